"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

Every error path is forced with argument values the host rejects before
enqueueing anything; the fake device addresses used here are never
dereferenced."""
import ctypes
import os
import re

import pytest

import oracle as R
from video_dit_sparse_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "vdsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libvdsa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(L.EXPORTED), names
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert L.abi_version() == 5
    for code in L.STATUS_NAMES:
        assert L.lib().vdsa_status_string(code)


def test_kernel_choice_per_workload():
    # the kernel sta_attn_fwd launches, by the largest query tile's token count
    # (and dtype / head_dim): the workloads' tiles and two edge cases
    from video_dit_sparse_amd import workloads as WL
    want = {"tiny_f32": "box_attn_f32_kernel<64>", "sta_720p": "box_attn_bf16_pp_kernel<1>",
            "dual_1080p": "box_attn_bf16_pp_kernel<0>", "local_global_4k": "box_attn_bf16_m16_kernel<8, 1, true>",
            "cross_window_2k": "box_attn_bf16_kernel<128>"}
    for name, kernel in want.items():
        w = WL.WORKLOADS[name]
        for s in w.shifts:
            assert L.sta_kernel_name(w.batch, w.heads, w.head_dim, w.grid, w.tile, w.window, s,
                                     dtype=w.dtype) == kernel, (name, s)
    # the 384-query kernel's key walk: tile by tile when every tile is full and
    # a tile frame is 64 tokens (on the rolled grid for the cyclic mode), else
    # raster (a lattice shift makes edge tiles partial; so does a ragged grid)
    g720, t720, w720 = (30, 48, 80), (6, 8, 8), (3, 3, 5)
    assert L.sta_kernel_name(1, 24, 128, g720, t720, w720, (3, 4, 4), "cyclic") == "box_attn_bf16_pp_kernel<2>"
    assert L.sta_kernel_name(1, 24, 128, g720, t720, w720, (0, 0, 0), "inward") == "box_attn_bf16_pp_kernel<1>"
    assert L.sta_kernel_name(1, 24, 128, g720, t720, w720, (3, 4, 4)) == "box_attn_bf16_pp_kernel<0>"
    assert L.sta_kernel_name(1, 24, 128, (30, 48, 81), t720, w720) == "box_attn_bf16_pp_kernel<0>"
    assert L.sta_kernel_name(1, 24, 128, (30, 48, 80), (6, 4, 16), w720) == "box_attn_bf16_pp_kernel<1>"
    # the 192-query kernel walks whole tiles too, but keeps the raster walk
    # in the cyclic mode
    g4k, t4k, w4k = (21, 136, 240), (3, 8, 8), (3, 5, 5)
    assert L.sta_kernel_name(1, 24, 128, g4k, t4k, w4k, (1, 4, 4), "cyclic") == "box_attn_bf16_m16_kernel<4, 0>"
    assert L.sta_kernel_name(1, 24, 128, g4k, t4k, w4k, (1, 4, 4)) == "box_attn_bf16_m16_kernel<4, 0>"
    # head_dim 64 always takes the 128-query kernel; a 384-token tile in a
    # grid that clips it to 40 tokens pads a 384-query block by far more than
    # 1/8, so the 128-query kernel takes it
    assert L.sta_kernel_name(1, 2, 64, (12, 16, 24), (6, 8, 8), (1, 3, 3)) == "box_attn_bf16_kernel<64>"
    assert L.sta_kernel_name(1, 2, 128, (5, 1, 8), (6, 8, 8), (1, 1, 1)) == "box_attn_bf16_kernel<128>"
    with pytest.raises(ValueError, match="window"):
        L.sta_kernel_name(1, 2, 128, (4, 8, 8), (2, 4, 4), (2, 3, 3))


# fake, 256-aligned device addresses: validation fails before any use
Q, K, V, O, LSE, WS = (0x10000000 * (i + 1) for i in range(6))


def prob(**kw):
    d = dict(batch=1, heads=2, head_dim=128, grid=(4, 8, 8), dtype=L.VDSA_BF16, scale=0.125)
    d.update(kw)
    return L.make_problem(d["batch"], d["heads"], d["head_dim"], d["grid"], d["dtype"], d["scale"])


def st(p, D=128):
    N = p.grid_t * p.grid_h * p.grid_w
    return L.Strides(p.heads * N * D, N * D, D)


def sta(p, cfg, q=Q, k=K, v=V, o=O, lse=None, strides=None):
    s = strides or {}
    d = st(p, p.head_dim)
    return L.lib().sta_attn_fwd(ctypes.byref(p), ctypes.byref(cfg) if cfg is not None else None,
                                q, ctypes.byref(s.get("q", d)), k, ctypes.byref(s.get("k", d)),
                                v, ctypes.byref(s.get("v", d)), o, ctypes.byref(s.get("o", d)), lse, None)


GOOD_CFG = dict(tile=(2, 4, 4), window=(3, 3, 3), shift=(0, 0, 0))


def cfg(**kw):
    d = dict(GOOD_CFG)
    d.update(kw)
    c = L.make_cfg(d["tile"], d["window"], d["shift"])
    if "window_mode" in d:
        c.window_mode = d["window_mode"]
    return c


@pytest.mark.parametrize("kw,code", [
    (dict(tile=(0, 4, 4)), "VDSA_ERR_WINDOW"),
    (dict(window=(2, 3, 3)), "VDSA_ERR_WINDOW"),
    (dict(window=(3, 0, 3)), "VDSA_ERR_WINDOW"),
    (dict(shift=(2, 0, 0)), "VDSA_ERR_WINDOW"),
    (dict(shift=(0, -1, 0)), "VDSA_ERR_WINDOW"),
    (dict(window_mode=3), "VDSA_ERR_WINDOW"),
    (dict(window_mode=-1), "VDSA_ERR_WINDOW"),
])
def test_bad_window_config(kw, code):
    assert sta(prob(), cfg(**kw)) == L.STATUS[code]
    assert L.lib().vdsa_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), "VDSA_ERR_UNSUPPORTED"),
    (dict(dtype=7), "VDSA_ERR_UNSUPPORTED"),
    (dict(scale=float("nan")), "VDSA_ERR_UNSUPPORTED"),
    (dict(scale=-1.0), "VDSA_ERR_UNSUPPORTED"),
    (dict(heads=0), "VDSA_ERR_SHAPE"),
    (dict(grid=(0, 8, 8)), "VDSA_ERR_SHAPE"),
])
def test_bad_problem(kw, code):
    assert sta(prob(**kw), cfg()) == L.STATUS[code]


def test_null_pointers():
    p = prob()
    assert L.lib().sta_attn_fwd(None, ctypes.byref(cfg()), Q, None, K, None, V, None, O, None, None, None) == 1
    assert sta(p, None) == L.STATUS["VDSA_ERR_NULL"]
    assert sta(p, cfg(), q=None) == L.STATUS["VDSA_ERR_NULL"]
    assert sta(p, cfg(), o=None) == L.STATUS["VDSA_ERR_NULL"]


def test_misaligned_pointer_and_stride():
    p = prob()
    assert sta(p, cfg(), k=K + 2) == L.STATUS["VDSA_ERR_ALIGN"]
    bad = L.Strides(2 * 256 * 136, 256 * 136, 132)   # 132 bf16 = 264 bytes: not a multiple of 16
    assert sta(p, cfg(), strides={"v": bad}) == L.STATUS["VDSA_ERR_ALIGN"]
    assert sta(p, cfg(), lse=LSE + 2) == L.STATUS["VDSA_ERR_ALIGN"]


def test_aliasing():
    p = prob()
    assert sta(p, cfg(), o=Q) == L.STATUS["VDSA_ERR_ALIAS"]
    assert sta(p, cfg(), o=V + 1024) == L.STATUS["VDSA_ERR_ALIAS"]
    assert sta(p, cfg(), lse=O + 64) == L.STATUS["VDSA_ERR_ALIAS"]
    # output rows overlapping each other (token stride smaller than head_dim)
    assert sta(p, cfg(), strides={"o": L.Strides(2 * 256 * 64, 256 * 64, 64)}) == L.STATUS["VDSA_ERR_ALIAS"]


def test_offset_limit():
    # 2^32 elements of token offset inside one head is beyond the kernels' addressing
    p = prob(grid=(64, 256, 256))
    big = L.Strides(0, 0, 1 << 20)
    assert sta(p, cfg(), strides={"q": big}) == L.STATUS["VDSA_ERR_SHAPE"]


def test_global_workspace_checks():
    p = prob()
    pool = (ctypes.c_int32 * 2)(4, 4)
    n = ctypes.c_size_t()
    assert L.lib().global_pooled_attn_workspace_size(ctypes.byref(p), pool, ctypes.byref(n)) == 0
    M = 4 * 2 * 2
    assert n.value == 2 * (((1 * 2 * M * 128 * 2) + 255) // 256 * 256)
    d = st(p)
    args = lambda ws, wsb, pl=pool: L.lib().global_pooled_attn_fwd(
        ctypes.byref(p), pl, Q, ctypes.byref(d), K, ctypes.byref(d), V, ctypes.byref(d), O, ctypes.byref(d),
        None, ws, wsb, None)
    assert args(None, n.value) == L.STATUS["VDSA_ERR_WORKSPACE"]
    assert args(WS, n.value - 1) == L.STATUS["VDSA_ERR_WORKSPACE"]
    assert args(Q + 256, n.value) == L.STATUS["VDSA_ERR_ALIAS"]
    assert args(WS, n.value, (ctypes.c_int32 * 2)(0, 4)) == L.STATUS["VDSA_ERR_WINDOW"]


def test_merge_checks():
    p = prob()
    d = st(p)
    m = lambda a, g, wl, wg, o: L.lib().dual_branch_merge(ctypes.byref(p), a, ctypes.byref(d), g, ctypes.byref(d),
                                                           wl, wg, o, ctypes.byref(d), None)
    assert m(Q, K, None, None, O) == L.STATUS["VDSA_ERR_NULL"]
    assert m(Q, K, None, WS, K) == L.STATUS["VDSA_ERR_ALIAS"]          # out == o_global
    assert m(Q, K, None, WS, Q + 512) == L.STATUS["VDSA_ERR_ALIAS"]    # partial overlap with o_local
    assert m(Q, K, None, WS + 2, O) == L.STATUS["VDSA_ERR_ALIGN"]


def test_merge_lse_checks():
    p = prob()
    d = st(p)
    LSE2 = WS   # a second LSE array
    m = lambda a, la, g, lg, o, lo: L.lib().dual_branch_merge_lse(
        ctypes.byref(p), a, ctypes.byref(d), la, g, ctypes.byref(d), lg, o, ctypes.byref(d), lo, None)
    assert m(Q, None, K, LSE2, O, None) == L.STATUS["VDSA_ERR_NULL"]
    assert m(Q, LSE, K, None, O, None) == L.STATUS["VDSA_ERR_NULL"]
    assert m(Q, LSE + 2, K, LSE2, O, None) == L.STATUS["VDSA_ERR_ALIGN"]
    assert m(Q, LSE, K, LSE2, Q + 512, None) == L.STATUS["VDSA_ERR_ALIAS"]    # partial overlap with o_local
    assert m(Q, LSE, K, LSE2, K + 256, None) == L.STATUS["VDSA_ERR_ALIAS"]    # partial overlap with o_global
    assert m(Q, LSE, K, LSE2, O, O + 64) == L.STATUS["VDSA_ERR_ALIAS"]        # lse_out inside out
    assert m(Q, LSE, K, LSE2, O, LSE + 4) == L.STATUS["VDSA_ERR_ALIAS"]       # lse_out straddles lse_local
    assert m(Q, LSE, K, LSE2, O, LSE2 + 8) == L.STATUS["VDSA_ERR_ALIAS"]      # lse_out straddles lse_global
    assert m(Q, LSE, K, LSE2, LSE, None) == L.STATUS["VDSA_ERR_ALIAS"]        # out over lse_local


def test_fused_global_merge_checks():
    p = prob()
    d = st(p)
    pool = (ctypes.c_int32 * 2)(4, 4)
    n = ctypes.c_size_t()
    assert L.lib().global_pooled_attn_workspace_size(ctypes.byref(p), pool, ctypes.byref(n)) == 0
    OL, GATE = 0x80000000, 0x90000000

    def f(mode, ol=OL, lse_l=None, wl=None, wg=GATE, out=O, lse_out=None, ws=WS, wsb=None):
        return L.lib().global_pooled_attn_merge_fwd(
            ctypes.byref(p), pool, Q, ctypes.byref(d), K, ctypes.byref(d), V, ctypes.byref(d), mode,
            ol, ctypes.byref(d), lse_l, wl, wg, out, ctypes.byref(d), lse_out, ws,
            n.value if wsb is None else wsb, None)
    assert f(7) == L.STATUS["VDSA_ERR_UNSUPPORTED"]
    assert f(-1) == L.STATUS["VDSA_ERR_UNSUPPORTED"]
    assert f(L.VDSA_MERGE_GATED, wg=None) == L.STATUS["VDSA_ERR_NULL"]
    assert f(L.VDSA_MERGE_GATED, wg=GATE + 2) == L.STATUS["VDSA_ERR_ALIGN"]
    assert f(L.VDSA_MERGE_LSE, lse_l=None) == L.STATUS["VDSA_ERR_NULL"]
    assert f(L.VDSA_MERGE_LSE, lse_l=LSE + 1) == L.STATUS["VDSA_ERR_ALIGN"]
    assert f(L.VDSA_MERGE_GATED, ol=None) == L.STATUS["VDSA_ERR_NULL"]
    assert f(L.VDSA_MERGE_GATED, out=OL + 512) == L.STATUS["VDSA_ERR_ALIAS"]       # out straddles o_local
    assert f(L.VDSA_MERGE_GATED, ol=WS + 256) == L.STATUS["VDSA_ERR_ALIAS"]        # o_local in the workspace
    assert f(L.VDSA_MERGE_GATED, out=Q) == L.STATUS["VDSA_ERR_ALIAS"]              # out over q
    assert f(L.VDSA_MERGE_LSE, lse_l=LSE, lse_out=LSE + 4) == L.STATUS["VDSA_ERR_ALIAS"]
    assert f(L.VDSA_MERGE_LSE, lse_l=O + 64) == L.STATUS["VDSA_ERR_ALIAS"]         # lse_local inside out
    assert f(L.VDSA_MERGE_GATED, wsb=n.value - 1) == L.STATUS["VDSA_ERR_WORKSPACE"]


def test_backward_checks():
    p = prob()
    d = st(p)
    c = cfg()
    n = ctypes.c_size_t()
    assert L.lib().sta_attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value >= 1 * 2 * 256 * 4   # delta: [batch, heads, N] fp32
    DO, DQ, DK, DV = 0x80000000, 0x90000000, 0xA0000000, 0xB0000000

    def b(pp=p, lse=LSE, dq=DQ, dk=DK, dv=DV, ws=WS, wsb=None, o=O):
        return L.lib().sta_attn_bwd(ctypes.byref(pp), ctypes.byref(c), Q, ctypes.byref(d), K, ctypes.byref(d),
                                    V, ctypes.byref(d), o, ctypes.byref(d), DO, ctypes.byref(d), lse,
                                    dq, ctypes.byref(d), dk, ctypes.byref(d), dv, ctypes.byref(d), ws,
                                    n.value if wsb is None else wsb, None)
    assert b(lse=None) == L.STATUS["VDSA_ERR_NULL"]
    assert b(dq=None) == L.STATUS["VDSA_ERR_NULL"]
    assert b(dk=Q + 512) == L.STATUS["VDSA_ERR_ALIAS"]        # dk over q
    assert b(dv=DK + 256) == L.STATUS["VDSA_ERR_ALIAS"]       # dv straddles dk
    assert b(dq=LSE) == L.STATUS["VDSA_ERR_ALIAS"]            # dq over lse
    assert b(ws=None) == L.STATUS["VDSA_ERR_WORKSPACE"]
    assert b(wsb=n.value - 1) == L.STATUS["VDSA_ERR_WORKSPACE"]
    assert b(ws=DV + 256) == L.STATUS["VDSA_ERR_ALIAS"]       # workspace inside dv
    assert b(pp=prob(head_dim=64)) == L.STATUS["VDSA_ERR_UNSUPPORTED"]   # bf16 backward: head_dim 128
    pool = (ctypes.c_int32 * 2)(4, 4)
    gn = ctypes.c_size_t()
    assert L.lib().global_pooled_attn_bwd_workspace_size(ctypes.byref(p), pool, ctypes.byref(gn)) == 0
    assert gn.value > n.value

    def gb(lse=LSE, wsb=None, pl=pool):
        return L.lib().global_pooled_attn_bwd(ctypes.byref(p), pl, Q, ctypes.byref(d), K, ctypes.byref(d),
                                              V, ctypes.byref(d), O, ctypes.byref(d), DO, ctypes.byref(d), lse,
                                              DQ, ctypes.byref(d), DK, ctypes.byref(d), DV, ctypes.byref(d), WS,
                                              gn.value if wsb is None else wsb, None)
    assert gb(lse=None) == L.STATUS["VDSA_ERR_NULL"]
    assert gb(wsb=gn.value - 1) == L.STATUS["VDSA_ERR_WORKSPACE"]
    assert gb(pl=(ctypes.c_int32 * 2)(0, 4)) == L.STATUS["VDSA_ERR_WINDOW"]


def test_variant_checks():
    p = prob()
    d = st(p)
    c = cfg()
    pool = (ctypes.c_int32 * 2)(2, 2)
    n = ctypes.c_size_t()
    assert L.lib().hier_pooled_attn_workspace_size(ctypes.byref(p), pool, ctypes.byref(n)) == 0
    h = lambda wsb, pl=pool, cc=c: L.lib().hier_pooled_attn_fwd(
        ctypes.byref(p), ctypes.byref(cc), pl, Q, ctypes.byref(d), K, ctypes.byref(d), V, ctypes.byref(d),
        O, ctypes.byref(d), None, WS, wsb, None)
    assert h(n.value - 1) == L.STATUS["VDSA_ERR_WORKSPACE"]
    assert h(n.value, (ctypes.c_int32 * 2)(2, 0)) == L.STATUS["VDSA_ERR_WINDOW"]
    assert h(n.value, pool, cfg(window=(2, 3, 3))) == L.STATUS["VDSA_ERR_WINDOW"]
    # the hierarchical variant is defined for clipped windows only
    for mode in (1, 2):
        assert h(n.value, pool, cfg(window_mode=mode)) == L.STATUS["VDSA_ERR_WINDOW"]
        f = ctypes.c_double()
        assert L.lib().vdsa_hier_flops(ctypes.byref(p), ctypes.byref(cfg(window_mode=mode)), pool,
                                       ctypes.byref(f)) == L.STATUS["VDSA_ERR_WINDOW"]
    m = ctypes.c_size_t()
    assert L.lib().compressed_global_attn_workspace_size(ctypes.byref(p), pool, ctypes.byref(m)) == 0
    assert m.value == 2 * n.value
    g = lambda wsb, o=O: L.lib().compressed_global_attn_fwd(
        ctypes.byref(p), pool, Q, ctypes.byref(d), K, ctypes.byref(d), V, ctypes.byref(d), o, ctypes.byref(d),
        WS, wsb, None)
    assert g(m.value - 1) == L.STATUS["VDSA_ERR_WORKSPACE"]
    assert g(m.value, Q + 256) == L.STATUS["VDSA_ERR_ALIAS"]


FLOP_CASES = [
    ((4, 8, 8), (2, 4, 4), (3, 3, 3), (0, 0, 0)),
    ((30, 48, 80), (6, 8, 8), (3, 3, 5), (0, 0, 0)),
    ((21, 68, 120), (21, 17, 30), (1, 1, 1), (0, 0, 0)),
    ((21, 90, 160), (4, 8, 8), (1, 1, 1), (0, 0, 0)),
    ((21, 90, 160), (4, 8, 8), (1, 1, 1), (2, 4, 4)),
    ((7, 13, 21), (3, 4, 8), (3, 3, 1), (1, 2, 4)),
    ((5, 9, 11), (2, 3, 3), (1, 3, 5), (1, 0, 2)),
]


@pytest.mark.parametrize("grid,tile,window,shift", FLOP_CASES)
def test_flop_counter_matches_oracle(grid, tile, window, shift):
    got = L.sta_flops(1, 3, 128, grid, tile, window, shift)
    assert got == R.sta_flops_ref(grid, tile, window, shift, head_dim=128, heads=3)


@pytest.mark.parametrize("mode", ["inward", "cyclic"])
@pytest.mark.parametrize("grid,tile,window,shift", FLOP_CASES + [
    ((6, 10, 14), (2, 4, 4), (3, 3, 3), (1, 2, 2)),
    ((3, 12, 16), (1, 4, 4), (1, 5, 3), (0, 2, 3)),
])
def test_flop_counter_window_modes(grid, tile, window, shift, mode):
    got = L.sta_flops(1, 3, 128, grid, tile, window, shift, window_mode=mode)
    assert got == R.sta_flops_ref(grid, tile, window, shift, head_dim=128, heads=3, window_mode=mode)


def test_global_flop_counter_matches_oracle():
    for grid, pool in [((21, 68, 120), (4, 4)), ((21, 136, 240), (8, 8)), ((3, 9, 10), (4, 3))]:
        assert L.global_flops(1, 24, 128, grid, pool) == R.global_flops_ref(grid, pool, head_dim=128, heads=24)


@pytest.mark.parametrize("grid,tile,window,shift,pool", [
    ((3, 8, 16), (1, 4, 4), (1, 3, 3), (0, 0, 0), (2, 2)),
    ((2, 9, 11), (1, 3, 4), (1, 3, 3), (0, 1, 1), (2, 2)),
    ((21, 68, 120), (21, 17, 30), (1, 1, 1), (0, 0, 0), (2, 2)),
    ((4, 10, 14), (2, 4, 6), (3, 1, 3), (1, 2, 3), (4, 3)),
])
def test_hier_flop_counter_matches_oracle(grid, tile, window, shift, pool):
    got = L.hier_flops(1, 2, 128, grid, tile, window, pool, shift)
    assert got == 4.0 * 128 * 2 * R.hier_pair_count_ref(grid, tile, window, shift, pool)


def test_compressed_global_flop_counter():
    T, H, W = 21, 68, 120
    M = T * 17 * 30
    assert L.compressed_global_flops(1, 24, 128, (T, H, W), (4, 4)) == 4.0 * 128 * 24 * M * M


def test_last_error_is_per_thread():
    """vdsa_last_error is thread-local: threads failing with different
    errors each read back their own detail, and a successful host-only call
    clears only its own thread's message."""
    import threading
    results = {}
    barrier = threading.Barrier(4)

    def worker(i):
        lib = L.lib()
        bad = cfg(window=(2 * i + 2, 3, 3))          # even window: VDSA_ERR_WINDOW
        barrier.wait()
        st = sta(prob(), bad)
        barrier.wait()                              # every thread has failed before anyone reads
        msg = lib.vdsa_last_error().decode()
        ok = L.sta_flops(1, 2, 128, (4, 8, 8), (2, 4, 4), (3, 3, 3))
        results[i] = (st, msg, lib.vdsa_last_error().decode(), ok)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i in range(4):
        st, msg, after, ok = results[i]
        assert st == L.STATUS["VDSA_ERR_WINDOW"]
        assert f"= {2 * i + 2}" in msg, msg
        assert after == "" and ok > 0


def test_noalloc_global_host_checks():
    # every check of the entry point that allocates nothing runs before its
    # first HIP call (the scratch lookup), so each path is forced here
    def g(p, pool=(4, 4), o=O, lse=None):
        d = st(p, p.head_dim)
        return L.lib().global_pooled_attn_fwd_noalloc(ctypes.byref(p), L._pool(pool), Q, ctypes.byref(d), K,
                                                      ctypes.byref(d), V, ctypes.byref(d), o, ctypes.byref(d),
                                                      lse, None)
    # 4K latent, 4 x 4 pooling: pooled K + V = 2 x 263 MB, beyond the 128 MiB scratch
    big = prob(heads=24, grid=(21, 136, 240))
    assert g(big) == L.STATUS["VDSA_ERR_WORKSPACE"]
    assert "static scratch" in L.lib().vdsa_last_error().decode()
    # the same latent at 8 x 8 pooling fits (2 x 65.8 MB); it fails here only at the alignment check
    assert g(big, pool=(8, 8), o=O + 8) == L.STATUS["VDSA_ERR_ALIGN"]
    assert 2 * 24 * 21 * 17 * 30 * 128 * 2 <= L.STATIC_SCRATCH_BYTES
    p = prob()
    assert g(p, pool=(0, 4)) == L.STATUS["VDSA_ERR_WINDOW"]
    assert g(p, o=None) == L.STATUS["VDSA_ERR_NULL"]
    assert g(p, lse=LSE + 2) == L.STATUS["VDSA_ERR_ALIGN"]
    assert g(p, o=Q) == L.STATUS["VDSA_ERR_ALIAS"]
