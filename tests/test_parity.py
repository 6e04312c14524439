"""GPU parity: the HIP path through the C ABI against the CPU fp64 oracle.

Small shapes are compared on every output element; the five workloads at
their full sizes are compared on sampled query rows (corner, edge and random
tiles), which the oracle evaluates exactly (rows are independent)."""
import sys

import numpy as np
import pytest
import torch

import oracle as R
import video_dit_sparse_amd as V
from video_dit_sparse_amd import pipeline as P
from video_dit_sparse_amd import workloads as WL
from _parity import compare, head_f64, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    V.lib()  # fail loudly if the library is missing


def qkv(shape, dtype, seed, scale=1.0):
    return [WL.make_tensor(shape, dtype, DEV, seed=seed + i, scale=scale) for i in range(3)]


TDT = {"bf16": torch.bfloat16, "f32": torch.float32}

SMALL_STA = [
    # name, grid, tile, window, shift, heads, head_dim, dtype
    ("tiny_dense_f32", (4, 8, 8), (2, 4, 4), (3, 3, 3), (0, 0, 0), 2, 64, "f32"),
    ("sparse_bf16", (8, 16, 16), (2, 4, 4), (3, 3, 3), (0, 0, 0), 2, 128, "bf16"),
    ("partial_shift_bf16", (7, 13, 21), (3, 4, 8), (3, 3, 1), (1, 2, 4), 2, 128, "bf16"),
    ("d64_bf16", (5, 9, 11), (2, 3, 3), (1, 3, 5), (1, 0, 2), 3, 64, "bf16"),
    ("sparse_f32", (6, 12, 12), (2, 4, 4), (3, 1, 3), (1, 2, 0), 2, 128, "f32"),
    ("d64_f32", (5, 9, 11), (2, 3, 3), (1, 3, 5), (1, 0, 2), 2, 64, "f32"),
    ("window1_shift_bf16", (4, 16, 24), (4, 8, 8), (1, 1, 1), (2, 4, 4), 2, 128, "bf16"),
    ("unit_tiles_bf16", (3, 6, 10), (1, 1, 1), (3, 3, 5), (0, 0, 0), 1, 128, "bf16"),
    ("full_window_bf16", (4, 12, 20), (2, 4, 4), (3, 5, 9), (0, 0, 0), 1, 128, "bf16"),
    ("big_tile_bf16", (3, 17, 30), (3, 17, 30), (1, 1, 1), (0, 0, 0), 1, 128, "bf16"),
    ("single_token_grid_bf16", (1, 1, 1), (1, 1, 1), (1, 1, 1), (0, 0, 0), 1, 128, "bf16"),
    # 384- and 192-token tiles run the 48-queries-per-wave kernel
    ("tile384_bf16", (12, 16, 24), (6, 8, 8), (1, 3, 3), (0, 0, 0), 2, 128, "bf16"),
    ("tile384_shift_bf16", (11, 13, 21), (6, 8, 8), (3, 1, 3), (3, 4, 4), 1, 128, "bf16"),
    # self-window with shifted partial tiles: key boxes of 1, 2 (ragged), 3 and 6 blocks
    ("tile384_self_shift_bf16", (12, 16, 16), (6, 8, 8), (1, 1, 1), (3, 4, 4), 2, 128, "bf16"),
    ("tile192_bf16", (6, 16, 24), (3, 8, 8), (3, 3, 3), (0, 0, 0), 2, 128, "bf16"),
    ("tile192_shift_bf16", (7, 12, 20), (3, 8, 8), (1, 3, 1), (1, 4, 4), 1, 128, "bf16"),
    # 256-token tiles (the 2K workload's tile), plain and shifted with ragged edges
    ("tile256_bf16", (8, 16, 24), (4, 8, 8), (3, 1, 3), (0, 0, 0), 2, 128, "bf16"),
    ("tile256_shift_ragged_bf16", (9, 19, 21), (4, 8, 8), (1, 3, 3), (2, 4, 4), 1, 128, "bf16"),
]


def oracle_sta(q, k, v, grid, tile, window, shift, scale, rows=None, heads=None):
    B, Hh = q.shape[:2]
    outs, lses = [], []
    for b in range(B):
        for h in (range(Hh) if heads is None else heads):
            o, l = R.sta_ref(head_f64(q, b, h), head_f64(k, b, h), head_f64(v, b, h), grid, tile, window,
                             shift, scale=scale, rows=rows)
            outs.append(o)
            lses.append(l)
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("case", SMALL_STA, ids=[c[0] for c in SMALL_STA])
def test_sta_small_all_rows(case):
    name, grid, tile, window, shift, heads, D, dt = case
    say(f"[sta small] {name}")
    N = int(np.prod(grid))
    q, k, v = qkv((1, heads, N, D), TDT[dt], seed=100)
    scale = D ** -0.5
    o, lse = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_sta(q, k, v, grid, tile, window, shift, scale)
    compare(o[0].cpu(), ro, dt, name)
    compare(lse[0].cpu(), rl, dt, name + " lse")


OUTLIER_STA = [
    # name, grid, tile, window, shift, dtype: each attention kernel in turn
    ("tile384_bf16", (12, 16, 24), (6, 8, 8), (1, 3, 3), (0, 0, 0), "bf16"),
    ("tile192_bf16", (6, 16, 24), (3, 8, 8), (3, 1, 3), (1, 4, 4), "bf16"),
    ("tile32_bf16", (8, 16, 16), (2, 4, 4), (3, 3, 3), (0, 0, 0), "bf16"),
    ("tile32_f32", (6, 12, 12), (2, 4, 4), (3, 1, 3), (1, 2, 0), "f32"),
]


@pytest.mark.parametrize("case", OUTLIER_STA, ids=[c[0] for c in OUTLIER_STA])
def test_sta_outlier_keys(case):
    """Large logits: 5% of the key rows scaled by 8 (exact in bf16), the
    structure of the 2K workload's inputs.  A kernel that rounds anything
    proportional to the logit (a pre-scaled bf16 Q, say) fails here first."""
    name, grid, tile, window, shift, dt = case
    say(f"[sta outliers] {name}")
    N = int(np.prod(grid))
    heads, D = 2, 128
    q, k, v = qkv((1, heads, N, D), TDT[dt], seed=950)
    gen = torch.Generator(device="cpu").manual_seed(951)
    for h in range(heads):
        rows = torch.randperm(N, generator=gen)[: N // 20].to(DEV)
        k[0, h, rows] *= 8
    o, lse = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_sta(q, k, v, grid, tile, window, shift, D ** -0.5)
    compare(o[0].cpu(), ro, dt, name)
    compare(lse[0].cpu(), rl, dt, name + " lse")


BATCH_STA = [
    # name, grid, tile, window, shift, dtype: each attention kernel with batch 2 and 3 heads
    ("tile384_bf16", (6, 16, 16), (6, 8, 8), (1, 3, 1), (0, 0, 0), "bf16"),
    ("tile192_bf16", (6, 16, 16), (3, 8, 8), (1, 1, 3), (1, 4, 4), "bf16"),
    ("tile32_bf16", (4, 12, 12), (2, 4, 4), (3, 1, 3), (0, 2, 0), "bf16"),
    ("tile32_f32", (4, 12, 12), (2, 4, 4), (1, 3, 3), (1, 0, 2), "f32"),
]


@pytest.mark.parametrize("case", BATCH_STA, ids=[c[0] for c in BATCH_STA])
def test_sta_batch2_heads3(case):
    """Batch and head decoding of the workgroup index in every kernel shape:
    two batches of three heads, each (batch, head) pair with its own inputs."""
    name, grid, tile, window, shift, dt = case
    say(f"[sta batch 2] {name}")
    N = int(np.prod(grid))
    q, k, v = qkv((2, 3, N, 128), TDT[dt], seed=970)
    o, lse = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_sta(q, k, v, grid, tile, window, shift, 128 ** -0.5)
    compare(o.reshape(6, N, 128).cpu(), ro, dt, name)
    compare(lse.reshape(6, N).cpu(), rl, dt, name + " lse")


@pytest.mark.parametrize("case", OUTLIER_STA, ids=[c[0] for c in OUTLIER_STA])
def test_sta_scale_zero(case):
    """Degenerate softmax: scale 0 gives every key of the window the same
    weight, so each row is the mean of V over its key box and LSE is the log
    of the box's key count."""
    name, grid, tile, window, shift, dt = case
    say(f"[sta scale 0] {name}")
    N = int(np.prod(grid))
    q, k, v = qkv((1, 2, N, 128), TDT[dt], seed=960)
    o, lse = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, scale=0.0, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_sta(q, k, v, grid, tile, window, shift, 0.0)
    compare(o[0].cpu(), ro, dt, name)
    compare(lse[0].cpu(), rl, dt, name + " lse")


def test_sta_bnhd_equals_bhnd():
    grid, tile, window, shift = (7, 13, 21), (3, 4, 8), (3, 3, 1), (1, 2, 4)
    N = int(np.prod(grid))
    q, k, v = qkv((1, 3, N, 128), torch.bfloat16, seed=7)
    qb, kb, vb = [x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for x in (q, k, v)]
    assert qb.stride(2) == 3 * 128
    o1 = V.sta_attn_fwd(q, k, v, grid, tile, window, shift)
    ob = torch.empty_like(qb)
    o2 = V.sta_attn_fwd(qb, kb, vb, grid, tile, window, shift, out=ob)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    ro, _ = oracle_sta(q, k, v, grid, tile, window, shift, 128 ** -0.5)
    compare(o2[0].cpu(), ro, "bf16", "bnhd")


def test_sta_deterministic_and_no_stray_writes():
    grid, tile, window, shift = (5, 9, 11), (2, 3, 3), (1, 3, 5), (1, 0, 2)
    N = int(np.prod(grid))
    q, k, v = qkv((2, 2, N, 128), torch.bfloat16, seed=11)
    pad = 64
    canary = torch.full((2 * 2 * N + 2 * pad, 128), -12345.0, dtype=torch.bfloat16, device=DEV)
    o = canary[pad:pad + 2 * 2 * N].view(2, 2, N, 128)
    V.sta_attn_fwd(q, k, v, grid, tile, window, shift, out=o)
    first = o.clone()
    V.sta_attn_fwd(q, k, v, grid, tile, window, shift, out=o)
    torch.cuda.synchronize()
    assert torch.equal(first, o)
    assert (canary[:pad] == -12345.0).all() and (canary[pad + 2 * 2 * N:] == -12345.0).all()
    ro, _ = oracle_sta(q, k, v, grid, tile, window, shift, 128 ** -0.5)
    compare(o.reshape(4, N, 128).cpu(), ro, "bf16", "batch 2")


TILE_WALK = [
    # name, grid, tile, window, shift, mode, kernel: every tile full and a
    # tile frame of 64 tokens, so the key boxes are walked tile by tile (walk
    # 1), on the rolled grid in the cyclic mode (walk 2)
    ("whole_tiles", (12, 16, 24), (6, 8, 8), (3, 3, 3), (0, 0, 0), "clip", "box_attn_bf16_pp_kernel<1>"),
    ("whole_tiles_4x16", (6, 8, 32), (6, 4, 16), (1, 3, 3), (0, 0, 0), "clip", "box_attn_bf16_pp_kernel<1>"),
    ("whole_tiles_inward", (12, 16, 40), (6, 8, 8), (1, 1, 3), (0, 0, 0), "inward", "box_attn_bf16_pp_kernel<1>"),
    ("rolled_whole_tiles", (12, 16, 24), (6, 8, 8), (3, 3, 5), (3, 4, 4), "cyclic", "box_attn_bf16_pp_kernel<2>"),
    # 192-token tiles: two tiles along w per workgroup (an odd count leaves the
    # last workgroup one tile; windows clipped at the edges), or one tile per
    # row of the lattice
    ("whole_tiles_192", (9, 16, 24), (3, 8, 8), (3, 3, 3), (0, 0, 0), "clip", "box_attn_bf16_m16_kernel<8, 1, true>"),
    ("whole_tiles_192_inward", (6, 24, 32), (3, 4, 16), (1, 5, 1), (0, 0, 0), "inward",
     "box_attn_bf16_m16_kernel<8, 1, true>"),
    ("whole_tiles_192_pairs_w5", (6, 16, 32), (3, 8, 8), (3, 3, 5), (0, 0, 0), "clip",
     "box_attn_bf16_m16_kernel<8, 1, true>"),
    ("whole_tiles_192_one_per_row", (6, 16, 8), (3, 8, 8), (3, 3, 1), (0, 0, 0), "clip",
     "box_attn_bf16_m16_kernel<4, 1>"),
]


@pytest.mark.parametrize("case", TILE_WALK, ids=[c[0] for c in TILE_WALK])
def test_tile_walk_bnhd_batch2(case):
    """The 384- and 192-query kernels' tile-by-tile key walks on batch 2, 2
    heads, token-major [B, N, heads, D] inputs, with LSE, against the oracle."""
    name, grid, tile, window, shift, mode, kernel = case
    assert V.sta_kernel_name(2, 2, 128, grid, tile, window, shift, mode) == kernel
    say(f"[tile walk] {name}")
    N = int(np.prod(grid))
    q, k, v = [WL.make_tensor((2, 2, N, 128), torch.bfloat16, DEV, seed=1500 + i) for i in range(3)]
    qb, kb, vb = [x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for x in (q, k, v)]
    o, lse = V.sta_attn_fwd(qb, kb, vb, grid, tile, window, shift, return_lse=True, window_mode=mode)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(2):
            ro, rl = R.sta_ref(head_f64(q, b, h), head_f64(k, b, h), head_f64(v, b, h), grid, tile, window, shift,
                               scale=128 ** -0.5, window_mode=mode)
            compare(o[b, h].cpu(), ro, "bf16", f"{name} b{b} h{h}")
            compare(lse[b, h].cpu(), rl, "bf16", f"{name} lse b{b} h{h}")


def test_reference_raise_pass():
    """Keys late in each key box whose logits jump far above the first keys'
    seen: the kernel must raise its softmax reference and repeat the walk."""
    grid, tile, window = (2, 16, 32), (2, 8, 8), (1, 3, 5)
    N = int(np.prod(grid))
    q, k, v = [WL.make_tensor((1, 2, N, 128), torch.float32, DEV, seed=31 + i) for i in range(3)]
    w = torch.arange(N, device=DEV) % grid[2]
    k[:, :, w >= 20] *= 40.0
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    o, lse = V.sta_attn_fwd(q, k, v, grid, tile, window, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_sta(q, k, v, grid, tile, window, (0, 0, 0), 128 ** -0.5)
    compare(o[0].cpu(), ro, "bf16", "reference raise")
    compare(lse[0].cpu(), rl, "bf16", "reference raise lse")


def test_heads_permute():
    grid, tile, window = (4, 16, 16), (2, 4, 4), (1, 3, 3)
    N = int(np.prod(grid))
    q, k, v = qkv((1, 4, N, 128), torch.bfloat16, seed=21)
    perm = [2, 0, 3, 1]
    o = V.sta_attn_fwd(q, k, v, grid, tile, window)
    op = V.sta_attn_fwd(q[:, perm].contiguous(), k[:, perm].contiguous(), v[:, perm].contiguous(), grid, tile, window)
    torch.cuda.synchronize()
    assert torch.equal(o[:, perm], op)
    # and every head of the permuted call against the oracle of the head it came from
    for i, hsrc in enumerate(perm):
        ro, _ = R.sta_ref(head_f64(q, 0, hsrc), head_f64(k, 0, hsrc), head_f64(v, 0, hsrc), grid, tile, window)
        compare(op[0, i].cpu(), ro, "bf16", f"permuted head {i} (from {hsrc})")


SMALL_GLOBAL = [
    ("pool4x4_bf16", (4, 8, 12), (4, 4), 2, 128, "bf16"),
    ("pool_ragged_bf16", (3, 9, 10), (4, 3), 2, 128, "bf16"),
    ("pool8x8_bf16", (2, 17, 30), (8, 8), 1, 128, "bf16"),
    ("pool_f32_d64", (3, 9, 10), (2, 3), 2, 64, "f32"),
    ("pool1_dense_bf16", (2, 6, 10), (1, 1), 1, 128, "bf16"),
    # 384-query blocks over the whole grid, the pooled keys walked in token
    # order: 540 keys (eight full 64-key blocks and a partial one), and 512
    # (whole blocks only)
    ("pool2x2_multi_block_bf16", (3, 20, 36), (2, 2), 2, 128, "bf16"),
    ("pool2x2_whole_blocks_bf16", (4, 16, 32), (2, 2), 1, 128, "bf16"),
]


@pytest.mark.parametrize("case", SMALL_GLOBAL, ids=[c[0] for c in SMALL_GLOBAL])
def test_global_small_all_rows(case):
    name, grid, pool, heads, D, dt = case
    say(f"[global small] {name}")
    N = int(np.prod(grid))
    q, k, v = qkv((1, heads, N, D), TDT[dt], seed=300)
    kp = V.kv_avgpool_fwd(k, grid, pool)
    o, lse = V.global_pooled_attn_fwd(q, k, v, grid, pool, return_lse=True)
    torch.cuda.synchronize()
    for h in range(heads):
        Kh, Vh, Qh = head_f64(k, 0, h), head_f64(v, 0, h), head_f64(q, 0, h)
        kpr, vpr = R.pool_ref(Kh, grid, pool), R.pool_ref(Vh, grid, pool)
        compare(kp[0, h].cpu(), kpr, dt, name + " pooled k")
        ro, rl = R.global_ref(Qh, kpr, vpr, scale=D ** -0.5)
        compare(o[0, h].cpu(), ro, dt, name + " global")
        compare(lse[0, h].cpu(), rl, dt, name + " global lse")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_merge_small(dt):
    N, heads = 1000, 3
    a, g, _ = qkv((2, heads, N, 128), TDT[dt], seed=400)
    wg = torch.rand(heads, device=DEV)
    wl = torch.rand(heads, device=DEV)
    out = V.dual_branch_merge(a, g, wg)
    out2 = V.dual_branch_merge(a, g, wg, w_local=wl)
    ref = R.merge_ref(R.to_f64(a).transpose(1, 0, 2, 3), R.to_f64(g).transpose(1, 0, 2, 3), None, wg.cpu())
    ref2 = R.merge_ref(R.to_f64(a).transpose(1, 0, 2, 3), R.to_f64(g).transpose(1, 0, 2, 3), wl.cpu(), wg.cpu())
    compare(out.cpu().transpose(0, 1), ref, dt, "merge")
    compare(out2.cpu().transpose(0, 1), ref2, dt, "merge w_local")
    V.dual_branch_merge(a, g, wg, out=a)   # in place on o_local
    torch.cuda.synchronize()
    assert torch.equal(a, out)


# ---------------------------------------------------------------- full-size workloads
def _check_workload(name, heads_to_check, n_random_tiles=4, rows_per_tile=24):
    w = WL.WORKLOADS[name]
    say(f"[workload] {name}: generating inputs")
    q, k, v = WL.make_qkv(w, DEV)
    gate = WL.make_gate(w, DEV)
    buf = P.Buffers(w, q)
    say(f"[workload] {name}: running")
    out = P.run(w, q, k, v, gate, buf, with_lse=True, fused=False)
    torch.cuda.synchronize()
    merged_fused = None
    if w.pool_hw is not None:
        # the fused global + merge call must give the same merged output
        merged_unfused = out["merged"].clone()
        out_f = P.run(w, q, k, v, gate, buf, with_lse=True, fused=True)
        torch.cuda.synchronize()
        merged_fused = out_f["merged"]
        d = (merged_fused.float() - merged_unfused.float()).abs()
        say(f"[workload] {name}: fused vs unfused merge max diff {d.max().item():.3e}")
        assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3
    for i, shift in enumerate(w.shifts):
        rows = sample_rows(w.grid, w.tile, shift, n_random_tiles, rows_per_tile, seed=i)
        for h in heads_to_check:
            say(f"[workload] {name}: local shift {shift} head {h}: {len(rows)} rows")
            ro, rl = R.sta_ref(head_f64(q, 0, h), head_f64(k, 0, h), head_f64(v, 0, h), w.grid, w.tile,
                               w.window, shift, scale=w.softmax_scale, rows=rows)
            compare(out["local"][i][0, h, rows].cpu(), ro, w.dtype, f"{name} local h{h}")
            compare(out["lse"][i][0, h, rows].cpu(), rl, w.dtype, f"{name} local lse h{h}")
            if w.pool_hw is not None and i == 0:
                kpr = R.pool_ref(head_f64(k, 0, h), w.grid, w.pool_hw)
                vpr = R.pool_ref(head_f64(v, 0, h), w.grid, w.pool_hw)
                M = kpr.shape[0]
                ws = out["workspace"]
                kpool = ws[: w.batch * w.heads * M * w.head_dim * 2].view(torch.bfloat16).view(
                    w.batch, w.heads, M, w.head_dim)
                compare(kpool[0, h].cpu(), kpr, w.dtype, f"{name} pooled k h{h}")
                # pooled V follows pooled K in the workspace, 256-byte aligned
                voff = -(-(w.batch * w.heads * M * w.head_dim * 2) // 256) * 256
                vpool = ws[voff: voff + w.batch * w.heads * M * w.head_dim * 2].view(torch.bfloat16).view(
                    w.batch, w.heads, M, w.head_dim)
                compare(vpool[0, h].cpu(), vpr, w.dtype, f"{name} pooled v h{h}")
                go, gl = R.global_ref(head_f64(q, 0, h), kpr, vpr, scale=w.softmax_scale, rows=rows)
                compare(out["glob"][0, h, rows].cpu(), go, w.dtype, f"{name} global h{h}")
                compare(out["glob_lse"][0, h, rows].cpu(), gl, w.dtype, f"{name} global lse h{h}")
                g = float(gate[h])
                mr = R.merge_ref(ro[None], go[None], None, np.array([g]))[0]
                compare(out["merged"][0, h, rows].cpu(), mr, w.dtype, f"{name} merged h{h}")
                compare(merged_fused[0, h, rows].cpu(), mr, w.dtype, f"{name} merged (fused) h{h}")
    # properties over every output element
    for t in out["local"]:
        assert torch.isfinite(t.float()).all()
    if w.pool_hw is not None:
        assert torch.isfinite(out["merged"].float()).all()


def test_workload_tiny_all_rows():
    w = WL.WORKLOADS["tiny_f32"]
    q, k, v = WL.make_qkv(w, DEV)
    o = V.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, scale=w.softmax_scale)
    torch.cuda.synchronize()
    ro, _ = oracle_sta(q, k, v, w.grid, w.tile, w.window, (0, 0, 0), w.softmax_scale)
    compare(o[0].cpu(), ro, "f32", "tiny_f32")
    # the tiny workload's window covers its 2x2x2 tile lattice: dense attention
    rd = np.stack([R.dense_ref(head_f64(q, 0, h), head_f64(k, 0, h), head_f64(v, 0, h), w.softmax_scale)[0]
                   for h in range(w.heads)])
    compare(o[0].cpu(), rd, "f32", "tiny_f32 dense")


def test_workload_sta_720p():
    _check_workload("sta_720p", heads_to_check=[0, 23])


def test_workload_sta_720p_full_head():
    # every element of one whole 720P head, O and LSE: all 300 query tiles,
    # corner, edge and interior, against the oracle
    w = WL.WORKLOADS["sta_720p"]
    h = 11
    q, k, v = WL.make_qkv(w, DEV)
    say(f"[workload] sta_720p full head {h}: running")
    o, lse = V.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, scale=w.softmax_scale, return_lse=True)
    torch.cuda.synchronize()
    say(f"[workload] sta_720p full head {h}: oracle over all {w.n_tokens} rows")
    ro, rl = R.sta_ref(head_f64(q, 0, h), head_f64(k, 0, h), head_f64(v, 0, h), w.grid, w.tile, w.window,
                       (0, 0, 0), scale=w.softmax_scale)
    compare(o[0, h].cpu(), ro, w.dtype, f"sta_720p full head {h}")
    compare(lse[0, h].cpu(), rl, w.dtype, f"sta_720p full head {h} lse")


def test_workload_dual_1080p():
    _check_workload("dual_1080p", heads_to_check=[5], rows_per_tile=16)


def test_workload_local_global_4k():
    _check_workload("local_global_4k", heads_to_check=[17], n_random_tiles=3, rows_per_tile=12)


def test_workload_cross_window_2k():
    _check_workload("cross_window_2k", heads_to_check=[0, 9])
