"""GPU parity of short key walks with many work items, through the C ABI
against the CPU fp64 oracle, on every output element.

Windows of one tile (UltraGen section 4.3: unshifted and half-shifted
partitions, each tile attending to itself) and of three tiles along one dim,
on 256-token tiles (the 2K workload's), with more tiles than an MI355X has
compute units and with partial tiles along every dim: key boxes of one to
twelve 64-key blocks, partial last blocks, and query blocks with lanes past
the tile's end.  The last test checks one whole head of the 2K workload in
both calls of the pair: with its outlier keys, the worst of its 38.7 million
output elements stay within the bar only when the softmax denominator sums the
probabilities as rounded to bf16 for the P.V product."""
import sys

import numpy as np
import pytest
import torch

import oracle as R
import video_dit_sparse_amd as V
from video_dit_sparse_amd import workloads as WL
from _parity import compare, head_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    V.lib()  # fail loudly if the library is missing


def n_items(batch, heads, grid, tile, shift, mode):
    sh = (0, 0, 0) if mode == "cyclic" else shift
    return batch * heads * int(np.prod([(L + s + b - 1) // b for L, b, s in zip(grid, tile, sh)]))


SHORT_WALK_CASES = [
    # name, batch, heads, grid, tile, window, shift, mode, with_lse
    # self windows on a shifted lattice: tiles of 2..4 frames, 4 or 8 rows and
    # columns, i.e. key boxes of 32 to 256 keys (one to four blocks, partial)
    ("self_shift", 1, 8, (9, 40, 48), (4, 8, 8), (1, 1, 1), (2, 4, 4), "clip", True),
    ("self_plain_no_lse", 1, 6, (9, 36, 56), (4, 8, 8), (1, 1, 1), (0, 0, 0), "clip", False),
    # windows of three tiles along w or h: key boxes of up to 12 blocks
    ("window_1x1x3", 1, 12, (7, 20, 40), (4, 8, 8), (1, 1, 3), (0, 0, 0), "clip", True),
    ("window_1x3x1_shift_batch2", 2, 4, (6, 24, 32), (4, 8, 8), (1, 3, 1), (2, 4, 4), "clip", True),
    ("self_cyclic", 1, 8, (9, 40, 48), (4, 8, 8), (1, 1, 1), (2, 4, 4), "cyclic", True),
    ("window_1x1x3_inward_no_lse", 1, 12, (7, 20, 40), (4, 8, 8), (1, 1, 3), (0, 0, 0), "inward", False),
]


@pytest.mark.parametrize("case", SHORT_WALK_CASES, ids=[c[0] for c in SHORT_WALK_CASES])
def test_short_walks_all_rows(case):
    name, B, H, grid, tile, window, shift, mode, with_lse = case
    items = n_items(B, H, grid, tile, shift, mode)
    say(f"[short walks] {name}: {items} items")
    assert items > 256
    N = int(np.prod(grid))
    q, k, v = [WL.make_tensor((B, H, N, 128), torch.bfloat16, DEV, seed=1200 + i) for i in range(3)]
    res = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, return_lse=with_lse, window_mode=mode)
    o, lse = res if with_lse else (res, None)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            ro, rl = R.sta_ref(head_f64(q, b, h), head_f64(k, b, h), head_f64(v, b, h), grid, tile, window, shift,
                               scale=128 ** -0.5, window_mode=mode)
            compare(o[b, h].cpu(), ro, "bf16", f"{name} b{b} h{h}")
            if with_lse:
                compare(lse[b, h].cpu(), rl, "bf16", f"{name} lse b{b} h{h}")


def test_short_walks_outliers_bnhd_canaries():
    """Large logits (5% of key rows scaled by 8, the 2K workload's inputs),
    token-major [B, N, heads, D] strides, and output and LSE buffers set
    inside larger ones filled with a sentinel: nothing outside the rows the
    call owns may change."""
    grid, tile, window, shift = (9, 40, 48), (4, 8, 8), (1, 1, 1), (2, 4, 4)
    H, N, D = 8, int(np.prod(grid)), 128
    q, k, v = [WL.make_tensor((1, H, N, D), torch.bfloat16, DEV, seed=1300 + i) for i in range(3)]
    gen = torch.Generator(device="cpu").manual_seed(1310)
    for h in range(H):
        rows = torch.randperm(N, generator=gen)[: N // 20].to(DEV)
        k[0, h, rows] *= 8
    qb, kb, vb = [x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for x in (q, k, v)]
    pad = 4096
    canary = torch.full((N * H * D + 2 * pad,), -12345.0, dtype=torch.bfloat16, device=DEV)
    ob = canary[pad:pad + N * H * D].view(1, N, H, D).permute(0, 2, 1, 3)
    lcan = torch.full((H * N + 2 * pad,), -777.0, dtype=torch.float32, device=DEV)
    lse = lcan[pad:pad + H * N].view(1, H, N)
    V.sta_attn_fwd(qb, kb, vb, grid, tile, window, shift, out=ob, lse=lse)
    o2 = V.sta_attn_fwd(q, k, v, grid, tile, window, shift)
    torch.cuda.synchronize()
    assert (canary[:pad] == -12345.0).all() and (canary[pad + N * H * D:] == -12345.0).all()
    assert (lcan[:pad] == -777.0).all() and (lcan[pad + H * N:] == -777.0).all()
    assert torch.equal(ob, o2)
    for h in range(H):
        ro, rl = R.sta_ref(head_f64(q, 0, h), head_f64(k, 0, h), head_f64(v, 0, h), grid, tile, window, shift,
                           scale=D ** -0.5)
        compare(ob[0, h].cpu(), ro, "bf16", f"outliers bnhd h{h}")
        compare(lse[0, h].cpu(), rl, "bf16", f"outliers bnhd lse h{h}")


def test_short_walks_deterministic_and_scale_zero():
    grid, tile, window, shift = (9, 36, 56), (4, 8, 8), (1, 1, 3), (2, 4, 4)
    H, N = 6, int(np.prod(grid))
    q, k, v = [WL.make_tensor((1, H, N, 128), torch.bfloat16, DEV, seed=1400 + i) for i in range(3)]
    a = V.sta_attn_fwd(q, k, v, grid, tile, window, shift)
    b = V.sta_attn_fwd(q, k, v, grid, tile, window, shift)
    # scale 0: each row is the mean of V over its key box, LSE the log of its size
    o0, l0 = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, scale=0.0, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    for h in (0, H - 1):
        ro, rl = R.sta_ref(head_f64(q, 0, h), head_f64(k, 0, h), head_f64(v, 0, h), grid, tile, window, shift,
                           scale=0.0)
        compare(o0[0, h].cpu(), ro, "bf16", f"scale 0 h{h}")
        compare(l0[0, h].cpu(), rl, "bf16", f"scale 0 lse h{h}")


def test_workload_cross_window_2k_full_head():
    """Every element of one whole head of the 2K workload, O and LSE, in both
    calls of the pair (unshifted, then shifted by half a tile), against the
    oracle: 302,400 rows each, 1,440 and 1,512 tiles."""
    w = WL.WORKLOADS["cross_window_2k"]
    h = 5
    q, k, v = WL.make_qkv(w, DEV)
    for shift in w.shifts:
        say(f"[workload] cross_window_2k full head {h}, shift {shift}: running")
        o, lse = V.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, shift, scale=w.softmax_scale, return_lse=True)
        torch.cuda.synchronize()
        say(f"[workload] cross_window_2k full head {h}, shift {shift}: oracle over all {w.n_tokens} rows")
        ro, rl = R.sta_ref(head_f64(q, 0, h), head_f64(k, 0, h), head_f64(v, 0, h), w.grid, w.tile, w.window,
                           shift, scale=w.softmax_scale)
        compare(o[0, h].cpu(), ro, w.dtype, f"2k full head {h} shift {shift}")
        compare(lse[0, h].cpu(), rl, w.dtype, f"2k full head {h} shift {shift} lse")
        del o, lse
