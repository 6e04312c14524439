"""GPU parity of the backward passes (``sta_attn_bwd``,
``global_pooled_attn_bwd``) through the C ABI against the CPU fp64 oracle,
on every gradient element.

Tolerance (bf16): the kernels round P and dS to bf16 for the matrix-core
products (relative rounding up to 2^-8, RMS about 2^-9) and take delta =
rowsum(dO * O) from the bf16 forward output; the global branch also rounds
the pooled K and V to bf16.  Each gradient element sums many such terms in
fp32, so its typical error is 2^-9 to sqrt(3) 2^-9 of the gradient's RMS
(measured 1.7e-3 to 2.7e-3).  Elements whose terms share a sign accumulate their rounding
linearly instead of as a random walk, giving a tail about ten times the mean;
and key gradients through the pooling are the cell gradient divided by the
cell's token count, so tokens of small ragged cells carry gradients many
times the RMS.  The bar: mean abs error <= 5e-3 * RMS (a dropped or wrong
term shows at the scale of the RMS itself) and, element by element,
abs error <= 6e-2 * (RMS + |reference|).  fp32: 1e-5 * RMS and
1e-4 * (RMS + |reference|).  Heavy-tailed gradients (keys with large
logits) break the RMS scaling; there the bar is the element-wise bound that
those roundings imply (``bwd_rounding_bound``).
"""
import sys

import numpy as np
import pytest
import torch

import oracle as R
import video_dit_sparse_amd as V
from video_dit_sparse_amd import workloads as WL
from _parity import bound_compare, bwd_rounding_bound, head_f64, rel_compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    V.lib()  # fail loudly if the library is missing


def tensors(shape, dtype, seed, n=4):
    return [WL.make_tensor(shape, dtype, DEV, seed=seed + i) for i in range(n)]


STA_BWD = [
    # name, batch, grid, tile, window, shift, heads, head_dim, dtype
    ("tile32_bf16", 1, (4, 8, 12), (2, 4, 4), (1, 3, 3), (0, 0, 0), 2, 128, "bf16"),
    ("shift_partial_bf16", 2, (3, 10, 13), (2, 4, 4), (3, 1, 3), (1, 2, 2), 1, 128, "bf16"),
    ("tile384_bf16", 1, (6, 16, 16), (6, 8, 8), (1, 3, 1), (0, 0, 0), 1, 128, "bf16"),
    ("tile384_b2h3_bf16", 2, (6, 8, 16), (6, 8, 8), (1, 1, 3), (0, 0, 0), 3, 128, "bf16"),
    # whole tiles of 64-token frames (4x16 and 2x32), walked tile by tile
    ("tile4x16_bf16", 1, (6, 8, 32), (6, 4, 16), (1, 3, 3), (0, 0, 0), 2, 128, "bf16"),
    ("tile2x32_bf16", 1, (4, 6, 64), (2, 2, 32), (3, 3, 1), (0, 0, 0), 1, 128, "bf16"),
    # self windows: boxes of one 32-token chunk (the dQ pass's odd-chunk group
    # has none), of two chunks, and of three with ragged edge tiles (a partial
    # last chunk in the 48-token tiles)
    ("self_1chunk_bf16", 1, (4, 8, 8), (2, 4, 4), (1, 1, 1), (0, 0, 0), 2, 128, "bf16"),
    ("self_2chunks_bf16", 1, (4, 8, 8), (2, 4, 8), (1, 1, 1), (0, 0, 0), 1, 128, "bf16"),
    ("self_3chunks_ragged_bf16", 2, (3, 8, 12), (3, 4, 8), (1, 1, 1), (0, 0, 0), 1, 128, "bf16"),
    ("f32_d64", 1, (3, 6, 8), (3, 3, 4), (1, 3, 1), (0, 1, 2), 2, 64, "f32"),
    ("f32_d128", 1, (2, 6, 8), (1, 3, 4), (1, 1, 3), (0, 0, 0), 1, 128, "f32"),
]


@pytest.mark.parametrize("case", STA_BWD, ids=[c[0] for c in STA_BWD])
def test_sta_bwd_small(case):
    name, B, grid, tile, window, shift, heads, D, dt = case
    say(f"[sta bwd] {name}")
    N = int(np.prod(grid))
    q, k, v, do = tensors((B, heads, N, D), TDT[dt], seed=800)
    o, lse = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, return_lse=True)
    dq, dk, dv = V.sta_attn_bwd(q, k, v, o, do, lse, grid, tile, window, shift)
    dq2, dk2, dv2 = V.sta_attn_bwd(q, k, v, o, do, lse, grid, tile, window, shift)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)   # deterministic
    for b in range(B):
        for h in range(heads):
            ref = R.sta_bwd_ref(head_f64(q, b, h), head_f64(k, b, h), head_f64(v, b, h), head_f64(do, b, h),
                                grid, tile, window, shift, scale=D ** -0.5)
            for nm, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
                rel_compare(got[b, h].cpu(), r, dt, f"{name} {nm} b{b} h{h}")


def test_sta_bwd_outlier_keys():
    """Large logits in the backward: 5% of the key rows scaled by 8 (exact in
    bf16), 384-token tiles (dK/dV pass over 64-query blocks, dQ pass over
    32-key blocks), compared on every gradient element against twice the
    element's rounding bound.  A CPU emulation of exactly those roundings
    (exact logits; P, dS and O rounded to bf16) reaches 0.36-0.83 of the
    bound on such inputs, and 0.06-0.09 x (RMS + |reference|) on dK, beyond
    the RMS-scaled bar of the other cases."""
    grid, tile, window, shift = (6, 16, 24), (6, 8, 8), (1, 1, 3), (0, 0, 0)
    say("[sta bwd] outlier keys")
    N, D = int(np.prod(grid)), 128
    q, k, v, do = tensors((1, 2, N, D), torch.bfloat16, seed=860)
    gen = torch.Generator(device="cpu").manual_seed(861)
    for h in range(2):
        k[0, h, torch.randperm(N, generator=gen)[: N // 20].to(DEV)] *= 8
    o, lse = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, return_lse=True)
    dq, dk, dv = V.sta_attn_bwd(q, k, v, o, do, lse, grid, tile, window, shift)
    torch.cuda.synchronize()
    for h in range(2):
        args = [head_f64(x, 0, h) for x in (q, k, v, do)]
        ref = R.sta_bwd_ref(*args, grid, tile, window, shift, scale=D ** -0.5)
        bounds = bwd_rounding_bound(*args, grid, tile, window, shift, D ** -0.5)
        for nm, got, r, bd in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, bounds):
            bound_compare(got[0, h].cpu(), r, bd, f"outlier {nm} h{h}")


def test_sta_bwd_720p_full_head():
    """The 720P workload's shape (30x48x80 grid, 6x8x8 tiles, 3x3x5 window) in
    the launch configuration the bench times, one head, every gradient
    element against the oracle (about half a minute of CPU)."""
    w = WL.WORKLOADS["sta_720p"]
    say("[sta bwd] 720P, one head, all elements")
    shape = (1, 1, w.n_tokens, w.head_dim)
    q, k, v, do = tensors(shape, torch.bfloat16, seed=880)
    o, lse = V.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, return_lse=True)
    dq, dk, dv = V.sta_attn_bwd(q, k, v, o, do, lse, w.grid, w.tile, w.window)
    torch.cuda.synchronize()
    ref = R.sta_bwd_ref(head_f64(q, 0, 0), head_f64(k, 0, 0), head_f64(v, 0, 0), head_f64(do, 0, 0),
                        w.grid, w.tile, w.window, scale=w.softmax_scale)
    for nm, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        rel_compare(got[0, 0].cpu(), r, "bf16", f"720p {nm}")


def test_global_bwd_1080p_full_head():
    """The 1080P workload's global branch (171,360 queries against 4x4-pooled
    K/V, M = 10,710), one head, every gradient element against the oracle."""
    w = WL.WORKLOADS["dual_1080p"]
    say("[global bwd] 1080P, one head, all elements")
    shape = (1, 1, w.n_tokens, w.head_dim)
    q, k, v, do = tensors(shape, torch.bfloat16, seed=890)
    o, lse = V.global_pooled_attn_fwd(q, k, v, w.grid, w.pool_hw, return_lse=True)
    dq, dk, dv = V.global_pooled_attn_bwd(q, k, v, o, do, lse, w.grid, w.pool_hw)
    torch.cuda.synchronize()
    ref = R.global_bwd_ref(head_f64(q, 0, 0), head_f64(k, 0, 0), head_f64(v, 0, 0), head_f64(do, 0, 0),
                           w.grid, w.pool_hw, scale=w.softmax_scale)
    for nm, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        rel_compare(got[0, 0].cpu(), r, "bf16", f"1080p global {nm}")


def _bnhd(x):
    """The same values as a [B, heads, N, D] view of a [B, N, heads, D] buffer."""
    return x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_bwd_bnhd_equals_bhnd(dt):
    """Strided (token-major) inputs and gradient outputs give the same
    gradients bit for bit, for the sliding-tile and the global backward."""
    grid, tile, window, shift, pool = (3, 12, 16), (3, 4, 8), (1, 3, 1), (1, 2, 4), (2, 4)
    N, D, heads = int(np.prod(grid)), 128, 3
    say(f"[bwd bnhd] {dt}")
    q, k, v, do = tensors((1, heads, N, D), TDT[dt], seed=870)
    qs, ks, vs, dos = (_bnhd(x) for x in (q, k, v, do))
    assert qs.stride(2) == heads * D
    o, lse = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, return_lse=True)
    os_ = _bnhd(o)
    g1 = V.sta_attn_bwd(q, k, v, o, do, lse, grid, tile, window, shift)
    g2 = V.sta_attn_bwd(qs, ks, vs, os_, dos, lse, grid, tile, window, shift,
                        dq=_bnhd(torch.empty_like(q)), dk=_bnhd(torch.empty_like(q)), dv=_bnhd(torch.empty_like(q)))
    og, lg = V.global_pooled_attn_fwd(q, k, v, grid, pool, return_lse=True)
    h1 = V.global_pooled_attn_bwd(q, k, v, og, do, lg, grid, pool)
    h2 = V.global_pooled_attn_bwd(qs, ks, vs, _bnhd(og), dos, lg, grid, pool,
                                  dq=_bnhd(torch.empty_like(q)), dk=_bnhd(torch.empty_like(q)), dv=_bnhd(torch.empty_like(q)))
    torch.cuda.synchronize()
    for nm, a, b in zip(("dq", "dk", "dv"), g1, g2):
        assert b.stride(2) == heads * D
        assert torch.equal(a, b), f"sta {nm}"
    for nm, a, b in zip(("dq", "dk", "dv"), h1, h2):
        assert torch.equal(a, b), f"global {nm}"


GLOBAL_BWD = [
    # name, batch, grid, pool, heads, head_dim, dtype
    ("pool2x4_bf16", 1, (3, 8, 12), (2, 4), 2, 128, "bf16"),
    ("pool_ragged_bf16", 2, (2, 9, 10), (4, 3), 1, 128, "bf16"),
    ("pool_f32_d64", 1, (3, 9, 10), (2, 3), 2, 64, "f32"),
]


@pytest.mark.parametrize("case", GLOBAL_BWD, ids=[c[0] for c in GLOBAL_BWD])
def test_global_bwd_small(case):
    name, B, grid, pool, heads, D, dt = case
    say(f"[global bwd] {name}")
    N = int(np.prod(grid))
    q, k, v, do = tensors((B, heads, N, D), TDT[dt], seed=820)
    o, lse = V.global_pooled_attn_fwd(q, k, v, grid, pool, return_lse=True)
    dq, dk, dv = V.global_pooled_attn_bwd(q, k, v, o, do, lse, grid, pool)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(heads):
            ref = R.global_bwd_ref(head_f64(q, b, h), head_f64(k, b, h), head_f64(v, b, h), head_f64(do, b, h),
                                   grid, pool, scale=D ** -0.5)
            for nm, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
                rel_compare(got[b, h].cpu(), r, dt, f"{name} {nm} b{b} h{h}")
