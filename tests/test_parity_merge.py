"""GPU parity of the exact log-sum-exp merge and of the global branch with a
merge fused into its epilogue, through the C ABI against the CPU fp64
oracle, on every output element.

The fused cases are sized so that the global branch (one query tile covering
the grid) runs each attention kernel in turn: 768 queries (384-query
kernel), 576 (192-query kernel), head_dim 64 (128-query kernel) and fp32."""
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
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    V.lib()  # fail loudly if the library is missing


def qkv(shape, dtype, seed):
    return [WL.make_tensor(shape, dtype, DEV, seed=seed + i) for i in range(3)]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_merge_lse_small(dt):
    B, heads, N, D = 2, 3, 1000, 128
    a, g, _ = qkv((B, heads, N, D), TDT[dt], seed=700)
    gen = torch.Generator(device="cpu").manual_seed(701)
    la = (3.0 * torch.randn((B, heads, N), generator=gen)).to(DEV)
    lg = (3.0 * torch.randn((B, heads, N), generator=gen)).to(DEV)
    out, lo = V.dual_branch_merge_lse(a, la, g, lg, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = R.merge_lse_ref(R.to_f64(a), R.to_f64(la), R.to_f64(g), R.to_f64(lg))
    compare(out.cpu(), ro, dt, "merge lse")
    compare(lo.cpu(), rl, "f32", "merge lse lse_out")
    # without lse_out, and in place on either input (and on its LSE)
    out1 = V.dual_branch_merge_lse(a, la, g, lg)
    a2, la2 = a.clone(), la.clone()
    V.dual_branch_merge_lse(a2, la2, g, lg, out=a2, lse_out=la2)
    g3 = g.clone()
    V.dual_branch_merge_lse(a, la, g3, lg, out=g3)
    torch.cuda.synchronize()
    assert torch.equal(out1, out) and torch.equal(a2, out) and torch.equal(la2, lo) and torch.equal(g3, out)


MERGE_CASES = [
    # name, batch, grid, tile, window, shift, pool, heads, head_dim, dtype
    ("q768_bf16", 2, (4, 12, 16), (2, 4, 4), (1, 3, 3), (0, 0, 0), (2, 4), 2, 128, "bf16"),
    ("tile384_b2h3_bf16", 2, (6, 16, 16), (6, 8, 8), (1, 1, 3), (0, 0, 0), (4, 4), 3, 128, "bf16"),
    ("q576_bf16", 1, (3, 12, 16), (3, 4, 4), (1, 1, 3), (1, 2, 2), (3, 4), 1, 128, "bf16"),
    # 2160 queries in six 384-query blocks of the global call, the last one ragged
    ("q2160_ragged_bf16", 1, (3, 20, 36), (3, 4, 4), (1, 3, 3), (0, 0, 0), (2, 2), 2, 128, "bf16"),
    ("d64_bf16", 1, (3, 9, 10), (3, 3, 5), (1, 3, 1), (0, 1, 2), (2, 3), 2, 64, "bf16"),
    ("d64_f32", 1, (3, 9, 10), (3, 3, 5), (1, 3, 1), (0, 0, 0), (2, 3), 2, 64, "f32"),
]


def _branch_refs(q, k, v, b, h, grid, pool, D):
    Qh, Kh, Vh = head_f64(q, b, h), head_f64(k, b, h), head_f64(v, b, h)
    kpr, vpr = R.pool_ref(Kh, grid, pool), R.pool_ref(Vh, grid, pool)
    return Qh, Kh, Vh, kpr, vpr


@pytest.mark.parametrize("case", MERGE_CASES, ids=[c[0] for c in MERGE_CASES])
def test_fused_gated_merge(case):
    name, B, grid, tile, window, shift, pool, heads, D, dt = case
    say(f"[fused gated] {name}")
    N = int(np.prod(grid))
    q, k, v = qkv((B, heads, N, D), TDT[dt], seed=710)
    o_loc = V.sta_attn_fwd(q, k, v, grid, tile, window, shift)
    wg = torch.rand(heads, device=DEV)
    wl = torch.rand(heads, device=DEV)
    out, lg = V.global_pooled_attn_merge_fwd(q, k, v, grid, pool, o_loc, mode="gated", w_global=wg, w_local=wl,
                                             return_lse=True)
    out1 = V.global_pooled_attn_merge_fwd(q, k, v, grid, pool, o_loc, mode="gated", w_global=wg)
    inplace = o_loc.clone()
    V.global_pooled_attn_merge_fwd(q, k, v, grid, pool, inplace, mode="gated", w_global=wg, w_local=wl, out=inplace)
    torch.cuda.synchronize()
    assert torch.equal(inplace, out)
    for b in range(B):
        for h in range(heads):
            Qh, _, _, kpr, vpr = _branch_refs(q, k, v, b, h, grid, pool, D)
            go, gl = R.global_ref(Qh, kpr, vpr, scale=D ** -0.5)
            ol = R.to_f64(o_loc[b, h])
            ref = R.merge_ref(ol[None], go[None], wl[h:h + 1].cpu(), wg[h:h + 1].cpu())[0]
            ref1 = R.merge_ref(ol[None], go[None], None, wg[h:h + 1].cpu())[0]
            compare(out[b, h].cpu(), ref, dt, f"{name} fused gated b{b} h{h}")
            compare(out1[b, h].cpu(), ref1, dt, f"{name} fused gated w_local=1 b{b} h{h}")
            compare(lg[b, h].cpu(), gl, dt, f"{name} fused gated global lse b{b} h{h}")


@pytest.mark.parametrize("case", MERGE_CASES, ids=[c[0] for c in MERGE_CASES])
def test_fused_lse_merge_is_union_attention(case):
    name, B, grid, tile, window, shift, pool, heads, D, dt = case
    say(f"[fused lse] {name}")
    N = int(np.prod(grid))
    q, k, v = qkv((B, heads, N, D), TDT[dt], seed=720)
    o_loc, l_loc = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, return_lse=True)
    out, lo = V.global_pooled_attn_merge_fwd(q, k, v, grid, pool, o_loc, mode="lse", lse_local=l_loc,
                                             return_lse=True)
    # the unfused path: global branch, then the standalone LSE merge
    og, lg = V.global_pooled_attn_fwd(q, k, v, grid, pool, return_lse=True)
    um, ul = V.dual_branch_merge_lse(o_loc, l_loc, og, lg, return_lse=True)
    ip_o, ip_l = o_loc.clone(), l_loc.clone()
    V.global_pooled_attn_merge_fwd(q, k, v, grid, pool, ip_o, mode="lse", lse_local=ip_l, out=ip_o, lse_out=ip_l)
    torch.cuda.synchronize()
    assert torch.equal(ip_o, out) and torch.equal(ip_l, lo)
    for b in range(B):
        for h in range(heads):
            Qh, Kh, Vh, kpr, vpr = _branch_refs(q, k, v, b, h, grid, pool, D)
            ou, lu = R.union_attention_ref(Qh, Kh, Vh, grid, tile, window, shift, kpr, vpr, scale=D ** -0.5)
            compare(out[b, h].cpu(), ou, dt, f"{name} fused lse b{b} h{h}")
            compare(lo[b, h].cpu(), lu, dt, f"{name} fused lse lse_out b{b} h{h}")
            compare(um[b, h].cpu(), ou, dt, f"{name} unfused lse b{b} h{h}")
            compare(ul[b, h].cpu(), lu, dt, f"{name} unfused lse lse_out b{b} h{h}")
