"""GPU parity of UltraGen's hierarchical windows over pooled keys
(``hier_pooled_attn_fwd``) and its compressed global attention with bilinear
upsampling (``compressed_global_attn_fwd``), through the C ABI against the
CPU fp64 oracle, on every output element (bf16: max 2e-2, mean 2e-3;
fp32: 1e-4)."""
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


def qkv(shape, dtype, seed, layout="bhnd"):
    return [WL.make_tensor(shape, dtype, DEV, seed=seed + i) for i in range(3)]


HIER = [
    # name, batch, grid, tile, window, shift, pool, heads, head_dim, dtype
    ("aligned_bf16", 1, (3, 8, 16), (1, 4, 4), (1, 3, 3), (0, 0, 0), (2, 2), 2, 128, "bf16"),
    ("shift_bf16", 2, (2, 10, 12), (2, 4, 4), (1, 3, 1), (0, 2, 2), (2, 2), 1, 128, "bf16"),
    ("unaligned_bf16", 1, (2, 9, 11), (1, 3, 4), (1, 3, 3), (0, 1, 1), (2, 2), 1, 128, "bf16"),
    ("tile384_bf16", 1, (6, 16, 16), (6, 8, 8), (1, 3, 1), (0, 0, 0), (2, 2), 1, 128, "bf16"),
    ("pool4x2_f32_d64", 1, (2, 8, 8), (1, 4, 4), (1, 1, 3), (0, 0, 0), (4, 2), 2, 64, "f32"),
]


@pytest.mark.parametrize("case", HIER, ids=[c[0] for c in HIER])
def test_hier_pooled_small_all_rows(case):
    name, B, grid, tile, window, shift, pool, heads, D, dt = case
    say(f"[hier] {name}")
    N = int(np.prod(grid))
    q, k, v = qkv((B, heads, N, D), TDT[dt], seed=900)
    o, lse = V.hier_pooled_attn_fwd(q, k, v, grid, tile, window, pool, shift, return_lse=True)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(heads):
            ro, rl = R.hier_pooled_ref(head_f64(q, b, h), head_f64(k, b, h), head_f64(v, b, h), grid, tile, window,
                                       shift, pool, scale=D ** -0.5)
            compare(o[b, h].cpu(), ro, dt, f"{name} b{b} h{h}")
            compare(lse[b, h].cpu(), rl, dt, f"{name} lse b{b} h{h}")


def test_hier_pooled_bnhd_strides():
    grid, tile, window, pool = (2, 8, 12), (1, 4, 4), (1, 3, 3), (2, 2)
    N = int(np.prod(grid))
    q, k, v = (WL.make_tensor((1, N, 2, 128), torch.bfloat16, DEV, seed=910 + i).transpose(1, 2) for i in range(3))
    o = V.hier_pooled_attn_fwd(q, k, v, grid, tile, window, pool)
    o2 = V.hier_pooled_attn_fwd(q.contiguous(), k.contiguous(), v.contiguous(), grid, tile, window, pool)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    # the BNHD call against the oracle, head by head
    for h in range(2):
        ro, _ = R.hier_pooled_ref(head_f64(q, 0, h), head_f64(k, 0, h), head_f64(v, 0, h), grid, tile, window,
                                  (0, 0, 0), pool, scale=128 ** -0.5)
        compare(o[0, h].cpu(), ro, "bf16", f"hier BNHD h{h}")


COMP = [
    # name, batch, grid, pool, heads, head_dim, dtype
    ("pool4_bf16", 1, (3, 8, 12), (4, 4), 2, 128, "bf16"),
    ("ragged_bf16", 2, (2, 9, 10), (4, 3), 1, 128, "bf16"),
    ("pooled384_bf16", 1, (4, 32, 48), (4, 4), 1, 128, "bf16"),
    ("pool2_f32_d64", 1, (2, 6, 8), (2, 2), 2, 64, "f32"),
]


@pytest.mark.parametrize("case", COMP, ids=[c[0] for c in COMP])
def test_compressed_global_small_all_rows(case):
    name, B, grid, pool, heads, D, dt = case
    say(f"[compressed global] {name}")
    N = int(np.prod(grid))
    q, k, v = qkv((B, heads, N, D), TDT[dt], seed=920)
    o = V.compressed_global_attn_fwd(q, k, v, grid, pool)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(heads):
            ro = R.compressed_global_ref(head_f64(q, b, h), head_f64(k, b, h), head_f64(v, b, h), grid, pool,
                                         scale=D ** -0.5)
            compare(o[b, h].cpu(), ro, dt, f"{name} b{b} h{h}")
