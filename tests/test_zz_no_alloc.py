"""The global branch's entry point that allocates nothing
(global_pooled_attn_fwd_noalloc: pooled K/V in the library's static device
scratch) against the one that takes a workspace (global_pooled_attn_fwd),
called through the C ABI.  Two calls in a row, the second on a smaller
input, so the second runs on scratch the first left full."""
import ctypes

import numpy as np
import pytest
import torch

import video_dit_sparse_amd as V
from video_dit_sparse_amd import _lib as L
from video_dit_sparse_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def noalloc(q, k, v, grid, pool, o, lse, scale):
    prob = L._problem_for(q, grid, scale)
    st = [L._strides(t) for t in (q, k, v, o)]
    return L.lib().global_pooled_attn_fwd_noalloc(
        ctypes.byref(prob), L._pool(pool), q.data_ptr(), ctypes.byref(st[0]), k.data_ptr(), ctypes.byref(st[1]),
        v.data_ptr(), ctypes.byref(st[2]), o.data_ptr(), ctypes.byref(st[3]), lse.data_ptr(),
        torch.cuda.current_stream().cuda_stream)


def check_case(q, k, v, grid, pool, scale, name):
    o_ref, lse_ref = V.global_pooled_attn_fwd(q, k, v, grid, pool, scale=scale, return_lse=True)
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    assert noalloc(q, k, v, grid, pool, o, lse, scale) == 0, L.lib().vdsa_last_error().decode()
    torch.cuda.synchronize()
    # the bar of the bf16 path (max 2e-2, mean 2e-3), and in fact bit-identical:
    # the same kernels on the same pooled values
    err = (o.float() - o_ref.float()).abs()
    say(f"[noalloc] {name}: max |diff| {err.max().item():.3e}")
    assert err.max().item() <= 2e-2 and err.mean().item() <= 2e-3
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_noalloc_matches_workspace_call_twice():
    # first: the 1080P latent with 4 x 4 pooling (pooled K + V = 131.6 MB of
    # the 134.2 MB scratch); second: a small ragged grid with 4 x 3 cells
    w = WL.WORKLOADS["dual_1080p"]
    q, k, v = WL.make_qkv(w, DEV)
    say("[noalloc] call 1: 1080P latent, pool 4x4")
    check_case(q, k, v, w.grid, w.pool_hw, w.softmax_scale, "1080P")
    del q, k, v
    grid, pool = (5, 13, 22), (4, 3)
    q, k, v = (WL.make_tensor((1, 3, 5 * 13 * 22, 128), torch.bfloat16, DEV, seed=s) for s in (11, 12, 13))
    say("[noalloc] call 2: grid 5x13x22, pool 4x3, 3 heads")
    check_case(q, k, v, grid, pool, None, "small ragged")


def test_noalloc_python_binding_and_oversize():
    grid, pool = (3, 9, 10), (4, 3)
    q, k, v = (WL.make_tensor((2, 2, 270, 128), torch.bfloat16, DEV, seed=s) for s in (21, 22, 23))
    out = torch.empty_like(q)
    V.global_pooled_attn_fwd_noalloc(q, k, v, grid, pool, out)
    ref = V.global_pooled_attn_fwd(q, k, v, grid, pool)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    # pooled K + V beyond the scratch: refused before anything is launched
    big = torch.empty((1, 24, 21 * 136 * 240, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(L.VdsaError, match="VDSA_ERR_WORKSPACE"):
        V.global_pooled_attn_fwd_noalloc(big, big, big, (21, 136, 240), (4, 4), torch.empty_like(big))
    del big
    assert np.isfinite(out.float().cpu().numpy()).all()
