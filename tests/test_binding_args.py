"""The Python binding rejects every malformed tensor argument before it calls
the library: the C ABI derives all extents from the problem descriptor, so an
output buffer of the wrong shape or dtype, or a host tensor, must never reach
a kernel.  CPU only: the tensors here are host tensors, so a call that got
past the shape and dtype checks stops at the device check, which is what the
last case asserts."""
import pytest
import torch

import video_dit_sparse_amd as V

GRID, TILE, WIN = (2, 4, 6), (1, 2, 3), (1, 1, 1)
B, H, N, D = 1, 2, 48, 64


def qkv(dtype=torch.bfloat16):
    return [torch.zeros(B, H, N, D, dtype=dtype) for _ in range(3)]


def f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def test_sta_out_and_lse_checked():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="out must have shape"):
        V.sta_attn_fwd(q, k, v, GRID, TILE, WIN, out=torch.zeros(B, H, N - 1, D, dtype=q.dtype))
    with pytest.raises(ValueError, match="out must be"):
        V.sta_attn_fwd(q, k, v, GRID, TILE, WIN, out=torch.zeros(B, H, N, D, dtype=torch.float32))
    with pytest.raises(ValueError, match="lse must be torch.float32"):
        V.sta_attn_fwd(q, k, v, GRID, TILE, WIN, lse=torch.zeros(B, H, N, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse must have shape"):
        V.sta_attn_fwd(q, k, v, GRID, TILE, WIN, lse=f32(B, H, N + 1))
    with pytest.raises(ValueError, match="lse must be contiguous"):
        V.sta_attn_fwd(q, k, v, GRID, TILE, WIN, lse=f32(B, N, H).transpose(1, 2))
    with pytest.raises(ValueError, match="share shape and dtype"):
        V.sta_attn_fwd(q, k[:, :1], v, GRID, TILE, WIN)
    with pytest.raises(TypeError):
        V.sta_attn_fwd(q, object(), v, GRID, TILE, WIN)


def test_global_and_fused_merge_checked():
    q, k, v = qkv()
    pool = (2, 3)
    with pytest.raises(ValueError, match="workspace must be contiguous"):
        V.global_pooled_attn_fwd(q, k, v, GRID, pool, workspace=torch.zeros(64, 64, dtype=torch.uint8).t())
    with pytest.raises(ValueError, match="out must have shape"):
        V.global_pooled_attn_fwd(q, k, v, GRID, pool, out=torch.zeros(B, H, 8, D, dtype=q.dtype))
    o_local = torch.zeros_like(q)
    with pytest.raises(ValueError, match="w_global must have shape"):
        V.global_pooled_attn_merge_fwd(q, k, v, GRID, pool, o_local, w_global=f32(H + 1))
    with pytest.raises(ValueError, match="w_local must be torch.float32"):
        V.global_pooled_attn_merge_fwd(q, k, v, GRID, pool, o_local, w_global=f32(H),
                                       w_local=torch.zeros(H, dtype=torch.float64))
    with pytest.raises(ValueError, match="lse_local must have shape"):
        V.global_pooled_attn_merge_fwd(q, k, v, GRID, pool, o_local, mode="lse", lse_local=f32(B, H, N - 2))
    with pytest.raises(ValueError, match="mode must be one of"):
        V.global_pooled_attn_merge_fwd(q, k, v, GRID, pool, o_local, mode="sum")


def test_merges_checked():
    a, g, _ = qkv()
    with pytest.raises(ValueError, match="w_global must have shape"):
        V.dual_branch_merge(a, g, f32(3 * H))
    with pytest.raises(ValueError, match="w_global is required"):
        V.dual_branch_merge(a, g, None)
    with pytest.raises(ValueError, match="out must have shape"):
        V.dual_branch_merge(a, g, f32(H), out=torch.zeros(B, H, N, D // 2, dtype=a.dtype))
    with pytest.raises(ValueError, match="lse_global must be torch.float32"):
        V.dual_branch_merge_lse(a, f32(B, H, N), g, torch.zeros(B, H, N, dtype=torch.float16))
    with pytest.raises(ValueError, match="lse_out must have shape"):
        V.dual_branch_merge_lse(a, f32(B, H, N), g, f32(B, H, N), lse_out=f32(B, H))


def test_pool_and_variants_checked():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="out must have shape"):
        # pooled out sized for 2 x 2 cells passed to a 2 x 3 pooling
        V.kv_avgpool_fwd(k, GRID, (2, 3), out=torch.zeros(B, H, 2 * 2 * 3, D, dtype=k.dtype))
    with pytest.raises(ValueError, match="out must be"):
        V.kv_avgpool_fwd(k, GRID, (2, 3), out=torch.zeros(B, H, 2 * 2 * 2, D, dtype=torch.float32))
    with pytest.raises(ValueError, match="lse must have shape"):
        V.hier_pooled_attn_fwd(q, k, v, GRID, TILE, WIN, (2, 2), lse=f32(B, H, 3))
    with pytest.raises(ValueError, match="out must have shape"):
        V.compressed_global_attn_fwd(q, k, v, GRID, (2, 2), out=torch.zeros(1, dtype=q.dtype))


def test_backward_checked():
    q, k, v = qkv()
    o, do = torch.zeros_like(q), torch.zeros_like(q)
    lse = f32(B, H, N)
    with pytest.raises(ValueError, match="lse must have shape"):
        V.sta_attn_bwd(q, k, v, o, do, f32(B, H), GRID, TILE, WIN)
    with pytest.raises(ValueError, match="dq must be"):
        V.sta_attn_bwd(q, k, v, o, do, lse, GRID, TILE, WIN, dq=torch.zeros(B, H, N, D, dtype=torch.float32))
    with pytest.raises(ValueError, match="dv must have shape"):
        V.global_pooled_attn_bwd(q, k, v, o, do, lse, GRID, (2, 2), dv=torch.zeros(B, H, N, D + 8, dtype=q.dtype))
    with pytest.raises(ValueError, match="share shape and dtype"):
        V.sta_attn_bwd(q, k, v, o, do.float(), lse, GRID, TILE, WIN)


def test_host_tensors_rejected_before_any_call():
    # well-formed in every respect but host memory: refused by the device check
    q, k, v = qkv()
    lse = f32(B, H, N)
    calls = [
        lambda: V.sta_attn_fwd(q, k, v, GRID, TILE, WIN),
        lambda: V.global_pooled_attn_fwd(q, k, v, GRID, (2, 2)),
        lambda: V.dual_branch_merge(q, k, f32(H)),
        lambda: V.dual_branch_merge_lse(q, lse, k, lse),
        lambda: V.global_pooled_attn_merge_fwd(q, k, v, GRID, (2, 2), torch.zeros_like(q), w_global=f32(H)),
        lambda: V.hier_pooled_attn_fwd(q, k, v, GRID, TILE, WIN, (2, 2)),
        lambda: V.compressed_global_attn_fwd(q, k, v, GRID, (2, 2)),
        lambda: V.sta_attn_bwd(q, k, v, torch.zeros_like(q), torch.zeros_like(q), lse, GRID, TILE, WIN),
        lambda: V.global_pooled_attn_bwd(q, k, v, torch.zeros_like(q), torch.zeros_like(q), lse, GRID, (2, 2)),
        lambda: V.kv_avgpool_fwd(k, GRID, (2, 2)),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="GPU device"):
            call()
