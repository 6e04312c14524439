"""GPU parity at the largest head slice the in-head byte offsets allow.

One (batch, head) slice of Q, K, V, O and the gradients is addressed with
32-bit byte offsets from a 64-bit base: within a head, ((N-1) * stride_n + D)
elements of 2 bytes must stay below 2^32.  The 4K workload's latent
(21x136x240, 685,440 tokens) in token-major layout with 24 heads (token
stride 24 * 128 elements) reaches 4.21e9 bytes, so the last half of every
head's tokens sit beyond 2^31, at offsets that are negative as signed 32-bit
integers.  The forward is compared with the oracle on sampled rows that
include the last tokens, and forward and backward with the same calls on the
head-major layout (whose slices stay below 2^31 and are parity-checked
element by element at smaller sizes), bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as R
import video_dit_sparse_amd as V
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


def _bnhd(x):
    """The same values as a [B, heads, N, D] view of a [B, N, heads, D] buffer."""
    return x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


W4K = WL.WORKLOADS["local_global_4k"]


def _max_offset(x):
    """Largest byte offset of an element from the start of its head slice."""
    return ((x.shape[2] - 1) * x.stride(2) + (x.shape[3] - 1) * x.stride(3) + 1) * x.element_size()


@pytest.fixture(scope="module")
def qkv_4k():
    w = W4K
    say("[limits] 4K BNHD: generating inputs")
    q, k, v = WL.make_qkv(w, DEV)
    qs, ks, vs = (_bnhd(x) for x in (q, k, v))
    assert qs.stride(2) == w.heads * w.head_dim
    assert 2 ** 31 < _max_offset(qs) < 2 ** 32
    return q, k, v, qs, ks, vs


def test_4k_bnhd_forward_beyond_2_31(qkv_4k):
    w = W4K
    q, k, v, qs, ks, vs = qkv_4k
    say("[limits] 4K BNHD forward")
    o1, l1 = V.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, scale=w.softmax_scale, return_lse=True)
    o2, l2 = V.sta_attn_fwd(qs, ks, vs, w.grid, w.tile, w.window, scale=w.softmax_scale, return_lse=True,
                            out=_bnhd(torch.empty_like(q)))
    torch.cuda.synchronize()
    assert o2.stride(2) == w.heads * w.head_dim
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # sampled rows, the lattice's corner tiles (the last token among them) and
    # the last 32 tokens of the head, whose offsets are the largest
    rows = sample_rows(w.grid, w.tile, (0, 0, 0), n_random_tiles=2, rows_per_tile=8, seed=41)
    rows = np.unique(np.concatenate([rows, np.arange(w.n_tokens - 32, w.n_tokens)]))
    far = rows[rows * qs.stride(2) * 2 > 2 ** 31]
    assert len(far) >= 32
    h = w.heads - 1
    say(f"[limits] 4K BNHD forward: oracle on {len(rows)} rows of head {h} ({len(far)} beyond 2^31 bytes)")
    ro, rl = R.sta_ref(head_f64(q, 0, h), head_f64(k, 0, h), head_f64(v, 0, h), w.grid, w.tile, w.window,
                       (0, 0, 0), scale=w.softmax_scale, rows=rows)
    compare(o2[0, h, rows].cpu(), ro, "bf16", f"4K BNHD head {h}")
    compare(l2[0, h, rows].cpu(), rl, "bf16", f"4K BNHD lse head {h}")


def test_4k_bnhd_backward_beyond_2_31(qkv_4k):
    w = W4K
    q, k, v, qs, ks, vs = qkv_4k
    do = WL.make_tensor(q.shape, torch.bfloat16, DEV, seed=991)
    dos = _bnhd(do)
    say("[limits] 4K BNHD backward")
    o, lse = V.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, scale=w.softmax_scale, return_lse=True)
    g1 = V.sta_attn_bwd(q, k, v, o, do, lse, w.grid, w.tile, w.window, scale=w.softmax_scale)
    os_ = _bnhd(o)
    g2 = V.sta_attn_bwd(qs, ks, vs, os_, dos, lse, w.grid, w.tile, w.window, scale=w.softmax_scale,
                        dq=_bnhd(torch.empty_like(q)), dk=_bnhd(torch.empty_like(q)), dv=_bnhd(torch.empty_like(q)))
    torch.cuda.synchronize()
    for nm, a, b in zip(("dq", "dk", "dv"), g1, g2):
        assert b.stride(2) == w.heads * w.head_dim
        assert 2 ** 31 < _max_offset(b) < 2 ** 32
        assert torch.equal(a, b), f"4K BNHD {nm}"
        assert torch.isfinite(a.float()).all()
