"""The library's calls under HIP graph capture: no call allocates, frees or
records a memset, so a captured step replays the same kernels on the same
buffers.  Each graph is replayed several times with eager work and
synchronisations between the replays, and every replay is checked bit for
bit against the eager result."""
import sys

import numpy as np
import pytest
import torch

import video_dit_sparse_amd as V
from video_dit_sparse_amd import _lib as L
from video_dit_sparse_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    V.lib()  # fail loudly if the library is missing


def test_forward_step_graph():
    """Local branch, then the global branch with the gated merge fused."""
    grid, tile, window, pool = (4, 24, 32), (2, 8, 8), (1, 3, 3), (4, 4)
    B, heads, D = 1, 2, 128
    N = int(np.prod(grid))
    q, k, v = (WL.make_tensor((B, heads, N, D), torch.bfloat16, DEV, seed=980 + i) for i in range(3))
    gate = torch.rand(heads, device=DEV)
    loc = torch.empty_like(q)
    lse = torch.empty((B, heads, N), dtype=torch.float32, device=DEV)
    merged = torch.empty_like(q)
    ws = torch.empty(L.global_pooled_attn_workspace_size(B, heads, D, grid, pool), dtype=torch.uint8, device=DEV)

    def step():
        V.sta_attn_fwd(q, k, v, grid, tile, window, out=loc, lse=lse)
        V.global_pooled_attn_merge_fwd(q, k, v, grid, pool, loc, mode="gated", w_global=gate, out=merged,
                                       workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_loc, ref_lse, ref_merged = loc.clone(), lse.clone(), merged.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        say(f"[graph fwd] replay {r}")
        for t in (loc, lse, merged):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(loc, ref_loc) and torch.equal(lse, ref_lse) and torch.equal(merged, ref_merged), r
        step()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(merged, ref_merged)


def test_backward_graph():
    grid, tile, window, shift = (6, 16, 16), (6, 8, 8), (1, 1, 1), (0, 0, 0)
    B, heads, D = 1, 2, 128
    N = int(np.prod(grid))
    q, k, v, do = (WL.make_tensor((B, heads, N, D), torch.bfloat16, DEV, seed=990 + i) for i in range(4))
    o, lse = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, return_lse=True)
    grads = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(V.sta_attn_bwd_workspace_size(B, heads, D, grid), dtype=torch.uint8, device=DEV)

    def step():
        V.sta_attn_bwd(q, k, v, o, do, lse, grid, tile, window, shift, dq=grads[0], dk=grads[1], dv=grads[2],
                       workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [g.clone() for g in grads]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        say(f"[graph bwd] replay {r}")
        for g in grads:
            g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for g, rg in zip(grads, ref):
            assert torch.equal(g, rg), r
        step()
        torch.cuda.synchronize()
