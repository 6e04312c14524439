"""The hot path of one workload as a sequence of library calls.

Local branch: one ``sta_attn_fwd`` per lattice shift (two for the
cross-window pair: the plain tile lattice, then the half-tile-shifted one, as
in UltraGen's alternating window partitions, summary section 4.3).  Global
branch, where the workload has one: attention over K/V pooled k_h x k_w and
the gated merge with the per-head gate (w_local = 1), either as one call with
the merge fused into the attention epilogue (``global_pooled_attn_merge_fwd``,
the default) or as ``global_pooled_attn_fwd`` then ``dual_branch_merge``.
Every step runs in libvdsa.so's kernels on the current torch stream.
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import _lib as L
from .workloads import Workload


class Buffers:
    """Outputs and workspace of one workload, allocated once and reused."""

    def __init__(self, w: Workload, q: torch.Tensor):
        self.local = [torch.empty_like(q, memory_format=torch.contiguous_format) for _ in w.shifts]
        self.lse = [torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) for _ in w.shifts]
        self.glob = self.glob_lse = self.merged = self.workspace = None
        if w.pool_hw is not None:
            self.glob = torch.empty_like(q, memory_format=torch.contiguous_format)
            self.glob_lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
            self.merged = torch.empty_like(q, memory_format=torch.contiguous_format)
            nbytes = L.global_pooled_attn_workspace_size(w.batch, w.heads, w.head_dim, w.grid, w.pool_hw,
                                                         L.VDSA_BF16 if w.dtype == "bf16" else L.VDSA_F32)
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)


def run(w: Workload, q, k, v, gate: Optional[torch.Tensor], buf: Buffers, with_lse: bool = False,
        fused: bool = True) -> Dict:
    """One pass of the workload's hot path; returns the output tensors.  With
    ``fused`` the global branch's own output is never materialised
    (``glob`` is None; ``glob_lse`` still holds its LSE when requested)."""
    for i, shift in enumerate(w.shifts):
        L.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, shift, scale=w.softmax_scale,
                       out=buf.local[i], lse=buf.lse[i] if with_lse else None)
    out = {"local": buf.local, "lse": buf.lse if with_lse else None}
    if w.pool_hw is not None:
        out.update(run_global(w, q, k, v, gate, buf, with_lse, fused))
    return out


def run_global(w: Workload, q, k, v, gate, buf: Buffers, with_lse: bool = False, fused: bool = True) -> Dict:
    """The global branch and the merge with the local output in ``buf.local[0]``."""
    glse = buf.glob_lse if with_lse else None
    if fused:
        L.global_pooled_attn_merge_fwd(q, k, v, w.grid, w.pool_hw, buf.local[0], mode="gated", w_global=gate,
                                       scale=w.softmax_scale, out=buf.merged, lse_out=glse,
                                       workspace=buf.workspace)
    else:
        L.global_pooled_attn_fwd(q, k, v, w.grid, w.pool_hw, scale=w.softmax_scale, out=buf.glob, lse=glse,
                                 workspace=buf.workspace)
        L.dual_branch_merge(buf.local[0], buf.glob, gate, out=buf.merged)
    return {"glob": None if fused else buf.glob, "glob_lse": glse, "merged": buf.merged, "workspace": buf.workspace}


def flops(w: Workload) -> Dict[str, float]:
    """Effective FLOP per step, per branch."""
    f = {"local": sum(L.sta_flops(w.batch, w.heads, w.head_dim, w.grid, w.tile, w.window, s) for s in w.shifts)}
    if w.pool_hw is not None:
        f["global"] = L.global_flops(w.batch, w.heads, w.head_dim, w.grid, w.pool_hw)
    return f
