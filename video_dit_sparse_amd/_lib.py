"""ctypes binding of libvdsa.so (include/vdsa.h).

Argument marshalling only: torch tensors become device pointers and element
strides, torch's current stream becomes the HIP stream, and every step of the
computation runs in the library's kernels.  Torch supplies device memory for
outputs and workspaces.  If the library is missing this module raises; there
is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvdsa.so")

VDSA_F32, VDSA_BF16 = 0, 1
STATUS_NAMES = {
    0: "VDSA_OK", 1: "VDSA_ERR_NULL", 2: "VDSA_ERR_SHAPE", 3: "VDSA_ERR_WINDOW",
    4: "VDSA_ERR_UNSUPPORTED", 5: "VDSA_ERR_ALIGN", 6: "VDSA_ERR_ALIAS",
    7: "VDSA_ERR_WORKSPACE", 8: "VDSA_ERR_HIP",
}
STATUS = {v: k for k, v in STATUS_NAMES.items()}

# every symbol include/vdsa.h declares
EXPORTED = [
    "sta_attn_fwd", "global_pooled_attn_workspace_size", "global_pooled_attn_fwd",
    "global_pooled_attn_fwd_noalloc", "dual_branch_merge", "dual_branch_merge_lse", "global_pooled_attn_merge_fwd",
    "hier_pooled_attn_workspace_size", "hier_pooled_attn_fwd", "compressed_global_attn_workspace_size",
    "compressed_global_attn_fwd",
    "sta_attn_bwd_workspace_size", "sta_attn_bwd", "global_pooled_attn_bwd_workspace_size",
    "global_pooled_attn_bwd",
    "kv_avgpool_fwd", "vdsa_sta_flops", "vdsa_global_flops", "vdsa_hier_flops", "vdsa_compressed_global_flops",
    "vdsa_status_string", "vdsa_last_error", "vdsa_abi_version", "vdsa_sta_kernel",
]
VDSA_MERGE_GATED, VDSA_MERGE_LSE = 0, 1
MERGE_MODES = {"gated": VDSA_MERGE_GATED, "lse": VDSA_MERGE_LSE}


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("grid_t", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("dtype", ctypes.c_int), ("scale", ctypes.c_float)]


class StaCfg(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int32 * 3), ("window", ctypes.c_int32 * 3), ("shift", ctypes.c_int32 * 3),
                ("window_mode", ctypes.c_int32)]


# vdsa_window_mode: how windows meet the grid edge
WINDOW_MODES = {"clip": 0, "inward": 1, "cyclic": 2}


class Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64)]


class VdsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libvdsa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m video_dit_sparse_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, C, S = ctypes.POINTER(Problem), ctypes.POINTER(StaCfg), ctypes.POINTER(Strides)
    vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
    fp = ctypes.c_void_p  # float* passed as an address
    L.sta_attn_fwd.argtypes = [P, C, vp, S, vp, S, vp, S, vp, S, fp, vp]
    L.global_pooled_attn_workspace_size.argtypes = [P, i32p, ctypes.POINTER(ctypes.c_size_t)]
    L.global_pooled_attn_fwd.argtypes = [P, i32p, vp, S, vp, S, vp, S, vp, S, fp, vp, ctypes.c_size_t, vp]
    L.global_pooled_attn_fwd_noalloc.argtypes = [P, i32p, vp, S, vp, S, vp, S, vp, S, fp, vp]
    L.dual_branch_merge.argtypes = [P, vp, S, vp, S, fp, fp, vp, S, vp]
    L.dual_branch_merge_lse.argtypes = [P, vp, S, fp, vp, S, fp, vp, S, fp, vp]
    L.global_pooled_attn_merge_fwd.argtypes = [P, i32p, vp, S, vp, S, vp, S, ctypes.c_int, vp, S, fp, fp, fp,
                                               vp, S, fp, vp, ctypes.c_size_t, vp]
    L.kv_avgpool_fwd.argtypes = [P, i32p, vp, S, vp, S, vp]
    L.hier_pooled_attn_workspace_size.argtypes = [P, i32p, ctypes.POINTER(ctypes.c_size_t)]
    L.hier_pooled_attn_fwd.argtypes = [P, C, i32p, vp, S, vp, S, vp, S, vp, S, fp, vp, ctypes.c_size_t, vp]
    L.compressed_global_attn_workspace_size.argtypes = [P, i32p, ctypes.POINTER(ctypes.c_size_t)]
    L.compressed_global_attn_fwd.argtypes = [P, i32p, vp, S, vp, S, vp, S, vp, S, vp, ctypes.c_size_t, vp]
    L.sta_attn_bwd_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    L.sta_attn_bwd.argtypes = [P, C, vp, S, vp, S, vp, S, vp, S, vp, S, fp, vp, S, vp, S, vp, S,
                               vp, ctypes.c_size_t, vp]
    L.global_pooled_attn_bwd_workspace_size.argtypes = [P, i32p, ctypes.POINTER(ctypes.c_size_t)]
    L.global_pooled_attn_bwd.argtypes = [P, i32p, vp, S, vp, S, vp, S, vp, S, vp, S, fp, vp, S, vp, S, vp, S,
                                         vp, ctypes.c_size_t, vp]
    L.vdsa_sta_flops.argtypes = [P, C, ctypes.POINTER(ctypes.c_double)]
    L.vdsa_global_flops.argtypes = [P, i32p, ctypes.POINTER(ctypes.c_double)]
    L.vdsa_hier_flops.argtypes = [P, C, i32p, ctypes.POINTER(ctypes.c_double)]
    L.vdsa_compressed_global_flops.argtypes = [P, i32p, ctypes.POINTER(ctypes.c_double)]
    L.vdsa_status_string.argtypes = [ctypes.c_int]
    L.vdsa_status_string.restype = ctypes.c_char_p
    L.vdsa_last_error.argtypes = []
    L.vdsa_last_error.restype = ctypes.c_char_p
    L.vdsa_abi_version.argtypes = []
    L.vdsa_sta_kernel.argtypes = [P, C]
    L.vdsa_sta_kernel.restype = ctypes.c_char_p
    for name in ("sta_attn_fwd", "global_pooled_attn_workspace_size", "global_pooled_attn_fwd",
                 "dual_branch_merge", "kv_avgpool_fwd", "vdsa_sta_flops", "vdsa_global_flops",
                 "vdsa_abi_version"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def check(status: int) -> None:
    if status != 0:
        raise VdsaError(status, lib().vdsa_last_error().decode())


# ---------------------------------------------------------------- descriptors
def make_problem(batch, heads, head_dim, grid, dtype: int, scale: float) -> Problem:
    return Problem(int(batch), int(heads), int(head_dim), int(grid[0]), int(grid[1]), int(grid[2]),
                   int(dtype), float(scale))


def make_cfg(tile, window, shift=(0, 0, 0), window_mode: str = "clip") -> StaCfg:
    if window_mode not in WINDOW_MODES:
        raise ValueError(f"window_mode must be one of {tuple(WINDOW_MODES)}, got {window_mode!r}")
    c = StaCfg()
    for i in range(3):
        c.tile[i], c.window[i], c.shift[i] = int(tile[i]), int(window[i]), int(shift[i])
    c.window_mode = WINDOW_MODES[window_mode]
    return c


def _pool(pool_hw) -> ctypes.Array:
    return (ctypes.c_int32 * 2)(int(pool_hw[0]), int(pool_hw[1]))


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return VDSA_BF16
    if t.dtype == torch.float32:
        return VDSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _strides(t) -> Strides:
    if t.dim() != 4:
        raise ValueError(f"expected a [batch, heads, N, head_dim] tensor, got shape {tuple(t.shape)}")
    if t.stride(3) != 1:
        raise ValueError("head_dim must be the contiguous dimension")
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return int(stream) if not hasattr(stream, "cuda_stream") else stream.cuda_stream


def _problem_for(q, grid, scale) -> Problem:
    B, Hh, N, D = q.shape
    T, H, W = grid
    if T * H * W != N:
        raise ValueError(f"grid {tuple(grid)} has {T * H * W} tokens but tensors have N = {N}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return make_problem(B, Hh, D, grid, _dtype_code(q), scale)


def _same(q, *others):
    """q and every tensor in ``others``: equal shape and dtype (devices are
    checked by ``_on_device`` once every shape is known to be right)."""
    torch = _torch()
    for t in (q,) + others:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"expected a torch tensor, got {type(t).__name__}")
    for t in others:
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v (and outputs) must share shape and dtype: "
                             f"{tuple(q.shape)} {q.dtype} against {tuple(t.shape)} {t.dtype}")


def _arg(t, name, shape, dtype, contiguous=False):
    """A caller-supplied tensor argument: exactly ``shape`` and ``dtype``
    (and contiguous if asked).  The C ABI derives every extent from the
    problem descriptor, so a smaller or mistyped buffer would be written past
    its end; this check runs before any library call.  Returns ``t``."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _workspace_arg(t):
    """A caller's workspace: a contiguous tensor (its byte size is checked by
    the library against the size the call needs).  ``None`` passes."""
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"workspace must be a torch tensor, got {type(t).__name__}")
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return t


def _on_device(q, *tensors):
    """Every tensor is GPU memory on q's device (a host pointer handed to a
    kernel would fault the GPU).  ``None`` entries are skipped."""
    if not q.is_cuda:
        raise ValueError(f"tensors must be on a GPU device, got {q.device}")
    for t in tensors:
        if t is not None and t.device != q.device:
            raise ValueError(f"every tensor must be on {q.device}, got one on {t.device}")


# ---------------------------------------------------------------- entry points
def _out_like(q, out, name="out"):
    torch = _torch()
    if out is None:
        return torch.empty_like(q, memory_format=torch.contiguous_format)
    return _arg(out, name, q.shape, q.dtype)


def _lse_buf(q, lse, want, name="lse"):
    """LSE output: fp32 [B, heads, N] contiguous; allocated if wanted and not given."""
    torch = _torch()
    shape = tuple(q.shape[:3])
    if lse is not None:
        return _arg(lse, name, shape, torch.float32, contiguous=True)
    return torch.empty(shape, dtype=torch.float32, device=q.device) if want else None


def _lse_in(q, t, name):
    return _arg(t, name, tuple(q.shape[:3]), _torch().float32, contiguous=True)


def _gate(w, heads, name):
    return None if w is None else _arg(w, name, (heads,), _torch().float32, contiguous=True)


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _workspace(q, workspace, need):
    torch = _torch()
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=q.device)
    return workspace


def _nbytes(t):
    return t.numel() * t.element_size()


def sta_attn_fwd(q, k, v, grid: Sequence[int], tile: Sequence[int], window: Sequence[int],
                 shift: Sequence[int] = (0, 0, 0), scale: Optional[float] = None, out=None,
                 lse=None, return_lse: bool = False, stream=None, window_mode: str = "clip"):
    """Sliding-tile attention (see ``sta_attn_fwd`` in include/vdsa.h).

    q, k, v: [B, heads, N, D] device tensors (bf16 or fp32), N = T*H*W.
    window_mode: "clip" (default), "inward" or "cyclic" (vdsa_window_mode).
    Returns O (and LSE [B, heads, N] fp32 if requested).
    """
    _same(q, k, v)
    prob = _problem_for(q, grid, scale)
    cfg = make_cfg(tile, window, shift, window_mode)
    o = _out_like(q, out)
    lse = _lse_buf(q, lse, return_lse)
    _on_device(q, k, v, o, lse)
    check(lib().sta_attn_fwd(ctypes.byref(prob), ctypes.byref(cfg),
                             q.data_ptr(), ctypes.byref(_strides(q)), k.data_ptr(), ctypes.byref(_strides(k)),
                             v.data_ptr(), ctypes.byref(_strides(v)), o.data_ptr(), ctypes.byref(_strides(o)),
                             _ptr(lse), _stream(stream)))
    return (o, lse) if (return_lse or lse is not None) else o


def global_pooled_attn_workspace_size(batch, heads, head_dim, grid, pool_hw, dtype_code=VDSA_BF16) -> int:
    prob = make_problem(batch, heads, head_dim, grid, dtype_code, 1.0)
    n = ctypes.c_size_t()
    check(lib().global_pooled_attn_workspace_size(ctypes.byref(prob), _pool(pool_hw), ctypes.byref(n)))
    return n.value


def global_pooled_attn_fwd(q, k, v, grid, pool_hw, scale=None, out=None, lse=None, return_lse=False,
                           workspace=None, stream=None):
    """Global branch: queries attend k_h x k_w average-pooled K/V
    (``global_pooled_attn_fwd`` in include/vdsa.h).  Returns O (and LSE)."""
    _same(q, k, v)
    prob = _problem_for(q, grid, scale)
    o = _out_like(q, out)
    lse = _lse_buf(q, lse, return_lse)
    _on_device(q, k, v, o, lse, _workspace_arg(workspace))
    need = ctypes.c_size_t()
    check(lib().global_pooled_attn_workspace_size(ctypes.byref(prob), _pool(pool_hw), ctypes.byref(need)))
    workspace = _workspace(q, workspace, need.value)
    check(lib().global_pooled_attn_fwd(
        ctypes.byref(prob), _pool(pool_hw), q.data_ptr(), ctypes.byref(_strides(q)),
        k.data_ptr(), ctypes.byref(_strides(k)), v.data_ptr(), ctypes.byref(_strides(v)),
        o.data_ptr(), ctypes.byref(_strides(o)), _ptr(lse),
        workspace.data_ptr(), _nbytes(workspace), _stream(stream)))
    return (o, lse) if (return_lse or lse is not None) else o


# bytes of the static device scratch behind global_pooled_attn_fwd_noalloc
STATIC_SCRATCH_BYTES = 128 << 20


def global_pooled_attn_fwd_noalloc(q, k, v, grid, pool_hw, out, lse=None, scale=None, stream=None):
    """The global branch with pooled K/V in the library's static device
    scratch (``global_pooled_attn_fwd_noalloc``): nothing is allocated, so
    ``out`` (and ``lse`` if wanted) must be given.  Calls that overlap in time
    on one GPU share that scratch and race.  Returns ``out``."""
    _same(q, k, v)
    prob = _problem_for(q, grid, scale)
    if out is None:
        raise ValueError("out is required: this entry point allocates nothing")
    o = _out_like(q, out)
    lse = _lse_buf(q, lse, False)
    _on_device(q, k, v, o, lse)
    check(lib().global_pooled_attn_fwd_noalloc(
        ctypes.byref(prob), _pool(pool_hw), q.data_ptr(), ctypes.byref(_strides(q)),
        k.data_ptr(), ctypes.byref(_strides(k)), v.data_ptr(), ctypes.byref(_strides(v)),
        o.data_ptr(), ctypes.byref(_strides(o)), _ptr(lse), _stream(stream)))
    return o


def dual_branch_merge(o_local, o_global, w_global, w_local=None, out=None, stream=None):
    """out = w_local[h] * o_local + w_global[h] * o_global (``dual_branch_merge``).

    ``out=o_local`` merges in place."""
    _same(o_local, o_global)
    B, Hh, N, D = o_local.shape
    prob = make_problem(B, Hh, D, (1, 1, N), _dtype_code(o_local), 1.0)
    o = _out_like(o_local, out)
    if w_global is None:
        raise ValueError("w_global is required")
    w_global, w_local = _gate(w_global, Hh, "w_global"), _gate(w_local, Hh, "w_local")
    _on_device(o_local, o_global, o, w_global, w_local)
    check(lib().dual_branch_merge(ctypes.byref(prob), o_local.data_ptr(), ctypes.byref(_strides(o_local)),
                                  o_global.data_ptr(), ctypes.byref(_strides(o_global)),
                                  _ptr(w_local), w_global.data_ptr(),
                                  o.data_ptr(), ctypes.byref(_strides(o)), _stream(stream)))
    return o


def dual_branch_merge_lse(o_local, lse_local, o_global, lse_global, out=None, lse_out=None,
                          return_lse=False, stream=None):
    """One softmax over the union of both branches' keys, from their LSEs
    (``dual_branch_merge_lse``).  ``out=o_local`` merges in place.  Returns O
    (and the merged LSE if requested)."""
    _same(o_local, o_global)
    B, Hh, N, D = o_local.shape
    prob = make_problem(B, Hh, D, (1, 1, N), _dtype_code(o_local), 1.0)
    o = _out_like(o_local, out)
    lse_local, lse_global = _lse_in(o_local, lse_local, "lse_local"), _lse_in(o_local, lse_global, "lse_global")
    lse_out = _lse_buf(o_local, lse_out, return_lse, "lse_out")
    _on_device(o_local, o_global, o, lse_local, lse_global, lse_out)
    check(lib().dual_branch_merge_lse(
        ctypes.byref(prob), o_local.data_ptr(), ctypes.byref(_strides(o_local)), lse_local.data_ptr(),
        o_global.data_ptr(), ctypes.byref(_strides(o_global)), lse_global.data_ptr(),
        o.data_ptr(), ctypes.byref(_strides(o)), _ptr(lse_out), _stream(stream)))
    return (o, lse_out) if (return_lse or lse_out is not None) else o


def global_pooled_attn_merge_fwd(q, k, v, grid, pool_hw, o_local, mode="gated", lse_local=None,
                                 w_global=None, w_local=None, scale=None, out=None, lse_out=None,
                                 return_lse=False, workspace=None, stream=None):
    """Global branch with the merge fused into its epilogue
    (``global_pooled_attn_merge_fwd``): ``mode`` "gated" (w_global, optional
    w_local) or "lse" (lse_local).  ``out=o_local`` merges in place.  Returns
    the merged O (and lse_out if requested)."""
    if mode not in MERGE_MODES:
        raise ValueError(f"mode must be one of {tuple(MERGE_MODES)}, got {mode!r}")
    _same(q, k, v, o_local)
    B, Hh, N, D = q.shape
    prob = _problem_for(q, grid, scale)
    o = _out_like(q, out)
    lse_out = _lse_buf(q, lse_out, return_lse, "lse_out")
    lse_local = _lse_in(q, lse_local, "lse_local") if lse_local is not None else None
    w_global, w_local = _gate(w_global, Hh, "w_global"), _gate(w_local, Hh, "w_local")
    _on_device(q, k, v, o_local, o, lse_out, lse_local, w_global, w_local, _workspace_arg(workspace))
    need = ctypes.c_size_t()
    check(lib().global_pooled_attn_workspace_size(ctypes.byref(prob), _pool(pool_hw), ctypes.byref(need)))
    workspace = _workspace(q, workspace, need.value)
    check(lib().global_pooled_attn_merge_fwd(
        ctypes.byref(prob), _pool(pool_hw), q.data_ptr(), ctypes.byref(_strides(q)),
        k.data_ptr(), ctypes.byref(_strides(k)), v.data_ptr(), ctypes.byref(_strides(v)),
        MERGE_MODES[mode], o_local.data_ptr(), ctypes.byref(_strides(o_local)),
        _ptr(lse_local), _ptr(w_local), _ptr(w_global),
        o.data_ptr(), ctypes.byref(_strides(o)), _ptr(lse_out),
        workspace.data_ptr(), _nbytes(workspace), _stream(stream)))
    return (o, lse_out) if (return_lse or lse_out is not None) else o


def hier_pooled_attn_fwd(q, k, v, grid, tile, window, pool_hw, shift=(0, 0, 0), scale=None, out=None, lse=None,
                         return_lse=False, workspace=None, stream=None):
    """Full-resolution queries against the pooled K/V of their sliding-tile
    window (``hier_pooled_attn_fwd``).  Returns O (and LSE)."""
    _same(q, k, v)
    prob = _problem_for(q, grid, scale)
    cfg = make_cfg(tile, window, shift)
    o = _out_like(q, out)
    lse = _lse_buf(q, lse, return_lse)
    _on_device(q, k, v, o, lse, _workspace_arg(workspace))
    need = ctypes.c_size_t()
    check(lib().hier_pooled_attn_workspace_size(ctypes.byref(prob), _pool(pool_hw), ctypes.byref(need)))
    workspace = _workspace(q, workspace, need.value)
    check(lib().hier_pooled_attn_fwd(
        ctypes.byref(prob), ctypes.byref(cfg), _pool(pool_hw), q.data_ptr(), ctypes.byref(_strides(q)),
        k.data_ptr(), ctypes.byref(_strides(k)), v.data_ptr(), ctypes.byref(_strides(v)),
        o.data_ptr(), ctypes.byref(_strides(o)), _ptr(lse),
        workspace.data_ptr(), _nbytes(workspace), _stream(stream)))
    return (o, lse) if (return_lse or lse is not None) else o


def compressed_global_attn_fwd(q, k, v, grid, pool_hw, scale=None, out=None, workspace=None, stream=None):
    """Pooled Q, K, V, full attention among pooled tokens, bilinear upsampling
    (``compressed_global_attn_fwd``).  Returns O."""
    _same(q, k, v)
    prob = _problem_for(q, grid, scale)
    o = _out_like(q, out)
    _on_device(q, k, v, o, _workspace_arg(workspace))
    need = ctypes.c_size_t()
    check(lib().compressed_global_attn_workspace_size(ctypes.byref(prob), _pool(pool_hw), ctypes.byref(need)))
    workspace = _workspace(q, workspace, need.value)
    check(lib().compressed_global_attn_fwd(
        ctypes.byref(prob), _pool(pool_hw), q.data_ptr(), ctypes.byref(_strides(q)),
        k.data_ptr(), ctypes.byref(_strides(k)), v.data_ptr(), ctypes.byref(_strides(v)),
        o.data_ptr(), ctypes.byref(_strides(o)),
        workspace.data_ptr(), _nbytes(workspace), _stream(stream)))
    return o


def _bwd_outputs(q, dq, dk, dv):
    return tuple(_out_like(q, t, name) for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")))


def sta_attn_bwd_workspace_size(batch, heads, head_dim, grid, dtype_code=VDSA_BF16) -> int:
    prob = make_problem(batch, heads, head_dim, grid, dtype_code, 1.0)
    n = ctypes.c_size_t()
    check(lib().sta_attn_bwd_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    return n.value


def sta_attn_bwd(q, k, v, o, do, lse, grid, tile, window, shift=(0, 0, 0), scale=None, dq=None, dk=None, dv=None,
                 workspace=None, stream=None, window_mode: str = "clip"):
    """Gradients of ``sta_attn_fwd`` (``sta_attn_bwd`` in include/vdsa.h), from
    the forward's inputs, output ``o`` and ``lse``.  Returns (dQ, dK, dV)."""
    _same(q, k, v, o, do)
    prob = _problem_for(q, grid, scale)
    cfg = make_cfg(tile, window, shift, window_mode)
    lse = _lse_in(q, lse, "lse")
    dq, dk, dv = _bwd_outputs(q, dq, dk, dv)
    _on_device(q, k, v, o, do, lse, dq, dk, dv, _workspace_arg(workspace))
    need = ctypes.c_size_t()
    check(lib().sta_attn_bwd_workspace_size(ctypes.byref(prob), ctypes.byref(need)))
    workspace = _workspace(q, workspace, need.value)
    check(lib().sta_attn_bwd(
        ctypes.byref(prob), ctypes.byref(cfg), q.data_ptr(), ctypes.byref(_strides(q)),
        k.data_ptr(), ctypes.byref(_strides(k)), v.data_ptr(), ctypes.byref(_strides(v)),
        o.data_ptr(), ctypes.byref(_strides(o)), do.data_ptr(), ctypes.byref(_strides(do)),
        lse.data_ptr(), dq.data_ptr(), ctypes.byref(_strides(dq)),
        dk.data_ptr(), ctypes.byref(_strides(dk)), dv.data_ptr(), ctypes.byref(_strides(dv)),
        workspace.data_ptr(), _nbytes(workspace), _stream(stream)))
    return dq, dk, dv


def global_pooled_attn_bwd_workspace_size(batch, heads, head_dim, grid, pool_hw, dtype_code=VDSA_BF16) -> int:
    prob = make_problem(batch, heads, head_dim, grid, dtype_code, 1.0)
    n = ctypes.c_size_t()
    check(lib().global_pooled_attn_bwd_workspace_size(ctypes.byref(prob), _pool(pool_hw), ctypes.byref(n)))
    return n.value


def global_pooled_attn_bwd(q, k, v, o, do, lse, grid, pool_hw, scale=None, dq=None, dk=None, dv=None,
                           workspace=None, stream=None):
    """Gradients of ``global_pooled_attn_fwd`` through the pooling
    (``global_pooled_attn_bwd``).  Returns (dQ, dK, dV)."""
    _same(q, k, v, o, do)
    prob = _problem_for(q, grid, scale)
    lse = _lse_in(q, lse, "lse")
    dq, dk, dv = _bwd_outputs(q, dq, dk, dv)
    _on_device(q, k, v, o, do, lse, dq, dk, dv, _workspace_arg(workspace))
    need = ctypes.c_size_t()
    check(lib().global_pooled_attn_bwd_workspace_size(ctypes.byref(prob), _pool(pool_hw), ctypes.byref(need)))
    workspace = _workspace(q, workspace, need.value)
    check(lib().global_pooled_attn_bwd(
        ctypes.byref(prob), _pool(pool_hw), q.data_ptr(), ctypes.byref(_strides(q)),
        k.data_ptr(), ctypes.byref(_strides(k)), v.data_ptr(), ctypes.byref(_strides(v)),
        o.data_ptr(), ctypes.byref(_strides(o)), do.data_ptr(), ctypes.byref(_strides(do)),
        lse.data_ptr(), dq.data_ptr(), ctypes.byref(_strides(dq)),
        dk.data_ptr(), ctypes.byref(_strides(dk)), dv.data_ptr(), ctypes.byref(_strides(dv)),
        workspace.data_ptr(), _nbytes(workspace), _stream(stream)))
    return dq, dk, dv


def kv_avgpool_fwd(x, grid, pool_hw, out=None, stream=None):
    """k_h x k_w frame-wise average pooling of a [B, heads, N, D] tensor."""
    torch = _torch()
    _same(x)
    B, Hh, N, D = x.shape
    prob = _problem_for(x, grid, 1.0)
    T, H, W = grid
    M = T * (-(-H // pool_hw[0])) * (-(-W // pool_hw[1]))
    y = torch.empty((B, Hh, M, D), dtype=x.dtype, device=x.device) if out is None else \
        _arg(out, "out", (B, Hh, M, D), x.dtype)
    _on_device(x, y)
    check(lib().kv_avgpool_fwd(ctypes.byref(prob), _pool(pool_hw), x.data_ptr(), ctypes.byref(_strides(x)),
                               y.data_ptr(), ctypes.byref(_strides(y)), _stream(stream)))
    return y


def sta_flops(batch, heads, head_dim, grid, tile, window, shift=(0, 0, 0), window_mode: str = "clip") -> float:
    """Effective FLOP of one sta_attn_fwd call (4*D per attended token pair)."""
    prob = make_problem(batch, heads, head_dim, grid, VDSA_BF16, 1.0)
    cfg = make_cfg(tile, window, shift, window_mode)
    f = ctypes.c_double()
    check(lib().vdsa_sta_flops(ctypes.byref(prob), ctypes.byref(cfg), ctypes.byref(f)))
    return f.value


def sta_kernel_name(batch, heads, head_dim, grid, tile, window, shift=(0, 0, 0), window_mode: str = "clip",
                    dtype: str = "bf16") -> str:
    """Name of the kernel sta_attn_fwd launches for this configuration
    (``vdsa_sta_kernel``; host only).  dtype: "bf16" or "f32"."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    prob = make_problem(batch, heads, head_dim, grid, VDSA_BF16 if dtype == "bf16" else VDSA_F32, 1.0)
    cfg = make_cfg(tile, window, shift, window_mode)
    name = lib().vdsa_sta_kernel(ctypes.byref(prob), ctypes.byref(cfg))
    if name is None:
        raise ValueError(lib().vdsa_last_error().decode())
    return name.decode()


def global_flops(batch, heads, head_dim, grid, pool_hw) -> float:
    prob = make_problem(batch, heads, head_dim, grid, VDSA_BF16, 1.0)
    f = ctypes.c_double()
    check(lib().vdsa_global_flops(ctypes.byref(prob), _pool(pool_hw), ctypes.byref(f)))
    return f.value


def hier_flops(batch, heads, head_dim, grid, tile, window, pool_hw, shift=(0, 0, 0)) -> float:
    prob = make_problem(batch, heads, head_dim, grid, VDSA_BF16, 1.0)
    cfg = make_cfg(tile, window, shift)
    f = ctypes.c_double()
    check(lib().vdsa_hier_flops(ctypes.byref(prob), ctypes.byref(cfg), _pool(pool_hw), ctypes.byref(f)))
    return f.value


def compressed_global_flops(batch, heads, head_dim, grid, pool_hw) -> float:
    prob = make_problem(batch, heads, head_dim, grid, VDSA_BF16, 1.0)
    f = ctypes.c_double()
    check(lib().vdsa_compressed_global_flops(ctypes.byref(prob), _pool(pool_hw), ctypes.byref(f)))
    return f.value


def abi_version() -> int:
    return lib().vdsa_abi_version()
