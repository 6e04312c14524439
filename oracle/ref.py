"""Plain fp64 NumPy definitions of what the attention path computes.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path, and it
imports nothing from it.

Sources (all read as the definition of a masked softmax, nothing blocked,
fused or reordered beyond what the definition states):

* UltraGen: High-Resolution Video Generation with Hierarchical Attention
  (arXiv 2510.18775), summary page, §3 "Preliminaries": a video latent of
  T x H x W positions becomes N = T*H*W tokens; full self-attention forms an
  N x N map.  Token order here is raster, n = (t*H + h)*W + w.
* Fast Video Generation with Sliding Tile Attention (arXiv 2502.04507),
  abstract: attention proceeds tile by tile, each query tile attending the key
  tiles of a local 3D window around it, in contrast to token-wise sliding
  windows.
* UltraGen summary, §4.3 "Cross-window Hierarchical Local Attention": window
  partitions alternate between layers, the second one shifted so that K
  windows per side become K+1.  Read here as a non-cyclic offset ``shift`` of
  the tile lattice (tile index = floor((x + s) / b)), so edge tiles are partial.
* UltraGen summary, §4.2 "Spatially-Compressed Global Attention": frame-wise
  compression with stride k before global attention.  Read here as k_h x k_w
  average pooling within each frame (a stride-k depthwise convolution whose
  weights all equal 1/(k_h k_w)); cells that run past the frame edge average
  only their real tokens.
* AtlasVid (arXiv 2605.16649), abstract: "asymmetric" global-local attention.
  Read here as full-resolution queries against pooled keys and values.
* UltraGen summary, §4.1 "Time-Aware Global-Local Attention": a fusion factor
  combines the local and the global latent.  Read here as a per-head gate:
  O = w_loc[h] * O_loc + w_glob[h] * O_glob.
* UltraGen summary, App. B "Efficiency Analysis": attention cost counted as
  proportional to (attended query-key pairs) x D; here 4*D FLOP per pair
  (2*D for q.k, 2*D for p*v).

Every array argument is a single head, ``[N, D]``, unless stated otherwise.
Inputs are converted to fp64 from exactly the values the caller holds
(bf16 bit patterns widen exactly to fp32 and then to fp64).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "to_f64", "token_coords", "tile_index", "tile_counts", "tile_extent",
    "window_radius", "sta_mask_row", "WINDOW_MODES", "mode_tile_index", "mode_tile_counts",
    "window_tiles", "mode_mask_row", "sta_ref", "dense_ref",
    "attention_weights_ref", "pooled_grid", "pool_ref", "global_ref",
    "merge_ref", "merge_lse_ref", "union_attention_ref", "upsample_bilinear_ref",
    "compressed_global_ref", "hier_pooled_ref", "attention_bwd_ref", "sta_bwd_ref",
    "global_bwd_ref", "sta_pair_count_ref",
    "sta_flops_ref", "global_flops_ref", "dense_flops_ref", "hier_pair_count_ref",
]


# --------------------------------------------------------------------------
# inputs
# --------------------------------------------------------------------------
def to_f64(x) -> np.ndarray:
    """Widen to fp64 without changing any value.

    Accepts NumPy arrays (a ``uint16`` array is taken as raw bf16 bit
    patterns) or any object with ``detach()/cpu()/float()/numpy()`` (a torch
    tensor; bf16 -> fp32 is exact).
    """
    if hasattr(x, "detach"):
        return x.detach().cpu().float().numpy().astype(np.float64)
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# --------------------------------------------------------------------------
# token grid and tile lattice
# --------------------------------------------------------------------------
def token_coords(grid) -> np.ndarray:
    """(t, h, w) of every token in raster order n = (t*H + h)*W + w.

    UltraGen §3: the T x H x W latent is flattened to N = T*H*W tokens.
    Returns int64 ``[N, 3]``.
    """
    T, H, W = (int(g) for g in grid)
    n = np.arange(T * H * W, dtype=np.int64)
    return np.stack([n // (H * W), (n // W) % H, n % W], axis=1)


def tile_index(coords, tile, shift=(0, 0, 0)) -> np.ndarray:
    """Tile coordinate of each token: i_d = floor((x_d + s_d) / b_d).

    The shifted lattice is the second window partition of UltraGen §4.3.
    """
    b = np.asarray(tile, dtype=np.int64)
    s = np.asarray(shift, dtype=np.int64)
    return (np.asarray(coords, dtype=np.int64) + s) // b


def tile_counts(grid, tile, shift=(0, 0, 0)) -> tuple:
    """Number of tiles per dim: ceil((L_d + s_d) / b_d)."""
    return tuple(-(-(int(L) + int(s)) // int(b)) for L, b, s in zip(grid, tile, shift))


def tile_extent(i, L, b, s) -> tuple:
    """Token range [lo, hi) of tile ``i`` along one dim of length ``L``."""
    return max(0, i * b - s), min(L, (i + 1) * b - s)


def window_radius(window) -> tuple:
    """Window of w tiles centred on the query tile has radius (w - 1) / 2.

    Only odd windows are centred; even ones are rejected.
    """
    for w in window:
        if int(w) < 1 or int(w) % 2 == 0:
            raise ValueError(f"window must be odd and >= 1, got {tuple(window)}")
    return tuple((int(w) - 1) // 2 for w in window)


WINDOW_MODES = ("clip", "inward", "cyclic")


def mode_tile_index(grid, tile, shift=(0, 0, 0), window_mode="clip") -> np.ndarray:
    """Tile coordinate of every token under a window mode.

    ``clip`` and ``inward``: the shifted lattice of ``tile_index``.
    ``cyclic``: the token grid is first rolled by the shift, x' = (x + s) mod L
    (a Swin-style cyclic shift, here without a seam mask), then tiled from 0:
    i = x' // b, so the tiles at the seam hold tokens of both grid edges.
    """
    coords = token_coords(grid)
    if window_mode == "cyclic":
        rolled = (coords + np.asarray(shift, dtype=np.int64)) % np.asarray(grid, dtype=np.int64)
        return rolled // np.asarray(tile, dtype=np.int64)
    return tile_index(coords, tile, shift)


def mode_tile_counts(grid, tile, shift=(0, 0, 0), window_mode="clip") -> tuple:
    return tile_counts(grid, tile, (0, 0, 0) if window_mode == "cyclic" else shift)


def window_tiles(query_tile, radius, counts, window_mode="clip"):
    """Per dim, the inclusive range [lo, hi] of key tiles in the window of
    ``query_tile``.  ``clip`` / ``cyclic``: the tiles within ``radius``,
    clipped at the lattice edge.  ``inward``: the same number of tiles, 2r+1,
    moved inward at the edges (all tiles when the lattice has fewer)."""
    lo, hi = [], []
    for a, r, n in zip(query_tile, radius, counts):
        a, r, n = int(a), int(r), int(n)
        if window_mode == "inward":
            c0 = max(0, min(a - r, n - (2 * r + 1)))
            lo.append(c0)
            hi.append(min(n - 1, c0 + 2 * r))
        else:
            lo.append(max(0, a - r))
            hi.append(min(n - 1, a + r))
    return np.asarray(lo), np.asarray(hi)


def mode_mask_row(tiles_of_keys, query_tile, radius, counts, window_mode="clip") -> np.ndarray:
    """Boolean mask over all keys for one query under a window mode."""
    lo, hi = window_tiles(query_tile, radius, counts, window_mode)
    return np.all((tiles_of_keys >= lo[None, :]) & (tiles_of_keys <= hi[None, :]), axis=1)


def sta_mask_row(tiles_of_keys: np.ndarray, query_tile, radius) -> np.ndarray:
    """Boolean mask over all keys for one query: key m is attended iff its
    tile is within ``radius`` tiles of the query's tile in every dim.

    Sliding Tile Attention, abstract: the window is a 3D neighbourhood of
    tiles; windows are clipped at the grid edge (never moved inward).
    """
    d = np.abs(tiles_of_keys - np.asarray(query_tile, dtype=np.int64)[None, :])
    return np.all(d <= np.asarray(radius, dtype=np.int64)[None, :], axis=1)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def _softmax_attend(qb, kb, vb, scale):
    """softmax(scale * q k^T) v over the given keys, plus LSE (natural log)."""
    s = scale * (qb @ kb.T)
    mx = s.max(axis=1, keepdims=True)
    p = np.exp(s - mx)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ vb) / l
    return o, mx[:, 0] + np.log(l[:, 0])


def sta_ref(q, k, v, grid, tile, window, shift=(0, 0, 0), scale=None, rows=None, window_mode="clip"):
    """Sliding-tile attention for one head.

    For query token n: O_n = sum_m softmax_m(scale * q_n . k_m) v_m with m over
    the keys whose tile lies in the window around n's tile (``sta_mask_row``).

    Queries are grouped by their tile index; the explicit boolean mask row
    over all N keys depends on the query only through that index, so it is
    built once per group and checked non-empty (the query's own tile is
    always in its window), then the group's rows are evaluated on exactly the
    selected keys, which equals masking every other key to -inf.

    ``rows``: optional query token indices to evaluate (rows are independent).
    Returns (O [len(rows), D], LSE [len(rows)]).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    N, D = q.shape
    T, H, W = grid
    assert N == T * H * W and k.shape[0] == N and v.shape[0] == N
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    radius = window_radius(window)
    ti = mode_tile_index(grid, tile, shift, window_mode)
    counts = mode_tile_counts(grid, tile, shift, window_mode)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((len(rows), v.shape[1]))
    lse = np.empty(len(rows))
    uniq, inv = np.unique(ti[rows], axis=0, return_inverse=True)
    inv = np.asarray(inv).reshape(-1)
    for g in range(len(uniq)):
        pos = np.nonzero(inv == g)[0]
        mask = mode_mask_row(ti, uniq[g], radius, counts, window_mode)
        assert mask.any(), "a query row with no key"
        keys = np.nonzero(mask)[0]
        o[pos], lse[pos] = _softmax_attend(q[rows[pos]], k[keys], v[keys], scale)
    return o, lse


def dense_ref(q, k, v, scale=None, rows=None):
    """Full softmax attention over all keys (UltraGen §3's N x N map)."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[1])
    qr = q if rows is None else q[np.asarray(rows, dtype=np.int64)]
    return _softmax_attend(qr, k, v, scale)


def attention_weights_ref(q, k, grid, tile, window, shift=(0, 0, 0), scale=None):
    """Full N x N attention weights of sliding-tile attention (tiny inputs).

    Entry [n, m] is softmax weight of key m for query n, exactly 0 where the
    tile window excludes m.
    """
    q, k = to_f64(q), to_f64(k)
    N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    radius = window_radius(window)
    ti = tile_index(token_coords(grid), tile, shift)
    P = np.zeros((N, N))
    for n in range(N):
        keys = np.nonzero(sta_mask_row(ti, ti[n], radius))[0]
        s = scale * (k[keys] @ q[n])
        e = np.exp(s - s.max())
        P[n, keys] = e / e.sum()
    return P


# --------------------------------------------------------------------------
# compressed global branch
# --------------------------------------------------------------------------
def pooled_grid(grid, pool_hw) -> tuple:
    """Grid of pooled tokens: T x ceil(H / k_h) x ceil(W / k_w).

    Frames are not pooled (the compression of UltraGen §4.2 is frame-wise).
    """
    T, H, W = grid
    kh, kw = pool_hw
    return (int(T), -(-int(H) // int(kh)), -(-int(W) // int(kw)))


def pool_ref(x, grid, pool_hw) -> np.ndarray:
    """k_h x k_w spatial average pooling of one head's tokens, frame by frame.

    Output row (t, i, j) in raster order is the mean of x over
    {(t, h, w): i*k_h <= h < min(H, (i+1)*k_h), j*k_w <= w < min(W, (j+1)*k_w)}.
    """
    x = to_f64(x)
    T, H, W = grid
    kh, kw = pool_hw
    _, Hp, Wp = pooled_grid(grid, pool_hw)
    X = x.reshape(T, H, W, -1)
    out = np.empty((T, Hp, Wp, X.shape[-1]))
    for t in range(T):
        for i in range(Hp):
            for j in range(Wp):
                cell = X[t, i * kh:min(H, (i + 1) * kh), j * kw:min(W, (j + 1) * kw)]
                out[t, i, j] = cell.mean(axis=(0, 1))
    return out.reshape(T * Hp * Wp, -1)


def global_ref(q, k_pooled, v_pooled, scale=None, rows=None):
    """Every full-resolution query attends all pooled keys, no mask.

    AtlasVid's asymmetric global-local attention: queries are not compressed.
    """
    return dense_ref(q, k_pooled, v_pooled, scale=scale, rows=rows)


def merge_ref(o_local, o_global, w_local, w_global) -> np.ndarray:
    """O = w_loc[h] * O_loc + w_glob[h] * O_glob, per head.

    ``o_local``/``o_global``: ``[heads, ..., D]``; ``w_local`` may be None
    (all ones).  UltraGen §4.1's fusion factor, taken as a per-head gate.
    """
    ol, og = to_f64(o_local), to_f64(o_global)
    heads = ol.shape[0]
    wl = np.ones(heads) if w_local is None else to_f64(w_local).reshape(heads)
    wg = to_f64(w_global).reshape(heads)
    shape = (heads,) + (1,) * (ol.ndim - 1)
    return wl.reshape(shape) * ol + wg.reshape(shape) * og


def merge_lse_ref(o_a, lse_a, o_b, lse_b):
    """Exact merge of two attention results over disjoint key sets A and B.

    Reading of UltraGen §4.1's fusion of the local and the global latent as
    one softmax over the union of both key sets: with Z_X = exp(LSE_X),
    O = (Z_A O_A + Z_B O_B) / (Z_A + Z_B) and LSE = log(Z_A + Z_B).
    ``o_*``: ``[..., D]``; ``lse_*``: ``[...]`` (natural log).  Returns (O, LSE).
    """
    oa, ob = to_f64(o_a), to_f64(o_b)
    la, lb = to_f64(lse_a), to_f64(lse_b)
    m = np.maximum(la, lb)
    ea, eb = np.exp(la - m), np.exp(lb - m)
    z = ea + eb
    return (ea[..., None] * oa + eb[..., None] * ob) / z[..., None], m + np.log(z)


def union_attention_ref(q, k, v, grid, tile, window, shift, k_pooled, v_pooled, scale=None, rows=None):
    """Each query attends the union of its sliding-tile window keys (as in
    ``sta_ref``) and every pooled key (as in ``global_ref``): one softmax over
    the concatenated key list, evaluated by the definition.  Returns (O, LSE).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    kp, vp = to_f64(k_pooled), to_f64(v_pooled)
    N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    radius = window_radius(window)
    ti = tile_index(token_coords(grid), tile, shift)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((len(rows), v.shape[1]))
    lse = np.empty(len(rows))
    for j, n in enumerate(rows):
        keys = np.nonzero(sta_mask_row(ti, ti[n], radius))[0]
        kk = np.concatenate([k[keys], kp], axis=0)
        vv = np.concatenate([v[keys], vp], axis=0)
        oj, lj = _softmax_attend(q[n:n + 1], kk, vv, scale)
        o[j], lse[j] = oj[0], lj[0]
    return o, lse


def upsample_bilinear_ref(xp, grid, pool_hw):
    """Frame-wise bilinear upsampling of a pooled [T*Hp*Wp, D] tensor back to
    the grid's H x W (UltraGen §4.2: bilinear upsampling restores the latent
    resolution; here without the learned 3D convolution that follows it).
    Half-pixel sample positions: output row y samples pooled row
    max((y + 1/2) Hp/H - 1/2, 0), interpolating the two nearest rows (the
    last row repeats at the far edge); the same along W.
    """
    xp = to_f64(xp)
    T, H, W = grid
    _, Hp, Wp = pooled_grid(grid, pool_hw)
    x = xp.reshape(T, Hp, Wp, -1)

    def taps(n_out, n_in):
        i0 = np.empty(n_out, dtype=np.int64)
        i1 = np.empty(n_out, dtype=np.int64)
        lam = np.empty(n_out)
        for y in range(n_out):
            src = max((y + 0.5) * n_in / n_out - 0.5, 0.0)
            a = int(math.floor(src))
            i0[y], i1[y], lam[y] = a, min(a + 1, n_in - 1), src - a
        return i0, i1, lam
    y0, y1, ly = taps(H, Hp)
    x0, x1, lx = taps(W, Wp)
    out = np.empty((T, H, W, x.shape[-1]))
    for y in range(H):
        for xx in range(W):
            out[:, y, xx] = ((1 - ly[y]) * (1 - lx[xx]) * x[:, y0[y], x0[xx]] + (1 - ly[y]) * lx[xx] * x[:, y0[y], x1[xx]]
                             + ly[y] * (1 - lx[xx]) * x[:, y1[y], x0[xx]] + ly[y] * lx[xx] * x[:, y1[y], x1[xx]])
    return out.reshape(T * H * W, -1)


def compressed_global_ref(q, k, v, grid, pool_hw, scale=None):
    """UltraGen's compressed global attention (§4.2, App. B's (THW)^2 D / K^4
    term): Q, K and V pooled k_h x k_w within each frame, full attention among
    the pooled tokens, bilinear upsampling of the pooled output to the grid."""
    qp, kp, vp = (pool_ref(x, grid, pool_hw) for x in (q, k, v))
    if scale is None:
        scale = 1.0 / math.sqrt(qp.shape[1])
    op, _ = dense_ref(qp, kp, vp, scale=scale)
    return upsample_bilinear_ref(op, grid, pool_hw)


def hier_pooled_ref(q, k, v, grid, tile, window, shift, pool_hw, scale=None, rows=None):
    """Intermediate-scale attention (UltraGen §4.3 hierarchical local
    attention; App. B's (THW)^2 D / (4 K^2) term for 2 x 2 pooling): each
    full-resolution query attends the k_h x k_w pooled keys and values of its
    sliding-tile window, i.e. every pooling cell that holds a token of the
    window (``sta_mask_row``'s keys mapped to their cells).  Returns (O, LSE).
    """
    q = to_f64(q)
    N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kp, vp = pool_ref(k, grid, pool_hw), pool_ref(v, grid, pool_hw)
    T, H, W = grid
    kh, kw = pool_hw
    _, Hp, Wp = pooled_grid(grid, pool_hw)
    coords = token_coords(grid)
    cell = (coords[:, 0] * Hp + coords[:, 1] // kh) * Wp + coords[:, 2] // kw
    radius = window_radius(window)
    ti = tile_index(coords, tile, shift)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.empty((len(rows), D))
    lse = np.empty(len(rows))
    for j, n in enumerate(rows):
        cells = np.unique(cell[sta_mask_row(ti, ti[n], radius)])
        oj, lj = _softmax_attend(q[n:n + 1], kp[cells], vp[cells], scale)
        o[j], lse[j] = oj[0], lj[0]
    return o, lse


# --------------------------------------------------------------------------
# backward (gradients of the forward definitions above)
# --------------------------------------------------------------------------
def attention_bwd_ref(q, k, v, do, scale):
    """Gradients of O = softmax(scale * q k^T) v over the given keys.

    With P the softmax, dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O))
    (the softmax Jacobian applied row by row), dQ = scale dS K and
    dK = scale dS^T Q.  Returns (dQ, dK, dV) for these rows and keys.
    """
    s = scale * (q @ k.T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o = p @ v
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (do * o).sum(axis=1, keepdims=True))
    return scale * (ds @ k), scale * (ds.T @ q), dv


def sta_bwd_ref(q, k, v, do, grid, tile, window, shift=(0, 0, 0), scale=None, window_mode="clip"):
    """Gradients of ``sta_ref`` for one head: every query tile's rows
    contribute through its own selected keys (the explicit mask of
    ``sta_mask_row``); key gradients are summed over all query tiles that
    select the key.  Returns (dQ, dK, dV), each [N, D].
    """
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    radius = window_radius(window)
    ti = mode_tile_index(grid, tile, shift, window_mode)
    counts = mode_tile_counts(grid, tile, shift, window_mode)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    uniq, inv = np.unique(ti, axis=0, return_inverse=True)
    inv = np.asarray(inv).reshape(-1)
    for g in range(len(uniq)):
        rows = np.nonzero(inv == g)[0]
        keys = np.nonzero(mode_mask_row(ti, uniq[g], radius, counts, window_mode))[0]
        gq, gk, gv = attention_bwd_ref(q[rows], k[keys], v[keys], do[rows], scale)
        dq[rows] += gq
        dk[keys] += gk
        dv[keys] += gv
    return dq, dk, dv


def global_bwd_ref(q, k, v, do, grid, pool_hw, scale=None):
    """Gradients of the global branch for one head, through the pooling:
    dQ, dKp, dVp of dense attention over the pooled keys, then every token of
    a cell receives its cell's gradient divided by the cell's token count
    (the derivative of the cell mean).  Returns (dQ, dK, dV), each [N, D].
    """
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kp, vp = pool_ref(k, grid, pool_hw), pool_ref(v, grid, pool_hw)
    dq, dkp, dvp = attention_bwd_ref(q, kp, vp, do, scale)
    T, H, W = grid
    kh, kw = pool_hw
    _, Hp, Wp = pooled_grid(grid, pool_hw)
    dk, dv = np.empty_like(k), np.empty_like(v)
    for t in range(T):
        for i in range(Hp):
            for j in range(Wp):
                hs = range(i * kh, min(H, (i + 1) * kh))
                ws = range(j * kw, min(W, (j + 1) * kw))
                cnt = len(hs) * len(ws)
                m = (t * Hp + i) * Wp + j
                for h in hs:
                    for w in ws:
                        n = (t * H + h) * W + w
                        dk[n] = dkp[m] / cnt
                        dv[n] = dvp[m] / cnt
    return dq, dk, dv


# --------------------------------------------------------------------------
# effective work
# --------------------------------------------------------------------------
def sta_pair_count_ref(grid, tile, window, shift=(0, 0, 0), window_mode="clip") -> int:
    """Attended (query, key) token pairs of one head: sum over tile pairs
    (a, c) with c in a's window of tokens(a) * tokens(c).

    Built from the explicit tile-level mask, so partial tiles count only
    their real tokens.
    """
    radius = window_radius(window)
    sh = (0, 0, 0) if window_mode == "cyclic" else shift
    counts = tile_counts(grid, tile, sh)
    sizes = [np.array([tile_extent(i, int(L), int(b), int(s))[1] - tile_extent(i, int(L), int(b), int(s))[0]
                       for i in range(n)], dtype=np.int64)
             for L, b, s, n in zip(grid, tile, sh, counts)]
    idx = np.stack(np.meshgrid(*[np.arange(n) for n in counts], indexing="ij"), axis=-1).reshape(-1, 3)
    tok = sizes[0][idx[:, 0]] * sizes[1][idx[:, 1]] * sizes[2][idx[:, 2]]
    A = np.stack([mode_mask_row(idx, a, radius, counts, window_mode) for a in idx])
    return int(tok @ A.astype(np.int64) @ tok)


def sta_flops_ref(grid, tile, window, shift=(0, 0, 0), head_dim=128, heads=1, batch=1, window_mode="clip") -> float:
    """4 * D FLOP per attended pair (2D for q.k, 2D for the p*v update)."""
    return 4.0 * head_dim * heads * batch * sta_pair_count_ref(grid, tile, window, shift, window_mode)


def global_flops_ref(grid, pool_hw, head_dim=128, heads=1, batch=1) -> float:
    T, H, W = grid
    M = int(np.prod(pooled_grid(grid, pool_hw)))
    return 4.0 * head_dim * heads * batch * (T * H * W) * M


def dense_flops_ref(grid, head_dim=128, heads=1, batch=1) -> float:
    N = int(np.prod(grid))
    return 4.0 * head_dim * heads * batch * N * N


def hier_pair_count_ref(grid, tile, window, shift, pool_hw) -> int:
    """(query, pooled cell) pairs of ``hier_pooled_ref`` for one head, counted
    query by query through the explicit token -> cell map."""
    T, H, W = grid
    kh, kw = pool_hw
    _, Hp, Wp = pooled_grid(grid, pool_hw)
    coords = token_coords(grid)
    cell = (coords[:, 0] * Hp + coords[:, 1] // kh) * Wp + coords[:, 2] // kw
    ti = tile_index(coords, tile, shift)
    radius = window_radius(window)
    uniq, inv, cnt = np.unique(ti, axis=0, return_inverse=True, return_counts=True)
    total = 0
    for g in range(len(uniq)):
        total += int(cnt[g]) * len(np.unique(cell[sta_mask_row(ti, uniq[g], radius)]))
    return total

