"""Shared helpers of the GPU parity tests: tolerances, comparison and row
sampling.  Test infrastructure only."""
import sys

import numpy as np

import oracle as R

# bf16 inputs: max abs error <= 2e-2 and mean abs error <= 2e-3 against the
# fp64 oracle; fp32 path: max abs error <= 1e-4.
TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-4)}
# gradients, relative to the reference gradient's RMS (derivation in the
# backward parity tests' docstring): (elementwise bound on
# |err| / (RMS + |ref|), bound on mean |err| / RMS)
TOL_BWD = {"bf16": (6e-2, 5e-3), "f32": (1e-4, 1e-5)}


def compare(got, ref, dtype, what=""):
    """Element-by-element comparison of a GPU result (any array-like) with the
    oracle's fp64 result; returns (max, mean) abs error, asserts the bar."""
    g = R.to_f64(got)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    err = np.abs(g - r)
    mx, mean = float(err.max()), float(err.mean())
    tmax, tmean = TOL[dtype]
    assert mx <= tmax and mean <= tmean, f"{what}: max err {mx:.3e} (<= {tmax}), mean {mean:.3e} (<= {tmean})"
    return mx, mean


def sample_rows(grid, tile, shift, n_random_tiles=6, rows_per_tile=48, seed=0):
    """Query rows from the corner tiles of the tile lattice, a few edge tiles
    and random tiles; per tile its first and last token (tile-local raster
    order) plus random ones.  Returns sorted token indices."""
    rng = np.random.default_rng(seed)
    counts = R.tile_counts(grid, tile, shift)
    T, H, W = grid
    picks = set()
    for ct in (0, counts[0] - 1):
        for ch in (0, counts[1] - 1):
            for cw in (0, counts[2] - 1):
                picks.add((ct, ch, cw))
    picks.add((counts[0] // 2, 0, counts[2] // 2))
    picks.add((0, counts[1] // 2, counts[2] - 1))
    for _ in range(n_random_tiles):
        picks.add(tuple(int(rng.integers(0, c)) for c in counts))
    rows = []
    for a in sorted(picks):
        ext = [R.tile_extent(i, L, b, s) for i, L, b, s in zip(a, grid, tile, shift)]
        tt, hh, ww = np.meshgrid(*[np.arange(lo, hi) for lo, hi in ext], indexing="ij")
        toks = ((tt * H + hh) * W + ww).reshape(-1)
        chosen = {int(toks[0]), int(toks[-1])}
        if len(toks) > 2:
            chosen.update(int(x) for x in rng.choice(toks, size=min(rows_per_tile, len(toks)), replace=False))
        rows.extend(chosen)
    return np.array(sorted(set(rows)), dtype=np.int64)


def head_f64(x, b, h):
    """One (batch, head) slice of a [B, heads, N, D] tensor as fp64 NumPy."""
    return R.to_f64(x[b, h])


def rel_compare(got, ref, dt, what):
    """Gradient comparison against the oracle at the TOL_BWD bar; prints the
    measured errors."""
    g = R.to_f64(got)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    rms = float(np.sqrt(np.mean(r * r)))
    err = np.abs(g - r)
    tmax, tmean = TOL_BWD[dt]
    worst = float((err / (rms + np.abs(r))).max())
    mean = float(err.mean()) / rms
    print(f"  {what}: max err {worst:.2e} (rms + |ref|), mean {mean:.2e} rms (rms {rms:.3e})",
          file=sys.stderr, flush=True)
    assert worst <= tmax and mean <= tmean, \
        f"{what}: max err {worst:.3e} x (rms + |ref|) (<= {tmax}), mean {mean:.3e} rms (<= {tmean})"


def bwd_rounding_bound(q, k, v, do, grid, tile, window, shift, scale, window_mode="clip"):
    """Element-wise bound on the gradient error that the bf16 backward's own
    roundings can cause, from fp64 quantities of one head (forward error
    analysis, |fl(ab) - ab| <= u |a||b| with bf16 unit roundoff u = 2^-8).
    The kernels round dS = P (dP - delta) and P to bf16 and take delta from
    the bf16 forward output O, so per query tile, with E = u (|dS| +
    P rowsum(|dO| |O|)):
        |err dQ| <= scale E |K|,   |err dK| <= scale E^T |Q|,
        |err dV| <= u P^T |dO|.
    Returns the three bounds, each [N, D]."""
    u = 2.0 ** -8
    q, k, v, do = (np.asarray(R.to_f64(x)) for x in (q, k, v, do))
    ti = R.mode_tile_index(grid, tile, shift, window_mode)
    counts = R.mode_tile_counts(grid, tile, shift, window_mode)
    radius = R.window_radius(window)
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for a in np.unique(ti, axis=0):
        qi = np.nonzero(np.all(ti == a, axis=1))[0]
        ki = np.nonzero(R.mode_mask_row(ti, a, radius, counts, window_mode))[0]
        s = scale * q[qi] @ k[ki].T
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ v[ki]
        delta = (do[qi] * o).sum(axis=1, keepdims=True)
        ds = p * (do[qi] @ v[ki].T - delta)
        e = u * (np.abs(ds) + p * (np.abs(do[qi]) * np.abs(o)).sum(axis=1, keepdims=True))
        bq[qi] += scale * e @ np.abs(k[ki])
        bk[ki] += scale * e.T @ np.abs(q[qi])
        bv[ki] += u * p.T @ np.abs(do[qi])
    return bq, bk, bv


def bound_compare(got, ref, bound, what, slack=2.0, mean_tol=5e-3):
    """|got - ref| <= slack * bound element by element (slack for the fp32
    accumulation and the forward's LSE), and mean |err| <= mean_tol * RMS."""
    g = R.to_f64(got)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    err = np.abs(g - r)
    rms = float(np.sqrt(np.mean(r * r)))
    ratio = float((err / (slack * bound + 1e-6 * rms)).max())
    mean = float(err.mean()) / rms
    print(f"  {what}: max err / ({slack} x bound) {ratio:.3f}, mean {mean:.2e} rms", file=sys.stderr, flush=True)
    assert ratio <= 1.0 and mean <= mean_tol, \
        f"{what}: max err {ratio:.3f} x ({slack} x rounding bound) (<= 1), mean {mean:.3e} rms (<= {mean_tol})"
