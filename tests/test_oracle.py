"""Pins for the CPU oracle: each test checks the oracle against something other
than itself (a library routine, a closed form, an invariant, a brute force
built differently, or a fact the pages state).  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def randn(seed, *shape):
    return rng(seed).standard_normal(shape)


def coords_lib(grid):
    """Token coordinates via numpy's own index decomposition (not the oracle's)."""
    T, H, W = grid
    t, h, w = np.unravel_index(np.arange(T * H * W), (T, H, W))
    return np.stack([t, h, w], axis=1)


# ---------------------------------------------------------------- softmax core
def test_dense_matches_torch_sdpa_fp64():
    q, k, v = randn(1, 40, 32), randn(2, 55, 32), randn(3, 55, 24)
    for scale in (None, 0.3):
        o, lse = R.dense_ref(q, k, v, scale=scale)
        s = scale if scale is not None else 1 / math.sqrt(32)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], scale=s)[0]
        np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
        lse_lib = torch.logsumexp(s * torch.from_numpy(q) @ torch.from_numpy(k).T, dim=1).numpy()
        np.testing.assert_allclose(lse, lse_lib, rtol=0, atol=1e-12)


def test_two_key_closed_form():
    # logits 0 and ln 3 -> weights 1/4, 3/4 exactly
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 5.0], [math.log(3.0), -2.0]])
    v = np.array([[4.0, -8.0], [8.0, 4.0]])
    o, lse = R.dense_ref(q, k, v, scale=1.0)
    np.testing.assert_allclose(o[0], [0.25 * 4 + 0.75 * 8, 0.25 * -8 + 0.75 * 4], atol=1e-14)
    np.testing.assert_allclose(lse[0], math.log(1 + 3), atol=1e-14)


def test_single_key_returns_value():
    q, k, v = randn(4, 3, 8), randn(5, 1, 8), randn(6, 1, 8)
    o, lse = R.dense_ref(q, k, v)
    np.testing.assert_allclose(o, np.repeat(v, 3, axis=0), atol=1e-15)
    np.testing.assert_allclose(lse, (q @ k.T)[:, 0] / math.sqrt(8), atol=1e-14)


def test_bf16_bits_widen_exactly():
    x = torch.randn(64, dtype=torch.float32).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(R.to_f64(bits), x.float().numpy().astype(np.float64))
    np.testing.assert_array_equal(R.to_f64(x), x.float().numpy().astype(np.float64))


# ---------------------------------------------------------------- token grid
@pytest.mark.parametrize("grid", [(4, 8, 8), (3, 5, 7), (1, 1, 9), (21, 90, 160)])
def test_token_coords_raster(grid):
    np.testing.assert_array_equal(R.token_coords(grid), coords_lib(grid))


def test_tile_partition_sizes_closed_form():
    # 2K workload: T=21 tile 4 shift 2 -> [2,4,4,4,4,3]; H=90 tile 8 shift 4 ->
    # [4, 8 x 10, 6]; W=160 tile 8 shift 4 -> [4, 8 x 19, 4]; unshifted H -> [8 x 11, 2].
    def sizes(L, b, s):
        n = R.tile_counts((L, 1, 1), (b, 1, 1), (s, 0, 0))[0]
        return [R.tile_extent(i, L, b, s)[1] - R.tile_extent(i, L, b, s)[0] for i in range(n)]
    assert sizes(21, 4, 2) == [2, 4, 4, 4, 4, 3]
    assert sizes(90, 8, 4) == [4] + [8] * 10 + [6]
    assert sizes(160, 8, 4) == [4] + [8] * 19 + [4]
    assert sizes(90, 8, 0) == [8] * 11 + [2]
    assert sizes(21, 4, 0) == [4] * 5 + [1]
    # extents agree with the tile index of every coordinate
    for L, b, s in [(21, 4, 2), (13, 4, 3), (7, 3, 1), (10, 5, 0)]:
        x = np.arange(L)
        ti = R.tile_index(np.stack([x, 0 * x, 0 * x], 1), (b, 1, 1), (s, 0, 0))[:, 0]
        n = R.tile_counts((L, 1, 1), (b, 1, 1), (s, 0, 0))[0]
        assert ti.max() == n - 1 and ti.min() == 0
        for i in range(n):
            lo, hi = R.tile_extent(i, L, b, s)
            np.testing.assert_array_equal(np.nonzero(ti == i)[0], np.arange(lo, hi))


def test_shifted_partition_page_fact():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))["shifted_partition"]
    for K, expect in zip(facts["K"], facts["shifted_windows_per_side"]):
        b = 8
        L = K * b
        assert R.tile_counts((L, L, L), (b, b, b), (0, 0, 0)) == (K, K, K)
        assert R.tile_counts((L, L, L), (b, b, b), (0, b // 2, b // 2)) == (K, expect, expect)
        # the two edge windows of the shifted partition are half windows
        assert R.tile_extent(0, L, b, b // 2) == (0, b // 2)
        assert R.tile_extent(expect - 1, L, b, b // 2) == (L - b // 2, L)


def test_window_rejects_even():
    with pytest.raises(ValueError):
        R.window_radius((3, 2, 3))
    with pytest.raises(ValueError):
        R.window_radius((0, 1, 1))


# ---------------------------------------------------------------- STA pins
FULL_WINDOW_CASES = [
    # grid, tile, window, shift
    ((4, 8, 8), (2, 4, 4), (3, 3, 3), (0, 0, 0)),        # the tiny fp32 workload: dense
    ((3, 5, 7), (2, 2, 3), (3, 5, 5), (1, 1, 2)),        # partial tiles + shift, full window
    ((2, 6, 6), (1, 1, 1), (3, 11, 11), (0, 0, 0)),
]


@pytest.mark.parametrize("grid,tile,window,shift", FULL_WINDOW_CASES)
def test_full_window_is_dense(grid, tile, window, shift):
    N = int(np.prod(grid))
    q, k, v = randn(10, N, 16), randn(11, N, 16), randn(12, N, 16)
    o, lse = R.sta_ref(q, k, v, grid, tile, window, shift, scale=0.25)
    od, lsed = R.dense_ref(q, k, v, scale=0.25)
    np.testing.assert_allclose(o, od, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, atol=1e-12)


SPARSE_CASES = [
    ((8, 16, 16), (2, 4, 4), (3, 3, 3), (0, 0, 0)),
    ((7, 13, 21), (3, 4, 8), (3, 3, 1), (1, 2, 4)),
    ((5, 9, 11), (2, 3, 3), (1, 3, 5), (1, 0, 2)),
    ((4, 8, 12), (2, 4, 4), (1, 3, 3), (1, 2, 0)),
]


@pytest.mark.parametrize("grid,tile,window,shift", [c for c in SPARSE_CASES if np.prod(c[0]) <= 1200])
def test_weights_row_stochastic_and_zero_outside(grid, tile, window, shift):
    N = int(np.prod(grid))
    q, k = randn(20, N, 8), randn(21, N, 8)
    P = R.attention_weights_ref(q, k, grid, tile, window, shift)
    assert (P >= 0).all()
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
    # independent zero pattern: per-dim 1-D tile ids from integer division of raw coordinates
    c = coords_lib(grid)
    tid = (c + np.array(shift)) // np.array(tile)
    r = (np.array(window) - 1) // 2
    allowed = np.ones((N, N), bool)
    for d in range(3):
        allowed &= np.abs(tid[:, d][:, None] - tid[:, d][None, :]) <= r[d]
    assert (P[~allowed] == 0).all()
    assert (P[allowed] > 0).all()


@pytest.mark.parametrize("grid,tile,window,shift", [c for c in SPARSE_CASES if np.prod(c[0]) <= 1200]
                         + FULL_WINDOW_CASES[:2])
@pytest.mark.parametrize("scale", [None, 0.7])
def test_weights_equal_torch_softmax_of_masked_scores(grid, tile, window, shift, scale):
    # the values themselves, not only their pattern: torch's softmax of the
    # scaled logits with every key outside an independently built mask at -inf
    # (a wrong scale, a dropped max shift or a transposed operand fails here)
    N = int(np.prod(grid))
    D = 8
    q, k = randn(22, N, D), randn(23, N, D)
    P = R.attention_weights_ref(q, k, grid, tile, window, shift, scale=scale)
    s = (1.0 / math.sqrt(D)) if scale is None else scale
    logits = s * torch.from_numpy(q) @ torch.from_numpy(k).T
    mask = torch.from_numpy(_sta_mask_by_coords(grid, tile, window, shift))
    ref = torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=1).numpy()
    np.testing.assert_allclose(P, ref, rtol=0, atol=1e-13)
    # and the weights reproduce the oracle's output: O = P V
    v = randn(24, N, 5)
    o, _ = R.sta_ref(q, k, v, grid, tile, window, shift, scale=scale)
    np.testing.assert_allclose(P @ v, o, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [(1, 1, 1), (3, 3, 3), (1, 3, 5), (3, 5, 1)])
def test_unit_tiles_equal_token_sliding_window(window):
    grid = (4, 7, 9)
    N = int(np.prod(grid))
    q, k, v = randn(30, N, 12), randn(31, N, 12), randn(32, N, 12)
    o, lse = R.sta_ref(q, k, v, grid, (1, 1, 1), window, (0, 0, 0), scale=0.4)
    c = coords_lib(grid)
    r = (np.array(window) - 1) // 2
    for n in range(N):
        keys = np.nonzero(np.all(np.abs(c - c[n]) <= r, axis=1))[0]
        on, ln = R.dense_ref(q[n:n + 1], k[keys], v[keys], scale=0.4)
        np.testing.assert_allclose(o[n], on[0], atol=1e-12)
        np.testing.assert_allclose(lse[n], ln[0], atol=1e-12)


def _box_1d(L, b, s, r, x):
    """Interval of coordinates whose 1-D tile is within r of x's tile (scan)."""
    tiles = [(xx + s) // b for xx in range(L)]
    sel = [xx for xx in range(L) if abs(tiles[xx] - tiles[x]) <= r]
    assert sel == list(range(sel[0], sel[-1] + 1))
    return sel[0], sel[-1] + 1


@pytest.mark.parametrize("grid,tile,window,shift", SPARSE_CASES + [((4, 8, 8), (2, 4, 4), (3, 3, 3), (0, 0, 0))])
def test_zero_keys_give_window_box_mean(grid, tile, window, shift):
    """K = 0 makes all logits 0: O is the plain mean of V over the window's
    tokens, here via a 3-D summed-area table; LSE is log(count)."""
    T, H, W = grid
    N = T * H * W
    D = 6
    v = randn(40, N, D)
    q = randn(41, N, D)
    k = np.zeros((N, D))
    rows = np.arange(N) if N <= 800 else rng(42).choice(N, 400, replace=False)
    o, lse = R.sta_ref(q, k, v, grid, tile, window, shift, rows=rows)
    S = np.zeros((T + 1, H + 1, W + 1, D))
    S[1:, 1:, 1:] = v.reshape(T, H, W, D).cumsum(0).cumsum(1).cumsum(2)
    r = [(w - 1) // 2 for w in window]
    c = coords_lib(grid)
    for i, n in enumerate(rows):
        (t0, t1), (h0, h1), (w0, w1) = [
            _box_1d(L, b, s, rr, x) for L, b, s, rr, x in zip(grid, tile, shift, r, c[n])]
        tot = (S[t1, h1, w1] - S[t0, h1, w1] - S[t1, h0, w1] - S[t1, h1, w0]
               + S[t0, h0, w1] + S[t0, h1, w0] + S[t1, h0, w0] - S[t0, h0, w0])
        cnt = (t1 - t0) * (h1 - h0) * (w1 - w0)
        np.testing.assert_allclose(o[i], tot / cnt, atol=1e-12)
        np.testing.assert_allclose(lse[i], math.log(cnt), atol=1e-12)


def test_constant_values_pass_through():
    grid, tile, window, shift = (5, 9, 11), (2, 3, 3), (1, 3, 5), (1, 0, 2)
    N = int(np.prod(grid))
    q, k = randn(50, N, 8) * 3, randn(51, N, 8) * 3
    c = randn(52, 1, 5)
    v = np.repeat(c, N, axis=0)
    o, _ = R.sta_ref(q, k, v, grid, tile, window, shift)
    np.testing.assert_allclose(o, v, atol=1e-13)


def test_translation_by_whole_tiles():
    """Rolling the grid by one tile in w moves interior outputs by one tile."""
    grid, tile, window = (4, 8, 24), (2, 4, 4), (3, 3, 3)
    T, H, W = grid
    N = T * H * W
    q, k, v = randn(60, N, 8), randn(61, N, 8), randn(62, N, 8)
    roll = lambda x: np.roll(x.reshape(T, H, W, -1), 4, axis=2).reshape(N, -1)
    o, _ = R.sta_ref(q, k, v, grid, tile, window)
    o2, _ = R.sta_ref(roll(q), roll(k), roll(v), grid, tile, window)
    o = o.reshape(T, H, W, -1)
    o2 = o2.reshape(T, H, W, -1)
    # w tiles 1..3 (window stays clear of both edges before and after the roll)
    np.testing.assert_allclose(o2[:, :, 8:20], o[:, :, 4:16], atol=1e-12)


def test_row_subset_equals_full():
    grid, tile, window, shift = (7, 13, 21), (3, 4, 8), (3, 3, 1), (1, 2, 4)
    N = int(np.prod(grid))
    q, k, v = randn(70, N, 8), randn(71, N, 8), randn(72, N, 8)
    rows = rng(73).choice(N, 97, replace=False)
    o_all, l_all = R.sta_ref(q, k, v, grid, tile, window, shift)
    o_s, l_s = R.sta_ref(q, k, v, grid, tile, window, shift, rows=rows)
    # same values up to the summation order of a different-sized BLAS call
    np.testing.assert_allclose(o_s, o_all[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_s, l_all[rows], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- pooling / global / merge
@pytest.mark.parametrize("grid,pool", [((3, 8, 12), (4, 4)), ((2, 9, 10), (4, 3)), ((2, 5, 7), (8, 8)), ((1, 6, 6), (1, 1))])
def test_pool_ramp_closed_form(grid, pool):
    T, H, W = grid
    kh, kw = pool
    c = coords_lib(grid).astype(np.float64)
    x = np.stack([c[:, 1] * W + c[:, 2], c[:, 0] * 1000.0 + c[:, 2], np.full(len(c), 7.5)], axis=1)
    p = R.pool_ref(x, grid, pool)
    Tp, Hp, Wp = R.pooled_grid(grid, pool)
    assert (Tp, Hp, Wp) == (T, -(-H // kh), -(-W // kw))
    for t in range(T):
        for i in range(Hp):
            for j in range(Wp):
                h0, h1 = i * kh, min(H, (i + 1) * kh)
                w0, w1 = j * kw, min(W, (j + 1) * kw)
                mh, mw = (h0 + h1 - 1) / 2, (w0 + w1 - 1) / 2      # mean of an integer range
                row = p[(t * Hp + i) * Wp + j]
                np.testing.assert_allclose(row, [mh * W + mw, t * 1000.0 + mw, 7.5], atol=1e-12)


def test_pool_identity_and_global_dense():
    grid = (2, 6, 5)
    N = 60
    x = randn(80, N, 4)
    np.testing.assert_array_equal(R.pool_ref(x, grid, (1, 1)), x)
    q, k, v = randn(81, N, 4), randn(82, N, 4), randn(83, N, 4)
    og, lg = R.global_ref(q, R.pool_ref(k, grid, (1, 1)), R.pool_ref(v, grid, (1, 1)))
    od, ld = R.dense_ref(q, k, v)
    np.testing.assert_array_equal(og, od)
    np.testing.assert_array_equal(lg, ld)


def test_pool_matches_torch_avg_pool_when_divisible():
    grid, pool = (3, 8, 12), (4, 3)
    T, H, W = grid
    x = randn(84, T * H * W, 5)
    ref = torch.nn.functional.avg_pool2d(
        torch.from_numpy(x.reshape(T, H, W, 5)).permute(0, 3, 1, 2), pool, stride=pool)
    ref = ref.permute(0, 2, 3, 1).reshape(-1, 5).numpy()
    np.testing.assert_allclose(R.pool_ref(x, grid, pool), ref, atol=1e-13)


def test_merge_special_cases_and_linearity():
    ol, og = randn(90, 3, 10, 4), randn(91, 3, 10, 4)
    g = rng(92).uniform(size=3)
    np.testing.assert_array_equal(R.merge_ref(ol, og, None, np.zeros(3)), ol)
    np.testing.assert_array_equal(R.merge_ref(ol, og, np.zeros(3), np.ones(3)), og)
    m = R.merge_ref(ol, og, None, g)
    for h in range(3):
        np.testing.assert_allclose(m[h], ol[h] + g[h] * og[h], atol=1e-15)
    # heads are independent: permuting heads permutes outputs
    perm = [2, 0, 1]
    np.testing.assert_array_equal(R.merge_ref(ol[perm], og[perm], None, g[perm]), m[perm])


# ---------------------------------------------------------------- exact (LSE) merge
@pytest.mark.parametrize("grid,tile,window,shift,pool", [
    ((4, 6, 8), (2, 3, 4), (1, 1, 1), (0, 0, 0), (2, 2)),
    ((3, 7, 9), (2, 4, 4), (3, 1, 3), (1, 2, 2), (3, 4)),
])
def test_merge_lse_equals_one_softmax_over_union(grid, tile, window, shift, pool):
    # merging the two branch results by their LSEs must equal attention over
    # the explicit union of window keys and pooled keys, built row by row
    N = int(np.prod(grid))
    q, k, v = randn(100, N, 8), randn(101, N, 8), randn(102, N, 8)
    kp, vp = R.pool_ref(k, grid, pool), R.pool_ref(v, grid, pool)
    ol, ll = R.sta_ref(q, k, v, grid, tile, window, shift)
    og, lg = R.global_ref(q, kp, vp)
    om, lm = R.merge_lse_ref(ol, ll, og, lg)
    ou, lu = R.union_attention_ref(q, k, v, grid, tile, window, shift, kp, vp)
    np.testing.assert_allclose(om, ou, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm, lu, rtol=0, atol=1e-12)


def test_merge_lse_limits_and_invariance():
    oa, ob = randn(110, 5, 6), randn(111, 5, 6)
    la, lb = randn(112, 5) * 4, randn(113, 5) * 4
    # an empty second branch (LSE -inf) leaves the first unchanged
    o, l = R.merge_lse_ref(oa, la, ob, np.full(5, -np.inf))
    np.testing.assert_allclose(o, oa, atol=1e-15)
    np.testing.assert_allclose(l, la, atol=1e-15)
    # equal partition functions average the outputs and add log 2
    o, l = R.merge_lse_ref(oa, la, ob, la)
    np.testing.assert_allclose(o, 0.5 * (oa + ob), atol=1e-15)
    np.testing.assert_allclose(l, la + math.log(2.0), atol=1e-14)
    # a common offset of both LSEs moves the merged LSE and nothing else
    o1, l1 = R.merge_lse_ref(oa, la, ob, lb)
    o2, l2 = R.merge_lse_ref(oa, la + 7.5, ob, lb + 7.5)
    np.testing.assert_allclose(o2, o1, atol=1e-14)
    np.testing.assert_allclose(l2, l1 + 7.5, atol=1e-13)
    # symmetric in the two branches
    o3, l3 = R.merge_lse_ref(ob, lb, oa, la)
    np.testing.assert_allclose(o3, o1, atol=1e-15)
    np.testing.assert_allclose(l3, l1, atol=1e-15)


def test_union_attention_two_key_closed_form():
    # grid 1x1x2, unit tiles, window 1: each query's local key is itself; one
    # pooled key (cell 1x2) is the mean of the two keys.  Logits chosen so the
    # weights are 1/4 and 3/4 exactly for query 0.
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    k = np.array([[0.0, 2.0], [2.0 * math.log(3.0), -2.0]])   # pooled key = (ln 3, 0)
    v = np.array([[4.0, -8.0], [6.0, 2.0]])                     # pooled value = (5, -3)
    kp, vp = R.pool_ref(k, (1, 1, 2), (1, 2)), R.pool_ref(v, (1, 1, 2), (1, 2))
    np.testing.assert_allclose(kp, [[math.log(3.0), 0.0]], atol=1e-15)
    o, lse = R.union_attention_ref(q, k, v, (1, 1, 2), (1, 1, 1), (1, 1, 1), (0, 0, 0), kp, vp, scale=1.0)
    # query 0: logits 0 (own key) and ln 3 (pooled)
    np.testing.assert_allclose(o[0], [0.25 * 4 + 0.75 * 5, 0.25 * -8 + 0.75 * -3], atol=1e-14)
    np.testing.assert_allclose(lse[0], math.log(4.0), atol=1e-14)
    # query 1: logits -2 (own key) and 0 (pooled)
    w = 1.0 / (1.0 + math.exp(-2.0))
    np.testing.assert_allclose(o[1], [(1 - w) * 6 + w * 5, (1 - w) * 2 + w * -3], atol=1e-14)
    np.testing.assert_allclose(lse[1], math.log(math.exp(-2.0) + 1.0), atol=1e-14)


# ---------------------------------------------------------------- effective work
@pytest.mark.parametrize("grid,tile,window,shift", SPARSE_CASES[1:] + FULL_WINDOW_CASES)
def test_pair_count_brute_force(grid, tile, window, shift):
    N = int(np.prod(grid))
    c = coords_lib(grid)
    tid = (c + np.array(shift)) // np.array(tile)
    r = (np.array(window) - 1) // 2
    count = 0
    for n in range(N):
        count += int(np.all(np.abs(tid - tid[n]) <= r, axis=1).sum())
    assert R.sta_pair_count_ref(grid, tile, window, shift) == count


def test_pair_count_720p_by_hand():
    # tile lattice 5 x 6 x 10; clipped window tile counts per dim (radius 1, 1, 2):
    # T: 2+3+3+3+2 = 13, H: 2+3+3+3+3+2 = 16, W: 3+4+5*6+4+3 = 44; 384 tokens per tile
    assert R.sta_pair_count_ref((30, 48, 80), (6, 8, 8), (3, 3, 5)) == 13 * 16 * 44 * 384 * 384
    assert R.sta_flops_ref((30, 48, 80), (6, 8, 8), (3, 3, 5), head_dim=128, heads=24) == 4 * 128 * 24 * 9152 * 384 ** 2


def test_full_attention_growth_page_fact():
    f = json.load(open(os.path.join(GOLDEN, "page_facts.json")))["full_attention_growth"]
    g1, g2 = (5, 12, 20), (5, 12 * f["hw_factor"], 20 * f["hw_factor"])
    assert np.prod(g2) == f["token_factor"] * np.prod(g1)
    assert R.dense_flops_ref(g2) == f["map_factor"] * R.dense_flops_ref(g1)


def test_cost_estimate_page_fact():
    """Local K x K windows give 1/K^2 of dense; queries against 2x2-pooled keys
    in those windows give 1/(4K^2); Q, K, V all compressed by K per side give
    1/K^4.  The sum reproduces the page's about-12-fold estimate at K = 4."""
    f = json.load(open(os.path.join(GOLDEN, "page_facts.json")))["cost_estimate"]
    K = f["K"]
    grid = (3, 8 * K, 8 * K)
    T, H, W = grid
    dense = R.dense_flops_ref(grid)
    local = R.sta_flops_ref(grid, (T, H // K, W // K), (1, 1, 1))
    assert local * K ** 2 == dense
    # hierarchical term (reading): each window's queries vs its keys pooled 2x2
    hier = local / 4
    glob_c = R.dense_flops_ref(R.pooled_grid(grid, (K, K)))
    assert glob_c * K ** f["formula_global_power"] == dense
    speedup = dense / (local + hier + glob_c)
    formula = 1 / (f["formula_local_coeff"] / K ** 2 + f["formula_hier_coeff"] / K ** 2 + 1 / K ** 4)
    assert abs(speedup - formula) < 1e-12
    assert round(speedup) == f["approx_speedup"]
    # asymmetric global (full-resolution Q against K x K pooled K/V) is 1/K^2
    assert R.global_flops_ref(grid, (K, K)) * K ** 2 == dense


# ---------------------------------------------------------------- backward
def _autograd_masked_attention(q, k, v, do, mask, scale):
    """Gradients by torch autograd (fp64, CPU) of softmax(scale q k^T + mask) v."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * tq @ tk.T
    if mask is not None:
        s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    o = torch.softmax(s, dim=1) @ tv
    o.backward(torch.from_numpy(do))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def _sta_mask_by_coords(grid, tile, window, shift):
    """Token-level window mask built independently of the oracle: tile
    indices from numpy's own index decomposition, then the window test."""
    c = coords_lib(grid)
    ti = (c + np.asarray(shift)) // np.asarray(tile)
    r = (np.asarray(window) - 1) // 2
    return np.all(np.abs(ti[:, None, :] - ti[None, :, :]) <= r[None, None, :], axis=2)


def test_attention_bwd_matches_autograd():
    q, k, v, do = randn(200, 7, 16), randn(201, 11, 16), randn(202, 11, 16), randn(203, 7, 16)
    got = R.attention_bwd_ref(q, k, v, do, 0.3)
    ref = _autograd_masked_attention(q, k, v, do, None, 0.3)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-12)


@pytest.mark.parametrize("grid,tile,window,shift", [
    ((4, 6, 8), (2, 3, 4), (3, 1, 1), (0, 0, 0)),
    ((3, 7, 9), (2, 4, 4), (1, 3, 3), (1, 2, 2)),
    ((2, 5, 6), (1, 2, 3), (3, 3, 1), (0, 1, 2)),
])
def test_sta_bwd_matches_autograd_of_masked_dense(grid, tile, window, shift):
    N = int(np.prod(grid))
    q, k, v, do = randn(210, N, 8), randn(211, N, 8), randn(212, N, 8), randn(213, N, 8)
    mask = _sta_mask_by_coords(grid, tile, window, shift)
    got = R.sta_bwd_ref(q, k, v, do, grid, tile, window, shift, scale=0.4)
    ref = _autograd_masked_attention(q, k, v, do, mask, 0.4)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-11)


def test_sta_bwd_finite_differences():
    grid, tile, window, shift = (2, 2, 3), (1, 2, 2), (1, 1, 3), (0, 1, 0)
    N, D = 12, 3
    q, k, v, g = randn(220, N, D), randn(221, N, D), randn(222, N, D), randn(223, N, D)
    loss = lambda qq, kk, vv: float((R.sta_ref(qq, kk, vv, grid, tile, window, shift, scale=0.7)[0] * g).sum())
    dq, dk, dv = R.sta_bwd_ref(q, k, v, g, grid, tile, window, shift, scale=0.7)
    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        args = [q, k, v]
        fd = np.zeros_like(grad)
        for n in range(N):
            for d in range(D):
                up = [a.copy() for a in args]
                dn = [a.copy() for a in args]
                up[which][n, d] += eps
                dn[which][n, d] -= eps
                fd[n, d] = (loss(*up) - loss(*dn)) / (2 * eps)
        np.testing.assert_allclose(grad, fd, rtol=0, atol=1e-7)


def test_sta_bwd_invariants():
    # softmax rows sum to one: keys' value gradients sum to the output
    # gradients' sum, and key gradients sum to zero
    grid, tile, window, shift = (3, 6, 8), (2, 3, 4), (1, 3, 1), (1, 1, 2)
    N = int(np.prod(grid))
    q, k, v, do = randn(230, N, 8), randn(231, N, 8), randn(232, N, 8), randn(233, N, 8)
    dq, dk, dv = R.sta_bwd_ref(q, k, v, do, grid, tile, window, shift)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-11)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    # a full window is dense attention's backward
    full = tuple(2 * c - 1 for c in R.tile_counts(grid, tile, shift))
    dense = R.attention_bwd_ref(q, k, v, do, 1.0 / math.sqrt(8))
    for g, r in zip(R.sta_bwd_ref(q, k, v, do, grid, tile, full, shift), dense):
        np.testing.assert_allclose(g, r, atol=1e-12)


@pytest.mark.parametrize("grid,pool", [((2, 4, 6), (2, 3)), ((3, 6, 4), (3, 2)), ((1, 4, 4), (1, 1))])
def test_global_bwd_matches_autograd_through_avg_pool(grid, pool):
    T, H, W = grid
    N = T * H * W
    q, k, v, do = randn(240, N, 5), randn(241, N, 5), randn(242, N, 5), randn(243, N, 5)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    pool2d = lambda x: torch.nn.functional.avg_pool2d(x.reshape(T, H, W, 5).permute(0, 3, 1, 2), pool,
                                                      stride=pool).permute(0, 2, 3, 1).reshape(-1, 5)
    o = torch.softmax(0.5 * tq @ pool2d(tk).T, dim=1) @ pool2d(tv)
    o.backward(torch.from_numpy(do))
    got = R.global_bwd_ref(q, k, v, do, grid, pool, scale=0.5)
    for g, r in zip(got, (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-12)


def test_global_bwd_ragged_cells_finite_differences():
    grid, pool = (1, 3, 5), (2, 2)   # cells of 4, 2 and 1 tokens
    N, D = 15, 2
    q, k, v, g = randn(250, N, D), randn(251, N, D), randn(252, N, D), randn(253, N, D)

    def loss(qq, kk, vv):
        o, _ = R.global_ref(qq, R.pool_ref(kk, grid, pool), R.pool_ref(vv, grid, pool), scale=0.8)
        return float((o * g).sum())
    grads = R.global_bwd_ref(q, k, v, g, grid, pool, scale=0.8)
    eps = 1e-6
    for which in range(3):
        fd = np.zeros((N, D))
        for n in range(N):
            for d in range(D):
                up = [q.copy(), k.copy(), v.copy()]
                dn = [q.copy(), k.copy(), v.copy()]
                up[which][n, d] += eps
                dn[which][n, d] -= eps
                fd[n, d] = (loss(*up) - loss(*dn)) / (2 * eps)
        np.testing.assert_allclose(grads[which], fd, rtol=0, atol=1e-7)


# ---------------------------------------------------------------- compressed global, hierarchical windows
@pytest.mark.parametrize("grid,pool", [((2, 8, 12), (4, 4)), ((3, 9, 10), (4, 3)), ((1, 6, 5), (2, 2)),
                                       ((2, 4, 4), (1, 1))])
def test_upsample_matches_torch_bilinear(grid, pool):
    T, H, W = grid
    _, Hp, Wp = R.pooled_grid(grid, pool)
    xp = randn(300, T * Hp * Wp, 3)
    ref = torch.nn.functional.interpolate(torch.from_numpy(xp.reshape(T, Hp, Wp, 3)).permute(0, 3, 1, 2),
                                          size=(H, W), mode="bilinear", align_corners=False)
    ref = ref.permute(0, 2, 3, 1).reshape(-1, 3).numpy()
    np.testing.assert_allclose(R.upsample_bilinear_ref(xp, grid, pool), ref, rtol=0, atol=1e-12)


def test_upsample_constant_and_identity():
    grid = (2, 6, 9)
    c = np.full((2 * 2 * 3, 4), 1.25)
    np.testing.assert_allclose(R.upsample_bilinear_ref(c, grid, (3, 3)), 1.25, atol=1e-15)
    x = randn(301, 2 * 6 * 9, 4)
    np.testing.assert_allclose(R.upsample_bilinear_ref(x, grid, (1, 1)), x, atol=1e-15)


def test_compressed_global_special_cases():
    grid = (2, 4, 6)
    N = 48
    q, k, v = randn(310, N, 8), randn(311, N, 8), randn(312, N, 8)
    # no pooling: plain dense attention
    np.testing.assert_allclose(R.compressed_global_ref(q, k, v, grid, (1, 1)), R.dense_ref(q, k, v)[0], atol=1e-13)
    # one cell per frame: every output row of a frame is that frame's pooled
    # value (one key; the upsampling of a 1x1 frame is constant)
    o = R.compressed_global_ref(q, k, v, grid, (4, 6))
    vbar = v.reshape(2, 24, 8).mean(axis=1)
    frame_of = np.arange(N) // 24
    np.testing.assert_allclose(o, R.dense_ref(R.pool_ref(q, grid, (4, 6)), R.pool_ref(k, grid, (4, 6)),
                                              R.pool_ref(v, grid, (4, 6)))[0][frame_of], atol=1e-13)
    np.testing.assert_allclose(R.dense_ref(np.zeros((1, 8)), R.pool_ref(k, grid, (4, 6)), vbar)[0][0],
                               vbar.mean(axis=0), atol=1e-14)


@pytest.mark.parametrize("grid,tile,window,shift,pool", [
    ((3, 8, 12), (1, 4, 4), (1, 1, 3), (0, 0, 0), (2, 2)),
    ((2, 9, 10), (2, 3, 4), (1, 3, 1), (1, 1, 2), (2, 2)),
])
def test_hier_pooled_by_explicit_cells(grid, tile, window, shift, pool):
    # pooled keys of a query = the cells holding a token of its window,
    # found here through a dense token -> cell assignment built with numpy
    T, H, W = grid
    N = T * H * W
    q, k, v = randn(320, N, 6), randn(321, N, 6), randn(322, N, 6)
    o, lse = R.hier_pooled_ref(q, k, v, grid, tile, window, shift, pool, scale=0.5)
    mask = _sta_mask_by_coords(grid, tile, window, shift)
    c = coords_lib(grid)
    Hp, Wp = -(-H // pool[0]), -(-W // pool[1])
    cell = (c[:, 0] * Hp + c[:, 1] // pool[0]) * Wp + c[:, 2] // pool[1]
    kp, vp = R.pool_ref(k, grid, pool), R.pool_ref(v, grid, pool)
    for n in range(0, N, 7):
        cells = sorted(set(cell[mask[n]].tolist()))
        ref_o, ref_l = R.dense_ref(q[n:n + 1], kp[cells], vp[cells], scale=0.5)
        np.testing.assert_allclose(o[n], ref_o[0], atol=1e-13)
        np.testing.assert_allclose(lse[n], ref_l[0], atol=1e-13)
    # unit pooling: plain sliding-tile attention
    o1, l1 = R.hier_pooled_ref(q, k, v, grid, tile, window, shift, (1, 1), scale=0.5)
    so, sl = R.sta_ref(q, k, v, grid, tile, window, shift, scale=0.5)
    np.testing.assert_allclose(o1, so, atol=1e-13)
    np.testing.assert_allclose(l1, sl, atol=1e-13)


HIER_COUNT_CASES = [
    # grid, tile, window, shift, pool: aligned, shifted, ragged cells, (4, 3) pooling
    ((3, 8, 16), (1, 4, 4), (1, 3, 3), (0, 0, 0), (2, 2)),
    ((2, 9, 11), (1, 3, 4), (1, 3, 3), (0, 1, 1), (2, 2)),
    ((4, 10, 14), (2, 4, 6), (3, 1, 3), (1, 2, 3), (4, 3)),
    ((3, 7, 9), (2, 3, 2), (1, 3, 5), (1, 1, 1), (3, 2)),
    ((2, 6, 6), (1, 1, 1), (3, 11, 11), (0, 0, 0), (2, 2)),   # full window: every cell
]


@pytest.mark.parametrize("grid,tile,window,shift,pool", HIER_COUNT_CASES)
def test_hier_pair_count_brute_force(grid, tile, window, shift, pool):
    # query by query: the distinct pooling cells among the tokens of an
    # independently built token mask (raw coordinates, numpy's own index
    # decomposition, a token -> cell map written here)
    T, H, W = grid
    mask = _sta_mask_by_coords(grid, tile, window, shift)
    t, h, w = np.unravel_index(np.arange(T * H * W), (T, H, W))
    Wp = -(-W // pool[1])
    cell = (t * (-(-H // pool[0])) + h // pool[0]) * Wp + w // pool[1]
    brute = sum(len(set(cell[mask[n]].tolist())) for n in range(T * H * W))
    assert R.hier_pair_count_ref(grid, tile, window, shift, pool) == brute


def test_hier_pair_count_1080p_closed_form():
    # 1080P local windows (21 x 17 x 30 tokens, one window per tile) over
    # 2 x 2 cells: along H a window [17i, 17i + 17) meets cells
    # floor(17i / 2) .. floor((17i + 16) / 2), nine for every i in 0..3; along
    # W the 30-token windows hold exactly 15 cells; T is not pooled
    assert R.hier_pair_count_ref((21, 68, 120), (21, 17, 30), (1, 1, 1), (0, 0, 0), (2, 2)) \
        == 21 * 68 * 120 * (21 * 9 * 15)
    # pooling 1 x 1 is sliding-tile attention's own pair count
    for grid, tile, window, shift, _ in HIER_COUNT_CASES:
        assert R.hier_pair_count_ref(grid, tile, window, shift, (1, 1)) == R.sta_pair_count_ref(grid, tile, window, shift)


# ---------------------------------------------------------------- window modes
def _mode_mask_by_coords(grid, tile, window, shift, mode):
    """Token-level mask of a window mode, built independently of the oracle."""
    c = coords_lib(grid)
    L = np.asarray(grid)
    b = np.asarray(tile)
    if mode == "cyclic":
        ti = ((c + np.asarray(shift)) % L) // b
        n = -(-L // b)
    else:
        ti = (c + np.asarray(shift)) // b
        n = -(-(L + np.asarray(shift)) // b)
    r = (np.asarray(window) - 1) // 2
    w = 2 * r + 1
    if mode == "inward":
        start = np.empty_like(ti)
        for d in range(3):
            for i in range(ti.shape[0]):
                s0 = ti[i, d] - r[d]
                if s0 + w[d] > n[d]:
                    s0 = n[d] - w[d]
                if s0 < 0:
                    s0 = 0
                start[i, d] = s0
        return np.all((ti[None, :, :] >= start[:, None, :]) & (ti[None, :, :] < start[:, None, :] + w[None, None, :]),
                      axis=2)
    return np.all(np.abs(ti[:, None, :] - ti[None, :, :]) <= r[None, None, :], axis=2)


def _masked_dense(q, k, v, mask, scale):
    s = scale * q @ k.T
    s = np.where(mask, s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return (p / p.sum(axis=1, keepdims=True)) @ v


def test_cyclic_mode_is_clip_on_rolled_grid():
    grid, tile, window, shift = (3, 8, 10), (1, 4, 4), (1, 1, 3), (1, 2, 3)
    T, H, W = grid
    N = T * H * W
    q, k, v = randn(400, N, 6), randn(401, N, 6), randn(402, N, 6)
    o, lse = R.sta_ref(q, k, v, grid, tile, window, shift, scale=0.5, window_mode="cyclic")
    roll = lambda x, s: np.roll(x.reshape(T, H, W, -1), s, axis=(0, 1, 2)).reshape(N, -1)
    ro, rl = R.sta_ref(roll(q, shift), roll(k, shift), roll(v, shift), grid, tile, window, (0, 0, 0), scale=0.5)
    neg = tuple(-s for s in shift)
    np.testing.assert_allclose(o, roll(ro, neg), atol=1e-13)
    np.testing.assert_allclose(lse, roll(rl[:, None], neg)[:, 0], atol=1e-13)


@pytest.mark.parametrize("grid,tile,window,shift,mode", [
    ((4, 9, 12), (2, 3, 4), (3, 1, 3), (0, 0, 0), "inward"),
    ((3, 10, 13), (2, 4, 4), (1, 3, 3), (1, 2, 2), "inward"),
    ((5, 8, 8), (2, 4, 4), (5, 3, 1), (1, 0, 2), "inward"),   # window wider than the T lattice
    ((3, 8, 10), (2, 4, 4), (1, 3, 3), (1, 2, 3), "cyclic"),
])
def test_window_mode_by_independent_mask(grid, tile, window, shift, mode):
    N = int(np.prod(grid))
    q, k, v = randn(410, N, 6), randn(411, N, 6), randn(412, N, 6)
    mask = _mode_mask_by_coords(grid, tile, window, shift, mode)
    o, _ = R.sta_ref(q, k, v, grid, tile, window, shift, scale=0.5, window_mode=mode)
    np.testing.assert_allclose(o, _masked_dense(q, k, v, mask, 0.5), atol=1e-13)
    assert R.sta_pair_count_ref(grid, tile, window, shift, mode) == int(mask.sum())
    if mode == "inward":
        # every window spans min(w, n) tiles per dim
        ti = R.mode_tile_index(grid, tile, shift, mode)
        counts = R.mode_tile_counts(grid, tile, shift, mode)
        r = R.window_radius(window)
        for a in np.unique(ti, axis=0):
            lo, hi = R.window_tiles(a, r, counts, mode)
            np.testing.assert_array_equal(hi - lo + 1, np.minimum(2 * np.asarray(r) + 1, counts))


@pytest.mark.parametrize("mode,shift", [("inward", (1, 2, 0)), ("cyclic", (1, 2, 3))])
def test_window_mode_bwd_matches_autograd(mode, shift):
    grid, tile, window = (3, 8, 10), (2, 4, 4), (1, 3, 3)
    N = int(np.prod(grid))
    q, k, v, do = randn(420, N, 6), randn(421, N, 6), randn(422, N, 6), randn(423, N, 6)
    mask = _mode_mask_by_coords(grid, tile, window, shift, mode)
    got = R.sta_bwd_ref(q, k, v, do, grid, tile, window, shift, scale=0.5, window_mode=mode)
    ref = _autograd_masked_attention(q, k, v, do, mask, 0.5)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-11)
