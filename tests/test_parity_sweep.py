"""Seeded random sweep of small sliding-tile configurations, through the C ABI
against the CPU fp64 oracle, on every output element.

The hand-picked parity cases pin each kernel on chosen shapes; this sweep
draws grids, tiles, windows, lattice shifts, window modes, batch, heads,
head_dim, dtype and with / without LSE from a fixed seed, so that the kernels'
tile decode, box walk, partial blocks and edge tiles meet combinations nobody
chose.  Tiles are drawn from families whose token counts send the call to each
attention kernel (384-, 192- and 128-query bf16, head_dim 64, fp32; for the
384- and 192-query kernels half the draws are whole-tile lattices, which they
walk tile by tile); the CPU
test checks, with the library's own selection (``vdsa_sta_kernel``), that the
sweep reaches every kernel several times.  Sizes stay small enough for the
oracle to finish each case in about a second.  The backward sweep draws from
the same generator at smaller sizes."""
import sys

import numpy as np
import pytest
import torch

import oracle as R
import video_dit_sparse_amd as V
from video_dit_sparse_amd import workloads as WL
from _parity import compare, head_f64, rel_compare

DEV = "cuda:0"
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}

# name, tiles, head_dim, dtype: the tiles' token counts pick the kernel
FAMILIES = [
    ("t384", [(6, 8, 8), (3, 8, 16), (6, 4, 16), (4, 8, 12)], 128, "bf16"),
    ("t192", [(3, 8, 8), (6, 4, 8), (3, 4, 16), (2, 8, 12)], 128, "bf16"),
    ("t128", [(4, 8, 8), (2, 4, 4), (1, 5, 7), (3, 3, 3)], 128, "bf16"),
    ("d64", [(2, 4, 8), (3, 4, 4), (2, 3, 5), (6, 8, 8)], 64, "bf16"),
    ("f32", [(2, 4, 4), (3, 3, 4), (1, 4, 8)], None, "f32"),
]
N_FWD, N_BWD = 40, 12


def draw_cases(n, seed, max_tokens):
    """n configurations: (name, batch, heads, grid, tile, window, shift, mode,
    head_dim, dtype, with_lse)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        fam, tiles, D, dt = FAMILIES[i % len(FAMILIES)]
        if D is None:
            D = int(rng.choice([64, 128]))
        # alternate 384- and 192-token draws: whole tiles with 64-token frames
        # and no lattice shift, which those kernels walk tile by tile
        whole = fam in ("t384", "t192") and (i // len(FAMILIES)) % 2 == 0
        pick = [t for t in tiles if t[1] * t[2] == 64] if whole else tiles
        tile = pick[int(rng.integers(len(pick)))]
        while True:
            # each dim holds at least one full tile and up to about three
            if whole:
                grid = tuple(b * int(rng.integers(1, 4)) for b in tile)
            else:
                grid = tuple(int(rng.integers(b, 3 * b + 3)) for b in tile)
            if int(np.prod(grid)) <= max_tokens:
                break
        counts = [(L + b - 1) // b for L, b in zip(grid, tile)]
        window = tuple(int(rng.choice([w for w in (1, 3, 5) if w <= 2 * c + 1])) for c in counts)
        shift = tuple(int(rng.integers(b)) if rng.random() < 0.6 else 0 for b in tile)
        mode = str(rng.choice(["clip", "clip", "inward", "cyclic"]))
        if whole and mode != "cyclic":
            shift = (0, 0, 0)
        batch = 2 if rng.random() < 0.25 else 1
        heads = 1 if batch == 2 else int(rng.integers(1, 3))
        with_lse = bool(rng.random() < 0.7)
        name = f"{i:02d}_{fam}_{mode}_g{'x'.join(map(str, grid))}_t{'x'.join(map(str, tile))}"
        cases.append((name, batch, heads, grid, tile, window, shift, mode, D, dt, with_lse))
    return cases


FWD = draw_cases(N_FWD, seed=20261203, max_tokens=5000)
BWD = draw_cases(N_BWD, seed=20261204, max_tokens=1500)


def test_sweep_reaches_every_kernel():
    # host only: the library's kernel choice for each drawn case
    seen = {}
    for c in FWD:
        name, B, H, grid, tile, window, shift, mode, D, dt, _ = c
        k = V.sta_kernel_name(B, H, D, grid, tile, window, shift, mode, dtype=dt)
        seen[k] = seen.get(k, 0) + 1
    want = ["box_attn_bf16_pp_kernel<0>", "box_attn_bf16_m16_kernel<4, 0>", "box_attn_bf16_kernel<128>",
            "box_attn_bf16_kernel<64>", "box_attn_f32_kernel<64>", "box_attn_f32_kernel<128>"]
    for k in want:
        assert seen.get(k, 0) >= 2, (k, seen)
    # the tile walks: the 384-query kernel's, plain and on the rolled grid,
    # and the 192-query kernel's
    assert seen.get("box_attn_bf16_pp_kernel<1>", 0) + seen.get("box_attn_bf16_pp_kernel<2>", 0) >= 2, seen
    assert seen.get("box_attn_bf16_m16_kernel<4, 1>", 0) + seen.get("box_attn_bf16_m16_kernel<8, 1, true>", 0) >= 1, seen
    modes = [c[7] for c in FWD]
    assert min(modes.count(m) for m in ("clip", "inward", "cyclic")) >= 5
    assert sum(1 for c in FWD if any(c[6])) >= 15   # shifted lattices
    assert sum(1 for c in FWD if c[1] == 2) >= 4     # batch 2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    V.lib()  # fail loudly if the library is missing


@pytest.mark.gpu
@pytest.mark.parametrize("case", FWD, ids=[c[0] for c in FWD])
def test_sweep_fwd(case, _gpu):
    name, B, H, grid, tile, window, shift, mode, D, dt, with_lse = case
    say(f"[sweep fwd] {name} window {window} shift {shift} B{B} H{H} D{D} {dt} lse={with_lse}")
    N = int(np.prod(grid))
    idx = int(name[:2])
    q, k, v = [WL.make_tensor((B, H, N, D), TDT[dt], DEV, seed=3000 + 10 * idx + i) for i in range(3)]
    res = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, return_lse=with_lse, window_mode=mode)
    o, lse = res if with_lse else (res, None)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            ro, rl = R.sta_ref(head_f64(q, b, h), head_f64(k, b, h), head_f64(v, b, h), grid, tile, window, shift,
                               scale=D ** -0.5, window_mode=mode)
            compare(o[b, h].cpu(), ro, dt, f"{name} b{b} h{h}")
            if with_lse:
                compare(lse[b, h].cpu(), rl, dt, f"{name} lse b{b} h{h}")


@pytest.mark.gpu
@pytest.mark.parametrize("case", BWD, ids=[c[0] for c in BWD])
def test_sweep_bwd(case, _gpu):
    name, B, H, grid, tile, window, shift, mode, D, dt, _ = case
    say(f"[sweep bwd] {name} window {window} shift {shift} B{B} H{H} D{D} {dt}")
    N = int(np.prod(grid))
    idx = int(name[:2])
    q, k, v, do = [WL.make_tensor((B, H, N, D), TDT[dt], DEV, seed=4000 + 10 * idx + i) for i in range(4)]
    o, lse = V.sta_attn_fwd(q, k, v, grid, tile, window, shift, return_lse=True, window_mode=mode)
    if dt == "bf16" and D != 128:
        # the bf16 backward is built for head_dim 128 only: refused before any launch
        with pytest.raises(V.VdsaError, match="UNSUPPORTED"):
            V.sta_attn_bwd(q, k, v, o, do, lse, grid, tile, window, shift, window_mode=mode)
        return
    dq, dk, dv = V.sta_attn_bwd(q, k, v, o, do, lse, grid, tile, window, shift, window_mode=mode)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            ref = R.sta_bwd_ref(head_f64(q, b, h), head_f64(k, b, h), head_f64(v, b, h), head_f64(do, b, h),
                                grid, tile, window, shift, scale=D ** -0.5, window_mode=mode)
            for nm, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
                rel_compare(got[b, h].cpu(), r, dt, f"{name} {nm} b{b} h{h}")
