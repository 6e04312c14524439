#!/usr/bin/env python3
"""Benchmark of the sliding-tile attention hot path on one MI355X.

A step is one pass of the workload's hot path over one batch of synthetic
inputs already resident in HBM.  The default workload is the 720P sliding-tile
attention latent (T=30, H=48, W=80; tile 6x8x8; window 3x3x5 tiles; 24 heads;
head_dim 128; bf16), where a step is one ``sta_attn_fwd`` call.  The value is
effective TFLOP/s: 4*head_dim FLOP per attended (query, key) token pair, only
pairs inside the tile windows counted.

Prints one JSON line (rank 0).  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective attention TFLOP/s + ms/call (720P-shape STA, bf16); % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
PEAK_F32_VECTOR_TFLOPS = 157.3   # fp32 vector ALU (the fp32 path has no matrix-core products)
NOMINAL_CLOCK_MHZ = 2400.0   # the clock the published bf16 peak assumes
COUNTERS_FILE = os.path.join(ROOT, "profiles", "sta_bf16_720p_counters.md")
# the 720P workload's 384-token (6x8x8) tiles at head_dim 128 run the 8-wave
# kernel of attn_bf16_pp.hip; its traffic counters are tied to these sources
KERNEL_SOURCES = [os.path.join(ROOT, "video_dit_sparse_amd", "csrc", f)
                  for f in ("attn_bf16_pp.hip", "box_common.h", "internal.h")]


def roofline_of(dtype: str, flop: float, nbytes: float, ms: float) -> dict:
    """Roofline of one attention launch from its effective FLOP, its compulsory
    bytes (Q, K, V read once, O written once) and its time: the fp32 path is
    bound by the vector ALU; a bf16 launch by the matrix cores when its FLOP
    per compulsory byte reach the ridge of the two published peaks
    (2500 TFLOP/s over 8 TB/s, 312.5 FLOP/B), else by HBM (a window of one
    tile is 116-121 FLOP/B)."""
    intensity = flop / nbytes
    if dtype == "f32":
        bound, achieved, peak, unit = "alu", flop / (ms * 1e-3) / 1e12, PEAK_F32_VECTOR_TFLOPS, "TFLOP/s"
    elif intensity >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        bound, achieved, peak, unit = "mfma", flop / (ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", nbytes / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "bytes_per_launch": nbytes, "flop_per_byte": round(intensity, 1)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the sliding-tile kernel from the committed
    rocprofv3 counter summary, or None if absent or taken on other source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    text = open(COUNTERS_FILE).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_bytes) or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def parse_gfx_clocks(text: str):
    """Current clock (MHz) of every GFX_<i> block in `amd-smi metric -c` text."""
    return [int(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", text)]


def gfx_clock_mhz():
    """Mean current GFX clock over the XCDs, read with amd-smi (None if that
    tool is unavailable or its output has no GFX clocks)."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-c"], capture_output=True, text=True, timeout=30)
    except (OSError, subprocess.SubprocessError):
        return None
    mhz = parse_gfx_clocks(r.stdout)
    return sum(mhz) / len(mhz) if mhz else None


def cpu_model_name() -> str:
    """The host CPU's model name (/proc/cpuinfo, as lscpu reports it)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# one CPU-baseline work item: a whole query tile of one head through the
# oracle as it stands, on the head's Q/K/V memory-mapped from fp64 .npy files
# (one copy in the page cache, shared by every worker)
def _cpu_tile(job):
    import numpy as np
    import oracle as R
    paths, slot, grid, tile, window, shift, scale, a = job
    qh, kh, vh = (np.load(pth, mmap_mode="r")[slot] for pth in paths)
    ti = R.tile_index(R.token_coords(grid), tile, shift)
    rows = np.nonzero(np.all(ti == np.asarray(a)[None, :], axis=1))[0]
    nkeys = int(R.sta_mask_row(ti, a, R.window_radius(window)).sum())
    R.sta_ref(qh, kh, vh, grid, tile, window, shift, scale=scale, rows=rows)
    return 4.0 * qh.shape[1] * len(rows) * nkeys


def cpu_baseline(w, q, k, v, budget_s: float, n_heads: int = 6):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    whole query tiles of ``n_heads`` seeded heads, in a seeded random order,
    over a pool of worker processes (one per core of the host's CPU share,
    each with one BLAS thread) until the time budget is spent.  The rate is
    effective FLOP of the finished tiles over the wall time; the full call's
    CPU time is extrapolated from it.  Returns the JSON object."""
    import multiprocessing as mp
    import shutil
    import tempfile

    import numpy as np
    import oracle as R

    nproc = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = nproc
    # the host share a GPU machine grants one GPU is 16 cores, whatever nproc shows
    workers = max(1, min(avail, 16))
    rng = np.random.default_rng(0)
    heads = sorted(rng.choice(w.heads, size=min(n_heads, w.heads), replace=False).tolist())
    tmp = tempfile.mkdtemp(prefix="vdsa_cpu_")
    saved_env = {e: os.environ.get(e) for e in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    try:
        paths = []
        for name, x in (("q", q), ("k", k), ("v", v)):
            pth = os.path.join(tmp, f"{name}.npy")
            np.save(pth, R.to_f64(x[0, heads]))
            paths.append(pth)
        shift = w.shifts[0]
        counts = R.tile_counts(w.grid, w.tile, shift)
        jobs = [(paths, slot, w.grid, w.tile, w.window, shift, w.softmax_scale,
                 tuple(int(c) for c in np.unravel_index(flat, counts)))
                for slot in range(len(heads)) for flat in range(int(np.prod(counts)))]
        jobs = [jobs[i] for i in rng.permutation(len(jobs))]
        for e in saved_env:
            os.environ[e] = "1"
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers) as pool:
            pool.map(int, range(workers))   # start every worker before the clock
            done_flops, tiles, pending, it = 0.0, 0, [], iter(jobs)
            t0 = time.perf_counter()
            for _ in range(workers):
                pending.append(pool.apply_async(_cpu_tile, (next(it),)))
            while pending:
                r = pending.pop(0)
                done_flops += r.get()
                tiles += 1
                if time.perf_counter() - t0 < budget_s:
                    nxt = next(it, None)
                    if nxt is not None:
                        pending.append(pool.apply_async(_cpu_tile, (nxt,)))
            el = time.perf_counter() - t0
    finally:
        for e, val in saved_env.items():
            if val is None:
                os.environ.pop(e, None)
            else:
                os.environ[e] = val
        shutil.rmtree(tmp, ignore_errors=True)
    rate = done_flops / el
    full_flop = R.sta_flops_ref(w.grid, w.tile, w.window, w.shifts[0], head_dim=w.head_dim, heads=w.heads,
                                batch=w.batch)
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{tiles} whole query tiles drawn at random from heads {heads} of {w.name}, "
                      f"fp64 NumPy oracle in {workers} worker processes (1 BLAS thread each), {el:.1f} s wall",
            "nproc": nproc, "cpus_available": avail, "cpu_model": cpu_model_name(),
            "wall_s": round(el, 2), "effective_flop_done": done_flops,
            "extrapolated_full_call_s": round(full_flop / rate, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sta_720p")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget (0 = skip)")
    ap.add_argument("--dense-steps", type=int, default=3, help="full-window comparison calls (0 = skip)")
    ap.add_argument("--bwd-steps", type=int, default=3,
                    help="backward-pass calls of the local branch to time (0 = skip)")
    ap.add_argument("--variant-steps", type=int, default=10,
                    help="calls per timed global-branch form and UltraGen variant (pooled workloads; 0 = skip)")
    ap.add_argument("--mode-steps", type=int, default=3,
                    help="calls per window mode (inward, cyclic) of the local branch to time (0 = skip)")
    ap.add_argument("--hbm-steps", type=int, default=10,
                    help="calls per HBM-bound kernel (pooling, gated merge, LSE merge) to time (0 = skip)")
    ap.add_argument("--clock-seconds", type=float, default=2.0,
                    help="run the dominant kernel back to back this long while reading the GFX clock (0 = skip)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the sliding-tile path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch
    import video_dit_sparse_amd as V
    from video_dit_sparse_amd import _lib as L
    from video_dit_sparse_amd import pipeline as P
    from video_dit_sparse_amd import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    V.lib()  # fail loudly without the HIP library
    dev = "cuda:0"
    w = WL.WORKLOADS[args.workload]
    log(f"[bench] workload {w.name}: {w.description}")
    q, k, v = WL.make_qkv(w, dev)
    gate = WL.make_gate(w, dev)
    buf = P.Buffers(w, q)
    fl = P.flops(w)
    step_flops = sum(fl.values())

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        P.run(w, q, k, v, gate, buf)
    torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        P.run(w, q, k, v, gate, buf)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ev_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall_ms / args.steps
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (events {ev_ms / args.steps:.3f}), "
        f"{value:.1f} effective TFLOP/s")

    # dominant kernel: the sliding-tile attention launch(es) alone, timed with
    # events on the stream it is launched on
    n_local = len(w.shifts)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        for i, s in enumerate(w.shifts):
            V.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, s, scale=w.softmax_scale, out=buf.local[i])
    e1.record(stream)
    torch.cuda.synchronize()
    launch_ms = e0.elapsed_time(e1) / (args.steps * n_local)
    # the same calls one by one, each between its own pair of events: median
    # and minimum per call
    per_call = []
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    for a, z in pairs:
        a.record(stream)
        V.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, w.shifts[0], scale=w.softmax_scale, out=buf.local[0])
        z.record(stream)
    torch.cuda.synchronize()
    per_call = sorted(a.elapsed_time(z) for a, z in pairs)
    launch_flops = fl["local"] / n_local
    achieved = launch_flops / (launch_ms * 1e-3) / 1e12
    traffic = measured_traffic() if w.name == "sta_720p" else None
    launch_bytes = 4.0 * q.numel() * q.element_size()   # Q, K, V read once, O written once
    roofline = roofline_of(w.dtype, launch_flops, launch_bytes, launch_ms)
    roofline.update({"traffic": traffic,
                     "kernel": V.sta_kernel_name(w.batch, w.heads, w.head_dim, w.grid, w.tile, w.window, w.shifts[0],
                                                 dtype=w.dtype),
                     "launch_ms": round(launch_ms, 4),
                     "flop_per_launch": launch_flops,
                     "tflops": round(achieved, 2),
                     "per_call_ms": {"n": len(per_call), "median": round(per_call[len(per_call) // 2], 4),
                                     "min": round(per_call[0], 4)}})

    clock = None
    if args.clock_seconds > 0:
        # the sustained GFX clock under this kernel, read while it runs back to
        # back; the bf16 peak scales with the clock (2.5 PFLOP/s at 2.4 GHz)
        import threading
        reads = []
        th = threading.Thread(target=lambda: [time.sleep(args.clock_seconds / 3), reads.append(gfx_clock_mhz()),
                                              time.sleep(args.clock_seconds / 3), reads.append(gfx_clock_mhz())])
        th.start()
        t_end = time.perf_counter() + args.clock_seconds
        while th.is_alive() or time.perf_counter() < t_end:
            for i, s in enumerate(w.shifts):
                V.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, s, scale=w.softmax_scale, out=buf.local[i])
            torch.cuda.synchronize()
        th.join()
        reads = [r for r in reads if r is not None]
        if reads:
            mhz = sum(reads) / len(reads)
            peak_at = PEAK_BF16_TFLOPS * mhz / NOMINAL_CLOCK_MHZ
            clock = {"source": "amd-smi metric -c (mean over XCDs)", "gfx_mhz": round(mhz, 1), "samples": len(reads),
                     "bf16_peak_at_clock": round(peak_at, 1), "frac_at_clock": round(achieved / peak_at, 4)}
            log(f"[bench] GFX clock under the kernel: {mhz:.0f} MHz; {achieved:.0f} TFLOP/s is "
                f"{100 * achieved / peak_at:.1f}% of the bf16 peak at that clock")

    def timed(fn, n):
        """Average ms of fn over n calls after one untimed call, with events
        on the stream the library launches on."""
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        a.record(stream)
        for _ in range(n):
            fn()
        z.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(z) / n

    extra = {}
    if w.pool_hw is not None and args.variant_steps > 0:
        # global branch: fused global + merge call against the two separate
        # calls, and the standalone exact (LSE) merge, each timed with events
        lse_l = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        V.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, w.shifts[0], scale=w.softmax_scale,
                       out=buf.local[0], lse=lse_l)
        n = args.variant_steps
        fused_ms = timed(lambda: P.run_global(w, q, k, v, gate, buf, fused=True), n)
        unfused_ms = timed(lambda: P.run_global(w, q, k, v, gate, buf, fused=False), n)
        lse_g = torch.empty_like(lse_l)
        V.global_pooled_attn_fwd(q, k, v, w.grid, w.pool_hw, scale=w.softmax_scale, out=buf.glob, lse=lse_g,
                                 workspace=buf.workspace)
        merge_lse_ms = timed(lambda: V.dual_branch_merge_lse(buf.local[0], lse_l, buf.glob, lse_g,
                                                             out=buf.merged), n)
        tensor_bytes = q.numel() * q.element_size()
        lse_bytes = lse_l.numel() * 4
        merge_lse_bytes = 3 * tensor_bytes + 2 * lse_bytes   # read two rows and two LSEs, write one row
        extra["global_branch"] = {
            "fused_global_merge_ms": round(fused_ms, 3), "global_then_merge_ms": round(unfused_ms, 3),
            "merge_lse_ms": round(merge_lse_ms, 4),
            "merge_lse_GBps": round(merge_lse_bytes / (merge_lse_ms * 1e-3) / 1e9, 1),
            "merge_lse_hbm_frac": round(merge_lse_bytes / (merge_lse_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"[bench] global branch: fused {fused_ms:.3f} ms, global then merge {unfused_ms:.3f} ms; "
            f"LSE merge {merge_lse_ms:.3f} ms ({merge_lse_bytes / (merge_lse_ms * 1e-3) / 1e9:.0f} GB/s)")
        # UltraGen's variants on the same inputs: hierarchical windows over
        # 2x2-pooled keys (the local tiling), compressed global attention
        # (Q pooled too, bilinear upsampling; the workload's pooling)
        sh0 = w.shifts[0]
        ws_h = torch.empty(L.global_pooled_attn_workspace_size(w.batch, w.heads, w.head_dim, w.grid, (2, 2),
                                                               1 if w.dtype == "bf16" else 0),
                           dtype=torch.uint8, device=dev)
        ws_c = torch.empty(2 * buf.workspace.numel(), dtype=torch.uint8, device=dev)
        hier_ms = timed(lambda: V.hier_pooled_attn_fwd(q, k, v, w.grid, w.tile, w.window, (2, 2), sh0,
                                                       scale=w.softmax_scale, out=buf.glob, workspace=ws_h), n)
        comp_ms = timed(lambda: V.compressed_global_attn_fwd(q, k, v, w.grid, w.pool_hw, scale=w.softmax_scale,
                                                             out=buf.glob, workspace=ws_c), n)
        hier_fl = V.hier_flops(w.batch, w.heads, w.head_dim, w.grid, w.tile, w.window, (2, 2), sh0)
        comp_fl = V.compressed_global_flops(w.batch, w.heads, w.head_dim, w.grid, w.pool_hw)
        extra["ultragen_variants"] = {
            "hier_pool2x2_ms": round(hier_ms, 3), "hier_effective_flop": hier_fl,
            "hier_tflops": round(hier_fl / (hier_ms * 1e-3) / 1e12, 1),
            "compressed_global_ms": round(comp_ms, 3), "compressed_global_effective_flop": comp_fl,
            "compressed_global_tflops": round(comp_fl / (comp_ms * 1e-3) / 1e12, 1)}
        log(f"[bench] hierarchical (2x2-pooled keys): {hier_ms:.3f} ms ({hier_fl / (hier_ms * 1e-3) / 1e12:.0f} TFLOP/s); "
            f"compressed global: {comp_ms:.3f} ms ({comp_fl / (comp_ms * 1e-3) / 1e12:.0f} TFLOP/s)")
    if args.hbm_steps > 0:
        # the HBM-bound steps on this workload's tensors: K/V pooling (the
        # workload's pooling, else 4x4), the gated merge and the LSE merge of
        # two branch outputs; compulsory bytes (inputs read once, output
        # written once) over the event-timed call
        n = args.hbm_steps
        pool = tuple(w.pool_hw) if w.pool_hw is not None else (4, 4)
        tensor_bytes = q.numel() * q.element_size()
        pooled = V.kv_avgpool_fwd(k, w.grid, pool)
        pool_ms = timed(lambda: V.kv_avgpool_fwd(k, w.grid, pool, out=pooled), n)
        pool_bytes = tensor_bytes + pooled.numel() * pooled.element_size()
        o_m = torch.empty_like(q)
        gm_ms = timed(lambda: V.dual_branch_merge(q, k, gate if gate is not None else torch.rand(w.heads, device=dev),
                                                  out=o_m), n)
        lse_a = torch.zeros(q.shape[:3], dtype=torch.float32, device=dev)
        lse_b = torch.ones_like(lse_a)
        lm_ms = timed(lambda: V.dual_branch_merge_lse(q, lse_a, k, lse_b, out=o_m), n)
        lse_bytes = lse_a.numel() * 4

        def rate(nbytes, ms):
            gbs = nbytes / (ms * 1e-3) / 1e9
            return {"ms": round(ms, 4), "bytes": nbytes, "GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        extra["hbm_kernels"] = {
            "tensor": list(q.shape), "dtype": w.dtype,
            "kv_avgpool_fwd": {"pool_hw": list(pool), **rate(pool_bytes, pool_ms)},
            "dual_branch_merge": rate(3 * tensor_bytes, gm_ms),
            "dual_branch_merge_lse": rate(3 * tensor_bytes + 2 * lse_bytes, lm_ms)}
        log(f"[bench] HBM kernels: pooling {pool_ms:.3f} ms ({pool_bytes / (pool_ms * 1e-3) / 1e9:.0f} GB/s), "
            f"gated merge {gm_ms:.3f} ms ({3 * tensor_bytes / (gm_ms * 1e-3) / 1e9:.0f} GB/s), "
            f"LSE merge {lm_ms:.3f} ms ({(3 * tensor_bytes + 2 * lse_bytes) / (lm_ms * 1e-3) / 1e9:.0f} GB/s)")
        del o_m, lse_a, lse_b, pooled
    if args.mode_steps > 0 and w.pool_hw is None:
        # the local branch under the other window modes: edge windows moved
        # inward (more attended pairs), and the grid rolled by half a tile
        half = tuple(b // 2 for b in w.tile)
        modes = {}
        for mode, sh in (("inward", w.shifts[0]), ("cyclic", half)):
            ms = timed(lambda: V.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, sh, scale=w.softmax_scale,
                                              out=buf.local[0], window_mode=mode), args.mode_steps)
            mf = V.sta_flops(w.batch, w.heads, w.head_dim, w.grid, w.tile, w.window, sh, window_mode=mode)
            modes[mode] = {"shift": list(sh), "ms_per_call": round(ms, 3), "effective_flop": mf,
                           "tflops": round(mf / (ms * 1e-3) / 1e12, 1)}
            log(f"[bench] window mode {mode} (shift {sh}): {ms:.2f} ms, {mf / (ms * 1e-3) / 1e12:.0f} TFLOP/s")
        extra["window_modes"] = modes
    if args.bwd_steps > 0:
        # backward of the local branch (first lattice shift): dQ, dK, dV from
        # the forward's output and LSE; effective work 10 * head_dim FLOP per
        # attended pair (S, dP, dV, dQ, dK), 2.5x the forward's
        lse_f = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        o_f = V.sta_attn_fwd(q, k, v, w.grid, w.tile, w.window, w.shifts[0], scale=w.softmax_scale, lse=lse_f)[0]
        do = WL.make_tensor(q.shape, q.dtype, dev, seed=99)
        grads = [torch.empty_like(q) for _ in range(3)]
        ws = torch.empty(V.sta_attn_bwd_workspace_size(w.batch, w.heads, w.head_dim, w.grid,
                                                       1 if w.dtype == "bf16" else 0),
                         dtype=torch.uint8, device=dev)
        def bwd():
            V.sta_attn_bwd(q, k, v, o_f, do, lse_f, w.grid, w.tile, w.window, w.shifts[0],
                           scale=w.softmax_scale, dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws)
        bwd()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(args.bwd_steps):
            bwd()
        b1.record(stream)
        torch.cuda.synchronize()
        bwd_ms = b0.elapsed_time(b1) / args.bwd_steps
        bwd_flops = 2.5 * fl["local"] / len(w.shifts)
        extra["backward"] = {"call": "sta_attn_bwd", "ms_per_call": round(bwd_ms, 3),
                             "effective_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 1),
                             "effective_flop_per_call": bwd_flops,
                             "frac_of_peak": round(bwd_flops / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"[bench] backward: {bwd_ms:.2f} ms per call, {bwd_flops / (bwd_ms * 1e-3) / 1e12:.1f} effective TFLOP/s")
        if w.pool_hw is not None:
            # backward of the global branch from its own output and LSE:
            # delta, K/V pooling, the dQ and dK/dV passes over the pooled
            # keys and the pooling gradient; 2.5x the forward's FLOP
            lse_g = torch.empty_like(lse_f)
            o_g = V.global_pooled_attn_fwd(q, k, v, w.grid, w.pool_hw, scale=w.softmax_scale, lse=lse_g)[0]
            ws_g = torch.empty(V.global_pooled_attn_bwd_workspace_size(w.batch, w.heads, w.head_dim, w.grid,
                                                                       w.pool_hw, 1 if w.dtype == "bf16" else 0),
                               dtype=torch.uint8, device=dev)
            gbwd_ms = timed(lambda: V.global_pooled_attn_bwd(q, k, v, o_g, do, lse_g, w.grid, w.pool_hw,
                                                             scale=w.softmax_scale, dq=grads[0], dk=grads[1],
                                                             dv=grads[2], workspace=ws_g), args.bwd_steps)
            gbwd_flops = 2.5 * fl["global"]
            extra["backward_global"] = {"call": "global_pooled_attn_bwd", "ms_per_call": round(gbwd_ms, 3),
                                        "effective_tflops": round(gbwd_flops / (gbwd_ms * 1e-3) / 1e12, 1),
                                        "effective_flop_per_call": gbwd_flops,
                                        "frac_of_peak": round(gbwd_flops / (gbwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
            log(f"[bench] global backward: {gbwd_ms:.2f} ms per call, "
                f"{gbwd_flops / (gbwd_ms * 1e-3) / 1e12:.1f} effective TFLOP/s")
            del o_g, lse_g, ws_g
        del grads, do, o_f, lse_f
    if args.dense_steps > 0 and w.pool_hw is None:
        # the same kernel with a window covering the whole tile lattice = dense attention
        n_tiles = [-(-(L + s) // b) for L, b, s in zip(w.grid, w.tile, w.shifts[0])]
        full = tuple(2 * n - 1 for n in n_tiles)
        V.sta_attn_fwd(q, k, v, w.grid, w.tile, full, scale=w.softmax_scale, out=buf.local[0])
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for _ in range(args.dense_steps):
            V.sta_attn_fwd(q, k, v, w.grid, w.tile, full, scale=w.softmax_scale, out=buf.local[0])
        d1.record(stream)
        torch.cuda.synchronize()
        dense_ms = d0.elapsed_time(d1) / args.dense_steps
        dense_flops = V.sta_flops(w.batch, w.heads, w.head_dim, w.grid, w.tile, full)
        extra["dense_same_kernel"] = {"window": list(full), "ms_per_call": round(dense_ms, 3),
                                      "tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 1),
                                      "speedup_vs_dense": round(dense_ms / launch_ms, 2)}
        log(f"[bench] dense (window {full}): {dense_ms:.2f} ms, speed-up {dense_ms / launch_ms:.2f}x")

    cpu = None
    if args.cpu_seconds > 0:
        log(f"[bench] CPU oracle sample ({args.cpu_seconds:.0f} s budget)")
        cpu = cpu_baseline(w, q, k, v, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "grid": list(w.grid), "tile": list(w.tile), "window": list(w.window),
                   "shifts": [list(s) for s in w.shifts], "pool_hw": w.pool_hw, "batch": w.batch,
                   "heads": w.heads, "head_dim": w.head_dim, "tokens": w.n_tokens,
                   "effective_flop_per_step": step_flops},
        "pct_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "clock": clock,
        "cpu_baseline": cpu,
        **extra,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
