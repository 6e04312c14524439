"""Host logic of bench.py that runs without a GPU: the multi-GPU refusal,
the counter-summary reader and the clock parser."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_only_for_matching_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "counters.md"
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(f))
    assert bench.measured_traffic() is None          # no summary
    f.write_text(f"traffic_bytes_per_launch: 1234567\nkernel_source_sha256_16: {bench.kernel_source_hash()}\n")
    assert bench.measured_traffic() == 1234567.0
    f.write_text("traffic_bytes_per_launch: 1234567\nkernel_source_sha256_16: 0000000000000000\n")
    assert bench.measured_traffic() is None          # taken on other source


def test_parse_gfx_clocks():
    text = """GPU: 0
    CLOCK:
        GFX_0:
            CLK: 2056 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 2008 MHz
            MIN_CLK: 500 MHz
        MEM_0:
            CLK: 2000 MHz
"""
    assert bench.parse_gfx_clocks(text) == [2056, 2008]
    assert bench.parse_gfx_clocks("no clocks here") == []


def test_cpu_baseline_fields_on_a_small_workload():
    # the oracle on whole query tiles, in worker processes, on the host
    from video_dit_sparse_amd import workloads as WL
    w = WL.Workload("small_sparse", (4, 8, 12), heads=3, head_dim=64, dtype="bf16", tile=(2, 4, 4),
                    window=(1, 1, 3))
    q, k, v = WL.make_qkv(w, "cpu")
    r = bench.cpu_baseline(w, q, k, v, 0.3, n_heads=2)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert 1 <= r["cores"] <= min(16, r["cpus_available"]) and r["nproc"] == os.cpu_count()
    assert r["cpu_model"] and "whole query tiles" in r["sample"]
    assert r["effective_flop_done"] > 0 and r["extrapolated_full_call_s"] > 0


def test_roofline_bound_by_flop_per_byte():
    # 720P call: 16.583 TFLOP over 2.831 GB compulsory (5,857 FLOP/B) is
    # matrix-core bound; a 2K window-1 call, 0.601 TFLOP over 4.955 GB
    # (121 FLOP/B), is HBM bound; the fp32 path is vector-ALU bound
    r = bench.roofline_of("bf16", 16.583e12, 2.831e9, 14.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["achieved"] - 16.583e12 / 14e-3 / 1e12) < 0.01 and abs(r["frac"] - r["achieved"] / 2500.0) < 1e-4
    r = bench.roofline_of("bf16", 0.601e12, 4.955e9, 1.3)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - 4.955e9 / 1.3e-3 / 1e9) < 0.01
    r = bench.roofline_of("f32", 33.6e6, 0.52e6, 0.01)
    assert r["bound"] == "alu" and r["peak"] == 157.3
    # the ridge itself (312.5 FLOP/B) counts as matrix-core bound
    assert bench.roofline_of("bf16", 312.5e9, 1e9, 1.0)["bound"] == "mfma"
    assert bench.roofline_of("bf16", 312.4e9, 1e9, 1.0)["bound"] == "hbm"
