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
