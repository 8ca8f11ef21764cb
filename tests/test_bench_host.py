"""Host-side logic of bench.py that needs no GPU: the kernel-source hash that
decides whether recorded traffic counters still apply, the clock-table
parsing of the clock probe, and the single-GPU guard."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_source_hash_ignores_comments_not_code(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("// header\nint f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n")
    b = tmp_path / "b.hip"
    b.write_text("int f(int x) {   return x + 1; }\n// a different comment\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) { return x + 2; }\n")
    ha, hb, hc = (bench.kernel_sources_hash([str(p)]) for p in (a, b, c))
    assert ha == hb          # comments and blank space do not count
    assert ha != hc          # code does


def test_recorded_traffic_follows_the_gemv_sources():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)["decode_gemv"]
    h = bench.kernel_sources_hash(bench.GEMV_SOURCES)
    if rec["kernel_sources_hash"] == h:
        assert bench.recorded_traffic(h) == rec["hbm_bytes_per_launch"]
    assert bench.recorded_traffic("0" * 16) is None


def test_clock_table_parsing(tmp_path):
    d = tmp_path / "dev"
    d.mkdir()
    (d / "pp_dpm_sclk").write_text("S: 1784Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    assert bench.ClockSampler(str(d))._sclk() == 1784.0
    (d / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 2400Mhz *\n")
    assert bench.ClockSampler(str(d))._sclk() == 2400.0
    (d / "pp_dpm_sclk").write_text("garbage\n")
    assert bench.ClockSampler(str(d))._sclk() is None
    hw = d / "hwmon" / "hwmon0"
    hw.mkdir(parents=True)
    (hw / "power1_input").write_text("714000000\n")
    (d / "pp_dpm_sclk").write_text("S: 2034Mhz *\n")
    with bench.ClockSampler(str(d)) as cs:
        import time
        time.sleep(0.05)
    s = cs.summary()
    assert s["sclk_MHz_median"] == 2034 and s["power_W_median"] == 714.0 and s["samples"] >= 1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
