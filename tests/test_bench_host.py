"""Host-side logic of bench.py (no GPU): the flop counts, the clock scaling,
the traffic summary's source check and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_causal_flops_counts_half_the_square():
    # 4 T^2 d Hq / 2: two products of 2 d flop per (query, key) pair, T^2/2 pairs
    assert bench.causal_flops(4096, 32) == 68719476736.0
    assert bench.causal_flops(2, 1, d=1) == 8.0


def test_backward_flops_are_five_products():
    assert bench.backward_flops(4096, 32) == 2.5 * bench.causal_flops(4096, 32)


def test_clock_fields_scale_the_peak_to_the_measured_clock():
    out = bench.clock_fields({"gfx_mhz": 1200.0, "samples": 3, "source": "x"}, 629.15)
    assert out["peak_at_clock"] == pytest.approx(bench.PEAK_FP16_TFLOPS / 2, abs=0.05)
    assert out["frac_at_clock"] == pytest.approx(0.5, abs=1e-4)
    assert out["samples"] == 3 and out["source"] == "x"
    assert bench.clock_fields(None, 100.0) is None


def test_traffic_summary_matches_the_kernel_source():
    # the committed counter summary is used only while its source hash matches
    got = bench.measured_traffic()
    assert got is not None, "profiles/ traffic summary is stale or missing"
    assert 42467328 <= got <= 1.05 * 42467328


def test_counter_summary_matches_the_kernel_source():
    got = bench.measured_utilisation()
    assert got is not None, "profiles/ SQ counter summary is stale or missing"
    assert 0.0 < got["mfma_busy"] < 1.0 and 0.0 < got["valu_active"] < 1.0


def test_backward_traffic_summary_matches_the_kernel_source():
    got = bench.measured_traffic(bench.BWD_TRAFFIC_FILE, bench.BWD_KERNEL_SRC)
    assert got is not None, "profiles/ backward traffic summary is stale or missing"
    assert 193986560 <= got <= 1.05 * 193986560


def test_backward_counter_summary_matches_the_kernel_source():
    got = bench.measured_utilisation_backward()
    assert got is not None, "profiles/ backward SQ counter summary is stale or missing"
    assert 0.0 < got["mfma_busy"] < 1.0 and 0.0 < got["valu_active"] < 1.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_sha_ignores_comments_but_not_code(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("// header\nint f(int x) {  /* note */\n  return x + 1;  // one\n}\n")
    b.write_text("int f(int x)\n{\n  return x + 1;\n}\n// trailing remark\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_sha(str(a)) == bench.kernel_sha(str(b))
    assert bench.kernel_sha(str(a)) != bench.kernel_sha(str(c))
