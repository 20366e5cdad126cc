"""CPU checks of bench.py that need no GPU: a request for more than one GPU
exits with a message (the library has no multi-GPU path), and the committed
HBM-traffic counters of the grouped gate/up GEMM still belong to the GEMM
sources in the tree (bench.py reports `roofline.traffic` only while the
sources hash to the value recorded beside the counters; a change to the GEMM
without re-taking them would turn the field into null)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_counters_match_the_gemm_sources():
    b = _bench()
    t = b.measured_traffic()
    assert t is not None, "GEMM sources changed since profiles/moe_decode_t32_hbm_traffic.md"
    assert 2.4e9 < t < 2.6e9
