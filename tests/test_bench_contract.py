"""The bench line's host-side contract (no GPU): the committed HBM-traffic
record belongs to the attention sources as they stand, and the multi-GPU flag
is refused with a message."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_is_reported_only_for_the_sources_it_was_taken_on():
    """bench.py reports `traffic` only while the attention kernel's sources
    hash to the value stored with the counter runs in profiles/; once they
    change, the line carries null until the counters are taken again."""
    bench = load_bench()
    rec = json.load(open(os.path.join(ROOT, "profiles", "k_block_attn_llama8b-bf16-c128-ctx8192_traffic.json")))
    got = bench.traffic_from_profile("llama8b-bf16-c128-ctx8192")
    if rec["source_hash"] == bench.kernel_source_hash():
        assert got == rec["hbm_bytes_per_launch"]
    else:
        assert got is None
    assert 0.99 < rec["hbm_bytes_per_launch"] / rec["kernels"]["k_block_attn"]["algorithmic_bytes"] < 1.1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)
