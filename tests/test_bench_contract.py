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


def test_roofline_bytes_match_the_hand_counts():
    """The roofline numerators of the 128-request, 8192-token workload, counted
    by hand from its shapes (bf16, 8 kv heads of 128, 32 query heads, K = 16,
    d_model 4096, state 16 x 64 x 32): attention = KV read in place
    (128 x 8192 tokens x 8 heads x 128 x 2 tensors x 2 B) + q and out
    (2 x 128 x 16 x 32 x 128 x 2 B) + block K/V (2 x 128 x 16 x 8 x 128 x 2 B);
    projection = W (4096 x 32768 x 2 B) + u (128 x 4096 x 2 B) + h0
    (128 x 32768 x 4 B); scan = h0 in + x (bf16) and y (fp32) + B and Cm +
    the step sizes."""
    import numpy as np
    bench = load_bench()
    sys.path.insert(0, ROOT)
    from hybrid_mamba_attention_amd import workloads as wl
    w = wl.WORKLOADS[3]
    ctx = np.full(w.C, 8192, np.int64)
    kv = 128 * 8192 * 8 * 128 * 2 * 2
    assert kv == 4_294_967_296
    assert bench.attention_bytes(w, ctx) == kv + 2 * 128 * 16 * 32 * 128 * 2 + 2 * 128 * 16 * 8 * 128 * 2 \
        == 4_336_910_336
    assert bench.init_bytes(w) == 4096 * 32768 * 2 + 128 * 4096 * 2 + 128 * 32768 * 4 == 286_261_248
    assert bench.ssd_bytes(w) == (128 * 32768 * 4 + 128 * 16 * 16 * 64 * (2 + 4) + 2 * 128 * 16 * 1 * 32 * 2
                                  + 128 * 16 * 16 * 4) == 29_753_344
