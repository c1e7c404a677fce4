"""GPU parity: the HIP path (through the C ABI) against the float64 oracle's
whole drafter layer (oracle.draft_layer) on the same seeded inputs, for all
five drafter-layer workloads.

Workloads 0-2 are compared element by element on every output.  Workloads 3
and 4 (full size, launch configuration as benchmarked) are compared in full on
the projection and the scan, and on a seeded sample of requests for the
attention output, which the oracle computes one request at a time.  Attention
outputs are also checked row by row (per request, block position and head).
"""
import numpy as np
import pytest

import oracle
from hybrid_mamba_attention_amd import workloads as wl

from helpers import assert_attn_close, assert_close, flush, layer_from_inputs, to_host64

pytestmark = pytest.mark.gpu


def _check_layer(idx, sample_requests=None):
    w = wl.WORKLOADS[idx]
    flush(f"[parity] workload {idx} {w.name}: drawing inputs")
    inp = wl.make_inputs(w)
    flush(f"[parity] workload {idx}: running the layer on the GPU (max_ctx={inp.max_ctx})")
    layer = layer_from_inputs(inp)
    reqs = sample_requests(inp) if sample_requests else None
    flush(f"[parity] workload {idx}: oracle layer (attention requests: {'all' if reqs is None else reqs})")
    ref = oracle.draft_layer(inp.arrays, inp.ctx_lens, inp.page_table, dtype=w.dtype, w=w, requests=reqs)
    res = {"h0": assert_close(to_host64(layer.h0), ref["h0"], w.dtype, f"w{idx} h0"),
           "y": assert_close(to_host64(layer.y), ref["y"], w.dtype, f"w{idx} y"),
           "h_final": assert_close(to_host64(layer.h_final), ref["h_final"], w.dtype, f"w{idx} h_final")}
    got, o = to_host64(layer.out), ref["o"]
    if reqs is not None:
        got, o = got[reqs], o[reqs]
    res["out"] = assert_attn_close(got, o, w.dtype, f"w{idx} attention out")
    flush(f"[parity] workload {idx}: " + ", ".join(f"{k} rel-L2 {v[0]:.2e} max-abs {v[1]:.2e}"
                                                   for k, v in res.items()))
    # the int32 work plan at the head of the workspace, bit for bit (the
    # capacity w_max is the host's sizing bound, read from the plan)
    plan = layer.plan().cpu().numpy()
    want = oracle.range_plan(inp.ctx_lens, K=w.K, w_max=int(plan[3]), rows=(w.Hq // w.Hkv) * w.K)
    assert np.array_equal(plan, want), "work plan differs from the oracle planner"
    flush(f"[parity] workload {idx}: ok")


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_workload_parity_full(idx):
    _check_layer(idx)


def _sample(inp):
    g = np.random.default_rng(7)
    ctx = inp.ctx_lens
    picks = {int(np.argmax(ctx)), int(np.argmin(ctx)), 0, len(ctx) - 1}
    picks |= set(int(i) for i in g.choice(len(ctx), size=2, replace=False))
    return sorted(picks)


@pytest.mark.parametrize("idx", [3, 4])
def test_workload_parity_full_size_sampled(idx):
    _check_layer(idx, sample_requests=_sample)
