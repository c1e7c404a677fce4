"""Shared test plumbing: moving seeded host arrays to the GPU and comparing
HIP outputs with the oracle under the stated tolerances.

Tolerances (per output tensor, over all compared elements):
  fp32 workloads:  relative L2 error <= 1e-5
  bf16 workloads:  relative L2 error <= 1e-2 and max |error| <= 3e-2
(bf16 inputs, fp32 accumulation; the attention output is itself bf16).

Attention outputs are also compared row by row (one row = one request, block
position and query head, D values): every row's relative L2 error must stay
within ROW_REL.  |o| is only ~0.02-0.2, so one wrong row (a wrong page, head
or split) could hide under the whole-tensor bounds, but not under this one.
The bf16 bound, 2e-2, is twice the tensor bound: a row's error is the bf16
rounding of its D outputs and of the probabilities (~2^-9 relative each),
measured at ~2e-3 over whole tensors.
"""
import numpy as np
import torch

import oracle

TOL = {"f32": dict(rel=1e-5, abs=None), "bf16": dict(rel=1e-2, abs=3e-2)}
ROW_REL = {"f32": 1e-4, "bf16": 2e-2}


def flush(msg: str):
    print(msg, flush=True)


def to_dev(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Stored host array -> device tensor of the activation type (bf16 from its bits)."""
    if arr.dtype == np.uint16:
        assert dtype == "bf16"
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    if arr.dtype == np.int32:
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    diff = got - want
    den = np.linalg.norm(want)
    rel = np.linalg.norm(diff) / (den if den > 0 else 1.0)
    return float(rel), float(np.abs(diff).max()) if diff.size else 0.0


def assert_close(got, want, dtype: str, what: str):
    rel, mx = errors(got, want)
    t = TOL[dtype]
    ok = rel <= t["rel"] and (t["abs"] is None or mx <= t["abs"])
    assert np.isfinite(np.asarray(got, np.float64)).all(), f"{what}: non-finite output"
    assert ok, f"{what}: rel-L2 {rel:.3e} max-abs {mx:.3e} exceeds {t}"
    return rel, mx


def row_errors(got, want):
    """Relative L2 error of every row (last axis) and the row index of the worst."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    num = np.linalg.norm(got - want, axis=-1)
    den = np.linalg.norm(want, axis=-1)
    rel = num / np.maximum(den, 1e-30)
    worst = np.unravel_index(int(np.argmax(rel)), rel.shape) if rel.size else ()
    return rel, worst


def assert_attn_close(got, want, dtype: str, what: str):
    """assert_close over the whole tensor, then every row [..., D] on its own."""
    res = assert_close(got, want, dtype, what)
    rel, worst = row_errors(got, want)
    if rel.size:
        assert rel.max() <= ROW_REL[dtype], (
            f"{what}: row {tuple(int(i) for i in worst)} rel-L2 {rel.max():.3e} exceeds {ROW_REL[dtype]}")
    return res


def layer_from_inputs(inp, *, kv_split_pages=0, want_final=True, with_dskip=False,
                      block_causal=False, no_init=False):
    """Build and run one drafter-layer call on the GPU for a workload's inputs
    (no_init: the direct-reuse-only ablation, u = w_init = None)."""
    from hybrid_mamba_attention_amd import ops
    w, a = inp.w, inp.arrays
    dt = w.dtype
    layer = ops.DraftLayer(
        u=None if no_init else to_dev(a["u"], dt),
        w_init=None if no_init else to_dev(a["w_init"], dt), x=to_dev(a["x"], dt),
        delta=to_dev(a["delta"], dt), A=to_dev(a["A"], dt), B=to_dev(a["B"], dt),
        Cm=to_dev(a["Cm"], dt), chunk=w.chunk, q=to_dev(a["q"], dt), k_blk=to_dev(a["k_blk"], dt),
        v_blk=to_dev(a["v_blk"], dt), k_cache=to_dev(a["k_cache"], dt),
        v_cache=to_dev(a["v_cache"], dt), page_table=to_dev(inp.page_table, dt),
        ctx_lens=to_dev(inp.ctx_lens, dt), max_ctx=inp.max_ctx, kv_split_pages=kv_split_pages,
        block_causal=block_causal, Dskip=to_dev(a["Dskip"], dt) if with_dskip else None,
        want_final=want_final)
    layer()
    torch.cuda.synchronize()
    return layer


def oracle_h0(inp, col_block=16384):
    """Oracle projection computed in column blocks (bounded host memory)."""
    w, a = inp.w, inp.arrays
    u = oracle.decode(a["u"], w.dtype)
    out = np.empty((w.C, w.S))
    for c0 in range(0, w.S, col_block):
        out[:, c0:c0 + col_block] = oracle.init_state(u, oracle.decode(a["w_init"][:, c0:c0 + col_block], w.dtype))
    return out


def oracle_scan(inp, h0):
    w, a = inp.w, inp.arrays
    return oracle.ssd_recurrence(oracle.decode(a["x"], w.dtype), a["delta"], a["A"],
                                 oracle.decode(a["B"], w.dtype), oracle.decode(a["Cm"], w.dtype),
                                 h0=h0.reshape(w.C, w.H, w.P, w.N), Dskip=a.get("Dskip"))


def oracle_attn(inp, requests=None, **kw):
    w, a = inp.w, inp.arrays
    return oracle.block_attention(a["q"], a["k_blk"], a["v_blk"], a["k_cache"], a["v_cache"],
                                  inp.page_table, inp.ctx_lens, dtype=w.dtype, requests=requests, **kw)
