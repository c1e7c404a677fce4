"""GPU parity of the drafter stack (hspec_draft_stack) and its HIP-graph form
against the oracle: parallel-hybrid layers (both halves), alternating Mamba /
attention layers, single-half stacks, fp32; every graph replay equals the
eager run, also after the inputs change in place between replays.

The Llama-shaped cases run the stack at the shapes the benchmark times
(d_model 4096, 32 query / 8 kv heads of 128, Mamba-2 16 x 64 x 32): a few
requests with 2k-8k-token contexts (split attention, and the head-pair path
at 256-page splits), and 128 requests with short contexts, where the
projections take the 2048-row tile plans of the benchmark.  Besides the
output stream, the layers' update (output minus input) is compared on its
own: the N(0,1) input stream is carried exactly and would otherwise dilute
the error of everything the GPU rounds to bf16 (normed activations, q/k/v,
attention output, the block's normed activations, both halves' outputs)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from hybrid_mamba_attention_amd import ops
from hybrid_mamba_attention_amd import workloads as wl

from helpers import assert_close, flush, row_errors, to_dev, to_host64

pytestmark = pytest.mark.gpu

W1 = replace(wl.WORKLOADS[1], name="stack-small", C=3, d_model=256, Hq=8, Hkv=2, ctx=("uniform", 0, 300), seed=61)


def build(w, a, kv_split_pages=0):
    dt = w.dtype
    layers = []
    for L in a["layers"]:
        Ld = {}
        for k, v in L.items():
            if k == "eps":
                continue
            Ld[k] = to_dev(v, dt) if v.dtype != np.float32 or k in ("k_cache", "v_cache") else to_dev(v, "f32")
        layers.append(Ld)
    return ops.DraftStack(hidden_in=to_dev(a["hidden_in"], dt), u=to_dev(a["u"], dt), layers=layers,
                          page_table=to_dev(a["page_table"], dt), ctx_lens=to_dev(a["ctx_lens"], dt),
                          max_ctx=int(a["ctx_lens"].max()), H=w.H, P=w.P, N=w.N, chunk=w.chunk, Hq=w.Hq,
                          Hkv=w.Hkv, D=w.D, eps=wl.BLOCK_EPS, kv_split_pages=kv_split_pages)


def oracle_stack(w, a):
    return oracle.stack_forward(a["hidden_in"], a["u"], a["layers"], a["page_table"], a["ctx_lens"],
                                dtype=w.dtype, H=w.H, P=w.P, ng=w.ng, N=w.N, Hq=w.Hq, Hkv=w.Hkv, D=w.D)[-1]


@pytest.mark.parametrize("kinds", [("MA", "MA"), ("M", "A", "M", "A"), ("A",), ("M",)],
                         ids=lambda k: "-".join(k))
def test_stack_parity(kinds):
    flush(f"[stack] {kinds}")
    a = wl.make_stack_inputs(W1, kinds)
    st = build(W1, a)()
    torch.cuda.synchronize()
    assert_close(to_host64(st.hidden_out), oracle_stack(W1, a), "bf16", f"stack {kinds}")


def test_stack_fp32():
    w = replace(wl.WORKLOADS[0], name="stack-f32", C=2, ctx=("uniform", 0, 70), seed=62)
    a = wl.make_stack_inputs(w, ("MA", "A"))
    st = build(w, a)()
    torch.cuda.synchronize()
    assert_close(to_host64(st.hidden_out), oracle_stack(w, a), "f32", "fp32 stack")


def test_graph_replays_match_eager():
    """Replays with eager work between them; the input is changed in place
    between replays, and each replay must equal an eager run on that input."""
    a = wl.make_stack_inputs(W1, ("MA", "M", "A"))
    st = build(W1, a)
    hidden = st._keep[0]
    st()
    torch.cuda.synchronize()
    eager = st.hidden_out.clone()
    st.graph()
    for rep in range(4):
        st.hidden_out.fill_(float("nan"))
        st.launch_graph()
        torch.cuda.synchronize()
        assert torch.equal(st.hidden_out, eager), f"replay {rep}"
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
    g = torch.Generator(device="cuda").manual_seed(5)
    hidden.copy_(torch.randn(hidden.shape, generator=g, device="cuda").to(hidden.dtype))
    st()
    torch.cuda.synchronize()
    eager2 = st.hidden_out.clone()
    assert not torch.equal(eager2, eager)
    for rep in range(2):
        st.hidden_out.zero_()
        st.launch_graph()
        torch.cuda.synchronize()
        assert torch.equal(st.hidden_out, eager2), f"replay {rep} after the input changed"
    del junk


LLAMA = wl.WORKLOADS[3]   # the benchmark's shapes


@pytest.mark.parametrize("C,ctx,split", [(3, (2048, 8192), 0), (3, (2048, 8192), 256), (128, (16, 300), 0)],
                         ids=["c3-ctx2k-8k-auto", "c3-ctx2k-8k-split256", "c128-short-2048rows"])
def test_stack_parity_llama_shapes(C, ctx, split):
    w = replace(LLAMA, name=f"stack-llama-c{C}", C=C, ctx=("uniform",) + ctx, seed=63 + C + split)
    flush(f"[stack] llama shapes C={C} ctx={ctx} split={split}: drawing inputs")
    a = wl.make_stack_inputs(w, ("MA", "MA"))
    st = build(w, a, kv_split_pages=split)()
    torch.cuda.synchronize()
    flush("[stack] oracle")
    want = oracle_stack(w, a)
    got = to_host64(st.hidden_out)
    h_in = oracle.decode(a["hidden_in"], w.dtype)
    rel, mx = assert_close(got, want, "bf16", "stack output")
    urel, umx = assert_close(got - h_in, want - h_in, "bf16", "stack update (output - input)")
    rows, worst = row_errors(got - h_in, want - h_in)
    flush(f"[stack] output rel-L2 {rel:.2e} max-abs {mx:.2e}; update rel-L2 {urel:.2e} max-abs {umx:.2e}, "
          f"worst token row {rows.max():.2e} at {worst}")
    assert rows.max() <= 2e-2, f"update row {worst}: rel-L2 {rows.max():.3e}"
