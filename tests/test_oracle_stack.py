"""Pins of the oracle's drafter stack: it is wiring around pieces pinned on
their own (the Mamba-2 block, the block attention, the state projection), so
the pins check the wiring.  Zero output weights leave the residual stream
unchanged; one layer equals the pieces composed here with torch's float64
rms_norm and linear; each attention half reads its own target layer's KV; a
layer sees the previous layer's output; a both-halves layer adds the two
halves' outputs."""
from dataclasses import replace

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from hybrid_mamba_attention_amd import workloads as wl

W = replace(wl.WORKLOADS[0], name="stack-pins", C=2, ctx=("uniform", 0, 40), seed=55)
SH = dict(H=W.H, P=W.P, ng=W.ng, N=W.N, Hq=W.Hq, Hkv=W.Hkv, D=W.D)


def run(a, layers=None):
    return oracle.stack_forward(a["hidden_in"], a["u"], a["layers"] if layers is None else layers,
                                a["page_table"], a["ctx_lens"], dtype=W.dtype, **SH)


def _t(x):
    return torch.from_numpy(np.asarray(x, np.float64))


def test_zero_output_weights_keep_the_stream():
    a = wl.make_stack_inputs(W, ("MA", "M", "A"))
    for L in a["layers"]:
        if "w_out" in L:
            L["w_out"] = np.zeros_like(L["w_out"])
        if "wo" in L:
            L["wo"] = np.zeros_like(L["wo"])
    for h in run(a):
        np.testing.assert_array_equal(h, oracle.decode(a["hidden_in"], W.dtype))


def test_one_layer_is_the_pieces():
    a = wl.make_stack_inputs(W, ("MA",))
    L = a["layers"][0]
    h_in = oracle.decode(a["hidden_in"], W.dtype)
    x = F.rms_norm(_t(h_in), (W.d_model,), weight=_t(L["pre_norm_w"]), eps=L["eps"]).numpy()
    h0 = oracle.init_state(oracle.decode(a["u"], W.dtype), L["w_init"]).reshape(W.C, W.H, W.P, W.N)
    ym = oracle.mamba_block(x, L["w_in"], L["conv_w"], L["conv_b"], L["dt_bias"], L["A"], L["Dskip"],
                            L["norm_w"], L["eps"], L["w_out"], H=W.H, P=W.P, ng=1, N=W.N, h0=h0)["out"]
    lin = lambda v, w: F.linear(_t(v), _t(w)).numpy()
    q = lin(x, L["wq"]).reshape(W.C, W.K, W.Hq, W.D)
    kb = lin(x, L["wk"]).reshape(W.C, W.K, W.Hkv, W.D)
    vb = lin(x, L["wv"]).reshape(W.C, W.K, W.Hkv, W.D)
    o = oracle.block_attention(q, kb, vb, L["k_cache"], L["v_cache"], a["page_table"], a["ctx_lens"],
                               dtype=W.dtype, block_dtype="f64")
    ya = lin(o.reshape(W.C, W.K, -1), L["wo"])
    np.testing.assert_allclose(run(a)[0], h_in + ym + ya, rtol=1e-12, atol=1e-12)


def test_each_attention_half_reads_its_own_target_layer():
    a = wl.make_stack_inputs(W, ("A", "A"))
    base = run(a)[-1]
    swapped = [dict(a["layers"][0]), dict(a["layers"][1])]
    for k in ("k_cache", "v_cache"):
        swapped[0][k], swapped[1][k] = a["layers"][1][k], a["layers"][0][k]
    assert np.abs(run(a, swapped)[-1] - base).max() > 1e-3


def test_layers_are_sequential():
    a = wl.make_stack_inputs(W, ("M", "A"))
    h1, h2 = run(a)
    # layer 2 applied to hidden_in instead of h1 gives something else
    alone = oracle.stack_forward(a["hidden_in"], a["u"], [a["layers"][1]], a["page_table"], a["ctx_lens"],
                                 dtype=W.dtype, **SH)[0]
    assert np.abs((h2 - h1) - (alone - oracle.decode(a["hidden_in"], W.dtype))).max() > 1e-6


def test_both_halves_add():
    a = wl.make_stack_inputs(W, ("MA",))
    L = a["layers"][0]
    m_only = {k: v for k, v in L.items() if k not in ("wq", "wk", "wv", "wo", "k_cache", "v_cache")}
    a_only = {k: v for k, v in L.items() if k not in ("w_init", "w_in", "conv_w", "conv_b", "dt_bias", "A",
                                                      "Dskip", "norm_w", "w_out")}
    h_in = oracle.decode(a["hidden_in"], W.dtype)
    both = run(a)[0] - h_in
    np.testing.assert_allclose(both, (run(a, [m_only])[0] - h_in) + (run(a, [a_only])[0] - h_in),
                               rtol=1e-12, atol=1e-12)
