"""Pins of the oracle's Mamba-2 block periphery (CPU only).

Each piece is checked against something other than itself: torch's own
conv1d / silu / softplus / rms_norm / linear in float64 (library routines
that state the same definitions independently), impulse responses of the
convolution, closed forms of the scan under constant inputs (which tell the
B and C channel slices apart), and exact zeros.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from hybrid_mamba_attention_amd import workloads as wl


def _t(a):
    return torch.from_numpy(np.asarray(a, np.float64))


@pytest.mark.parametrize("K", [1, 2, 3, 4, 7, 16])
def test_causal_conv_matches_torch_conv1d(K):
    g = np.random.default_rng(K)
    C, ch = 3, 10
    xr = g.standard_normal((C, K, ch))
    w = g.standard_normal((ch, 4))
    b = g.standard_normal(ch)
    got = oracle.causal_conv(xr, w, b)
    # torch: [C, ch, K] input, depthwise weight [ch, 1, 4], left padding 3 = causal
    want = F.conv1d(F.pad(_t(xr).permute(0, 2, 1), (3, 0)), _t(w)[:, None, :], _t(b), groups=ch)
    np.testing.assert_allclose(got, want.permute(0, 2, 1).numpy(), rtol=1e-13, atol=1e-13)


def test_causal_conv_impulses():
    g = np.random.default_rng(1)
    xr = g.standard_normal((2, 9, 5))
    w = np.zeros((5, 4))
    w[:, 3] = 1.0                                # current token only: identity
    np.testing.assert_array_equal(oracle.causal_conv(xr, w), xr)
    w = np.zeros((5, 4))
    w[:, 0] = 1.0                                # three tokens back, zeros before the block
    got = oracle.causal_conv(xr, w)
    np.testing.assert_array_equal(got[:, :3], 0.0)
    np.testing.assert_array_equal(got[:, 3:], xr[:, :-3])
    b = g.standard_normal(5)
    np.testing.assert_array_equal(oracle.causal_conv(np.zeros_like(xr), g.standard_normal((5, 4)), b),
                                  np.broadcast_to(b, xr.shape))


def test_activations_match_torch_and_closed_values():
    v = np.linspace(-30, 30, 241)
    np.testing.assert_allclose(oracle.silu(v), F.silu(_t(v)).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(oracle.softplus(v), F.softplus(_t(v), threshold=1e9).numpy(), rtol=1e-14)
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    assert oracle.softplus(800.0) == 800.0                          # no overflow
    assert oracle.softplus(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-12)
    assert oracle.silu(0.0) == 0.0 and oracle.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)))


def test_gated_rmsnorm_matches_torch_and_closed_form():
    g = np.random.default_rng(2)
    y, z = g.standard_normal((3, 4, 64)), g.standard_normal((3, 4, 64))
    wt = 1.0 + 0.1 * g.standard_normal(64)
    want = F.rms_norm(_t(y) * F.silu(_t(z)), (64,), weight=_t(wt), eps=1e-5)
    np.testing.assert_allclose(oracle.gated_rmsnorm(y, z, wt, 1e-5), want.numpy(), rtol=1e-13, atol=1e-14)
    # a constant gated row c normalises to c / sqrt(c^2 + eps)
    c, eps = 0.7, 1e-3
    zz = np.full((1, 8), 2.0)
    yy = np.full((1, 8), c / oracle.silu(2.0))
    np.testing.assert_allclose(oracle.gated_rmsnorm(yy, zz, np.ones(8), eps), c / math.sqrt(c * c + eps), rtol=1e-14)
    # with eps = 0 the result does not depend on the scale of y
    np.testing.assert_allclose(oracle.gated_rmsnorm(5.0 * y, z, wt, 0.0), oracle.gated_rmsnorm(y, z, wt, 0.0),
                               rtol=1e-13)


def _block(w, a, **kw):
    dec = lambda k: oracle.decode(a[k], w.dtype)
    return oracle.mamba_block(dec("hidden"), dec("w_in"), a["conv_w"], a["conv_b"], a["dt_bias"], a["A"],
                              a.get("Dskip"), a["norm_w"], a["eps"], dec("w_out"),
                              H=w.H, P=w.P, ng=w.ng, N=w.N, h0=a.get("h0"), **kw)


def test_block_matches_torch_composition():
    """The block against torch's linear / conv1d / silu / softplus / rms_norm
    around the (separately pinned) scan recurrence."""
    w = wl.WORKLOADS[0]
    a = wl.make_block_inputs(w)
    got = _block(w, a)
    d_inner, conv_dim, d_proj = wl.block_sizes(w)
    hid = _t(a["hidden"])
    zxbcdt = F.linear(hid, _t(a["w_in"]))
    z, xbc, dt = torch.split(zxbcdt, [d_inner, conv_dim, w.H], dim=-1)
    xbc = F.conv1d(F.pad(xbc.permute(0, 2, 1), (3, 0)), _t(a["conv_w"])[:, None, :], _t(a["conv_b"]),
                   groups=conv_dim)
    xbc = F.silu(xbc).permute(0, 2, 1)
    x, B, Cm = torch.split(xbc, [d_inner, w.N, w.N], dim=-1)
    delta = F.softplus(dt + _t(a["dt_bias"]), threshold=1e9)
    C, K = w.C, w.K
    y, hf = oracle.ssd_recurrence(x.reshape(C, K, w.H, w.P).numpy(), delta.numpy(), a["A"],
                                  B.reshape(C, K, 1, w.N).numpy(), Cm.reshape(C, K, 1, w.N).numpy(),
                                  h0=a["h0"], Dskip=a["Dskip"])
    normed = F.rms_norm(_t(y).reshape(C, K, d_inner) * F.silu(z), (d_inner,), weight=_t(a["norm_w"]),
                        eps=a["eps"])
    out = F.linear(normed, _t(a["w_out"]))
    np.testing.assert_allclose(got["zxbcdt"], zxbcdt.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["delta"], delta.numpy(), rtol=1e-12)
    np.testing.assert_allclose(got["y"], y, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(got["h_final"], hf, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(got["out"], out.numpy(), rtol=1e-10, atol=1e-10)


def test_zero_input_zero_state_gives_zero_output():
    w = wl.WORKLOADS[0]
    a = wl.make_block_inputs(w, with_h0=False)
    a["hidden"] = np.zeros_like(a["hidden"])
    a["conv_b"] = np.zeros_like(a["conv_b"])
    r = _block(w, a)
    assert np.all(r["x"] == 0) and np.all(r["y"] == 0) and np.all(r["out"] == 0)


def test_constant_inputs_closed_form_scan():
    """hidden = 0: every position sees x = silu(b_x), B = silu(b_B), C = silu(b_C)
    and delta = softplus(dt_bias), so with a = exp(delta*A)
        H_t = a^(t+1) h0 + delta * x (outer) B * (1 - a^(t+1)) / (1 - a)
        y_t = H_t @ C + D * x.
    h0 pairs with C alone, which tells the B and C slices apart."""
    w = wl.WORKLOADS[0]
    a = wl.make_block_inputs(w)
    a["hidden"] = np.zeros_like(a["hidden"])
    r = _block(w, a)
    d_inner = w.H * w.P
    sb = oracle.silu(np.asarray(a["conv_b"], np.float64))
    x = sb[:d_inner].reshape(w.H, w.P)
    Bv, Cv = sb[d_inner:d_inner + w.N], sb[d_inner + w.N:]
    dlt = oracle.softplus(np.asarray(a["dt_bias"], np.float64))
    av = np.exp(dlt * np.asarray(a["A"], np.float64))
    h0 = np.asarray(a["h0"], np.float64)[0]
    for t in range(w.K):
        p = av ** (t + 1)
        Ht = p[:, None, None] * h0 + (dlt * (1 - p) / (1 - av))[:, None, None] * x[:, :, None] * Bv[None, None, :]
        yt = Ht @ Cv + np.asarray(a["Dskip"], np.float64)[:, None] * x
        np.testing.assert_allclose(r["y"][0, t], yt, rtol=1e-11, atol=1e-12)


def test_out_is_linear_in_w_out_and_norm_weight():
    w = wl.WORKLOADS[0]
    a = wl.make_block_inputs(w)
    r1 = _block(w, a)
    b = dict(a, norm_w=3.0 * np.asarray(a["norm_w"], np.float64))
    np.testing.assert_allclose(_block(w, b)["out"], 3.0 * r1["out"], rtol=1e-12, atol=1e-12)
    c = dict(a, w_out=-2.0 * np.asarray(a["w_out"], np.float64))
    np.testing.assert_allclose(_block(w, c)["out"], -2.0 * r1["out"], rtol=1e-12, atol=1e-12)
