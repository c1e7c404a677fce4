"""The Mamba-2 block around the scan: input projection, short causal
convolution, gated RMS normalisation and output projection.

H-Spec (Abstract; the review page's Summary) builds its drafter from Mamba-2
modules and attention modules; the pages name Mamba-2 but print none of its
block.  The block here is the Mamba-2 block as Dao & Gu (2024, "Transformers
are SSMs") describe it, written out from that description:

  * one input projection produces, per token and in parallel, the gate z, the
    scan input x, the shared B and C and the raw step size (no bias);
  * x, B and C pass through a depthwise causal convolution of width 4 and a
    SiLU;
  * delta = softplus(dt_raw + dt_bias);  the scan (E2, from the state h0,
    with the skip term) gives y;
  * y is gated by SiLU(z), normalised by its RMS over the d_inner = H*P
    channels of the token and scaled by a learned weight;
  * an output projection (no bias) maps back to d_model.

Readings where the pages (and the Mamba-2 description) leave a choice:
  * the convolution starts at the draft block: positions before the block are
    zero (the pages keep no convolution state);
  * the normalisation spans all d_inner channels of a token (one group);
  * projection weights follow the [out_features, in_features] convention;
    the projection's output rows are ordered z | x | B | C | dt.

Channel layouts: x channel h*P + p is head h, element p; B and C channels are
g*N + n for group g.  Everything is float64.
"""
import numpy as np

from .ssd import ssd_recurrence

D_CONV = 4


def in_proj_sizes(H: int, P: int, ng: int, N: int):
    """(d_inner, conv_dim, d_in_proj) of the block."""
    d_inner = H * P
    conv_dim = d_inner + 2 * ng * N
    return d_inner, conv_dim, 2 * d_inner + 2 * ng * N + H


def silu(v):
    v = np.asarray(v, np.float64)
    return v / (1.0 + np.exp(-v))


def softplus(v):
    """log(1 + e^v), evaluated without overflow."""
    return np.logaddexp(0.0, np.asarray(v, np.float64))


def causal_conv(xr, w, b=None):
    """Depthwise causal convolution along the block.

    xr [C, K, ch], w [ch, 4], b [ch] or None:
        out[:, t, c] = b[c] + sum_j w[c, j] * xr[:, t - 3 + j, c],
    with xr at positions before 0 taken as zero.  Tap 3 is the current token.
    """
    xr = np.asarray(xr, np.float64)
    w = np.asarray(w, np.float64)
    C, K, ch = xr.shape
    out = np.zeros((C, K, ch)) if b is None else np.broadcast_to(np.asarray(b, np.float64), (C, K, ch)).copy()
    for t in range(K):
        for j in range(D_CONV):
            s = t - (D_CONV - 1) + j
            if s >= 0:
                out[:, t, :] += w[None, :, j] * xr[:, s, :]
    return out


def gated_rmsnorm(y, z, weight, eps):
    """g = y * silu(z);  g / sqrt(mean(g^2 over the last axis) + eps) * weight."""
    g = np.asarray(y, np.float64) * silu(z)
    r = 1.0 / np.sqrt(np.mean(g * g, axis=-1, keepdims=True) + eps)
    return g * r * np.asarray(weight, np.float64)


def mamba_block(hidden, w_in, conv_w, conv_b, dt_bias, A, Dskip, norm_w, eps, w_out,
                *, H, P, ng, N, h0=None):
    """One Mamba-2 block over the draft block.

    hidden [C, K, d_model]; w_in [2*H*P + 2*ng*N + H, d_model]; conv_w
    [H*P + 2*ng*N, 4]; conv_b same channels or None; dt_bias, A [H]; Dskip [H]
    or None; norm_w [H*P]; w_out [d_model, H*P]; h0 [C, H, P, N] or None.
    Returns a dict of float64 arrays: zxbcdt (the projection), x, B, Cm,
    delta (scan inputs), y (scan output), normed (normalised gated y),
    out [C, K, d_model] and h_final [C, H, P, N].
    """
    hidden = np.asarray(hidden, np.float64)
    C, K, _ = hidden.shape
    d_inner, conv_dim, d_proj = in_proj_sizes(H, P, ng, N)
    w_in = np.asarray(w_in, np.float64)
    if w_in.shape[0] != d_proj:
        raise ValueError("w_in rows must be 2*H*P + 2*ng*N + H")
    zxbcdt = hidden @ w_in.T                                         # [C, K, d_proj]
    z = zxbcdt[..., :d_inner]
    xbc_raw = zxbcdt[..., d_inner:d_inner + conv_dim]
    dt_raw = zxbcdt[..., d_inner + conv_dim:]
    xbc = silu(causal_conv(xbc_raw, conv_w, conv_b))
    x = xbc[..., :d_inner].reshape(C, K, H, P)
    B = xbc[..., d_inner:d_inner + ng * N].reshape(C, K, ng, N)
    Cm = xbc[..., d_inner + ng * N:].reshape(C, K, ng, N)
    delta = softplus(dt_raw + np.asarray(dt_bias, np.float64)[None, None, :])
    y, h_final = ssd_recurrence(x, delta, A, B, Cm, h0=h0, Dskip=Dskip)
    normed = gated_rmsnorm(y.reshape(C, K, d_inner), z, norm_w, eps)
    out = normed @ np.asarray(w_out, np.float64).T                   # [C, K, d_model]
    return dict(zxbcdt=zxbcdt, x=x, B=B, Cm=Cm, delta=delta, y=y, normed=normed,
                out=out, h_final=h_final)
