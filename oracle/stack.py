"""A drafter stack of hybrid layers over the draft block.

H-Spec (Abstract, and the runtime analysis of Figure 8) builds its drafter
from Mamba-2 and attention modules stacked into a backbone, and admits that
the deeper stack drafts slower at low concurrency.  The pages do
not print the stack; the reading here, kept to the pieces defined elsewhere in
this package:

  h = hidden_in                                    (fp64 residual stream)
  for each layer l:
      x  = RMSNorm(h) * pre_norm_w[l]              (over d_model, eps)
      ym = Mamba-2 block of x, from h0 = u . W_init[l]          (if the layer has one)
      ya = (block attention of q, k, v over the target KV of the
            layer's mapped target layer, read in place) . Wo[l]^T (if the layer has one)
           with q = x . Wq[l]^T, k = x . Wk[l]^T, v = x . Wv[l]^T
      h  = h + ym + ya

A layer with both halves is the drafter layer's two complementary modules
side by side; layers with one half each alternate Mamba and attention.
Weights are [out, in]; no RoPE, no bias, no MLP (the pages name none).
"""
import numpy as np

from .attention import block_attention
from .init_state import init_state
from .mamba_block import mamba_block
from .numerics import decode


def rmsnorm(h, w, eps):
    h = np.asarray(h, np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def stack_forward(hidden_in, u, layers, page_table, ctx_lens, *, dtype, H, P, ng, N, Hq, Hkv, D,
                  eps=1e-5, scale=None):
    """hidden_in [C, K, d] and u [C, d] stored activations; layers: list of dicts
    with 'pre_norm_w' and optionally the Mamba half ('w_init' [d, S], 'w_in',
    'conv_w', 'conv_b', 'dt_bias', 'A', 'Dskip', 'norm_w', 'w_out') and the
    attention half ('wq', 'wk', 'wv', 'wo', 'k_cache', 'v_cache').  Stored
    arrays are decoded with `dtype`; fp32 parameters are used as given.
    Returns the fp64 residual stream after every layer: list of [C, K, d]."""
    h = decode(hidden_in, dtype)
    uu = decode(u, dtype)
    C, K, d = h.shape
    outs = []
    for L in layers:
        x = rmsnorm(h, L["pre_norm_w"], eps)
        upd = np.zeros_like(h)
        if L.get("w_in") is not None:
            h0 = init_state(uu, decode(L["w_init"], dtype)).reshape(C, H, P, N)
            r = mamba_block(x, decode(L["w_in"], dtype), L["conv_w"], L.get("conv_b"), L["dt_bias"], L["A"],
                            L.get("Dskip"), L["norm_w"], L["eps"], decode(L["w_out"], dtype),
                            H=H, P=P, ng=ng, N=N, h0=h0)
            upd += r["out"]
        if L.get("wq") is not None:
            q = (x @ decode(L["wq"], dtype).T).reshape(C, K, Hq, D)
            kb = (x @ decode(L["wk"], dtype).T).reshape(C, K, Hkv, D)
            vb = (x @ decode(L["wv"], dtype).T).reshape(C, K, Hkv, D)
            o = block_attention(q, kb, vb, L["k_cache"], L["v_cache"], page_table, ctx_lens,
                                dtype=dtype, scale=scale, block_dtype="f64")
            upd += o.reshape(C, K, Hq * D) @ decode(L["wo"], dtype).T
        h = h + upd
        outs.append(h.copy())
    return outs
