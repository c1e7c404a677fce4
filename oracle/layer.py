"""The whole drafter layer: E1 -> E2 for the Mamba half, E4 for the attention half.

H-Spec (Abstract): the drafter takes two kinds of target context through two
complementary modules -- the Mamba module starts from the projected last-token
hidden state, the attention module reads the target KV in place.  The layer
here runs both over the same draft block and returns both outputs; the pages
say nothing about residuals, norms or projections between them, and none are
applied.
"""
from .numerics import decode
from .init_state import init_state
from .ssd import ssd_recurrence
from .attention import block_attention


def draft_layer(arrays: dict, ctx_lens, page_table, *, dtype: str, w, scale=None,
                requests=None, with_attention=True, with_mamba=True) -> dict:
    """arrays: the stored inputs (see the workload generator's Inputs.arrays).

    w: workload shapes (C, K, H, P, N, ...).  requests limits the attention
    half to some requests (the Mamba half always covers all of them).
    Returns float64 h0 [C,S], y [C,K,H,P], h_final [C,H,P,N], o [C,K,Hq,D].
    """
    out = {}
    if with_mamba:
        u = decode(arrays["u"], dtype)
        W = decode(arrays["w_init"], dtype)
        h0 = init_state(u, W)
        y, hf = ssd_recurrence(decode(arrays["x"], dtype), arrays["delta"], arrays["A"],
                               decode(arrays["B"], dtype), decode(arrays["Cm"], dtype),
                               h0=h0.reshape(w.C, w.H, w.P, w.N), Dskip=arrays.get("Dskip"))
        out.update(h0=h0, y=y, h_final=hf)
    if with_attention:
        out["o"] = block_attention(arrays["q"], arrays["k_blk"], arrays["v_blk"],
                                   arrays["k_cache"], arrays["v_cache"], page_table, ctx_lens,
                                   dtype=dtype, scale=scale, requests=requests)
    return out
