"""Drafter-side KV injection: the cost H-Spec removes (contrast workload).

H-Spec, Abstract, Table 1 and Figure 3: the parallel drafters the pages
compare against project the target's hidden state at every input
position into a drafter-side KV cache of their own, which adds KV memory per
token and an injection step whose time grows with concurrency.  H-Spec reads
the target's KV in place instead, so it never runs this step.  The pages give
no formula for the injection; the plainest reading, used here, is one
bias-free linear projection per drafter layer followed by a write into a
paged cache laid out like the target's:

    kv[b, i, :] = w_kv . hidden[b, i, :]             (w_kv is [2*Hkv*D, d_model])
    K rows are kv[..., :Hkv*D], V rows kv[..., Hkv*D:], head h at columns h*D .. h*D+D-1
    position p = start[b] + i  ->  page page_table[b, p // P], slot p % P
    (P = tokens per page, the pools' second extent)

Everything else in the pools is left as it was.  float64 throughout; the
returned pools hold float64 values (the caller compares written slots within
the tolerance and untouched ones exactly).
"""
import numpy as np

from .numerics import decode

PAGE = 16


def kv_project(hidden, w_kv):
    """[C, n, d] x [2*Hkv*D, d] -> [C, n, 2*Hkv*D] in float64."""
    return np.asarray(hidden, np.float64) @ np.asarray(w_kv, np.float64).T


def kv_inject(hidden, w_kv, k_cache, v_cache, page_table, start, *, Hkv: int, D: int, dtype: str):
    """Return (k_pool, v_pool, kv): float64 copies of the pools with the new
    positions written, and the projected rows [C, n, 2*Hkv*D].

    hidden [C, n, d] and w_kv are stored activations (decoded here); the pools
    are stored arrays [pages, P, Hkv, D] (NHD)."""
    kv = kv_project(decode(hidden, dtype), decode(w_kv, dtype))
    kp = decode(k_cache, dtype).copy()
    vp = decode(v_cache, dtype).copy()
    C, n, _ = kv.shape
    HD = Hkv * D
    P = kp.shape[1]
    for b in range(C):
        for i in range(n):
            p = int(start[b]) + i
            page = int(page_table[b, p // P])
            slot = p % P
            kp[page, slot] = kv[b, i, :HD].reshape(Hkv, D)
            vp[page, slot] = kv[b, i, HD:].reshape(Hkv, D)
    return kp, vp, kv


def extra_kv_bytes_per_token(Hkv: int, D: int, elem_bytes: int, layers: int = 1) -> int:
    """KV bytes a drafter-side cache adds per context token (K and V, per layer)."""
    return 2 * Hkv * D * elem_bytes * layers
