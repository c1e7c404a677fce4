"""E4 / E5: block-query attention over the target's paged KV, read in place.

H-Spec (Abstract; review page, Summary): the drafter's attention modules use
the target model's own KV cache where it lies, so no drafter-side KV cache is
ever built.  The K queries of the draft block attend to the request's whole
target context plus the block's own K keys (read here as no mask inside the
block: every block query sees every context key and every block key).

Definition, per request b and query head i (kv head j = i // G, G = Hq/Hkv):

    Kall = concat(Kctx_b,j, k_blk[b, :, j]),  Vall likewise
    Kctx_b,j[n] = Kc[PT[b, n // 16], n % 16, j]     for n < ctx_b
    o[b, :, i] = softmax(scale * q[b, :, i] @ Kall^T) @ Vall,   scale = 1/sqrt(D)

Pages hold page_size tokens (the pool's second extent; 16 in the workloads,
other sizes are the same tokens laid out in bigger pages).  The split-KV form
below counts its splits in 16-token slabs whatever the page size.

Page reads here are strict: a page-table entry outside the pool, or a NaN in
a token that should be valid, raises PoisonedRead.  The workloads fill spare
pages and the tail slots past ctx_b with NaN, so reading the wrong page or the
wrong slot cannot go unnoticed.

Block-causal variant (block_causal=True): block query t sees every context
key and the block keys s <= t only (mask inside the block); the no-mask form
above is the default reading.

block_attention is the definition.  block_attention_ranges restates it as
split-KV over the work plan of plan.py: each piece of a request's keys yields
a partial (running max m, sum l, unnormalised output); partials merge as
    M = max_s m_s,   o = sum_s e^(m_s - M) O_s / sum_s e^(m_s - M) l_s,
with an empty split contributing m = -inf, l = 0, O = 0.
"""
import numpy as np

from .numerics import decode

PAGE = 16


class PoisonedRead(RuntimeError):
    """The oracle was asked to read a page or slot that holds no valid token."""


def gather_context(cache, page_row, ctx_len: int, j: int, dtype: str) -> np.ndarray:
    """Target keys (or values) of one request and kv head as [ctx_len, D] float64.

    cache: stored pool [num_pages, page_size, Hkv, D] (the page size is the
    pool's second extent, 16 in the workloads); page_row: that request's page
    table row, token n at slot n % page_size of page page_row[n // page_size].
    Reads only the pages and slots that hold valid tokens.
    """
    ctx_len = int(ctx_len)
    P = cache.shape[1]
    D = cache.shape[-1]
    if ctx_len == 0:
        return np.zeros((0, D))
    n_pages = -(-ctx_len // P)
    pages = np.asarray(page_row[:n_pages], dtype=np.int64)
    if len(pages) < n_pages or (pages < 0).any() or (pages >= cache.shape[0]).any():
        raise PoisonedRead(f"page table entry out of range: {pages}")
    rows = np.asarray(cache[pages, :, j, :]).reshape(n_pages * P, D)[:ctx_len]
    rows = decode(rows, dtype)
    if np.isnan(rows).any():
        raise PoisonedRead("read a NaN-poisoned token")
    return rows


def _scale(D, scale):
    return 1.0 / np.sqrt(D) if not scale else float(scale)


def block_mask(K: int, G: int, ctx: int, block_causal: bool) -> np.ndarray:
    """Visibility [K*G, ctx+K] of the keys to the query rows (row r is block
    position r // G): all True, except block keys s > t when block_causal."""
    vis = np.ones((K * G, ctx + K), dtype=bool)
    if block_causal:
        t = np.arange(K * G)[:, None] // G
        s = np.arange(K)[None, :]
        vis[:, ctx:] = s <= t
    return vis


def block_attention(q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_lens, *,
                    dtype: str, scale=None, requests=None, block_causal=False,
                    block_dtype=None) -> np.ndarray:
    """Brute-force attention over (context read through the page table) + block.

    q [C,K,Hq,D], k_blk/v_blk [C,K,Hkv,D] and the caches in stored form
    (q and the block K/V decoded with block_dtype, default dtype).
    Returns o [C,K,Hq,D] float64 (rows of requests not in `requests` stay 0).
    """
    C, K, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    G = Hq // Hkv
    sc = _scale(D, scale)
    out = np.zeros((C, K, Hq, D))
    reqs = range(C) if requests is None else requests
    for b in reqs:
        bd = dtype if block_dtype is None else block_dtype
        qb = decode(q[b], bd)                                          # [K,Hq,D]
        kb = decode(k_blk[b], bd)
        vb = decode(v_blk[b], bd)
        for j in range(Hkv):
            kall = np.concatenate([gather_context(k_cache, page_table[b], ctx_lens[b], j, dtype), kb[:, j]])
            vall = np.concatenate([gather_context(v_cache, page_table[b], ctx_lens[b], j, dtype), vb[:, j]])
            qj = qb[:, j * G:(j + 1) * G, :].reshape(K * G, D)
            s = sc * (qj @ kall.T)                                     # [K*G, ctx+K]
            s = np.where(block_mask(K, G, int(ctx_lens[b]), block_causal), s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[b, :, j * G:(j + 1) * G, :] = (p @ vall).reshape(K, G, D)
    return out


def split_partials(qj, kall, vall, sc, bounds, vis=None):
    """Partials (m [R], l [R], O [R,D]) of query rows qj over key ranges `bounds`;
    vis [R, keys] (optional) hides keys from rows."""
    parts = []
    for lo, hi in bounds:
        R = qj.shape[0]
        if hi <= lo:
            parts.append((np.full(R, -np.inf), np.zeros(R), np.zeros((R, vall.shape[1]))))
            continue
        s = sc * (qj @ kall[lo:hi].T)
        if vis is not None:
            s = np.where(vis[:, lo:hi], s, -np.inf)
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        parts.append((m, p.sum(axis=1), p @ vall[lo:hi]))
    return parts


def merge_partials(parts):
    """Combine split partials into the normalised output [R, D]."""
    ms = np.stack([p[0] for p in parts])                               # [S,R]
    M = ms.max(axis=0)
    w = np.where(np.isneginf(ms), 0.0, np.exp(ms - np.where(np.isneginf(M), 0.0, M)[None]))
    num = sum(w[k][:, None] * parts[k][2] for k in range(len(parts)))
    den = sum(w[k] * parts[k][1] for k in range(len(parts)))
    return num / den[:, None]


def key_index(v: int, ctx: int, K: int) -> int:
    """Position in the concatenated key sequence (context, then block keys) of
    slab boundary v: context slab v starts at token 16v, block slab v - n_b
    (n_b = ceil(ctx/16)) at key ctx + 16 (v - n_b)."""
    n = -(-ctx // PAGE)
    return min(PAGE * v, ctx) if v <= n else ctx + min(PAGE * (v - n), K)


def block_attention_ranges(q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_lens, *, w_max: int,
                           range_pages: int = 0, dtype: str, scale=None, requests=None,
                           block_causal=False) -> np.ndarray:
    """Split-KV restatement of block_attention over the work plan of plan.py:
    each request's keys are cut where the batch's ranges cut them; every
    piece yields a partial (m, l, O), and the pieces merge as in the module
    docstring.  A request inside one range is a single piece."""
    from .plan import range_plan, request_pieces
    C, K, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    G = Hq // Hkv
    sc = _scale(D, scale)
    P = k_cache.shape[1]
    plan = range_plan(ctx_lens, K=K, w_max=w_max, page_size=P, range_pages=range_pages, rows=G * K)
    out = np.zeros((C, K, Hq, D))
    reqs = range(C) if requests is None else requests
    for b in reqs:
        ctx = int(ctx_lens[b])
        L = -(-ctx // PAGE) + -(-K // PAGE)
        bounds = [(key_index(lo, ctx, K), key_index(hi, ctx, K))
                  for _, _, lo, hi in request_pieces(plan, C, b, L)]
        assert bounds[0][0] == 0 and bounds[-1][1] == ctx + K
        assert all(bounds[i][1] == bounds[i + 1][0] for i in range(len(bounds) - 1))
        qb = decode(q[b], dtype)
        kb = decode(k_blk[b], dtype)
        vb = decode(v_blk[b], dtype)
        for j in range(Hkv):
            kall = np.concatenate([gather_context(k_cache, page_table[b], ctx, j, dtype), kb[:, j]])
            vall = np.concatenate([gather_context(v_cache, page_table[b], ctx, j, dtype), vb[:, j]])
            qj = qb[:, j * G:(j + 1) * G, :].reshape(K * G, D)
            vis = block_mask(K, G, ctx, block_causal)
            o = merge_partials(split_partials(qj, kall, vall, sc, bounds, vis))
            out[b, :, j * G:(j + 1) * G, :] = o.reshape(K, G, D)
    return out
