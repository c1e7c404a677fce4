"""Pins for the oracle's in-place paged block attention (E4) and its split-KV
restatement (E5): a hand-worked example, torch's own scaled-dot-product
attention on explicitly concatenated K/V, closed forms, invariances and the
strict (poison-aware) page reads."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

PAGE = 16


def _paged(ctx_lens, Hkv, D, seed, *, spare=5, identity=False, K=3, Hq=None):
    """Logical per-request context (float32) scattered into a NaN-poisoned pool."""
    g = np.random.default_rng(seed)
    Hq = Hq or 2 * Hkv
    C = len(ctx_lens)
    n_pages = [-(-c // PAGE) for c in ctx_lens]
    pool = sum(n_pages) + spare
    perm = np.arange(pool) if identity else np.random.default_rng(seed + 7919).permutation(pool)
    kc = np.full((pool, PAGE, Hkv, D), np.nan, dtype=np.float32)
    vc = np.full_like(kc, np.nan)
    pt = np.full((C, max(1, max(n_pages))), -1, dtype=np.int32)
    kctx, vctx = [], []
    off = 0
    for b, c in enumerate(ctx_lens):
        kl = g.standard_normal((c, Hkv, D)).astype(np.float32)
        vl = g.standard_normal((c, Hkv, D)).astype(np.float32)
        pages = perm[off:off + n_pages[b]]
        off += n_pages[b]
        pt[b, :len(pages)] = pages
        for n in range(c):
            kc[pages[n // PAGE], n % PAGE] = kl[n]
            vc[pages[n // PAGE], n % PAGE] = vl[n]
        kctx.append(kl)
        vctx.append(vl)
    q = g.standard_normal((C, K, Hq, D)).astype(np.float32)
    kb = g.standard_normal((C, K, Hkv, D)).astype(np.float32)
    vb = g.standard_normal((C, K, Hkv, D)).astype(np.float32)
    return dict(q=q, k_blk=kb, v_blk=vb, k_cache=kc, v_cache=vc, page_table=pt,
                ctx_lens=np.array(ctx_lens, np.int32), kctx=kctx, vctx=vctx)


def _run(d, **kw):
    return oracle.block_attention(d["q"], d["k_blk"], d["v_blk"], d["k_cache"], d["v_cache"],
                                  d["page_table"], d["ctx_lens"], dtype="f32", **kw)


def _close(a, b, tol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert np.abs(a - b).max() <= tol * max(1.0, np.abs(b).max()), np.abs(a - b).max()


def test_golden_hand(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "attn_hand.json")))
    pool = g["pool_pages"]
    kc = np.full((pool, PAGE, 1, 2), np.nan, np.float32)
    vc = np.full_like(kc, np.nan)
    kc[g["page_of_context"], 0, 0] = g["k_ctx"][0]
    vc[g["page_of_context"], 0, 0] = g["v_ctx"][0]
    pt = np.array([[g["page_of_context"]]], np.int32)
    o = oracle.block_attention(np.array(g["q"], np.float32), np.array(g["k_blk"], np.float32),
                               np.array(g["v_blk"], np.float32), kc, vc, pt, np.array([g["ctx_len"]]),
                               dtype="f32", scale=math.log(3.0))
    _close(o, g["o"], 1e-14)
    # one-granule ranges: the context token and the block token in one piece
    o2 = oracle.block_attention_ranges(np.array(g["q"], np.float32), np.array(g["k_blk"], np.float32),
                                       np.array(g["v_blk"], np.float32), kc, vc, pt,
                                       np.array([g["ctx_len"]]), w_max=4, range_pages=1, dtype="f32",
                                       scale=math.log(3.0))
    _close(o2, g["o"], 1e-14)


@pytest.mark.parametrize("ctx_lens,Hkv,G", [([37, 16, 5], 2, 2), ([64, 1], 1, 1), ([0, 20], 2, 4)])
def test_matches_torch_sdpa_on_concatenated_kv(ctx_lens, Hkv, G):
    D, K = 8, 3
    d = _paged(ctx_lens, Hkv, D, seed=sum(ctx_lens) + G, Hq=G * Hkv, K=K)
    o = _run(d)
    for b, c in enumerate(ctx_lens):
        kall = np.concatenate([d["kctx"][b], d["k_blk"][b]])          # [c+K, Hkv, D]
        vall = np.concatenate([d["vctx"][b], d["v_blk"][b]])
        qt = torch.from_numpy(d["q"][b].astype(np.float64)).permute(1, 0, 2)[None]   # [1,Hq,K,D]
        kt = torch.from_numpy(kall.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        vt = torch.from_numpy(vall.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0].permute(1, 0, 2).numpy()
        _close(o[b], ref)


def test_scrambled_equals_identity_page_table():
    a = _paged([50, 33, 16], 2, 8, seed=3)
    b = _paged([50, 33, 16], 2, 8, seed=3, identity=True)
    assert not np.array_equal(a["page_table"], b["page_table"])
    for k in ("q", "k_blk", "v_blk"):
        assert np.array_equal(a[k], b[k])
    _close(_run(a), _run(b))


@pytest.mark.parametrize("w_max,range_pages", [(64, 0), (3, 0), (1, 0), (1000, 1), (1000, 2), (1000, 7)])
def test_split_invariance(w_max, range_pages):
    """Cut where the batch's work ranges cut the keys (pieces of one or more
    slabs, cuts inside a context and at the context / block boundary), the
    merged partials equal the unsplit attention."""
    d = _paged([100, 0, 16, 17, 250], 2, 8, seed=4)
    ref = _run(d)
    o = oracle.block_attention_ranges(d["q"], d["k_blk"], d["v_blk"], d["k_cache"], d["v_cache"],
                                      d["page_table"], d["ctx_lens"], w_max=w_max, range_pages=range_pages,
                                      dtype="f32")
    _close(o, ref)


def test_ranges_cut_inside_the_block_keys():
    """K = 40 (three block slabs) with one-granule ranges: pieces start and
    end between block slabs, and the merge still gives the unsplit result."""
    d = _paged([0, 37], 2, 8, seed=24, K=40)
    plan = oracle.range_plan(d["ctx_lens"], K=40, w_max=64, range_pages=1)
    ps = oracle.request_pieces(plan, 2, 0, 3)
    assert [(lo, hi) for _, _, lo, hi in ps] == [(0, 2), (2, 3)]
    o = oracle.block_attention_ranges(d["q"], d["k_blk"], d["v_blk"], d["k_cache"], d["v_cache"],
                                      d["page_table"], d["ctx_lens"], w_max=64, range_pages=1, dtype="f32")
    _close(o, _run(d))


def test_key_index_of_slab_boundaries():
    # context of 37 tokens (3 slabs) then K = 40 block keys (3 slabs)
    assert [oracle.key_index(v, 37, 40) for v in range(7)] == [0, 16, 32, 37, 53, 69, 77]
    assert [oracle.key_index(v, 0, 5) for v in range(2)] == [0, 5]


def test_zero_query_is_mean_of_values():
    d = _paged([40, 7], 1, 4, seed=5)
    d["q"][:] = 0
    o = _run(d)
    for b in range(2):
        vall = np.concatenate([d["vctx"][b], d["v_blk"][b]]).astype(np.float64)[:, 0]
        for t in range(o.shape[1]):
            for i in range(o.shape[2]):
                _close(o[b, t, i], vall.mean(axis=0))


def test_dominant_key_selects_its_value():
    d = _paged([30], 1, 4, seed=6, K=1, Hq=1)
    d["q"][0, 0, 0] = [1, 0, 0, 0]
    d["kctx"][0][:] = 0
    pages = d["page_table"][0]
    for n in range(30):
        d["k_cache"][pages[n // PAGE], n % PAGE] = 0
    d["k_cache"][pages[17 // PAGE], 17 % PAGE, 0] = [60, 0, 0, 0]   # score 30 vs 0 for the rest
    d["k_blk"][:] = 0
    o = _run(d)
    v17 = d["vctx"][0][17, 0].astype(np.float64)
    assert np.abs(o[0, 0, 0] - v17).max() < 1e-10


def test_context_order_invariance():
    """Attention is a set operation over keys: permuting the context tokens
    (with their values) leaves the output unchanged."""
    d = _paged([45], 2, 8, seed=7)
    ref = _run(d)
    perm = np.random.default_rng(0).permutation(45)
    pages = d["page_table"][0]
    k_l = d["kctx"][0][perm]
    v_l = d["vctx"][0][perm]
    for n in range(45):
        d["k_cache"][pages[n // PAGE], n % PAGE] = k_l[n]
        d["v_cache"][pages[n // PAGE], n % PAGE] = v_l[n]
    _close(_run(d), ref)


def test_empty_context_is_block_only():
    d = _paged([0], 2, 8, seed=8)
    o = _run(d)
    qt = torch.from_numpy(d["q"][0].astype(np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(d["k_blk"][0].astype(np.float64)).permute(1, 0, 2).repeat_interleave(2, 0)
    vt = torch.from_numpy(d["v_blk"][0].astype(np.float64)).permute(1, 0, 2).repeat_interleave(2, 0)
    ref = torch.softmax(qt @ kt.transpose(1, 2) / math.sqrt(8), -1) @ vt
    _close(o[0], ref.permute(1, 0, 2).numpy())


def test_poisoned_reads_raise():
    d = _paged([20], 1, 4, seed=9)
    bad = d["page_table"].copy()
    used = set(bad[0, :2].tolist())
    spare = next(p for p in range(d["k_cache"].shape[0]) if p not in used)
    bad[0, 1] = spare                                        # a spare (NaN) page
    with pytest.raises(oracle.PoisonedRead):
        oracle.block_attention(d["q"], d["k_blk"], d["v_blk"], d["k_cache"], d["v_cache"], bad,
                               d["ctx_lens"], dtype="f32")
    with pytest.raises(oracle.PoisonedRead):                 # reading past ctx hits NaN tail slots
        oracle.block_attention(d["q"], d["k_blk"], d["v_blk"], d["k_cache"], d["v_cache"],
                               d["page_table"], np.array([21]), dtype="f32")
    bad2 = d["page_table"].copy()
    bad2[0, 0] = -1
    with pytest.raises(oracle.PoisonedRead):
        oracle.block_attention(d["q"], d["k_blk"], d["v_blk"], d["k_cache"], d["v_cache"], bad2,
                               d["ctx_lens"], dtype="f32")


def test_merge_of_empty_split():
    rows, D = 3, 4
    g = np.random.default_rng(1)
    qj = g.standard_normal((rows, D))
    kall = g.standard_normal((10, D))
    vall = g.standard_normal((10, D))
    parts = oracle.split_partials(qj, kall, vall, 0.5, [(0, 4), (4, 4), (4, 10)])
    assert np.isneginf(parts[1][0]).all() and not parts[1][1].any()
    s = 0.5 * qj @ kall.T
    p = np.exp(s - s.max(1, keepdims=True))
    _close(oracle.merge_partials(parts), (p / p.sum(1, keepdims=True)) @ vall)


def test_bf16_storage_decodes_exactly():
    bits = np.array([0x3F80, 0xC000, 0x3EAA, 0x0001], np.uint16)
    v = oracle.decode(bits, "bf16")
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == np.float64(np.array([0x3EAA0000], np.uint32).view(np.float32)[0])
    assert v[3] == 2.0 ** -133


def test_merge_is_overflow_safe():
    """Peaked logits (|s| ~ 1e3) overflow exp() unless each partial and the merge
    subtract their running maxima; the result must still be a convex mix of values."""
    g = np.random.default_rng(2)
    qj = 400.0 * g.standard_normal((4, 8))
    kall = g.standard_normal((20, 8))
    vall = g.standard_normal((20, 8))
    o = oracle.merge_partials(oracle.split_partials(qj, kall, vall, 1.0, [(0, 7), (7, 20)]))
    s = qj @ kall.T
    p = np.exp(s - s.max(1, keepdims=True))
    assert np.isfinite(o).all()
    _close(o, (p / p.sum(1, keepdims=True)) @ vall)


# ---------------------------------------------------------------------------
# block-causal variant: block query t sees the context and block keys s <= t
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ctx_lens,Hkv,G,K", [([37, 16, 5], 2, 2, 4), ([0, 20], 2, 4, 3), ([64], 1, 1, 5)])
def test_block_causal_matches_torch_sdpa_with_mask(ctx_lens, Hkv, G, K):
    D = 8
    d = _paged(ctx_lens, Hkv, D, seed=sum(ctx_lens) + 31 * G + K, Hq=G * Hkv, K=K)
    o = _run(d, block_causal=True)
    for b, c in enumerate(ctx_lens):
        kall = np.concatenate([d["kctx"][b], d["k_blk"][b]])
        vall = np.concatenate([d["vctx"][b], d["v_blk"][b]])
        allowed = torch.ones(K, c + K, dtype=torch.bool)
        for t in range(K):
            allowed[t, c + t + 1:] = False              # later block positions are hidden
        qt = torch.from_numpy(d["q"][b].astype(np.float64)).permute(1, 0, 2)[None]
        kt = torch.from_numpy(kall.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        vt = torch.from_numpy(vall.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed)
        _close(o[b], ref[0].permute(1, 0, 2).numpy())


def test_block_causal_with_one_position_is_the_unmasked_form():
    d = _paged([40, 0, 17], 2, 8, seed=12, K=1)
    _close(_run(d, block_causal=True), _run(d), 0.0)


def test_block_causal_ignores_later_block_keys():
    d = _paged([30, 5], 2, 8, seed=13, K=5)
    o = _run(d, block_causal=True)
    e = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d.items()}
    e["k_blk"][:, 3:] += 2.0
    e["v_blk"][:, 3:] -= 1.5
    o2 = _run(e, block_causal=True)
    assert np.array_equal(o[:, :3], o2[:, :3])           # positions 0..2 never see keys 3, 4
    assert not np.allclose(o[:, 3:], o2[:, 3:])
    assert not np.allclose(_run(d)[:, :3], _run(e)[:, :3])  # the unmasked form does


@pytest.mark.parametrize("range_pages", [0, 1, 3])
def test_block_causal_split_invariance(range_pages):
    d = _paged([100, 0, 16, 33], 2, 8, seed=14, K=6)
    ref = _run(d, block_causal=True)
    o = oracle.block_attention_ranges(d["q"], d["k_blk"], d["v_blk"], d["k_cache"], d["v_cache"],
                                      d["page_table"], d["ctx_lens"], w_max=1000, range_pages=range_pages,
                                      dtype="f32", block_causal=True)
    _close(o, ref)


def test_gather_with_bigger_pages_returns_the_logical_rows():
    """Pools of 32- and 64-token pages, built here by explicit loops from the
    logical context rows and a scrambled page table, gather back to those rows;
    slots past ctx are poisoned, so an off-by-one read raises."""
    g = np.random.default_rng(41)
    Hkv, D = 2, 8
    for P in (32, 64):
        for ctx in (1, P - 1, P, P + 1, 3 * P + 5):
            rows = g.standard_normal((ctx, Hkv, D)).astype(np.float32)
            n_pages = -(-ctx // P)
            perm = g.permutation(n_pages + 3)
            pool = np.full((n_pages + 3, P, Hkv, D), np.nan, np.float32)
            for n in range(ctx):
                pool[perm[n // P], n % P] = rows[n]
            row = np.full(n_pages + 2, -1, np.int32)
            row[:n_pages] = perm[:n_pages]
            for j in range(Hkv):
                np.testing.assert_array_equal(oracle.gather_context(pool, row, ctx, j, "f32"), rows[:, j])
            with pytest.raises(oracle.PoisonedRead):   # a poisoned slot, or a -1 page entry
                oracle.gather_context(pool, row, ctx + 1, 0, "f32")


def test_attention_is_independent_of_the_page_size():
    """The same context stored in 16- and 64-token pages gives the same output."""
    g = np.random.default_rng(42)
    C, K, Hq, Hkv, D = 2, 4, 4, 2, 16
    ctx = np.array([70, 129], np.int32)
    q = g.standard_normal((C, K, Hq, D)).astype(np.float32)
    kb = g.standard_normal((C, K, Hkv, D)).astype(np.float32)
    vb = g.standard_normal((C, K, Hkv, D)).astype(np.float32)
    outs = []
    for P in (16, 64):
        kl = [g.standard_normal((c, Hkv, D)).astype(np.float32) for c in ctx] if P == 16 else kl
        vl = [g.standard_normal((c, Hkv, D)).astype(np.float32) for c in ctx] if P == 16 else vl
        pages = [-(-int(c) // P) for c in ctx]
        pool_k = np.full((sum(pages), P, Hkv, D), np.nan, np.float32)
        pool_v = pool_k.copy()
        pt = np.full((C, max(pages)), -1, np.int32)
        perm = g.permutation(sum(pages))
        off = 0
        for b, c in enumerate(ctx):
            pt[b, :pages[b]] = perm[off:off + pages[b]]
            off += pages[b]
            for n in range(int(c)):
                pool_k[pt[b, n // P], n % P] = kl[b][n]
                pool_v[pt[b, n // P], n % P] = vl[b][n]
        outs.append(oracle.block_attention(q, kb, vb, pool_k, pool_v, pt, ctx, dtype="f32"))
    np.testing.assert_array_equal(outs[0], outs[1])
