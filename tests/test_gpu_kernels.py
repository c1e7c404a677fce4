"""GPU edge cases and invariants of each entry point, against the oracle.

Attention: ragged / empty / sub-page contexts, block lengths that are not a
multiple of 16, GQA group sizes 1..8, D = 64 and 128, fp32 and bf16, every
split size; results must not depend on the split size beyond the tolerance,
must repeat bit for bit for a fixed split size, must be bit-identical when the
same context sits in a scrambled or an identity page table or in an NHD or
HND pool, and the call must leave the KV pools untouched ("no drafter-side KV
cache": the library reads the target's cache and writes only `out` and its
workspace).
Scan: multi-chunk and partial-chunk blocks, B/C groups, the skip term, a zero
initial state.  Projection: C across the M-tile boundaries.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from hybrid_mamba_attention_amd import ops
from hybrid_mamba_attention_amd import workloads as wl

from helpers import assert_attn_close, assert_close, flush, to_dev, to_host64

pytestmark = pytest.mark.gpu
PAGE = 16


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def make_attn_case(seed, ctx, K, Hq, Hkv, D, dtype, *, identity=False, q_scale=1.0, spare=7, page=PAGE):
    """Logical context per request, scattered into a NaN-poisoned pool of
    `page`-token pages (the logical rows do not depend on the page size)."""
    g = np.random.default_rng(seed)
    bf = dtype == "bf16"
    enc = (lambda a: wl.f32_to_bf16_bits(a)) if bf else (lambda a: a.astype(np.float32))
    nan = wl.BF16_NAN if bf else np.float32("nan")
    C = len(ctx)
    n_pages = [-(-c // page) for c in ctx]
    pool = sum(n_pages) + spare
    perm = np.arange(pool) if identity else np.random.default_rng(seed + 99).permutation(pool)
    kc = np.full((pool, page, Hkv, D), nan, dtype=np.uint16 if bf else np.float32)
    vc = kc.copy()
    pt = np.full((C, max(1, max(n_pages))), -1, np.int32)
    off = 0
    for b, c in enumerate(ctx):
        kl = enc(g.standard_normal((c, Hkv, D)).astype(np.float32))
        vl = enc(g.standard_normal((c, Hkv, D)).astype(np.float32))
        pages = perm[off:off + n_pages[b]]
        off += n_pages[b]
        pt[b, :len(pages)] = pages
        for pi, pg in enumerate(pages):
            n = min(page, c - pi * page)
            kc[pg, :n] = kl[pi * page:pi * page + n]
            vc[pg, :n] = vl[pi * page:pi * page + n]
    q = enc(q_scale * g.standard_normal((C, K, Hq, D)).astype(np.float32))
    kb = enc(g.standard_normal((C, K, Hkv, D)).astype(np.float32))
    vb = enc(g.standard_normal((C, K, Hkv, D)).astype(np.float32))
    return dict(q=q, k_blk=kb, v_blk=vb, k_cache=kc, v_cache=vc, page_table=pt,
                ctx_lens=np.array(ctx, np.int32), dtype=dtype)


def run_attn(case, *, split=0, layout="NHD", out=None, causal=False):
    dt = case["dtype"]
    t = {k: to_dev(case[k], dt) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache", "page_table", "ctx_lens")}
    kc, vc = t["k_cache"], t["v_cache"]
    if layout == "HND":  # the same pool stored as [pages, Hkv, 16, D]
        kc = kc.permute(0, 2, 1, 3).contiguous()
        vc = vc.permute(0, 2, 1, 3).contiguous()
    max_ctx = int(case["ctx_lens"].max())
    o, ws = ops.block_attn_inplace(t["q"], t["k_blk"], t["v_blk"], kc, vc, t["page_table"], t["ctx_lens"],
                                   max_ctx=max_ctx, kv_split_pages=split, out=out, layout=layout,
                                   block_causal=causal)
    torch.cuda.synchronize()
    return o, ws, (kc, vc)


def oracle_attn(case, causal=False):
    return oracle.block_attention(case["q"], case["k_blk"], case["v_blk"], case["k_cache"], case["v_cache"],
                                  case["page_table"], case["ctx_lens"], dtype=case["dtype"],
                                  block_causal=causal)


ATTN_CASES = [
    # (name, ctx, K, Hq, Hkv, D, dtype)
    ("bf16-llama-ragged", [0, 1, 15, 16, 17, 300, 1000], 16, 32, 8, 128, "bf16"),
    ("bf16-d64-k13", [33, 100, 7], 13, 8, 2, 64, "bf16"),
    ("f32-mha-k4", [50, 0], 4, 4, 4, 128, "f32"),
    ("f32-d64-k1", [64, 3], 1, 4, 2, 64, "f32"),
    ("bf16-g8-k32-rows256", [500, 31], 32, 16, 2, 128, "bf16"),
    ("bf16-k64-g4-rows256", [200], 64, 8, 2, 128, "bf16"),
    ("bf16-k33-three-block-pages", [37, 16], 33, 4, 2, 128, "bf16"),
    ("bf16-g8-k16-rows128", [2000, 17], 16, 64, 8, 128, "bf16"),
    ("f32-rows128", [90], 16, 16, 2, 64, "f32"),
]


@pytest.mark.parametrize("name,ctx,K,Hq,Hkv,D,dtype", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_shapes(name, ctx, K, Hq, Hkv, D, dtype):
    flush(f"[attn] {name}")
    case = make_attn_case(sum(ctx) + K, ctx, K, Hq, Hkv, D, dtype)
    want = oracle_attn(case)
    for split in (0, 1, 3):
        o, ws, _ = run_attn(case, split=split)
        assert_attn_close(to_host64(o), want, dtype, f"{name} split={split}")
        # the device's work plan, bit for bit (automatic ranges charge by rows)
        plan = ops.plan_of(ws, len(ctx)).cpu().numpy()
        want_plan = oracle.range_plan(case["ctx_lens"], K=K, w_max=int(plan[3]), page_size=PAGE,
                                      range_pages=split, rows=(Hq // Hkv) * K)
        assert np.array_equal(plan, want_plan), f"{name} split={split}: work plan"


CAUSAL_CASES = [
    # (name, ctx, K, Hq, Hkv, D, dtype): partial and multiple block pages,
    # a block alone (empty context), GQA groups 1..8, both types
    ("bf16-llama", [0, 5, 16, 300, 1000], 16, 32, 8, 128, "bf16"),
    ("bf16-k33-three-block-pages", [37, 0], 33, 4, 2, 128, "bf16"),
    ("bf16-k64-rows256", [200, 1], 64, 8, 2, 128, "bf16"),
    ("bf16-g8-k7", [64, 90], 7, 64, 8, 128, "bf16"),
    ("f32-d64-k13", [33, 100, 0], 13, 8, 2, 64, "f32"),
    ("f32-mha-k20", [17], 20, 4, 4, 128, "f32"),
]


@pytest.mark.parametrize("name,ctx,K,Hq,Hkv,D,dtype", CAUSAL_CASES, ids=[c[0] for c in CAUSAL_CASES])
def test_attention_block_causal(name, ctx, K, Hq, Hkv, D, dtype):
    flush(f"[attn causal] {name}")
    case = make_attn_case(3 * sum(ctx) + K, ctx, K, Hq, Hkv, D, dtype)
    want = oracle_attn(case, causal=True)
    for split in (0, 1, 3):
        o, _, _ = run_attn(case, split=split, causal=True)
        assert_attn_close(to_host64(o), want, dtype, f"{name} causal split={split}")


def test_block_causal_edges():
    """K = 1 (the mask removes nothing) is bit-identical to the mask-free call;
    the last block position sees every key, so its output matches the
    mask-free one to the tolerance; earlier positions differ from it."""
    c1 = make_attn_case(21, [100, 0, 17], 1, 32, 8, 128, "bf16")
    a, _, _ = run_attn(c1, causal=True)
    b, _, _ = run_attn(c1, causal=False)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    c = make_attn_case(22, [300, 40], 16, 32, 8, 128, "bf16")
    oc, _, _ = run_attn(c, causal=True)
    of, _, _ = run_attn(c, causal=False)
    oc, of = to_host64(oc), to_host64(of)
    assert_attn_close(oc[:, -1], of[:, -1], "bf16", "last block position")
    assert np.abs(oc[:, 0] - of[:, 0]).max() > 0.05


@pytest.mark.parametrize("P", [32, 64, 128, 256])
def test_bigger_pages(P):
    """Pages of P tokens: parity with the oracle at several range sizes; and,
    for contexts whose keys (context slabs + the block slab) fill whole pages,
    the same bits as the 16-token layout of the same context with ranges of
    the same length in slabs: the kernel walks both in the same 16-token
    slabs and cuts them at the same slabs, only the slab addresses differ."""
    flush(f"[attn page {P}]")
    ctx = [0, 1, P - 1, P, P + 1, 1000, 3000]
    case = make_attn_case(900 + P, ctx, 16, 32, 8, 128, "bf16", page=P)
    want = oracle_attn(case)
    for split in (0, 1, 3):
        o, _, _ = run_attn(case, split=split)
        assert_attn_close(to_host64(o), want, "bf16", f"page {P} split={split}")
    spp = P // 16
    aligned = [16 * (m * spp - 1) - r for m, r in ((1, 0), (2, 5), (3, 15), (9, 1))]
    case = make_attn_case(910 + P, aligned, 16, 32, 8, 128, "bf16", page=P)
    ref16 = make_attn_case(910 + P, aligned, 16, 32, 8, 128, "bf16", page=16)
    for split in (1, 3):
        o, _, _ = run_attn(case, split=split)
        o16, _, _ = run_attn(ref16, split=split * spp)
        assert torch.equal(o.view(torch.int16), o16.view(torch.int16)), f"page {P} split={split}"
    oc, _, _ = run_attn(case, split=1, causal=True)
    assert_attn_close(to_host64(oc), oracle_attn(case, causal=True), "bf16", f"page {P} causal")


def test_bigger_pages_hnd():
    case = make_attn_case(950, [300, 45, 700], 16, 8, 2, 128, "bf16", page=64)
    on, _, _ = run_attn(case, layout="NHD")
    oh, _, _ = run_attn(case, layout="HND")
    assert torch.equal(on.view(torch.int16), oh.view(torch.int16))
    assert_attn_close(to_host64(oh), oracle_attn(case), "bf16", "HND page 64")


def test_split_invariance_and_repeatability():
    case = make_attn_case(5, [1000, 513, 0, 40], 16, 32, 8, 128, "bf16")
    want = oracle_attn(case)
    for split in (1, 2, 3, 7, 0, 10 ** 6):
        o1, ws, _ = run_attn(case, split=split)
        o2, _, _ = run_attn(case, split=split)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"split={split} not repeatable"
        assert_attn_close(to_host64(o1), want, "bf16", f"split={split}")
        plan = ops.plan_of(ws, len(case["ctx_lens"])).cpu().numpy()
        want_plan = oracle.range_plan(case["ctx_lens"], K=16, w_max=int(plan[3]), range_pages=split, rows=64)
        assert np.array_equal(plan, want_plan), split


def test_scrambled_page_table_is_bit_identical():
    a = make_attn_case(11, [700, 65, 16], 16, 32, 8, 128, "bf16")
    b = make_attn_case(11, [700, 65, 16], 16, 32, 8, 128, "bf16", identity=True)
    assert not np.array_equal(a["page_table"], b["page_table"])
    for split in (0, 5):
        oa, _, _ = run_attn(a, split=split)
        ob, _, _ = run_attn(b, split=split)
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_hnd_pool_layout_is_bit_identical():
    case = make_attn_case(12, [300, 45], 16, 8, 2, 128, "bf16")
    on, _, _ = run_attn(case, layout="NHD")
    oh, _, (kc, _) = run_attn(case, layout="HND")
    assert kc.shape[1] == 2 and ops.kv_strides(kc, "HND") == (16 * 2 * 128, 128, 16 * 128)
    assert torch.equal(on.view(torch.int16), oh.view(torch.int16))
    assert_attn_close(to_host64(oh), oracle_attn(case), "bf16", "HND")


@pytest.mark.parametrize("hq", [32, 64], ids=["64-rows", "128-rows"])
@pytest.mark.parametrize("page", [16, 64])
@pytest.mark.parametrize("causal", [False, True], ids=["mask-free", "block-causal"])
def test_head_pair_workgroups_match_single_heads(causal, page, hq):
    """NHD pools (adjacent kv heads) take two heads per workgroup; the HND
    layout of the same pools keeps one head per workgroup.  Same bits, and the oracle within tolerance (ragged
    contexts, one split and 2048-token splits with a merge, the block keys,
    16- and 64-token pages; 64 query rows per kv head, one row tile per wave,
    and 128, two row tiles per wave)."""
    case = make_attn_case(960, [2100, 4000, 2048, 3000], 16, hq, 8, 128, "bf16", page=page)
    for split in (10 ** 6, 2048 // page):
        on, _, _ = run_attn(case, split=split, layout="NHD", causal=causal)
        oh, _, _ = run_attn(case, split=split, layout="HND", causal=causal)
        assert torch.equal(on.view(torch.int16), oh.view(torch.int16)), split
        assert_attn_close(to_host64(on), oracle_attn(case, causal=causal), "bf16", f"head pair split={split}")


@pytest.mark.parametrize("page", [16, 32, 64])
@pytest.mark.parametrize("hq", [32, 64], ids=["64-rows", "128-rows"])
def test_contexts_across_page_table_windows(page, hq):
    """One split per request over contexts that span the kernel's 128-page
    windows of the page table: a window starting at the last stage of full
    pages (fetched during the loop over full pages, made current by the stages
    after it) or right after them, and two window crossings.  NHD pools (two
    heads per workgroup) and HND pools (one head) agree bit for bit, and both
    match the oracle; 64 and 128 query rows per kv head (one and two row
    tiles per wave)."""
    flush(f"[attn windows page {page} hq {hq}]")
    w = 64 * (page // 16)                 # stages (two 16-token slabs each) per window
    ctx = [16 * (2 * w + 2) + 5,          # full-page stages end one past the first window start
           16 * (2 * w) + 2,              # they end right before it
           16 * (4 * w + 2) + 9]          # two window crossings
    case = make_attn_case(970 + page, ctx, 16, hq, 8, 128, "bf16", page=page)
    want = oracle_attn(case)
    on, _, _ = run_attn(case, split=10 ** 6, layout="NHD")
    oh, _, _ = run_attn(case, split=10 ** 6, layout="HND")
    assert torch.equal(on.view(torch.int16), oh.view(torch.int16)), page
    assert_attn_close(to_host64(on), want, "bf16", f"windows page {page}")


@pytest.mark.parametrize("causal", [False, True], ids=["mask-free", "block-causal"])
def test_ranges_without_keys(causal):
    """128 query rows per kv head charge each request 24 slabs (12 units of
    2-slab granules), more than the 8-unit shortest range: with short
    requests some ranges hold only charges and no keys (ranges 0, 2, 5 and
    10 of this batch, by the oracle's plan).  Their workgroups do nothing;
    the output matches the oracle, NHD and HND pools agree bit for bit, and
    the device's plan equals the oracle's."""
    ctx = [0, 1, 5, 16, 17, 0, 3, 40]
    want_plan = oracle.range_plan(ctx, K=16, w_max=64, rows=128)
    f = oracle.plan.unpack(want_plan, len(ctx))
    G = oracle.request_granules(np.array(ctx), 16, PAGE)
    keys = [(int(f["S"][b]), int(f["S"][b] + G[b])) for b in range(len(ctx))]
    empty = [w for w in range(f["W"]) if not any(lo < f["B"][w + 1] and hi > f["B"][w] for lo, hi in keys)]
    assert empty == [0, 2, 5, 10]
    case = make_attn_case(980 + causal, ctx, 16, 64, 8, 128, "bf16")
    on, ws, _ = run_attn(case, split=0, layout="NHD", causal=causal)
    oh, _, _ = run_attn(case, split=0, layout="HND", causal=causal)
    assert torch.equal(on.view(torch.int16), oh.view(torch.int16))
    assert_attn_close(to_host64(on), oracle_attn(case, causal=causal), "bf16", f"empty ranges causal={causal}")
    plan = ops.plan_of(ws, len(ctx)).cpu().numpy()
    assert np.array_equal(plan, oracle.range_plan(ctx, K=16, w_max=int(plan[3]), rows=128))


def test_kv_pool_untouched_and_output_bounded():
    case = make_attn_case(13, [400, 3], 16, 32, 8, 128, "bf16")
    dt = case["dtype"]
    q = to_dev(case["q"], dt)
    canary = torch.full((q.numel() + 4096,), 12345, dtype=torch.int16, device="cuda")
    out = canary[:q.numel()].view(torch.bfloat16).view(q.shape)
    t = {k: to_dev(case[k], dt) for k in ("k_blk", "v_blk", "k_cache", "v_cache", "page_table", "ctx_lens")}
    before = (t["k_cache"].view(torch.int16).clone(), t["v_cache"].view(torch.int16).clone(),
              t["k_blk"].view(torch.int16).clone(), t["v_blk"].view(torch.int16).clone())
    ops.block_attn_inplace(q, t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["page_table"],
                           t["ctx_lens"], max_ctx=400, out=out)
    torch.cuda.synchronize()
    after = (t["k_cache"].view(torch.int16), t["v_cache"].view(torch.int16),
             t["k_blk"].view(torch.int16), t["v_blk"].view(torch.int16))
    for x, y in zip(before, after):
        assert torch.equal(x, y), "an input buffer was written"
    assert (canary[q.numel():] == 12345).all(), "wrote past the output tensor"
    assert torch.isfinite(out.float()).all()
    assert_attn_close(to_host64(out), oracle_attn(case), dt, "canary case")


def test_peaked_logits():
    """Scaled-up queries make the softmax sharp, so errors are not averaged away."""
    case = make_attn_case(14, [900, 100], 16, 32, 8, 128, "bf16", q_scale=4.0)
    want = oracle_attn(case)
    for split in (0, 8):
        o, _, _ = run_attn(case, split=split)
        assert_attn_close(to_host64(o), want, "bf16", f"peaked split={split}")


# ----------------------------------------------------------------------------
# SSD scan
# ----------------------------------------------------------------------------

SSD_CASES = [
    # (C, K, H, P, ng, N, chunk, dtype, dskip, zero_state)
    (2, 16, 4, 64, 1, 32, 4, "bf16", False, False),
    (3, 13, 4, 64, 1, 32, 4, "bf16", True, False),
    (2, 16, 8, 64, 2, 64, 16, "bf16", False, False),
    (1, 4, 4, 64, 1, 16, 4, "f32", False, False),
    (2, 9, 2, 32, 1, 16, 2, "f32", True, True),
    (2, 16, 2, 128, 1, 64, 8, "f32", False, False),
    (1, 5, 2, 64, 1, 128, 1, "bf16", False, False),
    (4, 16, 32, 64, 1, 64, 16, "bf16", True, False),
    # two row blocks per head with the largest state; partial row block
    (2, 16, 2, 128, 1, 128, 16, "bf16", True, False),
    (2, 16, 4, 100, 1, 24, 16, "bf16", False, False),
    # four waves per head sharing one staged state block of fewer than 64
    # rows, with a state narrower than its capacity
    (2, 16, 4, 48, 1, 24, 16, "bf16", True, False),
    # N not a multiple of 4 (scalar state-row loads); heads per group not a
    # multiple of 4 (2- and 1-head workgroups)
    (2, 11, 6, 64, 1, 7, 4, "f32", True, False),
    (3, 16, 12, 64, 4, 32, 8, "bf16", False, False),
    (2, 16, 6, 128, 2, 16, 16, "f32", False, False),
    # many chunks
    (2, 64, 4, 64, 1, 32, 16, "bf16", False, False),
    (1, 64, 4, 64, 1, 32, 1, "f32", True, False),
    # chunks of 32 and 64: several chunks with a partial last one, a block
    # shorter than one chunk, groups, the skip term, the largest state they take
    (2, 80, 4, 64, 1, 32, 32, "bf16", True, False),
    (3, 70, 8, 64, 2, 64, 64, "bf16", False, False),
    (2, 40, 4, 64, 1, 16, 64, "f32", True, False),
    (1, 33, 2, 128, 1, 8, 32, "f32", False, True),
    (2, 128, 4, 64, 1, 32, 64, "bf16", True, False),
]


@pytest.mark.parametrize("C,K,H,P,ng,N,chunk,dtype,dskip,zero_state", SSD_CASES)
def test_ssd_scan(C, K, H, P, ng, N, chunk, dtype, dskip, zero_state):
    g = np.random.default_rng(C * 1000 + K * 10 + N)
    bf = dtype == "bf16"
    enc = (lambda a: wl.f32_to_bf16_bits(a.astype(np.float32))) if bf else (lambda a: a.astype(np.float32))
    x = enc(g.standard_normal((C, K, H, P)))
    B = enc(g.standard_normal((C, K, ng, N)))
    Cm = enc(g.standard_normal((C, K, ng, N)))
    delta = np.logaddexp(0, g.standard_normal((C, K, H)) - 4.0).astype(np.float32)
    A = (-np.exp(g.uniform(0, 1, H))).astype(np.float32)
    h0 = None if zero_state else g.standard_normal((C, H, P, N)).astype(np.float32)
    D = g.standard_normal(H).astype(np.float32) if dskip else None
    y, hf = ops.ssd_scan(to_dev(x, dtype), to_dev(delta, dtype), to_dev(A, dtype), to_dev(B, dtype),
                         to_dev(Cm, dtype), chunk=chunk, h0=None if h0 is None else to_dev(h0, dtype),
                         Dskip=None if D is None else to_dev(D, dtype), want_final=True)
    torch.cuda.synchronize()
    yo, hfo = oracle.ssd_recurrence(oracle.decode(x, dtype), delta, A, oracle.decode(B, dtype),
                                    oracle.decode(Cm, dtype), h0=h0, Dskip=D)
    assert_close(to_host64(y), yo, dtype, "y")
    assert_close(to_host64(hf), hfo, dtype, "h_final")


@pytest.mark.parametrize("K,chunk,N", [(16, 16, 32), (40, 16, 64), (13, 4, 32)])
def test_scan_position_split_is_bit_identical(K, chunk, N):
    """A batch with few heads runs four waves per head, each taking every
    fourth position; 65 requests of 16 heads run one wave per head.  The same
    requests must get the same bits either way (y and h_final)."""
    C, H, P, ng = 65, 16, 64, 1
    g = np.random.default_rng(7000 + K + N)
    enc = lambda a: wl.f32_to_bf16_bits(a.astype(np.float32))
    x = enc(g.standard_normal((C, K, H, P)))
    B = enc(g.standard_normal((C, K, ng, N)))
    Cm = enc(g.standard_normal((C, K, ng, N)))
    delta = np.logaddexp(0, g.standard_normal((C, K, H)) - 4.0).astype(np.float32)
    A = (-np.exp(g.uniform(0, 1, H))).astype(np.float32)
    h0 = g.standard_normal((C, H, P, N)).astype(np.float32)
    D = g.standard_normal(H).astype(np.float32)

    def run(c):
        return ops.ssd_scan(to_dev(x[:c], "bf16"), to_dev(delta[:c], "bf16"), to_dev(A, "bf16"),
                            to_dev(B[:c], "bf16"), to_dev(Cm[:c], "bf16"), chunk=chunk, h0=to_dev(h0[:c], "bf16"),
                            Dskip=to_dev(D, "bf16"), want_final=True)
    y_all, hf_all = run(C)     # C * H = 1040: one wave per head
    y_few, hf_few = run(5)     # C * H = 80: four waves per head
    torch.cuda.synchronize()
    assert torch.equal(y_few, y_all[:5]) and torch.equal(hf_few, hf_all[:5])
    yo, hfo = oracle.ssd_recurrence(oracle.decode(x[:5], "bf16"), delta[:5], A, oracle.decode(B[:5], "bf16"),
                                    oracle.decode(Cm[:5], "bf16"), h0=h0[:5], Dskip=D)
    assert_close(to_host64(y_few), yo, "bf16", "y")
    assert_close(to_host64(hf_few), hfo, "bf16", "h_final")


# ----------------------------------------------------------------------------
# projection
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("C,d,S,dtype", [
    # 128-column kernel (bf16, d % 64 == 0, S % 128 == 0): 32/64/128-row blocks,
    # several row blocks, column-block counts with and without a multiple of 8,
    # step counts below, at and above the prefetch depth
    (1, 256, 4096, "bf16"), (5, 512, 8192, "bf16"), (17, 256, 4096, "bf16"), (33, 4096, 2048, "bf16"),
    (64, 1024, 4096, "bf16"), (65, 256, 4096, "bf16"), (130, 256, 8192, "bf16"), (256, 128, 1024, "bf16"),
    (3, 256, 640, "bf16"), (200, 192, 1152, "bf16"), (97, 320, 1024, "bf16"),
    # its 256-column form without the k split (>= 512 column blocks of up to 64
    # rows): 32- and 64-row blocks, block counts with and without a multiple
    # of 8, one step (below the prefetch depth) and several
    (1, 128, 131072, "bf16"), (40, 64, 131072, "bf16"), (64, 192, 131072, "bf16"),
    (17, 64, 131328, "bf16"), (64, 128, 131328, "bf16"),
    # general kernel: fp32, or d % 64 == 32, or S % 128 == 64
    (1, 256, 4096, "f32"), (100, 512, 4096, "f32"), (7, 96, 4096, "bf16"), (40, 256, 4160, "bf16"),
    (129, 160, 1088, "bf16"),
])
def test_init_state(C, d, S, dtype):
    g = np.random.default_rng(C + d + S)
    bf = dtype == "bf16"
    enc = (lambda a: wl.f32_to_bf16_bits(a.astype(np.float32))) if bf else (lambda a: a.astype(np.float32))
    u = enc(g.standard_normal((C, d)))
    w = enc(0.02 * g.standard_normal((d, S)))
    h0 = ops.init_state(to_dev(u, dtype), to_dev(w, dtype))
    torch.cuda.synchronize()
    assert_close(to_host64(h0), oracle.init_state(oracle.decode(u, dtype), oracle.decode(w, dtype)), dtype, "h0")


def test_layer_with_skip_term():
    from dataclasses import replace
    from helpers import layer_from_inputs, oracle_h0, oracle_scan
    w = replace(wl.WORKLOADS[1], name="small-layer-dskip", C=3, ctx=("uniform", 0, 200), d_model=512,
                H=4, N=32, seed=4242)
    inp = wl.make_inputs(w, with_dskip=True)
    layer = layer_from_inputs(inp, with_dskip=True)
    h0 = oracle_h0(inp)
    y, hf = oracle_scan(inp, h0)
    assert_close(to_host64(layer.y), y, "bf16", "y with skip")
    assert_close(to_host64(layer.h_final), hf, "bf16", "h_final with skip")


def test_layer_block_causal_and_direct_reuse_ablation():
    """The layer with the block-causal mask, and the direct-reuse-only
    ablation (no state projection: the scan starts from the zero state)."""
    from dataclasses import replace
    from helpers import layer_from_inputs, oracle_attn as oracle_attn_inp, oracle_h0, oracle_scan
    w = replace(wl.WORKLOADS[1], name="small-layer-ablation", C=3, ctx=("uniform", 0, 300), d_model=512,
                H=4, N=32, seed=4343)
    inp = wl.make_inputs(w)
    full = layer_from_inputs(inp, block_causal=True)
    assert_attn_close(to_host64(full.out), oracle_attn_inp(inp, block_causal=True), "bf16", "causal out")
    y, hf = oracle_scan(inp, oracle_h0(inp))
    assert_close(to_host64(full.y), y, "bf16", "y")
    abl = layer_from_inputs(inp, no_init=True)
    assert abl.h0 is None
    y0, hf0 = oracle_scan(inp, np.zeros((w.C, w.S)))
    assert_close(to_host64(abl.y), y0, "bf16", "y from the zero state")
    assert_close(to_host64(abl.h_final), hf0, "bf16", "h_final from the zero state")
    assert_attn_close(to_host64(abl.out), oracle_attn_inp(inp), "bf16", "ablation out")
    assert np.abs(to_host64(abl.y) - y).max() > 1e-3, "the projected state must matter"


def test_layer_graph_replays_match_eager():
    """The layer's HIP graph (captured on one stream) against the eager layer,
    bit for bit, over replays with eager work in between."""
    from helpers import layer_from_inputs
    w = wl.sweep_workload(4)
    w = replace_workload(w, ctx=("uniform", 100, 3000), seed=4545)
    inp = wl.make_inputs(w)
    layer = layer_from_inputs(inp)
    ref = [t.clone() for t in (layer.out, layer.y, layer.h0, layer.h_final)]
    layer.graph()
    for rep in range(3):
        for t in (layer.out, layer.y, layer.h0, layer.h_final):
            t.zero_()
        layer.launch_graph()
        torch.cuda.synchronize()
        for got, want in zip((layer.out, layer.y, layer.h0, layer.h_final), ref):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want), rep
        torch.randn(1 << 18, device="cuda").sum()
        torch.cuda.synchronize()


@pytest.mark.parametrize("C,ctx,split", [(4, ("uniform", 100, 3000), True), (1, ("fixed", 8192), True),
                                         (64, ("fixed", 2048), False), (96, ("uniform", 2048, 3000), True),
                                         (128, ("fixed", 8192), False)],
                         ids=["c4-ragged-pieces", "c1-33-pieces", "c64-whole", "c96-ragged-pieces",
                              "c128-whole-head-pair"])
def test_layer_equals_its_entry_points_bitwise(C, ctx, split):
    """When some request spans several ranges the layer runs the scan and the
    attention's merge in one launch; when every range holds whole requests
    (C = 64 at 2048 tokens: one request per range; C = 128 at 8192: two kv
    heads per workgroup) the merge finds nothing to do.  Either way its outputs
    must be the bits of the separate entry points (a1, a2, a3 + a4) on the
    same inputs."""
    from helpers import layer_from_inputs
    from hybrid_mamba_attention_amd import ops
    flush(f"[layer vs entry points C={C} ctx={ctx}]")
    w = replace_workload(wl.sweep_workload(C), ctx=ctx, seed=4646 + C)
    inp = wl.make_inputs(w)
    layer = layer_from_inputs(inp)
    plan = layer.plan().cpu().numpy()
    assert (plan[4 + 2 * C:4 + 3 * C].max() > 1) == split, "the case must (not) cut requests into pieces"
    a, dt = inp.arrays, w.dtype
    h0 = ops.init_state(to_dev(a["u"], dt), to_dev(a["w_init"], dt))
    y, hf = ops.ssd_scan(to_dev(a["x"], dt), to_dev(a["delta"], dt), to_dev(a["A"], dt), to_dev(a["B"], dt),
                         to_dev(a["Cm"], dt), chunk=w.chunk, h0=h0, want_final=True)
    out, _ = ops.block_attn_inplace(to_dev(a["q"], dt), to_dev(a["k_blk"], dt), to_dev(a["v_blk"], dt),
                                    to_dev(a["k_cache"], dt), to_dev(a["v_cache"], dt),
                                    to_dev(inp.page_table, dt), to_dev(inp.ctx_lens, dt), max_ctx=inp.max_ctx)
    torch.cuda.synchronize()
    assert torch.equal(layer.h0, h0)
    assert torch.equal(layer.y, y)
    assert torch.equal(layer.h_final, hf)
    assert torch.equal(layer.out.view(torch.int16), out.view(torch.int16))


def replace_workload(w, **kw):
    from dataclasses import replace
    return replace(w, **kw)
