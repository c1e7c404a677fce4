"""Seeded synthetic workloads for the H-Spec drafter layer.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no projection, no scan, no softmax).  Both the CPU oracle
(through the tests and the bench's CPU leg) and the HIP path receive the very
same host arrays produced here.

Shapes follow the five workloads of the drafter layer (the tiny fp32 case, the
Llama-3-8B-shaped cases at concurrency 1 / 32 / 128, and the wider 64-head
case).  The method itself comes from "H-Spec: Parallel Speculative Decoding
Without a Drafter-Side KV Cache" (Abstract): the Mamba state is initialised
from a projection of the target's last-token hidden state, and attention reads
the target's paged KV cache in place.  The pages print no shapes or value
distributions; those below are the stated synthetic recipe.

Value recipe (every workload):
  * u, x, B, Cm, q, k_blk, v_blk and both KV pools: N(0, 1)
  * W_init: N(0, 0.02^2)  (0.02 read as a standard deviation)
  * delta = softplus(N(0,1) - 4)  (already positive; the kernel takes it as is)
  * A = -exp(U(0, 1))
  * bf16 tensors are drawn in fp32 and rounded once to bf16 (round to
    nearest even); delta and A stay fp32.
Paged KV recipe:
  * page size 16; pool = sum_b ceil(ctx_b/16) pages + 64 spare pages
  * a seeded permutation of the pool hands pages to requests, so pages of
    different requests interleave in the one shared pool
  * spare pages and the tail slots past ctx_b of each last page hold NaN
  * page-table entries past a request's last page are -1
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

PAGE = 16
SPARE_PAGES = 64
BF16_NAN = np.uint16(0x7FC0)
F32_NAN = np.float32("nan")

# Fixed order of the per-tensor random streams (SeedSequence(seed).spawn).
STREAMS = ("ctx", "perm", "u", "w_init", "x", "delta", "A", "B", "Cm",
           "q", "k_blk", "v_blk", "k_cache", "v_cache", "Dskip")
CHUNK = 1 << 22  # elements per independently seeded chunk of a big tensor


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16": element type of the activation tensors
    C: int                # concurrent requests
    ctx: tuple            # ("fixed", n) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    K: int                # draft block length
    d_model: int
    Hq: int
    Hkv: int
    D: int                # attention head dim
    H: int                # Mamba-2 heads
    P: int                # Mamba-2 head dim
    N: int                # Mamba-2 state size
    chunk: int            # SSD chunk length
    seed: int
    ng: int = 1           # B/C groups

    @property
    def S(self) -> int:
        return self.H * self.P * self.N

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    0: Workload("tiny-f32-c1-ctx64", "f32", 1, ("fixed", 64), 4, 256, 4, 2, 64,
                4, 64, 16, 4, 1000),
    1: Workload("llama8b-bf16-c1-ctx2048", "bf16", 1, ("fixed", 2048), 16, 4096,
                32, 8, 128, 16, 64, 32, 16, 1001),
    2: Workload("llama8b-bf16-c32-ctx512to4096", "bf16", 32, ("uniform", 512, 4096),
                16, 4096, 32, 8, 128, 16, 64, 32, 16, 1002),
    3: Workload("llama8b-bf16-c128-ctx8192", "bf16", 128, ("fixed", 8192), 16, 4096,
                32, 8, 128, 16, 64, 32, 16, 1003),
    4: Workload("wide64h-bf16-c64-ctx1024to16384", "bf16", 64,
                ("loguniform", 1024, 16384), 16, 5120, 64, 8, 128, 32, 64, 64, 16, 1004),
}


def sweep_workload(C: int) -> Workload:
    """Concurrency sweep point: the C=128 workload's shapes at another C."""
    base = WORKLOADS[3]
    return replace(base, name=f"llama8b-bf16-c{C}-ctx8192", C=C, seed=2000 + C)


# ----------------------------------------------------------------------------
# helpers (format conversion only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    out = ((u + (((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF))) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_chunked(ss: np.random.SeedSequence, n: int, std: float, bf16: bool,
                    out: np.ndarray | None = None) -> np.ndarray:
    """n draws of N(0, std^2), produced in CHUNK-sized independently seeded pieces.

    The result does not depend on the thread count.  Returns fp32 or bf16 bits.
    """
    if out is None:
        out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    nchunks = max(1, -(-n // CHUNK))
    kids = ss.spawn(nchunks)

    def work(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        g = np.random.default_rng(kids[i])
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(v) if bf16 else v

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


# ----------------------------------------------------------------------------
# context lengths, page pool and page table
# ----------------------------------------------------------------------------

def draw_ctx_lens(w: Workload, ss: np.random.SeedSequence) -> np.ndarray:
    g = np.random.default_rng(ss)
    kind = w.ctx[0]
    if kind == "fixed":
        return np.full(w.C, w.ctx[1], dtype=np.int32)
    if kind == "uniform":
        lo, hi = w.ctx[1], w.ctx[2]
        return g.integers(lo, hi, endpoint=True, size=w.C).astype(np.int32)
    if kind == "loguniform":
        lo, hi = w.ctx[1], w.ctx[2]
        v = np.floor(np.exp(g.uniform(math.log(lo), math.log(hi), size=w.C)))
        return np.clip(v, lo, hi).astype(np.int32)
    raise ValueError(kind)


def build_page_table(ctx_lens: np.ndarray, ss: np.random.SeedSequence,
                     spare: int = SPARE_PAGES, identity: bool = False, page_size: int = PAGE):
    """Shared page pool with interleaved pages of page_size tokens.

    Returns (page_table int32 [C, max_pages] with -1 padding, num_pages, pages_of
    list of int arrays).  identity=True hands out pages in order (no shuffle).
    """
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    n_pages = (ctx_lens + page_size - 1) // page_size
    total = int(n_pages.sum())
    pool = total + spare
    if identity:
        perm = np.arange(pool, dtype=np.int64)
    else:
        perm = np.random.default_rng(ss).permutation(pool)
    max_pages = max(1, int(n_pages.max()) if len(n_pages) else 1)
    pt = np.full((len(ctx_lens), max_pages), -1, dtype=np.int32)
    off = 0
    pages_of = []
    for b, n in enumerate(n_pages):
        p = perm[off:off + n]
        pt[b, :n] = p
        pages_of.append(p.astype(np.int64))
        off += n
    return pt, pool, pages_of


def _poison_kv(pool_arr: np.ndarray, ctx_lens, pages_of, used_pages, nan_value):
    """NaN into spare pages and into the tail slots past ctx of each last page."""
    spare = np.ones(pool_arr.shape[0], dtype=bool)
    spare[used_pages] = False
    pool_arr[spare] = nan_value
    for L, pages in zip(ctx_lens, pages_of):
        r = int(L) % PAGE
        if r:
            pool_arr[pages[-1], r:] = nan_value


# ----------------------------------------------------------------------------
# full input set
# ----------------------------------------------------------------------------

@dataclass
class Inputs:
    w: Workload
    ctx_lens: np.ndarray          # int32 [C]
    page_table: np.ndarray        # int32 [C, max_pages]
    num_pages: int
    arrays: dict = field(default_factory=dict)
    # arrays: u [C,d], w_init [d,S], x [C,K,H,P], B/Cm [C,K,ng,N] (act dtype: fp32 or
    # bf16 bits as uint16); delta f32 [C,K,H]; A f32 [H]; q [C,K,Hq,D];
    # k_blk/v_blk [C,K,Hkv,D]; k_cache/v_cache [num_pages,16,Hkv,D] (act dtype)

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def max_ctx(self) -> int:
        return int(self.ctx_lens.max()) if len(self.ctx_lens) else 0


def make_inputs(w: Workload, *, ctx_lens=None, identity_pages: bool = False,
                with_dskip: bool = False, parts=("mamba", "attn")) -> Inputs:
    """Draw every input of workload `w` from its seed.

    ctx_lens overrides the drawn context lengths (edge-case tests).  parts
    selects which halves to draw ("mamba": u, W_init, x, delta, A, B, Cm;
    "attn": q, block K/V, KV pools); the streams stay the same either way.
    """
    root = np.random.SeedSequence(w.seed)
    ss = dict(zip(STREAMS, root.spawn(len(STREAMS))))
    bf16 = w.dtype == "bf16"
    act = np.uint16 if bf16 else np.float32

    if ctx_lens is None:
        ctx_lens = draw_ctx_lens(w, ss["ctx"])
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    pt, pool, pages_of = build_page_table(ctx_lens, ss["perm"], identity=identity_pages)
    inp = Inputs(w, ctx_lens, pt, pool)
    a = inp.arrays

    def normal(name, shape, std=1.0):
        n = int(np.prod(shape))
        return _normal_chunked(ss[name], n, std, bf16).reshape(shape)

    if "mamba" in parts:
        a["u"] = normal("u", (w.C, w.d_model))
        a["w_init"] = normal("w_init", (w.d_model, w.S), 0.02)
        a["x"] = normal("x", (w.C, w.K, w.H, w.P))
        z = np.random.default_rng(ss["delta"]).standard_normal((w.C, w.K, w.H)) - 4.0
        a["delta"] = np.logaddexp(0.0, z).astype(np.float32)          # softplus
        a["A"] = (-np.exp(np.random.default_rng(ss["A"]).uniform(0.0, 1.0, w.H))).astype(np.float32)
        a["B"] = normal("B", (w.C, w.K, w.ng, w.N))
        a["Cm"] = normal("Cm", (w.C, w.K, w.ng, w.N))
        if with_dskip:
            a["Dskip"] = np.random.default_rng(ss["Dskip"]).standard_normal(w.H).astype(np.float32)
    if "attn" in parts:
        a["q"] = normal("q", (w.C, w.K, w.Hq, w.D))
        a["k_blk"] = normal("k_blk", (w.C, w.K, w.Hkv, w.D))
        a["v_blk"] = normal("v_blk", (w.C, w.K, w.Hkv, w.D))
        shape = (pool, PAGE, w.Hkv, w.D)
        used = np.concatenate(pages_of) if pages_of else np.zeros(0, np.int64)
        nan = BF16_NAN if bf16 else F32_NAN
        for name in ("k_cache", "v_cache"):
            arr = normal(name, shape)
            _poison_kv(arr, ctx_lens, pages_of, used, nan)
            a[name] = arr
    assert all(v.dtype in (act, np.float32) for v in a.values())
    return inp


# ----------------------------------------------------------------------------
# the Mamba-2 block around the scan
# ----------------------------------------------------------------------------

BLOCK_STREAMS = ("hidden", "w_in", "conv_w", "conv_b", "norm_w", "w_out", "h0", "A", "Dskip")
BLOCK_DT_BIAS = -4.0
BLOCK_EPS = 1e-5


def block_sizes(w: Workload):
    """(d_inner, conv_dim, d_in_proj) of the Mamba-2 block of workload w."""
    d_inner = w.H * w.P
    conv_dim = d_inner + 2 * w.ng * w.N
    return d_inner, conv_dim, 2 * d_inner + 2 * w.ng * w.N + w.H


def make_block_inputs(w: Workload, *, with_dskip: bool = True, with_h0: bool = True) -> dict:
    """Inputs of one Mamba-2 block call over workload w's draft blocks.

    Recipe (its own seed branch, so the layer's streams are unchanged):
      * hidden [C,K,d_model]: N(0,1); h0 [C,H,P,N] fp32: N(0,1)
      * w_in [2*H*P + 2*ng*N + H, d_model] and w_out [d_model, H*P]: N(0, 0.02^2)
      * conv_w [conv_dim, 4], conv_b [conv_dim]: U(-0.5, 0.5) (fan-in 4)
      * dt_bias [H] = -4, so delta = softplus(dt_raw - 4) as in the layer recipe
      * A [H] = -exp(U(0,1)); Dskip [H]: N(0,1); norm_w [H*P]: 1 + 0.1 N(0,1)
      * eps = 1e-5; fp32 for everything but hidden, w_in and w_out (act dtype)
    """
    root = np.random.SeedSequence([w.seed, 77])
    ss = dict(zip(BLOCK_STREAMS, root.spawn(len(BLOCK_STREAMS))))
    bf16 = w.dtype == "bf16"
    d_inner, conv_dim, d_proj = block_sizes(w)

    def normal(name, shape, std=1.0):
        return _normal_chunked(ss[name], int(np.prod(shape)), std, bf16).reshape(shape)

    def rng(name):
        return np.random.default_rng(ss[name])

    a = dict(
        hidden=normal("hidden", (w.C, w.K, w.d_model)),
        w_in=normal("w_in", (d_proj, w.d_model), 0.02),
        conv_w=rng("conv_w").uniform(-0.5, 0.5, (conv_dim, 4)).astype(np.float32),
        conv_b=rng("conv_b").uniform(-0.5, 0.5, conv_dim).astype(np.float32),
        dt_bias=np.full(w.H, BLOCK_DT_BIAS, np.float32),
        A=(-np.exp(rng("A").uniform(0.0, 1.0, w.H))).astype(np.float32),
        norm_w=(1.0 + 0.1 * rng("norm_w").standard_normal(d_inner)).astype(np.float32),
        w_out=normal("w_out", (w.d_model, d_inner), 0.02),
        eps=BLOCK_EPS,
    )
    if with_dskip:
        a["Dskip"] = rng("Dskip").standard_normal(w.H).astype(np.float32)
    if with_h0:
        a["h0"] = rng("h0").standard_normal((w.C, w.H, w.P, w.N), dtype=np.float32)
    return a


# ----------------------------------------------------------------------------
# drafter-side KV injection (the contrast workload)
# ----------------------------------------------------------------------------

def make_inject_inputs(w: Workload, n_new: int, *, ctx_lens=None, spare: int = 8,
                       page_size: int = PAGE) -> dict:
    """Inputs of one injection step: n_new new positions per request after
    ctx_lens[b] existing ones, written into a drafter-side paged pool shaped
    like the target's ([pages, page_size, Hkv, D], shuffled page table).

      * hidden [C, n_new, d_model]: N(0,1); w_kv [2*Hkv*D, d_model]: N(0, 0.02^2)
      * the pools hold N(0,1) values (the existing cache) plus NaN in spare pages
      * start = ctx_lens (drawn as for the layer unless given)
    """
    root = np.random.SeedSequence([w.seed, 91])
    ss = dict(zip(("ctx", "perm", "hidden", "w_kv", "k", "v"), root.spawn(6)))
    bf16 = w.dtype == "bf16"
    if ctx_lens is None:
        ctx_lens = draw_ctx_lens(w, ss["ctx"])
    start = np.asarray(ctx_lens, dtype=np.int32)
    pt, pool, pages_of = build_page_table(start.astype(np.int64) + n_new, ss["perm"], spare=spare,
                                          page_size=page_size)

    def normal(name, shape, std=1.0):
        return _normal_chunked(ss[name], int(np.prod(shape)), std, bf16).reshape(shape)

    a = dict(hidden=normal("hidden", (w.C, n_new, w.d_model)),
             w_kv=normal("w_kv", (2 * w.Hkv * w.D, w.d_model), 0.02),
             page_table=pt, start=start, num_pages=pool)
    used = np.concatenate(pages_of) if pages_of else np.zeros(0, np.int64)
    nan = BF16_NAN if bf16 else F32_NAN
    for name in ("k", "v"):
        arr = normal(name, (pool, page_size, w.Hkv, w.D))
        spare_mask = np.ones(pool, dtype=bool)
        spare_mask[used] = False
        arr[spare_mask] = nan
        a[name + "_cache"] = arr
    return a


# ----------------------------------------------------------------------------
# a drafter stack of hybrid layers
# ----------------------------------------------------------------------------

def make_stack_inputs(w: Workload, kinds=("MA", "MA"), *, ctx_lens=None) -> dict:
    """Inputs of a drafter stack: kinds[l] holds "M" (Mamba half) and/or "A"
    (attention half) for layer l.  Every layer gets its own weights and, for
    an attention half, its own target KV pools (the target layer it reads);
    the page table and context lengths are shared, as a target's layers
    share them.

      * hidden_in [C, K, d_model], u [C, d_model]: N(0,1)
      * pre_norm_w: 1 + 0.1 N(0,1); Mamba half as the block recipe, plus
        w_init [d_model, S] N(0, 0.02^2) and h0 from u
      * wq [Hq*D, d], wk/wv [Hkv*D, d], wo [d, Hq*D]: N(0, 0.02^2)
      * pools: N(0,1) with NaN in spare pages and tail slots, as the layer's
    """
    root = np.random.SeedSequence([w.seed, 123])
    nl = len(kinds)
    kids = root.spawn(3 + nl)
    bf16 = w.dtype == "bf16"

    def normal(ss, shape, std=1.0):
        return _normal_chunked(ss, int(np.prod(shape)), std, bf16).reshape(shape)

    g_ctx, g_perm, g_io = kids[0], kids[1], kids[2].spawn(2)
    if ctx_lens is None:
        ctx_lens = draw_ctx_lens(w, g_ctx)
    ctx_lens = np.asarray(ctx_lens, np.int32)
    pt, pool, pages_of = build_page_table(ctx_lens, g_perm)
    used = np.concatenate(pages_of) if pages_of else np.zeros(0, np.int64)
    nan = BF16_NAN if bf16 else F32_NAN
    out = dict(hidden_in=normal(g_io[0], (w.C, w.K, w.d_model)), u=normal(g_io[1], (w.C, w.d_model)),
               page_table=pt, ctx_lens=ctx_lens, num_pages=pool, layers=[])
    d_inner, conv_dim, d_proj = block_sizes(w)
    for l, kind in enumerate(kinds):
        ss = kids[3 + l].spawn(16)
        rng = lambda i: np.random.default_rng(ss[i])
        L = dict(pre_norm_w=(1.0 + 0.1 * rng(0).standard_normal(w.d_model)).astype(np.float32), eps=BLOCK_EPS)
        if "M" in kind:
            L.update(w_init=normal(ss[1], (w.d_model, w.S), 0.02),
                     w_in=normal(ss[2], (d_proj, w.d_model), 0.02),
                     conv_w=rng(3).uniform(-0.5, 0.5, (conv_dim, 4)).astype(np.float32),
                     conv_b=rng(4).uniform(-0.5, 0.5, conv_dim).astype(np.float32),
                     dt_bias=np.full(w.H, BLOCK_DT_BIAS, np.float32),
                     A=(-np.exp(rng(5).uniform(0.0, 1.0, w.H))).astype(np.float32),
                     Dskip=rng(6).standard_normal(w.H).astype(np.float32),
                     norm_w=(1.0 + 0.1 * rng(7).standard_normal(d_inner)).astype(np.float32),
                     w_out=normal(ss[8], (w.d_model, d_inner), 0.02))
        if "A" in kind:
            L.update(wq=normal(ss[9], (w.Hq * w.D, w.d_model), 0.02),
                     wk=normal(ss[10], (w.Hkv * w.D, w.d_model), 0.02),
                     wv=normal(ss[11], (w.Hkv * w.D, w.d_model), 0.02),
                     wo=normal(ss[12], (w.d_model, w.Hq * w.D), 0.02))
            for name, i in (("k_cache", 13), ("v_cache", 14)):
                arr = normal(ss[i], (pool, PAGE, w.Hkv, w.D))
                _poison_kv(arr, ctx_lens, pages_of, used, nan)
                L[name] = arr
        out["layers"].append(L)
    return out


def kv_bytes(w: Workload, ctx_lens) -> int:
    """Bytes of target KV a layer call must read in place (K and V, valid tokens)."""
    e = 2 if w.dtype == "bf16" else 4
    return int(np.sum(np.asarray(ctx_lens, np.int64))) * w.Hkv * w.D * 2 * e


def w_init_bytes(w: Workload) -> int:
    e = 2 if w.dtype == "bf16" else 4
    return w.d_model * w.S * e
