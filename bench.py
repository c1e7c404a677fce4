"""Benchmark of the H-Spec drafter layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 3] [--no-sweep] [--no-cpu]

One step is one call of the whole layer (hspec_draft_layer: split plan,
W_init projection, SSD scan, in-place paged block attention and split merge)
over one batch of synthetic inputs already resident in HBM.  The default
workload is the concurrency-128 case (8192-token contexts, Llama-3-8B-shaped
attention, 4.3 GB of target KV read in place per call).  Each timed step is
preceded by a 2 GiB streaming read that evicts L2 and the 256 MiB Infinity
Cache, so no step reads W_init or KV from a previous step's cache; the events
bracket only the layer call.  (The flush reads rather than writes: a write
flush would leave the Infinity Cache full of dirty lines whose write-back then
competes with the timed kernel's reads -- measured on this chip, it halves the
read bandwidth of a 256 MiB stream.)

Printed: one JSON line with the metric (drafted block-tokens/s per drafter
layer), the per-kernel breakdown, the roofline of the dominant kernel (the
in-place KV attention), a concurrency sweep C = 1..128 at the same shapes, and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor peak
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
FP32_MATRIX_TFLOPS = 157.3     # MI355X dense fp32 matrix peak
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD)
    p.add_argument("--kv-split-pages", type=int, default=0)
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-flush", action="store_true")
    p.add_argument("--no-probe", action="store_true", help="skip the stream-read bandwidth probe")
    p.add_argument("--no-variants", action="store_true",
                   help="skip the block-causal and direct-reuse-only layer timings")
    p.add_argument("--no-block", action="store_true",
                   help="skip the Mamba-2 block (projections, conv, scan, gated norm) timings")
    p.add_argument("--no-inject", action="store_true",
                   help="skip the drafter-side KV injection contrast timings")
    p.add_argument("--no-stack", action="store_true",
                   help="skip the drafter-stack (eager vs HIP graph) timings")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-workload table (all five workloads, one entry each)")
    p.add_argument("--sweep", default="1,2,4,8,16,32,64,128")
    p.add_argument("--summarize-profiles", nargs="+", metavar="DIR",
                   help="write the profiles/ records from rocprofv3 output directories (no GPU work): "
                        "a --kernel-trace --stats run, FETCH_SIZE and WRITE_SIZE --pmc runs (with "
                        "--calib-copy) and an MFMA --pmc run of this script")
    p.add_argument("--calib-copy", action="store_true",
                   help="also launch a plain 1 GiB device copy (counter calibration under rocprofv3)")
    return p.parse_args()


# ----------------------------------------------------------------------------
# device-side plumbing (torch only for memory, streams and events)
# ----------------------------------------------------------------------------

def dev(arr, torch):
    import numpy as np
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def build_layer(inp, kv_split_pages, torch, block_causal=False, no_init=False):
    """The layer of a workload; no_init: direct-reuse-only ablation (no state projection)."""
    from hybrid_mamba_attention_amd import ops
    a = inp.arrays
    w = inp.w
    t = {k: dev(v, torch) for k, v in a.items()}
    return ops.DraftLayer(
        u=None if no_init else t["u"], w_init=None if no_init else t["w_init"], x=t["x"],
        delta=t["delta"], A=t["A"], B=t["B"], Cm=t["Cm"],
        chunk=w.chunk, q=t["q"], k_blk=t["k_blk"], v_blk=t["v_blk"], k_cache=t["k_cache"],
        v_cache=t["v_cache"], page_table=dev(inp.page_table, torch), ctx_lens=dev(inp.ctx_lens, torch),
        max_ctx=inp.max_ctx, kv_split_pages=kv_split_pages, block_causal=block_causal), t


def timed(fn, steps, warmup, flush, torch):
    """Per-call event times (ms) with the cache flush outside the events."""
    for _ in range(warmup):
        flush()
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def stats(ts):
    import numpy as np
    a = np.array(ts)
    return dict(mean=float(a.mean()), median=float(np.median(a)), p10=float(np.percentile(a, 10)),
                p90=float(np.percentile(a, 90)))


def attention_bytes(w, ctx_lens):
    """Algorithmic bytes of one attention call: the target KV read in place once,
    plus the block queries, the block's own K/V and the output."""
    from hybrid_mamba_attention_amd import workloads as wl
    e = 2 if w.dtype == "bf16" else 4
    io = (w.C * w.K * w.Hq * w.D * 2 + w.C * w.K * w.Hkv * w.D * 2) * e
    return wl.kv_bytes(w, ctx_lens) + io


def init_bytes(w):
    e = 2 if w.dtype == "bf16" else 4
    return w.d_model * w.S * e + w.C * w.d_model * e + w.C * w.S * 4


def ssd_bytes(w):
    e = 2 if w.dtype == "bf16" else 4
    return (w.C * w.S * 4 + w.C * w.K * w.H * w.P * (e + 4) + 2 * w.C * w.K * w.ng * w.N * e
            + w.C * w.K * w.H * 4)


def plan_summary(plan, C):
    """The work plan's shape: ranges used and their capacity, requests cut
    into pieces by range boundaries, and the pieces in all."""
    pieces = plan[4 + 2 * C:4 + 3 * C]
    return dict(ranges=int(plan[0]), range_capacity=int(plan[3]), granule_slabs=int(plan[1]),
                requests_cut=int((pieces > 1).sum()), pieces=int(pieces.sum()))


def measure(w, inp, args, torch, flush, with_parts=True):
    from hybrid_mamba_attention_amd import ops
    layer, t = build_layer(inp, args.kv_split_pages, torch)
    steps = stats(timed(layer, args.steps, args.warmup, flush, torch))
    layer.graph()
    res = dict(step=steps, step_graph=stats(timed(layer.launch_graph, args.steps, args.warmup, flush, torch)))
    if with_parts:
        ws = layer.workspace
        pt, cl = dev(inp.page_table, torch), dev(inp.ctx_lens, torch)
        out = torch.empty_like(t["q"])

        def attn():
            ops.block_attn_inplace(t["q"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], pt, cl,
                                   max_ctx=inp.max_ctx, kv_split_pages=args.kv_split_pages, out=out,
                                   workspace=ws)
        h0 = torch.empty((w.C, w.S), dtype=torch.float32, device="cuda")
        y = torch.empty((w.C, w.K, w.H, w.P), dtype=torch.float32, device="cuda")
        res["attention"] = stats(timed(attn, args.steps, args.warmup, flush, torch))
        res["init_state"] = stats(timed(lambda: ops.init_state(t["u"], t["w_init"], h0), args.steps,
                                        args.warmup, flush, torch))
        res["ssd_scan"] = stats(timed(lambda: ops.ssd_scan(t["x"], t["delta"], t["A"], t["B"], t["Cm"],
                                                           chunk=w.chunk, h0=h0, y=y),
                                      args.steps, args.warmup, flush, torch))
        res["plan"] = plan_summary(layer.plan().cpu().numpy(), w.C)
    del layer, t
    torch.cuda.empty_cache()
    return res


def part_metrics(w, inp, r):
    """Per-kernel figures of one measure() result: event times, algorithmic
    bytes and their rate, and the projection's matrix-core share."""
    from hybrid_mamba_attention_amd import workloads as wl
    att_b = attention_bytes(w, inp.ctx_lens)
    kv_b = wl.kv_bytes(w, inp.ctx_lens)
    att_ms, init_ms, ssd_ms = r["attention"]["mean"], r["init_state"]["mean"], r["ssd_scan"]["mean"]
    peak = BF16_DENSE_TFLOPS if w.dtype == "bf16" else FP32_MATRIX_TFLOPS
    ib = init_bytes(w)
    return {
        "attention": dict(ms=att_ms, algorithmic_bytes=att_b, kv_bytes=kv_b,
                          gbs=att_b / (att_ms * 1e-3) / 1e9, hbm_frac=att_b / (att_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          kv_frac=kv_b / (att_ms * 1e-3) / 1e9 / HBM_PEAK_GBS),
        "init_state": dict(ms=init_ms, algorithmic_bytes=ib, gbs=ib / (init_ms * 1e-3) / 1e9,
                           hbm_frac=ib / (init_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           mfma_frac=2.0 * w.C * w.d_model * w.S / (init_ms * 1e-3) / 1e12 / peak,
                           mfma_peak_tflops=peak),
        "ssd_scan": dict(ms=ssd_ms, algorithmic_bytes=ssd_bytes(w), gbs=ssd_bytes(w) / (ssd_ms * 1e-3) / 1e9),
    }


def measure_configs(args, torch, flush, main_idx, main_result, main_inp):
    """All five workloads, one entry each: the layer step and its parts."""
    from hybrid_mamba_attention_amd import workloads as wl
    out = {}
    for idx in sorted(wl.WORKLOADS):
        w = wl.WORKLOADS[idx]
        print(f"[bench] workload {idx} {w.name}", file=sys.stderr, flush=True)
        inp = main_inp if idx == main_idx else wl.make_inputs(w)
        r = main_result if idx == main_idx else measure(w, inp, args, torch, flush)
        ms = r["step"]["mean"]
        out[str(idx)] = dict(workload=w.name, C=w.C, K=w.K, ctx=list(w.ctx), dtype=w.dtype,
                             ctx_tokens=int(inp.ctx_lens.sum()), ms_per_step=ms,
                             ms_per_step_graph=r["step_graph"]["mean"],
                             block_tokens_per_s=w.C * w.K / (ms * 1e-3), plan=r["plan"],
                             kernels=part_metrics(w, inp, r))
        if inp is not main_inp:
            del inp
        torch.cuda.empty_cache()
    return out


def host_metadata(torch):
    """Where the line was measured: the host CPU and thread count the CPU
    baseline runs on, NumPy and its BLAS, and the ROCm / HIP / torch builds."""
    import platform
    import numpy as np
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [dict(library=os.path.basename(i.get("filepath", "")), internal_api=i.get("internal_api"),
                     version=i.get("version"), threads=i.get("num_threads"))
                for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        pass
    rocm = None
    for f in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(f):
            rocm = open(f).read().strip()
            break
    return dict(cpu_model=cpu, host_threads=len(os.sched_getaffinity(0)), python=platform.python_version(),
                numpy=np.__version__, blas=blas, rocm=rocm, hip_runtime=torch.version.hip, torch=torch.__version__,
                gpu=torch.cuda.get_device_name(0))


def measure_variants(w, inp, args, torch, flush):
    """The layer with the block-causal mask, the direct-reuse-only ablation,
    and the attention over the same pools viewed as 64-token pages."""
    import numpy as np
    from hybrid_mamba_attention_amd import ops
    out = {}
    for name, kw in (("block_causal", dict(block_causal=True)), ("direct_reuse_only", dict(no_init=True))):
        layer, t = build_layer(inp, args.kv_split_pages, torch, **kw)
        st = stats(timed(layer, args.steps, args.warmup, flush, torch))
        out[name] = dict(ms_per_step=st["mean"], block_tokens_per_s=w.C * w.K / (st["mean"] * 1e-3))
        del layer, t
        torch.cuda.empty_cache()
    # 64-token pages: the pool memory regrouped four 16-token pages at a time
    # and a fresh shuffled table of 64-token pages (same context lengths; the
    # token values differ, which does not change the work)
    t = {k: dev(inp.arrays[k], torch) for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
    n64 = t["k_cache"].shape[0] // 4
    kc = t["k_cache"][:4 * n64].view(n64, 64, w.Hkv, w.D)
    vc = t["v_cache"][:4 * n64].view(n64, 64, w.Hkv, w.D)
    need = [-(-int(c) // 64) for c in inp.ctx_lens]
    if sum(need) <= n64:
        perm = np.random.default_rng(w.seed + 64).permutation(n64)
        pt = np.full((w.C, max(need)), 0, np.int32)
        off = 0
        for b, n in enumerate(need):
            pt[b, :n] = perm[off:off + n]
            off += n
        pt, cl = dev(pt, torch), dev(inp.ctx_lens, torch)
        o = torch.empty_like(t["q"])
        ws = None

        def attn64():
            ops.block_attn_inplace(t["q"], t["k_blk"], t["v_blk"], kc, vc, pt, cl, max_ctx=inp.max_ctx,
                                   out=o, workspace=ws)
        _, ws = ops.block_attn_inplace(t["q"], t["k_blk"], t["v_blk"], kc, vc, pt, cl, max_ctx=inp.max_ctx, out=o)
        st = stats(timed(attn64, args.steps, args.warmup, flush, torch))
        out["page_size_64"] = dict(attention_ms=st["mean"],
                                   algorithmic_gbs=attention_bytes(w, inp.ctx_lens) / (st["mean"] * 1e-3) / 1e9)
    del t
    torch.cuda.empty_cache()
    return out


def block_flops(w):
    """Matrix-core flops of one Mamba-2 block call: both projections."""
    from hybrid_mamba_attention_amd import workloads as wl
    d_inner, _, d_proj = wl.block_sizes(w)
    T = w.C * w.K
    return 2 * T * w.d_model * d_proj + 2 * T * d_inner * w.d_model


def measure_block(w, args, torch, flush):
    """The Mamba-2 block around the scan (projections, conv, scan, gated norm)."""
    from hybrid_mamba_attention_amd import ops, workloads as wl
    a = wl.make_block_inputs(w)
    f32 = lambda k: dev(a[k].astype("float32"), torch)
    blk = ops.MambaBlock(hidden=dev(a["hidden"], torch), w_in=dev(a["w_in"], torch), conv_w=f32("conv_w"),
                         conv_b=f32("conv_b"), dt_bias=f32("dt_bias"), A=f32("A"), Dskip=f32("Dskip"),
                         h0=f32("h0"), norm_w=f32("norm_w"), w_out=dev(a["w_out"], torch), eps=a["eps"],
                         H=w.H, P=w.P, N=w.N, ng=w.ng, chunk=w.chunk, want_final=True)
    st = stats(timed(blk, args.steps, args.warmup, flush, torch))
    fl = block_flops(w)
    d_inner, _, d_proj = wl.block_sizes(w)
    e = 2 if w.dtype == "bf16" else 4
    wbytes = (d_proj + d_inner) * w.d_model * e
    del blk
    torch.cuda.empty_cache()
    return dict(ms=st["mean"], block_tokens_per_s=w.C * w.K / (st["mean"] * 1e-3),
                projection_gflop=fl / 1e9, tflops_whole_block=fl / (st["mean"] * 1e-3) / 1e12,
                mfma_frac_whole_block=fl / (st["mean"] * 1e-3) / 1e12 / BF16_DENSE_TFLOPS,
                weight_bytes=wbytes)


def measure_injection(w, args, torch, flush, Cs=(4, 8, 16, 32, 64, 128)):
    """The contrast workload: one drafter-side KV injection step (hspec_kv_inject)
    of the K block positions per request after a ctx-token context, at each C.
    Each request's new positions fall in one page of its own, so the pools need
    only C pages; the projection and the paged writes are the full step."""
    import numpy as np
    from hybrid_mamba_attention_amd import ops
    ctx = w.ctx[1] if w.ctx[0] == "fixed" else w.ctx[2]
    e = 2 if w.dtype == "bf16" else 4
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {}
    for C in Cs:
        g = torch.Generator(device="cuda").manual_seed(5000 + C)
        hidden = torch.randn((C, w.K, w.d_model), generator=g, device="cuda").to(dt)
        w_kv = (0.02 * torch.randn((2 * w.Hkv * w.D, w.d_model), generator=g, device="cuda")).to(dt)
        kc = torch.zeros((C, 16, w.Hkv, w.D), dtype=dt, device="cuda")
        vc = torch.zeros_like(kc)
        max_pages = (ctx + w.K + 15) // 16
        pt = np.full((C, max_pages), -1, np.int32)
        pt[:, ctx // 16] = np.arange(C)          # ctx % 16 + K <= 16 here (ctx 8192, K 16)
        pt = torch.from_numpy(pt).cuda()
        start = torch.full((C,), ctx, dtype=torch.int32, device="cuda")
        ws = ops.kv_inject(hidden, w_kv, kc, vc, pt, start)
        st = stats(timed(lambda: ops.kv_inject(hidden, w_kv, kc, vc, pt, start, workspace=ws),
                         args.steps, args.warmup, flush, torch))
        out[str(C)] = dict(ms=st["mean"], written_bytes=C * w.K * 2 * w.Hkv * w.D * e,
                           drafter_cache_bytes_one_layer=C * (ctx + w.K) * 2 * w.Hkv * w.D * e)
        del hidden, w_kv, kc, vc, pt, start, ws
    torch.cuda.empty_cache()
    lo, hi = str(Cs[0]), str(Cs[-1])
    return dict(per_C=out, growth_C4_to_C128=out[hi]["ms"] / out[lo]["ms"],
                extra_kv_bytes_per_token_per_layer=2 * w.Hkv * w.D * e,
                note="what H-Spec avoids: per-position projection into a drafter-side paged KV cache")


def measure_stack(w, args, torch, flush, kinds=("MA", "MA"), Cs=(1, 4, 16, 64, 128)):
    """The drafter stack (hspec_draft_stack) eager on one stream and as one HIP
    graph (hspec_draft_stack_graph), at several C, ctx as the workload.  Inputs
    are drawn on the device from seeded generators (N(0,1) activations and
    pools, N(0, 0.02^2) weights, the block recipe's fp32 parameters); each
    attention half reads its own pools through one shared shuffled page table."""
    from hybrid_mamba_attention_amd import ops, workloads as wl
    ctx = w.ctx[1] if w.ctx[0] == "fixed" else w.ctx[2]
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(w.seed + 4242)
    rn = lambda shape, std=1.0: (std * torch.randn(shape, generator=g, device="cuda")).to(dt)
    rf = lambda shape: torch.randn(shape, generator=g, device="cuda")
    d_inner, conv_dim, d_proj = wl.block_sizes(w)
    Cmax = max(Cs)
    pages_per = (ctx + 15) // 16
    layers = []
    for kind in kinds:
        L = dict(pre_norm_w=1.0 + 0.1 * rf(w.d_model))
        if "M" in kind:
            L.update(w_init=rn((w.d_model, w.S), 0.02), w_in=rn((d_proj, w.d_model), 0.02),
                     conv_w=torch.rand((conv_dim, 4), generator=g, device="cuda") - 0.5,
                     conv_b=torch.rand(conv_dim, generator=g, device="cuda") - 0.5,
                     dt_bias=torch.full((w.H,), wl.BLOCK_DT_BIAS, device="cuda"),
                     A=-torch.exp(torch.rand(w.H, generator=g, device="cuda")), Dskip=rf(w.H),
                     norm_w=1.0 + 0.1 * rf(d_inner), w_out=rn((w.d_model, d_inner), 0.02))
        if "A" in kind:
            L.update(wq=rn((w.Hq * w.D, w.d_model), 0.02), wk=rn((w.Hkv * w.D, w.d_model), 0.02),
                     wv=rn((w.Hkv * w.D, w.d_model), 0.02), wo=rn((w.d_model, w.Hq * w.D), 0.02),
                     k_cache=rn((Cmax * pages_per, 16, w.Hkv, w.D)), v_cache=rn((Cmax * pages_per, 16, w.Hkv, w.D)))
        layers.append(L)
    perm = torch.randperm(Cmax * pages_per, generator=g, device="cuda").to(torch.int32)
    pt_all = perm.view(Cmax, pages_per)
    out = {}
    for C in Cs:
        print(f"[bench] stack C={C}", file=sys.stderr, flush=True)
        st = ops.DraftStack(hidden_in=rn((C, w.K, w.d_model)), u=rn((C, w.d_model)), layers=layers,
                            page_table=pt_all[:C].contiguous(),
                            ctx_lens=torch.full((C,), ctx, dtype=torch.int32, device="cuda"), max_ctx=ctx,
                            H=w.H, P=w.P, N=w.N, chunk=w.chunk, Hq=w.Hq, Hkv=w.Hkv, D=w.D, eps=wl.BLOCK_EPS)
        eager = stats(timed(st, args.steps, args.warmup, flush, torch))
        st.graph()
        graph = stats(timed(st.launch_graph, args.steps, args.warmup, flush, torch))
        out[str(C)] = dict(eager_ms=eager["mean"], graph_ms=graph["mean"],
                           block_tokens_per_s=C * w.K / (graph["mean"] * 1e-3))
        del st
    del layers, pt_all, perm
    torch.cuda.empty_cache()
    return dict(layers="+".join(kinds), ctx=ctx, per_C=out)


# ----------------------------------------------------------------------------
# counters (traffic) from the committed rocprofv3 summary, if still current
# ----------------------------------------------------------------------------

def stream_read_probe(torch, gib=4, reps=6):
    """Sustained HBM read bandwidth of this GPU (hspec_probe_stream_read over a
    buffer far larger than L2 and the Infinity Cache), median of reps runs."""
    import numpy as np
    from hybrid_mamba_attention_amd import ops
    print("[bench] stream-read probe", file=sys.stderr, flush=True)
    buf = torch.zeros(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ts = []
    for i in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ops.stream_read_probe(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        if i:
            ts.append(e0.elapsed_time(e1))
    nbytes = buf.numel()
    del buf
    torch.cuda.empty_cache()
    ms = float(np.median(ts))
    return dict(bytes=nbytes, ms=ms, gbs=nbytes / (ms * 1e-3) / 1e9)


def kernel_source_hash():
    """Hash of what k_block_attn is compiled from: attention.hip, common.h and
    the AttnArgs definition in kernels.h (the rest of that header serves other
    kernels), so the committed counters are used only while they still apply."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hybrid_mamba_attention_amd", "csrc")
    for f in ("attention.hip", "common.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    text = open(os.path.join(csrc, "kernels.h")).read()
    i = text.index("struct AttnArgs")
    h.update(text[i:text.index("};", i) + 2].encode())
    return h.hexdigest()[:16]


def mfma_source_hash():
    """Hash of the matrix-core kernels' sources (the state projection and the
    block GEMMs), so the committed MFMA counters are used only while they apply."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hybrid_mamba_attention_amd", "csrc")
    for f in ("init_state.hip", "gemm.hip", "common.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def mfma_from_profile(workload_name):
    """Matrix-core utilisation per kernel from the committed counter record
    (rocprofv3: SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs), or
    None once the kernels have changed since it was taken."""
    path = os.path.join(PROFILE_DIR, f"mfma_{workload_name}_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != mfma_source_hash():
        return None
    return {k: dict(mfma_util=v["mfma_util"], counted_flops=v["counted_flops"], avg_us=v["avg_us"])
            for k, v in rec["kernels"].items()}


def traffic_from_profile(workload_name):
    path = os.path.join(PROFILE_DIR, f"k_block_attn_{workload_name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------
# profiles/ records from rocprofv3 output (no GPU work)
# ----------------------------------------------------------------------------

SIMDS = 256 * 4          # MI355X: 256 CUs x 4 SIMDs
XCDS = 8                 # GRBM_GUI_ACTIVE is reported summed over the 8 XCDs' instances
KERNEL_KEYS = ("k_block_attn", "k_attn_merge", "k_init_wide", "k_init_state", "k_ssd_scan", "k_scan_merge",
               "k_gemm_tn", "k_splitk_sum", "k_gate_norm", "__amd_rocclr_copyBuffer")
DEFAULT_WORKLOAD = 3   # the C = 128, 8192-token batch the headline line measures
_BENCH = "python3 bench.py --steps {steps} --warmup {warmup} --no-sweep --no-cpu --no-variants --no-stack --no-configs"
# The passes the profiles/ summaries come from, each a run of its own, from the
# repository root on one MI355X with TMPDIR=/tmp (counters are never combined
# with trace domains; each --pmc set fits one hardware pass).
PROFILE_PASSES = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_trace -o run -- "
             + _BENCH.format(steps=10, warmup=3) + " --calib-copy",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof_fetch -o run -- "
             + _BENCH.format(steps=3, warmup=1) + " --no-block --no-inject --no-probe --calib-copy",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof_write -o run -- "
             + _BENCH.format(steps=3, warmup=1) + " --no-block --no-inject --no-probe --calib-copy",
    "mfma": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE "
            "--output-format csv -d gpurun_out/prof_mfma -o run -- "
            + _BENCH.format(steps=3, warmup=1) + " --no-inject --no-probe",
    "sq": "rocprofv3 --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU "
          "SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU GRBM_GUI_ACTIVE "
          "--output-format csv -d gpurun_out/prof_sq -o run -- "
          + _BENCH.format(steps=3, warmup=1) + " --no-block --no-inject --no-probe",
}


def profile_passes(workload_idx):
    """The passes of PROFILE_PASSES for a workload (the default one needs no flag)."""
    if workload_idx == DEFAULT_WORKLOAD:
        return dict(PROFILE_PASSES)
    return {k: v + f" --workload {workload_idx}" for k, v in PROFILE_PASSES.items()}


def _rocprof_csv(d, what):
    import glob
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{what}.csv"), recursive=True))
    if not hits:
        return []
    import csv
    with open(hits[0]) as f:
        return list(csv.DictReader(f))


def _short(name):
    for k in KERNEL_KEYS:
        if k in name:
            return k
    return None


def _instance(name):
    """A kernel's name with its template arguments, without the parameter list."""
    n = (name[5:] if name.startswith("void ") else name).replace("(anonymous namespace)::", "")
    return n.split("(")[0]


def _counter_table(d):
    """{(kernel, grid): {counter: [value per dispatch], "_us": [...], "_name": [...]}} of a --pmc run."""
    import collections
    per = collections.defaultdict(dict)
    for r in _rocprof_csv(d, "counter_collection"):
        k = _short(r["Kernel_Name"])
        if k is None:
            continue
        key = (k, int(r["Grid_Size"]), r["Dispatch_Id"])
        per[key][r["Counter_Name"]] = per[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        per[key]["_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per[key]["_name"] = _instance(r["Kernel_Name"])
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for (k, grid, _), cs in per.items():
        for c, v in cs.items():
            out[(k, grid)][c].append(v)
    return out


def _write(path, text, written):
    with open(path, "w") as fh:
        fh.write(text)
    written.append(path)


def _stats_md(d, w, written, passes):
    """Kernel-time table of a --kernel-trace --stats run."""
    rows = _rocprof_csv(d, "kernel_stats")
    if not rows:
        return
    lines = [f"# Kernel time summary: drafter layer and Mamba-2 block, workload {w.name}", "",
             "Command (from the repository root, on one MI355X; TMPDIR=/tmp):", "", "    " + passes["trace"], "",
             "The run times 10 drafter-layer calls and 10 calls of each of its entry points alone, then the "
             "Mamba-2 block (hspec_mamba_block) and the drafter-side KV-injection contrast at C = 4 ... 128, each "
             "call after a 2 GiB read that evicts L2 and the Infinity Cache (the at::native reduce_kernel rows); "
             "the 1 GiB __amd_rocclr_copyBuffer rows are the counter-calibration copy and the k_stream_read rows "
             "the bandwidth probe.", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"] if "Name" in r else r.get("KernelName", "")
        lines.append(f"| `{_instance(name)[:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    _write(os.path.join(PROFILE_DIR, f"layer_and_block_{w.name}_kernel_stats.md"), "\n".join(lines) + "\n", written)


def summarize_profiles(dirs, workload_idx):
    """Write the profiles/ records of the benchmarked workload from rocprofv3
    csv directories (the PROFILE_PASSES runs): the kernel-time table of the
    trace run; k_block_attn_<w>_traffic.{json,md} from the FETCH_SIZE and
    WRITE_SIZE runs with their calibration copy; mfma_<w>_counters.{json,md}
    (matrix-core busy share per kernel) and sq_<w>_counters.md (where the
    waves of the main kernels spend their cycles)."""
    import numpy as np
    from hybrid_mamba_attention_amd import workloads as wl
    w = wl.WORKLOADS[workload_idx]
    passes = profile_passes(workload_idx)
    inp = wl.make_inputs(w, parts=())
    alg = {"k_block_attn": attention_bytes(w, inp.ctx_lens), "k_init_wide": init_bytes(w),
           "k_ssd_scan": ssd_bytes(w)}
    tables = {d: _counter_table(d) for d in dirs}
    trace = {}
    written = []
    for d in dirs:
        for r in _rocprof_csv(d, "kernel_trace"):
            k = _short(r["Kernel_Name"])
            if k:
                trace.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        _stats_md(d, w, written, passes)

    def find(counter):
        for d, t in tables.items():
            if any(counter in cs for cs in t.values()):
                return d, t
        return None, None

    def main_grid(t, k):
        """The kernel's most frequent grid (the benchmarked workload's launch)."""
        grids = [(len(cs.get("_us", [])), g) for (kk, g), cs in t.items() if kk == k]
        return max(grids)[1] if grids else None

    fd, ft = find("FETCH_SIZE")
    wd, wt = find("WRITE_SIZE")
    if ft and wt:
        def calib(t, c):
            v = [max(cs[c]) for (k, g), cs in t.items() if k == "__amd_rocclr_copyBuffer" and c in cs]
            return max(v)
        copy_bytes = float(1 << 30)
        fetch_factor = copy_bytes / (calib(ft, "FETCH_SIZE") * 1024)
        write_factor = copy_bytes / (calib(wt, "WRITE_SIZE") * 1024)
        rec = dict(workload=w.name, source_hash=kernel_source_hash(), fetch_factor=fetch_factor,
                   write_factor=write_factor, kernels={},
                   fetch_command=passes["fetch"], write_command=passes["write"])
        for k in ("k_block_attn", "k_init_wide", "k_ssd_scan"):
            g = main_grid(ft, k)
            if g is None:
                continue
            fk = float(np.mean(ft[(k, g)]["FETCH_SIZE"]))
            wk = float(np.mean(wt[(k, g)]["WRITE_SIZE"])) if (k, g) in wt else 0.0
            hb = fk * 1024 * fetch_factor + wk * 1024 * write_factor
            rec["kernels"][k] = dict(grid_threads=g, fetch_kib=fk, write_kib=wk, hbm_bytes=hb,
                                     algorithmic_bytes=alg.get(k), ratio=hb / alg[k] if k in alg else None)
        rec["hbm_bytes_per_launch"] = rec["kernels"]["k_block_attn"]["hbm_bytes"]
        if "k_block_attn" in trace:
            rec["k_block_attn_avg_us_kernel_trace"] = float(np.mean(trace["k_block_attn"]))
        path = os.path.join(PROFILE_DIR, f"k_block_attn_{w.name}_traffic.json")
        json.dump(rec, open(path, "w"), indent=1)
        written.append(path)
        lines = [f"# HBM traffic per launch: workload {w.name}", "",
                 "Two counter passes, each in a run of its own (from the repository root, on one MI355X; TMPDIR=/tmp):",
                 "", "    " + passes["fetch"], "    " + passes["write"], "",
                 "Calibration: the same runs launch a plain 1 GiB device copy (__amd_rocclr_copyBuffer). "
                 f"It reads {calib(ft, 'FETCH_SIZE'):.1f} KiB by FETCH_SIZE and writes {calib(wt, 'WRITE_SIZE'):.1f} KiB "
                 f"by WRITE_SIZE per dispatch, so bytes = FETCH_SIZE x 1024 x {fetch_factor:.4f} and "
                 f"WRITE_SIZE x 1024 x {write_factor:.4f} on this chip.", "",
                 "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | algorithmic bytes | ratio |",
                 "|---|---|---|---|---|---|"]
        for k, v in rec["kernels"].items():
            lines.append(f"| `{k}` | {v['fetch_kib']:.1f} | {v['write_kib']:.1f} | {v['hbm_bytes']:.4e} | "
                         f"{v['algorithmic_bytes']:.4e} | {v['ratio']:.3f} |")
        if "k_block_attn_avg_us_kernel_trace" in rec:
            lines += ["", f"Average k_block_attn duration in the kernel-trace run ({passes['trace'].split(' -d ')[0]} ...): "
                      f"{rec['k_block_attn_avg_us_kernel_trace']:.1f} us."]
        lines += ["", f"Attention sources hash (bench.py kernel_source_hash): {rec['source_hash']}."]
        _write(os.path.join(PROFILE_DIR, f"k_block_attn_{w.name}_traffic.md"), "\n".join(lines) + "\n", written)
    md_, mt = find("SQ_INSTS_VALU_MFMA_MOPS_BF16")
    if mt:
        rec = dict(workload=w.name, source_hash=mfma_source_hash(), simds=SIMDS, xcds=XCDS,
                   command=passes["mfma"], kernels={})
        for (k, g), cs in sorted(mt.items()):
            if k == "__amd_rocclr_copyBuffer" or "SQ_VALU_MFMA_BUSY_CYCLES" not in cs:
                continue
            busy = float(np.mean(cs["SQ_VALU_MFMA_BUSY_CYCLES"]))
            gui = float(np.mean(cs["GRBM_GUI_ACTIVE"])) / XCDS if "GRBM_GUI_ACTIVE" in cs else None
            mops = float(np.mean(cs.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0.0])))
            us = float(np.mean(cs["_us"]))
            rec["kernels"][f"{k} grid {g}"] = dict(
                instance=cs["_name"][0], dispatches=len(cs["SQ_VALU_MFMA_BUSY_CYCLES"]), avg_us=us,
                mfma_busy_cycles=busy, gui_active_cycles_per_xcd=gui,
                mfma_util=busy / (gui * SIMDS) if gui else None, counted_flops=mops * 512,
                counted_tflops=mops * 512 / (us * 1e-6) / 1e12 if us else None)
        path = os.path.join(PROFILE_DIR, f"mfma_{w.name}_counters.json")
        json.dump(rec, open(path, "w"), indent=1)
        written.append(path)
        lines = [f"# Matrix-core utilisation per kernel: workload {w.name}", "",
                 "Command (from the repository root, on one MI355X; TMPDIR=/tmp):", "", "    " + passes["mfma"], "",
                 "Per dispatch, averaged per kernel and grid (threads). `MFMA busy` = SQ_VALU_MFMA_BUSY_CYCLES "
                 f"/ (GRBM_GUI_ACTIVE of one XCD x {SIMDS} SIMDs): the csv gives GRBM_GUI_ACTIVE summed over the "
                 f"{XCDS} XCDs, 8 x 2.4 GHz x the kernel's time.  `counted TFLOP/s` = SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                 "x 512 flop / kernel time (dense bf16 peak 2500).", "",
                 "| kernel | grid | dispatches | avg us | MFMA busy | counted TFLOP/s |", "|---|---|---|---|---|---|"]
        for key, v in rec["kernels"].items():
            k, g = key.split(" grid ")
            lines.append(f"| `{v['instance'][:80]}` | {g} | {v['dispatches']} | {v['avg_us']:.1f} | "
                         f"{(v['mfma_util'] or 0) * 100:.1f}% | {(v['counted_tflops'] or 0):.0f} |")
        lines += ["", f"Matrix-core sources hash (bench.py mfma_source_hash): {rec['source_hash']}."]
        _write(os.path.join(PROFILE_DIR, f"mfma_{w.name}_counters.md"), "\n".join(lines) + "\n", written)
    sd, st = find("SQ_WAIT_INST_ANY")
    if st:
        lines = [f"# Where the waves spend their cycles: workload {w.name}", "",
                 "Command (from the repository root, on one MI355X; TMPDIR=/tmp):", "", "    " + passes["sq"], "",
                 "Per dispatch of each kernel's benchmarked launch, chip sums averaged over the dispatches, as "
                 "shares of SQ_WAVE_CYCLES (the cycles its waves were resident).  `MFMA busy` as in the "
                 "matrix-core table; `VALU / SIMD-cycle` = SQ_INSTS_VALU / (GRBM_GUI_ACTIVE of one XCD x SIMDs).", "",
                 "| kernel | dispatches | avg us | waiting (SQ_WAIT_INST_ANY) | VALU active | LDS active | "
                 "MFMA busy | VALU / SIMD-cycle |", "|---|---|---|---|---|---|---|---|"]
        for k in ("k_block_attn", "k_init_wide", "k_ssd_scan", "k_attn_merge", "k_scan_merge"):
            g = main_grid(st, k)
            if g is None:
                continue
            cs = st[(k, g)]
            m = {c: float(np.mean(v)) for c, v in cs.items() if c != "_name"}
            wc = m.get("SQ_WAVE_CYCLES", 0.0) or 1.0
            gui = m.get("GRBM_GUI_ACTIVE", 0.0) / XCDS or 1.0
            lines.append(f"| `{cs['_name'][0][:70]}` | {len(cs['_us'])} | {m['_us']:.1f} | "
                         f"{100 * m.get('SQ_WAIT_INST_ANY', 0) / wc:.1f}% | {100 * m.get('SQ_ACTIVE_INST_VALU', 0) / wc:.1f}% | "
                         f"{100 * m.get('SQ_ACTIVE_INST_LDS', 0) / wc:.1f}% | "
                         f"{100 * m.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / (gui * SIMDS):.1f}% | "
                         f"{m.get('SQ_INSTS_VALU', 0) / (gui * SIMDS):.3f} |")
        _write(os.path.join(PROFILE_DIR, f"sq_{w.name}_counters.md"), "\n".join(lines) + "\n", written)
    for p in written:
        print(p)


# ----------------------------------------------------------------------------
# CPU baseline: the oracle, untuned, on a bounded sample of the same workload
# ----------------------------------------------------------------------------

def cpu_baseline(w, inp, n_req, min_seconds=10.0, max_seconds=30.0):
    """The oracle (untuned) on batches of n_req requests of the workload, repeated
    over successive request batches until at least min_seconds of work."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    a = inp.arrays
    t0 = time.perf_counter()
    done = 0
    ctx_tokens = 0
    batch = 0
    while True:
        reqs = [(batch * n_req + i) % w.C for i in range(n_req)]
        sub = {k: a[k][reqs] for k in ("u", "x", "delta", "B", "Cm")}
        h0 = oracle.init_state(oracle.decode(sub["u"], w.dtype), oracle.decode(a["w_init"], w.dtype))
        oracle.ssd_recurrence(oracle.decode(sub["x"], w.dtype), sub["delta"], a["A"],
                              oracle.decode(sub["B"], w.dtype), oracle.decode(sub["Cm"], w.dtype),
                              h0=h0.reshape(n_req, w.H, w.P, w.N))
        oracle.block_attention(a["q"], a["k_blk"], a["v_blk"], a["k_cache"], a["v_cache"], inp.page_table,
                               inp.ctx_lens, dtype=w.dtype, requests=reqs)
        done += n_req
        ctx_tokens += int(inp.ctx_lens[reqs].sum())
        batch += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or dt * (batch + 1) / batch > max_seconds:
            break
    return dict(value=done * w.K / dt, unit="drafted block-tokens/s", cores=int(cores), kind="oracle",
                sample=f"{batch} batch(es) of {n_req} requests of {w.name} ({done} request-layers: projection "
                       f"incl. the full W_init decode per batch, scan, attention over {ctx_tokens} context "
                       f"tokens); {dt:.1f} s")


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the drafter layer shards by request across GPUs with no exchange).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from hybrid_mamba_attention_amd import ops, workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ops.lib()
    flush_buf = torch.ones(512 * 1024 * 1024, dtype=torch.float32, device="cuda")  # 2 GiB
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")

    def flush():
        if not args.no_flush:
            torch.sum(flush_buf, dim=0, out=flush_out)

    if args.calib_copy:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch
        # calibrate the HBM-traffic counters of the kernels profiled alongside
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            flush()
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    probe = None if args.no_probe else stream_read_probe(torch)
    w = wl.WORKLOADS[args.workload]
    print(f"[bench] drawing inputs for {w.name}", file=sys.stderr, flush=True)
    inp = wl.make_inputs(w)
    print("[bench] timing the layer", file=sys.stderr, flush=True)
    r = measure(w, inp, args, torch, flush)
    ms = r["step"]["mean"]
    tokens = w.C * w.K
    kv_b = wl.kv_bytes(w, inp.ctx_lens)
    parts = part_metrics(w, inp, r)
    att = parts["attention"]
    achieved = att["gbs"]
    traffic = traffic_from_profile(w.name)
    kernels = {
        "attention (k_block_attn; k_attn_merge when a request spans ranges)": att,
        "init_state (k_init_wide)": parts["init_state"],
        "ssd_scan (k_ssd_scan)": parts["ssd_scan"],
    }
    line = {
        "metric": "drafted block-tokens/sec per drafter layer",
        "value": tokens / (ms * 1e-3),
        "unit": "block-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": w.name, "C": w.C, "K": w.K, "ctx": list(w.ctx), "Hq": w.Hq, "Hkv": w.Hkv,
                   "D": w.D, "d_model": w.d_model, "mamba_H_P_N_chunk": [w.H, w.P, w.N, w.chunk],
                   "kv_bytes_in_place": kv_b, "w_init_bytes": wl.w_init_bytes(w),
                   "work_plan": r["plan"], "cache_flush_between_steps": not args.no_flush},
        "step_ms": r["step"],
        "step_ms_graph": r["step_graph"],
        "kernels": kernels,
        "kv_read_gbs": kv_b / (att["ms"] * 1e-3) / 1e9,
        "kv_read_frac_of_peak": att["kv_frac"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "k_block_attn"},
        "mfma_counters": mfma_from_profile(w.name),
        "host": host_metadata(torch),
    }
    if probe is not None:
        line["stream_read_probe"] = dict(probe, attention_frac_of_probe=achieved / probe["gbs"])
    if not args.no_variants:
        print("[bench] timing the layer variants", file=sys.stderr, flush=True)
        line["variants"] = measure_variants(w, inp, args, torch, flush)
    if not args.no_block:
        print("[bench] timing the Mamba-2 block", file=sys.stderr, flush=True)
        line["mamba_block"] = measure_block(w, args, torch, flush)
    if not args.no_inject:
        print("[bench] timing the drafter-side KV injection contrast", file=sys.stderr, flush=True)
        line["kv_injection_contrast"] = measure_injection(w, args, torch, flush)
    if not args.no_stack:
        print("[bench] timing the drafter stack", file=sys.stderr, flush=True)
        line["stack"] = measure_stack(w, args, torch, flush)
    if not args.no_sweep:
        sweep = {}
        for C in [int(c) for c in args.sweep.split(",")]:
            ws = wl.sweep_workload(C) if C != w.C or args.workload != 3 else w
            print(f"[bench] sweep C={C}", file=sys.stderr, flush=True)
            si = inp if ws is w else wl.make_inputs(ws)
            sr = r if ws is w else measure(ws, si, args, torch, flush, with_parts=True)
            sms = sr["step"]["mean"]
            akv = wl.kv_bytes(ws, si.ctx_lens)
            if not args.no_block:
                sweep_block = line["mamba_block"]["ms"] if ws is w else measure_block(ws, args, torch, flush)["ms"]
            sweep[str(C)] = dict(block_tokens_per_s=ws.C * ws.K / (sms * 1e-3), ms_per_step=sms,
                                 ms_per_step_graph=sr["step_graph"]["mean"],
                                 attention_ms=sr["attention"]["mean"], init_ms=sr["init_state"]["mean"],
                                 kv_read_gbs=akv / (sr["attention"]["mean"] * 1e-3) / 1e9,
                                 kv_read_frac=akv / (sr["attention"]["mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS)
            if not args.no_block:
                sweep[str(C)]["mamba_block_ms"] = sweep_block
            if si is not inp:
                del si
        line["sweep_ctx8192"] = sweep
    if not args.no_configs:
        line["configs"] = measure_configs(args, torch, flush, args.workload, r, inp)
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, inp, n_req=min(w.C, 64))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
