"""The C ABI on the host (no GPU work): the library loads, exports every entry
point include/hspec.h declares, and rejects bad arguments with the documented
status before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

from hybrid_mamba_attention_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("hspec.h", "hspec_probe.h")]
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = 1 << 20   # aligned, never dereferenced on the host (validation fails or size query)


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(hspec_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_loads_and_exports_every_declared_symbol():
    L = ops.lib()
    names = declared_functions()
    assert {"hspec_init_state", "hspec_ssd_scan", "hspec_block_attn_inplace",
            "hspec_draft_layer", "hspec_mamba_block", "hspec_kv_inject", "hspec_draft_stack",
            "hspec_draft_stack_graph", "hspec_graph_launch", "hspec_graph_destroy",
            "hspec_probe_stream_read", "hspec_probe_lds_pattern"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in hspec.h but not exported"
    assert L.hspec_abi_version() == ops.ABI_VERSION == 8
    assert L.hspec_layer_args_size() == ctypes.sizeof(ops.LayerArgs)
    assert L.hspec_mamba_args_size() == ctypes.sizeof(ops.MambaArgs)
    assert L.hspec_stack_args_size() == ctypes.sizeof(ops.StackArgs)
    assert L.hspec_status_string(-2) == b"HSPEC_ERR_UNSUPPORTED"


def _init(**kw):
    a = dict(stream=None, dtype=1, C=4, d=4096, S=32768, u=FAKE, w=FAKE, h0=FAKE)
    a.update(kw)
    return ops.lib().hspec_init_state(a["stream"], a["dtype"], a["C"], a["d"], a["S"], a["u"], a["w"], a["h0"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), INVALID), (dict(C=0), INVALID), (dict(u=None), INVALID),
    (dict(h0=FAKE + 4), INVALID), (dict(d=100), UNSUPPORTED), (dict(S=100), UNSUPPORTED),
    # the kernels' 32-bit row offsets and grid size bound S and C (a valid
    # shape would launch: this entry point has no size query)
    (dict(S=(1 << 25) + 64), UNSUPPORTED), (dict(C=(1 << 16) + 1), UNSUPPORTED),
])
def test_init_state_validation(kw, code):
    assert _init(**kw) == code


def _ssd(no_y=False, **kw):
    a = dict(dtype=1, C=2, K=16, H=16, P=64, ng=1, N=32, chunk=16)
    a.update(kw)
    # x, delta, A, B, Cm, Dskip, h0, y, h_final
    ptrs = [FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None if no_y else FAKE, None]
    return ops.lib().hspec_ssd_scan(None, a["dtype"], a["C"], a["K"], a["H"], a["P"], a["ng"],
                                    a["N"], a["chunk"], *ptrs)


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), INVALID), (dict(ng=3), INVALID), (dict(no_y=True), INVALID),
    (dict(chunk=12), UNSUPPORTED), (dict(chunk=128), UNSUPPORTED), (dict(P=256), UNSUPPORTED),
    # chunks of 32 and 64 take states of up to 64 with N % 4 == 0
    (dict(chunk=32, N=128), UNSUPPORTED), (dict(chunk=64, N=66), UNSUPPORTED),
])
def test_ssd_validation(kw, code):
    assert _ssd(**kw) == code


def _attn(ws=None, nbytes=0, **kw):
    a = dict(dtype=1, C=4, K=16, Hq=32, Hkv=8, D=128, ps=16 * 8 * 128, ts=8 * 128, hs=128,
             num_pages=100, max_pages=64, max_ctx=1000, split=0, scale=0.0, causal=0, page=16)
    a.update(kw)
    n = ctypes.c_size_t(nbytes)
    code = ops.lib().hspec_block_attn_inplace(
        None, a["dtype"], a["C"], a["K"], a["Hq"], a["Hkv"], a["D"], FAKE, FAKE, FAKE, FAKE, FAKE,
        a["ps"], a["ts"], a["hs"], a["num_pages"], a["page"], FAKE, a["max_pages"], FAKE, a["max_ctx"],
        a["split"], a["scale"], a["causal"], FAKE, ws, ctypes.byref(n))
    return code, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=30), INVALID), (dict(ts=100), INVALID), (dict(max_pages=10), INVALID),
    (dict(scale=-1.0), INVALID), (dict(split=-1), INVALID), (dict(K=0), INVALID),
    (dict(causal=2), INVALID), (dict(causal=-1), INVALID),
    (dict(page=0), INVALID), (dict(page=48), UNSUPPORTED), (dict(page=8), UNSUPPORTED),
    (dict(page=512), UNSUPPORTED), (dict(page=32, max_pages=31), INVALID),
    (dict(D=96), UNSUPPORTED), (dict(K=65), UNSUPPORTED), (dict(Hq=64, Hkv=2, K=16), UNSUPPORTED),
    # a slab's 16 row offsets are 32-bit byte offsets
    (dict(ts=1 << 26), OK), (dict(ts=(1 << 26) + 8), UNSUPPORTED),
])
def test_attention_validation(kw, code):
    assert _attn(**kw)[0] == code


def _ws_expect(C, w_max, rows, Hkv=8, D=128, esize=2):
    """Plan, then the pieces' outputs in the activation dtype (esize bytes) and
    their fp32 (m, l)."""
    up = lambda x: -(-x // 256) * 256
    plan = up((4 + 3 * C + w_max + 1) * 4)
    if w_max == 1:
        return plan
    return plan + up(2 * w_max * Hkv * rows * D * esize) + up(2 * w_max * Hkv * rows * 2 * 4)


def test_attention_workspace_query():
    """The workspace holds the int32 plan (4 + 3C + w_max + 1 entries) and,
    when a request can span ranges, partials for two slots per range (bf16
    outputs, fp32 (m, l)).
    C = 4, K = 16, max_ctx = 1000: a request's keys are 63 + 1 slabs, 32
    granules of 2 slabs; the batch at most 128 granules."""
    code, n = _attn(split=32)                           # 32 pages = 16 granules per range: 8 ranges
    assert code == OK and n == _ws_expect(4, 8, 64)
    code0, n0 = _attn(split=0)                          # automatic: at most floor(4 * (32 + 6) / 8) = 19 ranges
    assert code0 == OK and n0 == _ws_expect(4, 19, 64)
    code1, n1 = _attn(split=1000)                       # one range for the whole batch: no partials
    assert code1 == OK and n1 == _ws_expect(4, 1, 64)
    # 128 query rows per kv head: a charge of ceil(24/2) = 12 units per request,
    # at most floor(4 * (32 + 12) / 8) = 22 ranges
    code2, n2 = _attn(split=0, Hq=64)
    assert code2 == OK and n2 == _ws_expect(4, 22, 128)
    # a real (non-NULL) workspace that is too small is refused before any launch
    assert _attn(ws=FAKE, nbytes=n - 1, split=32)[0] == WORKSPACE


def test_probe_validation():
    f = ops.lib().hspec_probe_stream_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert f(None, FAKE, 0, FAKE) == INVALID
    assert f(None, FAKE, 100, FAKE) == INVALID          # not a multiple of 16
    assert f(None, FAKE + 8, 1 << 20, FAKE) == INVALID  # misaligned
    assert f(None, None, 1 << 20, FAKE) == INVALID
    g = ops.lib().hspec_probe_lds_pattern
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_uint32), ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    good = (ctypes.c_uint32 * 64)(*[16 * l for l in range(64)])
    bad_align = (ctypes.c_uint32 * 64)(*([8] + [16 * l for l in range(1, 64)]))
    past_end = (ctypes.c_uint32 * 64)(*([16384] + [0] * 63))
    assert g(None, 3, good, 64, 1, FAKE) == INVALID            # no such kind
    assert g(None, 0, good, 12, 1, FAKE) == INVALID            # not a multiple of 8
    assert g(None, 0, good, 64, 0, FAKE) == INVALID            # empty grid
    assert g(None, 0, good, 64, 1, None) == INVALID            # no sink
    assert g(None, 0, bad_align, 64, 1, FAKE) == INVALID       # 16-byte access at an 8-byte offset
    assert g(None, 2, past_end, 64, 1, FAKE) == INVALID        # 8-byte read past the 16 KiB


def _layer(**kw):
    """hspec_draft_layer size query (workspace NULL) with a valid bf16 shape."""
    a = ops.LayerArgs()
    a.dtype, a.C, a.K = 1, 4, 16
    a.d_model, a.H, a.P, a.ng, a.N, a.chunk = 4096, 32, 64, 1, 64, 16
    a.u = a.w_init = a.h0 = FAKE
    a.x = a.delta = a.A = a.B = a.Cm = a.y = FAKE
    a.Hq, a.Hkv, a.D = 32, 8, 128
    a.q = a.k_blk = a.v_blk = a.k_cache = a.v_cache = a.page_table = a.ctx_lens = a.out = FAKE
    a.page_stride, a.token_stride, a.head_stride = 16 * 8 * 128, 8 * 128, 128
    a.num_pages, a.max_pages, a.max_ctx, a.page_size = 100, 64, 1000, 16
    for k, v in kw.items():
        setattr(a, k, v)
    n = ctypes.c_size_t(0)
    return ops.lib().hspec_draft_layer(None, ctypes.byref(a), ctypes.byref(n)), n.value


def test_layer_validation_and_ablation():
    code, n = _layer()
    assert code == OK and n > 0
    # direct-reuse-only ablation: u and w_init both NULL, h0 may be NULL too
    assert _layer(u=None, w_init=None, h0=None) == (OK, n)
    assert _layer(u=None)[0] == INVALID
    assert _layer(w_init=None)[0] == INVALID
    assert _layer(h0=None)[0] == INVALID          # a1 runs and needs h0
    assert _layer(block_causal=1) == (OK, n)
    assert _layer(block_causal=3)[0] == INVALID


def _block(**kw):
    """hspec_mamba_block size query with a valid bf16 shape (C=128 requests)."""
    a = ops.MambaArgs()
    a.dtype, a.C, a.K, a.d_model = 1, 128, 16, 4096
    a.H, a.P, a.ng, a.N, a.chunk = 16, 64, 1, 32, 16
    a.hidden = a.w_in = a.conv_w = a.dt_bias = a.A = a.norm_w = a.w_out = a.out = FAKE
    a.norm_eps = 1e-5
    for k, v in kw.items():
        setattr(a, k, v)
    n = ctypes.c_size_t(0)
    return ops.lib().hspec_mamba_block(None, ctypes.byref(a), ctypes.byref(n)), n.value


def test_mamba_block_validation_and_workspace():
    code, n = _block()
    assert code == OK
    T, d_inner, ngN, H, d_proj = 128 * 16, 1024, 32, 16, 2128
    al = lambda b: -(-b // 256) * 256
    fixed = al(T * d_proj * 4) + al(T * d_inner * 4) + al(T * d_inner * 2)   # zx, y, normed
    assert n >= fixed and n - fixed < (1 << 30)           # + split-K partials, if any
    assert _block(conv_b=FAKE, Dskip=FAKE, h0=FAKE, h_final=FAKE) == (OK, n)
    assert _block(hidden=None)[0] == INVALID
    assert _block(A=None)[0] == INVALID
    assert _block(conv_w=FAKE + 4)[0] == INVALID           # float4 taps need 16-byte alignment
    assert _block(norm_w=FAKE + 4)[0] == INVALID
    assert _block(norm_eps=-1.0)[0] == INVALID
    assert _block(dtype=5)[0] == INVALID
    assert _block(ng=3)[0] == INVALID
    assert _block(d_model=4100)[0] == UNSUPPORTED          # d_model % 8
    assert _block(P=128 + 8)[0] == UNSUPPORTED             # scan limit P <= 128
    assert _block(chunk=32)[0] == UNSUPPORTED
    assert _block(C=(1 << 26) + 1, K=16)[0] == UNSUPPORTED  # C*K over 2^30 rows
    assert _block(C=1 << 25, K=16)[0] == UNSUPPORTED        # 2^29 rows x 4096 columns > 2^40
    assert _block(C=1 << 24, K=16)[0] == OK                 # 2^28 x 4096 = 2^40 (size query only)
    assert _block(workspace=FAKE, workspace_bytes=n - 1)[0] == WORKSPACE
    assert _block(workspace=FAKE + 16, workspace_bytes=n)[0] == WORKSPACE
    assert ops.lib().hspec_mamba_block(None, None, None) == INVALID


def _inject(ws=None, nbytes=0, **kw):
    a = dict(dtype=1, C=128, n=16, d=4096, Hkv=8, D=128, ps=16 * 8 * 128, ts=8 * 128, hs=128,
             num_pages=1000, max_pages=600, hidden=FAKE, w=FAKE, page=16)
    a.update(kw)
    n = ctypes.c_size_t(nbytes)
    code = ops.lib().hspec_kv_inject(None, a["dtype"], a["C"], a["n"], a["d"], a["Hkv"], a["D"], a["hidden"],
                                     a["w"], FAKE, FAKE, a["ps"], a["ts"], a["hs"], a["num_pages"], a["page"], FAKE,
                                     a["max_pages"], FAKE, ws, ctypes.byref(n))
    return code, n.value


def test_kv_inject_validation_and_workspace():
    code, n = _inject()
    assert code == OK and n == 256                         # 2048 x 2048 x 4096: no K slices
    code, n1 = _inject(C=1)                                 # 16 rows: K sliced, partials needed
    assert code == OK and n1 > 256 and n1 % 256 == 0
    assert _inject(n=0)[0] == INVALID
    assert _inject(hidden=FAKE + 8)[0] == INVALID
    assert _inject(ts=100)[0] == INVALID
    assert _inject(num_pages=0)[0] == INVALID
    assert _inject(d=4100)[0] == UNSUPPORTED
    assert _inject(page=24)[0] == UNSUPPORTED
    assert _inject(C=1 << 26, n=16)[0] == UNSUPPORTED      # 2^30 rows x 2048 columns > 2^40
    assert _inject(C=1 << 25, n=16)[0] == OK               # 2^29 x 2048 = 2^40 (size query only)
    assert _inject(ws=FAKE, nbytes=n1 - 1, C=1)[0] == WORKSPACE


def test_attention_workspace_with_bigger_pages():
    """Ranges are counted in granules of max(2, page / 16) slabs, so they
    start on page boundaries."""
    code, n16 = _attn(split=0, page=16, max_pages=64)
    assert code == OK
    for P in (32, 64, 128, 256):
        code, n = _attn(split=0, page=P, max_pages=-(-1000 // P))
        assert code == OK and n > 0
    # 64-token pages: granules of 4 slabs, a request at most 16 of them (63 + 1
    # slabs); a range of 4 pages is 16 slabs = 4 granules: 64 / 4 = 16 ranges
    code, n = _attn(split=4, page=64, max_pages=16)
    assert code == OK and n == _ws_expect(4, 16, 64)


def _stack(kinds=("MA", "MA"), mutate=None, **kw):
    """hspec_draft_stack size query for a bf16 stack of the C=128 shapes."""
    layers = (ops.StackLayer * len(kinds))()
    for l, kind in enumerate(kinds):
        layers[l].pre_norm_w = FAKE
        if "M" in kind:
            for k in ops._MAMBA_KEYS:
                setattr(layers[l], k, FAKE)
        if "A" in kind:
            for k in ops._ATTN_KEYS:
                setattr(layers[l], k, FAKE)
    a = ops.StackArgs()
    a.dtype, a.C, a.K, a.d_model, a.n_layers = 1, 128, 16, 4096, len(kinds)
    a.H, a.P, a.ng, a.N, a.chunk, a.eps = 16, 64, 1, 32, 16, 1e-5
    a.Hq, a.Hkv, a.D = 32, 8, 128
    a.page_stride, a.token_stride, a.head_stride = 16 * 8 * 128, 8 * 128, 128
    a.num_pages, a.page_size, a.page_table, a.max_pages = 70000, 16, FAKE, 512
    a.ctx_lens, a.max_ctx = FAKE, 8192
    a.hidden_in = a.u = a.hidden_out = FAKE
    a.layers = layers
    if mutate:
        mutate(layers)
    for k, v in kw.items():
        setattr(a, k, v)
    n = ctypes.c_size_t(0)
    return ops.lib().hspec_draft_stack(None, ctypes.byref(a), ctypes.byref(n)), n.value, layers


def test_stack_validation_and_workspace():
    code, n, _ = _stack()
    assert code == OK and n > 0
    assert _stack(("M", "A", "M", "A"))[:2] == (OK, n)      # same buffers whatever the layer mix
    assert _stack(n_layers=0)[0] == INVALID
    assert _stack(hidden_out=None)[0] == INVALID
    assert _stack(eps=-1.0)[0] == INVALID
    assert _stack(d_model=4100)[0] == UNSUPPORTED
    assert _stack(C=1 << 25)[0] == UNSUPPORTED              # 2^29 rows x 4096 columns > 2^40
    assert _stack(mutate=lambda L: setattr(L[1], "wk", None))[0] == INVALID   # half without a weight
    assert _stack(mutate=lambda L: setattr(L[0], "pre_norm_w", FAKE + 4))[0] == INVALID
    assert _stack(mutate=lambda L: setattr(L[0], "w_init", None))[0] == INVALID
    assert ops.lib().hspec_draft_stack(None, None, None) == INVALID
    g = ctypes.c_void_p()
    assert ops.lib().hspec_draft_stack_graph(None, ctypes.byref(g)) == INVALID
    assert ops.lib().hspec_graph_launch(None, None) == INVALID
    assert ops.lib().hspec_graph_destroy(None) == INVALID
