"""Thin ctypes binding over libhspec.so (include/hspec.h).

Argument marshalling only: tensors are passed by data pointer together with
torch's current HIP stream; every step of the layer runs in the library's
kernels.  There is no fallback of any kind -- if the library is missing or
refuses the arguments, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhspec.so")

F32, BF16 = 0, 1
_STATUS = {0: "HSPEC_OK", -1: "HSPEC_ERR_INVALID_ARG", -2: "HSPEC_ERR_UNSUPPORTED",
           -3: "HSPEC_ERR_WORKSPACE", -4: "HSPEC_ERR_HIP", -5: "HSPEC_ERR_SCRATCH"}
ABI_VERSION = 8

_vp, _i, _i64, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class LayerArgs(ctypes.Structure):
    """Mirror of hspec_layer_args (field order and types as in include/hspec.h)."""
    _fields_ = [
        ("dtype", _i), ("C", _i), ("K", _i),
        ("d_model", _i), ("H", _i), ("P", _i), ("ng", _i), ("N", _i), ("chunk", _i),
        ("u", _vp), ("w_init", _vp), ("h0", _vp),
        ("x", _vp), ("delta", _vp), ("A", _vp), ("B", _vp), ("Cm", _vp),
        ("Dskip", _vp), ("y", _vp), ("h_final", _vp),
        ("Hq", _i), ("Hkv", _i), ("D", _i),
        ("q", _vp), ("k_blk", _vp), ("v_blk", _vp),
        ("k_cache", _vp), ("v_cache", _vp),
        ("page_stride", _i64), ("token_stride", _i64), ("head_stride", _i64),
        ("num_pages", _i), ("page_size", _i), ("page_table", _vp), ("max_pages", _i),
        ("ctx_lens", _vp), ("max_ctx", _i),
        ("kv_split_pages", _i), ("scale", _f), ("block_causal", _i), ("out", _vp),
        ("workspace", _vp), ("workspace_bytes", _sz),
    ]


class MambaArgs(ctypes.Structure):
    """Mirror of hspec_mamba_args (field order and types as in include/hspec.h)."""
    _fields_ = [
        ("dtype", _i), ("C", _i), ("K", _i), ("d_model", _i), ("H", _i), ("P", _i), ("ng", _i),
        ("N", _i), ("chunk", _i),
        ("hidden", _vp), ("w_in", _vp),
        ("conv_w", _vp), ("conv_b", _vp), ("dt_bias", _vp),
        ("A", _vp), ("Dskip", _vp), ("h0", _vp),
        ("norm_w", _vp), ("norm_eps", _f),
        ("w_out", _vp),
        ("out", _vp), ("h_final", _vp),
        ("workspace", _vp), ("workspace_bytes", _sz),
    ]


class StackLayer(ctypes.Structure):
    """Mirror of hspec_stack_layer."""
    _fields_ = [
        ("pre_norm_w", _vp),
        ("w_init", _vp), ("w_in", _vp), ("conv_w", _vp), ("conv_b", _vp), ("dt_bias", _vp),
        ("A", _vp), ("Dskip", _vp), ("norm_w", _vp), ("w_out", _vp),
        ("wq", _vp), ("wk", _vp), ("wv", _vp), ("wo", _vp), ("k_cache", _vp), ("v_cache", _vp),
    ]


class StackArgs(ctypes.Structure):
    """Mirror of hspec_stack_args."""
    _fields_ = [
        ("dtype", _i), ("C", _i), ("K", _i), ("d_model", _i), ("n_layers", _i),
        ("H", _i), ("P", _i), ("ng", _i), ("N", _i), ("chunk", _i), ("eps", _f),
        ("Hq", _i), ("Hkv", _i), ("D", _i),
        ("page_stride", _i64), ("token_stride", _i64), ("head_stride", _i64),
        ("num_pages", _i), ("page_size", _i), ("page_table", _vp), ("max_pages", _i),
        ("ctx_lens", _vp), ("max_ctx", _i), ("kv_split_pages", _i), ("scale", _f),
        ("hidden_in", _vp), ("u", _vp), ("hidden_out", _vp),
        ("layers", ctypes.POINTER(StackLayer)),
        ("workspace", _vp), ("workspace_bytes", _sz),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libhspec.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                           "`python -m hybrid_mamba_attention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.hspec_status_string.restype = ctypes.c_char_p
    L.hspec_status_string.argtypes = [_i]
    L.hspec_abi_version.restype = _i
    L.hspec_layer_args_size.restype = _sz
    L.hspec_init_state.restype = _i
    L.hspec_init_state.argtypes = [_vp, _i, _i, _i, _i, _vp, _vp, _vp]
    L.hspec_ssd_scan.restype = _i
    L.hspec_ssd_scan.argtypes = [_vp, _i] + [_i] * 7 + [_vp] * 9
    L.hspec_block_attn_inplace.restype = _i
    L.hspec_block_attn_inplace.argtypes = ([_vp, _i, _i, _i, _i, _i, _i] + [_vp] * 5 +
                                           [_i64, _i64, _i64, _i, _i, _vp, _i, _vp, _i, _i, _f, _i,
                                            _vp, _vp, ctypes.POINTER(_sz)])
    L.hspec_draft_layer.restype = _i
    L.hspec_draft_layer.argtypes = [_vp, ctypes.POINTER(LayerArgs), ctypes.POINTER(_sz)]
    L.hspec_draft_layer_noalloc.restype = _i
    L.hspec_draft_layer_noalloc.argtypes = [_vp, ctypes.POINTER(LayerArgs)]
    L.hspec_mamba_args_size.restype = _sz
    L.hspec_mamba_block.restype = _i
    L.hspec_mamba_block.argtypes = [_vp, ctypes.POINTER(MambaArgs), ctypes.POINTER(_sz)]
    L.hspec_kv_inject.restype = _i
    L.hspec_kv_inject.argtypes = ([_vp, _i, _i, _i, _i, _i, _i] + [_vp] * 4 +
                                  [_i64, _i64, _i64, _i, _i, _vp, _i, _vp, _vp, ctypes.POINTER(_sz)])
    L.hspec_stack_args_size.restype = _sz
    L.hspec_draft_stack.restype = _i
    L.hspec_draft_stack.argtypes = [_vp, ctypes.POINTER(StackArgs), ctypes.POINTER(_sz)]
    L.hspec_draft_layer_graph.restype = _i
    L.hspec_draft_layer_graph.argtypes = [ctypes.POINTER(LayerArgs), ctypes.POINTER(_vp)]
    L.hspec_draft_stack_graph.restype = _i
    L.hspec_draft_stack_graph.argtypes = [ctypes.POINTER(StackArgs), ctypes.POINTER(_vp)]
    L.hspec_graph_launch.restype = _i
    L.hspec_graph_launch.argtypes = [_vp, _vp]
    L.hspec_graph_destroy.restype = _i
    L.hspec_graph_destroy.argtypes = [_vp]
    if L.hspec_abi_version() != ABI_VERSION:
        raise RuntimeError("libhspec.so ABI version mismatch")
    if L.hspec_layer_args_size() != ctypes.sizeof(LayerArgs):
        raise RuntimeError("hspec_layer_args layout mismatch between library and binding")
    if L.hspec_mamba_args_size() != ctypes.sizeof(MambaArgs):
        raise RuntimeError("hspec_mamba_args layout mismatch between library and binding")
    if L.hspec_stack_args_size() != ctypes.sizeof(StackArgs):
        raise RuntimeError("hspec_stack_args layout mismatch between library and binding")
    _lib = L
    return L


def status_string(code: int) -> str:
    return _STATUS.get(code, f"status {code}")


class HspecError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {status_string(code)}")
        self.code = code


def _check(fn: str, code: int):
    if code != 0:
        raise HspecError(fn, code)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"activation tensors must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _addr(t):
    """Device address of a tensor already checked by _checked (None stays None)."""
    return None if t is None else t.data_ptr()


def _checked(specs, act=None):
    """Check tensors before any of their addresses reaches the library.

    specs: (name, tensor, kind, shape, optional) with kind "act" (the
    activation type `act`), "f32", "i32" or "pool" (activation type, strides
    allowed); shape None skips the shape check.  Type, shape and layout are
    checked first, then that every tensor lives on the GPU -- all on one
    device -- so a host tensor or a wrong element type raises here instead of
    handing the kernels a pointer they would misread.  Returns the device."""
    want = {"f32": torch.float32, "i32": torch.int32}
    if act is not None and act not in (torch.float32, torch.bfloat16):
        raise TypeError(f"activation tensors must be float32 or bfloat16, got {act}")
    for name, t, kind, shape, optional in specs:
        if t is None:
            if optional:
                continue
            raise ValueError(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        dt = act if kind in ("act", "pool") else want[kind]
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if kind != "pool" and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    dev = None
    for name, t, *_ in specs:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must live on the GPU, not {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} lives on {t.device}, the other tensors on {dev}")
    return dev


def _pool_geometry(k_cache, v_cache, layout):
    """(Hkv, D, (page, token, head) strides) of a K/V pool pair, which must
    agree in shape and strides."""
    if k_cache.dim() != 4:
        raise ValueError("KV pools are 4-D: [pages, P, Hkv, D] (NHD) or [pages, Hkv, P, D] (HND)")
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("K and V pools must have the same shape")
    ps = kv_strides(k_cache, layout)
    if kv_strides(v_cache, layout) != ps:
        raise ValueError("K and V pools must share strides")
    Hkv = k_cache.shape[2] if layout == "NHD" else k_cache.shape[1]
    return int(Hkv), int(k_cache.shape[3]), ps


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------------------
# a1
# ---------------------------------------------------------------------------

def init_state(u: torch.Tensor, w_init: torch.Tensor, h0: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """h0[C, S] (fp32) = u[C, d] . w_init[d, S]."""
    if u.dim() != 2 or w_init.dim() != 2:
        raise ValueError("u is [C, d_model], w_init [d_model, S]")
    C, d = u.shape
    S = w_init.shape[1]
    dev = _checked([("u", u, "act", None, False), ("w_init", w_init, "act", (d, S), False),
                    ("h0", h0, "f32", (C, S), True)], u.dtype)
    if h0 is None:
        h0 = torch.empty((C, S), dtype=torch.float32, device=dev)
    _check("hspec_init_state", lib().hspec_init_state(
        _stream(stream), _dtype_code(u), C, d, S, _addr(u), _addr(w_init), _addr(h0)))
    return h0


# ---------------------------------------------------------------------------
# a2
# ---------------------------------------------------------------------------

def ssd_scan(x, delta, A, B, Cm, *, chunk: int, h0=None, Dskip=None, y=None, h_final=None,
             want_final: bool = False, stream=None):
    """y[C,K,H,P] (fp32) and optionally h_final[C,H,P,N] of the chunked SSD scan."""
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x is [C, K, H, P], B [C, K, ng, N]")
    C, K, H, P = x.shape
    ng, N = B.shape[2], B.shape[3]
    # the state may also come flat, as the projection writes it: [C, H*P*N]
    if h0 is not None and tuple(h0.shape) == (C, H * P * N):
        h0 = h0.view(C, H, P, N)
    dev = _checked([("x", x, "act", None, False), ("delta", delta, "f32", (C, K, H), False),
                    ("A", A, "f32", (H,), False), ("B", B, "act", None, False),
                    ("Cm", Cm, "act", (C, K, ng, N), False), ("h0", h0, "f32", (C, H, P, N), True),
                    ("Dskip", Dskip, "f32", (H,), True), ("y", y, "f32", (C, K, H, P), True),
                    ("h_final", h_final, "f32", (C, H, P, N), True)], x.dtype)
    if y is None:
        y = torch.empty((C, K, H, P), dtype=torch.float32, device=dev)
    if h_final is None and want_final:
        h_final = torch.empty((C, H, P, N), dtype=torch.float32, device=dev)
    _check("hspec_ssd_scan", lib().hspec_ssd_scan(
        _stream(stream), _dtype_code(x), C, K, H, P, ng, N, chunk,
        _addr(x), _addr(delta), _addr(A), _addr(B), _addr(Cm), _addr(Dskip), _addr(h0), _addr(y),
        _addr(h_final)))
    return y, h_final


# ---------------------------------------------------------------------------
# a0 + a3 + a4
# ---------------------------------------------------------------------------

def page_size_of(k_cache: torch.Tensor, layout: str = "NHD") -> int:
    """Tokens per page of a pool tensor: [pages, P, Hkv, D] (NHD) or [pages, Hkv, P, D] (HND)."""
    return int(k_cache.shape[1] if layout == "NHD" else k_cache.shape[2])


def kv_strides(k_cache: torch.Tensor, layout: str = "NHD"):
    """(page, token, head) strides in elements of a pool tensor.

    NHD pools are [pages, P, Hkv, D]; HND pools are [pages, Hkv, P, D]."""
    s = k_cache.stride()
    if k_cache.stride(-1) != 1:
        raise ValueError("the head dimension of the KV pool must be contiguous")
    if layout == "NHD":
        return s[0], s[1], s[2]
    if layout == "HND":
        return s[0], s[2], s[1]
    raise ValueError(layout)


def _attn_call(L, stream, q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_lens, max_ctx,
               kv_split_pages, scale, block_causal, out, ws, ws_bytes, layout):
    """out None: a size query (the library then only reads the sizes)."""
    if q.dim() != 4 or k_blk.dim() != 4 or page_table.dim() != 2:
        raise ValueError("q and k_blk are 4-D, page_table [C, max_pages]")
    C, K, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    pool_hkv, pool_d, (ps, ts, hs) = _pool_geometry(k_cache, v_cache, layout)
    if (pool_hkv, pool_d) != (Hkv, D):
        raise ValueError(f"KV pools hold {pool_hkv} heads of {pool_d}, the block {Hkv} of {D}")
    _checked([("q", q, "act", None, False), ("k_blk", k_blk, "act", (C, K, Hkv, D), False),
              ("v_blk", v_blk, "act", (C, K, Hkv, D), False), ("k_cache", k_cache, "pool", None, False),
              ("v_cache", v_cache, "pool", None, False),
              ("page_table", page_table, "i32", (C, page_table.shape[1]), False),
              ("ctx_lens", ctx_lens, "i32", (C,), False), ("out", out, "act", (C, K, Hq, D), True)], q.dtype)
    return L.hspec_block_attn_inplace(
        _stream(stream), _dtype_code(q), C, K, Hq, Hkv, D, _addr(q), _addr(k_blk), _addr(v_blk),
        _addr(k_cache), _addr(v_cache), ps, ts, hs, k_cache.shape[0], page_size_of(k_cache, layout),
        _addr(page_table), page_table.shape[1], _addr(ctx_lens), int(max_ctx), int(kv_split_pages), float(scale),
        int(bool(block_causal)), _addr(out if out is not None else q), ws, ctypes.byref(ws_bytes))


def plan_of(workspace: torch.Tensor, C: int) -> torch.Tensor:
    """The int32 work plan at the head of an attention workspace:
    [W, granule slabs, C, w_max], S_b, first range, pieces (C each), B_0..B_w_max."""
    w_max = int(workspace[12:16].view(torch.int32).item())
    return workspace[:4 * (4 + 3 * C + w_max + 1)].view(torch.int32)


def attn_workspace_bytes(q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_lens, *, max_ctx,
                         kv_split_pages=0, scale=0.0, block_causal=False, layout="NHD") -> int:
    n = _sz(0)
    _check("hspec_block_attn_inplace", _attn_call(
        lib(), None, q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_lens, max_ctx,
        kv_split_pages, scale, block_causal, None, None, n, layout))
    return n.value


def block_attn_inplace(q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_lens, *, max_ctx,
                       kv_split_pages=0, scale=0.0, block_causal=False, out=None, workspace=None,
                       layout="NHD", stream=None):
    """out[C,K,Hq,D] = attention of the block queries over paged target KV + block KV.

    block_causal: block query t sees block keys s <= t only (context keys all).
    workspace: a uint8 CUDA tensor of at least attn_workspace_bytes(...) bytes
    (allocated here if None).  Returns (out, workspace)."""
    L = lib()
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = attn_workspace_bytes(q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_lens,
                                      max_ctx=max_ctx, kv_split_pages=kv_split_pages, scale=scale,
                                      block_causal=block_causal, layout=layout)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    n = _sz(workspace.numel())
    _check("hspec_block_attn_inplace", _attn_call(
        L, stream, q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_lens, max_ctx,
        kv_split_pages, scale, block_causal, out, _ptr(workspace), n, layout))
    return out, workspace


# ---------------------------------------------------------------------------
# a5
# ---------------------------------------------------------------------------

class DraftLayer:
    """Holds the marshalled argument block of one drafter-layer configuration so
    that repeated calls (benchmarks, serving loops) only re-issue the C call.

    u = w_init = None is the direct-reuse-only ablation: no state projection,
    the scan starts from the zero state and h0 stays None."""

    def __init__(self, *, u, w_init, x, delta, A, B, Cm, chunk, q, k_blk, v_blk, k_cache, v_cache,
                 page_table, ctx_lens, max_ctx, kv_split_pages=0, scale=0.0, block_causal=False,
                 Dskip=None, want_final=False, layout="NHD"):
        if (u is None) != (w_init is None):
            raise ValueError("u and w_init are given together (or both None for the ablation)")
        if x.dim() != 4 or B.dim() != 4 or q.dim() != 4 or k_blk.dim() != 4:
            raise ValueError("x, B, q and k_blk are 4-D")
        C, K, H, P = x.shape
        ng, N = B.shape[2], B.shape[3]
        Hq, D = q.shape[2], q.shape[3]
        Hkv = k_blk.shape[2]
        d = u.shape[-1] if u is not None else 0
        act = x.dtype
        pool_hkv, pool_d, (ps, ts, hs) = _pool_geometry(k_cache, v_cache, layout)
        if (pool_hkv, pool_d) != (Hkv, D):
            raise ValueError(f"KV pools hold {pool_hkv} heads of {pool_d}, the block {Hkv} of {D}")
        if page_table.dim() != 2:
            raise ValueError("page_table is [C, max_pages]")
        dev = _checked([
            ("u", u, "act", (C, d), True), ("w_init", w_init, "act", (d, H * P * N), True),
            ("x", x, "act", None, False), ("delta", delta, "f32", (C, K, H), False),
            ("A", A, "f32", (H,), False), ("B", B, "act", (C, K, ng, N), False),
            ("Cm", Cm, "act", (C, K, ng, N), False), ("Dskip", Dskip, "f32", (H,), True),
            ("q", q, "act", (C, K, Hq, D), False), ("k_blk", k_blk, "act", (C, K, Hkv, D), False),
            ("v_blk", v_blk, "act", (C, K, Hkv, D), False),
            ("k_cache", k_cache, "pool", None, False), ("v_cache", v_cache, "pool", None, False),
            ("page_table", page_table, "i32", (C, page_table.shape[1]), False),
            ("ctx_lens", ctx_lens, "i32", (C,), False),
        ], act)
        self.h0 = (torch.empty((C, H * P * N), dtype=torch.float32, device=dev)
                   if u is not None else None)
        self.y = torch.empty((C, K, H, P), dtype=torch.float32, device=dev)
        self.h_final = (torch.empty((C, H, P, N), dtype=torch.float32, device=dev)
                        if want_final else None)
        self.out = torch.empty_like(q)
        a = LayerArgs()
        a.dtype = _dtype_code(x)
        a.C, a.K = C, K
        a.d_model, a.H, a.P, a.ng, a.N, a.chunk = d, H, P, ng, N, chunk
        a.u, a.w_init, a.h0 = _addr(u), _addr(w_init), _addr(self.h0)
        a.x, a.delta, a.A = _addr(x), _addr(delta), _addr(A)
        a.B, a.Cm = _addr(B), _addr(Cm)
        a.Dskip = _addr(Dskip)
        a.y = _addr(self.y)
        a.h_final = _addr(self.h_final)
        a.Hq, a.Hkv, a.D = Hq, Hkv, D
        a.q, a.k_blk, a.v_blk = _addr(q), _addr(k_blk), _addr(v_blk)
        a.k_cache, a.v_cache = _addr(k_cache), _addr(v_cache)
        a.page_stride, a.token_stride, a.head_stride = ps, ts, hs
        a.num_pages = k_cache.shape[0]
        a.page_size = page_size_of(k_cache, layout)
        a.page_table, a.max_pages = _addr(page_table), page_table.shape[1]
        a.ctx_lens, a.max_ctx = _addr(ctx_lens), int(max_ctx)
        a.kv_split_pages, a.scale = int(kv_split_pages), float(scale)
        a.block_causal = int(bool(block_causal))
        a.out = _addr(self.out)
        a.workspace, a.workspace_bytes = None, 0
        need = _sz(0)
        _check("hspec_draft_layer", lib().hspec_draft_layer(None, ctypes.byref(a), ctypes.byref(need)))
        self.workspace = torch.empty(max(need.value, 256), dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = self.workspace.data_ptr(), self.workspace.numel()
        self._args = a
        self._keep = (u, w_init, x, delta, A, B, Cm, Dskip, q, k_blk, v_blk, k_cache, v_cache,
                      page_table, ctx_lens)

    def __call__(self, stream=None):
        _check("hspec_draft_layer", lib().hspec_draft_layer(_stream(stream), ctypes.byref(self._args), None))
        return self

    def noalloc(self, stream=None):
        """The same layer through hspec_draft_layer_noalloc: the library's static
        scratch instead of this object's workspace (nothing is allocated)."""
        a = LayerArgs.from_buffer_copy(self._args)
        a.workspace, a.workspace_bytes = None, 0
        _check("hspec_draft_layer_noalloc", lib().hspec_draft_layer_noalloc(_stream(stream), ctypes.byref(a)))
        return self

    def graph(self):
        """Capture the layer into a HIP graph (once; the Mamba half on its own branch)."""
        if getattr(self, "_graph", None) is None:
            g = _vp()
            _check("hspec_draft_layer_graph", lib().hspec_draft_layer_graph(ctypes.byref(self._args), ctypes.byref(g)))
            self._graph = g
        return self

    def launch_graph(self, stream=None):
        self.graph()
        _check("hspec_graph_launch", lib().hspec_graph_launch(self._graph, _stream(stream)))
        return self

    def __del__(self):
        g = getattr(self, "_graph", None)
        if g is not None and _lib is not None:
            _lib.hspec_graph_destroy(g)
            self._graph = None

    def plan(self) -> torch.Tensor:
        """The int32 work plan at the head of the workspace (see include/hspec.h)."""
        return plan_of(self.workspace, self._args.C)


def draft_layer(**kw):
    """One drafter-layer call; returns the DraftLayer holding h0, y, h_final, out."""
    return DraftLayer(**kw)()


# ---------------------------------------------------------------------------
# the Mamba-2 block around the scan
# ---------------------------------------------------------------------------

class MambaBlock:
    """Marshalled arguments of one Mamba-2 block configuration (hspec_mamba_block).

    hidden [C,K,d_model] and w_in [d_proj,d_model], w_out [d_model,H*P] in the
    activation type; conv_w [conv_dim,4], conv_b, dt_bias, A, Dskip, norm_w and
    h0 [C,H,P,N] fp32 (conv_b, Dskip and h0 may be None)."""

    def __init__(self, *, hidden, w_in, conv_w, dt_bias, A, norm_w, w_out, H, P, N, chunk, ng=1,
                 conv_b=None, Dskip=None, h0=None, eps=1e-5, want_final=False):
        if hidden.dim() != 3:
            raise ValueError("hidden is [C, K, d_model]")
        C, K, d = hidden.shape
        d_inner = H * P
        conv_dim = d_inner + 2 * ng * N
        d_proj = 2 * d_inner + 2 * ng * N + H
        dev = _checked([
            ("hidden", hidden, "act", None, False), ("w_in", w_in, "act", (d_proj, d), False),
            ("conv_w", conv_w, "f32", (conv_dim, 4), False), ("conv_b", conv_b, "f32", (conv_dim,), True),
            ("dt_bias", dt_bias, "f32", (H,), False), ("A", A, "f32", (H,), False),
            ("Dskip", Dskip, "f32", (H,), True), ("h0", h0, "f32", (C, H, P, N), True),
            ("norm_w", norm_w, "f32", (d_inner,), False), ("w_out", w_out, "act", (d, d_inner), False),
        ], hidden.dtype)
        self.out = torch.empty_like(hidden)
        self.h_final = (torch.empty((C, H, P, N), dtype=torch.float32, device=dev)
                        if want_final else None)
        a = MambaArgs()
        a.dtype = _dtype_code(hidden)
        a.C, a.K, a.d_model, a.H, a.P, a.ng, a.N, a.chunk = C, K, d, H, P, ng, N, chunk
        a.hidden, a.w_in = _addr(hidden), _addr(w_in)
        a.conv_w, a.conv_b, a.dt_bias = _addr(conv_w), _addr(conv_b), _addr(dt_bias)
        a.A, a.Dskip, a.h0 = _addr(A), _addr(Dskip), _addr(h0)
        a.norm_w, a.norm_eps = _addr(norm_w), float(eps)
        a.w_out = _addr(w_out)
        a.out, a.h_final = _addr(self.out), _addr(self.h_final)
        a.workspace, a.workspace_bytes = None, 0
        need = _sz(0)
        _check("hspec_mamba_block", lib().hspec_mamba_block(None, ctypes.byref(a), ctypes.byref(need)))
        self.workspace = torch.empty(max(need.value, 256), dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = self.workspace.data_ptr(), self.workspace.numel()
        self._args = a
        self._keep = (hidden, w_in, conv_w, conv_b, dt_bias, A, Dskip, h0, norm_w, w_out)

    def __call__(self, stream=None):
        _check("hspec_mamba_block", lib().hspec_mamba_block(_stream(stream), ctypes.byref(self._args), None))
        return self


def mamba_block(**kw):
    """One Mamba-2 block call; returns the MambaBlock holding out and h_final."""
    return MambaBlock(**kw)()


# ---------------------------------------------------------------------------
# the drafter stack
# ---------------------------------------------------------------------------

_MAMBA_KEYS = ("w_init", "w_in", "conv_w", "conv_b", "dt_bias", "A", "Dskip", "norm_w", "w_out")
_ATTN_KEYS = ("wq", "wk", "wv", "wo", "k_cache", "v_cache")


class DraftStack:
    """Marshalled arguments of one drafter-stack configuration.

    layers: list of dicts of device tensors: 'pre_norm_w', and the Mamba half
    (_MAMBA_KEYS, w_in present) and/or the attention half (_ATTN_KEYS, wq
    present).  Calling the object runs the stack eagerly; graph() captures it
    once into a HIP graph (hspec_draft_stack_graph) and launch_graph() replays
    it.  hidden_out (fp32 [C, K, d_model]) holds the result either way."""

    def __init__(self, *, hidden_in, u, layers, page_table, ctx_lens, max_ctx, H, P, N, chunk, Hq, Hkv, D,
                 ng=1, eps=1e-5, kv_split_pages=0, scale=0.0, layout="NHD"):
        if hidden_in.dim() != 3 or page_table.dim() != 2 or not layers:
            raise ValueError("hidden_in is [C, K, d_model], page_table [C, max_pages], layers non-empty")
        C, K, d = hidden_in.shape
        act = hidden_in.dtype
        d_inner = H * P
        conv_dim = d_inner + 2 * ng * N
        d_proj = 2 * d_inner + 2 * ng * N + H
        specs = [("hidden_in", hidden_in, "act", None, False), ("u", u, "act", (C, d), False),
                 ("page_table", page_table, "i32", (C, page_table.shape[1]), False),
                 ("ctx_lens", ctx_lens, "i32", (C,), False)]
        # every attention half shares the one set of pool strides and the
        # page table, so all layers' pools must agree in shape and strides
        pools = None
        for l, Ld in enumerate(layers):
            unknown = set(Ld) - {"pre_norm_w", *_MAMBA_KEYS, *_ATTN_KEYS}
            if unknown:
                raise ValueError(f"layer {l}: unknown keys {sorted(unknown)}")
            specs.append((f"layers[{l}].pre_norm_w", Ld.get("pre_norm_w"), "f32", (d,), False))
            if Ld.get("w_in") is not None:
                mshape = dict(w_init=("act", (d, H * P * N), False), w_in=("act", (d_proj, d), False),
                              conv_w=("f32", (conv_dim, 4), False), conv_b=("f32", (conv_dim,), True),
                              dt_bias=("f32", (H,), False), A=("f32", (H,), False),
                              Dskip=("f32", (H,), True), norm_w=("f32", (d_inner,), False),
                              w_out=("act", (d, d_inner), False))
                specs += [(f"layers[{l}].{k}", Ld.get(k), kind, shp, opt) for k, (kind, shp, opt) in mshape.items()]
            if Ld.get("wq") is not None:
                ashape = dict(wq=(Hq * D, d), wk=(Hkv * D, d), wv=(Hkv * D, d), wo=(d, Hq * D))
                specs += [(f"layers[{l}].{k}", Ld.get(k), "act", shp, False) for k, shp in ashape.items()]
                kc, vc = Ld.get("k_cache"), Ld.get("v_cache")
                if kc is None or vc is None:
                    raise ValueError(f"layer {l}: an attention half needs k_cache and v_cache")
                geo = _pool_geometry(kc, vc, layout)
                if geo[:2] != (Hkv, D):
                    raise ValueError(f"layer {l}: KV pools hold {geo[0]} heads of {geo[1]}, not {Hkv} of {D}")
                if pools is not None and (geo[2] != pools[0] or kc.shape != pools[1]):
                    raise ValueError(f"layer {l}: KV pools differ in shape or strides from an earlier layer's")
                pools = (geo[2], kc.shape, kc)
                specs += [(f"layers[{l}].k_cache", kc, "pool", None, False),
                          (f"layers[{l}].v_cache", vc, "pool", None, False)]
        dev = _checked(specs, act)
        self.hidden_out = torch.empty((C, K, d), dtype=torch.float32, device=dev)
        arr = (StackLayer * len(layers))()
        for l, Ld in enumerate(layers):
            arr[l].pre_norm_w = _addr(Ld.get("pre_norm_w"))
            for k in _MAMBA_KEYS + _ATTN_KEYS:
                setattr(arr[l], k, _addr(Ld.get(k)))
        a = StackArgs()
        a.dtype = _dtype_code(hidden_in)
        a.C, a.K, a.d_model, a.n_layers = C, K, d, len(layers)
        a.H, a.P, a.ng, a.N, a.chunk, a.eps = H, P, ng, N, chunk, float(eps)
        a.Hq, a.Hkv, a.D = Hq, Hkv, D
        if pools is not None:
            a.page_stride, a.token_stride, a.head_stride = pools[0]
            a.num_pages, a.page_size = pools[2].shape[0], page_size_of(pools[2], layout)
        else:
            a.page_stride, a.token_stride, a.head_stride, a.num_pages, a.page_size = 8, 8, 8, 1, 16
        a.page_table, a.max_pages = _addr(page_table), page_table.shape[1]
        a.ctx_lens, a.max_ctx = _addr(ctx_lens), int(max_ctx)
        a.kv_split_pages, a.scale = int(kv_split_pages), float(scale)
        a.hidden_in, a.u, a.hidden_out = _addr(hidden_in), _addr(u), _addr(self.hidden_out)
        a.layers = arr
        need = _sz(0)
        _check("hspec_draft_stack", lib().hspec_draft_stack(None, ctypes.byref(a), ctypes.byref(need)))
        self.workspace = torch.empty(max(need.value, 256), dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = self.workspace.data_ptr(), self.workspace.numel()
        self._args, self._layers = a, arr
        self._keep = (hidden_in, u, layers, page_table, ctx_lens)
        self._graph = None

    def __call__(self, stream=None):
        _check("hspec_draft_stack", lib().hspec_draft_stack(_stream(stream), ctypes.byref(self._args), None))
        return self

    def graph(self):
        """Capture the stack into a HIP graph (once); returns self."""
        if self._graph is None:
            g = _vp()
            _check("hspec_draft_stack_graph", lib().hspec_draft_stack_graph(ctypes.byref(self._args), ctypes.byref(g)))
            self._graph = g
        return self

    def launch_graph(self, stream=None):
        self.graph()
        _check("hspec_graph_launch", lib().hspec_graph_launch(self._graph, _stream(stream)))
        return self

    def __del__(self):
        g = getattr(self, "_graph", None)
        if g is not None and _lib is not None:
            _lib.hspec_graph_destroy(g)
            self._graph = None


# ---------------------------------------------------------------------------
# contrast workload: drafter-side KV injection
# ---------------------------------------------------------------------------

def _inject_call(stream, hidden, w_kv, k_cache, v_cache, page_table, start_pos, ws, n, layout):
    if hidden.dim() != 3 or page_table.dim() != 2:
        raise ValueError("hidden is [C, n_new, d_model], page_table [C, max_pages]")
    C, n_new, d = hidden.shape
    Hkv, D, (ps, ts, hs) = _pool_geometry(k_cache, v_cache, layout)
    _checked([("hidden", hidden, "act", None, False), ("w_kv", w_kv, "act", (2 * Hkv * D, d), False),
              ("k_cache", k_cache, "pool", None, False), ("v_cache", v_cache, "pool", None, False),
              ("page_table", page_table, "i32", (C, page_table.shape[1]), False),
              ("start_pos", start_pos, "i32", (C,), False)], hidden.dtype)
    return lib().hspec_kv_inject(
        _stream(stream), _dtype_code(hidden), C, n_new, d, Hkv, D, _addr(hidden), _addr(w_kv), _addr(k_cache),
        _addr(v_cache), ps, ts, hs, k_cache.shape[0], page_size_of(k_cache, layout), _addr(page_table),
        page_table.shape[1], _addr(start_pos), ws, ctypes.byref(n))


def kv_inject(hidden, w_kv, k_cache, v_cache, page_table, start_pos, *, workspace=None, layout="NHD",
              stream=None):
    """Write w_kv . hidden[b, i] as K | V rows of positions start_pos[b] + i into
    the paged pools (in place).  Returns the workspace."""
    if workspace is None:
        n = _sz(0)
        _check("hspec_kv_inject", _inject_call(stream, hidden, w_kv, k_cache, v_cache, page_table,
                                               start_pos, None, n, layout))
        workspace = torch.empty(max(n.value, 256), dtype=torch.uint8, device=hidden.device)
    n = _sz(workspace.numel())
    _check("hspec_kv_inject", _inject_call(stream, hidden, w_kv, k_cache, v_cache, page_table,
                                           start_pos, _ptr(workspace), n, layout))
    return workspace


# ---------------------------------------------------------------------------
# measurement aid (include/hspec_probe.h)
# ---------------------------------------------------------------------------

def stream_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Enqueue one nontemporal streaming read of all of `buf` (see hspec_probe.h)."""
    L = lib()
    f = L.hspec_probe_stream_read
    f.restype = _i
    f.argtypes = [_vp, _vp, _sz, _vp]
    _check("hspec_probe_stream_read", f(_stream(stream), _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink)))
