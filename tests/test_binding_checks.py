"""The Python binding refuses misused tensors before any address reaches the
library: a host-resident tensor, a wrong element type (an int64 page table
would be read as int32 pairs), a wrong shape, activations of mixed types, or
K and V pools of different layouts.  Everything here runs on the CPU: the
checks raise before the first library or GPU call."""
import pytest
import torch

from hybrid_mamba_attention_amd import ops

C, K, H, P, N, d, Hq, Hkv, D, NP = 2, 4, 2, 8, 4, 32, 4, 2, 64, 6


def layer_kwargs(dt=torch.bfloat16):
    z = lambda *s: torch.zeros(s, dtype=dt)
    f = lambda *s: torch.zeros(s, dtype=torch.float32)
    return dict(u=z(C, d), w_init=z(d, H * P * N), x=z(C, K, H, P), delta=f(C, K, H), A=f(H),
                B=z(C, K, 1, N), Cm=z(C, K, 1, N), chunk=4, q=z(C, K, Hq, D), k_blk=z(C, K, Hkv, D),
                v_blk=z(C, K, Hkv, D), k_cache=z(NP, 16, Hkv, D), v_cache=z(NP, 16, Hkv, D),
                page_table=torch.zeros((C, 3), dtype=torch.int32),
                ctx_lens=torch.zeros(C, dtype=torch.int32), max_ctx=40)


MISUSE = [
    ("page_table", lambda t: t.long(), TypeError),
    ("ctx_lens", lambda t: t.long(), TypeError),
    ("delta", lambda t: t.bfloat16(), TypeError),
    ("A", lambda t: t.double(), TypeError),
    ("q", lambda t: t.float(), TypeError),              # activations of mixed types
    ("k_cache", lambda t: t.float(), TypeError),
    ("w_init", lambda t: t[:, :-8], ValueError),          # wrong state size
    ("k_blk", lambda t: t[:, :, :1], ValueError),         # wrong head count
    ("ctx_lens", lambda t: t[:1], ValueError),
    ("page_table", lambda t: t.t().contiguous().t(), ValueError),   # not contiguous
    ("v_cache", lambda t: t[:-1], ValueError),            # pools of different shapes
    ("Cm", lambda t: t[:, :, :, :2], ValueError),
]


@pytest.mark.parametrize("name,bad,exc", MISUSE, ids=[f"{m[0]}-{i}" for i, m in enumerate(MISUSE)])
def test_draft_layer_refuses_misuse(name, bad, exc):
    kw = layer_kwargs()
    kw[name] = bad(kw[name])
    with pytest.raises(exc):
        ops.DraftLayer(**kw)


def test_draft_layer_refuses_host_tensors():
    """Well-typed and well-shaped, but on the host: refused before any call."""
    with pytest.raises(ValueError, match="GPU"):
        ops.DraftLayer(**layer_kwargs())


def test_draft_layer_refuses_half_an_initialisation():
    kw = layer_kwargs()
    kw["w_init"] = None
    with pytest.raises(ValueError):
        ops.DraftLayer(**kw)


def test_attention_and_scan_wrappers_refuse_misuse():
    kw = layer_kwargs()
    args = [kw[k] for k in ("q", "k_blk", "v_blk", "k_cache", "v_cache", "page_table", "ctx_lens")]
    bad = list(args)
    bad[5] = bad[5].long()
    with pytest.raises(TypeError):
        ops.block_attn_inplace(*bad, max_ctx=40)
    with pytest.raises(ValueError, match="GPU"):
        ops.block_attn_inplace(*args, max_ctx=40)
    with pytest.raises(TypeError):
        ops.ssd_scan(kw["x"], kw["delta"].bfloat16(), kw["A"], kw["B"], kw["Cm"], chunk=4)
    with pytest.raises(ValueError):
        ops.init_state(kw["u"], kw["w_init"].t())


def block_kwargs():
    dt = torch.bfloat16
    d_inner, conv_dim, d_proj = H * P, H * P + 2 * N, 2 * H * P + 2 * N + H
    f = lambda *s: torch.zeros(s, dtype=torch.float32)
    return dict(hidden=torch.zeros((C, K, d), dtype=dt), w_in=torch.zeros((d_proj, d), dtype=dt),
                conv_w=f(conv_dim, 4), dt_bias=f(H), A=f(H), norm_w=f(d_inner),
                w_out=torch.zeros((d, d_inner), dtype=dt), H=H, P=P, N=N, chunk=4)


@pytest.mark.parametrize("name,bad,exc", [
    ("conv_w", lambda t: t.bfloat16(), TypeError), ("w_out", lambda t: t.t(), ValueError),
    ("norm_w", lambda t: t[:-1], ValueError), ("w_in", lambda t: t.float(), TypeError),
])
def test_mamba_block_refuses_misuse(name, bad, exc):
    kw = block_kwargs()
    kw[name] = bad(kw[name])
    with pytest.raises(exc):
        ops.MambaBlock(**kw)
    with pytest.raises(ValueError, match="GPU"):
        ops.MambaBlock(**block_kwargs())


def stack_kwargs(n_layers=2):
    dt = torch.bfloat16
    kw = layer_kwargs()
    blk = block_kwargs()
    layers = []
    for _ in range(n_layers):
        L = dict(pre_norm_w=torch.ones(d), w_init=kw["w_init"], w_in=blk["w_in"], conv_w=blk["conv_w"],
                 dt_bias=blk["dt_bias"], A=blk["A"], norm_w=blk["norm_w"], w_out=blk["w_out"],
                 wq=torch.zeros((Hq * D, d), dtype=dt), wk=torch.zeros((Hkv * D, d), dtype=dt),
                 wv=torch.zeros((Hkv * D, d), dtype=dt), wo=torch.zeros((d, Hq * D), dtype=dt),
                 k_cache=torch.zeros((NP, 16, Hkv, D), dtype=dt), v_cache=torch.zeros((NP, 16, Hkv, D), dtype=dt))
        layers.append(L)
    return dict(hidden_in=torch.zeros((C, K, d), dtype=dt), u=kw["u"], layers=layers,
                page_table=kw["page_table"], ctx_lens=kw["ctx_lens"], max_ctx=40, H=H, P=P, N=N, chunk=4,
                Hq=Hq, Hkv=Hkv, D=D)


def test_stack_refuses_pools_of_different_layouts():
    """All layers share one set of pool strides: a layer whose pools are laid
    out differently is refused."""
    kw = stack_kwargs()
    L = kw["layers"][1]
    L["k_cache"] = torch.zeros((NP + 1, 16, Hkv, D), dtype=torch.bfloat16)
    L["v_cache"] = torch.zeros((NP + 1, 16, Hkv, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="differ"):
        ops.DraftStack(**kw)


@pytest.mark.parametrize("key,bad,exc", [
    ("pre_norm_w", lambda t: t.bfloat16(), TypeError), ("wo", lambda t: t.t(), ValueError),
    ("k_cache", lambda t: t.float(), TypeError), ("dt_bias", lambda t: t[:1], ValueError),
])
def test_stack_refuses_misuse(key, bad, exc):
    kw = stack_kwargs()
    kw["layers"][0][key] = bad(kw["layers"][0][key])
    with pytest.raises(exc):
        ops.DraftStack(**kw)
    with pytest.raises(ValueError, match="GPU"):
        ops.DraftStack(**stack_kwargs())
