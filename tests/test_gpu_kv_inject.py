"""GPU parity of the drafter-side KV injection (hspec_kv_inject, the contrast
workload) against the oracle: written slots within the tolerance, every other
element of both pools bit-identical, positions crossing page boundaries,
ragged row / column / contraction tiles, split-K at small C, the HND layout,
and positions outside the page table skipped."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from hybrid_mamba_attention_amd import ops
from hybrid_mamba_attention_amd import workloads as wl

from helpers import assert_close, flush, to_dev, to_host64

pytestmark = pytest.mark.gpu


def written_mask(a, n_new):
    m = np.zeros(a["k_cache"].shape[:2], dtype=bool)
    P = a["k_cache"].shape[1]
    for b, s in enumerate(a["start"]):
        for i in range(n_new):
            p = int(s) + i
            m[a["page_table"][b, p // P], p % P] = True
    return m


def shifted(t, elems):
    """A contiguous copy of t whose data starts `elems` elements past an
    allocation's (aligned) start."""
    flat = torch.empty(t.numel() + elems, dtype=t.dtype, device=t.device)
    v = flat[elems:].view(t.shape)
    v.copy_(t)
    return v


def run_and_check(w, n_new, starts, layout="NHD", page_size=16, pool_offset=0):
    a = wl.make_inject_inputs(w, n_new, ctx_lens=starts, page_size=page_size)
    dt = w.dtype
    kc, vc = to_dev(a["k_cache"], dt), to_dev(a["v_cache"], dt)
    if pool_offset:
        kc, vc = shifted(kc, pool_offset), shifted(vc, pool_offset)
        assert kc.data_ptr() % 16 and vc.data_ptr() % 16
    if layout == "HND":
        kc, vc = kc.permute(0, 2, 1, 3).contiguous(), vc.permute(0, 2, 1, 3).contiguous()
    ops.kv_inject(to_dev(a["hidden"], dt), to_dev(a["w_kv"], dt), kc, vc, to_dev(a["page_table"], dt),
                  to_dev(a["start"], dt), layout=layout)
    torch.cuda.synchronize()
    if layout == "HND":
        kc, vc = kc.permute(0, 2, 1, 3).contiguous(), vc.permute(0, 2, 1, 3).contiguous()
    kp, vp, _ = oracle.kv_inject(a["hidden"], a["w_kv"], a["k_cache"], a["v_cache"], a["page_table"], a["start"],
                                 Hkv=w.Hkv, D=w.D, dtype=dt)
    wm = written_mask(a, n_new)
    for got, want, stored, name in ((kc, kp, a["k_cache"], "K"), (vc, vp, a["v_cache"], "V")):
        g = got.cpu()
        g_bits = g.view(torch.int16 if dt == "bf16" else torch.int32).numpy()
        s_bits = stored.view(np.int16 if dt == "bf16" else np.int32)
        assert np.array_equal(g_bits[~wm], s_bits[~wm]), f"{name}: an unwritten slot changed"
        assert_close(g.float().numpy().astype(np.float64)[wm], want[wm], dt, f"{w.name} {name} written")


CASES = [
    # (name, C, n_new, d_model, Hkv, D, dtype, starts)
    ("llama-c4-ragged-splitk", 4, 16, 4096, 8, 128, "bf16", [0, 13, 100, 2047]),
    ("llama-c128-2048rows", 128, 16, 4096, 8, 128, "bf16", None),
    ("n7-cross-page-d200", 3, 7, 200, 2, 128, "bf16", [14, 0, 31]),
    ("d64-hkv4-n21", 5, 21, 512, 4, 64, "bf16", [5, 16, 33, 0, 70]),
    ("f32-small", 2, 5, 64, 2, 64, "f32", [3, 15]),
    # 2*Hkv*D = 192 columns: 128-column tiles leave a 64-column tail, and at
    # 25600 rows (200 row tiles) that tail is launched on its own so the
    # whole tiles fill one round; its V columns must land in V, not in K
    ("tail-launch-hkv1-d96-25600rows", 100, 256, 64, 1, 96, "bf16", None),
]


@pytest.mark.parametrize("name,C,n,d,Hkv,D,dtype,starts", CASES, ids=[c[0] for c in CASES])
def test_kv_inject(name, C, n, d, Hkv, D, dtype, starts):
    flush(f"[inject] {name}")
    w = replace(wl.WORKLOADS[1], name=name, C=C, d_model=d, Hkv=Hkv, Hq=Hkv, D=D, dtype=dtype,
                ctx=("uniform", 0, 200), seed=700 + [c[0] for c in CASES].index(name))
    run_and_check(w, n, starts)


def test_kv_inject_bigger_pages():
    w = replace(wl.WORKLOADS[1], name="inject-p64", C=4, d_model=256, seed=779)
    run_and_check(w, 16, [0, 60, 100, 127], page_size=64)


def test_kv_inject_hnd_layout():
    w = replace(wl.WORKLOADS[1], name="inject-hnd", C=3, d_model=256, seed=777)
    run_and_check(w, 16, [0, 9, 40], layout="HND")


def test_kv_inject_skips_positions_outside_the_table():
    """Positions whose page-table slot lies past max_pages are not written."""
    w = replace(wl.WORKLOADS[1], name="inject-oob", C=2, d_model=256, seed=778)
    a = wl.make_inject_inputs(w, 16, ctx_lens=[0, 20])
    pt = a["page_table"][:, :2].copy()            # request 1 needs pages 0..2: page 2 is cut off
    dt = w.dtype
    kc, vc = to_dev(a["k_cache"], dt), to_dev(a["v_cache"], dt)
    before = kc.view(torch.int16).clone()
    ops.kv_inject(to_dev(a["hidden"], dt), to_dev(a["w_kv"], dt), kc, vc, to_dev(pt, dt), to_dev(a["start"], dt))
    torch.cuda.synchronize()
    third = a["page_table"][1, 2]
    assert torch.equal(kc.view(torch.int16)[third], before[third])           # positions 32..35 skipped
    assert not torch.equal(kc.view(torch.int16)[pt[1, 1]], before[pt[1, 1]])  # 20..31 written


def test_kv_inject_pools_off_16_byte_alignment():
    """Pools 8 bytes off a 16-byte boundary: the split-K sum (C = 2) writes
    the paged rows one element at a time instead of four."""
    w = replace(wl.WORKLOADS[1], name="inject-misaligned", C=2)
    run_and_check(w, 16, [5, 40], pool_offset=4)
