"""The seeded workload generator: reproducibility, page-pool structure, poison
placement and the bf16 rounding of inputs."""
import numpy as np
import pytest
import torch

from hybrid_mamba_attention_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    a = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 3.0e38, -1e-40, 1.00390625, 1.01171875], np.float32)])
    ours = wl.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert wl.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_reproducible_and_thread_independent(monkeypatch):
    w = wl.WORKLOADS[0]
    a = wl.make_inputs(w)
    monkeypatch.setattr(wl, "CHUNK", 1 << 22)
    monkeypatch.setattr(wl, "_threads", lambda: 1)
    b = wl.make_inputs(w)
    for k in a.arrays:
        assert np.array_equal(a.arrays[k], b.arrays[k], equal_nan=True), k
    assert np.array_equal(a.page_table, b.page_table)


def test_parts_share_streams():
    w = wl.WORKLOADS[0]
    full = wl.make_inputs(w)
    only = wl.make_inputs(w, parts=("attn",))
    assert "u" not in only.arrays
    assert np.array_equal(full.arrays["q"], only.arrays["q"])
    assert np.array_equal(full.arrays["k_cache"], only.arrays["k_cache"], equal_nan=True)


def test_page_pool_structure_and_poison():
    w = wl.WORKLOADS[0]
    inp = wl.make_inputs(w, ctx_lens=[37, 0, 16, 1, 80][:w.C] if w.C > 1 else [37])
    pt, ctx = inp.page_table, inp.ctx_lens
    used = []
    for b, L in enumerate(ctx):
        n = -(-int(L) // 16)
        assert (pt[b, :n] >= 0).all() and (pt[b, n:] == -1).all()
        used += pt[b, :n].tolist()
    assert len(set(used)) == len(used)                       # no page shared between requests
    assert inp.num_pages == len(used) + wl.SPARE_PAGES
    kc = inp.arrays["k_cache"]
    spare = sorted(set(range(inp.num_pages)) - set(used))
    assert np.isnan(kc[spare]).all()
    last = pt[0, (37 - 1) // 16]
    assert np.isnan(kc[last, 37 % 16:]).all() and not np.isnan(kc[last, :37 % 16]).any()


def test_multi_request_interleave():
    w = wl.WORKLOADS[2]
    ss = np.random.SeedSequence(5)
    ctx = wl.draw_ctx_lens(w, ss)
    assert ctx.min() >= 512 and ctx.max() <= 4096 and len(ctx) == 32
    pt, pool, pages_of = wl.build_page_table(ctx, np.random.SeedSequence(6))
    allp = np.concatenate(pages_of)
    assert len(np.unique(allp)) == len(allp) == pool - wl.SPARE_PAGES
    # pages of one request are not a contiguous run of the pool
    assert (np.diff(np.sort(pages_of[0])) > 1).any()


def test_loguniform_ctx_range():
    w = wl.WORKLOADS[4]
    ctx = wl.draw_ctx_lens(w, np.random.SeedSequence(1))
    assert ctx.min() >= 1024 and ctx.max() <= 16384
    assert np.median(ctx) < 8000                             # log-uniform, not uniform


def test_value_recipe():
    w = wl.WORKLOADS[0]
    inp = wl.make_inputs(w)
    a = inp.arrays
    assert (a["delta"] > 0).all() and np.median(a["delta"]) < 0.05
    assert (a["A"] <= -1).all() and (a["A"] >= -np.e).all()
    assert 0.015 < a["w_init"].std() < 0.025
    assert abs(a["u"].std() - 1) < 0.1


def test_shapes_of_all_workloads():
    for w in wl.WORKLOADS.values():
        assert w.Hq % w.Hkv == 0 and w.H % w.ng == 0
    assert wl.WORKLOADS[1].S == 32768 and wl.WORKLOADS[4].S == 131072 and wl.WORKLOADS[0].S == 4096
    assert wl.kv_bytes(wl.WORKLOADS[3], [8192] * 128) == 2 ** 32


def test_block_inputs_shapes_and_reproducibility():
    w = wl.WORKLOADS[1]
    small = wl.replace(w, C=2, d_model=256)
    a, b = wl.make_block_inputs(small), wl.make_block_inputs(small)
    d_inner, conv_dim, d_proj = wl.block_sizes(small)
    assert (d_inner, conv_dim, d_proj) == (1024, 1088, 2128)
    assert a["hidden"].shape == (2, 16, 256) and a["hidden"].dtype == np.uint16
    assert a["w_in"].shape == (d_proj, 256) and a["w_out"].shape == (256, d_inner)
    assert a["conv_w"].shape == (conv_dim, 4) and a["conv_w"].dtype == np.float32
    assert a["h0"].shape == (2, 16, 64, 32) and np.all(a["dt_bias"] == -4.0)
    for k in a:
        if isinstance(a[k], np.ndarray):
            assert np.array_equal(a[k], b[k]), k
    # the block's streams leave the layer's inputs untouched
    assert np.array_equal(wl.make_inputs(small, parts=("mamba",)).arrays["u"],
                          wl.make_inputs(small, parts=("mamba",)).arrays["u"])
