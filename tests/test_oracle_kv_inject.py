"""Pins of the oracle's drafter-side KV injection (the contrast workload).

The write convention is checked against the attention oracle's page gather
(pinned on its own): what the injection writes at positions start .. start+n
must come back, through the page table, as the last n context rows.  A
one-hot hidden state pins the [out, in] weight orientation and the K | V
split; torch's float64 linear pins the projection; everything not written
must be bit-identical.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from hybrid_mamba_attention_amd import workloads as wl

W = replace(wl.WORKLOADS[0], name="inject-pins", C=3, d_model=64, Hkv=2, D=64, seed=31)


@pytest.mark.parametrize("P", [16, 64])
def test_written_rows_come_back_through_the_page_table(P):
    n = 21                                               # crosses page boundaries
    a = wl.make_inject_inputs(W, n, ctx_lens=[0, 13, 60], page_size=P)
    kp, vp, kv = oracle.kv_inject(a["hidden"], a["w_kv"], a["k_cache"], a["v_cache"], a["page_table"],
                                  a["start"], Hkv=W.Hkv, D=W.D, dtype=W.dtype)
    HD = W.Hkv * W.D
    for b in range(W.C):
        L = int(a["start"][b]) + n
        for j in range(W.Hkv):
            kg = oracle.gather_context(kp, a["page_table"][b], L, j, "f32")
            vg = oracle.gather_context(vp, a["page_table"][b], L, j, "f32")
            # (the gather reads the float64 pool as stored fp32: round kv the same way)
            f32 = lambda x: x.astype(np.float32).astype(np.float64)
            np.testing.assert_array_equal(kg[-n:], f32(kv[b, :, j * W.D:(j + 1) * W.D]))
            np.testing.assert_array_equal(vg[-n:], f32(kv[b, :, HD + j * W.D:HD + (j + 1) * W.D]))
            # the existing context is untouched
            old = oracle.gather_context(oracle.decode(a["k_cache"], "f32"), a["page_table"][b],
                                        int(a["start"][b]), j, "f32")
            np.testing.assert_array_equal(kg[:-n], old)


def test_nothing_else_is_written():
    n = 5
    a = wl.make_inject_inputs(W, n, ctx_lens=[3, 16, 31])
    kp, vp, _ = oracle.kv_inject(a["hidden"], a["w_kv"], a["k_cache"], a["v_cache"], a["page_table"],
                                 a["start"], Hkv=W.Hkv, D=W.D, dtype=W.dtype)
    written = np.zeros(kp.shape[:2], dtype=bool)
    for b in range(W.C):
        for i in range(n):
            p = int(a["start"][b]) + i
            written[a["page_table"][b, p // 16], p % 16] = True
    assert written.sum() == W.C * n
    k0, v0 = oracle.decode(a["k_cache"], "f32"), oracle.decode(a["v_cache"], "f32")
    np.testing.assert_array_equal(kp[~written], k0[~written])     # NaN slots compare equal too
    np.testing.assert_array_equal(vp[~written], v0[~written])


def test_one_hot_hidden_selects_a_weight_column_and_the_k_v_split():
    r = 7
    hid = np.zeros((1, 1, W.d_model), np.float32)
    hid[0, 0, r] = 1.0
    w = np.random.default_rng(3).standard_normal((2 * W.Hkv * W.D, W.d_model)).astype(np.float32)
    kv = oracle.kv_project(hid, w)
    np.testing.assert_array_equal(kv[0, 0], w[:, r])
    a = wl.make_inject_inputs(replace(W, C=1), 1, ctx_lens=[17])
    kp, vp, _ = oracle.kv_inject(hid, w, a["k_cache"], a["v_cache"], a["page_table"], a["start"],
                                 Hkv=W.Hkv, D=W.D, dtype="f32")
    page = a["page_table"][0, 1]
    np.testing.assert_array_equal(kp[page, 1].ravel(), w[:W.Hkv * W.D, r])
    np.testing.assert_array_equal(vp[page, 1].ravel(), w[W.Hkv * W.D:, r])


def test_projection_matches_torch_linear():
    a = wl.make_inject_inputs(W, 9)
    got = oracle.kv_project(a["hidden"], a["w_kv"])
    want = F.linear(torch.from_numpy(a["hidden"].astype(np.float64)), torch.from_numpy(a["w_kv"].astype(np.float64)))
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-13, atol=1e-13)


def test_extra_bytes_per_token():
    # one drafter layer with the target's KV shape adds one target layer's KV per token
    assert oracle.extra_kv_bytes_per_token(8, 128, 2) == 4096
    assert oracle.extra_kv_bytes_per_token(8, 128, 2, layers=5) == 5 * 4096
