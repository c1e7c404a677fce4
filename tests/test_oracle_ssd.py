"""Pins for the oracle's Mamba-2 scan (E2 recurrence, E3 chunked restatement).

Each check fixes the scan by something other than the oracle's own code:
hand-derived values, the explicit-product solution of the linear recurrence,
and the special cases that reduce it to textbook forms.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle


def _rand(seed, C=2, K=6, H=4, P=3, ng=2, N=5, state=True):
    g = np.random.default_rng(seed)
    x = g.standard_normal((C, K, H, P))
    delta = np.logaddexp(0, g.standard_normal((C, K, H)) - 1.0)
    A = -np.exp(g.uniform(0, 1, H))
    B = g.standard_normal((C, K, ng, N))
    Cm = g.standard_normal((C, K, ng, N))
    h0 = g.standard_normal((C, H, P, N)) if state else None
    return x, delta, A, B, Cm, h0


def _explicit_products(x, delta, A, B, Cm, h0):
    """Solution of H_t = a_t H_{t-1} + b_t written with explicit products:
    H_t = (prod_{r<=t} a_r) h0 + sum_{s<=t} (prod_{s<r<=t} a_r) b_s."""
    C, K, H, P = x.shape
    ng, N = B.shape[2], B.shape[3]
    y = np.zeros((C, K, H, P))
    hf = np.zeros((C, H, P, N))
    for b in range(C):
        for h in range(H):
            grp = h // (H // ng)
            a = [math.exp(delta[b, r, h] * A[h]) for r in range(K)]
            for t in range(K):
                Ht = np.prod(a[:t + 1]) * h0[b, h]
                for s in range(t + 1):
                    Ht = Ht + np.prod(a[s + 1:t + 1]) * delta[b, s, h] * np.outer(x[b, s, h], B[b, s, grp])
                y[b, t, h] = Ht @ Cm[b, t, grp]
                if t == K - 1:
                    hf[b, h] = Ht
    return y, hf


def _close(a, b, tol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.abs(b).max()))
    assert np.abs(a - b).max() <= tol * scale, np.abs(a - b).max()


def test_golden_two_heads(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "ssd_two_heads.json")))
    A = np.array([-math.log(2.0), 0.0])
    args = [np.array(g[k], dtype=np.float64) for k in ("x", "delta")]
    x, delta = args
    B, Cm, h0 = (np.array(g[k], dtype=np.float64) for k in ("B", "Cm", "h0"))
    for fn in (oracle.ssd_recurrence, lambda *a, **k: oracle.ssd_chunked(*a, chunk=1, **k),
               lambda *a, **k: oracle.ssd_chunked(*a, chunk=2, **k)):
        y, hf = fn(x, delta, A, B, Cm, h0=h0)
        _close(y, g["y"], 1e-14)
        _close(hf, g["h_final"], 1e-14)


def test_recurrence_matches_explicit_products():
    x, delta, A, B, Cm, h0 = _rand(1)
    y, hf = oracle.ssd_recurrence(x, delta, A, B, Cm, h0=h0)
    ye, hfe = _explicit_products(x, delta, A, B, Cm, h0)
    _close(y, ye)
    _close(hf, hfe)


@pytest.mark.parametrize("K,Q", [(6, 1), (6, 2), (6, 3), (6, 6), (16, 4), (13, 4), (16, 16), (5, 8)])
def test_chunked_equals_recurrence_step_by_step(K, Q):
    x, delta, A, B, Cm, h0 = _rand(10 + K + Q, K=K)
    y_r, hf_r = oracle.ssd_recurrence(x, delta, A, B, Cm, h0=h0)
    y_c, hf_c = oracle.ssd_chunked(x, delta, A, B, Cm, h0=h0, chunk=Q)
    _close(y_c, y_r)
    _close(hf_c, hf_r)
    # the state at every chunk boundary equals the recurrence's state there
    for t_end in range(Q, K, Q):
        _, h_prefix_r = oracle.ssd_recurrence(x[:, :t_end], delta[:, :t_end], A, B[:, :t_end], Cm[:, :t_end], h0=h0)
        _, h_prefix_c = oracle.ssd_chunked(x[:, :t_end], delta[:, :t_end], A, B[:, :t_end], Cm[:, :t_end], h0=h0, chunk=Q)
        _close(h_prefix_c, h_prefix_r)


def test_zero_state_is_plain_scan():
    x, delta, A, B, Cm, _ = _rand(2, state=False)
    C, K, H, P = x.shape
    N = B.shape[3]
    y0, hf0 = oracle.ssd_recurrence(x, delta, A, B, Cm, h0=None)
    y1, hf1 = oracle.ssd_recurrence(x, delta, A, B, Cm, h0=np.zeros((C, H, P, N)))
    assert np.array_equal(y0, y1) and np.array_equal(hf0, hf1)
    # a zero last-token hidden state projects to a zero initial state
    h0 = oracle.init_state(np.zeros((C, 7)), np.random.default_rng(0).standard_normal((7, H * P * N)))
    assert not h0.any()
    y2, _ = oracle.ssd_chunked(x, delta, A, B, Cm, h0=h0.reshape(C, H, P, N), chunk=4)
    _close(y2, y0)


def test_superposition_and_state_closed_form():
    x, delta, A, B, Cm, h0 = _rand(3)
    y, _ = oracle.ssd_recurrence(x, delta, A, B, Cm, h0=h0)
    y_x, _ = oracle.ssd_recurrence(x, delta, A, B, Cm, h0=None)
    y_h, _ = oracle.ssd_recurrence(np.zeros_like(x), delta, A, B, Cm, h0=h0)
    _close(y, y_x + y_h)
    # the state-only response decays by exp(A * sum_{r<=t} delta_r)
    C, K, H, P = x.shape
    ng = B.shape[2]
    for t in range(K):
        for h in range(H):
            decay = np.exp(A[h] * delta[:, :t + 1, h].sum(axis=1))      # [C]
            want = decay[:, None] * np.einsum("cpn,cn->cp", h0[:, h], Cm[:, t, h // (H // ng)])
            _close(y_h[:, t, h], want)


def test_delta_zero_keeps_state():
    x, delta, A, B, Cm, h0 = _rand(4)
    dz = np.zeros_like(delta)
    for fn in (oracle.ssd_recurrence, oracle.ssd_chunked):
        y, hf = fn(x, dz, A, B, Cm, h0=h0)
        _close(hf, h0)
        H = x.shape[2]
        ng = B.shape[2]
        for h in range(H):
            _close(y[:, :, h], np.einsum("cpn,ctn->ctp", h0[:, h], Cm[:, :, h // (H // ng)]))


def test_no_decay_is_running_sum():
    x, delta, A, B, Cm, h0 = _rand(5)
    A0 = np.zeros_like(A)
    C, K, H, P = x.shape
    ng = B.shape[2]
    grp = np.arange(H) // (H // ng)
    y, hf = oracle.ssd_chunked(x, delta, A0, B, Cm, h0=h0, chunk=4)
    acc = h0.copy()
    for t in range(K):
        acc = acc + np.einsum("ch,chp,chn->chpn", delta[:, t], x[:, t], B[:, t][:, grp])
        _close(y[:, t], np.einsum("chpn,chn->chp", acc, Cm[:, t][:, grp]))
    _close(hf, acc)


def test_single_step():
    x, delta, A, B, Cm, h0 = _rand(6, K=1)
    y, hf = oracle.ssd_recurrence(x, delta, A, B, Cm, h0=h0)
    C, _, H, P = x.shape
    ng = B.shape[2]
    for b in range(C):
        for h in range(H):
            gi = h // (H // ng)
            H1 = math.exp(delta[b, 0, h] * A[h]) * h0[b, h] + delta[b, 0, h] * np.outer(x[b, 0, h], B[b, 0, gi])
            _close(hf[b, h], H1)
            _close(y[b, 0, h], H1 @ Cm[b, 0, gi])


def test_dskip_adds_skip_term():
    x, delta, A, B, Cm, h0 = _rand(7)
    D = np.random.default_rng(9).standard_normal(x.shape[2])
    y0, _ = oracle.ssd_recurrence(x, delta, A, B, Cm, h0=h0)
    y1, _ = oracle.ssd_recurrence(x, delta, A, B, Cm, h0=h0, Dskip=D)
    y2, _ = oracle.ssd_chunked(x, delta, A, B, Cm, h0=h0, chunk=4, Dskip=D)
    _close(y1, y0 + D[None, None, :, None] * x)
    _close(y2, y1)


def test_group_sharing():
    """ng groups: heads in one group see the same B/Cm; ng=H equals separate heads."""
    x, delta, A, B, Cm, h0 = _rand(8, H=4, ng=4)
    y, _ = oracle.ssd_recurrence(x, delta, A, B, Cm, h0=h0)
    for h in range(4):
        yh, _ = oracle.ssd_recurrence(x[:, :, h:h + 1], delta[:, :, h:h + 1], A[h:h + 1],
                                      B[:, :, h:h + 1], Cm[:, :, h:h + 1], h0=h0[:, h:h + 1])
        _close(y[:, :, h:h + 1], yh)
    # ng=1: every head reads group 0
    x, delta, A, B, Cm, h0 = _rand(9, H=4, ng=1)
    y, _ = oracle.ssd_recurrence(x, delta, A, B, Cm, h0=h0)
    yh, _ = oracle.ssd_recurrence(x[:, :, 3:4], delta[:, :, 3:4], A[3:4], B, Cm, h0=h0[:, 3:4])
    _close(y[:, :, 3:4], yh)
