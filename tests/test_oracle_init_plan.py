"""Pins for the oracle's state projection (E1) and the integer split plan (a0)."""
import json
import os

import numpy as np
import pytest

import oracle


def test_one_hot_hidden_selects_weight_row():
    """u = e_i projects to row i of W, and the flat state index is (h*P+p)*N+n."""
    H, P, N, d = 3, 4, 5, 7
    W = np.random.default_rng(0).standard_normal((d, H * P * N))
    u = np.zeros((2, d))
    u[0, 2] = 1.0
    u[1, 6] = -3.0
    h0 = oracle.init_state(u, W)
    assert np.array_equal(h0[0], W[2]) and np.array_equal(h0[1], -3.0 * W[6])
    st = h0.reshape(2, H, P, N)
    for h, p, n in [(0, 0, 0), (1, 2, 3), (2, 3, 4)]:
        assert st[0, h, p, n] == W[2, (h * P + p) * N + n]


def test_rank_one_weight_closed_form():
    g = np.random.default_rng(1)
    a, c = g.standard_normal(9), g.standard_normal(12)
    u = g.standard_normal((3, 9))
    h0 = oracle.init_state(u, np.outer(a, c))
    assert np.allclose(h0, (u @ a)[:, None] * c[None, :], rtol=1e-13, atol=1e-13)


def test_linear_no_bias():
    g = np.random.default_rng(2)
    W = g.standard_normal((6, 10))
    u1, u2 = g.standard_normal((2, 6)), g.standard_normal((2, 6))
    assert not oracle.init_state(np.zeros((2, 6)), W).any()
    assert np.allclose(oracle.init_state(2 * u1 - u2, W),
                       2 * oracle.init_state(u1, W) - oracle.init_state(u2, W), atol=1e-13)
    with pytest.raises(ValueError):
        oracle.init_state(u1, W.T)


def test_plan_hand(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "plan_hand.json")))
    plan = oracle.split_plan(g["ctx"], g["pps"], g["max_ctx"])
    assert plan.dtype == np.int32
    assert plan.tolist() == g["plan"]
    assert len(plan) == oracle.plan_len(len(g["ctx"]), plan[3])


@pytest.mark.parametrize("pps", [1, 3, 8, 64, 10 ** 6])
def test_plan_invariants(pps):
    ctx = np.random.default_rng(pps).integers(0, 700, size=23)
    plan = oracle.split_plan(ctx, pps, max_ctx=800)
    C = len(ctx)
    total, p, c, M = plan[:4]
    n_splits = plan[4:4 + C]
    first = plan[4 + C:4 + 2 * C]
    req = plan[4 + 2 * C:4 + 2 * C + M]
    spl = plan[4 + 2 * C + M:]
    assert p == pps and c == C and total == n_splits.sum() <= M
    assert M == C * max(1, -(-(-(-800 // 16)) // pps))
    pages = -(-ctx // 16)
    # every context page is covered by exactly one split of its request
    for b in range(C):
        covered = []
        for s in range(n_splits[b]):
            i = first[b] + s
            assert req[i] == b and spl[i] == s
            covered += list(range(s * pps, min(pages[b], (s + 1) * pps)))
        assert covered == list(range(pages[b]))
        assert n_splits[b] >= 1
    assert (req[total:] == -1).all() and (spl[total:] == -1).all()


def test_plan_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.split_plan([10], 0)
    with pytest.raises(ValueError):
        oracle.split_plan([100], 4, max_ctx=50)
