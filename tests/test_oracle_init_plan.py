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
    for case in g["cases"]:
        plan = oracle.range_plan(case["ctx"], K=case["K"], w_max=case["w_max"], page_size=case["page"],
                                 range_pages=case["range_pages"], rows=case.get("rows", 64))
        assert plan.dtype == np.int32
        head = case["plan_head"]
        assert plan[:len(head)].tolist() == head
        assert (plan[len(head):] == -1).all()
        assert len(plan) == oracle.plan_len(len(case["ctx"]), case["w_max"])
        C = len(case["ctx"])
        for b, want in case.get("pieces_of_request", {}).items():
            b = int(b)
            L = -(-case["ctx"][b] // 16) + -(-case["K"] // 16)
            assert [list(p) for p in oracle.request_pieces(plan, C, b, L)] == want


CASES = [(16, 64, 0, 64), (16, 7, 0, 64), (16, 64, 3, 64), (32, 64, 0, 64), (64, 16, 5, 64), (256, 64, 0, 64),
         (16, 3, 0, 64), (16, 64, 0, 128), (64, 16, 0, 256), (16, 64, 3, 128)]


def test_segment_charge():
    """The fixed cost of automatic ranges: ceil(12 / g) units, ceil(24 / g)
    above 64 query rows per kv head, none for fixed ranges."""
    assert [oracle.segment_granules(p, 0, 64) for p in (16, 32, 64, 128, 256)] == [6, 6, 3, 2, 1]
    assert [oracle.segment_granules(p, 0, 128) for p in (16, 32, 64, 128, 256)] == [12, 12, 6, 3, 2]
    assert oracle.segment_granules(16, 0, 65) == 12 and oracle.segment_granules(16, 0, 8) == 6
    assert oracle.segment_granules(16, 4, 128) == 0


@pytest.mark.parametrize("page,w_max,range_pages,rows", CASES)
def test_plan_invariants(page, w_max, range_pages, rows):
    """Every slab of every request lies in exactly one of its pieces, in
    order; each range's segments tile it; slots of partial pieces are unique;
    automatic ranges differ in size by at most one granule."""
    rng = np.random.default_rng(page + w_max + range_pages)
    for trial in range(20):
        C = int(rng.integers(1, 30))
        K = int(rng.integers(1, 65))
        ctx = rng.integers(0, 3000, size=C) * (rng.random(C) < 0.9)
        try:
            plan = oracle.range_plan(ctx, K=K, w_max=w_max, page_size=page, range_pages=range_pages, rows=rows)
        except ValueError:
            assert range_pages > 0   # fixed ranges beyond the capacity are refused
            continue
        f = oracle.plan.unpack(plan, C)
        W, T, g, B = f["W"], f["T"], f["g"], f["B"]
        G = oracle.request_granules(ctx, K, page)
        sigma = oracle.segment_granules(page, range_pages, rows)
        assert g == max(2, page // 16) and T == (G + sigma).sum() and 1 <= W <= min(w_max, T)
        assert B[0] == 0 and B[-1] == T and (np.diff(B) >= 1).all()
        if range_pages == 0:
            assert np.diff(B).max() - np.diff(B).min() <= 1
        else:
            R = max(1, -(-(range_pages * (page // 16)) // g))
            assert (np.diff(B)[:-1] == R).all() and 1 <= np.diff(B)[-1] <= R
        slots = []
        for b in range(C):
            L = -(-int(ctx[b]) // 16) + -(-K // 16)
            ps = oracle.request_pieces(plan, C, b, L)
            assert ps[0][2] == 0 and ps[-1][3] == L
            for (w0, s0, lo0, hi0), (w1, s1, lo1, hi1) in zip(ps, ps[1:]):
                assert hi0 == lo1 and w1 == w0 + 1
            for w, slot, lo, hi in ps:
                assert lo < hi and lo % g == 0 and slot // 2 == w
                assert B[w] <= f["S"][b] + lo // g and f["S"][b] + (hi - 1) // g < B[w + 1]
            if len(ps) > 1:
                slots += [p[1] for p in ps]
        assert len(slots) == len(set(slots))


def test_plan_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.range_plan([10], K=0, w_max=4)
    with pytest.raises(ValueError):
        oracle.range_plan([-1], K=4, w_max=4)
    with pytest.raises(ValueError):
        oracle.range_plan([10], K=4, w_max=4, page_size=48)
    with pytest.raises(ValueError):
        oracle.range_plan([4000], K=4, w_max=4, range_pages=1)
