"""Pins of the ratio-budget (D-cut) and packed-verification oracle.

CPU only.  Source: "AngelSpec", section 4.2, Eq. 20-24 and "Packing and
correctness".  The pages print no worked example for this part, so the pins are
hand-worked small cases, closed forms, brute force over every allocation, and
the identity between packed and unpacked verification.  A dropped bonus score
s_0, a budget off by one, a deep-first tie rule, a wrong argmax direction or a
shifted packed row fails at least one of them.
"""

import itertools

import numpy as np
import pytest

import oracle
from oracle import dcut as D


# --------------------------------------------------------------- Eq. 22

def test_budget_closed_forms():
    # B = 64, D = 15 (B(D+1) = 1024): the four ratios of the pages.
    assert [D.ratio_budget(r, 64, 15) for r in (0.25, 0.5, 0.75, 1.0)] == [256, 512, 768, 1024]
    # The floor max(B, .) binds: ceil(0.25 * 5 * 2) = 3 < 5.
    assert D.ratio_budget(0.25, 5, 1) == 5
    # Rounded up: 0.75 * 5 * 3 = 11.25 -> 12.
    assert D.ratio_budget(0.75, 5, 2) == 12
    # No drafts: only the bonus positions.
    assert all(D.ratio_budget(r, 3, 0) == 3 for r in (0.25, 0.5, 1.0))
    # The ratio is the float32 value: float32(0.3) = 0.30000001192..., so
    # 0.3 * 100 rounds up to 31, not 30.
    assert D.ratio_budget(0.3, 10, 9) == 31
    assert D.ratio_budget(0.5, 10, 9) == 50


# --------------------------------------------------------------- Eq. 20

def test_scores_prefix_product_with_bonus():
    s = D.scores(np.array([[0.5, 0.5, 0.5], [1.0, 0.25, 0.0]]))
    np.testing.assert_array_equal(s, [[1, 0.5, 0.25, 0.125], [1, 1, 0.25, 0]])


def test_scores_clamp_out_of_range_confidence():
    s = D.scores(np.array([[1.5, 0.5, -0.2, 0.5], [np.nan, 0.9, 0.9, 0.9]]))
    np.testing.assert_array_equal(s, [[1, 1, 0.5, 0, 0], [1, 0, 0, 0, 0]])


# ------------------------------------------------ hand-worked small case

def test_hand_worked_case():
    # c = [[1, .5], [.5, .5]] -> scores b0 = [1, 1, .5], b1 = [1, .5, .25].
    # Order (score desc, position asc, request asc):
    #   (0,0) (1,0) (0,1) | (1,1) (0,2) | (1,2)
    # B(D+1) = 6; K = max(2, ceil(rho * 6)) = 2, 3, 5, 6.
    #   K=2: n = [0, 0], U = 1 + 1                     = 2
    #   K=3: n = [1, 0], U = (1 + 1) + 1               = 3
    #   K=5: n = [2, 1], U = (1 + 1 + .5) + (1 + .5)   = 4
    #   K=6: n = [2, 2], U = 2.5 + 1.75                = 4.25
    # C = [1, 1.2, 1.5, 2]: U/C = 2, 2.5, 2.667, 2.125 -> rho = 0.75.
    c = np.array([[1.0, 0.5], [0.5, 0.5]])
    out = D.dcut(c, [0.25, 0.5, 0.75, 1.0], [1.0, 1.2, 1.5, 2.0])
    assert out["budgets"].tolist() == [2, 3, 5, 6]
    assert out["lengths"].tolist() == [[0, 0], [1, 0], [2, 1], [2, 2]]
    np.testing.assert_array_equal(out["utility"], [2.0, 3.0, 4.0, 4.25])
    assert out["ratio_index"] == 2 and out["total_rows"] == 5
    assert out["verify_len"].tolist() == [2, 1]
    assert out["row_offsets"].tolist() == [0, 3, 5]


def test_shallow_tie_rule_closed_form():
    """All scores equal (c = 1): depth is dealt out one level at a time, lower b first."""
    B, Dd = 5, 4
    s = D.scores(np.ones((B, Dd)))
    for m in range(B * Dd + 1):
        n = D.top_k_lengths(s, B + m)
        assert n.tolist() == [m // B + (b < m % B) for b in range(B)]


# ----------------------------------------------------- brute force, Eq. 21/23

def _brute_best(s, K):
    B, D1 = s.shape
    best = None
    for n in itertools.product(range(D1), repeat=B):
        if sum(n) + B != K:
            continue
        v = sum(float(s[b, : n[b] + 1].sum()) for b in range(B))
        best = v if best is None else max(best, v)
    return best


@pytest.mark.parametrize("seed", range(30))
def test_top_k_is_the_best_allocation(seed):
    g = np.random.default_rng(100 + seed)
    B = int(g.integers(1, 4))
    Dd = int(g.integers(1, 4))
    kind = seed % 3
    if kind == 0:
        c = g.uniform(0, 1, size=(B, Dd))
    elif kind == 1:
        c = g.choice([0.0, 0.5, 1.0], size=(B, Dd))         # many exact ties
    else:
        c = 1 / (1 + np.exp(-(g.normal(1.5, 1.0, size=(B, Dd)) - 0.08 * np.arange(Dd))))
    s = D.scores(c)
    draft_scores = np.sort(s[:, 1:].ravel())[::-1]
    for K in range(B, B * (Dd + 1) + 1):
        n = D.top_k_lengths(s, K)
        assert int((n + 1).sum()) == K and (n >= 0).all() and (n <= Dd).all()
        U = D.utility(s, n)
        # no allocation of K positions has more estimated progress ...
        assert abs(U - _brute_best(s, K)) <= 1e-12 * max(1.0, U)
        # ... and it is the B bonus scores plus the K - B best draft scores
        assert abs(U - (B + draft_scores[: K - B].sum())) <= 1e-12 * max(1.0, U)


# ------------------------------------------------------------- Eq. 24

def test_ratio_choice_extremes():
    g = np.random.default_rng(7)
    B, Dd = 6, 5
    c = g.uniform(0.05, 0.95, size=(B, Dd))
    ratios = [0.25, 0.5, 0.75, 1.0]
    # Equal costs: the largest progress wins (U never falls as K grows).
    out = D.dcut(c, ratios, [1.0] * 4)
    assert out["ratio_index"] == 3 and out["total_rows"] == B * (Dd + 1)
    assert np.all(np.diff(out["utility"]) > 0)
    # Zero confidence: U = B everywhere; the first of the cheapest wins.  The
    # budget is still filled: K = 18 keeps 12 zero-score drafts, 2 per request.
    out = D.dcut(np.zeros((B, Dd)), ratios, [2.0, 1.0, 1.0, 3.0])
    np.testing.assert_array_equal(out["utility"], [B] * 4)
    assert out["ratio_index"] == 1 and out["total_rows"] == 18
    assert out["verify_len"].tolist() == [2] * B
    # c = 1 and cost proportional to K: U / C is the same for every ratio -> the first.
    Ks = [D.ratio_budget(r, B, Dd) for r in ratios]
    out = D.dcut(np.ones((B, Dd)), ratios, [0.01 * k for k in Ks])
    assert out["ratio_index"] == 0
    # A steep cost for depth picks the smallest budget.
    out = D.dcut(c, ratios, [1.0, 10.0, 100.0, 1000.0])
    assert out["ratio_index"] == 0 and out["total_rows"] == Ks[0]


def test_ratio_order_is_the_callers():
    g = np.random.default_rng(8)
    c = g.uniform(0.05, 0.95, size=(4, 3))
    out = D.dcut(c, [1.0, 0.25], [1.0, 1.0])
    assert out["ratio_index"] == 0 and out["total_rows"] == 16


def test_dcut_outputs_are_consistent():
    g = np.random.default_rng(9)
    B, Dd = 16, 15
    c = 1 / (1 + np.exp(-(g.normal(1.5, 1.0, size=(B, Dd)) - 0.08 * np.arange(Dd))))
    K = np.array([D.ratio_budget(r, B, Dd) for r in (0.25, 0.5, 0.75, 1.0)])
    out = D.dcut(c, [0.25, 0.5, 0.75, 1.0], 1.0 + 0.02 * K)
    n, off = out["verify_len"], out["row_offsets"]
    assert off[0] == 0 and off[-1] == out["total_rows"] == int((n + 1).sum())
    np.testing.assert_array_equal(np.diff(off), n + 1)
    for i, Kr in enumerate(out["budgets"]):
        assert int((out["lengths"][i] + 1).sum()) == Kr


# ------------------------------------------------------ packed verification

def _tiny(seed, B=5, Dd=4, V=11, T=1.0):
    g = np.random.default_rng(seed)
    z = g.normal(0, 2, size=(B, Dd + 1, V))
    ql = z[:, :Dd] + g.normal(0, 0.7, size=(B, Dd, V))
    q = np.exp(ql - ql.max(-1, keepdims=True))
    q /= q.sum(-1, keepdims=True)
    x = np.array([[g.choice(V, p=q[b, k]) for k in range(Dd)] for b in range(B)])
    u = g.uniform(size=(B, Dd + 1))
    c = g.uniform(0.1, 1.0, size=(B, Dd))
    return z, q, x, u, c


@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
@pytest.mark.parametrize("seed", range(6))
def test_packed_verify_is_unpacked_verify(seed, T):
    """Packing changes which target rows exist, not how a kept row is verified."""
    z, q, x, u, c = _tiny(seed)
    B, Dd = x.shape
    out = D.dcut(c, [0.25, 0.5, 0.75, 1.0], [1.0, 1.3, 1.7, 2.2])
    off, n = out["row_offsets"], out["verify_len"]
    extra = seed % 3                                   # spare rows past the last request
    zp = D.pack_rows(z, off, rows=int(off[-1]) + extra)
    # the packed row of (b, k) is the target row of (b, k)
    for b in range(B):
        for k in range(n[b] + 1):
            np.testing.assert_array_equal(zp[off[b] + k], z[b, k])
    got = D.verify_packed(zp, off, q, x, u, T)
    ref = oracle.verify(z, q, x, u, T, verify_len=n)
    np.testing.assert_array_equal(got["accepted"], ref["accepted"])
    np.testing.assert_array_equal(got["tokens"], ref["tokens"])


def test_packed_verify_bad_offsets():
    z, q, x, u, _ = _tiny(3, B=4, Dd=3)
    n = np.array([1, 3, 0, 2])
    off = D.row_offsets(n)                              # [0, 2, 6, 7, 10]
    zp = D.pack_rows(z, off)
    ref = oracle.verify(z, q, x, u, 1.0, verify_len=n)
    bad = off.copy()
    bad[2] = 1                                          # request 1: 5 rows > D+1; request 2: 6 rows
    got = D.verify_packed(zp, bad, q, x, u, 1.0)
    assert got["accepted"].tolist()[1:3] == [-1, -1]
    assert (got["tokens"][1:3] == -1).all()
    for b in (0, 3):
        assert got["accepted"][b] == ref["accepted"][b]
        np.testing.assert_array_equal(got["tokens"][b], ref["tokens"][b])
    # rows past the buffer, a negative start, and an empty request
    for off_bad, who in (([0, 2, 6, 7, 11], 3), ([-1, 2, 6, 7, 10], 0), ([0, 2, 2, 7, 10], 1)):
        got = D.verify_packed(zp, np.array(off_bad), q, x, u, 1.0)
        assert got["accepted"][who] == -1 and (got["tokens"][who] == -1).all()
