"""Pins of the float64 oracle against what the pages and the mathematics fix.

CPU only.  Each test names the passage (page title, section / equation) or the
mathematical fact it checks.  A plausible slip in the oracle -- a dropped term
in the residual, a wrong comparison direction, an off-by-one in the first
rejection, a transposed p/q, a wrong uniform slot -- fails at least one of them.
"""

import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle


GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _one_request(p_rows, q_rows, x, u, T=1.0, verify_len=None):
    """Build oracle inputs from explicit probability rows (logits = ln p)."""
    with np.errstate(divide="ignore"):
        z = np.log(np.asarray(p_rows, np.float64))[None]
    q = np.asarray(q_rows, np.float64)[None]
    return oracle.verify(z, q, np.asarray(x)[None], np.asarray(u, np.float64)[None], T,
                         None if verify_len is None else [verify_len])


def _batch(p_rows, q_rows, xs, us, T=1.0, verify_len=None):
    """Same rows for every request; xs [N, G], us [N, G+1]."""
    N = len(xs)
    with np.errstate(divide="ignore"):
        z = np.broadcast_to(np.log(np.asarray(p_rows, np.float64)), (N,) + np.shape(p_rows))
    q = np.broadcast_to(np.asarray(q_rows, np.float64), (N,) + np.shape(q_rows))
    return oracle.verify(z, q, np.asarray(xs), np.asarray(us, np.float64), T, verify_len)


# --------------------------------------------------------------------------
# Worked example: "breaking down dspark and its lineage", section
# "Preserving the target distribution during verification".
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def page():
    with open(os.path.join(GOLDEN, "page_example.json")) as f:
        return json.load(f)


def test_page_table_arithmetic(page):
    p, q = np.array(page["p_target"]), np.array(page["q_draft"])
    # The oracle's residual is the "p sticks up" row, and its total is the table's.
    np.testing.assert_allclose(oracle.residual(p, q), page["p_sticks_up"], atol=1e-15)
    np.testing.assert_allclose(oracle.residual(p, q).sum(), page["p_sticks_up_sum"], atol=1e-15)
    np.testing.assert_allclose(oracle.residual(q, p), page["q_sticks_up"], atol=1e-15)
    # Eq. 4-5 of AngelSpec: overlap = 1 - TV.
    assert abs(np.minimum(p, q).sum() - page["overlap_sum"]) < 1e-15
    assert abs(0.5 * np.abs(p - q).sum() - page["tv"]) < 1e-15


def test_page_deterministic_decisions(page):
    p, q = page["p_target"], page["q_draft"]
    rows_p = [p, p]          # row 1 is the bonus row
    rows_q = [q]
    # Token 1 is over-proposed: accept probability 0.3/0.5 = 0.6.
    assert _one_request(rows_p, rows_q, [1], [0.59, 0.3])["accepted"][0] == 1
    r = _one_request(rows_p, rows_q, [1], [0.61, 0.3])
    assert r["accepted"][0] == 0
    # After a rejection the draw is from the normalised residual (0.5, 0, 0.5).
    assert abs(r["resid_mass"][0] - page["p_sticks_up_sum"]) < 1e-12
    for u1, tok in [(0.0, 0), (0.25, 0), (0.4999, 0), (0.5001, 2), (0.75, 2), (0.999999, 2)]:
        out = _one_request(rows_p, rows_q, [1], [0.99, u1])
        assert out["tokens"][0].tolist() == [tok, -1], (u1, out["tokens"])
    # Tokens 0 and 2 are under-proposed: always kept, for every u0 in [0,1).
    for x in (0, 2):
        for u0 in (0.0, 0.5, 0.999999):
            out = _one_request(rows_p, rows_q, [x], [u0, 0.1])
            assert out["accepted"][0] == 1
            # bonus token drawn from row 1 = p with u=0.1 -> token 0
            assert out["tokens"][0].tolist() == [x, 0]


def test_page_acceptance_mass_and_output_law(page):
    """Integrate the oracle exactly over (x ~ q, u0, u1) on a midpoint grid.

    Every threshold of this example (0.6 for u0, 0.5 for the residual draw,
    0.5 and 0.8 for a bonus draw) is a multiple of 1/M, so the midpoint rule is
    exact: the acceptance mass must be 0.8 and the first emitted token must
    follow p = (0.5, 0.3, 0.2).
    """
    p, q = np.array(page["p_target"]), np.array(page["q_draft"])
    M = 40
    grid = (np.arange(M) + 0.5) / M
    U0, U1 = np.meshgrid(grid, grid, indexing="ij")
    us = np.stack([U0.ravel(), U1.ravel()], axis=1)
    acc_mass = 0.0
    law = np.zeros(3)
    for x in range(3):
        out = _batch([p, p], [q], np.full((len(us), 1), x), us)
        acc_mass += q[x] * np.mean(out["accepted"] == 1)
        first = out["tokens"][:, 0]
        law += q[x] * np.bincount(first, minlength=3) / len(us)
    assert abs(acc_mass - page["overlap_sum"]) < 1e-12
    np.testing.assert_allclose(law, page["p_target"], atol=1e-12)


# --------------------------------------------------------------------------
# Exact enumeration with grid-aligned thresholds (tiny V, gamma).
# Checks: emitted law at each position = p_k given the position is reached;
# P(a >= k) = prod alpha_i; E[a + 1] = 1 + sum_j prod_{i<=j} alpha_i
# (UraionSpec, section "Speculative Decoding", Eq. expected_tau).
# --------------------------------------------------------------------------

# Per-position (p_k, q_k) whose ratios p/q and residual / bonus CDF breakpoints
# are all multiples of 1/10.
P_ROWS = [[0.5, 0.3, 0.2], [0.2, 0.4, 0.4], [0.3, 0.3, 0.4]]
Q_ROWS = [[0.4, 0.5, 0.1], [0.5, 0.25, 0.25]]


def _enumerate_law(P_rows, Q_rows, M=10):
    G = len(Q_rows)
    V = len(P_rows[0])
    grid = (np.arange(M) + 0.5) / M
    us = np.array(list(itertools.product(grid, repeat=G + 1)))
    pos_law = np.zeros((G + 1, V))       # P(emit v at k, reach k)
    reach = np.zeros(G + 2)              # P(a >= k)
    e_len = 0.0
    for xs in itertools.product(range(V), repeat=G):
        w = np.prod([Q_rows[k][xs[k]] for k in range(G)])
        out = _batch(P_rows, Q_rows, np.tile(xs, (len(us), 1)), us)
        a = out["accepted"]
        tok = out["tokens"]
        for k in range(G + 1):
            sel = a >= k
            reach[k] += w * sel.mean()
            pos_law[k] += w * np.bincount(tok[sel, k], minlength=V) / len(us)
        e_len += w * np.mean(a + 1)
    return pos_law, reach, e_len


def test_enumeration_lossless_law_and_tau():
    pos_law, reach, e_len = _enumerate_law(P_ROWS, Q_ROWS)
    P, Q = np.array(P_ROWS), np.array(Q_ROWS)
    alpha = np.minimum(P[:2], Q).sum(axis=1)          # (0.8, 0.7)
    G = 2
    for k in range(G + 1):
        np.testing.assert_allclose(pos_law[k] / reach[k], P[k], atol=1e-12)
        np.testing.assert_allclose(reach[k], np.prod(alpha[:k]), atol=1e-12)
    tau = 1 + sum(np.prod(alpha[: j + 1]) for j in range(G))
    assert abs(e_len - tau) < 1e-12
    assert abs(tau - (1 + 0.8 + 0.8 * 0.7)) < 1e-12


def test_enumeration_truncated_verify_len():
    """Verify length 1 of G=2: position 1 must be the bonus from row 1 (law p_1)."""
    grid = (np.arange(10) + 0.5) / 10
    us = np.array(list(itertools.product(grid, repeat=3)))
    law = np.zeros((2, 3))
    reach1 = 0.0
    for xs in itertools.product(range(3), repeat=2):
        w = Q_ROWS[0][xs[0]] * Q_ROWS[1][xs[1]]
        out = _batch(P_ROWS, Q_ROWS, np.tile(xs, (len(us), 1)), us, verify_len=np.ones(len(us), int))
        a, tok = out["accepted"], out["tokens"]
        assert a.max() <= 1
        assert np.all(tok[:, 2] == -1)
        law[0] += w * np.bincount(tok[:, 0], minlength=3) / len(us)
        sel = a >= 1
        reach1 += w * sel.mean()
        law[1] += w * np.bincount(tok[sel, 1], minlength=3) / len(us)
    np.testing.assert_allclose(law[0], P_ROWS[0], atol=1e-12)
    np.testing.assert_allclose(law[1] / reach1, P_ROWS[1], atol=1e-12)
    assert abs(reach1 - 0.8) < 1e-12


# --------------------------------------------------------------------------
# Monte Carlo on random distributions (losslessness at scale).
# --------------------------------------------------------------------------

def _mc(seed, V, G, N, verify_len=None, T=1.0):
    g = np.random.default_rng(seed)
    z = g.normal(0, 1.5, size=(G + 1, V))
    draft = z[:G] + g.normal(0, 0.7, size=(G, V))
    q = np.exp(draft - draft.max(1, keepdims=True))
    q /= q.sum(1, keepdims=True)
    p = np.exp((z - z.max(1, keepdims=True)) / T)
    p /= p.sum(1, keepdims=True)
    xs = np.stack([g.choice(V, size=N, p=q[k]) for k in range(G)], axis=1)
    us = g.random((N, G + 1))
    zz = np.broadcast_to(z, (N, G + 1, V))
    qq = np.broadcast_to(q, (N, G, V))
    out = oracle.verify(zz, qq, xs, us, T, verify_len)
    return p, q, out


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_monte_carlo_law_and_acceptance(T):
    V, G, N = 12, 3, 200_000
    p, q, out = _mc(7, V, G, N, T=T)
    a, tok = out["accepted"], out["tokens"]
    alpha = np.minimum(p[:G], q).sum(1)
    for k in range(G + 1):
        sel = a >= k
        n_k = sel.sum()
        counts = np.bincount(tok[sel, k], minlength=V)
        expected = n_k * p[k]
        chi2 = ((counts - expected) ** 2 / expected).sum()
        # chi-square with V-1 = 11 dof: P(chi2 > 35) ~ 2.5e-4
        assert chi2 < 35.0, (k, chi2)
        if k < G:
            rate = (a[sel] > k).mean()
            sd = np.sqrt(alpha[k] * (1 - alpha[k]) / n_k)
            assert abs(rate - alpha[k]) < 4.5 * sd, (k, rate, alpha[k])


def test_monte_carlo_truncated_is_lossless():
    V, G, N = 10, 4, 150_000
    g = np.random.default_rng(3)
    n = g.integers(0, G + 1, size=N)          # depends on nothing the target sees
    p, q, out = _mc(11, V, G, N, verify_len=n)
    a, tok = out["accepted"], out["tokens"]
    assert np.all(a <= n)
    for k in range(G + 1):
        sel = (a >= k) & (k <= n)
        counts = np.bincount(tok[sel, k], minlength=V)
        expected = sel.sum() * p[k]
        chi2 = ((counts - expected) ** 2 / expected).sum()
        assert chi2 < 33.0, (k, chi2)     # 9 dof


# --------------------------------------------------------------------------
# Special cases that reduce to a textbook result or a library routine.
# --------------------------------------------------------------------------

def test_q_equal_p_accepts_everything():
    """UraionSpec, section "Component Verification": p_t = p_d accepts all gamma drafts."""
    V, G, N = 8, 5, 2000
    g = np.random.default_rng(0)
    z = np.zeros((N, G + 1, V))                      # uniform rows: p = 1/8 exactly
    q = np.full((N, G, V), 1.0 / 8.0)
    xs = g.integers(0, V, size=(N, G))
    us = g.random((N, G + 1))
    out = oracle.verify(z, q, xs, us, 1.0)
    assert np.all(out["accepted"] == G)
    assert np.all(out["tokens"][:, :G] == xs)


def test_gamma_zero_is_plain_inverse_cdf_sampling():
    V, N = 50, 500
    g = np.random.default_rng(1)
    z = g.normal(0, 2, size=(N, 1, V))
    us = g.random((N, 1))
    out = oracle.verify(z, None, np.zeros((N, 0), int), us, 0.8)
    assert np.all(out["accepted"] == 0)
    for b in range(N):
        p = np.exp((z[b, 0] - z[b, 0].max()) / 0.8)
        c = np.cumsum(p)
        assert out["tokens"][b, 0] == np.searchsorted(c, us[b, 0] * c[-1], side="right")


def test_lse_matches_library_logsumexp():
    g = np.random.default_rng(2)
    z = g.normal(0, 3, size=(3, 4, 777))
    q = np.full((3, 3, 777), 1.0 / 777)
    out = oracle.verify(z, q, np.zeros((3, 3), int), g.random((3, 4)), 0.7)
    ref = logsumexp(z / 0.7, axis=2)
    used = ~np.isnan(out["lse"])
    assert used[:, 0].all()
    np.testing.assert_allclose(out["lse"][used], ref[used], rtol=1e-13)
    # p_draft is the softmax value at the draft token
    np.testing.assert_allclose(out["p_draft"][:, 0], np.exp(z[:, 0, 0] / 0.7 - ref[:, 0]), rtol=1e-12)


def test_onehot_draft_with_zero_target_mass_rejects_at_zero():
    V = 6
    p0 = np.array([0.1, 0.2, 0.0, 0.3, 0.25, 0.15])
    q0 = np.eye(V)[2]
    for u1 in (0.0, 0.05, 0.31, 0.61, 0.99):
        out = _one_request([p0, p0], [q0], [2], [0.0, u1])
        assert out["accepted"][0] == 0
        c = np.cumsum(p0)
        assert out["tokens"][0, 0] == np.searchsorted(c, u1 * c[-1], side="right")


def test_zero_mass_tokens_never_drawn():
    p = np.array([0.0, 0.5, 0.0, 0.5, 0.0])
    for u in np.linspace(0, 0.999999, 101):
        out = _one_request([p], np.zeros((0, 5)), np.zeros(0, int), [u])
        assert out["tokens"][0, 0] in (1, 3)
    # u at the exact breakpoint goes to the upper token (strict "exceeds")
    assert _one_request([p], np.zeros((0, 5)), np.zeros(0, int), [0.5])["tokens"][0, 0] == 3


def test_uniform_zero_accepts_positive_mass():
    out = _one_request([[0.01, 0.99], [0.5, 0.5]], [[0.99, 0.01]], [0], [0.0, 0.0])
    assert out["accepted"][0] == 1


def test_greedy_is_the_low_temperature_limit():
    """T=0 path equals the stochastic path at T -> 0 with one-hot drafts."""
    g = np.random.default_rng(5)
    B, G, V = 40, 4, 30
    z = np.round(g.normal(0, 4, size=(B, G + 1, V)))      # integer logits: gaps >= 1 or ties
    # break ties so the low-T softmax is one-hot (greedy tie rule is tested below)
    z = z + np.arange(V)[None, None, :] * -1e-3
    a = z.argmax(2)
    xs = np.where(g.random((B, G)) < 0.7, a[:, :G], g.integers(0, V, size=(B, G)))
    q = np.eye(V)[xs]
    us = g.random((B, G + 1)) * 0.999
    greedy = oracle.verify(z, None, xs, None, 0.0)
    cold = oracle.verify(z, q, xs, us, 1e-4)
    np.testing.assert_array_equal(greedy["accepted"], cold["accepted"])
    np.testing.assert_array_equal(greedy["tokens"], cold["tokens"])


def test_greedy_ties_take_lowest_index():
    V = 20
    z = np.zeros((1, 2, V))
    z[0, 0, [5, 9, 13]] = 3.0
    z[0, 1, [2, 17]] = 1.0
    z[0, 1, 0] = -0.0
    out = oracle.verify(z, None, np.array([[9]]), None, 0.0)
    assert out["accepted"][0] == 0 and out["tokens"][0].tolist() == [5, -1]
    out = oracle.verify(z, None, np.array([[5]]), None, 0.0)
    assert out["accepted"][0] == 1 and out["tokens"][0].tolist() == [5, 2]
    # brute-force argmax by a Python scan
    g = np.random.default_rng(9)
    zz = np.round(g.normal(0, 1, size=(30, 3, 40)) * 2) / 2       # many ties
    out = oracle.verify(zz, None, np.zeros((30, 2), int), None, 0.0)
    for b in range(30):
        best = 0
        for v in range(40):
            if zz[b, 0, v] > zz[b, 0, best]:
                best = v
        assert out["argmax"][b, 0] == best


def test_data_errors():
    V = 5
    z = np.zeros((4, 3, V))
    q = np.full((4, 2, V), 0.2)
    xs = np.array([[0, 1], [0, 7], [1, 1], [2, 2]])
    z[2, 1, 3] = np.nan                                  # used row with NaN
    z[3, 2, :] = np.nan                                  # row beyond verify_len=1: unused
    vl = np.array([2, 2, 2, 1])
    out = oracle.verify(z, q, xs, np.full((4, 3), 0.5), 1.0, vl)
    assert out["accepted"].tolist() == [2, -1, -1, 1]
    assert out["tokens"][1].tolist() == [-1, -1, -1]
    assert out["tokens"][2].tolist() == [-1, -1, -1]
    bad_len = oracle.verify(z[:1], q[:1], xs[:1], np.full((1, 3), 0.5), 1.0, [3])
    assert bad_len["accepted"][0] == -1
    allninf = np.full((1, 2, V), -np.inf)
    assert oracle.verify(allninf, q[:1, :1], xs[:1, :1], np.full((1, 2), 0.5), 1.0)["accepted"][0] == -1
    pinf = np.zeros((1, 2, V)); pinf[0, 0, 1] = np.inf
    assert oracle.verify(pinf, None, xs[:1, :1], None, 0.0)["accepted"][0] == -1


def test_bf16_decode_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x4049, 0x0001], np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[2] == 0.0
    assert np.signbit(vals[3]) and vals[4] == np.inf and vals[5] == -np.inf
    assert vals[6] == 3.140625
    assert vals[7] == 2.0 ** -133


# --------------------------------------------------------------------------
# Scheduler: AngelSpec section 4.2 Eq. 19-21 and UraionSpec Algorithm 1.
# --------------------------------------------------------------------------

def test_schedule_hand_worked_case():
    # s = [[0.9, 0.45], [0.8, 0.08]]; cost = 1 + 0.2 T.
    # T=2 tau=2 Theta=2/1.4; +0.9 -> 2.9/1.6; +0.8 -> 3.7/1.8; +0.45 -> 4.15/2.0;
    # +0.08 -> 4.23/2.2 < 4.15/2.0: stop.  len = [2, 1], T = 5, tau = 4.15.
    c = np.array([[0.9, 0.5], [0.8, 0.1]])
    cost = 1 + 0.2 * np.arange(10)
    lens, T, tau = oracle.schedule(c, cost, 9)
    assert lens.tolist() == [2, 1] and T == 5 and abs(tau - 4.15) < 1e-12
    # budget cap at 4 stops after two extensions
    lens, T, tau = oracle.schedule(c, cost, 4)
    assert lens.tolist() == [1, 1] and T == 4 and abs(tau - 3.7) < 1e-12


def test_schedule_survival_is_cumprod():
    c = np.array([[0.5, 0.5, 0.2], [1.0, 0.9, 0.0]])
    np.testing.assert_array_equal(oracle.survival(c), [[0.5, 0.25, 0.05], [1.0, 0.9, 0.0]])


def test_schedule_noncontiguous_candidate_is_skipped():
    # c > 1 makes survival rise: (0,1) sorts first but len_0 = 0 != 1 -> skipped;
    # (0,0) is then taken; (0,1) is never revisited.
    c = np.array([[0.5, 1.5]])
    lens, T, tau = oracle.schedule(c, np.ones(10), 9)
    assert lens.tolist() == [1] and T == 2 and tau == 1.5


@pytest.mark.parametrize("seed", range(40))
def test_schedule_matches_brute_force_on_linear_cost(seed):
    g = np.random.default_rng(seed)
    B, G = 3, 4
    c = 1 / (1 + np.exp(-(g.normal(1.0, 1.5, size=(B, G)))))
    a, b = 1.0, float(g.choice([0.005, 0.02, 0.1, 0.3]))
    budget = int(g.integers(B, B * (G + 1) + 2))
    cost = a + b * np.arange(B * (G + 1) + 3)
    lens, T, tau = oracle.schedule(c, cost, budget)
    best_val, _ = oracle.brute_force(c, cost, budget)
    val, T2, tau2 = oracle.schedule_value(c, cost, lens)
    assert T2 == T == B + lens.sum() and T <= budget
    assert abs(tau2 - tau) < 1e-12
    assert abs(val - best_val) <= 1e-12 * best_val
    # kept set is a top set of survivals (contiguous prefixes, Eq. 20-21 text)
    s = oracle.survival(c)
    kept = np.array([[k < lens[i] for k in range(G)] for i in range(B)])
    if kept.any() and (~kept).any():
        assert s[kept].min() >= s[~kept].max()


def test_schedule_extremes():
    g = np.random.default_rng(4)
    B, G = 6, 5
    c = g.uniform(0.05, 0.95, size=(B, G))
    # very expensive verification: nothing beyond the anchors
    lens, T, tau = oracle.schedule(c, 1 + 1e6 * np.arange(64), 63)
    assert lens.tolist() == [0] * B and T == B and tau == B
    # free verification with room for everything: full depth
    lens, T, tau = oracle.schedule(c, np.ones(64), 63)
    assert lens.tolist() == [G] * B and T == B * (G + 1)
    # zero confidence: no candidate survives epsilon = 0
    lens, T, _ = oracle.schedule(np.zeros((B, G)), np.ones(64), 63)
    assert lens.tolist() == [0] * B and T == B


def test_schedule_exact_tie_does_not_extend():
    """Algorithm 1 keeps an extension only when Theta strictly improves."""
    # Theta0 = 1/1 = 1; Theta1 = (1 + 0.5)/1.5 = 1 exactly: a tie -> stop.
    lens, T, tau = oracle.schedule(np.array([[0.5]]), np.array([9.0, 1.0, 1.5, 2.0]), 3)
    assert lens.tolist() == [0] and T == 1 and tau == 1.0
    # a hair cheaper and it extends
    lens, T, tau = oracle.schedule(np.array([[0.5]]), np.array([9.0, 1.0, 1.4999, 2.0]), 3)
    assert lens.tolist() == [1] and T == 2
