"""Pins of the acceptance-diagnostics and draft-logits oracle.

CPU only.  Sources: "AngelSpec", section 2, Eq. 2 (the drafter's softmax),
Eq. 4 (TV) and Eq. 5 (alpha = sum min(p, q) = 1 - TV, the expected
acceptance); "breaking down dspark and its lineage", the worked example
(overlap 0.8); "UraionSpec", the confidence-head target c* = 1 - TV.  A wrong
min/max, a dropped 1/2, a softmax at the wrong temperature or a mask on the
wrong positions fails at least one of them.
"""

import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import acceptance as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_page_example_overlap_and_tv():
    with open(os.path.join(GOLDEN, "page_example.json")) as f:
        g = json.load(f)
    p, q = np.array(g["p_target"]), np.array(g["q_draft"])
    assert abs(A.overlap(p, q) - g["overlap_sum"]) < 1e-15
    assert abs(A.total_variation(p, q) - g["tv"]) < 1e-15
    # the same through acceptance() from logits ln p and draft probabilities q
    z = np.log(np.stack([p, p]))[None]                      # rows 0 and 1 (bonus row)
    alpha = A.acceptance(z, q[None, None], 1.0)
    assert alpha.shape == (1, 1) and abs(alpha[0, 0] - 0.8) < 1e-12


@pytest.mark.parametrize("seed", range(10))
def test_overlap_is_one_minus_tv(seed):
    g = np.random.default_rng(seed)
    V = int(g.integers(2, 300))
    p = g.dirichlet(np.full(V, 0.3))
    q = g.dirichlet(np.full(V, 0.3))
    assert abs(A.overlap(p, q) + A.total_variation(p, q) - 1.0) < 1e-12
    assert abs(A.overlap(p, p) - 1.0) < 1e-12
    assert 0.0 <= A.overlap(p, q) <= 1.0


def test_disjoint_supports_overlap_zero():
    p = np.array([0.5, 0.5, 0.0, 0.0])
    q = np.array([0.0, 0.0, 0.25, 0.75])
    assert A.overlap(p, q) == 0.0 and A.total_variation(p, q) == 1.0


@pytest.mark.parametrize("T", [1.0, 0.7, 2.5])
def test_draft_softmax_is_library_softmax(T):
    g = np.random.default_rng(3)
    d = g.normal(0, 3, size=(2, 3, 50))
    np.testing.assert_allclose(A.draft_probs_from_logits(d, T), softmax(d / T, axis=-1), rtol=1e-13, atol=0)


def test_overlap_is_the_acceptance_probability():
    """Eq. 5: integrating the verify rule's accept decision over x ~ q and u ~ U[0,1) gives alpha."""
    g = np.random.default_rng(5)
    V = 7
    p = g.dirichlet(np.ones(V))
    q = g.dirichlet(np.ones(V))
    M = 4000                                           # midpoint grid of u
    us = (np.arange(M) + 0.5) / M
    acc = 0.0
    z = np.log(np.stack([p, p]))
    for x in range(V):
        N = M
        zz = np.broadcast_to(z, (N, 2, V))
        qq = np.broadcast_to(q, (N, 1, V))
        u = np.stack([us, np.full(N, 0.5)], axis=1)
        out = oracle.verify(zz, qq, np.full((N, 1), x), u, 1.0)
        acc += q[x] * float((out["accepted"] == 1).mean())
    assert abs(acc - A.overlap(p, q)) < 2.0 / M


def test_acceptance_masks_untested_positions_and_bad_requests():
    g = np.random.default_rng(6)
    B, G, V = 4, 3, 20
    z = g.normal(size=(B, G + 1, V))
    q = softmax(g.normal(size=(B, G, V)), axis=-1)
    n = np.array([3, 1, 0, 2])
    z[3, 1, 5] = np.nan                                # request 3, row 1: only alpha[3, 1] is lost
    z[1, 2, :] = -np.inf                               # request 1 tests row 0 only: no effect
    alpha = A.acceptance(z, q, 1.0, verify_len=n)
    p = softmax(z, axis=-1)
    for b in range(B):
        for k in range(G):
            if k < n[b] and not (b == 3 and k == 1):
                assert abs(alpha[b, k] - np.minimum(p[b, k], q[b, k]).sum()) < 1e-12
            else:
                assert np.isnan(alpha[b, k])
    # an invalid verify length: the whole request
    alpha = A.acceptance(z, q, 1.0, verify_len=np.array([4, 1, -1, 2]))
    assert np.isnan(alpha[0]).all() and np.isnan(alpha[2]).all() and not np.isnan(alpha[1, 0])
    with pytest.raises(ValueError):
        A.acceptance(z, q, 0.0)


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_draft_logits_acceptance_and_verify_match_explicit_softmax(T):
    g = np.random.default_rng(7)
    B, G, V = 6, 4, 40
    z = g.normal(0, 2, size=(B, G + 1, V))
    d = z[:, :G] + g.normal(0, 0.8, size=(B, G, V))
    q = softmax(d / T, axis=-1)
    x = np.array([[g.choice(V, p=q[b, k]) for k in range(G)] for b in range(B)])
    u = g.uniform(size=(B, G + 1))
    n = np.array([4, 2, 0, 3, 4, 1])
    ref = oracle.verify(z, q, x, u, T, verify_len=n)
    got = A.verify_logits(z, d, x, u, T, verify_len=n)
    np.testing.assert_array_equal(got["accepted"], ref["accepted"])
    np.testing.assert_array_equal(got["tokens"], ref["tokens"])
    np.testing.assert_allclose(A.acceptance(z, d, T, n, draft_is_logits=True),
                               A.acceptance(z, q, T, n), rtol=1e-12, equal_nan=True)


def test_bad_draft_rows_are_data_errors():
    g = np.random.default_rng(8)
    B, G, V = 3, 3, 16
    z = g.normal(size=(B, G + 1, V))
    d = g.normal(size=(B, G, V))
    x = g.integers(0, V, size=(B, G))
    u = g.uniform(size=(B, G + 1))
    d[0, 1, 3] = np.nan                                # verified row: error
    d[1, 2, :] = -np.inf                               # row 2 of request 1, not verified at n = 2: fine
    d[2, 0, 7] = np.inf                                # max +inf: error
    n = np.array([3, 2, 3])
    out = A.verify_logits(z, d, x, u, 1.0, verify_len=n)
    assert out["accepted"][0] == -1 and out["accepted"][2] == -1 and out["accepted"][1] >= 0
    alpha = A.acceptance(z, d, 1.0, n, draft_is_logits=True)
    # per position: the bad draft rows' positions only
    assert np.isnan(alpha[0, 1]) and np.isnan(alpha[2, 0])
    assert not np.isnan(alpha[0, [0, 2]]).any() and not np.isnan(alpha[2, 1:]).any()
    assert not np.isnan(alpha[1, :2]).any() and np.isnan(alpha[1, 2])
    # greedy ignores the draft logits
    g0 = A.verify_logits(z, d, x, u, 0.0, verify_len=n)
    ref = oracle.verify_greedy(z, x, n)
    np.testing.assert_array_equal(g0["tokens"], ref["tokens"])
