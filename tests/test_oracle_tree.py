"""Pins of the greedy tree-verification oracle.

CPU only.  Source: "breaking down dspark and its lineage", section "Tree
attention": each node is scored in the context of its own path, and the target
decides which candidate path survives.  A walk that follows a non-matching
child, stops early, takes the wrong argmax tie or mis-reads the parent array
fails at least one of these.
"""

import itertools

import numpy as np
import pytest

import oracle
from oracle import tree as TR


def _logits_with_argmax(g, B, M, V, amax):
    z = g.normal(size=(B, M, V))
    for b in range(B):
        for i in range(M):
            z[b, i, amax[b, i]] = z[b, i].max() + 1.0
    return z


def test_hand_worked_tree():
    # root -> {1: tok 1, 2: tok 2}; 2 -> {3: tok 3}.  argmax: root 2, node 2 -> 3, node 3 -> 0.
    V, M = 4, 4
    amax = np.array([[2, 1, 3, 0]])
    z = _logits_with_argmax(np.random.default_rng(0), 1, M, V, amax)
    out = TR.tree_verify_greedy(z, [[-1, 0, 0, 2]], [[0, 1, 2, 3]])
    assert out["accepted"].tolist() == [2]
    assert out["tokens"].tolist() == [[2, 3, 0, -1]]
    assert out["path"].tolist() == [[2, 3, -1, -1]]


@pytest.mark.parametrize("seed", range(8))
def test_chain_is_greedy_verification(seed):
    """A tree that is one chain is the greedy verification of that block."""
    g = np.random.default_rng(seed)
    B, G, V = 6, 5, 9
    z = g.normal(size=(B, G + 1, V))
    a = z.argmax(axis=2)
    x = np.where(g.random((B, G)) < 0.7, a[:, :G], g.integers(0, V, (B, G)))   # mostly matching drafts
    par = np.tile(TR.chain(G), (B, 1))
    tok = np.concatenate([np.zeros((B, 1), np.int64), x], axis=1)
    got = TR.tree_verify_greedy(z, par, tok)
    ref = oracle.verify_greedy(z, x)
    np.testing.assert_array_equal(got["accepted"], ref["accepted"])
    np.testing.assert_array_equal(got["tokens"], ref["tokens"])


def _consistent_paths(par, tok, amax, M):
    """Every root-to-node path whose each node carries the argmax of its parent."""
    paths = []
    for i in range(1, M):
        p, n = [], i
        while n != 0:
            p.append(n)
            n = par[n]
        p = p[::-1]
        prev, ok = 0, True
        for n in p:
            ok &= tok[n] == amax[prev]
            prev = n
        if ok:
            paths.append(p)
    return paths


@pytest.mark.parametrize("seed", range(20))
def test_walk_is_the_longest_consistent_path(seed):
    g = np.random.default_rng(100 + seed)
    B, M, V = 4, int(g.integers(2, 12)), 4
    # logits peaked on few tokens, so long consistent paths occur
    z = g.normal(size=(B, M, V))
    amax = z.argmax(axis=2)
    par = np.array([[-1] + [int(g.integers(0, i)) for i in range(1, M)] for _ in range(B)])
    # siblings carry distinct tokens (a candidate tree: each child a different continuation)
    tok = np.zeros((B, M), np.int64)
    for b in range(B):
        for i in range(1, M):
            used = {int(tok[b, j]) for j in range(1, i) if par[b, j] == par[b, i]}
            free = [v for v in range(V) if v not in used]
            if not free:
                par[b, i] = i - 1
                used = set()
                free = list(range(V))
            tok[b, i] = int(g.choice(free))
    out = TR.tree_verify_greedy(z, par, tok)
    for b in range(B):
        paths = _consistent_paths(par[b], tok[b], amax[b], M)
        n = int(out["accepted"][b])
        assert n == max([len(p) for p in paths], default=0)
        path = out["path"][b, :n].tolist()
        assert path in paths or n == 0
        # emitted = argmax chain along the path, then the bonus
        nodes = [0] + path
        assert out["tokens"][b, : n + 1].tolist() == [int(amax[b, v]) for v in nodes]
        assert (out["tokens"][b, n + 1:] == -1).all()


def test_duplicate_children_take_the_lowest_node():
    V, M = 3, 4
    amax = np.array([[1, 2, 0, 0]])
    z = _logits_with_argmax(np.random.default_rng(1), 1, M, V, amax)
    out = TR.tree_verify_greedy(z, [[-1, 0, 0, 0]], [[0, 2, 1, 1]])    # nodes 2 and 3 both carry 1
    assert out["path"][0, 0] == 2 and out["accepted"][0] == 1


def test_data_errors_only_on_visited_rows():
    g = np.random.default_rng(2)
    V, M = 5, 4
    amax = np.array([[1, 2, 3, 4]] * 4)
    z = _logits_with_argmax(g, 4, M, V, amax)
    par = np.array([[-1, 0, 0, 1]] * 4)
    tok = np.array([[0, 1, 4, 2]] * 4)                  # walk: root -> 1 -> 3
    z[0, 2, 0] = np.nan                                 # row 2 is never visited: fine
    z[1, 3, :] = -np.inf                                # row 3 is visited: error
    par_bad = par.copy(); par_bad[2, 2] = 2             # parent not before the node
    tok_bad = tok.copy(); tok_bad[3, 2] = V             # token out of range
    out = TR.tree_verify_greedy(z, np.stack([par[0], par[1], par_bad[2], par[3]]),
                                np.stack([tok[0], tok[1], tok[2], tok_bad[3]]))
    assert out["accepted"].tolist() == [2, -1, -1, -1]
    assert (out["tokens"][1:] == -1).all()
