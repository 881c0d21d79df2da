"""Pins for the oracle's token-tree verification (VerifyGreedy, MSS).

Lecture 5: Speculative Decoding and SpecInfer, sec. 6.4:
* MSS with children drawn i.i.d. from q keeps the target distribution
  (checked by exact enumeration of child tuples and of the uniform grid);
* MSS accepts at least as often as naive sampling (NS: draw from p and look
  for the token among the children);
* deterministic top-k children with the ratio rule are biased (the page
  reports TV 0.24-0.34), so the same check must fail for them;
* a tree whose nodes have one child each is chain verification.
"""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

from oracle import tree as otree
from oracle.sampling import verify_sequence
from oracle.tree import mss_node, verify_tree, verify_tree_batch
from uniform_grid import GRID, bucket_counts, count_accepting

TOL = 1e-6


def mss_first_token(p, q, child_tuples):
    """Exact distribution of the first emitted token and the acceptance
    probability, for child tuples given with their weights; every decision by
    the oracle's mss_node, enumerated over the uniform grid."""
    V = len(p)
    out = np.zeros(V)
    acc_total = 0.0
    for tup, weight in child_tuples:
        m = len(tup)
        prefix = 1.0
        for j in range(m):
            def accepted(u, j=j):
                us = [1.0] * m
                us[j] = u
                return mss_node(p, q, list(tup), us, 0.5)[0] == j
            a = count_accepting(accepted) / GRID
            out[tup[j]] += weight * prefix * a
            acc_total += weight * prefix * a
            prefix *= 1.0 - a
            if prefix == 0.0:
                break
        if prefix > 0.0:
            counts = bucket_counts(lambda v: mss_node(p, q, list(tup), [1.0] * m, v)[1], V)
            out += weight * prefix * np.array(counts) / GRID
    return out, acc_total


def iid_tuples(q, m):
    V = len(q)
    for tup in itertools.product(range(V), repeat=m):
        w = float(np.prod([q[t] for t in tup]))
        if w > 0:
            yield tup, w


@pytest.mark.parametrize("m,trials", [(1, 60), (2, 40), (3, 25)])
def test_mss_keeps_target_distribution(m, trials):
    rng = np.random.default_rng(100 + m)
    for _ in range(trials):
        V = 5
        p = softmax(rng.normal(0, 1.5, V))
        q = softmax(rng.normal(0, 1.5, V))
        out, acc = mss_first_token(p, q, list(iid_tuples(q, m)))
        assert np.max(np.abs(out - p)) < TOL
        # Naive sampling accepts with E[p(set of children)].
        ns = sum(w * p[list(set(t))].sum() for t, w in iid_tuples(q, m))
        assert acc >= ns - TOL


def test_deterministic_topk_children_are_biased():
    rng = np.random.default_rng(7)
    tvs = []
    for _ in range(10):
        V = 5
        p = softmax(rng.normal(0, 1.5, V))
        q = softmax(rng.normal(0, 1.5, V))
        top = tuple(int(j) for j in np.argsort(-q, kind="stable")[:2])
        out, _ = mss_first_token(p, q, [(top, 1.0)])
        tvs.append(0.5 * np.abs(out - p).sum())
    assert np.mean(tvs) > 0.05, tvs


def test_planted_missing_residual_update_is_caught(monkeypatch):
    # Dropping the r <- norm(max(0, r - q)) step after a rejection (testing
    # every child against the original p) must break the exactness check.
    monkeypatch.setattr(otree, "mss_residual", lambda r, q: r)
    rng = np.random.default_rng(41)
    worst = 0.0
    for _ in range(5):
        p = softmax(rng.normal(0, 1.5, 5))
        q = softmax(rng.normal(0, 1.5, 5))
        out, _ = mss_first_token(p, q, list(iid_tuples(q, 2)))
        worst = max(worst, np.max(np.abs(out - p)))
    assert worst > 0.01, worst


def test_chain_shaped_tree_equals_chain_verification():
    rng = np.random.default_rng(9)
    checked = 0
    for trial in range(200):
        V, gamma = int(rng.integers(2, 12)), int(rng.integers(1, 6))
        T = 0.0 if trial % 4 == 0 else float(rng.choice([0.7, 1.0]))
        target = rng.normal(0, 2, (gamma + 1, V))
        draft = np.vstack([target[:gamma] + rng.normal(0, 1, (gamma, V)),
                           rng.normal(0, 1, (1, V))])
        x = [int(rng.integers(V)) for _ in range(gamma)]
        u = list(rng.random(gamma) * 0.999 + 1e-4)
        v = float(rng.random() * 0.999 + 1e-4)
        chain = verify_sequence(target, draft, x, T, u, v)
        parent = [-1] + list(range(gamma))
        tokens = [0] + x
        tr = verify_tree(target, draft, parent, tokens, T, [0.0] + u, v)
        if chain.near_tie or tr.near_tie:
            continue
        assert tr.num_accepted == chain.k
        assert tr.path == list(range(1, chain.k + 1))
        assert tr.bonus == chain.bonus
        checked += 1
    assert checked > 180


def test_verify_greedy_walk():
    V = 6
    target = np.zeros((6, V))
    target[0, 3] = 5      # root argmax 3
    target[2, 1] = 5      # node 2 argmax 1
    target[4, 5] = 5      # node 4 (leaf) argmax 5
    parent = [-1, 0, 0, 0, 2, 2]
    tokens = [0, 2, 3, 3, 1, 1]   # nodes 2 and 3 both carry token 3; 4 and 5 carry 1
    r = verify_tree(target, None, parent, tokens, 0.0, [0.5] * 6, 0.5)
    assert r.path == [2, 4] and r.bonus == 5
    target[0, 3] = 0
    target[0, 0] = 5      # root argmax 0: no child matches
    r = verify_tree(target, None, parent, tokens, 0.0, [0.5] * 6, 0.5)
    assert r.path == [] and r.bonus == 0


def test_two_level_walk_monte_carlo():
    # Depth-2 tree with the same target row p1 at every depth-1 node: the first
    # emitted token follows p0, and after an accepted first token the next one
    # follows p1.
    rng = np.random.default_rng(31)
    V, B = 4, 12000
    l0, l1 = rng.normal(0, 1.2, V), rng.normal(0, 1.2, V)
    d0, d1 = l0 + rng.normal(0, 1, V), l1 + rng.normal(0, 1, V)
    q0, q1 = softmax(d0), softmax(d1)
    parent = [-1, 0, 0, 1, 1, 2]
    N = len(parent)
    target = np.stack([l0] + [l1] * (N - 1))
    draft = np.stack([d0, d1, d1, d1, d1, d1])
    P = np.tile(parent, (B, 1))
    toks = np.zeros((B, N), np.int64)
    for n in range(1, N):
        q = q0 if parent[n] == 0 else q1
        toks[:, n] = rng.choice(V, size=B, p=q)
    out = verify_tree_batch(np.broadcast_to(target, (B, N, V)),
                            np.broadcast_to(draft, (B, N, V)), P, toks,
                            np.ones(B), seed=5, offset=0)
    first = np.where(out["num_accepted"] > 0,
                     toks[np.arange(B), np.maximum(out["path"][:, 0], 0)],
                     out["bonus"])
    tv0 = 0.5 * np.abs(np.bincount(first, minlength=V) / B - softmax(l0)).sum()
    assert tv0 < 0.02, tv0
    sel = out["num_accepted"] >= 1
    second = np.where(out["num_accepted"][sel] >= 2,
                      toks[np.arange(B)[sel], np.maximum(out["path"][sel, 1], 0)],
                      out["bonus"][sel])
    tv1 = 0.5 * np.abs(np.bincount(second, minlength=V) / sel.sum() - softmax(l1)).sum()
    assert tv1 < 0.03, tv1


def test_mss_residual_keeps_r_when_mass_is_zero():
    r = np.array([0.2, 0.8])
    np.testing.assert_array_equal(otree.mss_residual(r, r.copy()), r)
    np.testing.assert_allclose(otree.mss_residual(r, np.array([0.5, 0.5])), [0, 1])
