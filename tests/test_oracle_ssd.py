"""Pins for the oracle's SSD/Saguaro extensions and the lenient rule
(oracle/ssd.py).

* Speculative Speculative Decoding, Appendix A.3, Theorem 19: Saguaro sampling
  with C = 47/147 turns p_d = (.49, .49, .01, .01) into (.47, .47, .03, .03);
  both have acceptance 0.98 against p_t = (.48, .48, .02, .02), and with F = 2
  the hit rate given a rejection is 50% for p_d and 100% for the biased draft.
* Theorem 15: the hit rate does not increase with C (checked on random rows,
  with the theorem's own definition of the hit rate).
* Exactness: verification with the Saguaro draft distribution as q outputs p_t
  (exact enumeration of the uniform grid, the oracle as a black box).
* Lenience [L5 sec. 2.8]: l = 1 is the exact rule; for l < 1 no output
  probability exceeds p(x)/l, and acceptance does not drop.
* Theorem 12: the geometric fan-out satisfies the budget and the Lagrange
  conditions of Appendix A.2, and matches a numerical optimum (scipy).
"""
import json
import os

import numpy as np
import pytest
from scipy.optimize import minimize
from scipy.special import softmax

from oracle import ssd
from oracle.sampling import verify_sequence
from oracle.topf import rank_order
from uniform_grid import GRID, bucket_counts, count_accepting

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL_GRID = 3 * 2.0 ** -24


def theorem19():
    with open(os.path.join(GOLDEN, "ssd_theorem19.json")) as f:
        return json.load(f)


def test_theorem19_saguaro_distribution():
    g = theorem19()
    z = np.log(np.array(g["p_draft"]))
    q = ssd.saguaro_probs(z, 1.0, g["F"], 47.0 / 147.0)
    np.testing.assert_allclose(q, g["p_draft_saguaro"], atol=1e-12)
    # a temperature rescales the logits, not the construction
    q2 = ssd.saguaro_probs(2.0 * z, 2.0, g["F"], 47.0 / 147.0)
    np.testing.assert_allclose(q2, g["p_draft_saguaro"], atol=1e-12)


def test_theorem19_acceptance_and_hit_rates():
    g = theorem19()
    pt = np.array(g["p_target"])
    z = np.log(np.array(g["p_draft"]))
    pd = softmax(z)
    q = ssd.saguaro_probs(z, 1.0, g["F"], 47.0 / 147.0)
    assert np.minimum(pt, pd).sum() == pytest.approx(g["printed"]["acceptance_rate_draft"], abs=1e-12)
    assert np.minimum(pt, q).sum() == pytest.approx(g["printed"]["acceptance_rate_draft_saguaro"], abs=1e-12)
    assert ssd.hit_given_rejection(pt, pd, z, g["F"]) == pytest.approx(g["printed"]["hit_rate_draft"], abs=1e-12)
    assert ssd.hit_given_rejection(pt, q, z, g["F"]) == pytest.approx(g["printed"]["hit_rate_draft_saguaro"], abs=1e-12)


def test_saguaro_special_cases():
    rng = np.random.default_rng(5)
    z = rng.normal(0, 2, 30)
    T = 0.8
    np.testing.assert_allclose(ssd.saguaro_probs(z, T, 5, 1.0), softmax(z / T), atol=1e-15)   # C = 1
    np.testing.assert_allclose(ssd.saguaro_probs(z, T, 0, 0.3), softmax(z / T), atol=1e-15)   # F = 0
    q = ssd.saguaro_probs(z, T, 4, 0.0)                                                         # C = 0
    top = rank_order(z)[:4]
    assert np.all(q[top] == 0.0)
    rest = np.setdiff1d(np.arange(30), top)
    np.testing.assert_allclose(q[rest], softmax(z[rest] / T), atol=1e-15)
    # ties at the F-th place: the lower id is inside top_F
    zt = np.array([3.0, 1.0, 2.0, 2.0, 0.5])
    qt = ssd.saguaro_probs(zt, 1.0, 2, 0.5)
    w = np.exp(zt - 3.0)
    w[[0, 2]] *= 0.5
    np.testing.assert_allclose(qt, w / w.sum(), atol=1e-15)


def theorem15_hit_rate(pt, q, S):
    """The hit rate as Theorem 15's proof defines it: the residual's mass on
    the cache set S over its total mass."""
    r = np.maximum(pt - q, 0.0)
    return r[S].sum() / r.sum() if r.sum() > 0 else 1.0


@pytest.mark.parametrize("seed", range(20))
def test_theorem15_hit_rate_monotone_in_C(seed):
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(4, 12))
    F = int(rng.integers(1, V))
    zt = rng.normal(0, 2, V)
    zd = zt + rng.normal(0, 1, V)
    pt = softmax(zt)
    S = rank_order(zd)[:F]
    Cs = np.linspace(0.0, 1.0, 41)
    hits = [theorem15_hit_rate(pt, ssd.saguaro_probs(zd, 1.0, F, C), S) for C in Cs]
    assert all(hits[i + 1] <= hits[i] + 1e-12 for i in range(len(hits) - 1)), hits


def output_distribution(pt_logits, q, T, lenience=1.0):
    """Exact distribution of the first emitted token at one position when the
    drafted token is drawn from q and the oracle takes every decision (uniform
    grid enumeration; the oracle is a black box)."""
    V = len(q)
    target = np.stack([pt_logits, pt_logits])
    draft = np.zeros((1, V))
    out = np.zeros(V)
    for x in range(V):
        if q[x] == 0:
            continue
        run = lambda u, v, x=x: verify_sequence(target, draft, [x], T, [u], v, q_rows=[q], lenience=lenience)
        a = count_accepting(lambda u: run(u, 0.5).k == 1) / GRID
        out[x] += q[x] * a
        if a < 1.0:
            counts = bucket_counts(lambda v: run(1.0, v).bonus, V)
            out += q[x] * (1.0 - a) * np.array(counts, np.float64) / GRID
    return out


@pytest.mark.parametrize("seed", range(6))
def test_verification_with_saguaro_draft_is_exact(seed):
    rng = np.random.default_rng(200 + seed)
    V = 7
    T = float(rng.choice([0.7, 1.0, 1.5]))
    zt = rng.normal(0, 2, V)
    zd = zt + rng.normal(0, 1, V)
    q = ssd.saguaro_probs(zd, T, int(rng.integers(1, 4)), float(rng.choice([0.1, 47 / 147, 0.6])))
    out = output_distribution(zt, q, T)
    np.testing.assert_allclose(out, softmax(zt / T), atol=V * TOL_GRID)


@pytest.mark.parametrize("seed", range(6))
def test_lenience_bound_and_limit(seed):
    rng = np.random.default_rng(300 + seed)
    V = 6
    zt = rng.normal(0, 2, V)
    zd = zt + rng.normal(0, 1.5, V)
    q = softmax(zd)
    pt = softmax(zt)
    exact = output_distribution(zt, q, 1.0, lenience=1.0)
    np.testing.assert_allclose(exact, pt, atol=V * TOL_GRID)
    for lenience in (0.8, 0.5, 0.1):
        out = output_distribution(zt, q, 1.0, lenience=lenience)
        assert out.sum() == pytest.approx(1.0, abs=V * TOL_GRID)
        assert np.all(out <= pt / lenience + V * TOL_GRID)
        # acceptance can only grow
        acc_l = sum(q[x] * count_accepting(lambda u, x=x: verify_sequence(
            np.stack([zt, zt]), np.zeros((1, V)), [x], 1.0, [u], 0.5, q_rows=[q], lenience=lenience).k == 1)
            for x in range(V)) / GRID
        assert acc_l >= np.minimum(pt, q).sum() - V * TOL_GRID


@pytest.mark.parametrize("K,a,r,budget", [(8, 0.7, 1.0, 64), (4, 0.5, 0.5, 20), (6, 0.9, 2.0, 100), (1, 0.3, 1.0, 5)])
def test_geometric_fanout_theorem12(K, a, r, budget):
    F = ssd.geometric_fanout(K, a, r, budget)
    assert F.sum() == pytest.approx(budget, rel=1e-12)
    # Appendix A.2: with dp/dF = r F^(-r-1), every F_k has the same marginal
    # weighted gain: a^k (1-a) r F_k^(-r-1) for k < K and a^K r F_K^(-r-1).
    gains = [a ** k * (1 - a) * r * F[k] ** (-r - 1) for k in range(K)] + [a ** K * r * F[K] ** (-r - 1)]
    np.testing.assert_allclose(gains, gains[0], rtol=1e-10)
    # A numerical optimum of the same objective under the budget agrees.
    weights = np.array([a ** k * (1 - a) for k in range(K)] + [a ** K])
    obj = lambda x: -np.sum(weights * (1 - np.maximum(x, 1e-9) ** (-r)))
    cons = {"type": "eq", "fun": lambda x: x.sum() - budget}
    res = minimize(obj, np.full(K + 1, budget / (K + 1)), constraints=[cons], bounds=[(1e-6, budget)] * (K + 1),
                   method="SLSQP", options={"ftol": 1e-14, "maxiter": 1000})
    np.testing.assert_allclose(res.x, F, rtol=2e-3)


def test_integer_fanout_rounding():
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(1, 12))
        budget = int(rng.integers(n, 200))
        Fr = ssd.geometric_fanout(n - 1, float(rng.uniform(0.1, 0.95)), float(rng.uniform(0.3, 3)), budget)
        Fi = ssd.integer_fanout(Fr, budget)
        assert Fi.sum() == budget
        assert np.all(np.abs(Fi - Fr) < 1.0)
    np.testing.assert_array_equal(ssd.integer_fanout([1.5, 1.5, 1.0], 4), [2, 1, 1])   # lower k first


def test_cache_candidates_and_hit():
    rng = np.random.default_rng(11)
    V, gamma = 9, 3
    zt = rng.normal(0, 1, (gamma + 1, V))
    zd = zt + rng.normal(0, 1, (gamma + 1, V))
    tokens = [int(rng.integers(V)) for _ in range(gamma)]
    fan = [2, 3, 0, 4]
    cands = ssd.cache_candidates(zd, tokens, fan)
    assert cands[2] == []   # F_k = 0: the cache does not cover position 2
    for k in range(gamma + 1):
        order = [int(j) for j in rank_order(zd[k]) if k == gamma or int(j) != tokens[k]]
        assert cands[k] == order[:fan[k]]
    # With F_k = V - 1 every bonus drawn after a rejection at k < gamma is
    # cached (the rejected token is the only one left out, and a rejected
    # token has zero residual mass).
    full = [V - 1] * (gamma + 1)
    for s in range(40):
        u = list(rng.uniform(0, 1, gamma))
        res, c, hit = ssd.verify_cached(zt, zd, tokens, 1.0, u, float(rng.uniform(0, 1)), full)
        if res.k < gamma:
            assert hit
        assert hit == (res.bonus in c[res.k])
