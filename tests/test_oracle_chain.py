"""Pins for the oracle's chain verification (accept rule, residual, bonus).

Each test checks the oracle against something other than itself: numbers the
pages print, closed forms, exact enumeration of the uniform grid, library
routines for special cases. Reference distributions come from
scipy.special.softmax, not from the oracle.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

from oracle import sampling
from oracle.sampling import verify_batch, verify_sequence
from uniform_grid import GRID, bucket_counts, count_accepting

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL_GRID = 3 * 2.0 ** -24      # per-token error of grid enumeration


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def accept_fraction(pt_logits, pd_logits, x, T):
    """Exact probability (over the 2^24-point grid) that the oracle accepts the
    drafted token x at a single position."""
    target = np.stack([pt_logits, pt_logits])
    draft = np.stack([pd_logits])
    n = count_accepting(
        lambda u: verify_sequence(target, draft, [x], T, [u], 0.5).k == 1)
    return n / GRID


def bonus_after_reject(pt_logits, pd_logits, x, T):
    """Exact bonus distribution (over the v grid) when x is rejected (u = 1)."""
    target = np.stack([pt_logits, pt_logits])
    draft = np.stack([pd_logits])
    V = len(pt_logits)
    counts = bucket_counts(
        lambda v: verify_sequence(target, draft, [x], T, [1.0], v).bonus, V)
    return np.array(counts, dtype=np.float64) / GRID


def output_distribution(pt_logits, pd_logits, T):
    """Exact distribution of the first emitted token at one position, with the
    draft token x drawn from p_d (weights from scipy) and the oracle taking
    every decision."""
    pd = softmax(np.asarray(pd_logits, np.float64) / T)
    out = np.zeros(len(pd))
    for x in range(len(pd)):
        if pd[x] == 0:
            continue
        a = accept_fraction(pt_logits, pd_logits, x, T)
        out[x] += pd[x] * a
        if a < 1.0:
            out += pd[x] * (1.0 - a) * bonus_after_reject(pt_logits, pd_logits, x, T)
    return out


def test_exercise1_printed_numbers():
    g = load("lecture5_exercise1.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    lp, lq = np.log(p), np.log(q)
    pr = g["printed"]
    acc = [accept_fraction(lp, lq, x, 1.0) for x in range(3)]
    np.testing.assert_allclose(acc, pr["accept_probability_by_token"], atol=2 * 2.0 ** -24)
    beta = sum(q[x] * acc[x] for x in range(3))
    assert abs(beta - pr["acceptance_rate"]) < 2 * 2.0 ** -24
    # Rejecting token 1 (the only way besides token 2 to reject) resamples from
    # the residual, which puts all mass on token 0.
    for x in (1, 2):
        np.testing.assert_allclose(bonus_after_reject(lp, lq, x, 1.0),
                                   pr["residual"], atol=2.0 ** -24)
    np.testing.assert_allclose(output_distribution(lp, lq, 1.0), pr["output"],
                               atol=TOL_GRID)


def test_four_token_example_printed_numbers():
    g = load("lecture5_sec2_3_four_tokens.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    lp, lq = np.log(p), np.log(q)
    pr = g["printed"]
    B = g["tokens"].index("B")
    assert p[B] == pr["p_B"]
    assert int(np.argmax(q)) == g["tokens"].index(pr["draft_favourite"])
    acc = [accept_fraction(lp, lq, x, 1.0) for x in range(4)]
    assert abs(acc[B] - pr["accept_probability_B"]) < 2 * 2.0 ** -24
    beta = sum(q[x] * acc[x] for x in range(4))
    assert abs(beta - pr["acceptance_rate"]) < 4 * 2.0 ** -24
    # The residual mass the oracle reports after a rejection is 1 - beta, and
    # it is shared A : C = 0.20 : 0.05.
    target = np.stack([lp, lp])
    res = verify_sequence(target, np.stack([lq]), [B], 1.0, [1.0], 0.5)
    assert res.k == 0
    assert abs(res.bonus_mass - pr["reject_mass"]) < 1e-12
    bonus = bonus_after_reject(lp, lq, B, 1.0) * pr["reject_mass"]
    A, C = g["tokens"].index("A"), g["tokens"].index("C")
    assert abs(bonus[A] - pr["residual_mass_A"]) < 1e-6
    assert abs(bonus[C] - pr["residual_mass_C"]) < 1e-6
    assert bonus[B] == 0 and bonus[g["tokens"].index("D")] == 0
    np.testing.assert_allclose(output_distribution(lp, lq, 1.0), p, atol=TOL_GRID)


def test_output_equals_target_random_pairs():
    # The exactness identity min(p_d, p_t) + [p_t - p_d]_+ = p_t, checked
    # through the oracle's decisions on random pairs and temperatures.
    rng = np.random.default_rng(11)
    worst = 0.0
    for trial in range(60):
        V = int(rng.integers(2, 8))
        T = float(rng.choice([0.5, 1.0, 1.7]))
        lt = rng.normal(0, 2, V)
        ld = lt + rng.normal(0, 1.5, V)
        if trial % 10 == 0:
            ld[rng.integers(V)] = -np.inf      # a token the draft never proposes
        out = output_distribution(lt, ld, T)
        worst = max(worst, np.max(np.abs(out - softmax(lt / T))))
    assert worst < TOL_GRID


def test_tiny_v16_every_position_exact():
    from workloads import make_workload
    w = make_workload("tiny_v16")
    for i in range(w.gamma):
        out = output_distribution(w.target[0, i].astype(np.float64),
                                  w.draft[0, i].astype(np.float64), 1.0)
        np.testing.assert_allclose(out, softmax(w.target[0, i].astype(np.float64)),
                                   atol=TOL_GRID)


def test_all_accepted_bonus_comes_from_last_target_row():
    rng = np.random.default_rng(3)
    V, gamma = 6, 3
    target = rng.normal(0, 2, (gamma + 1, V))
    draft = target[:gamma].copy()          # identical rows: ratio 1, always accepted
    x = [0, 1, 2]
    counts = bucket_counts(
        lambda v: verify_sequence(target, draft, x, 1.0, [1.0] * gamma, v).bonus, V)
    np.testing.assert_allclose(np.array(counts) / GRID, softmax(target[gamma]),
                               atol=2 * 2.0 ** -24)
    res = verify_sequence(target, draft, x, 1.0, [1.0] * gamma, 0.3)
    assert res.k == gamma and res.tokens[:gamma] == x


def test_theorem1_acceptance_rate_and_residual_mass():
    # alpha = sum_x min(p_t, p_d) = 1 - 0.5 * ||p_t - p_d||_1 (Speculative
    # Speculative Decoding, sec. 2.1, Theorem 1); the residual mass after a
    # rejection is 1 - alpha.
    rng = np.random.default_rng(5)
    for _ in range(40):
        V = int(rng.integers(3, 9))
        lt, ld = rng.normal(0, 2, V), rng.normal(0, 2, V)
        pt, pd = softmax(lt), softmax(ld)
        alpha = 1.0 - 0.5 * np.sum(np.abs(pt - pd))
        enum = sum(pd[x] * accept_fraction(lt, ld, x, 1.0) for x in range(V))
        assert abs(enum - alpha) < 2 * 2.0 ** -24
        x = int(np.argmax(pd / pt))         # the most over-proposed token
        res = verify_sequence(np.stack([lt, lt]), np.stack([ld]), [x], 1.0, [1.0], 0.5)
        assert res.k == 0
        assert abs(res.bonus_mass - (1.0 - alpha)) < 1e-12


@pytest.mark.parametrize("case", load("lecture5_expected_tokens.json")["cases"])
def test_expected_tokens_monte_carlo(case):
    alpha, gamma = case["alpha"], case["gamma"]
    E = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs(E - case["printed_E"]) < 0.0051
    # Two tokens: p_t = (0.5, 0.5); p_d = (0.5 + (1 - alpha), alpha - 0.5) gives
    # sum min = alpha. The same pair at every position, drafts drawn from p_d.
    pt = np.array([0.5, 0.5])
    pd = np.array([1.5 - alpha, alpha - 0.5])
    assert abs(np.minimum(pt, pd).sum() - alpha) < 1e-15
    B = 3000
    rng = np.random.default_rng(int(alpha * 100) + gamma)
    target = np.broadcast_to(np.log(pt), (B, gamma + 1, 2))
    draft = np.broadcast_to(np.log(pd), (B, gamma, 2))
    tokens = (rng.random((B, gamma)) < pd[1]).astype(np.int64)
    out = verify_batch(target, draft, tokens, np.ones(B), seed=99, offset=gamma)
    n = out["num_accepted"] + 1
    se = n.std() / np.sqrt(B)
    assert abs(n.mean() - E) < 4 * se, (n.mean(), E, se)


def test_exercise3_speedup_closed_form():
    g = load("lecture5_expected_tokens.json")["exercise3"]
    a, c = g["alpha"], g["c"]
    for gamma, printed in enumerate(g["printed_speedup"], start=1):
        s = (1 - a ** (gamma + 1)) / ((1 - a) * (gamma * c + 1))
        # Printed to two decimals; the page's gamma = 8 value (2.41) sits
        # 0.005 above the formula's 2.405.
        assert abs(s - printed) < 0.006


def test_first_token_distribution_monte_carlo_philox():
    # The batch path with Philox uniforms: the first emitted token follows p_t.
    rng = np.random.default_rng(21)
    V, B = 5, 20000
    lt = rng.normal(0, 1.5, V)
    ld = lt + rng.normal(0, 1.0, V)
    pd = softmax(ld)
    target = np.broadcast_to(np.stack([lt, lt]), (B, 2, V))
    draft = np.broadcast_to(ld[None, None, :], (B, 1, V))
    tokens = rng.choice(V, size=(B, 1), p=pd)
    out = verify_batch(target, draft, tokens, np.ones(B), seed=2024, offset=0)
    emp = np.bincount(out["tokens"][:, 0], minlength=V) / B
    tv = 0.5 * np.abs(emp - softmax(lt)).sum()
    assert tv < 0.015, tv


def test_greedy_ties_take_lowest_index():
    rng = np.random.default_rng(8)
    for _ in range(200):
        z = rng.integers(-3, 3, size=int(rng.integers(1, 40))).astype(np.float64)
        assert sampling.greedy_token(z) == int(np.argmax(z))
    assert sampling.greedy_token([-np.inf, 2.0, 2.0]) == 1
    assert sampling.greedy_token([-0.0, 0.0]) == 0


def test_greedy_chain_rule():
    target = np.array([[0, 5, 1], [2, 2, 0], [0, 0, 9.0]])
    # Position 0 argmax 1, position 1 argmax 0 (tie with 1 -> lowest id).
    r = verify_sequence(target, None, [1, 0], 0.0, [1.0, 1.0], 1.0)
    assert (r.k, r.bonus, r.tokens) == (2, 2, [1, 0, 2])
    r = verify_sequence(target, None, [1, 1], 0.0, [1.0, 1.0], 1.0)
    assert (r.k, r.bonus, r.tokens) == (1, 0, [1, 0])
    np.testing.assert_array_equal(r.probs, [[1, 1], [0, 1]])


def test_small_temperature_limit_is_greedy():
    # Lecture 5 sec. 2.7: with one-hot p and q the sampled rule reduces to
    # "accept iff the draft argmax is the target argmax; else emit the target
    # argmax".
    rng = np.random.default_rng(13)
    for _ in range(100):
        V, gamma = int(rng.integers(2, 30)), int(rng.integers(1, 6))
        target = rng.permuted(np.tile(np.arange(V) * 0.5, (gamma + 1, 1)), axis=1)
        draft = rng.permuted(np.tile(np.arange(V) * 0.5, (gamma, 1)), axis=1)
        x = [int(np.argmax(draft[i])) for i in range(gamma)]
        if rng.random() < 0.5:             # make some drafts agree
            for i in range(gamma):
                if rng.random() < 0.7:
                    draft[i] = target[i]
                    x[i] = int(np.argmax(target[i]))
        u = list(rng.random(gamma) * 0.999 + 0.0005)
        g = verify_sequence(target, draft, x, 0.0, u, 0.5)
        s = verify_sequence(target, draft, x, 1e-3, u, 0.5)
        assert (g.k, g.bonus) == (s.k, s.bonus)


def test_inverse_cdf_matches_searchsorted():
    rng = np.random.default_rng(17)
    for _ in range(2000):
        V = int(rng.integers(1, 50))
        w = rng.random(V) * (rng.random(V) < 0.6)
        if w.sum() == 0:
            w[rng.integers(V)] = 0.3
        v = float(rng.choice([2.0 ** -24, 1.0, rng.random() * 0.999 + 1e-6]))
        j, W, _ = sampling.inverse_cdf(w, v)
        S = np.cumsum(w)
        assert j == int(np.searchsorted(S, v * S[-1], side="left"))
        assert w[j] > 0


def test_zero_residual_falls_back_to_target(monkeypatch):
    monkeypatch.setattr(sampling, "residual_weights", lambda pt, pd: np.zeros_like(pt))
    lt = np.array([0.0, 1.0, 2.0])
    r = verify_sequence(np.stack([lt, lt]), np.stack([lt[::-1]]), [0], 1.0, [1.0], 0.999)
    assert r.k == 0 and r.bonus_mass == 0.0 and r.bonus == 2


def test_planted_wrong_variant_is_caught(monkeypatch):
    # Lecture 5 sec. 2.6, wrong variant A: after a rejection, sample again from
    # p instead of the residual. The exactness check above must reject it.
    lt = np.log(np.array([0.4, 0.3, 0.2, 0.1]))
    ld = np.log(np.array([0.2, 0.5, 0.15, 0.15]))
    monkeypatch.setattr(sampling, "residual_weights", lambda pt, pd: np.asarray(pt))
    out = output_distribution(lt, ld, 1.0)
    assert np.max(np.abs(out - softmax(lt))) > 0.02


def test_near_tie_flag():
    lt = np.log(np.array([0.5, 0.5]))
    ld = np.log(np.array([0.8, 0.2]))
    ratio = 0.5 / 0.8
    r = verify_sequence(np.stack([lt, lt]), np.stack([ld]), [0], 1.0,
                        [ratio + 5e-7], 0.5)
    assert r.near_tie and r.k == 0
    r = verify_sequence(np.stack([lt, lt]), np.stack([ld]), [0], 1.0,
                        [ratio + 5e-6], 0.5)
    assert not r.near_tie


def test_out_of_range_token_is_rejected():
    target = np.zeros((3, 4))
    draft = np.zeros((2, 4))
    for bad in (4, 9, -1):
        r = verify_sequence(target, draft, [1, bad], 1.0, [0.5, 2.0 ** -24], 0.5)
        assert r.k == 1 and r.probs[1].tolist() == [0.0, 0.0]
        g = verify_sequence(target, draft, [0, bad], 0.0, [0.5, 0.5], 0.5)
        assert g.k == 1
