"""Pins for the oracle's top-F bonus candidates (SSD/Saguaro outcome prediction).

* Brute force: a token's rank is the number of tokens that beat it (larger
  logit, or equal logit and lower id); the candidates are the tokens of rank
  < F, found by counting rather than sorting.
* Speculative Speculative Decoding, Appendix A.3, Theorem 19: with F = 2 and the
  drafted token excluded, the bonus lands in the cache 50% of the time for p_d
  and 100% for p'_d; without the exclusion it would be 0% for p_d.
"""
import json
import os

import numpy as np
from scipy.special import softmax

from oracle.sampling import verify_sequence
from oracle.topf import bonus_topf, bonus_topf_batch
from uniform_grid import GRID, bucket_counts, count_accepting

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def brute_topf(z, F, exclude=None):
    ids = [j for j in range(len(z)) if j != exclude]
    rank = {}
    for j in ids:
        rank[j] = sum(1 for i in ids if z[i] > z[j] or (z[i] == z[j] and i < j))
    return [j for j in sorted(ids, key=lambda j: rank[j]) if rank[j] < F]


def test_brute_force_with_ties():
    rng = np.random.default_rng(1)
    for trial in range(300):
        V = int(rng.integers(2, 120))
        pool = np.array([-np.inf, -1.5, -0.0, 0.0, 0.25, 1.0, 3.0])
        z = rng.choice(pool, size=V) if trial % 2 else rng.normal(0, 1, V).round(1)
        F = int(rng.integers(1, min(V, 17)))
        excl = None if trial % 3 == 0 else int(rng.integers(V))
        assert bonus_topf(z, F, excl) == brute_topf(list(z), F, excl)


def test_signed_zero_is_one_value():
    assert bonus_topf([-0.0, 0.0, -1.0], 2) == [0, 1]
    assert bonus_topf([0.0, -0.0, -1.0], 2) == [0, 1]


def test_last_position_has_no_exclusion():
    rng = np.random.default_rng(2)
    draft = rng.normal(0, 1, (2, 4, 30))
    toks = np.array([[int(np.argmax(draft[b, k])) for k in range(3)] for b in range(2)])
    out, vals = bonus_topf_batch(draft, toks, 3)
    for b in range(2):
        for k in range(3):
            assert toks[b, k] not in out[b, k]
        assert out[b, 3].tolist() == brute_topf(list(draft[b, 3]), 3)
        np.testing.assert_array_equal(vals[b, 3], draft[b, 3, out[b, 3]])
    out_none, _ = bonus_topf_batch(draft, None, 3)
    assert out_none[0, 0].tolist() == brute_topf(list(draft[0, 0]), 3)


def hit_rate(p_target, p_draft, F, exclude=True):
    """P(bonus in the cache | a rejection), every decision taken by the oracle:
    x ~ p_draft, accept fraction and bonus distribution enumerated over the
    uniform grid, cache = top-F draft logits excluding x."""
    lt, ld = np.log(p_target), np.log(p_draft)
    V = len(p_target)
    target, draft = np.stack([lt, lt]), np.stack([ld])
    rej, hit = 0.0, 0.0
    for x in range(V):
        a = count_accepting(lambda u: verify_sequence(target, draft, [x], 1.0, [u], 0.5).k == 1) / GRID
        if a == 1.0:
            continue
        bonus = np.array(bucket_counts(
            lambda v: verify_sequence(target, draft, [x], 1.0, [1.0], v).bonus, V)) / GRID
        cache = bonus_topf(ld, F, x if exclude else None)
        rej += p_draft[x] * (1 - a)
        hit += p_draft[x] * (1 - a) * bonus[cache].sum()
    return hit / rej


def test_theorem19_hit_rates():
    with open(os.path.join(GOLDEN, "ssd_theorem19.json")) as f:
        g = json.load(f)
    pt = np.array(g["p_target"])
    pd = np.array(g["p_draft"])
    pds = np.array(g["p_draft_saguaro"])
    pr, F = g["printed"], g["F"]
    assert abs(np.minimum(pt, pd).sum() - pr["acceptance_rate_draft"]) < 1e-12
    assert abs(np.minimum(pt, pds).sum() - pr["acceptance_rate_draft_saguaro"]) < 1e-12
    # The fixture's p'_d is Saguaro sampling of p_d with C = 47/147 on the top-2.
    C = 47 / 147
    w = pd.copy()
    w[bonus_topf(np.log(pd), F)] *= C
    np.testing.assert_allclose(w / w.sum(), pds, atol=1e-12)
    assert abs(hit_rate(pt, pd, F) - pr["hit_rate_draft"]) < 1e-6
    assert abs(hit_rate(pt, pds, F) - pr["hit_rate_draft_saguaro"]) < 1e-6
    # Without the exclusion the cache for p_d would never hold the bonus.
    assert hit_rate(pt, pd, F, exclude=False) < 1e-6


def test_temperature_does_not_change_the_order():
    rng = np.random.default_rng(4)
    z = rng.normal(0, 2, 500).round(2)
    for T in (0.3, 1.0, 2.5):
        p = softmax(z / T)
        assert bonus_topf(z, 8, 3) == brute_topf(list(p), 8, 3)
