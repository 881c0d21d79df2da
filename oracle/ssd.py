"""SSD/Saguaro extensions of chain verification, and the lenient accept rule
(oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (page title, section):
  [SSD] Speculative Speculative Decoding -- sec. 4.1.1 (the fan-out F_k is the
        number of cached outcomes with k accepted tokens; Saguaro outcome
        prediction caches, at every lookahead position k, the top-F_k draft
        tokens once the token sampled there is removed), sec. 4.1.2 and
        Appendix A.2 (Theorem 12: under a power-law hit rate the best fan-out
        is a capped geometric series, with F_0 in closed form), sec. 4.2.1
        (Saguaro sampling sigma_{F,C}: weight C * exp(z_t) on the top-F tokens
        and exp(z_t) elsewhere), Appendix A.3 (Theorem 15: the hit rate does
        not increase with C; Theorem 19: the worked example).
  [L5]  Lecture 5: Speculative Decoding and SpecInfer -- sec. 2.2 (the rule and
        the residual), sec. 2.8 (lenience: q(x) is multiplied by l in (0, 1]
        before the comparison; no output probability exceeds p(x)/l).

Readings where the pages are silent (each also listed in the design doc):
  * sigma_{F,C} is applied to the tempered logits z/T. For T > 0 top_F(z/T) =
    top_F(z); ties are ordered as in topf.rank_order. At position k it uses
    F = F_k, the cache's fan-out at that position, so that the down-weighted
    tokens are the cached ones (the cache also drops the sampled token).
  * Verification with Saguaro sampling: q = sigma_{F_k,C}(draft_k / T) is the
    distribution the drafted token was drawn from, so it is q both in the
    accept rule and in the residual. Greedy sequences are unchanged.
  * If sigma's total weight is 0 (C = 0 and nothing outside top_F has
    positive probability), sigma is taken to be softmax(z/T).
  * Lenience changes only the comparison, u <= p(x)/(l q(x)); the residual stays
    norm(max(p - q, 0)).
  * The outcome (k, t*) hits the cache iff t* is one of the F_k candidates at
    position k.
  * Integer fan-out: Theorem 12's real F_k are rounded by largest remainder
    (floors first, then +1 to the largest fractional parts, lower k first on
    equal parts) so that they sum to the budget.
"""

import numpy as np

from .philox import chain_uniforms
from .sampling import tempered_probs, verify_sequence
from .topf import bonus_topf, rank_order


def saguaro_probs(z, T, F, C):
    """sigma_{F,C}(z/T) [SSD sec. 4.2.1]: proportional to C * exp(z_t/T) for
    the F tokens of largest logit and exp(z_t/T) for the others."""
    p = tempered_probs(z, T)
    if F <= 0:
        return p
    w = p.copy()
    w[rank_order(z)[:F]] *= C
    total = np.sum(w)
    if not total > 0:
        return p
    return w / total


def draft_distributions(draft, T, fanout, C):
    """The distributions the drafted tokens were drawn from: sigma_{F_k,C} of
    draft rows 0..gamma-1 (plain softmax when C = 1)."""
    gamma = len(fanout) - 1
    return [saguaro_probs(draft[i], T, int(fanout[i]), C) for i in range(gamma)]


def cache_candidates(draft, draft_tokens, fanout):
    """The speculation cache's bonus guesses [SSD sec. 4.1.1]: for position
    k = 0..gamma the F_k tokens of largest draft logit, without the token
    drafted at k (position gamma has none)."""
    gamma = len(draft_tokens)
    out = []
    for k in range(gamma + 1):
        excl = int(draft_tokens[k]) if k < gamma else None
        out.append(bonus_topf(draft[k], int(fanout[k]), excl))
    return out


def verify_cached(target, draft, draft_tokens, T, u, v, fanout, C=1.0, lenience=1.0):
    """One sequence: verification with the draft distribution sigma_{F_k,C}
    (C = 1: plain softmax) and lenience l, plus the cache candidates and the
    hit flag. draft has gamma + 1 rows (row gamma only feeds the cache).
    Returns (ChainOutcome, candidates, hit)."""
    target = np.asarray(target, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.float64)
    if T > 0:
        q_rows = draft_distributions(draft, T, fanout, C)
        res = verify_sequence(target, draft, draft_tokens, T, u, v, q_rows=q_rows, lenience=lenience)
    else:
        res = verify_sequence(target, draft, draft_tokens, T, u, v)
    cands = cache_candidates(draft, draft_tokens, fanout)
    hit = res.bonus in cands[res.k]
    return res, cands, hit


def verify_cached_batch(target, draft, draft_tokens, temperature, seed, offset, fanout, C=1.0, lenience=1.0):
    """A batch with uniforms from the Philox stream (tag 0), shaped like the
    library's outputs: tokens [B, gamma+1] (-1 padded), num_accepted, probs
    [B, gamma, 2], bonus_mass, near_tie, topk [B, gamma+1, max F_k] (-1 padded),
    hit [B]."""
    draft_tokens = np.asarray(draft_tokens)
    B, gamma = draft_tokens.shape
    fmax = max(1, int(max(fanout)))
    out = dict(tokens=np.full((B, gamma + 1), -1, np.int64), num_accepted=np.zeros(B, np.int64),
               probs=np.zeros((B, gamma, 2)), bonus_mass=np.zeros(B), near_tie=np.zeros(B, bool),
               topk=np.full((B, gamma + 1, fmax), -1, np.int64), hit=np.zeros(B, np.int64))
    for b in range(B):
        u, v = chain_uniforms(seed, offset, b, gamma)
        res, cands, hit = verify_cached(target[b], draft[b], draft_tokens[b], float(temperature[b]), u, v,
                                        fanout, C, lenience)
        out["tokens"][b, :len(res.tokens)] = res.tokens
        out["num_accepted"][b] = res.k
        out["probs"][b] = res.probs
        out["bonus_mass"][b] = res.bonus_mass
        out["near_tie"][b] = res.near_tie
        for k, c in enumerate(cands):
            out["topk"][b, k, :len(c)] = c
        out["hit"][b] = int(hit)
    return out


def geometric_fanout(K, a, r, budget):
    """Theorem 12 [SSD sec. 4.1.2, Appendix A.2]: with acceptance rate a and a
    power-law hit rate 1 - F^-r, the best real fan-outs under sum F_k = budget
    are F_k = F_0 a^(k/(1+r)) for k < K and F_K = F_0 a^(K/(1+r))
    (1-a)^(-1/(1+r)), with F_0 fixed by the budget (closed form in A.2)."""
    g = a ** (1.0 / (1.0 + r))
    F0 = budget / (a ** (K / (1.0 + r)) * (1.0 - a) ** (-1.0 / (1.0 + r)) + (1.0 - g ** K) / (1.0 - g))
    F = [F0 * a ** (k / (1.0 + r)) for k in range(K)]
    F.append(F0 * a ** (K / (1.0 + r)) * (1.0 - a) ** (-1.0 / (1.0 + r)))
    return np.array(F)


def integer_fanout(F_real, budget):
    """Largest-remainder rounding of real fan-outs to integers summing to the
    budget (floors, then +1 to the largest fractional parts; lower k first
    among equal parts)."""
    F_real = np.asarray(F_real, dtype=np.float64)
    fl = np.floor(F_real).astype(np.int64)
    left = int(budget - fl.sum())
    frac = F_real - fl
    order = sorted(range(len(F_real)), key=lambda k: (-frac[k], k))
    for k in order[:max(0, left)]:
        fl[k] += 1
    return fl


def hit_given_rejection(pt, q, z, F):
    """Exact probability that, given a rejection at one position, the bonus
    lands in the cache [SSD sec. 4.1.1]: the drafted token x ~ q is rejected
    with probability 1 - min(1, p_t(x)/q(x)), the bonus is drawn from
    norm(max(p_t - q, 0)), and the cache holds the top-F draft logits z
    without x. Used by the tests of Theorem 19."""
    pt = np.asarray(pt, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    w = np.maximum(pt - q, 0.0)
    if not w.sum() > 0:
        return 1.0
    w = w / w.sum()
    rej = 0.0
    hit = 0.0
    for x in range(len(q)):
        if q[x] <= 0:
            continue
        p_rej = 1.0 - min(1.0, pt[x] / q[x])
        if p_rej <= 0:
            continue
        rej += q[x] * p_rej
        hit += q[x] * p_rej * w[bonus_topf(z, F, exclude=x)].sum()
    return hit / rej if rej > 0 else 1.0


__all__ = ["saguaro_probs", "draft_distributions", "cache_candidates", "verify_cached", "verify_cached_batch",
           "geometric_fanout", "integer_fanout", "hit_given_rejection"]
