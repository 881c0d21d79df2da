"""Chain verification: accept prefix, first rejection, bonus token (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (page title, section):
  [L5]  Lecture 5: Speculative Decoding and SpecInfer -- sec. 2.1 (every sampler
        is "sample from an adjusted p"; temperature = softmax(logits/T)),
        sec. 2.2 (the rule: accept x when u <= p(x)/q(x), else resample from
        norm(max(0, p - q))), sec. 2.7 (greedy is the one-hot special case),
        sec. 3.1 (one iteration: gamma guesses, gamma+1 target distributions,
        first rejection n+1, residual at n+1 or a free token from p_{gamma+1}).
  [DLN] Speculative Decoding (dl-note) -- sec. 2.2 Verification (alpha_i =
        min(1, p_t/p_d)), sec. 2.3 Rejection and Resampling (p_res =
        [p_t - p_d]_+ / sum), Appendix "Implementation Details" (vLLM accepts
        when p/q >= u and rejects when the draft probability is 0; greedy
        requests are handled apart).
  [SSD] Speculative Speculative Decoding -- sec. 2.1 (the verification outcome
        is (k, t*): k accepted draft tokens plus the bonus token).

Everything is fp64. Inputs are logits already decoded exactly to fp64.
Readings where the pages are silent (each also listed in the design doc):
  * T = 0 means greedy: one-hot at the argmax, lowest index on ties; greedy
    sequences never read draft logits.
  * Accept iff p_d(x) > 0 and u <= p_t(x)/p_d(x), with u in (0, 1].
  * Inverse CDF in index order: the bonus is the smallest j with S_j >= v*W,
    S_j = w_0 + ... + w_j summed left to right, W = S_{V-1}.
  * A residual with zero total mass (possible only through rounding) falls back
    to p_t of the same row.
  * A draft token outside [0, V) has probability 0 under both distributions,
    so it is rejected (greedy: it is never the argmax).
"""

from dataclasses import dataclass, field

import numpy as np

NEAR_TIE = 1e-6  # a threshold comparison this close to equality is a near tie


def tempered_probs(z, T):
    """softmax(z / T) for T > 0 [L5 sec. 2.1]. The max is subtracted first;
    logits of -inf get probability 0. At least one logit must be finite."""
    z = np.asarray(z, dtype=np.float64)
    if not T > 0:
        raise ValueError("tempered_probs needs T > 0; T = 0 is the greedy path")
    m = np.max(z)
    if not np.isfinite(m):
        raise ValueError("a row needs at least one finite logit")
    e = np.exp((z - m) / T)
    return e / np.sum(e)


def greedy_token(z):
    """The one-hot distribution's token: argmax, first occurrence on ties
    [L5 sec. 2.7]."""
    z = np.asarray(z, dtype=np.float64).tolist()
    best = 0
    for j in range(1, len(z)):
        if z[j] > z[best]:
            best = j
    return best


def prob_at(p, x):
    """p(x), with 0 for a token outside the vocabulary."""
    return float(p[x]) if 0 <= x < len(p) else 0.0


def accept(pt_x, pd_x, u, lenience=1.0):
    """Accept the drafted token iff u <= p_t(x)/p_d(x) [L5 sec. 2.2]; a draft
    probability of 0 rejects [DLN Appendix]. With a lenience l in (0, 1], q(x)
    is multiplied by l before the comparison [L5 sec. 2.8]: u <= p_t/(l p_d);
    l = 1 is the exact rule."""
    if not pd_x > 0:
        return False
    return u <= pt_x / (lenience * pd_x)


def accept_margin(pt_x, pd_x, u, lenience=1.0):
    """|u - p_t(x)/(l p_d(x))|, the distance of the accept decision from a tie
    (infinite when the decision does not depend on u)."""
    if not pd_x > 0:
        return np.inf
    return abs(u - pt_x / (lenience * pd_x))


def residual_weights(pt, pd):
    """[p_t - p_d]_+ elementwise [DLN sec. 2.3; L5 sec. 2.2 step 4]."""
    return np.maximum(np.asarray(pt) - np.asarray(pd), 0.0)


def inverse_cdf(w, v):
    """Sample index j from the unnormalised weights w >= 0 with the uniform v in
    (0, 1]: the smallest j with S_j >= v * W, where S is the running sum in
    index order and W = S_{V-1}.

    Returns (j, W, margin), margin = distance of v*W from the nearer edge of
    bucket j, divided by W."""
    S = np.cumsum(np.asarray(w, dtype=np.float64))
    W = S[-1]
    if not W > 0:
        raise ValueError("inverse_cdf needs positive total mass")
    t = v * W
    j = int(np.flatnonzero(S >= t)[0])
    lo = S[j - 1] if j > 0 else 0.0
    margin = min(t - lo, S[j] - t) / W
    return j, W, margin


@dataclass
class ChainOutcome:
    """Result of verifying one sequence: the verification outcome (k, t*)
    [SSD sec. 2.1] plus what the library reports beside it."""

    k: int                      # number of accepted draft tokens
    bonus: int                  # t*, from the residual, from p_t, or the argmax
    tokens: list                # x_0 .. x_{k-1}, then the bonus
    probs: np.ndarray           # [gamma, 2]: (p_t(x_i), p_d(x_i)) per position
    bonus_mass: float           # total mass of the weights the bonus came from
    near_tie: bool              # some decision taken lay within NEAR_TIE of a tie
    margins: list = field(default_factory=list)  # every decision's margin


def verify_sequence(target, draft, draft_tokens, T, u, v, q_rows=None, lenience=1.0):
    """Verify one sequence with the uniforms given explicitly.

    target: [gamma+1, V] logits; draft: [>= gamma, V] logits (only rows
    0..gamma-1 are read, and none when T = 0); draft_tokens: gamma ids;
    u: gamma accept uniforms; v: the bonus uniform.
    Follows [L5 sec. 3.1] steps 3-5 with the rule of [L5 sec. 2.2].
    q_rows: the draft distributions the tokens were drawn from, when they are
    not softmax(draft/T) (Saguaro sampling, oracle/ssd.py); lenience: l of
    [L5 sec. 2.8] (1 = exact). Neither changes the greedy path, where p and q
    are one-hot."""
    target = np.asarray(target, dtype=np.float64)
    gamma = len(draft_tokens)
    probs = np.zeros((gamma, 2), dtype=np.float64)

    if T == 0:
        # Greedy [L5 sec. 2.7]: accept iff the draft token is the target argmax;
        # the first mismatch emits the target argmax, and if every token is
        # accepted the argmax of row gamma is the free token.
        argmax = [greedy_token(target[i]) for i in range(gamma + 1)]
        for i in range(gamma):
            probs[i] = (1.0 if draft_tokens[i] == argmax[i] else 0.0, 1.0)
        k = gamma
        for i in range(gamma):
            if draft_tokens[i] != argmax[i]:
                k = i
                break
        bonus = argmax[k]
        tokens = [int(t) for t in draft_tokens[:k]] + [bonus]
        return ChainOutcome(k, bonus, tokens, probs, 1.0, False, [])

    draft = np.asarray(draft, dtype=np.float64)
    pt_rows = [tempered_probs(target[i], T) for i in range(gamma + 1)]
    pd_rows = list(q_rows) if q_rows is not None else [tempered_probs(draft[i], T) for i in range(gamma)]
    for i in range(gamma):
        x = int(draft_tokens[i])
        probs[i] = (prob_at(pt_rows[i], x), prob_at(pd_rows[i], x))

    margins = []
    k = gamma
    for i in range(gamma):
        pt_x, pd_x = probs[i]
        margins.append(accept_margin(pt_x, pd_x, u[i], lenience))
        if not accept(pt_x, pd_x, u[i], lenience):
            k = i
            break

    if k < gamma:
        w = residual_weights(pt_rows[k], pd_rows[k])
        if not np.sum(w) > 0:
            w = pt_rows[k]          # zero residual mass: fall back to p_t
            mass = 0.0
        else:
            mass = None
    else:
        w = pt_rows[gamma]          # every draft accepted: sample from p_t
        mass = None
    bonus, W, cdf_margin = inverse_cdf(w, v)
    if mass is None:
        mass = W
    margins.append(cdf_margin)
    near = any(mg <= NEAR_TIE for mg in margins)
    tokens = [int(t) for t in draft_tokens[:k]] + [bonus]
    return ChainOutcome(k, bonus, tokens, probs, float(mass), near, margins)


def verify_batch(target, draft, draft_tokens, temperature, seed, offset):
    """Verify a batch with uniforms from the Philox stream (tag 0).

    target [B, gamma+1, V], draft [B, >= gamma, V], draft_tokens [B, gamma],
    temperature [B] (0 = greedy). Returns a dict shaped like the library's
    outputs: tokens [B, gamma+1] padded with -1, num_accepted [B],
    probs [B, gamma, 2], bonus_mass [B], near_tie [B]."""
    from .philox import chain_uniforms

    B, gamma = np.asarray(draft_tokens).shape
    out_tokens = np.full((B, gamma + 1), -1, dtype=np.int64)
    num_acc = np.zeros(B, dtype=np.int64)
    probs = np.zeros((B, gamma, 2), dtype=np.float64)
    mass = np.zeros(B, dtype=np.float64)
    near = np.zeros(B, dtype=bool)
    for b in range(B):
        u, v = chain_uniforms(seed, offset, b, gamma)
        res = verify_sequence(target[b], draft[b], draft_tokens[b],
                              float(temperature[b]), u, v)
        out_tokens[b, :len(res.tokens)] = res.tokens
        num_acc[b] = res.k
        probs[b] = res.probs
        mass[b] = res.bonus_mass
        near[b] = res.near_tie
    return dict(tokens=out_tokens, num_accepted=num_acc, probs=probs,
                bonus_mass=mass, near_tie=near)
