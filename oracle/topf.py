"""SSD/Saguaro verification-outcome prediction: top-F bonus candidates (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: Speculative Speculative Decoding, sec. 4.1.1 ("Saguaro verification
outcome prediction"): at every lookahead position k the cache receives the F
tokens with the largest draft logits, after removing the token that was sampled
at that position and sent for verification (it can never be the bonus token).
Appendix A.3, Theorem 19, is the worked example that fixes this exclusion.

Readings (also listed in the design doc):
  * Order: larger logit first, lower token id first among equal logits; -0.0
    and +0.0 are equal.
  * Position k = gamma has no sampled token, so nothing is excluded there; every
    position yields F candidates, (gamma+1)*F per sequence.
  * Temperature does not enter: for T > 0 softmax(z/T) is monotone in z, and
    for T = 0 the order of the logits is the order of interest.
"""

import numpy as np


def rank_order(z):
    """Token ids sorted by (logit descending, id ascending). numpy's lexsort
    sorts by the last key first, so the keys are (id, -logit)."""
    z = np.asarray(z, dtype=np.float64)
    ids = np.arange(z.shape[0])
    return np.lexsort((ids, -z))


def bonus_topf(z, F, exclude=None):
    """The F candidate bonus tokens of one draft row: the first F ids of
    rank_order(z) once the excluded id (the drafted token, or None) is dropped.
    F = 0 gives no candidates (a position the cache does not cover)."""
    if F <= 0:
        return []
    picks = []
    for j in rank_order(z):
        if exclude is not None and int(j) == int(exclude):
            continue
        picks.append(int(j))
        if len(picks) == F:
            break
    return picks


def bonus_topf_batch(draft, draft_tokens, F):
    """draft [B, gamma+1, V], draft_tokens [B, gamma] or None (no exclusion)
    -> candidates [B, gamma+1, F] and their logits."""
    draft = np.asarray(draft, dtype=np.float64)
    B, rows, V = draft.shape
    out = np.zeros((B, rows, F), dtype=np.int64)
    vals = np.zeros((B, rows, F), dtype=np.float64)
    for b in range(B):
        for k in range(rows):
            excl = None
            if draft_tokens is not None and k < rows - 1:
                excl = int(draft_tokens[b][k])
            picks = bonus_topf(draft[b, k], F, excl)
            out[b, k] = picks
            vals[b, k] = draft[b, k, picks]
    return out, vals
