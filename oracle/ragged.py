"""Ragged batches and drafts without probabilities (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: Speculative Decoding (dl-note), Appendix "Implementation Details":
sequence b drafts its own number of tokens (a cumulative-count layout), and a
proposer without probabilities (NO_DRAFT_PROBS) makes the draft probability
of the drafted token 1, so the test becomes p(x) >= u; its resampling keeps
the target distribution with the drafted token masked out. That is the rule of
[Lecture 5: Speculative Decoding and SpecInfer, sec. 2.2] with q the point mass
at x: accept with min(1, p(x)/1), residual norm(max(p - onehot(x), 0)).

Readings (also in the design doc): draft rows and target rows are packed; sequence
b's draft tokens are tokens[off[b] .. off[b+1]) and its target rows 0..gamma_b
are packed rows off[b] + b + i; its bonus uniform uses j = gamma_b.
"""

import numpy as np

from .philox import chain_uniforms
from .sampling import verify_sequence


def point_masses(tokens, V):
    """q rows for drafts without probabilities: one-hot at each drafted token
    (all zero for a token outside the vocabulary, which is then rejected)."""
    rows = []
    for x in tokens:
        q = np.zeros(V)
        if 0 <= int(x) < V:
            q[int(x)] = 1.0
        rows.append(q)
    return rows


def verify_ragged_batch(target_rows, draft_rows, offsets, tokens, temperature, seed, offset, max_gamma):
    """target_rows [num_draft + B, V], draft_rows [num_draft, V] or None,
    offsets [B + 1], tokens [num_draft], temperature [B]. Returns tokens
    [B, max_gamma + 1] (-1 padded), num_accepted, probs [num_draft, 2],
    bonus_mass, near_tie."""
    target_rows = np.asarray(target_rows, dtype=np.float64)
    B = len(offsets) - 1
    V = target_rows.shape[1]
    out = dict(tokens=np.full((B, max_gamma + 1), -1, np.int64), num_accepted=np.zeros(B, np.int64),
               probs=np.zeros((len(tokens), 2)), bonus_mass=np.zeros(B), near_tie=np.zeros(B, bool))
    for b in range(B):
        o0, o1 = int(offsets[b]), int(offsets[b + 1])
        g = o1 - o0
        T = float(temperature[b])
        target = target_rows[o0 + b:o1 + b + 1]
        toks = [int(t) for t in tokens[o0:o1]]
        u, v = chain_uniforms(seed, offset, b, g)
        if draft_rows is None:
            q_rows = point_masses(toks, V) if T > 0 else None
            res = verify_sequence(target, np.zeros((max(g, 1), V)), toks, T, u, v, q_rows=q_rows)
        else:
            res = verify_sequence(target, np.asarray(draft_rows[o0:o1], np.float64), toks, T, u, v)
        out["tokens"][b, :len(res.tokens)] = res.tokens
        out["num_accepted"][b] = res.k
        out["probs"][o0:o1] = res.probs
        out["bonus_mass"][b] = res.bonus_mass
        out["near_tie"][b] = res.near_tie
    return out


__all__ = ["point_masses", "verify_ragged_batch"]
