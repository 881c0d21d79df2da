"""Pins for oracle/ragged.py: drafts without probabilities and ragged batches.

* A draft without probabilities is the point mass at its token; the rule then
  accepts x with probability exactly p_t(x) (uniform-grid count) and outputs
  p_t exactly (grid enumeration of accept + bonus, the oracle as a black box).
* A ragged batch whose sequences all draft gamma tokens gives the dense
  batch's outcome (same uniforms: the bonus uses j = gamma_b).
* With unequal counts (0 .. G), every sequence gives the outcome of the
  sequence verified on its own rows, built here from a dense block.
"""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import ragged
from oracle.philox import chain_uniforms
from oracle.sampling import verify_batch, verify_sequence
from uniform_grid import GRID, bucket_counts, count_accepting

TOL_GRID = 3 * 2.0 ** -24


@pytest.mark.parametrize("seed", range(5))
def test_no_draft_probabilities_is_exact(seed):
    rng = np.random.default_rng(40 + seed)
    V = 6
    T = float(rng.choice([0.8, 1.0, 1.3]))
    zt = rng.normal(0, 2, V)
    pt = softmax(zt / T)
    target = np.stack([zt, zt])
    for x in range(V):
        q = ragged.point_masses([x], V)
        run = lambda u, v: verify_sequence(target, np.zeros((1, V)), [x], T, [u], v, q_rows=q)
        a = count_accepting(lambda u: run(u, 0.5).k == 1) / GRID
        assert a == pytest.approx(pt[x], abs=TOL_GRID)            # accept iff u <= p_t(x)
        if a < 1.0:
            counts = np.array(bucket_counts(lambda v: run(1.0, v).bonus, V), np.float64) / GRID
            assert counts[x] == 0.0                                # the drafted token is masked out
            w = pt.copy()
            w[x] = 0.0
            np.testing.assert_allclose(counts, w / w.sum(), atol=V * TOL_GRID)
    # The emitted token is distributed as p_t whatever the (deterministic) draft.
    x = int(rng.integers(V))
    q = ragged.point_masses([x], V)
    run = lambda u, v: verify_sequence(target, np.zeros((1, V)), [x], T, [u], v, q_rows=q)
    a = count_accepting(lambda u: run(u, 0.5).k == 1) / GRID
    out = np.zeros(V)
    out[x] += a
    out += (1 - a) * np.array(bucket_counts(lambda v: run(1.0, v).bonus, V), np.float64) / GRID
    np.testing.assert_allclose(out, pt, atol=V * TOL_GRID)


def test_ragged_with_equal_counts_equals_dense():
    rng = np.random.default_rng(9)
    B, gamma, V = 5, 3, 40
    target = rng.normal(0, 2, (B, gamma + 1, V))
    draft = target + rng.normal(0, 1, (B, gamma + 1, V))
    tokens = rng.integers(0, V, (B, gamma))
    temps = np.array([1.0, 0.0, 0.7, 1.0, 2.0])
    dense = verify_batch(target, draft, tokens, temps, 5, 3)
    offsets = np.arange(B + 1) * gamma
    t_rows = target.reshape(B * (gamma + 1), V)
    d_rows = draft[:, :gamma].reshape(B * gamma, V)
    rag = ragged.verify_ragged_batch(t_rows, d_rows, offsets, tokens.reshape(-1), temps, 5, 3, gamma)
    np.testing.assert_array_equal(rag["tokens"], dense["tokens"])
    np.testing.assert_array_equal(rag["num_accepted"], dense["num_accepted"])
    np.testing.assert_allclose(rag["probs"].reshape(B, gamma, 2), dense["probs"])


@pytest.mark.parametrize("with_draft", [True, False])
@pytest.mark.parametrize("seed", range(4))
def test_ragged_with_unequal_counts_follows_each_sequence(seed, with_draft):
    # Sequence b of a ragged batch is verified exactly as the sequence on its
    # own: its first gamma_b + 1 target rows and gamma_b draft rows of a dense
    # [B, G + 1, V] block, its gamma_b tokens, and the uniforms
    # chain_uniforms(seed, offset, b, gamma_b) (the bonus uniform at j =
    # gamma_b). The packed layout is built here row by row, so a slip in the
    # oracle's packed addressing (target row i of sequence b is packed row
    # off[b] + b + i, draft row i is off[b] + i) changes p_t(x_i) or p_d(x_i).
    rng = np.random.default_rng(70 + seed)
    B, G, V = 9, 5, 48
    counts = rng.integers(0, G + 1, B)
    counts[0], counts[-1] = 0, G
    target = rng.normal(0, 2, (B, G + 1, V))
    draft = target + rng.normal(0, 1, (B, G + 1, V))
    tokens = rng.integers(0, V, (B, G))
    temps = np.array([1.0, 0.0, 0.7, 1.0, 2.0, 0.0, 1.3, 1.0, 0.5])
    t_rows, d_rows, toks = [], [], []
    for b in range(B):
        for i in range(counts[b] + 1):
            t_rows.append(target[b, i])
        for i in range(counts[b]):
            d_rows.append(draft[b, i])
            toks.append(tokens[b, i])
    offsets = np.concatenate([[0], np.cumsum(counts)])
    seed_, off_ = 1234 + seed, 7
    rag = ragged.verify_ragged_batch(np.array(t_rows), np.array(d_rows) if with_draft else None, offsets,
                                     np.array(toks, np.int64), temps, seed_, off_, G)
    for b in range(B):
        g = int(counts[b])
        u, v = chain_uniforms(seed_, off_, b, g)
        q_rows = None
        if not with_draft and temps[b] > 0:
            q_rows = ragged.point_masses(tokens[b, :g], V)
        res = verify_sequence(target[b, :g + 1], draft[b, :max(g, 1)], list(tokens[b, :g]), float(temps[b]), u, v,
                              q_rows=q_rows)
        assert rag["num_accepted"][b] == res.k, f"sequence {b}"
        np.testing.assert_array_equal(rag["tokens"][b, :len(res.tokens)], res.tokens, err_msg=f"sequence {b}")
        assert np.all(rag["tokens"][b, len(res.tokens):] == -1)
        np.testing.assert_array_equal(rag["probs"][offsets[b]:offsets[b + 1]], np.asarray(res.probs).reshape(g, 2))
        assert rag["bonus_mass"][b] == res.bonus_mass
