"""Pins for oracle/ragged.py: drafts without probabilities and ragged batches.

* A draft without probabilities is the point mass at its token; the rule then
  accepts x with probability exactly p_t(x) (uniform-grid count) and outputs
  p_t exactly (grid enumeration of accept + bonus, the oracle as a black box).
* A ragged batch whose sequences all draft gamma tokens gives the dense
  batch's outcome (same uniforms: the bonus uses j = gamma_b).
"""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import ragged
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
