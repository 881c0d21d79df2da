"""GPU parity of bonus draws from small residuals (MI355X).

Near-identical drafts make the residual max(p_t - p_d, 0) of [Lecture 5:
Speculative Decoding and SpecInfer, sec. 2.2; Speculative Decoding (dl-note),
sec. 2.3] small everywhere: every weight is a tiny fraction of p_t, which is
where a residual formed as a difference of two rounded probabilities loses
its relative accuracy. Here the draft is the target plus N(0, sigma^2) noise
(sigma in 0 .. 0.1, rounded to bf16 as the target), and at position 0 one
token of low target probability gets a draft probability of m (log-uniform in
1e-4 .. 1e-2) and is the drafted token: it is rejected almost surely, and the
bonus is drawn from a residual of mass about m (plus what the noise adds).
Outcomes must equal the oracle's except where the oracle flags a near tie.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import chain_to_dev, compare_chain, log, run_chain_oracle
from speculative_sampling_verification_04_amd import binding

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def near_identical(B, gamma, V, seed, T=1.0):
    """Inputs described in the module docstring (bf16 logits at fp32)."""
    rng = np.random.default_rng(seed)
    target = workloads.round_to_bf16((rng.standard_normal((B, gamma + 1, V), dtype=np.float32) * 4.0)
                                     + np.float32(8.0) * (rng.random((B, gamma + 1, V), dtype=np.float32) < 0.01))
    sigmas = np.array([0.0, 0.01, 0.03, 0.1])[np.arange(B) % 4]
    noise = rng.standard_normal((B, gamma + 1, V), dtype=np.float32) * sigmas[:, None, None].astype(np.float32)
    draft = workloads.round_to_bf16(target + noise)
    masses = 10.0 ** rng.uniform(-4, -2, B)
    temps = np.full(B, T, np.float32)
    tokens = np.zeros((B, gamma), np.int32)
    for b in range(B):
        z = target[b, 0].astype(np.float64)
        order = np.argsort(z)
        x = int(order[rng.integers(0, V // 2)])          # a token in the lower half of the target row
        d = draft[b, 0].astype(np.float64) / T
        rest = d.copy()
        rest[x] = -np.inf
        mx = rest.max()
        lz = mx + np.log(np.exp(rest - mx).sum())          # log of the draft row's mass without x
        draft[b, 0, x] = np.float32(T * (lz + np.log(masses[b] / (1 - masses[b]))))
        tokens[b, 0] = x
        for i in range(1, gamma):
            tokens[b, i] = workloads.gumbel_max_sample(rng, draft[b, i], T)
    draft = workloads.round_to_bf16(draft)
    return workloads.ChainInputs("near-identical", B, gamma, V, "bf16", target, draft, tokens, temps, seed % 1000)


@pytest.fixture(scope="module")
def small_residuals():
    return near_identical(320, 2, 128256, 2024)


@pytest.mark.parametrize("entry", ["verify", "verify_topk"])
def test_small_residuals_are_drawn_exactly(small_residuals, entry):
    w = small_residuals
    d = chain_to_dev(w)
    log(f"small residuals: {entry} B={w.B} gamma={w.gamma} V={w.V}")
    if entry == "verify":
        out = binding.verify(d["target"], d["draft"], d["tokens"], d["temperature"], w.seed, w.offset)
    else:
        out = binding.verify_topk(d["target"], d["draft"], d["tokens"], d["temperature"], 4, w.seed, w.offset)
    torch.cuda.synchronize()
    gpu = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
    ref, seqs = run_chain_oracle(w)
    rejected = ref["num_accepted"] < w.gamma
    mass = ref["bonus_mass"][rejected]
    log(f"{int(rejected.sum())} residual draws; masses {np.percentile(mass, [0, 10, 50, 90, 100])}")
    assert rejected.sum() >= 0.9 * w.B
    assert np.mean(mass < 1e-3) > 0.2 and np.mean(mass < 1e-2) > 0.6 and np.mean(mass < 3e-4) > 0.05
    compare_chain(gpu, ref, seqs, w.gamma, f"small residuals {entry}")


def test_small_residuals_tree():
    # A chain-shaped tree (one child per node) over the same kind of rows: the
    # first child of the root is the forced token, so the walk draws its bonus
    # from the root's small residual (multi-step sampling, tree oracle).
    from gpu_common import compare_tree, run_tree_oracle, tree_to_dev
    B, N, V = 96, 3, 128256
    w = near_identical(B, N - 1, V, 77)
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    tok = np.zeros((B, N), np.int32)
    tok[:, 1:] = w.draft_tokens
    t = workloads.TreeInputs("near-identical tree", B, N, V, "bf16", w.target, w.draft, parent, tok, w.temperature,
                             w.seed)
    d = tree_to_dev(t)
    log(f"small residuals: tree B={B} N={N} V={V}")
    out = binding.tree_verify(d["target"], d["draft"], d["parent"], d["tokens"], d["temperature"], t.seed, t.offset)
    torch.cuda.synchronize()
    gpu = {k: v.cpu().numpy() for k, v in out.items()}
    ref, seqs = run_tree_oracle(t)
    compare_tree(gpu, ref, seqs, "small residuals tree")
