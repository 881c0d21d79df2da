"""Seeded synthetic inputs for speculative-sampling verification.

The only module shared by the oracle side (tests) and the HIP side (tests,
bench.py, smoke). It holds none of the verification arithmetic: it draws logits
from numpy's PCG64, rounds them to bf16 where asked, draws draft tokens and
token trees, and nothing else. Draft tokens are drawn with the Gumbel-max trick
(argmax of z/T plus standard Gumbel noise), an exact sampler of softmax(z/T)
that is unrelated to the inverse-CDF sampling being verified.

The pages measure on real Llama-3 / Qwen3 logits over Alpaca, GSM8K,
UltraFeedback and HumanEval prompts (Speculative Speculative Decoding, sec. 4
and Appendix B.2); none of that is available here, so seeded synthetic logits
with the same vocabulary sizes stand in for them. Draft logits are target
logits plus Gaussian noise, as the toy drafts of Lecture 5 (sec. 2.5, sec. 3.3)
are built.
"""

from dataclasses import dataclass, field

import numpy as np

# Named workloads: (batch, draft length or tree size, vocabulary, dtype, logit
# distribution, temperature, seeds).
WORKLOADS = {
    # Tiny exact case: small enough for exhaustive enumeration.
    "tiny_v16": dict(kind="chain", B=1, gamma=4, V=16, dtype="f32", sigma=2.0,
                     noise=1.0, boost_frac=0.0, temps="all1", gen_seed=1000,
                     philox_seed=0),
    # fp32 logits over a 32000-token vocabulary.
    "v32000_f32": dict(kind="chain", B=8, gamma=4, V=32000, dtype="f32",
                       sigma=3.0, noise=1.0, boost_frac=0.0, temps="all1",
                       gen_seed=1001, philox_seed=1),
    # Peaked bf16 logits (1% of entries boosted by +8), T = 0.7.
    "v128256_bf16_peaked": dict(kind="chain", B=64, gamma=5, V=128256,
                                dtype="bf16", sigma=4.0, noise=1.5,
                                boost_frac=0.01, temps="all0.7", gen_seed=1002,
                                philox_seed=2),
    # The headline shape: B=256, gamma=8, V=128256 bf16, half the sequences
    # greedy and half at T=1, plus top-F=4 bonus candidates per position.
    "v128256_bf16_b256_g8": dict(kind="chain", B=256, gamma=8, V=128256,
                                 dtype="bf16", sigma=4.0, noise=1.5,
                                 boost_frac=0.01, temps="half0_half1", F=4,
                                 gen_seed=1003, philox_seed=3),
    # Token trees: 64 nodes, depth 6, branching <= 4, V=152064 bf16, T=1.
    "tree_v152064_n64": dict(kind="tree", B=32, N=64, depth=6, branching=4,
                             V=152064, dtype="bf16", sigma=4.0, noise=1.0,
                             boost_frac=0.0, temps="all1", gen_seed=1004,
                             philox_seed=4),
}


def round_to_bf16(a):
    """Round fp32 values to the nearest bf16 (ties to even) and return them as
    fp32, using torch's conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _logits(rng, shape, sigma, boost_frac, dtype):
    z = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    if boost_frac > 0:
        z += np.float32(8.0) * (rng.random(shape, dtype=np.float32) < boost_frac)
    return z


def _finish(z, dtype):
    return round_to_bf16(z) if dtype == "bf16" else np.ascontiguousarray(z, np.float32)


def _temperatures(spec, B):
    if spec == "all1":
        return np.ones(B, np.float32)
    if spec == "all0":
        return np.zeros(B, np.float32)
    if spec.startswith("all"):
        return np.full(B, float(spec[3:]), np.float32)
    if spec == "half0_half1":
        t = np.ones(B, np.float32)
        t[: B // 2] = 0.0
        return t
    raise ValueError(spec)


def gumbel_max_sample(rng, z, T):
    """One sample from softmax(z/T) (T > 0) by the Gumbel-max trick; T = 0
    returns the argmax (first occurrence)."""
    z = np.asarray(z, dtype=np.float64)
    if T == 0:
        return int(np.argmax(z))
    g = -np.log(-np.log(rng.random(z.shape[0]) * (1 - 2e-16) + 1e-16))
    return int(np.argmax(z / T + g))


@dataclass
class ChainInputs:
    name: str
    B: int
    gamma: int
    V: int
    dtype: str
    target: np.ndarray          # [B, gamma+1, V] fp32 (bf16-exact when dtype=bf16)
    draft: np.ndarray           # [B, gamma+1, V]
    draft_tokens: np.ndarray    # [B, gamma] int32
    temperature: np.ndarray     # [B] fp32, 0 = greedy
    seed: int
    offset: int = 0
    F: int = 4
    extra: dict = field(default_factory=dict)


@dataclass
class TreeInputs:
    name: str
    B: int
    N: int
    V: int
    dtype: str
    target: np.ndarray          # [B, N, V]
    draft: np.ndarray           # [B, N, V]
    parent: np.ndarray          # [B, N] int32, parent[:, 0] = -1
    tokens: np.ndarray          # [B, N] int32, tokens[:, 0] unused (0)
    temperature: np.ndarray     # [B]
    seed: int
    offset: int = 0


def make_chain(B, gamma, V, dtype="f32", sigma=2.0, noise=1.0, boost_frac=0.0,
               temps="all1", gen_seed=0, philox_seed=0, offset=0, F=4,
               name="chain"):
    """Target logits ~ N(0, sigma^2) (+8 on a boost_frac share of entries),
    draft = target + N(0, noise^2), both rounded to dtype. Draft tokens are
    sampled from the (rounded) draft row at the sequence's temperature."""
    rng = np.random.default_rng(gen_seed)
    target = _logits(rng, (B, gamma + 1, V), sigma, boost_frac, dtype)
    draft = target + rng.standard_normal(target.shape, dtype=np.float32) * np.float32(noise)
    target = _finish(target, dtype)
    draft = _finish(draft, dtype)
    temperature = _temperatures(temps, B) if isinstance(temps, str) else np.asarray(temps, np.float32)
    tokens = np.zeros((B, gamma), np.int32)
    for b in range(B):
        for i in range(gamma):
            tokens[b, i] = gumbel_max_sample(rng, draft[b, i], float(temperature[b]))
    return ChainInputs(name, B, gamma, V, dtype, target, draft, tokens,
                       temperature, philox_seed, offset, F)


def make_tree(B, N, V, depth=6, branching=4, dtype="bf16", sigma=4.0, noise=1.0,
              boost_frac=0.0, temps="all1", gen_seed=0, philox_seed=0, offset=0,
              name="tree"):
    """Random token trees: nodes 1..depth form a spine (so the depth is exact);
    every later node picks its parent uniformly among earlier nodes with depth
    < `depth` and fewer than `branching` children. Each node's token is an
    independent sample from softmax(draft[parent]/T)."""
    if N < depth + 1:
        raise ValueError("N must be at least depth+1")
    rng = np.random.default_rng(gen_seed)
    target = _finish(_logits(rng, (B, N, V), sigma, boost_frac, dtype), dtype)
    draft = _finish(target + rng.standard_normal((B, N, V), dtype=np.float32)
                    * np.float32(noise), dtype)
    temperature = _temperatures(temps, B) if isinstance(temps, str) else np.asarray(temps, np.float32)
    parent = np.full((B, N), -1, np.int32)
    tokens = np.zeros((B, N), np.int32)
    for b in range(B):
        d = [0] * N
        nkids = [0] * N
        for n in range(1, N):
            if n <= depth:
                p = n - 1
            else:
                cand = [x for x in range(n) if d[x] < depth and nkids[x] < branching]
                p = cand[int(rng.integers(len(cand)))]
            parent[b, n] = p
            d[n] = d[p] + 1
            nkids[p] += 1
            tokens[b, n] = gumbel_max_sample(rng, draft[b, p], float(temperature[b]))
    return TreeInputs(name, B, N, V, dtype, target, draft, parent, tokens,
                      temperature, philox_seed, offset)


def make_workload(name, **overrides):
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    kind = spec.pop("kind")
    if kind == "chain":
        return make_chain(name=name, **spec)
    return make_tree(name=name, **spec)
