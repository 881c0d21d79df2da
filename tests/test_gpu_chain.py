"""GPU parity of chain verification and of the uniform stream (MI355X).

The HIP path (through the C ABI) against the oracle on the same seeded inputs:
the named workloads at full size, plus edge cases."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_common import (chain_to_dev, compare_chain, log, run_chain_gpu,
                        run_chain_oracle, to_dev)
from speculative_sampling_verification_04_amd import binding

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


@pytest.mark.parametrize("seed,offset,tag", [(0, 0, 0), (3, 7, 1), (2**63 + 12345, 2**40 + 3, 0), (99, 1, 5)])
def test_uniform_stream_matches_oracle(seed, offset, tag):
    log(f"uniforms seed={seed} offset={offset} tag={tag}")
    B, J = 37, 19
    gpu = binding.uniforms(seed, offset, tag, B, J).cpu().numpy()
    ref = np.array([[oracle.philox.uniform(seed, offset, b, tag, j) for j in range(J)] for b in range(B)])
    np.testing.assert_array_equal(gpu.astype(np.float64), ref)


@pytest.mark.parametrize("name", ["tiny_v16", "v32000_f32", "v128256_bf16_peaked"])
def test_named_workloads(name):
    w = workloads.make_workload(name)
    log(f"chain {name} B={w.B} gamma={w.gamma} V={w.V} {w.dtype}")
    gpu = run_chain_gpu(w)
    ref, seqs = run_chain_oracle(w)
    good, bad = compare_chain(gpu, ref, seqs, w.gamma, name)
    assert bad <= max(1, w.B // 50)


@pytest.fixture(scope="module")
def headline():
    w = workloads.make_workload("v128256_bf16_b256_g8")
    return w, chain_to_dev(w)


def test_headline_workload_all_sequences(headline):
    w, d = headline
    log(f"chain headline B={w.B} gamma={w.gamma} V={w.V}")
    gpu = run_chain_gpu(w, d)
    ref, seqs = run_chain_oracle(w)
    good, bad = compare_chain(gpu, ref, seqs, w.gamma, "headline")
    assert bad <= 5
    # Greedy half: bit-exact by construction, never excluded.
    assert all(not ref["near_tie"][b] for b in range(w.B // 2))


def test_headline_repeat_is_identical(headline):
    w, d = headline
    log("chain headline repeated twice")
    a = run_chain_gpu(w, d)
    b = run_chain_gpu(w, d)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_split_factor_does_not_change_results():
    # Sequences 0 and 1 alone (each row split across ~31 workgroups) and inside
    # a batch of 128 (one workgroup per row) draw the same uniforms; every run
    # must match the oracle.
    w = workloads.make_chain(128, 8, 128256, dtype="bf16", sigma=4.0, noise=1.5, boost_frac=0.01,
                             temps=np.r_[[1.0, 0.0], np.ones(126)], gen_seed=77, philox_seed=5)
    log("chain split-factor invariance B=128 vs B=1 and B=2")
    full = run_chain_gpu(w)
    ref, seqs = run_chain_oracle(w, range(2))
    for n in (1, 2):
        sub = workloads.ChainInputs("sub", n, w.gamma, w.V, w.dtype, w.target[:n], w.draft[:n],
                                    w.draft_tokens[:n], w.temperature[:n], w.seed)
        one = run_chain_gpu(sub)
        sel = {k: (v[:n] if v is not None and v.ndim > 0 else v) for k, v in ref.items()}
        compare_chain(one, sel, list(range(n)), w.gamma, f"split B={n}")
        np.testing.assert_allclose(one["probs"], full["probs"][:n], atol=1e-6)
    compare_chain(full, ref, seqs, w.gamma, "split B=128")


EDGE = [
    # (B, gamma, V, dtype, temps, sigma, noise, seed)
    (3, 1, 1, "f32", "all1", 1.0, 1.0, 1),
    (4, 2, 2, "bf16", "all1", 2.0, 1.0, 2),
    (5, 3, 7, "f32", "all0.5", 2.0, 1.0, 3),
    (6, 4, 16, "bf16", "half0_half1", 3.0, 1.0, 4),
    (7, 5, 33, "f32", "all1", 2.0, 0.5, 5),
    (9, 16, 4097, "bf16", "all1", 4.0, 1.5, 6),
    (4, 12, 4097, "f32", "all2.5", 3.0, 1.0, 7),
    (16, 8, 513, "bf16", "all0", 4.0, 1.5, 8),
    (2, 64, 1000, "f32", "all1", 0.5, 0.2, 9),
    (300, 2, 300, "bf16", "all0.7", 4.0, 1.0, 10),
    # the bonus pass shared by H = ceil(tiles / 16) workgroups up to 64
    # sequences, ceil(tiles / 32) above (at most 16)
    (3, 3, 16385, "bf16", "all1", 3.0, 1.0, 11),          # 33 tiles: H = 3, uneven split
    (5, 6, 70000, "bf16", "half0_half1", 4.0, 1.5, 12),   # 137 tiles: H = 9
    (2, 4, 300000, "f32", "all0.8", 3.0, 1.0, 13),        # 586 tiles: H = 16
    (80, 2, 20000, "bf16", "half0_half1", 3.0, 1.0, 16),  # 40 tiles above 64 sequences: H = 2
    (4, 3, 40000, "bf16", "all1", 3.0, 0.02, 14),         # nearly all accepted: p_t of row gamma
    (4100, 1, 64, "f32", "half0_half1", 2.0, 1.0, 15),     # B > 4096: sequences taken in index order
    (2, 2, 1048576, "bf16", "half0_half1", 4.0, 1.0, 17),  # the largest vocabulary: 2048 tiles, 16 bonus workgroups
    (1, 64, 30000, "f32", "all1", 2.0, 0.05, 18),          # the longest draft, nearly all accepted
]


@pytest.mark.parametrize("B,gamma,V,dtype,temps,sigma,noise,seed", EDGE)
def test_edge_shapes(B, gamma, V, dtype, temps, sigma, noise, seed):
    w = workloads.make_chain(B, gamma, V, dtype=dtype, sigma=sigma, noise=noise, temps=temps,
                             gen_seed=seed, philox_seed=seed)
    log(f"chain edge B={B} gamma={gamma} V={V} {dtype} {temps}")
    gpu = run_chain_gpu(w)
    ref, seqs = run_chain_oracle(w)
    good, bad = compare_chain(gpu, ref, seqs, gamma, f"edge V={V}")
    assert bad <= max(1, B // 20)


def test_unaligned_and_strided_rows():
    # Rows that start off 16-byte boundaries (row stride V + 3) and a batch
    # stride with a gap; the kernels fall back to element loads there.
    w = workloads.make_chain(6, 4, 1001, dtype="bf16", sigma=3, noise=1, temps="half0_half1", gen_seed=12,
                             philox_seed=12)
    log("chain unaligned rows")
    big_t = torch.zeros((6, 5, 1004 + 2), dtype=torch.bfloat16, device="cuda")
    big_d = torch.zeros((6, 6, 1004 + 2), dtype=torch.bfloat16, device="cuda")
    tv = big_t[:, :, 1:1002]
    dv = big_d[:, 1:6, 3:1004]
    tv.copy_(to_dev(w.target, "bf16"))
    dv.copy_(to_dev(w.draft, "bf16")[:, :5])
    out = binding.verify(tv, dv, torch.from_numpy(w.draft_tokens).cuda(), torch.from_numpy(w.temperature).cuda(),
                         w.seed, 0)
    torch.cuda.synchronize()
    gpu = {k: v.cpu().numpy() for k, v in out.items()}
    ref, seqs = run_chain_oracle(w)
    compare_chain(gpu, ref, seqs, w.gamma, "unaligned")


def test_masked_identical_disjoint_and_out_of_range():
    B, gamma, V = 8, 4, 64
    rng = np.random.default_rng(3)
    target = rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    draft = (target + rng.normal(0, 1, target.shape)).astype(np.float32)
    temps = np.ones(B, np.float32)
    tokens = rng.integers(0, V, (B, gamma)).astype(np.int32)
    draft[0] = target[0]                           # identical rows: alpha = 1, every token accepted
    target[1, :, : V // 2] = -np.inf               # disjoint supports: alpha = 0
    draft[1, :, V // 2:] = -np.inf
    tokens[1] = rng.integers(0, V // 2, gamma)
    target[2, :, ::3] = -np.inf                    # masked logits
    tokens[3, 1] = V + 5                           # out of range: rejected at position 1
    tokens[4, 0] = -1
    temps[5] = 0.0
    tokens[5, 2] = V + 1
    temps[6] = 1e-3                                # nearly greedy
    temps[7] = 40.0                                # nearly uniform
    w = workloads.ChainInputs("special", B, gamma, V, "f32", target, draft, tokens, temps, 11)
    log("chain special rows")
    gpu = run_chain_gpu(w)
    ref, seqs = run_chain_oracle(w)
    compare_chain(gpu, ref, seqs, gamma, "special")
    assert gpu["num_accepted"][0] == gamma
    assert gpu["num_accepted"][1] == 0
    assert gpu["num_accepted"][3] <= 1 and gpu["num_accepted"][4] == 0 and gpu["num_accepted"][5] <= 2


def test_distribution_of_first_token_matches_target():
    # 2^18 copies of one position with independent uniforms: the first emitted
    # token follows p_t (a statistical check of the whole GPU path).
    V, B = 12, 1 << 18
    rng = np.random.default_rng(4)
    lt = rng.normal(0, 1.5, V)
    ld = lt + rng.normal(0, 1.0, V)
    pd = np.exp(ld - ld.max()); pd /= pd.sum()
    pt = np.exp(lt - lt.max()); pt /= pt.sum()
    target = np.broadcast_to(np.stack([lt, lt]).astype(np.float32), (B, 2, V)).copy()
    draft = np.broadcast_to(ld.astype(np.float32)[None, None, :], (B, 1, V)).copy()
    tokens = rng.choice(V, size=(B, 1), p=pd).astype(np.int32)
    w = workloads.ChainInputs("dist", B, 1, V, "f32", target, draft, tokens, np.ones(B, np.float32), 21)
    log("chain first-token distribution B=262144")
    gpu = run_chain_gpu(w)
    emp = np.bincount(gpu["tokens"][:, 0], minlength=V) / B
    tv = 0.5 * np.abs(emp - pt).sum()
    assert tv < 0.012, tv


def test_one_workspace_across_shapes():
    # Calls of different shapes sharing one workspace: each call must leave it
    # zero-filled, whatever region the previous layout used.
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    shapes = [(16, 8, 513), (300, 2, 300), (3, 16, 4097), (257, 1, 64), (40, 4, 1000), (6, 3, 70000),
              (2, 2, 300000)]
    assert max(binding.verify_workspace_bytes(B, g, V) for B, g, V in shapes) <= ws.numel()
    for i, (B, gamma, V) in enumerate(shapes * 2):
        w = workloads.make_chain(B, gamma, V, dtype="bf16", sigma=3, noise=1, temps="half0_half1",
                                 gen_seed=100 + i, philox_seed=i)
        log(f"shared workspace call {i}: B={B} gamma={gamma} V={V}")
        d = chain_to_dev(w)
        out = binding.verify(d["target"], d["draft"], d["tokens"], d["temperature"], w.seed, 0, workspace=ws)
        torch.cuda.synchronize()
        gpu = {k: v.cpu().numpy() for k, v in out.items()}
        ref, seqs = run_chain_oracle(w)
        compare_chain(gpu, ref, seqs, gamma, f"shared workspace {i}")
        assert int(ws.count_nonzero().item()) == 0


def test_bonus_pass_with_zero_tiles():
    # A draft far above the target on the first 1024 ids makes the residual
    # max(p_t - p_d, 0) exactly 0 on whole tiles; the tile words of the shared
    # bonus pass must still count as published (V = 20000: two bonus workgroups).
    rng = np.random.default_rng(21)
    B, gamma, V = 8, 2, 20000
    target = rng.normal(0, 1, (B, gamma + 1, V)).astype(np.float32)
    draft = target.copy()
    draft[:, :, :1024] += 3.0
    tokens = np.full((B, gamma), 5, np.int32)
    w = workloads.ChainInputs("zero-tiles", B, gamma, V, "f32", target, draft, tokens,
                              np.ones(B, np.float32), 8, 0, 4)
    log("chain zero tiles")
    gpu = run_chain_gpu(w)
    ref, seqs = run_chain_oracle(w)
    assert np.all(gpu["num_accepted"] >= 0)
    good, bad = compare_chain(gpu, ref, seqs, gamma, "zero tiles")
    assert bad <= 1
