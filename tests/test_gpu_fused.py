"""GPU parity of specv_verify_topk: the same outputs as specv_verify followed
by specv_bonus_topk, and as the oracle. One kernel streams every draft row
once; small batches split each row into chunks and merge the draft rows'
top-F keys in the bonus workgroups."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_common import chain_to_dev, compare_chain, log, oracle_topf_all, run_chain_oracle
from speculative_sampling_verification_04_amd import binding

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def run_both(w, F):
    d = chain_to_dev(w)
    fused = binding.verify_topk(d["target"], d["draft"], d["tokens"], d["temperature"], F, w.seed, w.offset)
    sep = binding.verify(d["target"], d["draft"], d["tokens"], d["temperature"], w.seed, w.offset)
    ids, vals = binding.bonus_topk(d["draft"], d["tokens"], F)
    torch.cuda.synchronize()
    f = {k: v.cpu().numpy() for k, v in fused.items() if v is not None}
    s = {k: v.cpu().numpy() for k, v in sep.items() if v is not None}
    s["topk"], s["topk_logits"] = ids.cpu().numpy(), vals.cpu().numpy()
    return f, s


@pytest.mark.parametrize("name,B,gamma,V,dtype,temps,F", [
    ("headline", None, None, None, None, None, 4),
    ("fused-f32-mixed", 300, 6, 7000, "f32", "half0_half1", 3),
    ("fused-F16", 256, 8, 9000, "bf16", "all1", 16),
    ("split-small-batch", 4, 5, 50000, "bf16", "half0_half1", 4),       # rows in 3 chunks
    ("split-one-sequence", 1, 8, 128256, "bf16", "all1", 4),        # 7 chunks per draft row
    ("split-F31", 2, 3, 40000, "f32", "half0_half1", 31),           # K = 32, 2 chunks
    ("split-31-chunks", 1, 2, 600000, "bf16", "half0_half1", 9),    # the most chunks
    ("split-greedy", 2, 3, 40000, "bf16", "all0", 5),                # greedy only, 2 chunks
    ("largest-vocab", 1, 2, 1048576, "bf16", "half0_half1", 31),    # V = 2^20, 31 chunks, F = 31
    ("longest-draft", 2, 64, 20000, "f32", "all1", 6),               # gamma = 64
    ("split-tiny", 3, 2, 40, "f32", "all0.8", 7),
    ("batch-over-4096", 4100, 1, 64, "f32", "half0_half1", 3),   # sequences taken in index order
])
def test_fused_equals_separate_and_oracle(name, B, gamma, V, dtype, temps, F):
    if name == "headline":
        w = workloads.make_workload("v128256_bf16_b256_g8")
    else:
        w = workloads.make_chain(B, gamma, V, dtype=dtype, sigma=4.0, noise=1.5, boost_frac=0.01, temps=temps,
                                 gen_seed=hash(name) % 1000, philox_seed=7)
    log(f"fused {name} B={w.B} gamma={w.gamma} V={w.V} F={F}")
    f, s = run_both(w, F)
    ref, seqs = run_chain_oracle(w)
    compare_chain(f, ref, seqs, w.gamma, f"fused {name}")
    # Top-F is integer work: identical. Away from near ties the outcomes are
    # identical too; the fp32 probabilities may differ in the last bit (the
    # fused kernel sums the draft rows in another order).
    for k in ("topk", "topk_logits"):
        np.testing.assert_array_equal(f[k], s[k], err_msg=f"{name}: {k} differs from the separate call")
    clear = ~ref["near_tie"]
    for k in ("tokens", "num_accepted"):
        np.testing.assert_array_equal(f[k][clear], s[k][clear], err_msg=f"{name}: {k} differs")
    for k in ("probs", "bonus_mass"):
        np.testing.assert_allclose(f[k], s[k], atol=1e-6, err_msg=f"{name}: {k} differs")
    if name == "headline":   # every row (the oracle's top-F, computed once per test process)
        ids, vals = oracle_topf_all("headline", workloads.round_to_bf16(w.draft), w.draft_tokens, F)
        np.testing.assert_array_equal(f["topk"], ids, err_msg=f"{name}: top-F ids")
        np.testing.assert_array_equal(f["topk_logits"].astype(np.float64), vals, err_msg=f"{name}: top-F logits")
        return
    sample = list(range(0, w.B, max(1, w.B // 24)))
    for b in sample:
        ids, vals = oracle.topf.bonus_topf_batch(w.draft[b:b + 1].astype(np.float64), w.draft_tokens[b:b + 1], F)
        np.testing.assert_array_equal(f["topk"][b], ids[0], err_msg=f"{name}: top-F of sequence {b}")
        np.testing.assert_array_equal(f["topk_logits"][b].astype(np.float64), vals[0])


def test_fused_small_batch_nearly_all_accepted():
    # Draft = target up to tiny noise: almost every draft is accepted and the
    # bonus comes from p_t of row gamma, merged from chunk words (2 chunks).
    w = workloads.make_chain(3, 4, 40000, dtype="bf16", sigma=3.0, noise=0.02, temps="all1", gen_seed=61,
                             philox_seed=61)
    log("fused small batch, nearly all accepted")
    f, s = run_both(w, 6)
    ref, seqs = run_chain_oracle(w)
    compare_chain(f, ref, seqs, w.gamma, "fused nearly all accepted")
    assert (f["num_accepted"] == w.gamma).sum() >= 2
    for k in ("topk", "topk_logits"):
        np.testing.assert_array_equal(f[k], s[k], err_msg=f"nearly all accepted: {k}")


def test_fused_leaves_workspace_zero():
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    for i, (B, gamma, V) in enumerate([(300, 3, 5000), (8, 2, 9000), (260, 3, 20000), (260, 7, 3000), (2, 2, 40000)]):
        w = workloads.make_chain(B, gamma, V, dtype="bf16", temps="half0_half1", gen_seed=50 + i, philox_seed=i)
        log(f"fused shared workspace {i}: B={B} gamma={gamma} V={V}")
        d = chain_to_dev(w)
        out = binding.verify_topk(d["target"], d["draft"], d["tokens"], d["temperature"], 4, w.seed, 0,
                                  workspace=ws)
        torch.cuda.synchronize()
        gpu = {k: v.cpu().numpy() for k, v in out.items() if v is not None}
        ref, seqs = run_chain_oracle(w)
        compare_chain(gpu, ref, seqs, gamma, f"fused shared workspace {i}")
        assert int(ws.count_nonzero().item()) == 0
