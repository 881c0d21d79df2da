"""Chain calls at the batch sizes where placement changes form (MI355X).

Every chain workgroup first reads the batch's temperatures to find its task
(T > 0 sequences first). Up to 256 sequences each lane of the reading wave
issues all of its loads at once and the workgroup keeps the temperatures
(and, in a ragged call, the offsets) in LDS; above 256 it reads them in a
loop of 64 at a time and a task reads its own values from memory. Both forms
must give the oracle's outcome: here at 255, 256 and 257 sequences, for
specv_verify, specv_verify_topk, specv_verify_cache and specv_verify_ragged
(with and without draft logits), with mixed temperatures so that the order
of the sequences is not the index order."""
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


def host(out):
    return {k: v.cpu().numpy() for k, v in out.items() if v is not None}


@pytest.mark.parametrize("B", [255, 256, 257])
def test_verify_and_fused_at_the_placement_edge(B):
    w = workloads.make_chain(B, 3, 700, dtype="bf16", sigma=3.0, noise=1.0, temps="half0_half1",
                             gen_seed=1200 + B, philox_seed=B)
    d = chain_to_dev(w)
    ref, seqs = run_chain_oracle(w)
    log(f"placement edge: verify and verify_topk, B={B}")
    v = host(binding.verify(d["target"], d["draft"], d["tokens"], d["temperature"], w.seed, w.offset))
    f = host(binding.verify_topk(d["target"], d["draft"], d["tokens"], d["temperature"], 4, w.seed, w.offset))
    torch.cuda.synchronize()
    compare_chain(v, ref, seqs, w.gamma, f"verify B={B}")
    compare_chain(f, ref, seqs, w.gamma, f"verify_topk B={B}")
    ids, _ = oracle_topf_all(("edge", B), w.draft, w.draft_tokens, 4)
    np.testing.assert_array_equal(f["topk"], ids, err_msg=f"verify_topk B={B}: top-F")


@pytest.mark.parametrize("B", [256, 257])
def test_cache_at_the_placement_edge(B):
    fan = (3, 2, 2)
    w = workloads.make_chain(B, 2, 600, dtype="f32", sigma=3.0, noise=1.0, temps="half0_half1",
                             gen_seed=1300 + B, philox_seed=B, F=max(fan))
    d = chain_to_dev(w)
    log(f"placement edge: verify_cache, B={B}")
    gpu = host(binding.verify_cache(d["target"], d["draft"], d["tokens"], d["temperature"], fan, w.seed, w.offset,
                                    saguaro_C=0.5, lenience=0.9))
    ref = oracle.ssd.verify_cached_batch(w.target.astype(np.float64), w.draft.astype(np.float64), w.draft_tokens,
                                         w.temperature, w.seed, w.offset, fan, C=float(np.float32(0.5)),
                                         lenience=float(np.float32(0.9)))
    compare_chain(gpu, ref, list(range(B)), w.gamma, f"verify_cache B={B}")
    np.testing.assert_array_equal(gpu["topk"][:, :, :max(fan)], ref["topk"], err_msg=f"verify_cache B={B}: candidates")


@pytest.mark.parametrize("B", [255, 256, 257])
@pytest.mark.parametrize("with_draft", [True, False])
def test_ragged_at_the_placement_edge(B, with_draft):
    from test_gpu_ragged import compare, make_ragged, run
    r = make_ragged(B, 3, 600, "bf16", "mixed", 1400 + B)
    log(f"placement edge: verify_ragged, B={B}, with_draft={with_draft}")
    gpu, ref = run(r, with_draft)
    assert compare(gpu, ref, r, f"ragged B={B} with_draft={with_draft}") <= max(1, B // 10)
