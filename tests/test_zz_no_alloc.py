"""specv_verify_topk_noalloc (no workspace argument: the library's static
device array) against specv_verify_topk on the same inputs, through the
C-ABI: two calls in a row, the second with a smaller batch, gamma and
vocabulary; every output must be identical (the same kernels run on the same
inputs). The oracle parity of specv_verify_topk itself is tested elsewhere."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import chain_to_dev, log
from speculative_sampling_verification_04_amd import binding

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def test_noalloc_matches_verify_topk_on_two_calls():
    for B, gamma, V, F, seed in [(96, 6, 65536, 4, 31), (10, 3, 32000, 2, 32)]:
        assert binding.verify_topk_workspace_bytes(B, gamma, V) <= 4 << 20
        w = workloads.make_chain(B, gamma, V, dtype="bf16", sigma=3.0, noise=1.0, temps="half0_half1",
                                 gen_seed=seed, philox_seed=seed)
        d = chain_to_dev(w)
        log(f"noalloc: B={B} gamma={gamma} V={V} F={F}")
        ref = binding.verify_topk(d["target"], d["draft"], d["tokens"], d["temperature"], F, w.seed, 3)
        out = binding.verify_topk_noalloc(d["target"], d["draft"], d["tokens"], d["temperature"], F, w.seed, 3)
        torch.cuda.synchronize()
        for k in ref:
            np.testing.assert_array_equal(out[k].cpu().numpy(), ref[k].cpu().numpy(), err_msg=f"B={B}: {k}")
