"""The failure path of the kernels' bounded waits, forced from the host.

Workgroups wait for each other's published words (row statistics, tile sums,
top-F keys, a tree's pass totals); every wait is bounded and a wait that runs
out makes its sequence or tree report -1. Here the bound is set to one tick of
the 100 MHz clock for one call: the call must still return, and every
sequence or tree must either report -1 or give the oracle's outcome. The
bound is then restored and the same call, on the same workspace (which the
failed call may have left with words written after their readers gave up:
every call tags its words with its own epoch, so those never count), must
match the oracle again and leave the workspace zero."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import (chain_to_dev, compare_chain, compare_tree, log, run_chain_oracle, run_tree_oracle,
                        tree_to_dev)
from speculative_sampling_verification_04_amd import binding

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()
    yield
    binding.set_wait_bound(0)


def with_short_waits(call):
    binding.set_wait_bound(1)
    try:
        out = call()
        torch.cuda.synchronize()
    finally:
        binding.set_wait_bound(0)
    return {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}


def check_chain_or_failed(gpu, ref, seqs, name):
    failed = [b for b in seqs if gpu["num_accepted"][b] == -1]
    for n, b in enumerate(seqs):
        if b in failed or ref["near_tie"][n]:
            continue
        assert gpu["num_accepted"][b] == ref["num_accepted"][n], f"{name}: sequence {b}"
        np.testing.assert_array_equal(gpu["tokens"][b], ref["tokens"][n], err_msg=f"{name}: sequence {b}")
    log(f"{name}: {len(failed)} of {len(seqs)} sequences reported a wait that ran out")
    assert failed, f"{name}: no wait ran out: the failure path was not exercised"


@pytest.mark.parametrize("B,gamma,V,entry", [(64, 4, 20000, "verify"), (3, 4, 40000, "verify_topk")])
def test_chain_waits_that_run_out_report_minus_one(B, gamma, V, entry):
    w = workloads.make_chain(B, gamma, V, dtype="bf16", sigma=3.0, noise=1.0, temps="half0_half1",
                             gen_seed=71 + B, philox_seed=71)
    d = chain_to_dev(w)
    if entry == "verify":
        ws = torch.zeros(binding.verify_workspace_bytes(B, gamma, V), dtype=torch.uint8, device="cuda")
        call = lambda: binding.verify(d["target"], d["draft"], d["tokens"], d["temperature"], w.seed, 0, workspace=ws)
    else:
        ws = torch.zeros(binding.verify_topk_workspace_bytes(B, gamma, V), dtype=torch.uint8, device="cuda")
        call = lambda: binding.verify_topk(d["target"], d["draft"], d["tokens"], d["temperature"], 4, w.seed, 0,
                                           workspace=ws)
    log(f"short waits: {entry} B={B} gamma={gamma} V={V}")
    ref, seqs = run_chain_oracle(w)
    check_chain_or_failed(with_short_waits(call), ref, seqs, f"{entry} short waits")
    out = call()
    torch.cuda.synchronize()
    gpu = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
    compare_chain(gpu, ref, seqs, gamma, f"{entry} after short waits")
    assert int(ws.count_nonzero().item()) == 0


def test_tree_waits_that_run_out_report_minus_one():
    t = workloads.make_tree(6, 40, 20000, depth=5, branching=4, dtype="bf16", temps="half0_half1",
                            gen_seed=73, philox_seed=73)
    d = tree_to_dev(t)
    ws = torch.zeros(binding.tree_workspace_bytes(t.B, t.N, t.V), dtype=torch.uint8, device="cuda")
    call = lambda: binding.tree_verify(d["target"], d["draft"], d["parent"], d["tokens"], d["temperature"], t.seed,
                                       0, workspace=ws)
    log("short waits: tree B=6 N=40 V=20000")
    ref, seqs = run_tree_oracle(t)
    gpu = with_short_waits(call)
    failed = [b for b in seqs if gpu["num_accepted"][b] == -1]
    for n, b in enumerate(seqs):
        if b in failed or ref["near_tie"][n]:
            continue
        assert gpu["num_accepted"][b] == ref["num_accepted"][n] and gpu["bonus"][b] == ref["bonus"][n], f"tree {b}"
    log(f"tree short waits: {len(failed)} of {len(seqs)} trees reported a wait that ran out")
    assert failed, "tree: no wait ran out: the failure path was not exercised"
    out = call()
    torch.cuda.synchronize()
    compare_tree({k: v.cpu().numpy() for k, v in out.items()}, ref, seqs, "tree after short waits")
    assert int(ws.count_nonzero().item()) == 0


def test_default_workspace_after_waits_ran_out():
    # The binding's own workspace (one per device and stream): a call whose
    # waits ran out, then ordinary calls on the same default workspace, which
    # must match the oracle (no zeroing by the caller).
    w = workloads.make_chain(48, 5, 30000, dtype="bf16", sigma=3.0, noise=1.0, temps="half0_half1",
                             gen_seed=75, philox_seed=75)
    d = chain_to_dev(w)
    call = lambda: binding.verify_topk(d["target"], d["draft"], d["tokens"], d["temperature"], 3, w.seed, 0)
    log("short waits on the default workspace, then ordinary calls")
    ref, seqs = run_chain_oracle(w)
    check_chain_or_failed(with_short_waits(call), ref, seqs, "default workspace short waits")
    for rep in range(2):
        out = call()
        torch.cuda.synchronize()
        gpu = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
        compare_chain(gpu, ref, seqs, w.gamma, f"default workspace after short waits ({rep})")
