"""The kernels' bounded waits, run out on purpose from the host.

Workgroups wait for each other's published words (row statistics, tile sums,
top-F keys, a tree's pass totals), and every wait is bounded. Here the bound
is set to one tick of the 100 MHz clock for one call, so that waits run out.
A chain launch (verify, verify_topk, verify_cache, verify_ragged) then leaves the sequences whose bonus
workgroups gave up to its finisher launch, which completes them: every
sequence must still give the oracle's outcome, and the workspace header's
count of sequences completed that way must have grown. A tree launch has no
finisher (its walkers need each other): a tree whose wait ran out reports -1,
the others give the oracle's outcome. The bound is then restored and the
same call on the same workspace must match the oracle again and leave the
workspace zero (but for that count). A guard region after the workspace
checks that no call writes past it."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_common import (chain_to_dev, compare_chain, compare_tree, log, run_chain_oracle, run_tree_oracle, to_dev,
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


def deferred_count(ws):
    return int(ws[8:16].view(torch.int64).item())


GUARD = 4096


def guarded_workspace(nbytes):
    """A zeroed workspace of nbytes and, right after it in the same buffer, a
    guard region of 0xAB bytes (returned too): no call may write past its
    workspace."""
    buf = torch.zeros(nbytes + GUARD, dtype=torch.uint8, device="cuda")
    buf[nbytes:] = 0xAB
    return buf[:nbytes], buf[nbytes:]


def assert_guard(guard, what):
    torch.cuda.synchronize()
    assert bool((guard == 0xAB).all().item()), f"{what}: memory past the workspace was written"


@pytest.mark.parametrize("B,gamma,V,entry", [(64, 4, 20000, "verify"), (3, 4, 40000, "verify_topk"),
                                             (48, 5, 30000, "verify_topk")])
def test_chain_waits_that_run_out_are_finished(B, gamma, V, entry):
    w = workloads.make_chain(B, gamma, V, dtype="bf16", sigma=3.0, noise=1.0, temps="half0_half1",
                             gen_seed=71 + B, philox_seed=71)
    d = chain_to_dev(w)
    if entry == "verify":
        ws, guard = guarded_workspace(binding.verify_workspace_bytes(B, gamma, V))
        call = lambda: binding.verify(d["target"], d["draft"], d["tokens"], d["temperature"], w.seed, 0, workspace=ws)
    else:
        ws, guard = guarded_workspace(binding.verify_topk_workspace_bytes(B, gamma, V))
        call = lambda: binding.verify_topk(d["target"], d["draft"], d["tokens"], d["temperature"], 4, w.seed, 0,
                                           workspace=ws)
    log(f"short waits: {entry} B={B} gamma={gamma} V={V}")
    ref, seqs = run_chain_oracle(w)
    gpu = with_short_waits(call)
    n = deferred_count(ws)
    log(f"{entry} short waits: the finisher completed {n} of {B} sequences")
    assert n > 0, f"{entry}: no wait ran out: the deferral path was not exercised"
    assert_guard(guard, f"{entry} short waits")
    compare_chain(gpu, ref, seqs, gamma, f"{entry} short waits")
    ws[8:16].zero_()
    out = call()
    torch.cuda.synchronize()
    again = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
    compare_chain(again, ref, seqs, gamma, f"{entry} after short waits")
    for k in ("tokens", "num_accepted", "probs", "bonus_mass", "topk", "topk_logits"):
        if k in gpu:   # the finisher's outcome is the main launch's, bit for bit
            np.testing.assert_array_equal(gpu[k], again[k], err_msg=f"{entry}: {k}")
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
    # must all match the oracle (no zeroing by the caller).
    w = workloads.make_chain(48, 5, 30000, dtype="bf16", sigma=3.0, noise=1.0, temps="half0_half1",
                             gen_seed=75, philox_seed=75)
    d = chain_to_dev(w)
    call = lambda: binding.verify_topk(d["target"], d["draft"], d["tokens"], d["temperature"], 3, w.seed, 0)
    log("short waits on the default workspace, then ordinary calls")
    ref, seqs = run_chain_oracle(w)
    compare_chain(with_short_waits(call), ref, seqs, w.gamma, "default workspace short waits")
    for rep in range(2):
        out = call()
        torch.cuda.synchronize()
        gpu = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
        compare_chain(gpu, ref, seqs, w.gamma, f"default workspace after short waits ({rep})")


@pytest.mark.parametrize("with_draft", [True, False])
def test_ragged_waits_that_run_out_are_finished(with_draft):
    # Ragged batches, sequence 5 with offsets that break the contract (its
    # rows publish skipped values and its finisher work only zeroes them).
    from test_gpu_ragged import compare, make_ragged
    r = make_ragged(40, 5, 20000, "bf16", "mixed", 77)
    offsets = r["offsets"].copy()
    d = {k: (to_dev(r[k], "bf16", "cuda") if k in ("target", "draft") else torch.from_numpy(r[k]).to("cuda"))
         for k in ("target", "draft", "tokens", "temperature")}
    bad = offsets.copy()
    bad[6] = bad[5] - 1                       # sequence 5: decreasing offsets
    ws, guard = guarded_workspace(binding.verify_ragged_workspace_bytes(40, 5, 20000, with_draft))
    draft = d["draft"] if with_draft else None

    def call(offs):
        return binding.verify_ragged(d["target"], draft, torch.from_numpy(offs).to("cuda"), d["tokens"],
                                     d["temperature"], r["G"], r["seed"], 0, workspace=ws)

    log(f"short waits: ragged B=40 G=5 V=20000 with_draft={with_draft}")
    gpu = with_short_waits(lambda: call(offsets))
    assert deferred_count(ws) > 0, "ragged: no wait ran out: the deferral path was not exercised"
    assert_guard(guard, "ragged short waits")
    ref = oracle.ragged.verify_ragged_batch(r["target"], r["draft"] if with_draft else None, offsets, r["tokens"],
                                            r["temperature"], r["seed"], 0, r["G"])
    compare(gpu, ref, r, "ragged short waits")
    bad_out = with_short_waits(lambda: call(bad))
    assert_guard(guard, "ragged short waits, bad offsets")
    assert bad_out["num_accepted"][5] == -2
    ws[8:16].zero_()
    out = call(offsets)
    torch.cuda.synchronize()
    again = {k: v.cpu().numpy() for k, v in out.items() if v is not None}
    for k in again:
        np.testing.assert_array_equal(gpu[k], again[k], err_msg=f"ragged: {k}")
    assert int(ws.count_nonzero().item()) == 0


@pytest.mark.parametrize("B,gamma,V", [(3, 4, 40000), (48, 5, 30000)])
def test_cache_waits_that_run_out_are_finished(B, gamma, V):
    # specv_verify_cache: with chunked rows (B = 3) the resolve waits for the
    # cache pairs that each draft row's chunk merge publishes, so a merge that
    # gives up defers the resolve too and the finisher runs both, merges
    # first; with one chunk per row (B = 48) the draft rows publish them.
    w = workloads.make_chain(B, gamma, V, dtype="bf16", sigma=3.0, noise=1.0, temps="half0_half1",
                             gen_seed=91 + B, philox_seed=91)
    d = chain_to_dev(w)
    fan = [5, 4, 3, 2, 2, 1][:gamma + 1]
    ws, guard = guarded_workspace(binding.verify_cache_workspace_bytes(B, gamma, V))
    call = lambda: binding.verify_cache(d["target"], d["draft"], d["tokens"], d["temperature"], fan, w.seed, 0,
                                        saguaro_C=0.5, workspace=ws)
    log(f"short waits: verify_cache B={B} gamma={gamma} V={V}")
    short = with_short_waits(call)
    n = deferred_count(ws)
    log(f"verify_cache short waits: the finisher completed {n} of {B} sequences")
    assert n > 0, "verify_cache: no wait ran out: the deferral path was not exercised"
    assert_guard(guard, "verify_cache short waits")
    ws[8:16].zero_()
    out = call()
    torch.cuda.synchronize()
    again = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
    for k in again:
        if again[k] is not None:
            np.testing.assert_array_equal(short[k], again[k], err_msg=f"verify_cache: {k}")
    assert int(ws.count_nonzero().item()) == 0


def test_finisher_with_most_sequences_deferred():
    # 40 sequences over long rows: every workgroup of the call is resident at
    # once, so with waits of one tick nearly every bonus task gives up and the
    # finisher completes nearly every sequence, those of slots 31 and up
    # included (the finisher reads each wave's 64-bit mask of deferred slots;
    # a mask widened with a sign would name slots past the batch). Outputs
    # must equal the oracle's and nothing past the workspace may be written.
    B, gamma, V = 40, 4, 128256
    w = workloads.make_chain(B, gamma, V, dtype="bf16", sigma=3.0, noise=1.0, temps="half0_half1",
                             gen_seed=41, philox_seed=41)
    d = chain_to_dev(w)
    ref, seqs = run_chain_oracle(w)
    for entry in ("verify", "verify_topk"):
        if entry == "verify":
            ws, guard = guarded_workspace(binding.verify_workspace_bytes(B, gamma, V))
            call = lambda: binding.verify(d["target"], d["draft"], d["tokens"], d["temperature"], w.seed, 0,
                                          workspace=ws)
        else:
            ws, guard = guarded_workspace(binding.verify_topk_workspace_bytes(B, gamma, V))
            call = lambda: binding.verify_topk(d["target"], d["draft"], d["tokens"], d["temperature"], 4, w.seed, 0,
                                               workspace=ws)
        log(f"most deferred: {entry} B={B} gamma={gamma} V={V}")
        gpu = with_short_waits(call)
        n = deferred_count(ws)
        log(f"{entry}: the finisher completed {n} of {B} sequences")
        assert n > 0
        assert_guard(guard, f"{entry}, most deferred")
        compare_chain(gpu, ref, seqs, gamma, f"{entry}, most deferred")
        ws[8:16].zero_()
        assert int(ws.count_nonzero().item()) == 0
