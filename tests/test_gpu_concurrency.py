"""Calls on two streams at once (MI355X).

Workgroups of one call wait for words published by other workgroups of the
same call; they take their task numbers from a ticket counter in the call's
workspace, so a waiting task only waits for tasks already claimed by running
workgroups, whatever else the GPU runs. Here a fused chain call and a tree
call run concurrently on two streams with separate workspaces (the binding's
default workspaces are per stream), repeatedly, and every outcome must match
the oracle with no -1 (a wait that ran out)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import chain_to_dev, compare_chain, compare_tree, log, run_chain_oracle, run_tree_oracle, tree_to_dev
from speculative_sampling_verification_04_amd import binding

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def test_fused_and_tree_on_two_streams():
    w = workloads.make_chain(96, 6, 65536, dtype="bf16", sigma=4.0, noise=1.5, boost_frac=0.01, temps="half0_half1",
                             gen_seed=301, philox_seed=301)
    t = workloads.make_tree(24, 48, 65536, depth=5, branching=4, dtype="bf16", temps="all1", gen_seed=302,
                            philox_seed=302)
    dc, dt = chain_to_dev(w), tree_to_dev(t)
    ref_c, seqs_c = run_chain_oracle(w)
    ref_t, seqs_t = run_tree_oracle(t)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(4):
        log(f"two streams, round {rep}")
        with torch.cuda.stream(s1):
            oc = binding.verify_topk(dc["target"], dc["draft"], dc["tokens"], dc["temperature"], 4, w.seed, w.offset)
        with torch.cuda.stream(s2):
            ot = binding.tree_verify(dt["target"], dt["draft"], dt["parent"], dt["tokens"], dt["temperature"], t.seed,
                                     t.offset)
        outs.append((oc, ot))
    torch.cuda.synchronize()
    for rep, (oc, ot) in enumerate(outs):
        gc = {k: (v.cpu().numpy() if v is not None else None) for k, v in oc.items()}
        gt = {k: v.cpu().numpy() for k, v in ot.items()}
        assert np.all(gc["num_accepted"] >= 0) and np.all(gt["num_accepted"] >= 0), "a wait ran out"
        compare_chain(gc, ref_c, seqs_c, w.gamma, f"two streams chain {rep}")
        compare_tree(gt, ref_t, seqs_t, f"two streams tree {rep}")
