"""Calls on two streams at once (MI355X).

Workgroups of one call wait for words published by other workgroups of the
same call. A chain call's waits are bounded and its finisher launch completes
whatever a wait left; a tree call's workgroups take their task numbers from a
ticket counter in the call's workspace, so a waiting task only waits for
tasks already claimed by running workgroups. Neither depends on what else the
GPU runs. Here a fused chain call and a tree
call run concurrently on two streams with separate workspaces (the binding's
default workspaces are per stream), repeatedly, and every outcome must match
the oracle with no -1 (a wait that ran out); then a ragged call and a cache
call, whose outcomes must equal the same calls made alone."""
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


def test_ragged_and_cache_on_two_streams():
    # The other two chain entry points, each with its own finisher launch,
    # concurrently on two streams; every concurrent outcome must equal the
    # same call made alone (the computation is deterministic), and neither
    # reports -1 or -2. Their parity with the oracle is tested elsewhere.
    rng = np.random.default_rng(303)
    B, G, V = 64, 6, 65536
    counts = rng.integers(0, G + 1, B)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    nd = int(offsets[-1])
    rt = torch.from_numpy(workloads.round_to_bf16(rng.normal(0, 3, (nd + B, V)).astype(np.float32))).cuda().bfloat16()
    rd = torch.from_numpy(workloads.round_to_bf16(rng.normal(0, 3, (nd, V)).astype(np.float32))).cuda().bfloat16()
    rtok = torch.from_numpy(rng.integers(0, V, nd).astype(np.int32)).cuda()
    rtemp = torch.from_numpy(np.where(np.arange(B) % 2 == 0, 0.0, 1.0).astype(np.float32)).cuda()
    roffs = torch.from_numpy(offsets).cuda()
    w = workloads.make_chain(48, 5, V, dtype="bf16", sigma=3.0, noise=1.0, temps="half0_half1", gen_seed=304,
                             philox_seed=304)
    dc = chain_to_dev(w)
    fan = [6, 5, 4, 3, 2, 2]

    def ragged():
        return binding.verify_ragged(rt, rd, roffs, rtok, rtemp, G, 303, 0)

    def cache():
        return binding.verify_cache(dc["target"], dc["draft"], dc["tokens"], dc["temperature"], fan, w.seed, 0,
                                    saguaro_C=0.5)

    def host(o):
        return {k: v.cpu().numpy() for k, v in o.items() if v is not None}

    alone_r, alone_c = host(ragged()), host(cache())
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(4):
        log(f"two streams (ragged, cache), round {rep}")
        with torch.cuda.stream(s1):
            o_r = ragged()
        with torch.cuda.stream(s2):
            o_c = cache()
        outs.append((o_r, o_c))
    torch.cuda.synchronize()
    assert np.all(alone_r["num_accepted"] >= 0) and np.all(alone_c["num_accepted"] >= 0)
    for rep, (o_r, o_c) in enumerate(outs):
        gr, gc = host(o_r), host(o_c)
        for k in alone_r:
            np.testing.assert_array_equal(gr[k], alone_r[k], err_msg=f"ragged {k}, round {rep}")
        for k in alone_c:
            np.testing.assert_array_equal(gc[k], alone_c[k], err_msg=f"cache {k}, round {rep}")
