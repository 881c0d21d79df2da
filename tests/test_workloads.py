"""The seeded input generator: determinism, shapes, bf16 exactness, tree
structure (topological order, exact depth, branching limit)."""
import numpy as np
import torch

import workloads


def test_chain_is_deterministic_and_bf16_exact():
    a = workloads.make_chain(3, 2, 50, dtype="bf16", sigma=4, noise=1.5,
                             boost_frac=0.01, temps="half0_half1", gen_seed=5)
    b = workloads.make_chain(3, 2, 50, dtype="bf16", sigma=4, noise=1.5,
                             boost_frac=0.01, temps="half0_half1", gen_seed=5)
    np.testing.assert_array_equal(a.target, b.target)
    np.testing.assert_array_equal(a.draft_tokens, b.draft_tokens)
    assert a.target.shape == (3, 3, 50) and a.draft.shape == (3, 3, 50)
    for arr in (a.target, a.draft):
        back = torch.from_numpy(arr).to(torch.bfloat16).float().numpy()
        np.testing.assert_array_equal(back, arr)
    np.testing.assert_array_equal(a.temperature, [0, 1, 1])
    # Greedy drafts are the draft argmax.
    assert a.draft_tokens[0, 0] == int(np.argmax(a.draft[0, 0]))


def test_tree_structure():
    t = workloads.make_tree(8, 64, 40, depth=6, branching=4, gen_seed=3)
    for b in range(8):
        par = t.parent[b]
        assert par[0] == -1
        depth = [0] * 64
        kids = [0] * 64
        for n in range(1, 64):
            assert 0 <= par[n] < n
            depth[n] = depth[par[n]] + 1
            kids[par[n]] += 1
            assert 0 <= t.tokens[b, n] < 40
        assert max(depth) == 6 and max(kids) <= 4


def test_named_workloads_have_the_stated_shapes():
    w = workloads.make_workload("tiny_v16")
    assert (w.B, w.gamma, w.V, w.dtype, w.seed) == (1, 4, 16, "f32", 0)
    spec = workloads.WORKLOADS["v128256_bf16_b256_g8"]
    assert (spec["B"], spec["gamma"], spec["V"], spec["F"]) == (256, 8, 128256, 4)
    spec = workloads.WORKLOADS["tree_v152064_n64"]
    assert (spec["B"], spec["N"], spec["V"]) == (32, 64, 152064)
