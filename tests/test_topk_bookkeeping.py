"""Host build of the top-K candidate list's bookkeeping (TopKAcc, in
csrc/specv_topk_list.hpp): tests/topk_list_host.cpp compiles the same header
with g++ against an emulated 64-lane wave and feeds it rows the way the
streaming loop does (all equal, strictly ascending, ascending by step,
descending, random, -inf/-0/+0), for U = 1, 2, 4 and 8 and every K. After every push and compaction the list must hold <= kCandCap entries,
and the keys gathered after the final compaction must fit topf_keys<K>() and
contain the K largest. A wider streaming shape must pass this before it runs
on a GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "speculative_sampling_verification_04_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_candidate_list_stays_within_its_bounds(tmp_path):
    exe = tmp_path / "topk_list_host"
    subprocess.run(["g++", "-std=c++20", "-O1", "-pthread", "-I", CSRC, os.path.join(HERE, "topk_list_host.cpp"),
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(r.stdout[-3000:])
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-2000:]
