"""Pins for the oracle's Philox4x32-10 generator and uniform mapping.

Two independent references:
* the known-answer vectors published with the Random123 library of Salmon et
  al. (SC'11) for philox4x32 with 10 rounds;
* rocRAND's philox4x32_10 engine, compiled on the host from its source header
  (/opt/rocm/include/rocrand/rocrand_philox4x32_10.h).
"""
import os
import random
import shutil
import subprocess

import pytest

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))

# (counter, key, output) -- Random123 known-answer vectors, philox4x32 10 rounds.
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_known_answer_vectors(ctr, key, out):
    assert philox.philox4x32_10(ctr, key) == out


def _rocrand_helper():
    inc = "/opt/rocm/include"
    if not os.path.exists(os.path.join(inc, "rocrand", "rocrand_philox4x32_10.h")):
        pytest.skip("rocRAND headers not installed")
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    bindir = os.path.join(HERE, "_bin")
    os.makedirs(bindir, exist_ok=True)
    exe = os.path.join(bindir, "rocrand_philox_kat")
    src = os.path.join(HERE, "rocrand_philox_kat.cpp")
    if not os.path.exists(exe) or os.path.getmtime(exe) < os.path.getmtime(src):
        subprocess.run([gxx, "-O1", "-x", "c++", "-D__HIP_PLATFORM_AMD__",
                        "-I", inc, src, "-o", exe], check=True,
                       capture_output=True)
    return exe


def test_matches_rocrand_engine():
    exe = _rocrand_helper()
    rng = random.Random(7)
    cases = []
    for _ in range(300):
        seed = rng.getrandbits(64)
        offset = rng.getrandbits(rng.choice([8, 32, 62]))
        b = rng.getrandbits(rng.choice([4, 16, 32]))
        tag = rng.randrange(4)
        j = rng.randrange(1 << rng.choice([3, 10, 26]))
        cases.append((seed, offset, b, tag, j))
    # Our layout -> rocRAND's (seed, subsequence, offset-in-words).
    lines = []
    for seed, offset, b, tag, j in cases:
        subsequence = b | (((tag << 24) | (j >> 2)) << 32)
        lines.append(f"{seed} {subsequence} {4 * offset + (j & 3)}")
    res = subprocess.run([exe], input="\n".join(lines) + "\n", text=True,
                         capture_output=True, check=True)
    words = [int(w, 16) for w in res.stdout.split()]
    assert len(words) == len(cases)
    for (seed, offset, b, tag, j), w in zip(cases, words):
        assert philox.stream_word(seed, offset, b, tag, j) == w


def test_uniform_mapping_edges():
    assert philox.word_to_uniform(0) == 2.0 ** -24
    assert philox.word_to_uniform(0xFF) == 2.0 ** -24          # low 8 bits ignored
    assert philox.word_to_uniform(0x100) == 2.0 * 2.0 ** -24
    assert philox.word_to_uniform(0xFFFFFFFF) == 1.0
    import numpy as np
    for w in (0, 1234567, 0x80000000, 0xFFFFFF00, 0xFFFFFFFF):
        u = philox.word_to_uniform(w)
        assert float(np.float32(u)) == u                     # exact in fp32
        assert 0.0 < u <= 1.0


def test_stream_layout_words_and_tags_differ():
    s = [philox.stream_word(5, 9, 3, tag, j) for tag in (0, 1) for j in range(8)]
    assert len(set(s)) == len(s)
    # Words 0..3 share one counter block, word 4 starts the next.
    blk = philox.philox4x32_10((9, 0, 3, 0), (5, 0))
    assert [philox.stream_word(5, 9, 3, 0, j) for j in range(4)] == list(blk)


def test_stream_rejects_out_of_layout():
    with pytest.raises(ValueError):
        philox.stream_word(0, 0, 0, 256, 0)
    with pytest.raises(ValueError):
        philox.stream_word(0, 0, 0, 0, 1 << 26)
