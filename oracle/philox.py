"""Philox4x32-10 and the uniform stream used by verification (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages treat the accept uniforms u_i and the bonus uniform v as given inputs
("take u ~ U(0,1)", Lecture 5: Speculative Decoding and SpecInfer, section 2.2;
vLLM passes ``uniform_probs`` in, Speculative Decoding (dl-note), Appendix
"Implementation Details"). This build draws them from a counter-based generator
so that any call can be replayed from (seed, offset). The generator is Philox4x32
with 10 rounds as published by Salmon, Moraes, Dror and Shaw ("Parallel random
numbers: as easy as 1, 2, 3", SC'11), written here in plain Python integers.

Stream layout (a reading the pages leave open):
    key     = (seed mod 2^32, seed >> 32)
    counter = (offset mod 2^32, offset >> 32, b, (tag << 24) | (j >> 2))
    word    = output[j & 3]
    U(word) = ((word >> 8) + 1) * 2^-24, a value in (0, 1] exact in fp32.

Tags: 0 = chain verification (j = position i for u_i, j = gamma for v),
      1 = tree verification  (j = child node id for its test, j = N for v).
"""

MASK32 = 0xFFFFFFFF

# Round multipliers and Weyl key increments of Philox4x32 (Salmon et al., SC'11).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
PHILOX_ROUNDS = 10

TAG_CHAIN = 0
TAG_TREE = 1


def philox_round(ctr, key):
    """One Philox4x32 S-box/P-box round: two 32x32->64 products, hi words xored
    with the other counter words and the key, then the word permutation."""
    c0, c1, c2, c3 = ctr
    prod0 = PHILOX_M0 * c0
    prod1 = PHILOX_M1 * c2
    hi0, lo0 = prod0 >> 32, prod0 & MASK32
    hi1, lo1 = prod1 >> 32, prod1 & MASK32
    return (hi1 ^ c1 ^ key[0], lo1, hi0 ^ c3 ^ key[1], lo0)


def philox4x32_10(ctr, key):
    """Ten rounds; the key is bumped by the Weyl constants between rounds."""
    ctr = tuple(int(c) & MASK32 for c in ctr)
    k0, k1 = int(key[0]) & MASK32, int(key[1]) & MASK32
    for r in range(PHILOX_ROUNDS):
        if r > 0:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        ctr = philox_round(ctr, (k0, k1))
    return ctr


def stream_word(seed, offset, b, tag, j):
    """The 32-bit word for (sequence b, tag, index j) of stream (seed, offset)."""
    if not (0 <= tag < 256 and 0 <= j < (1 << 26) and 0 <= b <= MASK32):
        raise ValueError("tag, j or b out of the stream layout's range")
    key = (seed & MASK32, (seed >> 32) & MASK32)
    ctr = (offset & MASK32, (offset >> 32) & MASK32, b, (tag << 24) | (j >> 2))
    return philox4x32_10(ctr, key)[j & 3]


def word_to_uniform(word):
    """Top 24 bits plus one, scaled by 2^-24: never 0, reaches exactly 1."""
    return ((int(word) >> 8) + 1) * 2.0 ** -24


def uniform(seed, offset, b, tag, j):
    return word_to_uniform(stream_word(seed, offset, b, tag, j))


def chain_uniforms(seed, offset, b, gamma):
    """(u_0..u_{gamma-1}, v) for one sequence of chain verification."""
    u = [uniform(seed, offset, b, TAG_CHAIN, i) for i in range(gamma)]
    v = uniform(seed, offset, b, TAG_CHAIN, gamma)
    return u, v


def tree_uniforms(seed, offset, b, n_nodes):
    """(u[c] for c in 0..N-1, v) for one tree; u[0] is never used (the root is
    not tested)."""
    u = [uniform(seed, offset, b, TAG_TREE, c) for c in range(n_nodes)]
    v = uniform(seed, offset, b, TAG_TREE, n_nodes)
    return u, v
