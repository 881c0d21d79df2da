"""Exact enumeration over the uniform grid.

The generator's uniforms take exactly 2^24 values, (k + 1) * 2^-24 for
k = 0 .. 2^24 - 1, each with probability 2^-24. For a decision that is
monotone in the uniform (accept iff u <= ratio; the inverse-CDF index grows
with v), the number of grid values leading to each outcome can be found
exactly by binary search, calling the function under test as a black box.
"""

GRID = 1 << 24


def grid_value(k):
    return (k + 1) * 2.0 ** -24


def first_true(pred, lo=0, hi=GRID):
    """Smallest k in [lo, hi) with pred(k) true, assuming pred is monotone
    false -> true; returns hi when pred is never true."""
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


def count_accepting(accepts):
    """accepts(u) is true for u below some threshold and false above; return
    the number of grid values for which it is true."""
    return first_true(lambda k: not accepts(grid_value(k)))


def bucket_counts(index_of, n_out):
    """index_of(v) is nondecreasing in v with values in [0, n_out); return how
    many grid values map to each index."""
    edges = [first_true(lambda k, j=j: index_of(grid_value(k)) >= j)
             for j in range(n_out + 1)]
    edges[0] = 0
    return [edges[j + 1] - edges[j] for j in range(n_out)]
