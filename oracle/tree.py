"""Token-tree verification: VerifyGreedy and multi-step speculative sampling.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: Lecture 5: Speculative Decoding and SpecInfer --
  sec. 6.2 (token tree: node u carries token t_u; the root is the last
           committed token),
  sec. 6.4 (VerifyGreedy: from the root, move to the child whose token is the
           target argmax at the current node, else emit that argmax;
           MSS: test the children in turn, accepting child j with probability
           min(1, p_j(x_j)/q(x_j)); after each rejection replace the target
           distribution by norm(max(0, p_j - q)); if every child is rejected,
           sample from the last residual. Children must be independent samples
           from q; duplicates stay separate nodes),
  sec. 2.2 for the single-candidate rule that MSS generalises.

Layout of one tree (a reading; also in the design doc): nodes 0..N-1 in topological
order, parent[0] = -1 and parent[n] < n; tokens[n] is node n's token (tokens[0]
is unused). target[n] holds the target logits after the path to node n (the
distribution of the token that follows n); draft[n] holds the draft logits at
node n, from which n's children were sampled, so q = softmax(draft[n]/T) for
every child of n. Children are tested in increasing node id. A walk that ends
on a leaf samples the bonus from p at that leaf. Uniforms: child c is tested
with u[c]; the bonus uses v.
"""

from dataclasses import dataclass, field

import numpy as np

from .sampling import (NEAR_TIE, accept, accept_margin, greedy_token,
                       inverse_cdf, prob_at, tempered_probs)


def children_of(parent, node):
    return [c for c in range(len(parent)) if parent[c] == node]


def mss_residual(r, q):
    """r <- norm(max(0, r - q)) [L5 sec. 6.4]. If the clipped mass is 0 (r <= q
    everywhere, hence r = q), r is kept."""
    w = np.maximum(r - q, 0.0)
    s = np.sum(w)
    if not s > 0:
        return r
    return w / s


def mss_node(p, q, child_tokens, u_children, v):
    """One MSS step at a node with target distribution p and draft q.

    child_tokens / u_children: the children's tokens and accept uniforms, in
    test order. Returns (index of the accepted child or None, bonus token or
    None, margins of the decisions taken)."""
    r = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    margins = []
    for j, t in enumerate(child_tokens):
        r_t, q_t = prob_at(r, t), prob_at(q, t)
        margins.append(accept_margin(r_t, q_t, u_children[j]))
        if accept(r_t, q_t, u_children[j]):
            return j, None, margins
        r = mss_residual(r, q)
    bonus, _, m = inverse_cdf(r, v)
    margins.append(m)
    return None, bonus, margins


@dataclass
class TreeOutcome:
    path: list                  # accepted node ids, root excluded, in order
    bonus: int
    near_tie: bool
    margins: list = field(default_factory=list)

    @property
    def num_accepted(self):
        return len(self.path)


def verify_tree(target, draft, parent, tokens, T, u, v):
    """Walk one tree from the root [L5 sec. 6.4]; greedy when T = 0."""
    target = np.asarray(target, dtype=np.float64)
    node, path, margins = 0, [], []
    while True:
        kids = children_of(parent, node)
        if T == 0:
            g = greedy_token(target[node])
            match = [c for c in kids if int(tokens[c]) == g]
            if not match:
                return TreeOutcome(path, g, False, [])
            node = match[0]
            path.append(node)
            continue
        p = tempered_probs(target[node], T)
        if not kids:
            bonus, _, m = inverse_cdf(p, v)
            margins.append(m)
            break
        q = tempered_probs(np.asarray(draft[node], dtype=np.float64), T)
        j, bonus, ms = mss_node(p, q, [int(tokens[c]) for c in kids],
                                [u[c] for c in kids], v)
        margins.extend(ms)
        if j is None:
            break
        node = kids[j]
        path.append(node)
    near = any(mg <= NEAR_TIE for mg in margins)
    return TreeOutcome(path, bonus, near, margins)


def verify_tree_batch(target, draft, parent, tokens, temperature, seed, offset):
    """target/draft [B, N, V], parent/tokens [B, N], temperature [B]; uniforms
    from the Philox stream (tag 1). Returns path [B, N] (-1 padded),
    num_accepted [B], bonus [B], near_tie [B]."""
    from .philox import tree_uniforms

    B, N = np.asarray(parent).shape
    path = np.full((B, N), -1, dtype=np.int64)
    nacc = np.zeros(B, dtype=np.int64)
    bonus = np.zeros(B, dtype=np.int64)
    near = np.zeros(B, dtype=bool)
    for b in range(B):
        u, v = tree_uniforms(seed, offset, b, N)
        res = verify_tree(target[b], draft[b], list(parent[b]), list(tokens[b]),
                          float(temperature[b]), u, v)
        path[b, :len(res.path)] = res.path
        nacc[b] = res.num_accepted
        bonus[b] = res.bonus
        near[b] = res.near_tie
    return dict(path=path, num_accepted=nacc, bonus=bonus, near_tie=near)
