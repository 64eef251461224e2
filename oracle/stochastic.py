"""Lossless stochastic acceptance of a drafted chain (speculative sampling), plain
numpy in float64.  TEST INFRASTRUCTURE ONLY (see oracle/__init__.py); it shares
nothing with the library.

The pages say only that the verification rule keeps the target's distribution
(DSpark, glossary "Speculative Decoding"); the rule itself is the standard
speculative-sampling rejection rule of the literature, restated here step by
step for a chain of request i with verify tokens 0..gamma (token 0 = root):
  - p_j = softmax(logits[o + j - 1] / temperature): the target's distribution
    of the token at position j (j = 1 .. gamma + 1);
  - q_j = draft_probs[o + j]: the drafter's distribution it drew draft x_j from;
  - for j = 1, 2, ...: accept x_j iff u[o + j] * q_j(x_j) < p_j(x_j), and stop
    at the first rejection;
  - n = accepted drafts; the next token y is drawn with w[i] by inverse CDF
    (the smallest v whose cumulative weight exceeds w * total) from
      max(0, p_{n+1} - q_{n+1})  if a draft was rejected (n < gamma),
      p_{gamma+1}                 if every draft was accepted;
    when the rejected position's residual has no mass (p == q), from p_{n+1};
  - accept_len = n + 1; accepted_path = 0..n; out_tokens = x_1..x_n, y.
Random numbers are inputs: u [T] and w [B], uniform in [0, 1)."""
from __future__ import annotations

import numpy as np


def target_probs(row_logits, temperature):
    x = np.asarray(row_logits, np.float64) / float(temperature)
    e = np.exp(x - x.max())
    return e / e.sum()


def inverse_cdf(weights, w):
    """Smallest index v with cumsum(weights)[v] > w * sum(weights)."""
    c = np.cumsum(np.asarray(weights, np.float64))
    target = float(w) * c[-1]
    v = int(np.searchsorted(c, target, side="right"))
    return min(v, len(c) - 1)


def accept_request(logits, draft_probs, draft, u, w, o, q, temperature):
    """One request (rows o .. o+q-1).  Returns (n, y, residual_used, target_row, cdf, target)."""
    gamma = q - 1
    n = 0
    for j in range(1, gamma + 1):
        p = target_probs(logits[o + j - 1], temperature)
        x = int(draft[o + j])
        if float(u[o + j]) * float(draft_probs[o + j][x]) < p[x]:
            n += 1
        else:
            break
    p = target_probs(logits[o + n], temperature)
    if n < gamma:
        r = np.maximum(0.0, p - np.asarray(draft_probs[o + n + 1], np.float64))
        if r.sum() <= 0.0:
            r = p
    else:
        r = p
    return n, inverse_cdf(r, w), r


def accept_stochastic(logits, draft_probs, draft_tokens, u, w, cu_q, temperature=1.0):
    """Returns (accept_len [B], accepted_path [T], out_tokens [T]); -1 past the path."""
    cu_q = np.asarray(cu_q, np.int64)
    B = len(cu_q) - 1
    T = int(cu_q[-1])
    acc = np.zeros(B, np.int32)
    path = np.full(T, -1, np.int32)
    toks = np.full(T, -1, np.int32)
    for i in range(B):
        o, q = int(cu_q[i]), int(cu_q[i + 1] - cu_q[i])
        if q == 0:
            continue
        n, y, _ = accept_request(logits, draft_probs, draft_tokens, u, w[i], o, q, temperature)
        acc[i] = n + 1
        path[o:o + n + 1] = np.arange(n + 1)
        toks[o:o + n] = np.asarray(draft_tokens[o + 1:o + n + 1])
        toks[o + n] = y
    return acc, path, toks


# ---------------------------------------------------------------------------
# Draft trees (SwiftSpec, "Tree-aware KV cache management": the verify tokens of
# a request form a tree; DSpark's glossary: the rule must keep the target's
# distribution).  The pages give no rule for trees; the plainest lossless one is
# speculative sampling applied to the siblings of a node one after another, each
# test against the target distribution left over by the siblings rejected before
# it (multi-draft rejection sampling).  For request i, node 0 = root, parent[o+k]
# in [0, k) for k >= 1:
#   at the current node c (c = 0 first) the distribution is p = softmax(row c / T);
#   its children are tested in index order; child k (draft x_k drawn from q_k =
#   draft_probs[o+k]) is accepted iff u[o+k] * q_k(x_k) < p'(x_k), p' being the
#   distribution in force (p at first);
#   on acceptance the walk moves to k (p' starts again from k's own row);
#   on rejection p' becomes max(0, p' - q_k) normalised, unless that has no mass
#   (then p' stays);
#   when no child of c is accepted, y is drawn with w[i] by inverse CDF from the
#   last residual max(0, p' - q_k) that had mass, or from p if none did.
# A chain is the special case of one child per node.  Outputs as for chains,
# except that accepted_path lists the node indices of the accepted path.
def accept_request_tree(logits, draft_probs, draft, parent, u, w, o, q, temperature):
    """One request of a tree.  Returns (path, y, weights, tests): path = node
    indices from the root, weights = the (unnormalised) draw weights, tests =
    (u*q(x), p'(x)) of every acceptance test made, in order."""
    c, path, tests = 0, [0], []
    while True:
        p = target_probs(logits[o + c], temperature)
        cur, last, moved = p, None, False
        for k in range(c + 1, q):
            if int(parent[o + k]) != c:
                continue
            x = int(draft[o + k])
            qk = np.asarray(draft_probs[o + k], np.float64)
            lhs = float(u[o + k]) * float(qk[x])
            tests.append((lhs, float(cur[x])))
            if lhs < cur[x]:
                path.append(k)
                c, moved = k, True
                break
            r = np.maximum(0.0, cur - qk)
            if r.sum() > 0.0:
                last = r
                cur = r / r.sum()
        if not moved:
            weights = p if last is None else last
            return path, inverse_cdf(weights, w), weights, tests


def accept_stochastic_tree(logits, draft_probs, draft_tokens, tree_parent, u, w, cu_q, temperature=1.0):
    """Returns (accept_len [B], accepted_path [T], out_tokens [T]); -1 past the path."""
    cu_q = np.asarray(cu_q, np.int64)
    B = len(cu_q) - 1
    T = int(cu_q[-1])
    acc = np.zeros(B, np.int32)
    path = np.full(T, -1, np.int32)
    toks = np.full(T, -1, np.int32)
    for i in range(B):
        o, q = int(cu_q[i]), int(cu_q[i + 1] - cu_q[i])
        if q == 0:
            continue
        pth, y, _, _ = accept_request_tree(logits, draft_probs, draft_tokens, tree_parent, u, w[i], o, q,
                                           temperature)
        n = len(pth) - 1
        acc[i] = n + 1
        path[o:o + n + 1] = pth
        toks[o:o + n] = [int(draft_tokens[o + k]) for k in pth[1:]]
        toks[o + n] = y
    return acc, path, toks
