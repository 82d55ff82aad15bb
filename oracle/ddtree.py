"""DDTree draft-tree construction (test infrastructure only).

"Accelerating Speculative Decoding with Block Diffusion Draft Trees" notes:

* §4.2 (Proposition 2): with a factorised draft q(u) = prod_i q_i(u_i) every
  strict descendant scores below its ancestors, so the B most probable
  prefixes form a prefix-closed tree, and that set is the optimal tree.
* §4.3 (Lemma 1): some optimal tree uses only each depth's top-K tokens,
  K = min(B, |V|).
* §5 (Algorithm 1): prefixes are tuples of per-depth ranks; a max-heap keyed
  by the prefix score sigma (the sum of log q over its ranks) starts with
  (rank 1 at depth 1); each pop adds the popped prefix to the tree and pushes
  its next sibling (last rank + 1, score - log q^(r) + log q^(r+1)) when that
  rank exists and its first child (rank 1 at the next depth, score + log q^(1)
  of that depth) when the depth is below L; B pops give the top-B prefixes in
  descending score order (§5.3).

Readings where the notes are open (the same ones the input generator of the
DDTree workloads follows):

* A depth's draft distribution is the softmax of its logits truncated to the
  top K tokens and renormalised over them: log q^(r) = z_(r) - lse, lse =
  z_(1) + log(sum_r exp(z_(r) - z_(1))) over the K kept logits, the sum taken
  in rank order.
* The top-K order is by logit, descending, then by token id, ascending.
* Equal scores pop in increasing rank-tuple order (a tuple before its
  extensions), as a heap of (-score, ranks) pairs does.
* Node i of the output is the i-th popped prefix; its parent is the node of
  the prefix without its last rank (-1 at depth 1) and its token the
  last-ranked token of its depth.

All in float64 with the logits widened exactly.
"""

import heapq
import math
from typing import List, Tuple

import numpy as np


def depth_topk(z_row, K: int) -> Tuple[np.ndarray, np.ndarray]:
    """(token ids, log q) of one depth's top-K, in rank order."""
    z = np.asarray(z_row, dtype=np.float64)
    order = np.lexsort((np.arange(z.size), -z))[:K]   # by -z, then by index
    zz = z[order]
    s = 0.0
    for v in zz:                                     # rank order
        s += math.exp(v - zz[0])
    lse = zz[0] + math.log(s)
    return order.astype(np.int64), zz - lse


def best_first(logq, budget: int) -> List[Tuple[int, ...]]:
    """Algorithm 1 over per-depth log q rows (each in rank order, length K):
    the popped rank tuples (0-based ranks), in pop order."""
    L = len(logq)
    heap = [(-logq[0][0], (0,))]
    popped: List[Tuple[int, ...]] = []
    while heap and len(popped) < budget:
        negs, ranks = heapq.heappop(heap)
        popped.append(ranks)
        d = len(ranks) - 1
        s = -negs
        r = ranks[-1]
        if r + 1 < len(logq[d]):
            heapq.heappush(heap, (-(s - logq[d][r] + logq[d][r + 1]), ranks[:-1] + (r + 1,)))
        if d + 1 < L:
            heapq.heappush(heap, (-(s + logq[d + 1][0]), ranks + (0,)))
    return popped


def build_tree(draft_logits, budget: int):
    """Parents and tokens (pop order) of one request's DDTree tree.

    draft_logits: [L, V] the drafter's per-depth logits."""
    z = np.asarray(draft_logits)
    L, V = z.shape
    K = min(budget, V)
    toks, logq = zip(*(depth_topk(z[d], K) for d in range(L)))
    popped = best_first(logq, budget)
    node_of = {ranks: i for i, ranks in enumerate(popped)}
    parents = [-1 if len(r) == 1 else node_of[r[:-1]] for r in popped]
    tokens = [int(toks[len(r) - 1][r[-1]]) for r in popped]
    return np.asarray(parents, dtype=np.int32), np.asarray(tokens, dtype=np.int32)
