"""Greedy acceptance: row argmax and the sequential walk (test infrastructure only).

What it follows:

* Decoding-extensions glossary, three-part semantics experiment (verify_tree):
  walk the target's next tokens depth by depth; at each depth keep only the
  candidates that extend the accepted prefix with the target token; stop at
  the first depth with no match; the accepted tokens are committed.
* "02 · Token Tree 与 Tree Attention", section 4: from the root, compare each
  child's token id with the target's choice (greedy); an accepted child
  becomes the current node; when no child matches, the target's own choice is
  emitted as the correction, and after a full match the choice at the last
  node is the bonus token.
* DDTree notes, section 7.2: the verifier walk starts at the committed root,
  follows the drafted child equal to the target's choice and otherwise stops,
  taking that choice as the next bonus token; no further target pass is
  needed because every node's logits come from the one verify pass.

Readings where the pages leave the step open:

* A request has N_b + 1 logits rows: row 0 is the target's prediction at the
  last committed token (the walk's root), row 1 + i the prediction after
  node i.  Nodes with parent -1 are the root's children.
* The target's choice is the argmax of the row, ties to the lowest token id;
  -0.0 equals +0.0 (``np.argmax`` on the exactly widened values does both).
* Among the current node's children, the lowest-index child whose token
  matches is taken.
* ``max_accept`` bounds the accepted nodes; reaching it while a further match
  exists sets error bit 16 and stops the walk there.
"""

from typing import Dict, List

import numpy as np

ERR_ACCEPT_OVERFLOW = 16


def row_argmax(rows: np.ndarray) -> List[int]:
    """Lowest index of the maximum of each row (rows widened exactly to float64)."""
    return [int(np.argmax(np.asarray(r, dtype=np.float64))) for r in rows]


def greedy_walk(choice: List[int], tokens, parents, max_accept: int) -> Dict[str, object]:
    """Sequential greedy walk of one request.

    choice[r] is the target's token for logits row r (row 0 = root).
    Returns accepted node indices, their tokens, the bonus token and err bits.
    """
    tokens = [int(t) for t in tokens]
    parents = [int(p) for p in parents]
    n = len(parents)
    accepted: List[int] = []
    err = 0
    current = -1                  # the committed root
    target = choice[0]
    while True:
        children = [j for j in range(n) if parents[j] == current]
        match = [j for j in children if tokens[j] == target]
        if not match:
            break
        if len(accepted) == max_accept:
            err |= ERR_ACCEPT_OVERFLOW
            break
        current = match[0]
        accepted.append(current)
        target = choice[1 + current]
    return dict(accepted=accepted, accepted_tokens=[tokens[j] for j in accepted],
                bonus=target, err=err)


def accept(logits_rows_f64_of, node_offsets, tokens_all, parents_all, max_accept: int):
    """Batched greedy acceptance.

    ``logits_rows_f64_of(b)`` returns request b's N_b + 1 logits rows as
    float64 (exact widening of fp32 or bf16).  Returns per-request lists plus
    the ABI-shaped arrays accept_len [B], accepted_nodes [B, max_accept],
    out_tokens [B, max_accept + 1] (unused entries -1), row_argmax [T + B].
    """
    node_offsets = np.asarray(node_offsets)
    B = len(node_offsets) - 1
    T = int(node_offsets[-1])
    accept_len = np.zeros(B, dtype=np.int32)
    accepted_nodes = np.full((B, max_accept), -1, dtype=np.int32)
    out_tokens = np.full((B, max_accept + 1), -1, dtype=np.int32)
    argmax_all = np.zeros(T + B, dtype=np.int32)
    err = np.zeros(B, dtype=np.int32)
    for b in range(B):
        s, e = int(node_offsets[b]), int(node_offsets[b + 1])
        choice = row_argmax(logits_rows_f64_of(b))
        argmax_all[s + b: e + b + 1] = choice
        w = greedy_walk(choice, tokens_all[s:e], parents_all[s:e], max_accept)
        a = len(w["accepted"])
        accept_len[b] = a
        accepted_nodes[b, :a] = w["accepted"]
        out_tokens[b, :a] = w["accepted_tokens"]
        out_tokens[b, a] = w["bonus"]
        err[b] = w["err"]
    return dict(accept_len=accept_len, accepted_nodes=accepted_nodes, out_tokens=out_tokens,
                row_argmax=argmax_all, err=err)
