"""KV commit and rollback as a copy (test infrastructure only).

What it follows:

* Decoding-extensions glossary, "Tree/Self Speculation" and the verify_tree
  experiment: with base cache [10, 11] and accepted path [4, 7] the committed
  cache becomes [10, 11, 4, 7]; every other tentative node is rolled back and
  released (6 of the 8 there).
* Tree-attention verification essay, KV cache section: the tree gets a
  contiguous cache region in node order; after verification the accepted
  path's nodes are kept and the rest is marked recyclable; with a paged cache
  that means releasing or reusing pages.
* "02 · Token Tree 与 Tree Attention", section 4: the chosen path's KV joins the
  cache as the next round's prompt; unchosen siblings and nodes past the
  rejection point are discarded.

Readings: the accepted node at depth d (node i_d) moves from slot ctx + i_d to
slot ctx + d for K and V of every KV head, taking the values the slots held
before the commit; the bonus token has no KV yet and is not committed;
new_len = ctx + a.  Paged cache: logical blocks whose index lies in
[ceil(new_len / bs), ceil((ctx + N) / bs)) are released, their physical ids
listed in logical order, and their table entries set to -1.  Slots at or past
new_len are undefined afterwards.
"""

import numpy as np


def commit_contiguous(k_cache, v_cache, ctx_lens, accept_len, accepted_nodes):
    """Return (k, v, new_lens) after committing every request (copies)."""
    k_old, v_old = np.array(k_cache), np.array(v_cache)
    k_new, v_new = np.array(k_cache), np.array(v_cache)
    B = len(ctx_lens)
    new_lens = np.zeros(B, dtype=np.int32)
    for b in range(B):
        c, a = int(ctx_lens[b]), int(accept_len[b])
        for d in range(a):
            src = c + int(accepted_nodes[b][d])
            k_new[b, :, c + d] = k_old[b, :, src]
            v_new[b, :, c + d] = v_old[b, :, src]
        new_lens[b] = c + a
    return k_new, v_new, new_lens


def commit_paged(k_pool, v_pool, block_table, ctx_lens, node_counts, accept_len, accepted_nodes,
                 block_size: int = 16):
    """Return (k, v, new_lens, new_table, released [list per request])."""
    k_old, v_old = np.array(k_pool), np.array(v_pool)
    k_new, v_new = np.array(k_pool), np.array(v_pool)
    table = np.array(block_table)
    B = len(ctx_lens)
    new_lens = np.zeros(B, dtype=np.int32)
    released = []

    def where(b, slot):
        return int(block_table[b, slot // block_size]), slot % block_size

    for b in range(B):
        c, a, n = int(ctx_lens[b]), int(accept_len[b]), int(node_counts[b])
        for d in range(a):
            sb, so = where(b, c + int(accepted_nodes[b][d]))
            db, do = where(b, c + d)
            k_new[db, :, do] = k_old[sb, :, so]
            v_new[db, :, do] = v_old[sb, :, so]
        new_lens[b] = c + a
        first = -(-(c + a) // block_size)
        last = -(-(c + n) // block_size)
        rel = [int(block_table[b, j]) for j in range(first, last)]
        for j in range(first, last):
            table[b, j] = -1
        released.append(rel)
    return k_new, v_new, new_lens, table, released
