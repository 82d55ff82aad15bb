"""Tree metadata, written out plainly (test infrastructure only).

What it follows:

* Decoding-extensions glossary ("Beam Search、约束解码与 Tree/Self
  Speculation"), section "Packed tree attention": unique nodes are packed in
  topological order; each node has a token, a parent, a depth and a position
  id; a node sees the whole committed prefix and its own ancestor chain (self
  included), never siblings or cousins; siblings share a position, and the
  packed index is never used as the position.
* Same page, packed-vs-branch experiment: depth by walking the parent chain,
  ancestor path by walking it and reversing.  The page counts depth from 1 and
  uses position = prefix + depth - 1; here depth counts from 0 (a node hanging
  off the committed prefix has depth 0) and position = context + depth, which
  is the same position.
* "02 · Token Tree 与 Tree Attention", section 3: positions are context length
  plus tree depth (depths [0,1,1,2] with a 7-token prompt give [7,8,8,9]); the
  mask is kept QLEN-only / bit-packed; retrieve_index, retrieve_next_token and
  retrieve_next_sibling are the indices used to walk the tree after verify.

Readings where the pages leave the step open:

* next_token[i] is i's first child (smallest index j with parent[j] == i),
  next_sibling[i] the next child of i's parent after i; -1 when none.
* retrieve_index[i] is the global logits row of node i: request b's rows start
  at node_offsets[b] + b, row 0 of a request is the last committed token and
  row 1 + i belongs to node i.
* Mask rows are uint32 words, bit j % 32 of word j // 32 (LSB first), row
  stride ``mask_words``, unused bits zero.  Context columns are always visible
  and are not stored.
* Error bits per request: 1 = a parent outside [-1, i-1]; 2 = more nodes than
  ``n_max``.  A flagged request's outputs are left as zeros here and are not
  compared.
"""

from typing import Dict, List

import numpy as np

ERR_BAD_PARENT = 1
ERR_TOO_MANY_NODES = 2
ERR_CAPACITY = 4
ERR_BAD_MASK = 64

MASK_QLEN_ONLY = 0   # dense [N_b] columns: the tree only
MASK_FULL = 1        # dense [ctx_b + N_b] columns: committed context, then the tree


def parents_valid(parents) -> bool:
    """Topological packing: every parent is -1 or an earlier node."""
    return all(-1 <= int(p) < i for i, p in enumerate(parents))


def depth_of(node: int, parents) -> int:
    """Number of ancestors of ``node`` (0 for a node hanging off the context)."""
    d, cur = 0, int(parents[node])
    while cur != -1:
        d += 1
        cur = int(parents[cur])
    return d


def ancestor_path(node: int, parents) -> List[int]:
    """Nodes from the top of the tree down to ``node`` (inclusive)."""
    path = []
    cur = int(node)
    while cur != -1:
        path.append(cur)
        cur = int(parents[cur])
    return path[::-1]


def build_request(parents, ctx_len: int) -> Dict[str, object]:
    """Metadata of one request's tree (local node indices)."""
    parents = [int(p) for p in parents]
    n = len(parents)
    depth = [depth_of(i, parents) for i in range(n)]
    positions = [int(ctx_len) + d for d in depth]
    visible = [ancestor_path(i, parents) for i in range(n)]
    next_token, next_sibling = [], []
    for i in range(n):
        kids = [j for j in range(n) if parents[j] == i]
        next_token.append(kids[0] if kids else -1)
        later = [j for j in range(i + 1, n) if parents[j] == parents[i]]
        next_sibling.append(later[0] if later else -1)
    return dict(depth=depth, positions=positions, visible=visible,
                next_token=next_token, next_sibling=next_sibling)


def build(parents_all, node_offsets, ctx_lens, n_max: int, mask_words: int) -> Dict[str, np.ndarray]:
    """Batched metadata in the layout the C ABI returns.

    Returns int32 arrays ``depth``, ``positions``, ``retrieve_index``,
    ``retrieve_next_token``, ``retrieve_next_sibling`` of length T, uint32
    ``mask`` [T, mask_words] and int32 ``err`` [B].
    """
    node_offsets = np.asarray(node_offsets)
    B = len(node_offsets) - 1
    T = int(node_offsets[-1])
    out = {k: np.zeros(T, dtype=np.int32) for k in
           ("depth", "positions", "retrieve_index", "retrieve_next_token", "retrieve_next_sibling")}
    out["mask"] = np.zeros((T, mask_words), dtype=np.uint32)
    out["err"] = np.zeros(B, dtype=np.int32)
    for b in range(B):
        s, e = int(node_offsets[b]), int(node_offsets[b + 1])
        par = [int(p) for p in parents_all[s:e]]
        if e - s > n_max:
            out["err"][b] |= ERR_TOO_MANY_NODES
        if not parents_valid(par):
            out["err"][b] |= ERR_BAD_PARENT
        if out["err"][b]:
            continue
        md = build_request(par, int(ctx_lens[b]))
        for i in range(e - s):
            out["depth"][s + i] = md["depth"][i]
            out["positions"][s + i] = md["positions"][i]
            out["retrieve_index"][s + i] = s + b + 1 + i
            out["retrieve_next_token"][s + i] = md["next_token"][i]
            out["retrieve_next_sibling"][s + i] = md["next_sibling"][i]
            for j in md["visible"][i]:
                out["mask"][s + i, j // 32] |= np.uint32(1 << (j % 32))
    return out


def mask_bool(mask_rows: np.ndarray, n: int) -> np.ndarray:
    """Unpack n bit-packed mask rows into a dense [n, n] bool matrix."""
    dense = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(n):
            dense[i, j] = bool((int(mask_rows[i, j // 32]) >> (j % 32)) & 1)
    return dense


def dense_mask(parents_all, node_offsets, ctx_lens, mode: int, row_stride: int):
    """The dense (one byte per column) masks of "02 · Token Tree 与 Tree
    Attention" §3's other two modes, in one [T, row_stride] uint8 array.

    QLEN_ONLY: byte j of node i's row is 1 iff j is i or an ancestor of i.
    FULL (the mask over the whole sequence, as the glossary's packed-vs-branch
    experiment's tree_mask [N, prefix + N]): bytes 0 .. ctx-1 are 1 (the
    committed context is always visible), byte ctx + j as QLEN_ONLY's byte j.
    Unused bytes are 0.  A request whose row does not fit row_stride gets
    err bit 4 and zero rows; bad parents / sizes as in ``build``.
    Returns (mask, err).
    """
    node_offsets = np.asarray(node_offsets)
    B = len(node_offsets) - 1
    T = int(node_offsets[-1])
    mask = np.zeros((T, row_stride), dtype=np.uint8)
    err = np.zeros(B, dtype=np.int32)
    for b in range(B):
        s, e = int(node_offsets[b]), int(node_offsets[b + 1])
        par = [int(p) for p in parents_all[s:e]]
        ctx = int(ctx_lens[b])
        if not parents_valid(par):
            err[b] |= ERR_BAD_PARENT
            continue
        base = ctx if mode == MASK_FULL else 0
        if base + (e - s) > row_stride:
            err[b] |= ERR_CAPACITY
            continue
        for i in range(e - s):
            mask[s + i, :base] = 1
            for j in ancestor_path(i, par):
                mask[s + i, base + j] = 1
    return mask, err


def pack_dense(dense, node_offsets, ctx_lens, mode: int, mask_words: int):
    """A caller's dense mask (either mode) packed into the bit-packed
    QLEN-only rows the attention reads: bit j of node i's row = byte j (or
    ctx + j) of its dense row.  A row is refused (err bit 64, row left zero)
    when it is not a mask the attention can run: a FULL row hiding a context
    column, a bit above the diagonal (a later node) or past the tree, or the
    node's own column clear.  Returns (packed, err)."""
    node_offsets = np.asarray(node_offsets)
    B = len(node_offsets) - 1
    T = int(node_offsets[-1])
    dense = np.asarray(dense)
    packed = np.zeros((T, mask_words), dtype=np.uint32)
    err = np.zeros(B, dtype=np.int32)
    for b in range(B):
        s, e = int(node_offsets[b]), int(node_offsets[b + 1])
        n, ctx = e - s, int(ctx_lens[b])
        base = ctx if mode == MASK_FULL else 0
        if base + n > dense.shape[1]:
            err[b] |= ERR_CAPACITY
            continue
        ok = True
        for i in range(n):
            row = dense[s + i]
            if mode == MASK_FULL and not all(row[:ctx] != 0):
                ok = False
            tree = row[base:base + n] != 0
            if not tree[i] or tree[i + 1:].any() or (row[base + n:] != 0).any():
                ok = False
        if not ok:
            err[b] |= ERR_BAD_MASK
            continue
        for i in range(n):
            row = dense[s + i]
            for j in range(n):
                if row[base + j]:
                    packed[s + i, j // 32] |= np.uint32(1 << (j % 32))
    return packed, err


def merge_sequences(seqs):
    """Draft sequences merged into one tree of their distinct prefixes
    (test infrastructure only).

    "02 · Token Tree 与 Tree Attention" §3: SpecInfer builds the tree bottom-up,
    merging independent drafts along their common prefixes; the glossary's
    packed node table shows three branches [4,5,6], [4,7,8], [9,0,1] becoming
    8 unique nodes.  Readings: a sequence ends at its first negative entry;
    nodes are numbered level by level (depth 0 first), and within a level in
    the order the sequences first reach them (sequence index, then nothing
    else: a sequence adds at most one node per level).  Returns (parents,
    tokens, node_of) with node_of[m][d] the node of sequence m's prefix of
    length d + 1 (-1 past its end).
    """
    M = len(seqs)
    L = max((len(s) for s in seqs), default=0)
    node_of = [[-1] * L for _ in range(M)]
    parents: List[int] = []
    tokens: List[int] = []
    for d in range(L):
        seen = {}
        for m in range(M):
            if d >= len(seqs[m]) or seqs[m][d] < 0 or (d > 0 and node_of[m][d - 1] < 0):
                continue
            key = (node_of[m][d - 1] if d > 0 else -1, int(seqs[m][d]))
            if key not in seen:
                seen[key] = len(parents)
                parents.append(key[0])
                tokens.append(key[1])
            node_of[m][d] = seen[key]
    return parents, tokens, node_of


def eagle_grow(root_tokens, root_conf, child_tokens, child_conf, budget: int):
    """EAGLE-style dynamic tree: layer-by-layer top-k expansion, then a global
    rerank (test infrastructure only).

    "02 · Token Tree 与 Tree Attention" §3: EAGLE grows the tree layer by layer,
    expanding the current layer's top-k nodes by top-k children ("layer x
    topk"); §5: the dynamic tree scores a node by its prefix survival
    probability (the product of the draft confidences along its path) and
    keeps the N_tree most promising nodes overall.

    Inputs: root_tokens / root_conf [k]: the first layer's k candidates;
    child_tokens / child_conf [L-1, k, k]: at layer l (1-based), the drafter's
    k children of the j-th expanded node of the previous layer.
    Readings: a node's score is its parent's score times its confidence
    (float64, in that order); a layer's expanded nodes are its k best by
    (score descending, creation index ascending), in that order; the kept
    nodes are the ``budget`` best of all created nodes by the same order (a
    parent comes before its children in that order, so the kept set is
    prefix-closed); they are renumbered in creation order.
    Returns (parents, tokens) of the kept tree.
    """
    k = len(root_tokens)
    par: List[int] = [-1] * k
    tok: List[int] = [int(t) for t in root_tokens]
    score: List[float] = [float(c) for c in root_conf]
    layer = list(range(k))
    for l in range(len(child_tokens)):
        expanded = sorted(layer, key=lambda i: (-score[i], i))[:k]
        layer = []
        for j, p in enumerate(expanded):
            for c in range(k):
                layer.append(len(par))
                par.append(p)
                tok.append(int(child_tokens[l][j][c]))
                score.append(score[p] * float(child_conf[l][j][c]))
    keep = sorted(sorted(range(len(par)), key=lambda i: (-score[i], i))[:budget])
    remap = {old: new for new, old in enumerate(keep)}
    return [-1 if par[i] < 0 else remap[par[i]] for i in keep], [tok[i] for i in keep]
