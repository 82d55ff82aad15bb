"""Seeded synthetic inputs for token-tree verification workloads.

This module draws inputs only: draft trees given as parent lists, token ids,
bf16 activations, KV caches and target logits with a planted argmax.  It holds
none of the verification arithmetic (no masks, depths, positions, RoPE,
attention, acceptance walk or commit).  The CPU oracle and the GPU path both
consume what it returns, and neither imports the other.

Every draw comes from ``np.random.default_rng([seed, cfg_id, stream, ...])``
with a separate stream per kind of input, so any one input can be regenerated
alone; the large normal arrays (Q/K/V, caches) are drawn in 2^24-value slabs,
each seeded by its index, so several threads can draw them.

Workload shapes follow the five verification workloads of the pages' setting:

* ``tiny_medusa``  -- Medusa top-2 x top-3 cartesian tree (8 nodes, 6 paths),
  context 7, 4 query / 2 KV heads, head_dim 64, vocab 1000 fp32 logits,
  acceptance 0.8, contiguous cache.
* ``eagle``        -- EAGLE-style layered tree (depth 6, top-4 leaves expanded
  by 4 children per layer, reranked to 64 nodes), context 4096, 32/8/128,
  vocab 128256 bf16, acceptance 0.8, contiguous cache.
* ``batched``      -- 32 requests, context U{512..8192}, random trees of
  U{16..64} nodes with at most 8 levels, 32/8/128, paged cache (block 16,
  shuffled tables), vocab 128256 bf16, acceptance U(0.5, 0.9) per request.
* ``ddtree``       -- 4 DDTree trees of the top-1024 prefixes of factorised
  per-depth drafts (16 depths, N(0, 2) logits over vocab 151936 truncated to
  the top 1024), context 16384, 64/8/128, bf16 logits, acceptance 0.7.
* ``medusa_long``  -- 64 Medusa cartesian trees with top-s = (10, 3, 2, 2)
  (220 nodes), context U{1024..32768}, paged cache, 40/8/128, vocab 32000
  bf16, acceptance 0.6.
* ``ddtree_deep``  -- stress variant of ``ddtree`` with N(0, 8^2) draft logits,
  which gives trees about 13 levels deep.
"""

from __future__ import annotations

import dataclasses
import heapq
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "CONFIGS", "Workload", "make_workload", "bf16_bits_from_f32", "f32_from_bf16_bits",
    "medusa_tree", "eagle_tree", "random_tree", "ddtree_tree", "BLOCK_SIZE", "make_trees", "TreeBatch",
    "gumbel_noise", "draft_distributions", "uniforms", "draft_logits",
]

BLOCK_SIZE = 16

# Input streams: each kind of input has its own generator.
_S_TREE, _S_TOKENS, _S_QKV, _S_CACHE, _S_LOGITS, _S_LENS, _S_PAGES, _S_PLANT = range(8)


def _rng(seed: int, cfg_id: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(cfg_id), int(stream)])


# --------------------------------------------------------------------------
# bf16 encoding of draws (round to nearest even).  Input drawing only.
# --------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _bf16_round_up(v: float) -> int:
    """Smallest bf16 value >= v (v finite), as bits."""
    f = np.array([v], dtype=np.float32)
    if float(f[0]) < v:  # float32 rounding went down: step up one float32 ulp
        f = np.nextafter(f, np.float32(np.inf)).astype(np.float32)
    u = int(f.view(np.uint32)[0])
    hi, lo = u >> 16, u & 0xFFFF
    if lo == 0:
        return hi
    if (u >> 31) == 0:  # positive: truncation is below v, step up
        return hi + 1
    return hi  # negative: truncation moves toward zero, i.e. up


def _f32_round_up(v: float) -> float:
    f = np.float32(v)
    if float(f) < v:
        f = np.nextafter(f, np.float32(np.inf))
    return float(f)


_SLAB = 1 << 24  # values per independently seeded slab of a normal draw


def _normal_bf16(key, shape, scale: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0, scale^2) float32 draws.

    ``key`` is a list of ints; slab i of 2^24 values comes from
    ``np.random.default_rng(key + [i])``, so the slabs can be drawn by
    several threads and the result depends only on the key and the shape.
    """
    from concurrent.futures import ThreadPoolExecutor

    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.uint16)

    def slab(i):
        s = i * _SLAB
        e = min(n, s + _SLAB)
        x = np.random.default_rng(list(key) + [i]).standard_normal(e - s, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[s:e] = bf16_bits_from_f32(x)

    n_slabs = (n + _SLAB - 1) // _SLAB
    if n_slabs <= 1:
        for i in range(n_slabs):
            slab(i)
    else:
        with ThreadPoolExecutor(max_workers=min(8, n_slabs)) as ex:
            list(ex.map(slab, range(n_slabs)))
    return out.reshape(shape)


# --------------------------------------------------------------------------
# Draft-tree generators (parent lists in topological order: parent[i] < i).
# --------------------------------------------------------------------------

def medusa_tree(tops: Sequence[int]) -> np.ndarray:
    """Cartesian Medusa tree in level order.

    Depth-0 nodes are head 0's top-s0 candidates (parent -1); every node at
    depth k-1 gets head k's top-s_k candidates as children.
    """
    parents: List[int] = []
    level = [-1]
    for s in tops:
        nxt = []
        for p in level:
            for _ in range(int(s)):
                nxt.append(len(parents))
                parents.append(p)
        level = nxt
    return np.asarray(parents, dtype=np.int32)


def medusa_tokens(rng: np.random.Generator, tops: Sequence[int], vocab: int) -> np.ndarray:
    """Token of every node of ``medusa_tree(tops)``: head k's distinct top-s_k ids."""
    heads = [rng.choice(vocab, size=int(s), replace=False) for s in tops]
    toks: List[int] = []
    count = 1
    for k, s in enumerate(tops):
        for _parent in range(count):
            toks.extend(int(t) for t in heads[k])
        count *= int(s)
    return np.asarray(toks, dtype=np.int32)


def eagle_tree(rng: np.random.Generator, levels: int = 6, width: int = 4,
               expand: int = 4, budget: int = 64) -> np.ndarray:
    """EAGLE-style layered tree.

    Level 0 holds ``width`` draft candidates.  Each further level takes the
    ``expand`` best nodes of the previous level, by the product of their
    U(0,1) confidences along the path, and gives each ``width`` children.
    The candidates are then reranked and the best ``budget`` kept; since a
    child's product is below its parent's, the kept set is prefix-closed.
    """
    score: List[float] = []
    parent: List[int] = []
    level: List[int] = []
    for _ in range(width):
        level.append(len(score))
        score.append(float(rng.uniform()))
        parent.append(-1)
    for _ in range(1, levels):
        best = sorted(level, key=lambda n: -score[n])[:expand]
        nxt = []
        for p in best:
            for _ in range(width):
                nxt.append(len(score))
                score.append(score[p] * float(rng.uniform()))
                parent.append(p)
        level = nxt
    keep = sorted(range(len(score)), key=lambda n: -score[n])[:budget]
    keep_set = set(keep)
    for n in keep:  # prefix closure holds by construction; check it anyway
        assert parent[n] == -1 or parent[n] in keep_set
    order = sorted(keep)  # candidate creation order is topological
    remap = {n: i for i, n in enumerate(order)}
    return np.asarray([-1 if parent[n] == -1 else remap[parent[n]] for n in order],
                      dtype=np.int32)


def random_tree(rng: np.random.Generator, n: int, max_parent_depth: int = 6) -> np.ndarray:
    """Node 0 is the root; node i's parent is uniform over earlier nodes whose
    0-based depth is at most ``max_parent_depth`` (so at most
    ``max_parent_depth + 2`` levels)."""
    parents = np.empty(n, dtype=np.int32)
    depth = np.empty(n, dtype=np.int32)
    eligible: List[int] = []
    for i in range(n):
        if i == 0:
            parents[i], depth[i] = -1, 0
        else:
            p = eligible[int(rng.integers(len(eligible)))]
            parents[i], depth[i] = p, depth[p] + 1
        if depth[i] <= max_parent_depth:
            eligible.append(i)
    return parents


def ddtree_tree(rng: np.random.Generator, vocab: int, depths: int = 16, topk: int = 1024,
                budget: int = 1024, sigma: float = 2.0):
    """DDTree draft: the ``budget`` most probable prefixes of a factorised draft.

    Per depth, logits z ~ N(0, sigma^2) over the vocab are truncated to their
    top ``topk`` tokens and renormalised (a softmax over those).  A prefix is a
    tuple of per-depth ranks; its score is the sum of its log-probabilities.
    Prefixes are popped best-first from a heap seeded with (rank 1 at depth 1):
    a popped prefix pushes its next sibling (last rank + 1) and its first child
    (rank 1 at the next depth).  Returns (parents, tokens) in pop order, which
    is topological because a prefix scores strictly above its extensions.
    """
    tok_by_rank = []
    logq = []
    k = min(topk, vocab)
    for _ in range(depths):
        z = rng.standard_normal(vocab) * sigma
        idx = np.argpartition(-z, k - 1)[:k]
        idx = idx[np.argsort(-z[idx], kind="stable")]
        zz = z[idx]
        lse = zz.max() + np.log(np.exp(zz - zz.max()).sum())
        tok_by_rank.append(idx.astype(np.int64))
        logq.append(zz - lse)
    heap = [(-logq[0][0], (0,))]
    node_of = {}
    parents: List[int] = []
    tokens: List[int] = []
    while heap and len(parents) < budget:
        negs, ranks = heapq.heappop(heap)
        d = len(ranks) - 1
        node_of[ranks] = len(parents)
        parents.append(-1 if d == 0 else node_of[ranks[:-1]])
        tokens.append(int(tok_by_rank[d][ranks[-1]]))
        s = -negs
        if ranks[-1] + 1 < k:
            sib = ranks[:-1] + (ranks[-1] + 1,)
            heapq.heappush(heap, (-(s - logq[d][ranks[-1]] + logq[d][ranks[-1] + 1]), sib))
        if d + 1 < depths:
            heapq.heappush(heap, (-(s + logq[d + 1][0]), ranks + (0,)))
    return np.asarray(parents, dtype=np.int32), np.asarray(tokens, dtype=np.int32)


def _distinct_sibling_tokens(rng: np.random.Generator, parents: np.ndarray, vocab: int) -> np.ndarray:
    """Random token per node, distinct among the children of each parent."""
    n = len(parents)
    tokens = np.empty(n, dtype=np.int32)
    used: Dict[int, set] = {}
    for i in range(n):
        s = used.setdefault(int(parents[i]), set())
        while True:
            t = int(rng.integers(vocab))
            if t not in s:
                break
        s.add(t)
        tokens[i] = t
    return tokens


# --------------------------------------------------------------------------
# Workload container
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    logits_dtype: str            # "fp32" or "bf16"
    layout: str                  # "contiguous" or "paged"
    parents: np.ndarray          # int32 [T], request-local parent (-1 = off the context)
    tokens: np.ndarray           # int32 [T]
    node_offsets: np.ndarray     # int32 [B+1]
    ctx_lens: np.ndarray         # int32 [B]
    accept_p: np.ndarray         # float64 [B] planted acceptance probability
    q: np.ndarray                # uint16 (bf16) [T, Hq, D]
    k_new: np.ndarray            # uint16 (bf16) [T, Hkv, D]
    v_new: np.ndarray            # uint16 (bf16) [T, Hkv, D]
    k_cache: np.ndarray          # uint16: contiguous [B, Hkv, cap, D] / paged [NB, Hkv, 16, D]
    v_cache: np.ndarray
    capacity: int                # contiguous: slots per request
    block_table: Optional[np.ndarray]  # paged: int32 [B, max_blocks], -1 = none
    logits: np.ndarray           # float32 or uint16 (bf16) [T+B, V]
    planted: np.ndarray          # int32 [T+B] planted target token per logits row
    rope_base: float = 10000.0

    @property
    def batch(self) -> int:
        return len(self.ctx_lens)

    @property
    def total_nodes(self) -> int:
        return int(self.node_offsets[-1])

    @property
    def n_max(self) -> int:
        return int(np.diff(self.node_offsets).max(initial=0))

    def request_nodes(self, b: int) -> slice:
        return slice(int(self.node_offsets[b]), int(self.node_offsets[b + 1]))


CONFIGS = {
    0: dict(name="tiny_medusa", batch=1, ctx=(7, 7), tree=("medusa", (2, 3)),
            heads=(4, 2, 64), vocab=1000, logits="fp32", p=(0.8, 0.8), layout="contiguous"),
    1: dict(name="eagle", batch=1, ctx=(4096, 4096), tree=("eagle", 64),
            heads=(32, 8, 128), vocab=128256, logits="bf16", p=(0.8, 0.8), layout="contiguous"),
    2: dict(name="batched", batch=32, ctx=(512, 8192), tree=("random", (16, 64)),
            heads=(32, 8, 128), vocab=128256, logits="bf16", p=(0.5, 0.9), layout="paged"),
    3: dict(name="ddtree", batch=4, ctx=(16384, 16384), tree=("ddtree", 2.0),
            heads=(64, 8, 128), vocab=151936, logits="bf16", p=(0.7, 0.7), layout="contiguous"),
    4: dict(name="medusa_long", batch=64, ctx=(1024, 32768), tree=("medusa", (10, 3, 2, 2)),
            heads=(40, 8, 128), vocab=32000, logits="bf16", p=(0.6, 0.6), layout="paged"),
    5: dict(name="ddtree_deep", batch=4, ctx=(16384, 16384), tree=("ddtree", 8.0),
            heads=(64, 8, 128), vocab=151936, logits="bf16", p=(0.7, 0.7), layout="contiguous"),
}


def _small_alphabet_tokens(rng: np.random.Generator, parents: np.ndarray, alphabet: int) -> np.ndarray:
    """Uniform tokens from [0, alphabet): siblings often share a token."""
    return rng.integers(0, alphabet, size=len(parents)).astype(np.int32)


def _tree_for(cfg: dict, rng_tree, rng_tok, vocab, draft_vocab, ddtree_budget):
    kind, arg = cfg["tree"]
    dup = int(cfg.get("dup_alphabet", 0))  # > 0: sibling tokens drawn from a tiny alphabet
    tok_of = ((lambda p: _small_alphabet_tokens(rng_tok, p, dup)) if dup > 0
              else (lambda p: _distinct_sibling_tokens(rng_tok, p, vocab)))
    if kind == "medusa":
        return medusa_tree(arg), medusa_tokens(rng_tok, arg, vocab)
    if kind == "eagle":
        p = eagle_tree(rng_tree, budget=int(arg))
        return p, tok_of(p)
    if kind == "random":
        lo, hi = arg
        p = random_tree(rng_tree, int(rng_tree.integers(lo, hi + 1)))
        return p, tok_of(p)
    if kind == "ddtree":
        return ddtree_tree(rng_tree, draft_vocab, topk=min(1024, draft_vocab),
                           budget=ddtree_budget, sigma=float(arg))
    if kind == "parents":  # explicit parent list
        p = np.asarray(arg, dtype=np.int32)
        return p, tok_of(p)
    raise ValueError(kind)


@dataclasses.dataclass
class TreeBatch:
    """Trees, tokens and context lengths of one batch (no activations)."""
    parents: np.ndarray
    tokens: np.ndarray
    node_offsets: np.ndarray
    ctx_lens: np.ndarray
    accept_p: np.ndarray
    per_request_parents: list
    per_request_tokens: list

    @property
    def batch(self) -> int:
        return len(self.ctx_lens)

    @property
    def total_nodes(self) -> int:
        return int(self.node_offsets[-1])

    @property
    def n_max(self) -> int:
        return int(np.diff(self.node_offsets).max(initial=0))

    def request_nodes(self, b: int) -> slice:
        return slice(int(self.node_offsets[b]), int(self.node_offsets[b + 1]))


def _config(cfg_id: int, over: dict) -> dict:
    cfg = dict(CONFIGS[cfg_id])
    cfg.update(over)
    return cfg


def make_trees(cfg_id: int, seed: int = 0, ddtree_budget: int = 1024, **over) -> TreeBatch:
    """The tree / token / context-length part of ``make_workload``."""
    cfg = _config(cfg_id, over)
    B = int(cfg["batch"])
    V = int(cfg["vocab"])
    r_tree, r_tok, r_len = _rng(seed, cfg_id, _S_TREE), _rng(seed, cfg_id, _S_TOKENS), _rng(seed, cfg_id, _S_LENS)
    parents, tokens, sizes = [], [], []
    for _b in range(B):
        p, t = _tree_for(cfg, r_tree, r_tok, V, V, ddtree_budget)
        parents.append(p)
        tokens.append(t)
        sizes.append(len(p))
    node_offsets = np.zeros(B + 1, dtype=np.int32)
    node_offsets[1:] = np.cumsum(sizes)
    lo, hi = cfg["ctx"]
    ctx = r_len.integers(lo, hi + 1, size=B).astype(np.int32)
    plo, phi = cfg["p"]
    accept_p = r_len.uniform(plo, phi, size=B) if phi > plo else np.full(B, plo)
    T = int(node_offsets[-1])
    parents_all = np.concatenate(parents).astype(np.int32) if T else np.zeros(0, np.int32)
    tokens_all = np.concatenate(tokens).astype(np.int32) if T else np.zeros(0, np.int32)
    return TreeBatch(parents_all, tokens_all, node_offsets, ctx, accept_p, parents, tokens)


def make_workload(cfg_id: int, seed: int = 0, **over) -> Workload:
    """Build one seeded workload.

    ``over`` may replace any CONFIGS field (``batch``, ``ctx``, ``tree``,
    ``heads``, ``vocab``, ``logits``, ``p``, ``layout``) to draw a scaled-down
    case of the same structure, plus ``ddtree_budget``, ``spare_slots`` and
    ``dup_alphabet`` (draw non-Medusa node tokens from that many ids, so
    siblings share tokens; the planted choice is still a child's token).
    """
    ddtree_budget = int(over.pop("ddtree_budget", 1024))
    spare = int(over.pop("spare_slots", 0))
    cfg = _config(cfg_id, over)
    tb = make_trees(cfg_id, seed, ddtree_budget=ddtree_budget, **over)
    B = tb.batch
    hq, hkv, D = cfg["heads"]
    V = int(cfg["vocab"])
    T = tb.total_nodes
    sizes = np.diff(tb.node_offsets)
    ctx = tb.ctx_lens

    qkv = [int(seed), int(cfg_id), _S_QKV]
    q = _normal_bf16(qkv + [0], (T, hq, D))
    k_new = _normal_bf16(qkv + [1], (T, hkv, D))
    v_new = _normal_bf16(qkv + [2], (T, hkv, D))

    kv = [int(seed), int(cfg_id), _S_CACHE]
    need = ctx + sizes.astype(np.int32)
    if cfg["layout"] == "contiguous":
        cap = int(-(-(int(need.max(initial=1)) + spare) // BLOCK_SIZE) * BLOCK_SIZE)
        k_cache = _normal_bf16(kv + [0], (B, hkv, cap, D))
        v_cache = _normal_bf16(kv + [1], (B, hkv, cap, D))
        block_table = None
    else:
        nblk = [-(-(int(n) + spare) // BLOCK_SIZE) for n in need]
        total = int(sum(nblk))
        perm = _rng(seed, cfg_id, _S_PAGES).permutation(total).astype(np.int32)
        mb = max(nblk) if nblk else 1
        block_table = np.full((B, mb), -1, dtype=np.int32)
        off = 0
        for b, nb in enumerate(nblk):
            block_table[b, :nb] = perm[off:off + nb]
            off += nb
        k_cache = _normal_bf16(kv + [0], (total, hkv, BLOCK_SIZE, D))
        v_cache = _normal_bf16(kv + [1], (total, hkv, BLOCK_SIZE, D))
        cap = 0

    logits, planted = _planted_logits(_rng(seed, cfg_id, _S_LOGITS), _rng(seed, cfg_id, _S_PLANT),
                                      tb.per_request_parents, tb.per_request_tokens, tb.accept_p, V,
                                      cfg["logits"])
    return Workload(name=cfg["name"], seed=seed, n_heads=hq, n_kv_heads=hkv, head_dim=D, vocab=V,
                    logits_dtype=cfg["logits"], layout=cfg["layout"], parents=tb.parents,
                    tokens=tb.tokens, node_offsets=tb.node_offsets, ctx_lens=ctx, accept_p=tb.accept_p,
                    q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, capacity=cap,
                    block_table=block_table, logits=logits, planted=planted)


# --------------------------------------------------------------------------
# Random inputs of the sampled walks (drawing only)
# --------------------------------------------------------------------------

_S_GUMBEL, _S_DRAFT, _S_UNIFORM, _S_DDRAFT = 8, 9, 10, 11


def gumbel_noise(seed: int, cfg_id: int, rows: int, vocab: int) -> np.ndarray:
    """float32 [rows, vocab] standard Gumbel draws (numpy's Gumbel(0, 1) sampler)."""
    rng = _rng(seed, cfg_id, _S_GUMBEL)
    return rng.gumbel(0.0, 1.0, size=(rows, vocab)).astype(np.float32)


def draft_distributions(seed: int, cfg_id: int, rows: int, vocab: int, tokens_of_row=None,
                        boost: float = 0.0) -> np.ndarray:
    """float32 [rows, vocab] probability vectors (flat Dirichlet draws: normalised
    exponential variates).  ``tokens_of_row(r)`` may name tokens whose weight is
    multiplied by (1 + boost), so drafted tokens carry visible draft mass."""
    rng = _rng(seed, cfg_id, _S_DRAFT)
    x = rng.exponential(1.0, size=(rows, vocab))
    if tokens_of_row is not None and boost:
        for r in range(rows):
            t = tokens_of_row(r)
            if len(t):
                x[r, np.asarray(t, dtype=np.int64)] *= 1.0 + boost
    return (x / x.sum(axis=1, keepdims=True)).astype(np.float32)


def draft_logits(seed: int, cfg_id: int, requests: int, depths: int, vocab: int, sigma: float = 2.0,
                 levels: int = 0) -> np.ndarray:
    """float32 [requests, depths, vocab] per-depth drafter logits, N(0, sigma^2);
    with ``levels`` > 0 rounded to multiples of 1 / levels (many exact ties)."""
    x = _rng(seed, cfg_id, _S_DDRAFT).standard_normal((requests, depths, vocab)) * sigma
    if levels:
        x = np.round(x * levels) / levels
    return x.astype(np.float32)


def uniforms(seed: int, cfg_id: int, n: int) -> np.ndarray:
    """float32 [n] U[0, 1) draws."""
    return _rng(seed, cfg_id, _S_UNIFORM).random(n, dtype=np.float32)


def _planted_logits(r_val, r_plant, parents, tokens, accept_p, vocab, dtype):
    """Target logits [sum(N_b + 1), V]: N(0,1) draws with one planted maximum per row.

    Request b owns rows node_offsets[b] + b ... (N_b + 1 rows).  Row 0 stands
    for the last committed token; row 1 + i belongs to node i.  With
    probability p_b a row's planted token is the token of one of the row's
    children (uniformly chosen; row 0's children are the nodes with parent -1);
    otherwise, and always when there are no children, it is a uniform token
    that no child carries.  The planted value is the row maximum + 1, rounded
    up in the logits dtype, so the maximum is unique.
    """
    rows = sum(len(p) + 1 for p in parents)
    if dtype == "fp32":
        out = np.empty((rows, vocab), dtype=np.float32)
    else:
        out = np.empty((rows, vocab), dtype=np.uint16)
    planted = np.empty(rows, dtype=np.int32)
    r0 = 0
    for b, (par, tok) in enumerate(zip(parents, tokens)):
        n = len(par)
        kids: Dict[int, List[int]] = {}
        for j in range(n):
            kids.setdefault(int(par[j]), []).append(j)
        for r in range(n + 1):
            row = r0 + r
            ch = kids.get(r - 1, [])
            ch_tok = [int(tok[j]) for j in ch]
            if ch and r_plant.uniform() < accept_p[b]:
                t = ch_tok[int(r_plant.integers(len(ch)))]
            else:
                ban = set(ch_tok)
                while True:
                    t = int(r_plant.integers(vocab))
                    if t not in ban:
                        break
            planted[row] = t
            x = r_val.standard_normal(vocab, dtype=np.float32)
            if dtype == "fp32":
                x[t] = _f32_round_up(float(x.max()) + 1.0)
                out[row] = x
            else:
                bits = bf16_bits_from_f32(x)
                rowmax = float(f32_from_bf16_bits(bits).max())
                bits[t] = _bf16_round_up(rowmax + 1.0)
                out[row] = bits
        r0 += n + 1
    return out, planted
