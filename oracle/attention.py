"""Tree attention as per-node causal attention on the linearised path (test infrastructure only).

Definition followed (float64 throughout):

* Decoding-extensions glossary, packed-vs-branch experiment: each candidate
  node, taken alone, attends over the committed base K/V followed by the K/V
  of its own root-to-node ancestor path (the "branch reference"); the packed
  ancestry-masked pass must reproduce it.  Scores are q.k / sqrt(D) and the
  softmax runs over that concatenated key list.
* Same page: RoPE in interleaved-pair form, inv_freq_m = base^(-2m/D) for pair
  (x_2m, x_2m+1), rotated as (x0 cos - x1 sin, x1 cos + x0 sin); candidate Q
  and K are rotated at their tree positions; the committed prefix K is already
  rotated when it sits in the cache.  V is never rotated.
* Tree-attention verification essay, mask section: the output of tree verify
  must equal token-by-token decoding of each path, which is what running
  ordinary causal attention on the linearised path computes.
* "02 · Token Tree 与 Tree Attention", section 3: position = context length +
  tree depth.

Readings: GQA maps query head h to KV head h // (Hq / Hkv); the softmax scale
defaults to 1/sqrt(D); the context is every committed slot 0..ctx-1.
"""

from typing import Iterable, Optional

import numpy as np

from . import bf16 as _bf16
from .tree import ancestor_path, depth_of


def rope(x: np.ndarray, positions, base: float = 10000.0) -> np.ndarray:
    """Rotate the last axis of ``x`` (float64, even length D) at ``positions``.

    ``positions`` broadcasts against ``x.shape[:-1]``.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    inv = float(base) ** (-(np.arange(0, D, 2, dtype=np.float64)) / D)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x1 * c + x0 * s
    return out


def softmax_attend(qg: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray,
                   k_path: np.ndarray, v_path: np.ndarray, scale: float) -> np.ndarray:
    """Attention of query rows ``qg`` [G, D] over the key list ctx ++ path.

    The scores of the concatenated key list are formed as the concatenation
    of the scores of its two parts, and the weighted sum over the list as the
    sum of its two parts; this is the same arithmetic as concatenating K and
    V first, without copying the context per node.
    """
    s = np.concatenate([qg @ k_ctx.T, qg @ k_path.T], axis=1) * scale   # [G, ctx + L]
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    c = k_ctx.shape[0]
    return p[:, :c] @ v_ctx + p[:, c:] @ v_path


def attention_request(q, k_new, v_new, k_ctx, v_ctx, parents, ctx_len: int,
                      rope_base: float = 10000.0, scale: Optional[float] = None,
                      nodes: Optional[Iterable[int]] = None) -> np.ndarray:
    """Outputs of one request's tree nodes.

    q      bf16 bits [N, Hq, D]       candidate queries (not yet rotated)
    k_new  bf16 bits [N, Hkv, D]      candidate keys (not yet rotated)
    v_new  bf16 bits [N, Hkv, D]
    k_ctx  bf16 bits [Hkv, ctx, D]    committed keys, already rotated
    v_ctx  bf16 bits [Hkv, ctx, D]
    Returns float64 [len(nodes), Hq, D] (all nodes by default).
    """
    N, Hq, D = q.shape
    Hkv = k_new.shape[1]
    G = Hq // Hkv
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(D)
    parents = [int(p) for p in parents]
    nodes = list(range(N)) if nodes is None else [int(i) for i in nodes]
    Kc = _bf16.to_f64(k_ctx[:, :ctx_len])
    Vc = _bf16.to_f64(v_ctx[:, :ctx_len])
    out = np.empty((len(nodes), Hq, D), dtype=np.float64)
    for oi, i in enumerate(nodes):
        path = ancestor_path(i, parents)
        pos_path = [ctx_len + depth_of(j, parents) for j in path]
        k_path = rope(_bf16.to_f64(k_new[path]), np.asarray(pos_path)[:, None], rope_base)  # [L, Hkv, D]
        v_path = _bf16.to_f64(v_new[path])
        q_i = rope(_bf16.to_f64(q[i]), ctx_len + depth_of(i, parents), rope_base)          # [Hq, D]
        for hk in range(Hkv):
            heads = slice(hk * G, (hk + 1) * G)
            out[oi, heads] = softmax_attend(q_i[heads], Kc[hk], Vc[hk],
                                            k_path[:, hk], v_path[:, hk], scale)
    return out


def context_of(k_cache, v_cache, b: int, ctx_len: int, layout: str, block_table=None,
               block_size: int = 16):
    """Committed K/V of request b as [Hkv, ctx, D] bf16 bits.

    Contiguous cache: [B, Hkv, capacity, D].  Paged cache: pool
    [num_blocks, Hkv, block_size, D] and logical slot t of request b lives in
    block block_table[b, t // block_size] at offset t % block_size.
    """
    if layout == "contiguous":
        return k_cache[b, :, :ctx_len], v_cache[b, :, :ctx_len]
    Hkv, D = k_cache.shape[1], k_cache.shape[3]
    kc = np.empty((Hkv, ctx_len, D), dtype=k_cache.dtype)
    vc = np.empty((Hkv, ctx_len, D), dtype=v_cache.dtype)
    for t in range(ctx_len):
        blk = int(block_table[b, t // block_size])
        kc[:, t] = k_cache[blk, :, t % block_size]
        vc[:, t] = v_cache[blk, :, t % block_size]
    return kc, vc


def tentative_k(k_new, parents, ctx_len: int, rope_base: float = 10000.0) -> np.ndarray:
    """The rotated candidate keys a verify pass leaves in slots ctx..ctx+N-1 (float64)."""
    pos = [ctx_len + depth_of(j, parents) for j in range(len(parents))]
    return rope(_bf16.to_f64(k_new), np.asarray(pos)[:, None], rope_base)
