"""Comparisons of GPU results with the CPU oracle (shared by the GPU tests and the smoke check).

Bars: bit-exact for metadata, row argmax, acceptance, tentative V and the
committed cache bytes; the rotated tentative K within one bf16 ulp of the
float64 rotation rounded to bf16 (RoPE is floating point); attention
outputs within |gpu - o64| <= 1e-2 + 1e-2 * |o64| elementwise against the
float64 oracle.
"""

from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

from oracle import accept as O_acc
from oracle import attention as O_att
from oracle import bf16 as O_bf16
from oracle import commit as O_com
from oracle import tree as O_tree

ATOL = 1e-2
RTOL = 1e-2


def mask_words_for(n_max: int) -> int:
    return max(1, (n_max + 31) // 32)


def check_build(wl, meta: Dict[str, np.ndarray], n_max: Optional[int] = None) -> None:
    n_max = wl.n_max if n_max is None else n_max
    W = meta["mask"].shape[1]
    ref = O_tree.build(wl.parents, wl.node_offsets, wl.ctx_lens, n_max, W)
    np.testing.assert_array_equal(meta["err"], ref["err"], err_msg="err")
    ok_nodes = np.ones(wl.total_nodes, dtype=bool)
    for b in range(wl.batch):
        if ref["err"][b]:
            ok_nodes[wl.request_nodes(b)] = False
    for k in ("depth", "positions", "retrieve_index", "retrieve_next_token", "retrieve_next_sibling"):
        np.testing.assert_array_equal(meta[k][ok_nodes], ref[k][ok_nodes], err_msg=k)
    np.testing.assert_array_equal(meta["mask"].view(np.uint32)[ok_nodes], ref["mask"][ok_nodes],
                                  err_msg="mask")


def logits_rows_f64(wl, b: int) -> np.ndarray:
    s, e = int(wl.node_offsets[b]), int(wl.node_offsets[b + 1])
    rows = wl.logits[s + b: e + b + 1]
    return O_bf16.to_f64(rows) if wl.logits_dtype == "bf16" else rows.astype(np.float64)


def check_accept(wl, acc: Dict[str, np.ndarray], max_accept: int) -> Dict[str, np.ndarray]:
    ref = O_acc.accept(lambda b: logits_rows_f64(wl, b), wl.node_offsets, wl.tokens, wl.parents,
                       max_accept)
    if "row_argmax" in acc:
        np.testing.assert_array_equal(acc["row_argmax"], ref["row_argmax"], err_msg="row_argmax")
    np.testing.assert_array_equal(acc["accept_len"], ref["accept_len"], err_msg="accept_len")
    np.testing.assert_array_equal(acc["accepted_nodes"], ref["accepted_nodes"], err_msg="accepted_nodes")
    np.testing.assert_array_equal(acc["out_tokens"], ref["out_tokens"], err_msg="out_tokens")
    return ref


def request_context(wl, b: int, k_cache: np.ndarray, v_cache: np.ndarray, table=None):
    """[Hkv, ctx, D] committed K/V of request b from a host cache image."""
    tab = wl.block_table if table is None else table
    return O_att.context_of(k_cache, v_cache, b, int(wl.ctx_lens[b]), wl.layout, tab)


def check_attention_request(wl, b: int, out_bits: np.ndarray, nodes: Optional[Sequence[int]] = None,
                            rope_base: float = 10000.0) -> float:
    """Compare one request's outputs (bits [N, Hq, D] or the selected nodes) with the oracle.

    Returns the largest |err| / (ATOL + RTOL |o64|) seen (<= 1 passes).
    """
    sl = wl.request_nodes(b)
    kc, vc = request_context(wl, b, wl.k_cache, wl.v_cache)
    ref = O_att.attention_request(wl.q[sl], wl.k_new[sl], wl.v_new[sl], kc, vc, wl.parents[sl],
                                  int(wl.ctx_lens[b]), rope_base, nodes=nodes)
    got = O_bf16.to_f64(out_bits)
    if nodes is not None and got.shape[0] != len(nodes):
        got = got[list(nodes)]
    ratio = np.abs(got - ref) / (ATOL + RTOL * np.abs(ref))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1.0, (f"request {b}: max |err|/(atol+rtol|ref|) = {worst:.3f}, "
                          f"max abs err {np.abs(got - ref).max():.3e}")
    return worst


def check_tentative(wl, b: int, k_slots_bits: np.ndarray, v_slots_bits: np.ndarray,
                    rope_base: float = 10000.0) -> None:
    """Slots ctx..ctx+N-1 after attention: K within 1 bf16 ulp of the rounded rotation, V exact.

    k_slots_bits / v_slots_bits: [Hkv, N, D] uint16.
    """
    sl = wl.request_nodes(b)
    ref_k = O_att.tentative_k(wl.k_new[sl], wl.parents[sl], int(wl.ctx_lens[b]), rope_base)  # [N, Hkv, D]
    ref_k = np.transpose(ref_k, (1, 0, 2))
    ref_bits = O_bf16.from_f64(ref_k)
    diff = np.abs(O_bf16.to_f64(k_slots_bits) - O_bf16.to_f64(ref_bits))
    assert (diff <= O_bf16.ulp(ref_bits) * (1 + 1e-12)).all(), f"request {b}: tentative K off by > 1 ulp"
    np.testing.assert_array_equal(v_slots_bits, np.transpose(wl.v_new[sl], (1, 0, 2)),
                                  err_msg=f"request {b}: tentative V")


def slots_of(wl, b: int, k_cache: np.ndarray, v_cache: np.ndarray, start: int, count: int,
             table=None) -> Tuple[np.ndarray, np.ndarray]:
    """[Hkv, count, D] of slots start.. of request b from a host cache image."""
    if wl.layout == "contiguous":
        return k_cache[b, :, start:start + count], v_cache[b, :, start:start + count]
    tab = wl.block_table if table is None else table
    Hkv, D = k_cache.shape[1], k_cache.shape[3]
    ko = np.empty((Hkv, count, D), dtype=k_cache.dtype)
    vo = np.empty((Hkv, count, D), dtype=v_cache.dtype)
    for t in range(count):
        slot = start + t
        blk = int(tab[b, slot // 16])
        ko[:, t] = k_cache[blk, :, slot % 16]
        vo[:, t] = v_cache[blk, :, slot % 16]
    return ko, vo
