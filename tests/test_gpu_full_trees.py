"""tree_attention_verify on 1024-node trees, every node compared with the oracle.

These cases reach the paths the sampled full-size rounds only touch: 32-word
ancestor masks, up to 32 tree tiles of 32 keys per item, 256-row items with
up to 32 tree tiles, the 128-row items a one-query-head-per-KV-head batch of
1024-node trees falls back to (the 256-row items' mask rows would not fit in
LDS), and the textbook special cases of the mask: a chain (the causal mask
over the context and the chain) and a star of 1024 depth-0 nodes (each node
sees the context and itself only).  A level-order tree and the same tree in
depth-first order must give the same outputs node for node.
Bar: |gpu - o64| <= 1e-2 + 1e-2 |o64| for every output element; tentative K
within one bf16 ulp of the rounded rotation, tentative V exact.
"""

import dataclasses

import numpy as np
import pytest

import synth
from gpu_helpers import region_bits, require_gpu, say
from oracle import bf16 as O_bf16
from parity import check_attention_request, check_tentative
from test_gpu_attention import run_attention

pytestmark = pytest.mark.gpu

CHAIN = [-1] + list(range(1023))
STAR = [-1] * 1024

FULL = {
    # 1024-node chain: the mask is lower triangular, positions ctx .. ctx + 1023
    "chain_1024_ctx40": (1, dict(batch=1, ctx=(40, 40), tree=("parents", CHAIN), heads=(8, 2, 128), vocab=64)),
    # 1024 depth-0 nodes: diagonal mask, every node at position ctx
    "star_1024_ctx300": (1, dict(batch=1, ctx=(300, 300), tree=("parents", STAR), heads=(32, 8, 128),
                                 vocab=4096)),
    # full-budget DDTree trees (1024 nodes, 64/8/128): 256-row items, 32 mask words
    "ddtree_1024_ctx200": (3, dict(batch=2, ctx=(200, 200), vocab=64)),
    "ddtree_deep_1024_ctx600": (5, dict(batch=2, ctx=(600, 600), vocab=64)),
    # one query head per KV head, 8 requests of 1024 nodes: enough row tiles
    # for 256-row items, whose mask rows would not fit; runs 128-row items
    "g1_1024_x8_ctx300": (2, dict(batch=8, ctx=(300, 300), tree=("random", (1024, 1024)), heads=(8, 8, 128),
                                  vocab=64, layout="contiguous")),
}


@pytest.mark.parametrize("name", sorted(FULL))
def test_full_tree_every_node(name):
    require_gpu()
    cfg, over = FULL[name]
    wl = synth.make_workload(cfg, 0, **over)
    assert wl.n_max == 1024
    say(f"tree_attention_verify {name}: B={wl.batch} T={wl.total_nodes} "
        f"heads={wl.n_heads}/{wl.n_kv_heads}/{wl.head_dim} ctx={wl.ctx_lens.tolist()}")
    d, out, err = run_attention(wl)
    assert (err == 0).all(), err
    for b in range(wl.batch):
        sl = wl.request_nodes(b)
        check_attention_request(wl, b, out[sl])
        n = sl.stop - sl.start
        kb = region_bits(d, wl, b, int(wl.ctx_lens[b]), n, "k")
        vb = region_bits(d, wl, b, int(wl.ctx_lens[b]), n, "v")
        check_tentative(wl, b, kb, vb)


def dfs_order(parents):
    """Pre-order of a parent list (children in increasing index): a permutation
    perm with perm[k] = the old index of new node k, parents still earlier."""
    kids = {}
    for i, p in enumerate(parents):
        kids.setdefault(int(p), []).append(i)
    order, stack = [], list(reversed(kids.get(-1, [])))
    while stack:
        i = stack.pop()
        order.append(i)
        stack.extend(reversed(kids.get(i, [])))
    return np.asarray(order, dtype=np.int64)


def permuted(wl, perm):
    """The same single-request workload with its nodes renumbered: new node k is old node perm[k]."""
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    par = np.asarray([-1 if wl.parents[o] < 0 else inv[wl.parents[o]] for o in perm], dtype=np.int32)
    return dataclasses.replace(wl, parents=par, tokens=wl.tokens[perm], q=wl.q[perm],
                               k_new=wl.k_new[perm], v_new=wl.v_new[perm])


@pytest.mark.parametrize("cfg, over", [
    (1, dict(ctx=(500, 500), vocab=64)),                                   # EAGLE tree, 64 nodes
    (4, dict(batch=1, ctx=(300, 300), vocab=64)),                          # Medusa (10,3,2,2), 220 nodes
])
def test_level_order_equals_depth_first_order(cfg, over):
    require_gpu()
    wl = synth.make_workload(cfg, 2, **over)
    assert wl.batch == 1
    perm = dfs_order(wl.parents)
    assert sorted(perm.tolist()) == list(range(wl.total_nodes))
    assert not np.array_equal(perm, np.arange(wl.total_nodes)), "the tree is already in DFS order"
    wl_dfs = permuted(wl, perm)
    say(f"level order vs DFS order, cfg={cfg}, N={wl.total_nodes}")
    _, out_lvl, err1 = run_attention(wl)
    _, out_dfs, err2 = run_attention(wl_dfs)
    assert (err1 == 0).all() and (err2 == 0).all()
    check_attention_request(wl, 0, out_lvl)
    check_attention_request(wl_dfs, 0, out_dfs)
    # node for node: new node k of the DFS order is old node perm[k]
    fa, fb = O_bf16.to_f64(out_lvl[perm]), O_bf16.to_f64(out_dfs)
    assert np.all(np.abs(fa - fb) <= 2e-2 + 2e-2 * np.abs(fa)), np.abs(fa - fb).max()
