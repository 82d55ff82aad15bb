"""Pins of the acceptance and commit oracles against the pages' worked examples."""

import numpy as np
import pytest

import synth
from oracle import accept as AC
from oracle import commit as CM
from oracle import tree as T
from oracle import bf16 as OB
from conftest import golden


def planted_rows(n_rows, vocab, targets):
    rows = np.zeros((n_rows, vocab))
    for r, t in targets.items():
        rows[r, t] = 1.0
    return rows


def test_verify_tree_example_pin():
    g = golden("verify_tree_example.json")
    pt = golden("packed_table.json")
    toks, par = pt["tokens"], pt["parents"]
    # target path [4, 7, 3]: root row -> 4; node 0 (token 4) row -> 7; node 3 (token 7) row -> 3
    tgt = g["target_next"]
    rows = planted_rows(9, 16, {0: tgt[0], 1 + 0: tgt[1], 1 + 3: tgt[2]})
    w = AC.greedy_walk(AC.row_argmax(rows), toks, par, 8)
    assert w["accepted_tokens"] == g["accepted_tokens"]
    assert w["accepted"] == [0, 3]
    assert w["bonus"] == tgt[2]
    # Commit: slot s of the cache holds token ids; base [10, 11] + tentative nodes in packed order.
    base = g["base_cache"]
    ctx = len(base)
    cache = np.array([[[[t] for t in base + toks]]])           # [B=1, Hkv=1, 10, D=1]
    k, v, new_lens = CM.commit_contiguous(cache, cache, [ctx], [2], [w["accepted"]])
    assert k[0, 0, :new_lens[0], 0].tolist() == g["committed_cache"]
    assert len(toks) - len(w["accepted"]) == g["rejected_tentative"]


def test_ddtree_walk_pin():
    g = golden("ddtree_walk.json")
    voc = g["vocab"]
    par = g["parents"]
    toks = [voc[s] for s in ["A", "B", "B", "A", "B", "C"]]
    md = T.build_request(par, 1)        # committed root b at position 0 -> context length 1
    assert [0] + md["positions"] == g["position_ids"]
    tg = g["target_greedy"]
    rows = planted_rows(7, 4, {0: voc[tg["b"]], 1 + 0: voc[tg["A"]], 1 + 2: voc[tg["AB"]]})
    w = AC.greedy_walk(AC.row_argmax(rows), toks, par, 8)
    assert [k for t in w["accepted_tokens"] for k, vv in voc.items() if vv == t] == g["accepted"]
    assert w["bonus"] == voc[g["bonus"]]
    assert len(w["accepted"]) + 1 == g["tokens_this_round"]


def brute_argmax(row):
    best, idx = None, None
    for i, v in enumerate(row):
        if best is None or v > best:
            best, idx = v, i
    return idx


def test_argmax_ties_and_signed_zero():
    rows = np.array([[1.0, 3.0, 3.0, 2.0], [-0.0, 0.0, -1.0, -0.0], [0.0, -0.0, -2.0, -3.0],
                     [-5.0, -4.0, -4.0, -6.0]])
    got = AC.row_argmax(rows)
    assert got == [1, 0, 0, 1]
    assert got == [brute_argmax(r.tolist()) for r in rows]
    rng = np.random.default_rng(0)
    for _ in range(200):
        r = rng.integers(-3, 3, size=17).astype(np.float64)  # many ties
        assert AC.row_argmax(r[None])[0] == brute_argmax(r.tolist())


def test_argmax_bf16_rows_widened_exactly():
    rng = np.random.default_rng(1)
    bits = synth.bf16_bits_from_f32(rng.standard_normal((6, 300)).astype(np.float32))
    rows = OB.to_f64(bits)
    assert AC.row_argmax(rows) == [brute_argmax(r.tolist()) for r in rows]


def test_walk_all_mismatch_and_empty():
    w = AC.greedy_walk([5, 1, 1], [3, 4], [-1, -1], 4)
    assert w["accepted"] == [] and w["bonus"] == 5
    w = AC.greedy_walk([7], [], [], 4)
    assert w["accepted"] == [] and w["bonus"] == 7 and w["err"] == 0


def test_walk_duplicate_sibling_tokens_lowest_index():
    # nodes 0 and 1 both carry token 9 under the root; node 2 is a child of 1 only
    w = AC.greedy_walk([9, 2, 2, 0], [9, 9, 2], [-1, -1, 1], 4)
    assert w["accepted"] == [0]       # lowest index matching child wins, then no child of 0
    assert w["bonus"] == 2


def test_walk_overflow_flag():
    par = [-1, 0, 1, 2]
    toks = [1, 2, 3, 4]
    choice = [1, 2, 3, 4, 5]
    w = AC.greedy_walk(choice, toks, par, 2)
    assert w["err"] & AC.ERR_ACCEPT_OVERFLOW and w["accepted"] == [0, 1]
    w = AC.greedy_walk(choice, toks, par, 4)
    assert w["err"] == 0 and w["accepted"] == [0, 1, 2, 3] and w["bonus"] == 5


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_walk_properties_on_planted_workload(seed):
    wl = synth.make_workload(2, seed, batch=6, ctx=(10, 20), vocab=500)
    rows_of = lambda b: OB.to_f64(wl.logits[int(wl.node_offsets[b]) + b: int(wl.node_offsets[b + 1]) + b + 1])
    res = AC.accept(rows_of, wl.node_offsets, wl.tokens, wl.parents, 16)
    for b in range(wl.batch):
        s = int(wl.node_offsets[b])
        par = wl.parents[wl.request_nodes(b)].tolist()
        a = int(res["accept_len"][b])
        nodes = res["accepted_nodes"][b, :a].tolist()
        # Depths 0..a-1, each the parent of the next, tokens equal the planted choices.
        for d, j in enumerate(nodes):
            assert T.depth_of(j, par) == d
            assert par[j] == (nodes[d - 1] if d else -1)
            row = s + b + (0 if d == 0 else 1 + nodes[d - 1])
            assert wl.tokens[s + j] == wl.planted[row]
        # The walk stopped because the planted token of the stop row is not a child's.
        stop_row = s + b + (0 if a == 0 else 1 + nodes[-1])
        assert res["out_tokens"][b, a] == wl.planted[stop_row]
        kids = [j for j in range(len(par)) if par[j] == (nodes[-1] if a else -1)]
        assert all(wl.tokens[s + j] != wl.planted[stop_row] for j in kids)


def test_commit_aliasing_chain_moves():
    # accepted nodes [0, 2, 5]: slot ctx+2 is a source (d=1) and later a destination (d=2)
    ctx, N = 3, 7
    par = [-1, -1, 0, 0, 1, 2, 2]
    acc = [0, 2, 5]
    slots = np.arange(ctx + N)
    cache = np.zeros((1, 2, ctx + N, 4), dtype=np.uint16)
    cache[0, :, :, 0] = slots
    k, v, nl = CM.commit_contiguous(cache, cache + 100, [ctx], [3], [acc])
    assert nl.tolist() == [6]
    assert k[0, 0, :6, 0].tolist() == [0, 1, 2, 3, 5, 8]
    assert v[0, 1, :6, 0].tolist() == [100, 101, 102, 103, 105, 108]
    # Same as list slicing of the linearised sequence.
    seq = list(range(ctx)) + [ctx + j for j in range(N)]
    assert k[0, 0, :6, 0].tolist() == seq[:ctx] + [seq[ctx + j] for j in acc]


def test_commit_paged_release():
    bs = 4
    ctx, N = 6, 9            # slots 0..14 -> blocks 0..3 (ceil(15/4) = 4)
    table = np.array([[7, 2, 5, 0, -1]], dtype=np.int32)
    pool = np.zeros((8, 1, bs, 1), dtype=np.int64)
    for slot in range(ctx + N):
        pool[table[0, slot // bs], 0, slot % bs, 0] = 1000 + slot
    acc = [1, 4]             # depth 0 node 1, depth 1 node 4 -> slots 7 and 10 move to 6 and 7
    k, v, nl, tab, rel = CM.commit_paged(pool, pool, table, [ctx], [N], [2], [acc], bs)
    assert nl.tolist() == [8]
    got = [k[table[0, s // bs], 0, s % bs, 0] for s in range(8)]
    assert got == [1000 + s for s in range(6)] + [1007, 1010]
    # new_len 8 -> keep blocks 0, 1; release logical 2, 3 (physical 5, 0) in logical order
    assert rel == [[5, 0]]
    assert tab.tolist() == [[7, 2, -1, -1, -1]]


def test_commit_accept_zero_releases_tail_blocks():
    bs = 16
    table = np.array([[3, 1, 0]], dtype=np.int32)
    pool = np.zeros((4, 1, bs, 1), dtype=np.int64)
    k, v, nl, tab, rel = CM.commit_paged(pool, pool, table, [32], [5], [0], [[]], bs)
    assert nl.tolist() == [32] and rel == [[0]] and tab.tolist() == [[3, 1, -1]]
