"""Pins of the tree-metadata oracle against the pages and brute force."""

import itertools

import numpy as np
import pytest

import synth
from oracle import tree as T
from conftest import golden


def test_packed_table_pin():
    g = golden("packed_table.json")
    md = T.build_request(g["parents"], g["prefix_length"])
    assert [d + 1 for d in md["depth"]] == g["depth_one_based"]
    assert md["positions"] == g["positions"]
    assert md["visible"] == g["visible_candidate_ancestors"]
    assert [len(v) + g["prefix_length"] for v in md["visible"]] == g["tree_mask_visible_counts_with_prefix"]
    # Bit-packed rows carry the same sets.
    out = T.build(np.array(g["parents"]), np.array([0, 8]), np.array([g["prefix_length"]]), 8, 1)
    dense = T.mask_bool(out["mask"], 8)
    for i, vis in enumerate(g["visible_candidate_ancestors"]):
        assert sorted(np.nonzero(dense[i])[0].tolist()) == vis
    assert (dense.sum(1) + g["prefix_length"]).tolist() == g["tree_mask_visible_counts_with_prefix"]


def test_branch_dedup_counts():
    g = golden("packed_table.json")
    prefixes = {tuple(br[:d]) for br in g["branches"] for d in range(1, len(br) + 1)}
    assert sum(len(br) for br in g["branches"]) == g["branch_expanded_nodes"]
    assert len(prefixes) == g["unique_tree_nodes"] == len(g["parents"])
    # Each unique prefix is exactly one packed node: token path from the root.
    toks, par = g["tokens"], g["parents"]
    paths = {tuple(toks[j] for j in T.ancestor_path(i, par)) for i in range(len(par))}
    assert paths == prefixes


def test_positions_pin():
    g = golden("positions_example.json")
    md = T.build_request([-1, 0, 0, 1], g["prompt_length"])
    assert md["depth"] == g["depths"]
    assert md["positions"] == g["positions"]


def test_medusa_counts_pin():
    import synth
    g = golden("medusa_counts.json")
    for case in g["cases"]:
        par = synth.medusa_tree(case["tops"])
        md = T.build_request(par, 0)
        assert len(par) == case["nodes"]
        leaves = sum(1 for x in md["next_token"] if x == -1)
        assert leaves == case["paths"]
        # Closed form of the page: sum_k prod_{i<=k} s_i nodes, prod s_i paths.
        assert case["nodes"] == sum(int(np.prod(case["tops"][:k + 1])) for k in range(len(case["tops"])))
        assert case["paths"] == int(np.prod(case["tops"]))


def _closure(parents):
    """Reflexive-transitive closure of the child->parent relation by boolean matrix powers."""
    n = len(parents)
    A = np.zeros((n, n), dtype=np.int64)
    for i, p in enumerate(parents):
        if p >= 0:
            A[i, p] = 1
    R = np.eye(n, dtype=np.int64)
    P = np.eye(n, dtype=np.int64)
    for _ in range(n):
        P = (P @ A > 0).astype(np.int64)
        R = R | P
    return R.astype(bool)


def _all_parent_lists(n):
    return itertools.product(*[range(-1, i) for i in range(n)])


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7])
def test_bruteforce_all_trees(n):
    for parents in _all_parent_lists(n):
        parents = list(parents)
        ctx = 5
        out = T.build(np.array(parents), np.array([0, n]), np.array([ctx]), n, 1)
        assert out["err"][0] == 0
        dense = T.mask_bool(out["mask"], n)
        R = _closure(parents)
        assert np.array_equal(dense, R)
        # Depth is the number of strict ancestors; positions follow it.
        assert out["depth"].tolist() == (R.sum(1) - 1).tolist()
        assert out["positions"].tolist() == (ctx + R.sum(1) - 1).tolist()
        # First child / next sibling from a sort of (parent, index) pairs.
        order = sorted(range(n), key=lambda j: (parents[j], j))
        first_child = [-1] * n
        next_sib = [-1] * n
        for a, b in zip(order, order[1:]):
            if parents[a] == parents[b]:
                next_sib[a] = b
        for j in reversed(order):
            if parents[j] >= 0:
                first_child[parents[j]] = j
        assert out["retrieve_next_token"].tolist() == first_child
        assert out["retrieve_next_sibling"].tolist() == next_sib
        # Rows of the logits: request 0 starts at row 0, node i at row 1 + i.
        assert out["retrieve_index"].tolist() == [1 + i for i in range(n)]


def test_unused_mask_bits_zero_and_stride():
    par = list(range(-1, 39))  # a 40-node chain
    out = T.build(np.array(par), np.array([0, 40]), np.array([3]), 64, 3)
    assert out["mask"].shape == (40, 3)
    assert (out["mask"][:, 2] == 0).all()
    dense = T.mask_bool(out["mask"], 40)
    assert np.array_equal(dense, np.tril(np.ones((40, 40), dtype=bool)))


def test_error_bits():
    # bad parent (>= i) in request 0, too many nodes in request 1, request 2 fine
    parents = [-1, 1, -1, 0, 1, -1, 0]
    offs = [0, 2, 5, 7]
    out = T.build(np.array(parents), np.array(offs), np.array([1, 1, 1]), 2, 1)
    assert out["err"][0] & T.ERR_BAD_PARENT
    assert out["err"][1] & T.ERR_TOO_MANY_NODES
    assert out["err"][2] == 0
    out2 = T.build(np.array([-2]), np.array([0, 1]), np.array([0]), 4, 1)
    assert out2["err"][0] & T.ERR_BAD_PARENT


def test_empty_request_and_retrieve_rows():
    parents = [-1, 0, -1, -1, 1]
    offs = [0, 2, 2, 5]      # request 1 is empty
    out = T.build(np.array(parents), np.array(offs), np.array([4, 9, 0]), 3, 1)
    assert out["err"].tolist() == [0, 0, 0]
    assert out["retrieve_index"].tolist() == [1, 2, 5, 6, 7]
    assert out["positions"].tolist() == [4, 5, 0, 0, 1]


# ---- dense mask modes (FULL_MASK / QLEN_ONLY) and packing a caller's dense mask ----

def test_full_mask_pin():
    """The glossary's packed node table: tree_mask is [8, 10] (prefix 2 + 8 nodes)
    and each row sees 3, 3, 4, 4, 4, 5, 5, 5 columns (prefix included)."""
    g = golden("packed_table.json")
    par, P = g["parents"], g["prefix_length"]
    full, err = T.dense_mask(par, [0, len(par)], [P], T.MASK_FULL, P + len(par))
    assert list(full.shape) == g["shapes"]["tree_mask"] and not err.any()
    assert full.sum(axis=1).tolist() == g["tree_mask_visible_counts_with_prefix"]
    for i, anc in enumerate(g["visible_candidate_ancestors"]):
        assert np.flatnonzero(full[i, P:]).tolist() == anc
        assert full[i, :P].all()
    qlen, _ = T.dense_mask(par, [0, len(par)], [P], T.MASK_QLEN_ONLY, len(par))
    assert np.array_equal(qlen, full[:, P:])


def test_full_mask_of_a_chain_is_causal_and_of_a_star_is_diagonal():
    n, ctx = 9, 4
    chain = [-1] + list(range(n - 1))
    full, _ = T.dense_mask(chain, [0, n], [ctx], T.MASK_FULL, ctx + n)
    # the rows of the last n positions of a causal mask over ctx + n tokens
    assert np.array_equal(full, np.tril(np.ones((ctx + n, ctx + n), np.uint8))[ctx:])
    star = [-1] * n
    full, _ = T.dense_mask(star, [0, n], [ctx], T.MASK_FULL, ctx + n)
    assert np.array_equal(full, np.concatenate([np.ones((n, ctx), np.uint8), np.eye(n, dtype=np.uint8)], 1))


def test_dense_mask_stride_and_errors():
    par = [-1, 0, 0, 1]
    full, err = T.dense_mask(par + [-1, 5], [0, 4, 6], [3, 2], T.MASK_FULL, 8)
    assert err.tolist() == [0, T.ERR_BAD_PARENT]
    assert (full[:4, 7] == 0).all() and full[0, :4].tolist() == [1, 1, 1, 1]
    _, err = T.dense_mask(par, [0, 4], [5], T.MASK_FULL, 8)
    assert err.tolist() == [T.ERR_CAPACITY]


@pytest.mark.parametrize("mode", [0, 1])
def test_pack_dense_round_trip_and_refusals(mode):
    rng = np.random.default_rng(9)
    sizes = [5, 40, 1, 0, 33]
    pars = [synth.random_tree(rng, k) if k else np.zeros(0, np.int32) for k in sizes]
    par_all = np.concatenate(pars).astype(np.int32)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    ctx = np.array([3, 0, 7, 2, 1], np.int32)
    stride = 64
    dense, err = T.dense_mask(par_all, offs, ctx, mode, stride)
    assert not err.any()
    packed, err = T.pack_dense(dense, offs, ctx, mode, 2)
    assert not err.any()
    assert np.array_equal(packed, T.build(par_all, offs, ctx, 40, 2)["mask"])
    base = (lambda b: int(ctx[b])) if mode == 1 else (lambda b: 0)
    # a later node's column set (a sibling or child), and the own column cleared
    for b, (row, col) in ((1, (5, 9)), (4, (2, 2))):
        bad = dense.copy()
        i = offs[b] + row
        bad[i, base(b) + col] ^= 1
        _, err = T.pack_dense(bad, offs, ctx, mode, 2)
        assert err[b] == T.ERR_BAD_MASK and err.sum() == T.ERR_BAD_MASK
    if mode == 1:  # a hidden context column
        bad = dense.copy()
        bad[offs[0] + 1, 0] = 0
        _, err = T.pack_dense(bad, offs, ctx, mode, 2)
        assert err[0] == T.ERR_BAD_MASK


def test_merge_sequences_pin():
    """The glossary's three branches merge into its packed node table."""
    g = golden("packed_table.json")
    par, tok, node_of = T.merge_sequences(g["branches"])
    assert par == g["parents"] and tok == g["tokens"]
    assert len(par) == g["unique_tree_nodes"]
    assert sum(len(b) for b in g["branches"]) == g["branch_expanded_nodes"]
    # every sequence's last node spells the sequence from the root
    for m, br in enumerate(g["branches"]):
        assert [tok[j] for j in T.ancestor_path(node_of[m][-1], par)] == br


def test_merge_sequences_against_prefix_set():
    rng = np.random.default_rng(4)
    for _ in range(20):
        M, L = int(rng.integers(1, 12)), int(rng.integers(1, 6))
        seqs = rng.integers(0, 3, size=(M, L)).tolist()
        for s in seqs:  # ragged ends
            cut = int(rng.integers(0, L + 1))
            for d in range(cut, L):
                s[d] = -1
        par, tok, node_of = T.merge_sequences(seqs)
        assert T.parents_valid(par)
        prefixes = {tuple(s[:d + 1]) for s in seqs for d in range(L) if all(x >= 0 for x in s[:d + 1])}
        paths = [tuple(tok[j] for j in T.ancestor_path(i, par)) for i in range(len(par))]
        assert len(paths) == len(set(paths)) and set(paths) == prefixes
        depth = [T.depth_of(i, par) for i in range(len(par))]
        assert depth == sorted(depth)  # level order


def test_eagle_grow_hand_case():
    # k = 2, two layers: roots A (0.9), B (0.5); layer 1 expands both:
    # A -> C (0.9 * 0.8 = 0.72), D (0.9 * 0.1 = 0.09); B -> E (0.5 * 0.6 = 0.30), F (0.05)
    A, B, C, D, E, F = 10, 11, 12, 13, 14, 15
    par, tok = T.eagle_grow([A, B], [0.9, 0.5], [[[C, D], [E, F]]], [[[0.8, 0.1], [0.6, 0.1]]], 4)
    # best four: A 0.9, C 0.72, B 0.5, E 0.30; creation order A, B, C, E
    assert tok == [A, B, C, E] and par == [-1, -1, 0, 1]
    # the second layer expands only the two best of layer 1 (C, E), in score order
    par, tok = T.eagle_grow([A, B], [0.9, 0.5], [[[C, D], [E, F]], [[1, 2], [3, 4]]],
                            [[[0.8, 0.1], [0.6, 0.1]], [[0.9, 0.5], [0.99, 0.2]]], 7)
    assert tok == [A, B, C, E, 1, 2, 3] and par == [-1, -1, 0, 1, 2, 2, 3]


def test_eagle_grow_selection_by_path_product():
    """Every kept node's path product (recomputed from the inputs along its
    path) is at least every dropped node's; with the whole budget the tree
    holds k roots and k * k children per further layer, each layer's children
    hanging off the k best nodes of the layer before."""
    rng = np.random.default_rng(6)
    for _ in range(30):
        k, L = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        rt = np.arange(k)
        rc = rng.uniform(0.01, 0.99, size=k)
        ct = rng.integers(0, 1000, size=(L - 1, k, k)) + 1000 * np.arange(1, L)[:, None, None]
        cc = rng.uniform(0.01, 0.99, size=(L - 1, k, k))
        total = k + (L - 1) * k * k
        par, tok = T.eagle_grow(rt, rc, ct, cc, total)
        assert len(par) == total and T.parents_valid(par)
        # path product of every node: the confidence of each (layer, expanded slot, child)
        conf = {}
        for i in range(k):
            conf[i] = rc[i]
        depth = [T.depth_of(i, par) for i in range(total)]
        score = [0.0] * total
        for i in range(total):
            if par[i] < 0:
                score[i] = rc[tok[i]]
                continue
            l = depth[i]
            # siblings of i are the children of par[i]; their slot j is par[i]'s rank in its layer
            layer_prev = [x for x in range(total) if depth[x] == l - 1]
            ranked = sorted(layer_prev, key=lambda x: (-score[x], x))[:k]
            j = ranked.index(par[i])
            c = [x for x in range(total) if par[x] == par[i]].index(i)
            score[i] = score[par[i]] * cc[l - 1][j][c]
        for budget in range(1, total + 1):
            kp, kt = T.eagle_grow(rt, rc, ct, cc, budget)
            kept = sorted(range(total), key=lambda x: (-score[x], x))[:budget]
            assert sorted(tok[x] for x in kept) == sorted(kt)
