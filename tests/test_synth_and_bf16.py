"""Input generators and bf16 helpers, pinned against library routines and brute force."""

import itertools

import numpy as np
import pytest
import torch

import synth
from oracle import bf16 as OB
from oracle import tree as T


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, -1e-42], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.bf16_bits_from_f32(x), ref)
    # Oracle's float64 -> bf16 rounding agrees on values exact in float32
    np.testing.assert_array_equal(OB.from_f64(x.astype(np.float64)), ref)
    np.testing.assert_array_equal(OB.to_f64(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_bf16_from_f64_ties_and_double_rounding():
    # 1 + 2^-8 is exactly half-way between bf16 1.0 and 1.0078125: ties to even -> 1.0
    assert OB.from_f64(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 is half-way between 1.0078125 (odd) and 1.015625 (even) -> up
    assert OB.from_f64(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
    # just above the half-way point rounds up (a float32 detour would lose this)
    assert OB.from_f64(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    assert OB.ulp(np.array([0x3F80], np.uint16))[0] == 2.0 ** -7


def test_medusa_tree_shape():
    par = synth.medusa_tree((10, 3, 2, 2))
    md = T.build_request(par, 0)
    assert len(par) == 220
    assert sorted(set(md["depth"])) == [0, 1, 2, 3]
    toks = synth.medusa_tokens(np.random.default_rng(0), (10, 3, 2, 2), 32000)
    for p in set(par.tolist()):
        kids = [toks[j] for j in range(len(par)) if par[j] == p]
        assert len(set(kids)) == len(kids)


def test_eagle_tree_shape():
    for seed in range(5):
        par = synth.eagle_tree(np.random.default_rng(seed))
        assert len(par) == 64
        assert T.parents_valid(par)
        md = T.build_request(par, 0)
        assert max(md["depth"]) <= 5      # 6 levels
        assert sum(1 for p in par if p == -1) <= 4


def test_random_tree_levels():
    for seed in range(5):
        rng = np.random.default_rng(seed)
        par = synth.random_tree(rng, 64)
        assert T.parents_valid(par) and par[0] == -1 and (par[1:] >= 0).all()
        assert max(T.build_request(par, 0)["depth"]) <= 7


def brute_top_prefixes(logq, budget):
    L, K = logq.shape
    scored = []
    for d in range(1, L + 1):
        for ranks in itertools.product(range(K), repeat=d):
            scored.append((sum(logq[i][r] for i, r in enumerate(ranks)), ranks))
    scored.sort(key=lambda t: -t[0])
    return [r for _, r in scored[:budget]]


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_ddtree_heap_equals_bruteforce(seed):
    vocab, L, B = 5, 3, 9
    rng = np.random.default_rng(seed)
    par, tok = synth.ddtree_tree(np.random.default_rng(seed), vocab, depths=L, topk=vocab, budget=B, sigma=1.5)
    # Rebuild the same draft logits to know the ranks.
    r2 = np.random.default_rng(seed)
    logq, order = [], []
    for _ in range(L):
        z = r2.standard_normal(vocab) * 1.5
        idx = np.argsort(-z, kind="stable")
        zz = z[idx]
        logq.append(zz - (zz.max() + np.log(np.exp(zz - zz.max()).sum())))
        order.append(idx)
    best = brute_top_prefixes(np.array(logq), B)
    got = []
    for i in range(len(par)):
        path = T.ancestor_path(i, par)
        got.append(tuple(int(np.nonzero(order[d] == tok[j])[0][0]) for d, j in enumerate(path)))
    assert sorted(got) == sorted(best)
    assert T.parents_valid(par)
    # prefix-closed
    gs = set(got)
    assert all(g[:-1] in gs for g in got if len(g) > 1)


def test_ddtree_literal_reading_is_flat():
    par, _ = synth.ddtree_tree(np.random.default_rng(0), 151936, depths=16, topk=1024, budget=1024, sigma=2.0)
    d = T.build_request(par, 0)["depth"]
    assert len(par) == 1024 and d.count(0) >= 1000


def test_planted_logits_unique_max():
    wl = synth.make_workload(2, 0, batch=3, ctx=(5, 9), vocab=300)
    vals = OB.to_f64(wl.logits)
    for r in range(vals.shape[0]):
        t = wl.planted[r]
        assert (vals[r] < vals[r, t]).sum() == vals.shape[1] - 1
    wl0 = synth.make_workload(0, 0)
    assert wl0.logits.dtype == np.float32 and wl0.logits.shape == (9, 1000)
    assert wl0.n_max == 8 and wl0.ctx_lens.tolist() == [7]
    for r in range(9):
        assert np.argmax(wl0.logits[r]) == wl0.planted[r]
        assert (wl0.logits[r] == wl0.logits[r].max()).sum() == 1


def test_paged_tables_cover_tree_and_shuffle():
    wl = synth.make_workload(2, 1, batch=5, ctx=(30, 90), vocab=64)
    assert wl.layout == "paged"
    used = []
    for b in range(5):
        need = -(-(int(wl.ctx_lens[b]) + int(np.diff(wl.node_offsets)[b])) // 16)
        row = wl.block_table[b]
        assert (row[:need] >= 0).all() and (row[need:] == -1).all()
        used.extend(row[:need].tolist())
    assert sorted(used) == list(range(wl.k_cache.shape[0]))
