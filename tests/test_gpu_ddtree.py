"""tree_ddtree_build on the GPU against the oracle, bit-exact: the pop order
(node numbering), parents, tokens and node count of every request, including
logits with many exact ties and a budget larger than the number of prefixes;
and the trees feed tree_build as they come out."""

import numpy as np
import pytest

import synth
import token_tree_attention_amd as tta
from gpu_helpers import host, require_gpu, say
from oracle import ddtree as O_dd
from oracle import tree as O_tree

pytestmark = pytest.mark.gpu

CASES = [
    # (requests, depths, vocab, budget, sigma, levels)
    (2, 3, 50, 20, 2.0, 0),
    (2, 2, 3, 20, 2.0, 0),          # 3 + 9 prefixes: the heap empties before the budget
    (3, 16, 4096, 300, 2.0, 0),
    (3, 16, 4096, 300, 8.0, 0),     # deep trees
    (2, 6, 2000, 500, 1.0, 2),      # logits on a 0.5 grid: ties in the top-K and in the scores
    (4, 16, 151936, 1024, 2.0, 0),  # the DDTree workload's shape
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_ddtree_build_matches_oracle(case):
    require_gpu()
    import torch
    R, L, V, budget, sigma, levels = CASES[case]
    z = synth.draft_logits(case, 3, R, L, V, sigma, levels)
    say(f"tree_ddtree_build R={R} L={L} V={V} budget={budget} sigma={sigma} levels={levels}")
    out = tta.tree_ddtree_build(torch.from_numpy(z).cuda(), budget)
    torch.cuda.synchronize()
    par, tok, nn = host(out["parents"]), host(out["tokens"]), host(out["n_nodes"])
    for r in range(R):
        rp, rt = O_dd.build_tree(z[r], budget)
        assert nn[r] == len(rp)
        np.testing.assert_array_equal(par[r, :nn[r]], rp, err_msg=f"parents of request {r}")
        np.testing.assert_array_equal(tok[r, :nn[r]], rt, err_msg=f"tokens of request {r}")
        assert (par[r, nn[r]:] == -1).all() and (tok[r, nn[r]:] == -1).all()


def test_ddtree_trees_feed_tree_build():
    require_gpu()
    import torch
    R, L, V, budget = 3, 16, 8192, 1024
    z = synth.draft_logits(9, 3, R, L, V, 4.0)
    out = tta.tree_ddtree_build(torch.from_numpy(z).cuda(), budget)
    nn = host(out["n_nodes"])
    offs = np.concatenate([[0], np.cumsum(nn)]).astype(np.int32)
    parents = torch.cat([out["parents"][r, :nn[r]] for r in range(R)]).contiguous()
    ctx = np.array([100, 0, 5000], np.int32)
    bt = tta.Batch(torch.from_numpy(offs).cuda(), torch.from_numpy(ctx).cuda(), int(nn.max()),
                   total_nodes=int(offs[-1]))
    meta = tta.tree_build(bt, parents)
    torch.cuda.synchronize()
    assert (host(meta["err"]) == 0).all()
    ref = O_tree.build(host(parents), offs, ctx, int(nn.max()), meta["mask"].shape[1])
    np.testing.assert_array_equal(host(meta["mask"]).view(np.uint32), ref["mask"])
    np.testing.assert_array_equal(host(meta["positions"]), ref["positions"])


@pytest.mark.parametrize("seed, R, M, L, alphabet", [(0, 1, 3, 3, 10), (1, 4, 16, 8, 3), (2, 3, 200, 6, 4),
                                                     (3, 2, 1024, 12, 2), (4, 5, 64, 40, 2)])
def test_merge_sequences_matches_oracle(seed, R, M, L, alphabet):
    require_gpu()
    import torch
    rng = np.random.default_rng(seed)
    seqs = rng.integers(0, alphabet, size=(R, M, L)).astype(np.int32)
    ends = rng.integers(0, L + 1, size=(R, M))
    for r in range(R):
        for m in range(M):
            seqs[r, m, ends[r, m]:] = -1
    if seed == 0:  # the glossary's three branches
        seqs[0] = np.array([[4, 5, 6], [4, 7, 8], [9, 0, 1]], np.int32)
    say(f"tree_merge_sequences R={R} M={M} L={L} alphabet={alphabet}")
    out = tta.tree_merge_sequences(torch.from_numpy(seqs).cuda(), 1024)
    torch.cuda.synchronize()
    par, tok, nn, err = (host(out[k]) for k in ("parents", "tokens", "n_nodes", "err"))
    for r in range(R):
        rp, rt, _ = O_tree.merge_sequences([[int(x) for x in s] for s in seqs[r]])
        if len(rp) > 1024:
            assert err[r] & tta.ERR_TOO_MANY_NODES and nn[r] == 0
            continue
        assert err[r] == 0 and nn[r] == len(rp)
        np.testing.assert_array_equal(par[r, :nn[r]], rp)
        np.testing.assert_array_equal(tok[r, :nn[r]], rt)
    if seed == 0:
        assert par[0, :8].tolist() == [-1, -1, 0, 0, 1, 2, 3, 4] and tok[0, :8].tolist() == [4, 9, 5, 7, 0, 6, 8, 1]


def test_merge_sequences_overflow_flag():
    require_gpu()
    import torch
    seqs = np.arange(2 * 30 * 5, dtype=np.int32).reshape(2, 30, 5)  # 150 distinct prefixes per request
    out = tta.tree_merge_sequences(torch.from_numpy(seqs).cuda(), 100)
    torch.cuda.synchronize()
    assert (host(out["err"]) & tta.ERR_TOO_MANY_NODES).all() and (host(out["n_nodes"]) == 0).all()


@pytest.mark.parametrize("seed, R, k, L, budget, tie", [(0, 1, 4, 6, 64, False), (1, 5, 4, 6, 64, False),
                                                        (2, 3, 8, 5, 200, False), (3, 2, 16, 16, 1024, False),
                                                        (4, 4, 4, 4, 1024, False), (5, 3, 6, 5, 100, True)])
def test_eagle_grow_matches_oracle(seed, R, k, L, budget, tie):
    require_gpu()
    import torch
    rng = np.random.default_rng(seed)
    rt = rng.integers(0, 32000, size=(R, k)).astype(np.int32)
    rc = rng.uniform(0.01, 0.99, size=(R, k)).astype(np.float32)
    ct = rng.integers(0, 32000, size=(R, L - 1, k, k)).astype(np.int32)
    cc = rng.uniform(0.01, 0.99, size=(R, L - 1, k, k)).astype(np.float32)
    if tie:  # confidences on a coarse grid: many equal path products
        rc = (np.round(rc * 4) / 4 + 0.25).clip(0.25, 0.75).astype(np.float32)
        cc = (np.round(cc * 2) / 2).clip(0.5, 0.5).astype(np.float32)
    say(f"tree_eagle_grow R={R} k={k} L={L} budget={budget} tie={tie}")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = tta.tree_eagle_grow(t(rt), t(rc), t(ct), t(cc), budget)
    torch.cuda.synchronize()
    par, tok, nn = host(out["parents"]), host(out["tokens"]), host(out["n_nodes"])
    for r in range(R):
        rp, rtk = O_tree.eagle_grow(rt[r], rc[r], ct[r], cc[r], budget)
        assert nn[r] == len(rp)
        np.testing.assert_array_equal(par[r, :nn[r]], rp, err_msg=f"parents {r}")
        np.testing.assert_array_equal(tok[r, :nn[r]], rtk, err_msg=f"tokens {r}")
        assert (par[r, nn[r]:] == -1).all()
