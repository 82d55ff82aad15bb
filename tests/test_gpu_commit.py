"""tree_kv_commit on the GPU against the oracle's copy-based commit: bit-exact."""

import numpy as np
import pytest

import synth
import token_tree_attention_amd as tta
from gpu_helpers import bits, host, region_bits, require_gpu, say
from oracle import commit as O_com

pytestmark = pytest.mark.gpu


def run_round(wl, max_accept=16):
    """build -> attention -> accept, snapshot the cache, then commit."""
    import torch
    from synth.device import to_device
    d = to_device(wl)
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], max(1, wl.n_max), total_nodes=wl.total_nodes)
    cache = tta.KVCache(d["k_cache"], d["v_cache"], d["block_table"])
    from token_tree_attention_amd.step import VerifyStep
    step = VerifyStep(bt, cache, wl.n_heads, wl.vocab, max_accept)
    step.build(d["parents"])
    step.attention(d["q"], d["k_new"], d["v_new"])
    step.accept(d["logits"], d["tokens"])
    torch.cuda.synchronize()
    pre_k, pre_v = bits(d["k_cache"]), bits(d["v_cache"])
    pre_table = None if d["block_table"] is None else host(d["block_table"]).copy()
    step.commit()
    torch.cuda.synchronize()
    return d, step, pre_k, pre_v, pre_table


@pytest.mark.parametrize("cfg,over", [
    (0, dict()),
    (1, dict(ctx=(70, 70), vocab=64)),
    (2, dict(batch=7, ctx=(20, 300), vocab=64)),
    (4, dict(batch=4, ctx=(10, 200), vocab=64, p=(1.0, 1.0))),
    (5, dict(ctx=(40, 40), vocab=64, ddtree_budget=150, batch=2, p=(1.0, 1.0))),
])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_commit_matches_copy(cfg, over, seed):
    require_gpu()
    import torch
    wl = synth.make_workload(cfg, seed, **over)
    say(f"tree_kv_commit cfg={cfg} seed={seed} {over} layout={wl.layout}")
    d, step, pre_k, pre_v, pre_table = run_round(wl)
    acc = {k: host(v) for k, v in step.acc.items()}
    com = {k: host(v) for k, v in step.com.items()}
    assert (host(step.meta["err"]) == 0).all()
    post_k, post_v = bits(d["k_cache"]), bits(d["v_cache"])
    a = acc["accept_len"]
    paths = [acc["accepted_nodes"][b, :a[b]].tolist() for b in range(wl.batch)]
    if wl.layout == "contiguous":
        rk, rv, nl = O_com.commit_contiguous(pre_k, pre_v, wl.ctx_lens, a, paths)
        np.testing.assert_array_equal(com["new_lens"], nl)
        for b in range(wl.batch):
            np.testing.assert_array_equal(post_k[b, :, :nl[b]], rk[b, :, :nl[b]])
            np.testing.assert_array_equal(post_v[b, :, :nl[b]], rv[b, :, :nl[b]])
    else:
        n = np.diff(wl.node_offsets)
        rk, rv, nl, tab, rel = O_com.commit_paged(pre_k, pre_v, pre_table, wl.ctx_lens, n, a, paths)
        np.testing.assert_array_equal(com["new_lens"], nl)
        np.testing.assert_array_equal(host(d["block_table"]), tab)
        for b in range(wl.batch):
            assert com["num_released"][b] == len(rel[b])
            assert com["released_blocks"][b, :len(rel[b])].tolist() == rel[b]
            assert (com["released_blocks"][b, len(rel[b]):] == -1).all()
            for slot in range(int(nl[b])):
                blk = int(pre_table[b, slot // 16])
                np.testing.assert_array_equal(post_k[blk, :, slot % 16], rk[blk, :, slot % 16])
                np.testing.assert_array_equal(post_v[blk, :, slot % 16], rv[blk, :, slot % 16])
    # Committed tokens beyond the context are the accepted nodes' tokens (slot bookkeeping).
    for b in range(wl.batch):
        s = int(wl.node_offsets[b])
        assert acc["out_tokens"][b, :a[b]].tolist() == [int(wl.tokens[s + j]) for j in paths[b]]


def test_commit_rejects_bad_paths():
    require_gpu()
    import torch
    wl = synth.make_workload(2, 9, batch=4, ctx=(20, 40), vocab=64)
    say("tree_kv_commit invalid accepted paths")
    d, step, pre_k, pre_v, pre_table = run_round(wl)
    # Corrupt: request 0 non-increasing ids, request 1 id out of range, request 2 len > max
    acc_nodes = step.acc["accepted_nodes"]
    acc_len = step.acc["accept_len"]
    acc_nodes[0, :2] = torch.tensor([3, 3], dtype=torch.int32)
    acc_len[0] = 2
    acc_nodes[1, 0] = 10 ** 6
    acc_len[1] = 1
    acc_len[2] = 17
    step.meta["err"].zero_()
    tbl_before = host(d["block_table"]).copy()
    k_before = bits(d["k_cache"])
    step.commit()
    torch.cuda.synchronize()
    err = host(step.meta["err"])
    assert err[0] & tta.ERR_ACCEPT and err[1] & tta.ERR_ACCEPT and err[2] & tta.ERR_ACCEPT
    nl = host(step.com["new_lens"])
    assert nl[:3].tolist() == wl.ctx_lens[:3].tolist()
    for b in range(3):
        assert (host(d["block_table"])[b] == tbl_before[b]).all()
