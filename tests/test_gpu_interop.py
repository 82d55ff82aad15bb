"""Interop forms on the GPU: the dense mask modes and graph buckets.

* tree_expand_mask after tree_build equals the oracle's dense FULL_MASK /
  QLEN_ONLY rows byte for byte; tree_pack_mask of those rows gives back
  tree_build's packed rows; planted bad rows are refused per request.
* A round replayed from a tree-size bucket's HIP graph (static buffers larger
  than the round) gives the eager round's metadata, acceptance and commit
  bit for bit and its attention within the oracle's tolerance, replay after
  replay, across buckets, with eager work in between.
"""

import numpy as np
import pytest

import synth
import token_tree_attention_amd as tta
from gpu_helpers import bits, host, require_gpu, say
from oracle import tree as O_tree
from parity import check_attention_request

pytestmark = pytest.mark.gpu


def built(wl):
    import torch
    from synth.device import to_device
    d = to_device(wl)
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], max(1, wl.n_max), total_nodes=wl.total_nodes)
    meta = tta.tree_build(bt, d["parents"])
    return torch, d, bt, meta


MASK_CASES = [
    (0, dict()),
    (2, dict(batch=9, ctx=(0, 700), vocab=64)),
    (4, dict(batch=3, ctx=(5, 300), vocab=64)),
    (3, dict(batch=1, ctx=(33, 33), vocab=64)),   # 1024-node DDTree tree: 32 words per row
]


@pytest.mark.parametrize("case", range(len(MASK_CASES)))
@pytest.mark.parametrize("mode", [0, 1])
def test_expand_and_pack_mask(case, mode):
    require_gpu()
    cfg, over = MASK_CASES[case]
    wl = synth.make_workload(cfg, 1, **over)
    stride = int((wl.ctx_lens + np.diff(wl.node_offsets)).max()) if mode == 1 else wl.n_max
    stride += 5  # not a multiple of 16 here: the byte path
    for st in (stride, -(-stride // 16) * 16):  # and a multiple of 16: the 16-byte path
        say(f"tree_expand_mask / tree_pack_mask cfg={cfg} mode={mode} stride={st} T={wl.total_nodes}")
        torch, d, bt, meta = built(wl)
        dense = tta.tree_expand_mask(bt, meta["mask"], mode, st, meta["err"])
        torch.cuda.synchronize()
        ref, rerr = O_tree.dense_mask(wl.parents, wl.node_offsets, wl.ctx_lens, mode, st)
        assert (host(meta["err"]) == rerr).all() and not rerr.any()
        np.testing.assert_array_equal(host(dense), ref)
        packed = tta.tree_pack_mask(bt, dense, mode, meta["err"], mask_words=meta["mask"].shape[1])
        torch.cuda.synchronize()
        assert (host(meta["err"]) == 0).all()
        np.testing.assert_array_equal(host(packed), host(meta["mask"]))


def test_pack_mask_refuses_bad_rows_per_request():
    require_gpu()
    wl = synth.make_workload(2, 3, batch=6, ctx=(10, 90), vocab=64)
    mode = 1
    stride = int((wl.ctx_lens + np.diff(wl.node_offsets)).max())
    dense, _ = O_tree.dense_mask(wl.parents, wl.node_offsets, wl.ctx_lens, mode, stride)
    off, ctx = wl.node_offsets, wl.ctx_lens
    bad = dense.copy()
    bad[off[1] + 0, 3] = 0                          # request 1: a hidden context column
    bad[off[3] + 2, ctx[3] + 2] = 0                 # request 3: a node that does not see itself
    bad[off[4] + 1, ctx[4] + 2] = 1                 # request 4: a later node visible
    torch, d, bt, meta = built(wl)
    packed = tta.tree_pack_mask(bt, torch.from_numpy(bad).cuda(), mode, meta["err"], mask_words=meta["mask"].shape[1])
    torch.cuda.synchronize()
    ref, rerr = O_tree.pack_dense(bad, off, ctx, mode, meta["mask"].shape[1])
    err = host(meta["err"])
    np.testing.assert_array_equal(err, rerr)
    assert [b for b in range(wl.batch) if err[b]] == [1, 3, 4]
    good = np.concatenate([np.arange(off[b], off[b + 1]) for b in range(wl.batch) if not err[b]])
    np.testing.assert_array_equal(host(packed).view(np.uint32)[good], ref[good])


def test_graph_buckets_replay_rounds_of_several_sizes():
    require_gpu()
    import torch
    from synth.device import to_device
    from token_tree_attention_amd.graphs import GraphBuckets
    from token_tree_attention_amd.step import VerifyStep
    B, V = 4, 3000
    rounds = [synth.make_workload(2, s, batch=B, ctx=(200, 900), tree=("random", tr), vocab=V, layout="contiguous",
                                  spare_slots=64)
              for s, tr in ((0, (5, 20)), (1, (30, 60)), (2, (70, 120)), (3, (8, 16)))]
    cap = max(wl.k_cache.shape[2] for wl in rounds)
    dev = torch.device("cuda")
    k = torch.zeros((B, 8, cap, 128), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    cache = tta.KVCache(k, v)
    gb = GraphBuckets(cache, B, 32, V, max_accept=16, buckets=[(128, 64), (512, 128)])

    def load_cache(wl):
        k.zero_()
        v.zero_()
        c = wl.k_cache.shape[2]
        k[:, :, :c].copy_(to_device(wl, dev)["k_cache"])
        v[:, :, :c].copy_(to_device(wl, dev)["v_cache"])

    for rep in range(2):
        for wl in rounds:
            d = to_device(wl, dev)
            say(f"graph bucket round rep={rep} T={wl.total_nodes} n_max={wl.n_max}")
            # eager reference on the exact sizes
            load_cache(wl)
            bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=wl.total_nodes)
            ref = VerifyStep(bt, cache, 32, V, 16)
            ref.run(d["parents"], d["tokens"], d["q"], d["k_new"], d["v_new"], d["logits"])
            torch.cuda.synchronize()
            ref_meta = {kk: host(t) for kk, t in ref.meta.items()}
            ref_acc = {kk: host(t) for kk, t in ref.acc.items() if kk != "row_argmax"}
            ref_new = host(ref.com["new_lens"])
            ref_k = host(k.view(torch.int16)).copy()
            ref_out = bits(ref.out)
            # the same round through the bucket's graph
            load_cache(wl)
            st = gb.run(d["node_offsets"], d["ctx_lens"], d["parents"], d["tokens"], d["q"], d["k_new"],
                        d["v_new"], d["logits"], wl.total_nodes, wl.n_max)
            torch.cuda.synchronize()
            T = wl.total_nodes
            for kk in ("depth", "positions", "retrieve_index", "retrieve_next_token", "retrieve_next_sibling"):
                np.testing.assert_array_equal(host(st.meta[kk])[:T], ref_meta[kk], err_msg=kk)
            W = ref_meta["mask"].shape[1]
            np.testing.assert_array_equal(host(st.meta["mask"])[:T, :W], ref_meta["mask"])
            assert not host(st.meta["mask"])[:T, W:].any()
            np.testing.assert_array_equal(host(st.meta["err"]), ref_meta["err"])
            for kk, val in ref_acc.items():
                np.testing.assert_array_equal(host(st.acc[kk]), val, err_msg=kk)
            np.testing.assert_array_equal(host(st.com["new_lens"]), ref_new)
            # committed slots (the whole context up to new_len) are bit-identical
            for b in range(B):
                nl = int(ref_new[b])
                np.testing.assert_array_equal(host(k.view(torch.int16))[b, :, :nl], ref_k[b, :, :nl])
            out = bits(st.out)[:T]
            for b in range(B):
                check_attention_request(wl, b, out[wl.request_nodes(b)])
                check_attention_request(wl, b, ref_out[wl.request_nodes(b)])
            # eager work between replays
            torch.cuda.synchronize()
