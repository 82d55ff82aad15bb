"""Full-size verification rounds on the GPU, in the launch configuration the
benchmark times, against the oracle: metadata, row argmax and acceptance in
full (bit-exact); attention on sampled nodes (tolerance); tentative K/V and
the commit on sampled requests (bit-exact / 1 ulp for rotated K)."""

import numpy as np
import pytest

import synth
import token_tree_attention_amd as tta
from gpu_helpers import bits, host, region_bits, require_gpu, say
from parity import check_accept, check_attention_request, check_build, check_tentative

pytestmark = pytest.mark.gpu

MAX_ACCEPT = 32


def sample_nodes(wl, b, k=4):
    n = int(wl.node_offsets[b + 1] - wl.node_offsets[b])
    par = wl.parents[wl.request_nodes(b)]
    depth = np.zeros(n, int)
    for i in range(n):
        depth[i] = 0 if par[i] < 0 else depth[par[i]] + 1
    picks = {0, n - 1, int(np.argmax(depth)), n // 2}
    return sorted(p for p in picks if 0 <= p < n)[:k]


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5])
def test_full_round(cfg):
    require_gpu()
    import torch
    from synth.device import to_device
    from token_tree_attention_amd.step import VerifyStep
    say(f"full round cfg={cfg}: generating inputs")
    wl = synth.make_workload(cfg, 0)
    d = to_device(wl)
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=wl.total_nodes)
    cache = tta.KVCache(d["k_cache"], d["v_cache"], d["block_table"])
    step = VerifyStep(bt, cache, wl.n_heads, wl.vocab, MAX_ACCEPT)
    say(f"full round cfg={cfg} {wl.name}: B={wl.batch} T={wl.total_nodes} layout={wl.layout}")
    step.build(d["parents"])
    step.attention(d["q"], d["k_new"], d["v_new"])
    step.accept(d["logits"], d["tokens"])
    torch.cuda.synchronize()
    meta = {k: host(v) for k, v in step.meta.items()}
    assert (meta["err"] == 0).all(), meta["err"]
    check_build(wl, meta)
    acc = {k: host(v) for k, v in step.acc.items()}
    check_accept(wl, acc, MAX_ACCEPT)
    out = bits(step.out)
    reqs = sorted({0, wl.batch - 1, wl.batch // 2})
    snap = {}
    for b in reqs:
        n = int(wl.node_offsets[b + 1] - wl.node_offsets[b])
        c = int(wl.ctx_lens[b])
        kb, vb = region_bits(d, wl, b, c, n, "k"), region_bits(d, wl, b, c, n, "v")
        check_tentative(wl, b, kb, vb)
        snap[b] = (kb, vb, region_bits(d, wl, b, max(0, c - 3), min(3, c), "k"))
        nodes = sample_nodes(wl, b)
        sl = wl.request_nodes(b)
        check_attention_request(wl, b, out[sl][nodes], nodes=nodes)
        say(f"  request {b}: ctx={c} n={n} sampled nodes {nodes} ok")
    table_before = None if d["block_table"] is None else host(d["block_table"]).copy()
    step.commit()
    torch.cuda.synchronize()
    com = {k: host(v) for k, v in step.com.items()}
    assert (host(step.meta["err"]) == 0).all()
    for b in reqs:
        a = int(acc["accept_len"][b])
        c = int(wl.ctx_lens[b])
        path = acc["accepted_nodes"][b, :a].tolist()
        assert com["new_lens"][b] == c + a
        kb, vb, ctx_tail = snap[b]
        ka = region_bits(d, wl, b, c, a, "k", table=torch.from_numpy(table_before).cuda() if table_before is not None else None)
        va = region_bits(d, wl, b, c, a, "v", table=torch.from_numpy(table_before).cuda() if table_before is not None else None)
        np.testing.assert_array_equal(ka, kb[:, path])
        np.testing.assert_array_equal(va, vb[:, path])
        tail_now = region_bits(d, wl, b, max(0, c - 3), min(3, c), "k",
                               table=torch.from_numpy(table_before).cuda() if table_before is not None else None)
        np.testing.assert_array_equal(tail_now, ctx_tail)
        if table_before is not None:
            n = int(wl.node_offsets[b + 1] - wl.node_offsets[b])
            first, last = -(-(c + a) // 16), -(-(c + n) // 16)
            assert com["num_released"][b] == last - first
            assert com["released_blocks"][b, :last - first].tolist() == table_before[b, first:last].tolist()
    say(f"full round cfg={cfg}: accept lengths {np.bincount(acc['accept_len']).tolist()}")


def test_round_with_empty_and_context_free_requests():
    """A paged batch where some requests have no tree (0 nodes) and some no
    committed context: every request's metadata, attention, acceptance and
    commit against the oracle; an empty request accepts nothing and commits
    nothing."""
    require_gpu()
    import torch
    from synth.device import to_device
    from token_tree_attention_amd.step import VerifyStep
    wl = synth.make_workload(2, 3, batch=24, ctx=(0, 300), tree=("random", (0, 5)), vocab=64)
    sizes = np.diff(wl.node_offsets)
    assert (sizes == 0).any() and (sizes > 0).any()
    d = to_device(wl)
    ctx = d["ctx_lens"].clone()
    ctx[1] = 0  # a request with a tree but no committed context
    d["ctx_lens"] = ctx
    wl.ctx_lens[1] = 0
    say(f"round with empty requests {np.flatnonzero(sizes == 0).tolist()}, B={wl.batch} T={wl.total_nodes}")
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=wl.total_nodes)
    cache = tta.KVCache(d["k_cache"], d["v_cache"], d["block_table"])
    step = VerifyStep(bt, cache, wl.n_heads, wl.vocab, MAX_ACCEPT)
    step.build(d["parents"])
    step.attention(d["q"], d["k_new"], d["v_new"])
    step.accept(d["logits"], d["tokens"])
    torch.cuda.synchronize()
    meta = {k: host(v) for k, v in step.meta.items()}
    assert (meta["err"] == 0).all(), meta["err"]
    check_build(wl, meta)
    acc = {k: host(v) for k, v in step.acc.items()}
    check_accept(wl, acc, MAX_ACCEPT)
    out = bits(step.out)
    for b in range(wl.batch):
        if sizes[b] > 0:
            check_attention_request(wl, b, out[wl.request_nodes(b)])
        else:
            assert acc["accept_len"][b] == 0
    step.commit()
    torch.cuda.synchronize()
    com = {k: host(v) for k, v in step.com.items()}
    assert (host(step.meta["err"]) == 0).all()
    np.testing.assert_array_equal(com["new_lens"], wl.ctx_lens + acc["accept_len"])
