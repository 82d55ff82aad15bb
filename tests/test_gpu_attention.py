"""tree_attention_verify on the GPU against the float64 oracle.

Scaled cases span several 32-slot tiles, 128- and 256-row items (the two
row-tile sizes of the main kernel), requests of one to five row tiles,
split and unsplit contexts and ragged tails; outputs must be within 1e-2 + 1e-2|ref|,
the tentative K within one bf16 ulp of the rounded rotation, V exact.
"""

import numpy as np
import pytest

import synth
import token_tree_attention_amd as tta
from gpu_helpers import bits, region_bits, require_gpu, say
from parity import check_attention_request, check_tentative

pytestmark = pytest.mark.gpu


def run_attention(wl, rope_base=10000.0):
    import torch
    from synth.device import to_device
    d = to_device(wl)
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], max(1, wl.n_max), total_nodes=wl.total_nodes)
    cache = tta.KVCache(d["k_cache"], d["v_cache"], d["block_table"])
    meta = tta.tree_build(bt, d["parents"])
    out = tta.tree_attention_verify(bt, d["q"], d["k_new"], d["v_new"], meta["mask"], meta["positions"],
                                    cache, meta["err"], rope_base=rope_base)
    torch.cuda.synchronize()
    return d, bits(out), meta["err"].cpu().numpy()


SCALED = [
    # (cfg, overrides): several tiles of rows and keys, ragged tails
    (0, dict()),
    (0, dict(ctx=(300, 300))),
    (1, dict(ctx=(700, 700), vocab=64)),
    (1, dict(ctx=(33, 33), vocab=64)),
    (2, dict(batch=5, ctx=(100, 1300), vocab=64)),
    (3, dict(ctx=(513, 513), vocab=64, ddtree_budget=100, batch=2)),
    (4, dict(batch=3, ctx=(40, 900), vocab=64)),
    (5, dict(ctx=(257, 257), vocab=64, ddtree_budget=130, batch=2)),
    (2, dict(batch=3, ctx=(0, 0), vocab=64)),
    # enough row tiles for the 256-row items: paged, with requests of at most
    # 128 rows per KV head (one 16-row block per wave) next to larger ones
    (2, dict(batch=64, ctx=(30, 300), vocab=64)),
    # 256-row items over a contiguous cache, every tile full
    (1, dict(batch=40, ctx=(20, 200), vocab=64)),
    # five 256-row tiles per request and KV head (220-node trees, 5 query
    # heads per KV head), the last one partial
    (4, dict(batch=8, ctx=(40, 700), vocab=64)),
    # one or two 256-row tiles per request and KV head (8 query heads per KV
    # head, 16..64-node trees)
    (2, dict(batch=40, ctx=(30, 400), vocab=64, heads=(64, 8, 128))),
    # five 256-row tiles per request and KV head over contexts of more than
    # 128 key tiles: the partial last tile (76 rows) runs its five row blocks
    # in pairs on three waves, and more items than workgroups go through the
    # per-XCD work queues
    (4, dict(batch=8, ctx=(4000, 4200), vocab=64)),
    # 12-node trees, 5 query heads per KV head: one 60-row tile per request
    # and KV head (four single-block waves), single-chunk contexts next to
    # ones split into two chunks
    (4, dict(batch=64, ctx=(300, 600), vocab=64, tree=("medusa", (3, 3)))),
]


@pytest.mark.parametrize("case", range(len(SCALED)))
@pytest.mark.parametrize("seed", [0, 1])
def test_attention_scaled(case, seed):
    require_gpu()
    cfg, over = SCALED[case]
    wl = synth.make_workload(cfg, seed, **over)
    say(f"tree_attention_verify cfg={cfg} seed={seed} {over} T={wl.total_nodes} "
        f"heads={wl.n_heads}/{wl.n_kv_heads}/{wl.head_dim} layout={wl.layout}")
    d, out, err = run_attention(wl)
    assert (err == 0).all(), err
    for b in range(wl.batch):
        sl = wl.request_nodes(b)
        check_attention_request(wl, b, out[sl])
        n = sl.stop - sl.start
        kb = region_bits(d, wl, b, int(wl.ctx_lens[b]), n, "k")
        vb = region_bits(d, wl, b, int(wl.ctx_lens[b]), n, "v")
        check_tentative(wl, b, kb, vb)


def test_attention_small_tiles_long_context():
    """80-row tiles (16-node trees, 5 query heads per KV head: five row
    blocks, run in pairs on three waves) over single-chunk contexts of at
    least 4096 slots; every node of three requests against the oracle."""
    require_gpu()
    wl = synth.make_workload(4, 0, batch=56, ctx=(4096, 4200), vocab=64, tree=("medusa", (4, 3)))
    say(f"tree_attention_verify 80-row tiles T={wl.total_nodes} ctx={int(wl.ctx_lens.min())}.."
        f"{int(wl.ctx_lens.max())}")
    d, out, err = run_attention(wl)
    assert (err == 0).all(), err
    for b in (0, wl.batch // 2, wl.batch - 1):
        sl = wl.request_nodes(b)
        check_attention_request(wl, b, out[sl])
        n = sl.stop - sl.start
        kb = region_bits(d, wl, b, int(wl.ctx_lens[b]), n, "k")
        vb = region_bits(d, wl, b, int(wl.ctx_lens[b]), n, "v")
        check_tentative(wl, b, kb, vb)


def test_attention_rope_base_and_capacity_flag():
    require_gpu()
    wl = synth.make_workload(1, 3, ctx=(90, 90), vocab=64)
    say("tree_attention_verify rope_base=500000")
    d, out, err = run_attention(wl, rope_base=500000.0)
    check_attention_request(wl, 0, out, rope_base=500000.0)
    # A contiguous cache too small for ctx + N flags the request and writes nothing outside.
    import torch
    small = wl.ctx_lens[0] + wl.total_nodes - 1
    k = d["k_cache"][:, :, :small].contiguous()
    v = d["v_cache"][:, :, :small].contiguous()
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=wl.total_nodes)
    meta = tta.tree_build(bt, d["parents"])
    tta.tree_attention_verify(bt, d["q"], d["k_new"], d["v_new"], meta["mask"], meta["positions"],
                              tta.KVCache(k, v), meta["err"])
    torch.cuda.synchronize()
    assert meta["err"].cpu().numpy()[0] & tta.ERR_CAPACITY


def test_attention_softmax_scale_argument():
    require_gpu()
    import torch
    wl = synth.make_workload(0, 5)
    d = __import__("synth.device", fromlist=["to_device"]).to_device(wl)
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=wl.total_nodes)
    meta = tta.tree_build(bt, d["parents"])
    cache = tta.KVCache(d["k_cache"], d["v_cache"])
    o0 = tta.tree_attention_verify(bt, d["q"], d["k_new"], d["v_new"], meta["mask"], meta["positions"],
                                   cache, meta["err"], softmax_scale=0.0).clone()
    o1 = tta.tree_attention_verify(bt, d["q"], d["k_new"], d["v_new"], meta["mask"], meta["positions"],
                                   cache, meta["err"], softmax_scale=1.0 / 8.0)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)  # 1/sqrt(64) explicitly == default


def test_attention_unmapped_block_flags_only_its_request():
    """A paged request whose tentative block is unmapped (-1) is flagged with
    ERR_BLOCK_TABLE; its neighbours are unaffected and match the oracle."""
    require_gpu()
    import torch
    from synth.device import to_device
    wl = synth.make_workload(2, 4, batch=3, ctx=(60, 400), vocab=64)
    assert wl.layout == "paged"
    d = to_device(wl)
    bad = 1
    c = int(wl.ctx_lens[bad])
    table = d["block_table"]
    table[bad, c // 16] = -1  # the block holding the request's first tree slot
    say(f"tree_attention_verify with block {c // 16} of request {bad} unmapped")
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=wl.total_nodes)
    meta = tta.tree_build(bt, d["parents"])
    out = tta.tree_attention_verify(bt, d["q"], d["k_new"], d["v_new"], meta["mask"], meta["positions"],
                                    tta.KVCache(d["k_cache"], d["v_cache"], table), meta["err"])
    torch.cuda.synchronize()
    err = meta["err"].cpu().numpy()
    assert err[bad] & tta.ERR_BLOCK_TABLE, err
    for b in range(wl.batch):
        if b == bad:
            continue
        assert err[b] == 0, err
        check_attention_request(wl, b, bits(out)[wl.request_nodes(b)])


def test_attention_unmapped_context_block_in_a_large_batch():
    """Enough items for cost-ordered placement (40 paged requests): an unmapped
    block in the middle of one request's context (a whole-tile load) flags
    only that request; every other request matches the oracle."""
    require_gpu()
    import torch
    from synth.device import to_device
    wl = synth.make_workload(2, 6, batch=40, ctx=(600, 1500), vocab=64)
    assert wl.layout == "paged"
    d = to_device(wl)
    bad = 7
    table = d["block_table"]
    table[bad, 5] = -1  # slots 80..95, inside the committed context
    say(f"tree_attention_verify, B=40, block 5 of request {bad} unmapped")
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=wl.total_nodes)
    meta = tta.tree_build(bt, d["parents"])
    out = tta.tree_attention_verify(bt, d["q"], d["k_new"], d["v_new"], meta["mask"], meta["positions"],
                                    tta.KVCache(d["k_cache"], d["v_cache"], table), meta["err"])
    torch.cuda.synchronize()
    err = meta["err"].cpu().numpy()
    assert err[bad] & tta.ERR_BLOCK_TABLE, err
    ob = bits(out)
    for b in range(wl.batch):
        if b == bad:
            continue
        assert err[b] == 0, (b, err[b])
        check_attention_request(wl, b, ob[wl.request_nodes(b)])


def test_attention_many_small_requests():
    """600 paged requests of 1..8 nodes, one query head per KV head, head_dim
    64: thousands of short items dealt in cost order, two nodes per prep
    workgroup; every request matches the oracle."""
    require_gpu()
    wl = synth.make_workload(2, 8, batch=600, ctx=(1, 200), tree=("random", (1, 8)),
                             heads=(8, 8, 64), vocab=64)
    say(f"tree_attention_verify B=600 T={wl.total_nodes} heads=8/8/64")
    d, out, err = run_attention(wl)
    assert (err == 0).all(), err
    for b in range(wl.batch):
        check_attention_request(wl, b, out[wl.request_nodes(b)])
