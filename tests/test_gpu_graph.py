"""A verification round captured in a HIP graph replays to the eager result.

Each replay is checked against the eager outputs, with eager work and
synchronisations in between, for a paged batch (with the block-table
restore the benchmark captures) and a contiguous one.
"""

import numpy as np
import pytest

import synth
import token_tree_attention_amd as tta
from gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,over", [
    (2, dict(batch=6, ctx=(100, 900), vocab=3000)),
    (1, dict(ctx=(600, 600), vocab=3000)),
])
def test_graph_replay_matches_eager(cfg, over):
    require_gpu()
    import torch
    from synth.device import to_device
    from token_tree_attention_amd.step import VerifyStep
    wl = synth.make_workload(cfg, 0, **over)
    say(f"graph replay cfg={cfg} {over}")
    d = to_device(wl)
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=wl.total_nodes)
    cache = tta.KVCache(d["k_cache"], d["v_cache"], d["block_table"])
    st = VerifyStep(bt, cache, wl.n_heads, wl.vocab, 16)
    table0 = None if d["block_table"] is None else d["block_table"].clone()
    k0, v0 = d["k_cache"].clone(), d["v_cache"].clone()

    def reset():
        d["k_cache"].copy_(k0)
        d["v_cache"].copy_(v0)
        if table0 is not None:
            d["block_table"].copy_(table0)

    def round_():
        if table0 is not None:
            d["block_table"].copy_(table0)
        st.run(d["parents"], d["tokens"], d["q"], d["k_new"], d["v_new"], d["logits"])

    def snapshot():
        torch.cuda.synchronize()
        snap = {"out": st.out.clone(), "k": d["k_cache"].clone(), "v": d["v_cache"].clone()}
        for name, group in (("meta", st.meta), ("acc", st.acc), ("com", st.com)):
            for k, t in group.items():
                snap[f"{name}.{k}"] = t.clone()
        if table0 is not None:
            snap["table"] = d["block_table"].clone()
        return snap

    reset()
    round_()
    ref = snapshot()
    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        round_()
    for rep in range(3):
        reset()
        st.out.zero_()
        for t in list(st.acc.values()) + list(st.com.values()):
            t.fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for k in ref:
            assert torch.equal(got[k], ref[k]), f"replay {rep}: {k} differs"
        # eager work between replays
        reset()
        round_()
        again = snapshot()
        for k in ref:
            assert torch.equal(again[k], ref[k]), f"eager after replay {rep}: {k} differs"
