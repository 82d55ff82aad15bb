"""tree_greedy_accept_noalloc (static device scratch, no workspace) against
tree_greedy_accept (caller's workspace): bit-exact on every output, on two
calls in a row, the second with a smaller input, and both against the oracle."""

import pytest

import synth
import token_tree_attention_amd as tta
from gpu_helpers import host, require_gpu, say
from parity import check_accept

pytestmark = pytest.mark.gpu

MAX_ACCEPT = 32


def accept_both(wl):
    import torch
    from synth.device import to_device
    d = to_device(wl)
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], max(1, wl.n_max), total_nodes=wl.total_nodes)
    meta = tta.tree_build(bt, d["parents"])
    ref = tta.tree_greedy_accept(bt, d["logits"], d["tokens"], meta["retrieve_next_token"],
                                 meta["retrieve_next_sibling"], MAX_ACCEPT, meta["err"])
    T, B = wl.total_nodes, wl.batch
    i32 = dict(dtype=torch.int32, device=d["logits"].device)
    # outputs prefilled with a pattern the call must overwrite
    out = {"accept_len": torch.full((B,), -7, **i32),
           "accepted_nodes": torch.full((B, MAX_ACCEPT), -7, **i32),
           "out_tokens": torch.full((B, MAX_ACCEPT + 1), -7, **i32),
           "row_argmax": torch.full((T + B,), -7, **i32)}
    err2 = meta["err"].clone()
    tta.tree_greedy_accept_noalloc(bt, d["logits"], d["tokens"], meta["retrieve_next_token"],
                                   meta["retrieve_next_sibling"], MAX_ACCEPT, err2, out=out)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in ref.items()}, {k: host(v) for k, v in out.items()}, host(meta["err"]), host(err2)


def test_noalloc_matches_workspace_call_twice():
    require_gpu()
    import numpy as np
    cases = [
        # larger first: 32 paged-style requests, vocab 128256 bf16 (several chunks per row)
        (2, dict(ctx=(4, 9), vocab=128256)),
        # then smaller: one 64-node EAGLE tree, vocab 5000 (one chunk per row)
        (1, dict(ctx=(4, 4), vocab=5000)),
    ]
    sizes = []
    for cfg, over in cases:
        wl = synth.make_workload(cfg, 4, **over)
        sizes.append((wl.total_nodes + wl.batch) * wl.vocab)
        say(f"tree_greedy_accept_noalloc cfg={cfg} rows={wl.total_nodes + wl.batch} V={wl.vocab}")
        ref, got, err_ref, err_got = accept_both(wl)
        assert (err_ref == 0).all() and (err_got == 0).all(), (err_ref, err_got)
        for k in ("accept_len", "accepted_nodes", "out_tokens", "row_argmax"):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
        check_accept(wl, got, MAX_ACCEPT)
    assert sizes[1] < sizes[0]
