"""The sampled verification walks on the GPU against the oracle, bit-exact.

tree_sample_accept: every row's Gumbel-max choice (float32, one rounding
per operation, as the oracle forms it) and the walk over those choices.
tree_stochastic_accept: accepted paths and the correction / bonus token of
the min(1, p/q) walk (float64 on both sides; the sums over the vocab are
added in different orders, so only a decision within a few float64 ulps of
its threshold could differ, which these seeded inputs do not reach).
"""

import numpy as np
import pytest

import synth
import token_tree_attention_amd as tta
from gpu_helpers import host, require_gpu, say
from oracle import accept as O_acc
from oracle import bf16 as O_bf16
from oracle import sampling as O_smp

pytestmark = pytest.mark.gpu

MAX_ACCEPT = 32


def logits_f32(wl):
    if wl.logits_dtype == "bf16":
        return O_bf16.to_f64(wl.logits).astype(np.float32)  # exact
    return wl.logits.astype(np.float32)


def rows_of(arr, wl):
    off = wl.node_offsets
    return lambda b: arr[int(off[b]) + b: int(off[b + 1]) + b + 1]


def children_tokens(wl):
    """Tokens of each logits row's children (row 0 of a request: its depth-0 nodes)."""
    kids = {}
    for b in range(wl.batch):
        s, e = int(wl.node_offsets[b]), int(wl.node_offsets[b + 1])
        for i in range(s, e):
            p = int(wl.parents[i])
            kids.setdefault(s + b + (0 if p < 0 else 1 + p), []).append(int(wl.tokens[i]))
    return kids


def device_round(wl):
    import torch
    from synth.device import to_device
    d = to_device(wl)
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], max(1, wl.n_max), total_nodes=wl.total_nodes)
    meta = tta.tree_build(bt, d["parents"])
    return torch, d, bt, meta


SAMPLE_CASES = [
    (0, dict(), 1.0),
    (1, dict(vocab=5000, ctx=(4, 4)), 0.7),
    (2, dict(vocab=3001, ctx=(4, 9), batch=12), 1.3),         # odd vocab: the scalar path
    (2, dict(vocab=4096, ctx=(4, 9), batch=12, logits="fp32"), 0.25),
    (3, dict(vocab=4096, ctx=(4, 4), ddtree_budget=300), 0.9),  # > 256 nodes: the parallel walk
    (4, dict(vocab=2000, ctx=(4, 9), batch=6), 2.0),
    (1, dict(ctx=(4, 4)), 0.8),                               # full 128256 vocab, bf16
]


@pytest.mark.parametrize("case", range(len(SAMPLE_CASES)))
@pytest.mark.parametrize("seed", [0, 1])
def test_sample_accept_matches_oracle(case, seed):
    require_gpu()
    cfg, over, T = SAMPLE_CASES[case]
    wl = synth.make_workload(cfg, seed, **over)
    R, V = wl.total_nodes + wl.batch, wl.vocab
    g = synth.gumbel_noise(seed, cfg, R, V)
    say(f"tree_sample_accept cfg={cfg} seed={seed} T={T} rows={R} V={V} {wl.logits_dtype}")
    torch, d, bt, meta = device_round(wl)
    out = tta.tree_sample_accept(bt, d["logits"], torch.from_numpy(g).to(d["logits"].device), T, d["tokens"],
                                 meta["retrieve_next_token"], meta["retrieve_next_sibling"], MAX_ACCEPT,
                                 meta["err"])
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in out.items()}
    assert (host(meta["err"]) == 0).all()
    ref = O_smp.sample_accept(rows_of(logits_f32(wl), wl), rows_of(g, wl), T, wl.node_offsets, wl.tokens,
                              wl.parents, MAX_ACCEPT)
    np.testing.assert_array_equal(got["row_argmax"], ref["row_argmax"], err_msg="row choices")
    for k in ("accept_len", "accepted_nodes", "out_tokens"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)


def test_sample_accept_zero_noise_is_the_greedy_call():
    require_gpu()
    wl = synth.make_workload(2, 7, vocab=128256, ctx=(4, 9), batch=8)
    torch, d, bt, meta = device_round(wl)
    zero = torch.zeros((wl.total_nodes + wl.batch, wl.vocab), dtype=torch.float32, device=d["logits"].device)
    s = tta.tree_sample_accept(bt, d["logits"], zero, 1.0, d["tokens"], meta["retrieve_next_token"],
                               meta["retrieve_next_sibling"], MAX_ACCEPT, meta["err"])
    gr = tta.tree_greedy_accept(bt, d["logits"], d["tokens"], meta["retrieve_next_token"],
                                meta["retrieve_next_sibling"], MAX_ACCEPT, meta["err"])
    torch.cuda.synchronize()
    for k in ("row_argmax", "accept_len", "accepted_nodes", "out_tokens"):
        assert torch.equal(s[k], gr[k]), k


def test_sample_accept_rejects_bad_temperature():
    require_gpu()
    wl = synth.make_workload(0, 0)
    torch, d, bt, meta = device_round(wl)
    g = torch.zeros((wl.total_nodes + wl.batch, wl.vocab), dtype=torch.float32, device=d["logits"].device)
    for T in (0.0, -1.0, float("inf"), 1e-45):
        with pytest.raises(RuntimeError, match="invalid"):
            tta.tree_sample_accept(bt, d["logits"], g, T, d["tokens"], meta["retrieve_next_token"],
                                   meta["retrieve_next_sibling"], MAX_ACCEPT, meta["err"])


STOCH_CASES = [
    # (cfg, overrides, temperature, draft boost on the drafted tokens)
    (0, dict(), 1.0, 0.0),
    (1, dict(vocab=5000, ctx=(4, 4)), 1.0, 20.0),
    (2, dict(vocab=3001, ctx=(4, 9), batch=12), 0.8, 0.0),
    (2, dict(vocab=3000, ctx=(4, 9), batch=12, logits="fp32"), 1.2, 20.0),
    (4, dict(vocab=2000, ctx=(4, 9), batch=6), 1.0, 5.0),
    (4, dict(vocab=2000, ctx=(4, 9), batch=6), 0.7, 200.0),   # mostly rejections: residual passes
    (3, dict(vocab=4096, ctx=(4, 4), ddtree_budget=300), 1.0, 20.0),
    (1, dict(ctx=(4, 4)), 0.9, 20.0),                          # full 128256 vocab: 16 workgroups walk it
    # vocab 32000: 15 workgroups per request, many residual passes each
    (2, dict(vocab=32000, ctx=(4, 9), batch=12), 0.7, 200.0),
    (2, dict(vocab=32000, ctx=(4, 9), batch=20), 1.0, 20.0),   # 20 requests: the grid padded to 24
]


@pytest.mark.parametrize("case", range(len(STOCH_CASES)))
@pytest.mark.parametrize("seed", [0, 1])
def test_stochastic_accept_matches_oracle(case, seed):
    require_gpu()
    cfg, over, T, boost = STOCH_CASES[case]
    wl = synth.make_workload(cfg, seed, **over)
    R, V = wl.total_nodes + wl.batch, wl.vocab
    kids = children_tokens(wl)
    q = synth.draft_distributions(seed, cfg, R, V, lambda r: kids.get(r, []), boost)
    u = synth.uniforms(seed, cfg, wl.total_nodes)
    g = synth.gumbel_noise(seed, cfg, R, V)
    say(f"tree_stochastic_accept cfg={cfg} seed={seed} T={T} boost={boost} rows={R} V={V} {wl.logits_dtype}")
    torch, d, bt, meta = device_round(wl)
    dev = d["logits"].device
    out = tta.tree_stochastic_accept(bt, d["logits"], T, torch.from_numpy(q).to(dev), torch.from_numpy(u).to(dev),
                                     torch.from_numpy(g).to(dev), d["tokens"], meta["retrieve_next_token"],
                                     meta["retrieve_next_sibling"], MAX_ACCEPT, meta["err"])
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in out.items()}
    assert (host(meta["err"]) == 0).all()
    ref = O_smp.stochastic_accept(rows_of(logits_f32(wl), wl), rows_of(q, wl), u, rows_of(g, wl), T,
                                  wl.node_offsets, wl.tokens, wl.parents, MAX_ACCEPT)
    for k in ("accept_len", "accepted_nodes", "out_tokens"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
    say(f"  accept lengths {got['accept_len'].tolist()[:12]}")


def test_stochastic_accept_masked_vocab_tail():
    """Logits of -inf over the last 12000 of 32000 tokens (a masked range):
    with 15 workgroups per request, the last ones' slices hold no finite
    logit and contribute nothing to a row's softmax; drafted tokens in the
    range are rejected (p = 0 there) and the walk still matches the oracle."""
    require_gpu()
    cfg, seed, T, boost = 2, 5, 1.0, 20.0
    wl = synth.make_workload(cfg, seed, vocab=32000, ctx=(4, 9), batch=12)
    assert wl.logits_dtype == "bf16"
    wl.logits[:, 20000:] = 0xFF80  # bf16 -inf
    R, V = wl.total_nodes + wl.batch, wl.vocab
    kids = children_tokens(wl)
    q = synth.draft_distributions(seed, cfg, R, V, lambda r: kids.get(r, []), boost)
    u = synth.uniforms(seed, cfg, wl.total_nodes)
    g = synth.gumbel_noise(seed, cfg, R, V)
    say(f"tree_stochastic_accept masked tail cfg={cfg} seed={seed} rows={R} V={V}")
    torch, d, bt, meta = device_round(wl)
    dev = d["logits"].device
    out = tta.tree_stochastic_accept(bt, d["logits"], T, torch.from_numpy(q).to(dev), torch.from_numpy(u).to(dev),
                                     torch.from_numpy(g).to(dev), d["tokens"], meta["retrieve_next_token"],
                                     meta["retrieve_next_sibling"], MAX_ACCEPT, meta["err"])
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in out.items()}
    assert (host(meta["err"]) == 0).all()
    ref = O_smp.stochastic_accept(rows_of(logits_f32(wl), wl), rows_of(q, wl), u, rows_of(g, wl), T,
                                  wl.node_offsets, wl.tokens, wl.parents, MAX_ACCEPT)
    for k in ("accept_len", "accepted_nodes", "out_tokens"):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
    assert (got["out_tokens"][np.arange(wl.batch), got["accept_len"]] < 20000).all()  # sampled from the support


def test_stochastic_accept_reused_workspace():
    """Two different walks in a row on one workspace (15 workgroups per
    request, vocab 32000): the second must not take any of the first's
    exchanged words for its own, so both match the oracle."""
    require_gpu()
    ws = None
    for seed, T, boost in ((7, 1.0, 20.0), (8, 0.8, 0.0), (7, 1.0, 200.0)):
        cfg = 2
        wl = synth.make_workload(cfg, seed, vocab=32000, ctx=(4, 9), batch=12)
        R, V = wl.total_nodes + wl.batch, wl.vocab
        kids = children_tokens(wl)
        q = synth.draft_distributions(seed, cfg, R, V, lambda r: kids.get(r, []), boost)
        u = synth.uniforms(seed, cfg, wl.total_nodes)
        g = synth.gumbel_noise(seed, cfg, R, V)
        say(f"tree_stochastic_accept reused workspace seed={seed} T={T} boost={boost}")
        torch, d, bt, meta = device_round(wl)
        dev = d["logits"].device
        if ws is None:
            ws = torch.empty(tta.tree_stochastic_accept_workspace_bytes(bt, V), dtype=torch.uint8, device=dev)
        assert ws.numel() >= tta.tree_stochastic_accept_workspace_bytes(bt, V)
        out = tta.tree_stochastic_accept(bt, d["logits"], T, torch.from_numpy(q).to(dev),
                                         torch.from_numpy(u).to(dev), torch.from_numpy(g).to(dev), d["tokens"],
                                         meta["retrieve_next_token"], meta["retrieve_next_sibling"], MAX_ACCEPT,
                                         meta["err"], workspace=ws)
        torch.cuda.synchronize()
        got = {k: host(v) for k, v in out.items()}
        assert (host(meta["err"]) == 0).all()
        ref = O_smp.stochastic_accept(rows_of(logits_f32(wl), wl), rows_of(q, wl), u, rows_of(g, wl), T,
                                      wl.node_offsets, wl.tokens, wl.parents, MAX_ACCEPT)
        for k in ("accept_len", "accepted_nodes", "out_tokens"):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)


def test_stochastic_accept_overflow_flag():
    """q = p at every row accepts first children down to a leaf; with max_accept
    below the depth the request is flagged and stops at max_accept."""
    require_gpu()
    wl = synth.make_workload(4, 3, vocab=500, ctx=(4, 9), batch=2)  # 4-level Medusa trees
    R, V = wl.total_nodes + wl.batch, wl.vocab
    f32 = logits_f32(wl)
    q = np.stack([O_smp.softmax_f64(r, 1.0) for r in f32]).astype(np.float32)
    u = (synth.uniforms(3, 4, wl.total_nodes) * np.float32(0.999)).astype(np.float32)
    g = synth.gumbel_noise(3, 4, R, V)
    torch, d, bt, meta = device_round(wl)
    dev = d["logits"].device
    out = tta.tree_stochastic_accept(bt, d["logits"], 1.0, torch.from_numpy(q).to(dev), torch.from_numpy(u).to(dev),
                                     torch.from_numpy(g).to(dev), d["tokens"], meta["retrieve_next_token"],
                                     meta["retrieve_next_sibling"], 2, meta["err"])
    torch.cuda.synchronize()
    err = host(meta["err"])
    assert (err & tta.ERR_ACCEPT).all(), err
    assert (host(out["accept_len"]) == 2).all()
