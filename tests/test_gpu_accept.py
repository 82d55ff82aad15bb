"""tree_greedy_accept on the GPU against the oracle: bit-exact."""

import numpy as np
import pytest

import synth
import token_tree_attention_amd as tta
from gpu_helpers import host, require_gpu, say
from parity import check_accept


pytestmark = pytest.mark.gpu


def run_accept(wl, max_accept=16, logits_override=None):
    import torch
    from synth.device import to_device
    d = to_device(wl)
    if logits_override is not None:
        d["logits"] = logits_override
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], max(1, wl.n_max), total_nodes=wl.total_nodes)
    meta = tta.tree_build(bt, d["parents"])
    acc = tta.tree_greedy_accept(bt, d["logits"], d["tokens"], meta["retrieve_next_token"],
                                 meta["retrieve_next_sibling"], max_accept, meta["err"])
    torch.cuda.synchronize()
    return {k: host(v) for k, v in acc.items()}, host(meta["err"])


SMALL = {
    0: dict(),
    1: dict(vocab=5000, ctx=(4, 4)),
    2: dict(vocab=3001, ctx=(4, 9), batch=12),
    3: dict(vocab=4096, ctx=(4, 4), ddtree_budget=200),
    4: dict(vocab=2000, ctx=(4, 9), batch=6),
    5: dict(vocab=4096, ctx=(4, 4), ddtree_budget=300),
}


@pytest.mark.parametrize("cfg", sorted(SMALL))
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_accept_scaled(cfg, seed):
    require_gpu()
    wl = synth.make_workload(cfg, seed, **SMALL[cfg])
    say(f"tree_greedy_accept cfg={cfg} seed={seed} T={wl.total_nodes} V={wl.vocab} {wl.logits_dtype}")
    acc, err = run_accept(wl)
    assert (err == 0).all()
    check_accept(wl, acc, 16)


def test_accept_ties_signed_zero_and_unaligned_vocab():
    require_gpu()
    import torch
    for dtype, V in (("bf16", 1001), ("fp32", 999), ("bf16", 8192 * 3 + 5)):
        wl = synth.make_workload(2, 3, vocab=V, ctx=(4, 9), batch=5, logits=dtype)
        rows = wl.logits.copy()
        # plant exact ties at two or three indices and a -0/+0 row
        rng = np.random.default_rng(V)
        for r in range(rows.shape[0]):
            a, b, c = sorted(rng.choice(V, 3, replace=False))
            if dtype == "bf16":
                top = rows[r].view(np.uint16)
                val = synth.f32_from_bf16_bits(top).max()
                hi = synth.bf16_bits_from_f32(np.array([val + 2.0], np.float32))[0]
                top[[b, c]] = hi
                if r % 3 == 0:
                    top[:] = 0x8000
                    top[a] = 0
            else:
                val = rows[r].max()
                rows[r, [b, c]] = val + 2.0
                if r % 3 == 0:
                    rows[r, :] = -0.0
                    rows[r, a] = 0.0
        wl.logits = rows
        say(f"tree_greedy_accept ties dtype={dtype} V={V}")
        acc, _ = run_accept(wl)
        check_accept(wl, acc, 16)


def test_accept_maxima_at_chunk_boundaries_full_vocab():
    """Full 128256-entry bf16 rows with the maximum planted next to multiples of 2048
    (every chunk the argmax splits a row into is a multiple of 2048 elements), in the
    last, shorter chunk, and as exact ties across two such positions."""
    require_gpu()
    V = 128256
    for batch in (1, 8):
        wl = synth.make_workload(2, 11 + batch, vocab=V, ctx=(4, 9), batch=batch, logits="bf16")
        rows = wl.logits.copy()
        rng = np.random.default_rng(batch)
        edges = [2048 * k + d for k in range(1, V // 2048 + 1) for d in (-1, 0) if 2048 * k + d < V]
        tail = list(range(V - 2048 // 2, V))
        for r in range(rows.shape[0]):
            bits = rows[r].view(np.uint16)
            hi = synth.bf16_bits_from_f32(
                np.array([synth.f32_from_bf16_bits(bits).max() + 2.0], np.float32))[0]
            kind = r % 4
            if kind == 0:
                bits[int(rng.choice(edges))] = hi
            elif kind == 1:
                bits[int(rng.choice(tail))] = hi
            elif kind == 2:
                a, b = sorted(int(x) for x in rng.choice(edges, 2, replace=False))
                bits[[a, b]] = hi
            else:
                bits[[int(rng.choice(edges[:8])), V - 1]] = hi
        wl.logits = rows
        say(f"tree_greedy_accept chunk-boundary maxima V={V} batch={batch} rows={rows.shape[0]}")
        acc, _ = run_accept(wl)
        check_accept(wl, acc, 16)


def test_accept_chain_and_star_trees_past_the_serial_walk():
    """Trees above 256 nodes take the parallel walk: a 1000-node chain accepted end to
    end (and cut at max_accept, which flags the overflow), and a root with 999
    children, every draft planted as the target's argmax."""
    require_gpu()
    chain = list(range(-1, 999))
    star = [-1] + [0] * 999
    for name, parents, max_accept in (("chain", chain, 1024), ("chain", chain, 100),
                                      ("star", star, 16)):
        wl = synth.make_workload(2, 21, vocab=2048, ctx=(4, 9), batch=2, p=(1.0, 1.0),
                                 tree=("parents", parents))
        say(f"tree_greedy_accept {name} tree of {len(parents)} nodes, max_accept={max_accept}")
        acc, err = run_accept(wl, max_accept=max_accept)
        check_accept(wl, acc, max_accept)
        if name == "chain":
            assert (acc["accept_len"] == min(max_accept, len(parents))).all(), acc["accept_len"]
            overflow = max_accept < len(parents)
            assert all(bool(e & tta.ERR_ACCEPT) == overflow for e in err), err
        else:
            assert (acc["accept_len"] == 2).all(), acc["accept_len"]  # the root and its matching child


def test_accept_overflow_flag():
    require_gpu()
    wl = synth.make_workload(2, 4, vocab=64, ctx=(4, 9), batch=3, p=(1.0, 1.0),
                             tree=("parents", list(range(-1, 11))))
    say("tree_greedy_accept max_accept overflow")
    acc, err = run_accept(wl, max_accept=3)
    assert (acc["accept_len"] <= 3).all()
    for b in range(wl.batch):
        if acc["accept_len"][b] == 3:
            assert err[b] & tta.ERR_ACCEPT


@pytest.mark.parametrize("n, seed", [(200, 0), (200, 1), (700, 0), (1000, 2)])
def test_accept_duplicate_sibling_tokens(n, seed):
    """Sibling tokens drawn from 3 ids, so most nodes share their token with a
    sibling: the walk must take the lowest-index matching child.  Trees of at
    most 256 nodes take the one-lane walk, larger ones the parallel walk."""
    require_gpu()
    wl = synth.make_workload(2, seed, batch=4, tree=("random", (n, n)), vocab=64, ctx=(4, 9),
                             p=(0.95, 0.95), dup_alphabet=3)
    seen = set()
    dups = 0
    for b in range(wl.batch):
        sl = wl.request_nodes(b)
        for p, t in zip(wl.parents[sl], wl.tokens[sl]):
            dups += (b, int(p), int(t)) in seen
            seen.add((b, int(p), int(t)))
    assert dups > 0
    say(f"tree_greedy_accept duplicate sibling tokens n={n} seed={seed}")
    acc, err = run_accept(wl, max_accept=64)
    assert (err == 0).all(), err
    ref = check_accept(wl, acc, 64)
    assert ref["accept_len"].max() >= 2  # the walks do go down the tree
