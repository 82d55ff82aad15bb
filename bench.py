#!/usr/bin/env python3
"""Benchmark of one token-tree verification round on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
tree_build -> tree_attention_verify (one layer) -> tree_greedy_accept ->
tree_kv_commit (plus, for paged caches, restoring the block table that the
previous round's commit released, i.e. re-mapping the tentative blocks).

Headline workload (the JSON line's ``value``): ``medusa_long``, the largest
of the five verification workloads: 64 requests, each a Medusa cartesian tree
with top-s (10, 3, 2, 2) = 220 nodes over a committed context drawn from
U{1024..32768}, 40 query / 8 KV heads, head_dim 128, bf16, paged cache with
block size 16 and shuffled block tables, vocab 32000 bf16 logits.
``--workload`` picks another headline.  ``per_config`` in the same line holds
every workload's step time (median and p10/p90 over replays), per-call
times, the attention call's roofline fractions and the acceptance stats.

Inputs sit in HBM before timing and are rotated over enough copies (> 512 MB
in play) that each step reads cold HBM rather than the 256 MB Infinity
Cache.  W eager warm-up steps; then exactly K steps are captured in one HIP
graph (the way a serving loop replays a verify step per tree-size bucket);
after two untimed replays (the GPU clock drops while idle and takes tens of
milliseconds to recover) one replay is timed between two synchronisations
with HIP events on the stream the kernels run on: that is ``ms_per_step``.
Further replays give the p10/p50/p90.  Each call's own time comes from a
graph of K back-to-back calls of it, timed the same way (commit: K
table-restore + commit pairs minus K restores).

Prints ONE JSON line: throughput in verified tree tokens/s (tree nodes per
second) and us per step, the attention roofline of the headline (algorithmic
bytes per call / call time against 8 TB/s HBM, or flops per call / call
time against the 2.5 PFLOP/s dense bf16 MFMA peak when the call's
arithmetic intensity is above the ridge of the two), the achievable
streaming bandwidth measured on the same GPU, and the CPU oracle's rate on a
bounded sample of the headline workload, stage by stage.
"""

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified tree tokens/sec + µs/verify step at 1 GPU; % of HBM roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    "tiny_medusa": 0, "eagle": 1, "batched": 2, "ddtree": 3, "medusa_long": 4, "ddtree_deep": 5,
}
# the five verification workloads reported in per_config (ddtree_deep, a
# deeper-tree stress variant of ddtree, with --deep)
PER_CONFIG = ("tiny_medusa", "eagle", "batched", "ddtree", "medusa_long")


def describe(wl):
    import numpy as np
    n = np.diff(wl.node_offsets)
    return {
        "workload": wl.name,
        "batch": int(wl.batch),
        "tree_nodes_total": int(wl.total_nodes),
        "tree_nodes_per_request": [int(n.min()), int(n.max())],
        "ctx_tokens": [int(wl.ctx_lens.min()), int(wl.ctx_lens.max())],
        "heads_q_kv_dim": [wl.n_heads, wl.n_kv_heads, wl.head_dim],
        "vocab": wl.vocab,
        "logits_dtype": wl.logits_dtype,
        "kv_layout": wl.layout,
        "rope_base": wl.rope_base,
        "seed": wl.seed,
    }


def algorithmic(wl):
    """Algorithmic bytes and flops of one attention call and one accept call."""
    import numpy as np
    D, Hq, Hkv = wl.head_dim, wl.n_heads, wl.n_kv_heads
    W = max(1, (wl.n_max + 31) // 32)
    attn_bytes = 0
    flops = 0
    for b in range(wl.batch):
        s, e = int(wl.node_offsets[b]), int(wl.node_offsets[b + 1])
        n, ctx = e - s, int(wl.ctx_lens[b])
        attn_bytes += ctx * Hkv * D * 4          # context K + V (bf16)
        attn_bytes += n * Hq * D * 4             # Q in + O out
        attn_bytes += n * Hkv * D * 8            # k/v_new in + tentative K/V out
        attn_bytes += n * W * 4 + n * 4          # mask rows + positions
        par = wl.parents[s:e]
        depth = np.zeros(n, np.int64)
        for i in range(n):
            depth[i] = 0 if par[i] < 0 else depth[par[i]] + 1
        flops += int(4 * D * Hq * np.sum(ctx + depth + 1))
    esz = 4 if wl.logits_dtype == "fp32" else 2
    accept_bytes = (wl.total_nodes + wl.batch) * wl.vocab * esz
    return attn_bytes, flops, accept_bytes


def blas_info():
    """(library name, threads) of the BLAS numpy uses."""
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            i = infos[0]
            return f"{i.get('internal_api')} {i.get('version')}", int(i.get("num_threads", 1))
    except Exception:  # pragma: no cover
        pass
    return "unknown", 1


def cpu_baseline(wl, budget_s):
    """Time the oracle stage by stage on a bounded sample of the workload:
    whole requests in order (build, per-node path attention, argmax + walk,
    copy commit of the request's own cache region) until the budget is
    spent."""
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import accept as O_acc
    from oracle import attention as O_att
    from oracle import bf16 as O_bf16
    from oracle import commit as O_com
    from oracle import tree as O_tree

    blas, blas_threads = blas_info()
    cores = min(len(os.sched_getaffinity(0)), max(1, blas_threads))
    stage = {"build": 0.0, "attention": 0.0, "accept": 0.0, "commit": 0.0}
    nodes_done = 0
    reqs_done = 0
    passes = 0
    t_start = time.perf_counter()

    def spent():
        return time.perf_counter() - t_start > budget_s

    while True:
        for b in range(wl.batch):
            s, e = int(wl.node_offsets[b]), int(wl.node_offsets[b + 1])
            n, ctx = e - s, int(wl.ctx_lens[b])
            sl = slice(s, e)
            t0 = time.perf_counter()
            O_tree.build(wl.parents[sl], np.array([0, n]), np.array([ctx]), max(1, n), max(1, (n + 31) // 32))
            stage["build"] += time.perf_counter() - t0
            kc, vc = O_att.context_of(wl.k_cache, wl.v_cache, b, ctx, wl.layout, wl.block_table)
            done = 0
            t0 = time.perf_counter()
            for i in range(n):
                O_att.attention_request(wl.q[sl], wl.k_new[sl], wl.v_new[sl], kc, vc, wl.parents[sl], ctx,
                                        nodes=[i])
                done += 1
                if spent():
                    break
            stage["attention"] += time.perf_counter() - t0
            t0 = time.perf_counter()
            rows = wl.logits[s + b: e + b + 1]
            rows = O_bf16.to_f64(rows) if wl.logits_dtype == "bf16" else rows.astype(np.float64)
            choice = O_acc.row_argmax(rows)
            walk = O_acc.greedy_walk(choice, wl.tokens[sl], wl.parents[sl], 64)
            stage["accept"] += time.perf_counter() - t0
            # the commit copies this request's own cache region (its blocks, for a paged cache)
            a = len(walk["accepted"])
            acc_nodes = np.full((1, max(1, a)), -1, np.int32)
            acc_nodes[0, :a] = walk["accepted"]
            if wl.layout == "contiguous":
                kr, vr = wl.k_cache[b:b + 1], wl.v_cache[b:b + 1]
                t0 = time.perf_counter()
                O_com.commit_contiguous(kr, vr, [ctx], [a], acc_nodes)
            else:
                nblk = -(-(ctx + n) // 16)
                ids = wl.block_table[b, :nblk]
                kr, vr = wl.k_cache[ids], wl.v_cache[ids]
                table = np.arange(nblk, dtype=np.int32)[None, :]
                t0 = time.perf_counter()
                O_com.commit_paged(kr, vr, table, [ctx], [n], [a], acc_nodes)
            stage["commit"] += time.perf_counter() - t0
            nodes_done += done
            reqs_done += 1
            if spent():
                break
        passes += 1
        if spent():
            break
    dt = sum(stage.values())
    return {"value": nodes_done / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "blas": blas,
            "stage_s": {k: round(v, 4) for k, v in stage.items()},
            "sample": f"{wl.name}: {nodes_done} tree nodes of {reqs_done} request round(s) ({passes} pass(es) over "
                      f"the workload's requests): float64 oracle build, per-node path attention, argmax + walk "
                      f"and copy commit of those requests ({dt:.1f} s; {blas}, {blas_threads} threads)"}


def copy_reference(args, dev):
    """K plain copies of a fixed buffer: the known-size kernel that FETCH_SIZE and
    WRITE_SIZE are scaled by."""
    import torch
    nbytes = int(args.copy_reference * 1e6) // 4096 * 4096
    src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).random_()
    dst = torch.empty_like(src)
    for _ in range(max(1, args.warmup)):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"copy_reference_bytes": nbytes, "steps": args.steps,
                      "us_per_copy": dt * 1e6, "GBps_read_plus_write": 2 * nbytes / dt / 1e9}))


def achievable_bandwidth(dev):
    """Streaming rates of plain library kernels on this GPU (GB/s): a sum over
    1 GiB (reads only) and a 1 GiB device copy (read + write)."""
    import torch
    n = (1 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)

    def best_of(fn, reps=10):
        ts = []
        for _ in range(reps + 2):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts = sorted(ts[2:])
        return ts[len(ts) // 2]
    read_ms = best_of(lambda: x.sum())
    copy_ms = best_of(lambda: y.copy_(x))
    del x, y
    torch.cuda.empty_cache()
    # this library's own streaming read: the argmax of tree_greedy_accept over
    # 1 GiB of bf16 logits (2048 one-node requests, 4096 rows of 131072)
    import token_tree_attention_amd as tta
    B, V = 2048, 131072
    i32 = dict(dtype=torch.int32, device=dev)
    bt = tta.Batch(torch.arange(B + 1, **i32), torch.zeros(B, **i32), 1, total_nodes=B)
    meta = tta.tree_build(bt, torch.full((B,), -1, **i32))
    logits = torch.randn((2 * B, V), device=dev).to(torch.bfloat16)
    tokens = torch.zeros(B, **i32)
    out = {"accept_len": torch.empty(B, **i32), "accepted_nodes": torch.empty((B, 1), **i32),
           "out_tokens": torch.empty((B, 2), **i32)}
    ws = torch.empty(max(256, tta.tree_greedy_accept_workspace_bytes(bt, V)), dtype=torch.uint8, device=dev)
    us = graph_call_us(lambda: tta.tree_greedy_accept(bt, logits, tokens, meta["retrieve_next_token"],
                                                      meta["retrieve_next_sibling"], 1, meta["err"], out=out,
                                                      workspace=ws, want_row_argmax=False), 10, reps=5)
    nbytes = logits.numel() * 2
    del logits, ws
    torch.cuda.empty_cache()
    return {"read_gbs": (1 << 30) / (read_ms * 1e-3) / 1e9,
            "copy_gbs": 2 * (1 << 30) / (copy_ms * 1e-3) / 1e9,
            "argmax_read_gbs": nbytes / (us * 1e-6) / 1e9,
            "kernels": "torch sum over 1 GiB fp32 (read), a 1 GiB device copy (read + write), median of 10; "
                       "tree_greedy_accept over 1 GiB of bf16 logits (its argmax streams them once), "
                       "10 calls in a HIP graph, median of 5"}


def stored_traffic(workload):
    """HBM bytes per attention call from the committed counter summary, or None
    when the summary is missing or the attention source changed since."""
    import hashlib
    src = os.path.join(ROOT, "token_tree_attention_amd", "csrc", "tree_attention.hip")
    path = os.path.join(ROOT, "profiles", f"tree_attention_{workload}_hbm_counters.md")
    try:
        text = open(path).read()
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = dict(re.findall(r"^- (\w+): (\S+)$", text, re.M))
    if fields.get("source_sha256") != digest:
        return None
    try:
        return int(fields["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def roofline_entry(wl, attn_bytes, flops, attn_ms):
    """Roofline of the tree_attention_verify call: HBM-bound when its arithmetic
    intensity (flops per algorithmic byte) is below the ridge of the bf16 MFMA
    peak over the HBM peak, MFMA-bound above it."""
    gbs = attn_bytes / (attn_ms * 1e-3) / 1e9
    tflops = flops / (attn_ms * 1e-3) / 1e12
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    mfma_bound = flops / attn_bytes > ridge
    entry = {
        "kernel": "tree_attention_verify call (all its launches), K calls back to back in one HIP graph, "
                  "HIP events on their stream",
        "bound": "mfma" if mfma_bound else "hbm",
        "achieved": tflops if mfma_bound else gbs,
        "peak": BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
        "unit": "TFLOP/s" if mfma_bound else "GB/s",
        "frac": tflops / BF16_PEAK_TFLOPS if mfma_bound else gbs / HBM_PEAK_GBS,
        "traffic": stored_traffic(wl.name),
        "algorithmic_bytes": attn_bytes,
        "flops": flops,
        "arithmetic_intensity": flops / attn_bytes,
        "attention_us": attn_ms * 1e3,
        "attention_gbs": gbs,
        "attention_tflops": tflops,
        "hbm_frac": gbs / HBM_PEAK_GBS,
        "mfma_frac": tflops / BF16_PEAK_TFLOPS,
    }
    return entry


def pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def measure(wl, args, dev):
    """Time one workload: the step, its dispersion and each call; returns a dict."""
    import numpy as np
    import torch

    import token_tree_attention_amd as tta
    from synth.device import to_device
    from token_tree_attention_amd.step import VerifyStep

    K, W = args.steps, args.warmup
    base = to_device(wl, dev)
    per_set = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    n_sets = int(max(1, min(64, np.ceil(args.rotate_mb * 1e6 / per_set))))
    free = torch.cuda.mem_get_info()[0]
    n_sets = int(max(1, min(n_sets, (free * 0.5) // max(1, per_set))))
    sets = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()} for _ in range(n_sets - 1)]
    steps = []
    pristine_tables = []
    for d in sets:
        bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=wl.total_nodes)
        cache = tta.KVCache(d["k_cache"], d["v_cache"], d["block_table"])
        steps.append((d, VerifyStep(bt, cache, wl.n_heads, wl.vocab, max_accept=64)))
        pristine_tables.append(None if d["block_table"] is None else d["block_table"].clone())
    stream = torch.cuda.current_stream()

    def restore(i):
        if pristine_tables[i % n_sets] is not None:
            steps[i % n_sets][0]["block_table"].copy_(pristine_tables[i % n_sets], non_blocking=True)

    def run(i):
        d, st = steps[i % n_sets]
        restore(i)
        st.build(d["parents"])
        st.attention(d["q"], d["k_new"], d["v_new"])
        st.accept(d["logits"], d["tokens"])
        st.commit()

    for i in range(W):
        run(i)
    torch.cuda.synchronize()
    errs = steps[0][1].meta["err"].cpu().numpy()
    if (errs != 0).any():
        print(f"{wl.name}: device error bits after warm-up: {errs.tolist()}", file=sys.stderr)
        sys.exit(1)
    ref_acc = {k: v.clone() for k, v in steps[0][1].acc.items()}
    num_released = steps[0][1].com.get("num_released")
    released = None if num_released is None else int(num_released.sum().item())

    def timed(fn):
        """fn() between two HIP events on the stream the kernels run on (ms)."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # Eager (host-launched) steps, for reference.
    eager_ms = timed(lambda: [run(W + k) for k in range(K)]) / K

    def check_replay():
        for key, ref in ref_acc.items():  # a replay reproduces the eager result
            if not torch.equal(steps[0][1].acc[key], ref):
                print(f"{wl.name}: graph replay differs from eager in {key}", file=sys.stderr)
                sys.exit(1)

    def restore_all():
        for i in range(n_sets):
            restore(i)
        torch.cuda.synchronize()

    def graph_of(body):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(K):
                body(k)
        return g

    def replay_ms(g, reps):
        """Two untimed replays (steady clocks), then `reps` timed ones (ms per replay)."""
        g.replay()
        g.replay()
        return [timed(g.replay) for _ in range(reps)]

    g_step = graph_of(run)
    g_step.replay()
    torch.cuda.synchronize()
    check_replay()
    # the timed region: exactly K steps, one replay; then the dispersion replays
    step_ms = replay_ms(g_step, 1 + args.replays)
    ms_step = step_ms[0] / K
    samples = [t / K for t in step_ms]
    check_replay()

    def call(name):
        def body(k):
            d, st = steps[k % n_sets]
            if name == "build":
                st.build(d["parents"])
            elif name == "attention":
                st.attention(d["q"], d["k_new"], d["v_new"])
            elif name == "accept":
                st.accept(d["logits"], d["tokens"])
            elif name == "restore":
                restore(k)
            elif name == "restore_commit":
                restore(k)
                st.commit()
            elif name == "commit":
                st.commit()
        return body

    calls_us = {}
    attn_samples = None
    # A paged commit releases the tentative blocks, so each timed commit runs
    # on restored tables (restore + commit, minus the restores); a contiguous
    # commit repeats the same moves.
    paged = wl.layout == "paged"
    for name in ("build", "attention", "accept") + (("restore", "restore_commit") if paged else ("commit",)):
        restore_all()
        g = graph_of(call(name))
        ts = replay_ms(g, 1 + (args.replays if name == "attention" else 2))
        calls_us[name] = float(np.median(ts)) / K * 1e3
        if name == "attention":
            attn_ms = ts[0] / K
            attn_samples = [t / K for t in ts]
        del g
    restore_all()
    check_replay()
    commit_us = max(0.0, calls_us["restore_commit"] - calls_us["restore"]) if paged else calls_us["commit"]

    attn_bytes, flops, accept_bytes = algorithmic(wl)
    roof = roofline_entry(wl, attn_bytes, flops, attn_ms)
    acc_len = steps[0][1].acc["accept_len"].cpu().numpy()
    res = {
        "workload": wl.name,
        "config": describe(wl),
        "ms_per_step": ms_step,
        "us_per_step": ms_step * 1e3,
        "us_per_step_p10_p50_p90": [pct(samples, 10) * 1e3, pct(samples, 50) * 1e3, pct(samples, 90) * 1e3],
        "replays": len(samples),
        "tokens_per_s": wl.total_nodes / (ms_step * 1e-3),
        "eager_us_per_step": eager_ms * 1e3,
        "calls_us": {"tree_build": calls_us["build"], "tree_attention_verify": calls_us["attention"],
                     "tree_greedy_accept": calls_us["accept"], "tree_kv_commit": commit_us,
                     "block_table_restore": calls_us["restore"] if paged else 0.0},
        "attention_us_p10_p50_p90": [pct(attn_samples, 10) * 1e3, pct(attn_samples, 50) * 1e3,
                                     pct(attn_samples, 90) * 1e3],
        "roofline": roof,
        "accept_gbs": accept_bytes / (calls_us["accept"] * 1e-6) / 1e9,
        "accept_bytes": accept_bytes,
        "accept_len_hist": np.bincount(acc_len).tolist(),
        "mean_accept_len": float(acc_len.mean()),
        "released_blocks": released,
        "input_sets_rotated": n_sets,
    }
    del steps, sets, base, g_step
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def graph_call_us(fn, K, reps=3):
    """fn() K times in one HIP graph: two untimed replays, then the median of
    `reps` timed ones (HIP events on the capture stream), in us per call."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(K):
            fn()
    g.replay()
    g.replay()
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del g
    return float(np.median(ts)) / K * 1e3


def measure_next(args, dev):
    """The calls beyond the four-step round, each timed like the round's calls
    (K back to back in a HIP graph) on seeded inputs of a workload's shape,
    with its algorithmic bytes against the 8 TB/s HBM peak where it streams
    memory, else its latency:
    - tree_sample_accept (Gumbel-max temperature sampling) and
      tree_stochastic_accept (min(1, p/q) walk) on the batched workload;
    - tree_ddtree_build on the DDTree workload's draft logits (4 requests, 16
      depths, vocab 151936, budget 1024);
    - tree_eagle_grow (32 requests of the EAGLE tree: 4 roots, 6 layers,
      budget 64) and tree_merge_sequences (32 requests of 64 drafts of 8
      tokens over 4 symbols);
    - tree_expand_mask / tree_pack_mask of the DDTree workload (T = 4096) in
      both dense forms."""
    import numpy as np
    import torch

    import synth
    import token_tree_attention_amd as tta
    from synth.device import to_device

    K = max(1, args.steps)
    res = {}

    def hbm(name, us, nbytes, **extra):
        res[name] = {"us": us, "algorithmic_bytes": int(nbytes), "gbs": nbytes / (us * 1e-6) / 1e9,
                     "hbm_frac": nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), **extra}

    # -- acceptance variants on the batched workload
    cfg = WORKLOADS["batched"]
    wl = synth.make_workload(cfg, args.seed)
    d = to_device(wl, dev)
    T, B, V = wl.total_nodes, wl.batch, wl.vocab
    R = T + B
    esz = 4 if wl.logits_dtype == "fp32" else 2
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=T)
    meta = tta.tree_build(bt, d["parents"])
    g = torch.from_numpy(synth.gumbel_noise(args.seed, cfg, R, V)).to(dev)
    kids = {}
    for b in range(B):
        s0, e0 = int(wl.node_offsets[b]), int(wl.node_offsets[b + 1])
        for i in range(s0, e0):
            p = int(wl.parents[i])
            kids.setdefault(s0 + b + (0 if p < 0 else 1 + p), []).append(int(wl.tokens[i]))
    q = torch.from_numpy(synth.draft_distributions(args.seed, cfg, R, V, lambda r: kids.get(r, []), 20.0)).to(dev)
    u = torch.from_numpy(synth.uniforms(args.seed, cfg, T)).to(dev)
    max_accept = 64
    out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
           "accepted_nodes": torch.empty((B, max_accept), dtype=torch.int32, device=dev),
           "out_tokens": torch.empty((B, max_accept + 1), dtype=torch.int32, device=dev),
           "row_argmax": torch.empty(R, dtype=torch.int32, device=dev)}
    ws = torch.empty(max(256, tta.tree_greedy_accept_workspace_bytes(bt, V)), dtype=torch.uint8, device=dev)
    sws = torch.empty(max(256, tta.tree_stochastic_accept_workspace_bytes(bt, V)), dtype=torch.uint8, device=dev)
    err = meta["err"]

    def sample():
        tta.tree_sample_accept(bt, d["logits"], g, 0.8, d["tokens"], meta["retrieve_next_token"],
                               meta["retrieve_next_sibling"], max_accept, err, out=out, workspace=ws)
    hbm("tree_sample_accept", graph_call_us(sample, K), R * V * (esz + 4), workload="batched", temperature=0.8)
    sout = {k: v for k, v in out.items() if k != "row_argmax"}

    def stochastic():
        tta.tree_stochastic_accept(bt, d["logits"], 1.0, q, u, g, d["tokens"], meta["retrieve_next_token"],
                                   meta["retrieve_next_sibling"], max_accept, err, out=sout, workspace=sws)
    us = graph_call_us(stochastic, K)
    a = sout["accept_len"].cpu().numpy()
    if (err.cpu().numpy() != 0).any():
        raise RuntimeError("device error bits in the acceptance variants")
    # visited rows: a_b + 1 per request (logits and draft row each), the final row's noise, the uniforms
    hbm("tree_stochastic_accept", us, int(((a + 1) * V * (esz + 4)).sum() + B * V * 4 + T * 4),
        workload="batched", temperature=1.0, draft_boost=20.0, mean_accept_len=float(a.mean()),
        bound_note="a group of workgroups per request walks its visited rows: latency of dependent full-vocab passes")
    del g, q, u, ws, sws, d

    # -- DDTree construction
    cfg = WORKLOADS["ddtree"]
    Rq, L, Vd, budget = 4, 16, 151936, 1024
    z = torch.from_numpy(synth.draft_logits(args.seed, cfg, Rq, L, Vd)).to(dev)
    dd_out = {"parents": torch.empty((Rq, budget), dtype=torch.int32, device=dev),
              "tokens": torch.empty((Rq, budget), dtype=torch.int32, device=dev),
              "n_nodes": torch.empty(Rq, dtype=torch.int32, device=dev)}
    dd_ws = torch.empty(tta.tree_ddtree_workspace_bytes(Rq, L, Vd, budget), dtype=torch.uint8, device=dev)
    hbm("tree_ddtree_build", graph_call_us(lambda: tta.tree_ddtree_build(z, budget, out=dd_out, workspace=dd_ws), K),
        Rq * L * Vd * 4 + Rq * budget * 8, requests=Rq, depths=L, vocab=Vd, budget=budget)
    del z, dd_ws

    # -- EAGLE growth and SpecInfer merge (latency)
    rng = np.random.default_rng([args.seed, 1, 99])
    Re, k, Le, be = 32, 4, 6, 64
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    rt = t(rng.integers(0, 128256, size=(Re, k)).astype(np.int32))
    rc = t(rng.uniform(0.01, 0.99, size=(Re, k)).astype(np.float32))
    ct = t(rng.integers(0, 128256, size=(Re, Le - 1, k, k)).astype(np.int32))
    cc = t(rng.uniform(0.01, 0.99, size=(Re, Le - 1, k, k)).astype(np.float32))
    eg = {"parents": torch.empty((Re, be), dtype=torch.int32, device=dev),
          "tokens": torch.empty((Re, be), dtype=torch.int32, device=dev),
          "n_nodes": torch.empty(Re, dtype=torch.int32, device=dev)}
    res["tree_eagle_grow"] = {"us": graph_call_us(lambda: tta.tree_eagle_grow(rt, rc, ct, cc, be, out=eg), K),
                              "requests": Re, "k": k, "layers": Le, "budget": be, "bound": "latency"}
    Rm, M, Lm = 32, 64, 8
    seqs = rng.integers(0, 4, size=(Rm, M, Lm)).astype(np.int32)
    ends = rng.integers(1, Lm + 1, size=(Rm, M))
    for r in range(Rm):
        for m in range(M):
            seqs[r, m, ends[r, m]:] = -1
    seqs = t(seqs)
    mg = {"parents": torch.empty((Rm, 1024), dtype=torch.int32, device=dev),
          "tokens": torch.empty((Rm, 1024), dtype=torch.int32, device=dev),
          "n_nodes": torch.empty(Rm, dtype=torch.int32, device=dev)}
    merr = torch.zeros(Rm, dtype=torch.int32, device=dev)
    res["tree_merge_sequences"] = {
        "us": graph_call_us(lambda: tta.tree_merge_sequences(seqs, 1024, err=merr, out=mg), K),
        "requests": Rm, "sequences": M, "seq_len": Lm, "alphabet": 4, "bound": "latency",
        "mean_nodes": float(mg["n_nodes"].float().mean().item())}

    # -- dense mask forms of the DDTree workload
    wl = synth.make_trees(WORKLOADS["ddtree"], args.seed)
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)
    bt = tta.Batch(i32(wl.node_offsets), i32(wl.ctx_lens), wl.n_max, total_nodes=wl.total_nodes)
    meta = tta.tree_build(bt, i32(wl.parents))
    T, W = wl.total_nodes, meta["mask"].shape[1]
    for mode, name in ((tta.MASK_QLEN_ONLY, "qlen_only"), (tta.MASK_FULL, "full")):
        stride = wl.n_max if mode == tta.MASK_QLEN_ONLY else int((wl.ctx_lens + np.diff(wl.node_offsets)).max())
        stride = -(-stride // 16) * 16
        dense = torch.empty((T, stride), dtype=torch.uint8, device=dev)
        packed = torch.empty((T, W), dtype=torch.int32, device=dev)
        hbm(f"tree_expand_mask_{name}",
            graph_call_us(lambda: tta.tree_expand_mask(bt, meta["mask"], mode, stride, meta["err"], out=dense), K),
            T * stride + T * W * 4, nodes=T, row_stride=stride)
        hbm(f"tree_pack_mask_{name}",
            graph_call_us(lambda: tta.tree_pack_mask(bt, dense, mode, meta["err"], mask_words=W, out=packed), K),
            T * stride + T * W * 4, nodes=T, row_stride=stride)
        if (meta["err"].cpu().numpy() != 0).any() or not torch.equal(packed, meta["mask"]):
            raise RuntimeError(f"dense mask round trip ({name}) failed")
        del dense, packed
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def summary(res):
    """The per_config entry: the figures a reader compares across workloads."""
    r = res["roofline"]
    return {
        "us_per_step": res["us_per_step"],
        "us_per_step_p10_p50_p90": res["us_per_step_p10_p50_p90"],
        "tokens_per_s": res["tokens_per_s"],
        "calls_us": res["calls_us"],
        "attention_us_p10_p50_p90": res["attention_us_p10_p50_p90"],
        "bound": r["bound"],
        "frac": r["frac"],
        "hbm_frac": r["hbm_frac"],
        "mfma_frac": r["mfma_frac"],
        "attention_gbs": r["attention_gbs"],
        "attention_tflops": r["attention_tflops"],
        "arithmetic_intensity": r["arithmetic_intensity"],
        "accept_gbs": res["accept_gbs"],
        "mean_accept_len": res["mean_accept_len"],
        "released_blocks": res["released_blocks"],
        "nodes": res["config"]["tree_nodes_total"],
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="medusa_long", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--seeds", default="0,1,2",
                    help="input seeds the headline workload is also measured with (reported per seed)")
    ap.add_argument("--replays", type=int, default=10, help="timed replays for the p10/p50/p90")
    ap.add_argument("--rotate-mb", type=float, default=600.0,
                    help="rotate input copies until this many MB are in play (defeats the MALL)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle CPU work")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", action="store_true", help="the headline workload only (no per_config)")
    ap.add_argument("--deep", action="store_true", help="also ddtree_deep in per_config")
    ap.add_argument("--no-next", action="store_true", help="skip the calls beyond the four-step round")
    ap.add_argument("--next-only", action="store_true",
                    help="time only the calls beyond the four-step round (one JSON object)")
    ap.add_argument("--eager-only", action="store_true",
                    help="host-launched steps of the headline only, no graphs (for counter collection)")
    ap.add_argument("--copy-reference", type=float, default=0.0, metavar="MB",
                    help="instead of the path, run K device-to-device copies of MB megabytes "
                         "(the reference kernel for scaling the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU (asked for --gpus {args.gpus}); the verification path "
              f"runs on a single GPU and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import token_tree_attention_amd as tta

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_reference > 0:
        copy_reference(args, dev)
        return
    tta.load_library()
    if args.eager_only:
        eager_only(args, dev)
        return
    if args.next_only:
        print(json.dumps({"next": measure_next(args, dev)}))
        return

    names = [args.workload] if args.only else list(PER_CONFIG) + (["ddtree_deep"] if args.deep else [])
    if args.workload not in names:
        names.append(args.workload)
    results = {}
    head_wl = None
    for name in names:
        t0 = time.perf_counter()
        wl = synth.make_workload(WORKLOADS[name], args.seed)
        t1 = time.perf_counter()
        results[name] = measure(wl, args, dev)
        print(f"[bench] {name}: inputs {t1 - t0:.1f} s, timing {time.perf_counter() - t1:.1f} s, "
              f"{results[name]['us_per_step']:.1f} us/step", file=sys.stderr, flush=True)
        if name == args.workload:
            head_wl = wl
        else:
            del wl
    head = results[args.workload]
    per_seed = []
    for sd in [int(x) for x in args.seeds.split(",") if x.strip()]:
        if sd == args.seed:
            r = head
        else:
            t0 = time.perf_counter()
            r = measure(synth.make_workload(WORKLOADS[args.workload], sd), args, dev)
            print(f"[bench] {args.workload} seed {sd}: {time.perf_counter() - t0:.1f} s, "
                  f"{r['us_per_step']:.1f} us/step", file=sys.stderr, flush=True)
        per_seed.append({"seed": sd, "us_per_step": r["us_per_step"], "tokens_per_s": r["tokens_per_s"],
                         "attention_us": r["roofline"]["attention_us"], "frac": r["roofline"]["frac"],
                         "nodes": r["config"]["tree_nodes_total"], "ctx_tokens": r["config"]["ctx_tokens"]})
    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "us_per_step": head["us_per_step"],
        "us_per_step_p10_p50_p90": head["us_per_step_p10_p50_p90"],
        "eager_us_per_step": head["eager_us_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "calls_us": head["calls_us"],
        "accept_len_hist": head["accept_len_hist"],
        "released_blocks": head["released_blocks"],
        "input_sets_rotated": head["input_sets_rotated"],
        "timing": "K steps in one HIP graph replay (after two untimed replays); p10/p50/p90 over "
                  f"{head['replays']} replays",
        "per_config": {name: summary(r) for name, r in results.items()},
        "seeds": per_seed,
        "achievable_bandwidth": achievable_bandwidth(dev),
    }
    if not args.no_next:
        t0 = time.perf_counter()
        result["next"] = measure_next(args, dev)
        print(f"[bench] calls beyond the round: {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(head_wl, args.cpu_budget)
    print(json.dumps(result))


def eager_only(args, dev):
    """Host-launched steps of one workload (the counter runs need no graphs)."""
    import torch

    import synth
    import token_tree_attention_amd as tta
    from synth.device import to_device
    from token_tree_attention_amd.step import VerifyStep

    wl = synth.make_workload(WORKLOADS[args.workload], args.seed)
    d = to_device(wl, dev)
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=wl.total_nodes)
    cache = tta.KVCache(d["k_cache"], d["v_cache"], d["block_table"])
    st = VerifyStep(bt, cache, wl.n_heads, wl.vocab, max_accept=64)
    table = None if d["block_table"] is None else d["block_table"].clone()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for k in range(args.warmup + args.steps):
        if k == args.warmup:
            torch.cuda.synchronize()
            e0.record()
        if table is not None:
            d["block_table"].copy_(table)
        st.run(d["parents"], d["tokens"], d["q"], d["k_new"], d["v_new"], d["logits"])
    e1.record()
    torch.cuda.synchronize()
    print(json.dumps({"workload": wl.name, "eager_us_per_step": e0.elapsed_time(e1) / args.steps * 1e3,
                      "steps": args.steps}))


if __name__ == "__main__":
    main()
