#!/usr/bin/env python3
"""Benchmark of one token-tree verification round on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
tree_build -> tree_attention_verify (one layer) -> tree_greedy_accept ->
tree_kv_commit (plus, for paged caches, restoring the block table that the
previous round's commit released, i.e. re-mapping the tentative blocks).

Default workload: an EAGLE-style 64-node tree (depth 6, top-4 expansion,
reranked), batch 1, committed context 4096, 32 query / 8 KV heads, head_dim
128, bf16 K/V/Q, vocab 128256 bf16 logits, contiguous cache.  ``--workload``
selects the other shapes (tiny_medusa, batched, ddtree, medusa_long,
ddtree_deep).

Inputs are uploaded before timing and rotated over enough copies (> 512 MB)
that each step reads cold HBM rather than the 256 MB Infinity Cache.  W
eager warm-up steps; then exactly K steps are captured in one HIP graph (the
way a serving loop replays a verify step per tree-size bucket) and one replay
is timed between two synchronisations, right after two untimed replays (the
GPU clock drops while idle and takes tens of milliseconds to recover).  The
attention call's duration comes from a second graph of K attention calls,
timed the same way with HIP events on its stream.  The eager (host-launched)
time per step is reported too.

Prints ONE JSON line: throughput in verified tree tokens/s (tree nodes per
second), ms and us per step, the attention roofline (algorithmic bytes per
call / measured call time against 8 TB/s HBM, or flops per call / call time
against the 2.5 PFLOP/s dense bf16 MFMA peak when the call's arithmetic
intensity is above the ridge of the two), and the CPU oracle's rate on a
bounded sample of the same workload.
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


def cpu_baseline(wl, budget_s):
    """Time the oracle on a bounded sample: whole requests' verify rounds."""
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import accept as O_acc
    from oracle import attention as O_att
    from oracle import bf16 as O_bf16
    from oracle import tree as O_tree

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = min(len(os.sched_getaffinity(0)), max(1, blas_threads))
    t0 = time.perf_counter()
    nodes_done = 0
    reqs_done = 0
    passes = 0
    # Whole requests in order, repeated (a small workload) until the budget is
    # spent; at least one node.
    while True:
        for b in range(wl.batch):
            s, e = int(wl.node_offsets[b]), int(wl.node_offsets[b + 1])
            n, ctx = e - s, int(wl.ctx_lens[b])
            sl = slice(s, e)
            O_tree.build(wl.parents[sl], np.array([0, n]), np.array([ctx]), max(1, n), max(1, (n + 31) // 32))
            kc, vc = O_att.context_of(wl.k_cache, wl.v_cache, b, ctx, wl.layout, wl.block_table)
            done_nodes = 0
            for i in range(n):
                O_att.attention_request(wl.q[sl], wl.k_new[sl], wl.v_new[sl], kc, vc, wl.parents[sl], ctx,
                                        nodes=[i])
                done_nodes += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            rows = wl.logits[s + b: e + b + 1]
            rows = O_bf16.to_f64(rows) if wl.logits_dtype == "bf16" else rows.astype(np.float64)
            choice = O_acc.row_argmax(rows)
            O_acc.greedy_walk(choice, wl.tokens[sl], wl.parents[sl], 64)
            nodes_done += done_nodes
            reqs_done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        passes += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": nodes_done / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{nodes_done} tree nodes in {reqs_done} request round(s) ({passes} pass(es) over the "
                      f"workload's requests): float64 oracle build, per-node path attention, argmax + walk "
                      f"of those requests ({dt:.1f} s)"}


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
        "kernel": "tree_attention_verify call (prep + main + combine launches), K calls back to back, HIP events on their stream",
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="eagle", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--rotate-mb", type=float, default=600.0,
                    help="rotate input copies until this many MB are in play (defeats the MALL)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle CPU work")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--eager-only", action="store_true",
                    help="host-launched steps only, no graph capture (for counter collection)")
    ap.add_argument("--copy-reference", type=float, default=0.0, metavar="MB",
                    help="instead of the path, run K device-to-device copies of MB megabytes "
                         "(the reference kernel for scaling the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU (asked for --gpus {args.gpus}); the verification path "
              f"runs on a single GPU and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import token_tree_attention_amd as tta
    from synth.device import to_device
    from token_tree_attention_amd.step import VerifyStep

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_reference > 0:
        copy_reference(args, dev)
        return
    tta.load_library()
    cfg = WORKLOADS[args.workload]
    wl = synth.make_workload(cfg, args.seed)
    base = to_device(wl, dev)
    per_set = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    n_sets = int(max(1, min(64, np.ceil(args.rotate_mb * 1e6 / per_set))))
    free = torch.cuda.mem_get_info()[0]
    n_sets = int(max(1, min(n_sets, (free * 0.6) // max(1, per_set))))
    sets = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()} for _ in range(n_sets - 1)]
    steps = []
    pristine_tables = []
    for d in sets:
        bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=wl.total_nodes)
        cache = tta.KVCache(d["k_cache"], d["v_cache"], d["block_table"])
        steps.append((d, VerifyStep(bt, cache, wl.n_heads, wl.vocab, max_accept=64)))
        pristine_tables.append(None if d["block_table"] is None else d["block_table"].clone())
    stream = torch.cuda.current_stream()

    def run(i):
        d, st = steps[i % n_sets]
        if pristine_tables[i % n_sets] is not None:
            d["block_table"].copy_(pristine_tables[i % n_sets], non_blocking=True)
        st.build(d["parents"])
        st.attention(d["q"], d["k_new"], d["v_new"])
        st.accept(d["logits"], d["tokens"])
        st.commit()

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    errs = steps[0][1].meta["err"].cpu().numpy()
    if (errs != 0).any():
        print(f"device error bits after warm-up: {errs.tolist()}", file=sys.stderr)
        sys.exit(1)
    ref_acc = {k: v.clone() for k, v in steps[0][1].acc.items()}

    # Eager timing (host-launched, for reference).
    t0e = torch.cuda.Event(enable_timing=True)
    t1e = torch.cuda.Event(enable_timing=True)
    t0e.record(stream)
    for k in range(args.steps):
        run(args.warmup + k)
    t1e.record(stream)
    torch.cuda.synchronize()
    eager_ms = t0e.elapsed_time(t1e) / args.steps

    def check_replay():
        for key, ref in ref_acc.items():  # a replay reproduces the eager result
            if not torch.equal(steps[0][1].acc[key], ref):
                print(f"graph replay differs from eager in {key}", file=sys.stderr)
                sys.exit(1)

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

    def restore_tables():
        # Commits release each round's tentative blocks; the attention-only
        # timing runs on the tables as the rounds found them (untimed copy).
        for (d, _), t in zip(steps, pristine_tables):
            if t is not None:
                d["block_table"].copy_(t)
        torch.cuda.synchronize()

    def attention_calls():
        for k in range(args.steps):
            d, st = steps[k % n_sets]
            st.attention(d["q"], d["k_new"], d["v_new"])

    if args.eager_only:
        ms_step = eager_ms
        restore_tables()
        attention_calls()
        attn_ms = timed(attention_calls) / args.steps
        timing = "host-launched steps"
    else:
        # The timed region: exactly K steps captured in one HIP graph (rotating
        # input sets), replayed once after one untimed replay.
        g_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step):
            for k in range(args.steps):
                run(k)
        g_attn = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_attn):
            attention_calls()
        g_step.replay()
        torch.cuda.synchronize()
        check_replay()
        # The GPU lowers its clock while idle (graph capture, the check above)
        # and needs tens of milliseconds of work to come back up: two untimed
        # replays right before the timed one, so it measures steady state.
        g_step.replay()
        g_step.replay()
        ms_step = timed(g_step.replay) / args.steps
        # Attention calls alone: K calls back to back in one replay (also
        # after two untimed ones).
        restore_tables()
        g_attn.replay()
        g_attn.replay()
        attn_ms = timed(g_attn.replay) / args.steps
        check_replay()
        timing = "K steps in one HIP graph replay"
    attn_bytes, flops, accept_bytes = algorithmic(wl)
    acc_len = steps[0][1].acc["accept_len"].cpu().numpy()
    result = {
        "metric": METRIC,
        "value": wl.total_nodes / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "us_per_step": ms_step * 1e3,
        "eager_us_per_step": eager_ms * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": describe(wl),
        "roofline": roofline_entry(wl, attn_bytes, flops, attn_ms),
        "accept_len_hist": np.bincount(acc_len).tolist(),
        "input_sets_rotated": n_sets,
        "timing": timing,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
