"""The debug build (TTV_DEBUG: device bounds checks in every kernel) on the
GPU: whole rounds of several workloads and the calls beyond the round run
with no failed check, and their results equal the release build's.

Both builds are loaded in one child process each (a library stays loaded for
the life of a process); the child prints what it computed, this test compares."""

import json
import os
import subprocess
import sys

import pytest

from gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import hashlib, json, os, sys
sys.path.insert(0, os.environ["TTV_ROOT"])
sys.path.insert(0, os.path.join(os.environ["TTV_ROOT"], "tests"))
import numpy as np, torch
import synth, token_tree_attention_amd as tta
from synth.device import to_device
from token_tree_attention_amd.step import VerifyStep

def digest(*ts):
    h = hashlib.sha256()
    for t in ts:
        h.update(t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()[:16]

out = {"library": os.path.basename(tta.library_path())}
dev = torch.device("cuda")
cases = [(0, {}), (1, dict(ctx=(1500, 1500))), (2, dict(batch=6, ctx=(100, 700))),
         (3, dict(batch=1, ctx=(300, 300), vocab=4096)), (4, dict(batch=3, ctx=(50, 900)))]
for cfg, over in cases:
    wl = synth.make_workload(cfg, 5, **over)
    d = to_device(wl, dev)
    bt = tta.Batch(d["node_offsets"], d["ctx_lens"], max(1, wl.n_max), total_nodes=wl.total_nodes)
    cache = tta.KVCache(d["k_cache"], d["v_cache"], d["block_table"])
    st = VerifyStep(bt, cache, wl.n_heads, wl.vocab, 64)
    st.run(d["parents"], d["tokens"], d["q"], d["k_new"], d["v_new"], d["logits"])
    torch.cuda.synchronize()
    out[f"round{cfg}"] = digest(st.meta["mask"], st.meta["positions"], st.out, st.acc["accept_len"],
                                st.acc["out_tokens"], st.com["new_lens"], d["k_cache"], d["v_cache"])
    out[f"err{cfg}"] = st.meta["err"].cpu().tolist()
# beyond the round: sampled and stochastic walks, DDTree, merge, EAGLE, dense masks
wl = synth.make_workload(2, 6, batch=5, ctx=(10, 40), vocab=3000)
d = to_device(wl, dev)
bt = tta.Batch(d["node_offsets"], d["ctx_lens"], wl.n_max, total_nodes=wl.total_nodes)
meta = tta.tree_build(bt, d["parents"])
R, V = wl.total_nodes + wl.batch, wl.vocab
g = torch.from_numpy(synth.gumbel_noise(6, 2, R, V)).to(dev)
q = torch.from_numpy(synth.draft_distributions(6, 2, R, V)).to(dev)
u = torch.from_numpy(synth.uniforms(6, 2, wl.total_nodes)).to(dev)
a = tta.tree_sample_accept(bt, d["logits"], g, 0.7, d["tokens"], meta["retrieve_next_token"],
                           meta["retrieve_next_sibling"], 32, meta["err"])
b = tta.tree_stochastic_accept(bt, d["logits"], 1.0, q, u, g, d["tokens"], meta["retrieve_next_token"],
                               meta["retrieve_next_sibling"], 32, meta["err"])
z = torch.from_numpy(synth.draft_logits(6, 3, 2, 6, 2000, 2.0, 2)).to(dev)
c = tta.tree_ddtree_build(z, 300)
seqs = torch.from_numpy(np.random.default_rng(6).integers(0, 3, size=(3, 40, 6)).astype(np.int32)).to(dev)
m = tta.tree_merge_sequences(seqs, 1024)
rng = np.random.default_rng(7)
e = tta.tree_eagle_grow(torch.from_numpy(rng.integers(0, 999, (2, 4)).astype(np.int32)).to(dev),
                        torch.from_numpy(rng.uniform(0.1, 0.9, (2, 4)).astype(np.float32)).to(dev),
                        torch.from_numpy(rng.integers(0, 999, (2, 5, 4, 4)).astype(np.int32)).to(dev),
                        torch.from_numpy(rng.uniform(0.1, 0.9, (2, 5, 4, 4)).astype(np.float32)).to(dev), 64)
stride = int((wl.ctx_lens + np.diff(wl.node_offsets)).max()) + 3
dense = tta.tree_expand_mask(bt, meta["mask"], tta.MASK_FULL, stride, meta["err"])
packed = tta.tree_pack_mask(bt, dense, tta.MASK_FULL, meta["err"], mask_words=meta["mask"].shape[1])
torch.cuda.synchronize()
out["next"] = digest(a["accept_len"], a["out_tokens"], a["row_argmax"], b["accept_len"], b["out_tokens"],
                     c["parents"], c["tokens"], m["parents"], m["tokens"], e["parents"], e["tokens"],
                     dense, packed)
out["next_err"] = meta["err"].cpu().tolist()
out["report"] = tta.ttv_debug_report(reset=True)
print("RESULT " + json.dumps(out), flush=True)
'''


def run_child(debug):
    env = dict(os.environ, TTV_ROOT=ROOT)
    env.pop("TTV_LIBRARY", None)
    env["TTV_DEBUG"] = "1" if debug else "0"
    r = subprocess.run([sys.executable, "-c", CHILD], env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    lines = [l for l in r.stdout.splitlines() if l.startswith("RESULT ")]
    assert r.returncode == 0 and lines, r.stdout[-3000:]
    return json.loads(lines[-1][len("RESULT "):])


def test_debug_build_checks_pass_and_match_release():
    require_gpu()
    if not os.path.exists(os.path.join(ROOT, "token_tree_attention_amd", "libtreeverify_debug.so")):
        pytest.skip("debug library not built")
    say("debug build: rounds of five workloads and the calls beyond the round")
    dbg = run_child(True)
    say(f"  report {dbg['report']}")
    rel = run_child(False)
    assert dbg["library"] == "libtreeverify_debug.so" and rel["library"] == "libtreeverify.so"
    assert rel["report"] is None
    assert dbg["report"] == [0, 0], f"failed device checks: {dbg['report']}"
    for k, v in rel.items():
        if k not in ("library", "report"):
            assert dbg[k] == v, k
