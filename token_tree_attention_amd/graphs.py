"""HIP graphs of a whole verification round, one per tree-size bucket.

"02 · Token Tree 与 Tree Attention" §6 counts the implementation cost of trees
in a serving loop: tree mask, RoPE rewriting, KV reclamation and the CUDA
graphs all have to be bucketed by the number of tree nodes, because a graph
replays fixed launch shapes.  ``GraphBuckets`` does that for the four calls:
for each bucket (node capacity T_cap, per-request node bound n_cap) it owns
static input buffers of that capacity and a ``VerifyStep`` built on them,
captures one round into a graph, and replays the smallest bucket a round
fits.

Why a smaller round can replay a larger bucket's graph: every kernel finds
its request's nodes through ``node_offsets`` on the device and treats the
host-side total node count and n_max as bounds only, so nodes past
``node_offsets[B]`` are never read as part of a request (the attention's
node workgroups past the last request's end exit; the argmax streams the
unused logits rows of the static buffer, which nothing reads).  The inputs
of a round are copied into the leading part of the static buffers before
the replay; the KV cache (and block table) is the caller's and is shared by
all buckets.
"""

from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import torch

from . import Batch, KVCache
from .step import VerifyStep


class GraphBuckets:
    def __init__(self, cache: KVCache, batch: int, n_heads: int, vocab: int, max_accept: int,
                 buckets: Sequence[Tuple[int, int]], logits_dtype=torch.bfloat16, rope_base: float = 10000.0,
                 device=None):
        device = device or cache.k.device
        self.cache, self.batch, self.vocab = cache, int(batch), int(vocab)
        self.n_heads, self.rope_base = int(n_heads), float(rope_base)
        Hkv, D = cache.n_kv_heads, cache.head_dim
        B = self.batch
        self.buckets: List[Dict] = []
        for T_cap, n_cap in sorted((int(t), int(n)) for t, n in buckets):
            i32 = dict(dtype=torch.int32, device=device)
            st = {
                "node_offsets": torch.zeros(B + 1, **i32),
                "ctx_lens": torch.zeros(B, **i32),
                "parents": torch.full((T_cap,), -1, **i32),
                "tokens": torch.zeros(T_cap, **i32),
                "q": torch.zeros((T_cap, n_heads, D), dtype=torch.bfloat16, device=device),
                "k_new": torch.zeros((T_cap, Hkv, D), dtype=torch.bfloat16, device=device),
                "v_new": torch.zeros((T_cap, Hkv, D), dtype=torch.bfloat16, device=device),
                "logits": torch.zeros((T_cap + B, vocab), dtype=logits_dtype, device=device),
            }
            bt = Batch(st["node_offsets"], st["ctx_lens"], n_cap, total_nodes=T_cap)
            step = VerifyStep(bt, cache, n_heads, vocab, max_accept)
            # one eager round on empty trees (no node, context 0: nothing in the
            # cache is touched) sets the kernels' launch attributes, then capture
            self._round(step, st)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._round(step, st)
            self.buckets.append({"T_cap": T_cap, "n_cap": n_cap, "static": st, "step": step, "graph": g})

    def _round(self, step: VerifyStep, st: Dict[str, torch.Tensor]) -> None:
        step.run(st["parents"], st["tokens"], st["q"], st["k_new"], st["v_new"], st["logits"], self.rope_base)

    def bucket_for(self, total_nodes: int, n_max: int) -> Dict:
        for bk in self.buckets:
            if total_nodes <= bk["T_cap"] and n_max <= bk["n_cap"]:
                return bk
        raise ValueError(f"no bucket holds {total_nodes} nodes with up to {n_max} per request")

    def run(self, node_offsets, ctx_lens, parents, tokens, q, k_new, v_new, logits, total_nodes: int,
            n_max: int) -> VerifyStep:
        """Copy one round's inputs into the fitting bucket and replay its graph.

        ``total_nodes`` (= node_offsets[B]) and ``n_max`` are the host-side
        sizes of the round.  Returns the bucket's VerifyStep, whose ``meta``,
        ``out``, ``acc`` and ``com`` hold the round's results (rows past
        ``total_nodes`` are not part of it)."""
        T, B = int(total_nodes), self.batch
        if node_offsets.numel() != B + 1 or ctx_lens.numel() != B:
            raise ValueError(f"the buckets were built for {B} requests")
        bk = self.bucket_for(T, int(n_max))
        st = bk["static"]
        st["node_offsets"].copy_(node_offsets)
        st["ctx_lens"].copy_(ctx_lens)
        st["parents"][:T].copy_(parents)
        st["tokens"][:T].copy_(tokens)
        st["q"][:T].copy_(q)
        st["k_new"][:T].copy_(k_new)
        st["v_new"][:T].copy_(v_new)
        st["logits"][:T + B].copy_(logits)
        bk["graph"].replay()
        return bk["step"]
