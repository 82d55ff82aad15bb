"""One verification round through the C ABI with preallocated buffers.

``VerifyStep`` owns the outputs and workspaces of the four calls for a fixed
batch shape, so a serving loop (or a benchmark) can run rounds without
allocating.  It only allocates and calls; the arithmetic is in the library.
"""

from __future__ import annotations

from typing import Dict

import torch

from . import (Batch, KVCache, tree_attention_verify, tree_attention_workspace_bytes, tree_build,
               tree_greedy_accept, tree_greedy_accept_workspace_bytes, tree_kv_commit, KV_PAGED)


class VerifyStep:
    def __init__(self, bt: Batch, cache: KVCache, n_heads: int, vocab: int, max_accept: int,
                 device=None):
        device = device or bt.node_offsets.device
        T, B, W = bt.total_nodes, bt.batch, bt.mask_words
        self.bt, self.cache, self.n_heads, self.vocab, self.max_accept = bt, cache, n_heads, vocab, max_accept
        i32 = dict(dtype=torch.int32, device=device)
        self.meta: Dict[str, torch.Tensor] = {"mask": torch.empty((T, W), **i32)}
        for k in ("depth", "positions", "retrieve_index", "retrieve_next_token", "retrieve_next_sibling"):
            self.meta[k] = torch.empty(T, **i32)
        self.meta["err"] = torch.empty(B, **i32)
        self.out = torch.empty((T, n_heads, cache.head_dim), dtype=torch.bfloat16, device=device)
        self.attn_ws = torch.empty(max(256, tree_attention_workspace_bytes(bt, cache, n_heads)),
                                   dtype=torch.uint8, device=device)
        self.acc: Dict[str, torch.Tensor] = {
            "accept_len": torch.empty(B, **i32),
            "accepted_nodes": torch.empty((B, max_accept), **i32),
            "out_tokens": torch.empty((B, max_accept + 1), **i32),
            "row_argmax": torch.empty(T + B, **i32),
        }
        self.acc_ws = torch.empty(max(256, tree_greedy_accept_workspace_bytes(bt, vocab)),
                                  dtype=torch.uint8, device=device)
        self.com: Dict[str, torch.Tensor] = {"new_lens": torch.empty(B, **i32)}
        if cache.layout == KV_PAGED:
            self.com["released_blocks"] = torch.empty((B, cache.max_blocks), **i32)
            self.com["num_released"] = torch.empty(B, **i32)

    def build(self, parents):
        return tree_build(self.bt, parents, out=self.meta)

    def attention(self, q, k_new, v_new, rope_base=10000.0, softmax_scale=0.0):
        return tree_attention_verify(self.bt, q, k_new, v_new, self.meta["mask"], self.meta["positions"],
                                     self.cache, self.meta["err"], rope_base=rope_base,
                                     softmax_scale=softmax_scale, out=self.out, workspace=self.attn_ws)

    def accept(self, logits, tokens):
        return tree_greedy_accept(self.bt, logits, tokens, self.meta["retrieve_next_token"],
                                  self.meta["retrieve_next_sibling"], self.max_accept, self.meta["err"],
                                  out=self.acc, workspace=self.acc_ws)

    def commit(self):
        return tree_kv_commit(self.bt, self.cache, self.acc["accept_len"], self.acc["accepted_nodes"],
                              self.meta["err"], out=self.com)

    def run(self, parents, tokens, q, k_new, v_new, logits, rope_base=10000.0):
        """tree_build -> tree_attention_verify -> tree_greedy_accept -> tree_kv_commit."""
        self.build(parents)
        self.attention(q, k_new, v_new, rope_base)
        self.accept(logits, tokens)
        self.commit()
