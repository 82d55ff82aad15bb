"""token_tree_attention_amd -- MI355X (gfx950) token-tree verification.

A thin ctypes binding of ``libtreeverify.so`` (declared in
``include/treeverify.h``).  Functions carry the C names and only marshal
arguments: torch tensors go in as raw device pointers on the caller's current
stream; every step of the path runs in the library's HIP kernels.  Importing
works without a GPU; calling a compute function needs the built library and
a ROCm device, and raises if either is missing (there is no CPU fallback).

Typical round (all tensors on one ``cuda`` device)::

    bt = Batch(node_offsets, ctx_lens, n_max)
    meta = tree_build(bt, parents)
    out = tree_attention_verify(bt, q, k_new, v_new, meta["mask"], meta["positions"], cache)
    acc = tree_greedy_accept(bt, logits, tokens, meta["retrieve_next_token"],
                             meta["retrieve_next_sibling"], max_accept=16, err=meta["err"])
    com = tree_kv_commit(bt, cache, acc["accept_len"], acc["accepted_nodes"], err=meta["err"])
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

__all__ = [
    "Batch", "KVCache", "library_path", "load_library", "ttv_version", "ttv_status_string", "ttv_debug_report",
    "tree_build", "tree_attention_workspace_bytes", "tree_attention_verify",
    "tree_greedy_accept_workspace_bytes", "tree_greedy_accept", "tree_greedy_accept_noalloc",
    "tree_sample_accept", "tree_stochastic_accept_workspace_bytes", "tree_stochastic_accept",
    "tree_kv_commit", "tree_expand_mask", "tree_pack_mask", "tree_ddtree_workspace_bytes",
    "tree_ddtree_build", "tree_merge_sequences", "tree_eagle_grow", "MASK_QLEN_ONLY", "MASK_FULL", "ERR_BAD_MASK", "ERR_SYNC",
    "TTV_OK", "TTV_EINVAL", "TTV_EHIP", "TTV_ENOSPC", "ERR_BAD_PARENT", "ERR_TOO_MANY_NODES",
    "ERR_CAPACITY", "ERR_BLOCK_TABLE", "ERR_ACCEPT", "ERR_BAD_LENGTH", "MAX_TREE_NODES",
    "BLOCK_SIZE", "EXPORTED_SYMBOLS",
]

TTV_OK, TTV_EINVAL, TTV_EHIP, TTV_ENOSPC = 0, -1, -2, -3
ERR_BAD_PARENT, ERR_TOO_MANY_NODES, ERR_CAPACITY = 1, 2, 4
ERR_BLOCK_TABLE, ERR_ACCEPT, ERR_BAD_LENGTH, ERR_BAD_MASK, ERR_SYNC = 8, 16, 32, 64, 128
MASK_QLEN_ONLY, MASK_FULL = 0, 1
MAX_TREE_NODES = 1024
BLOCK_SIZE = 16
DTYPE_FP32, DTYPE_BF16 = 0, 1
KV_CONTIGUOUS, KV_PAGED = 0, 1

EXPORTED_SYMBOLS = (
    "ttv_version", "ttv_status_string", "tree_build", "tree_attention_workspace_bytes",
    "tree_attention_verify", "tree_greedy_accept_workspace_bytes", "tree_greedy_accept",
    "tree_greedy_accept_noalloc", "tree_sample_accept", "tree_stochastic_accept_workspace_bytes",
    "tree_stochastic_accept", "tree_kv_commit", "tree_expand_mask", "tree_pack_mask",
    "tree_ddtree_workspace_bytes", "tree_ddtree_build", "tree_merge_sequences", "tree_eagle_grow",
    "ttv_debug_report",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None


def library_path() -> str:
    """The built library next to this file; with TTV_DEBUG=1 in the
    environment its debug build (device bounds checks, libtreeverify_debug.so);
    or the one TTV_LIBRARY names (for instance the host-sanitized build the
    argument-checking tests load)."""
    if os.environ.get("TTV_LIBRARY"):
        return os.environ["TTV_LIBRARY"]
    if os.environ.get("TTV_DEBUG", "") not in ("", "0"):
        return os.path.join(_HERE, "libtreeverify_debug.so")
    return os.path.join(_HERE, "libtreeverify.so")


class _CBatch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_max", ctypes.c_int32),
                ("total_nodes", ctypes.c_int64), ("node_offsets", ctypes.c_void_p),
                ("ctx_lens", ctypes.c_void_p)]


class _CCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("layout", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32)]


def load_library() -> ctypes.CDLL:
    """Load libtreeverify.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with python -m token_tree_attention_amd.build")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    BP, CP = ctypes.POINTER(_CBatch), ctypes.POINTER(_CCache)
    lib.ttv_version.restype = I32
    lib.ttv_version.argtypes = []
    lib.ttv_status_string.restype = ctypes.c_char_p
    lib.ttv_status_string.argtypes = [I32]
    lib.ttv_debug_report.restype = ctypes.c_int
    lib.ttv_debug_report.argtypes = [P, P, I32]
    lib.tree_build.restype = ctypes.c_int
    lib.tree_build.argtypes = [BP, P, P, I32, P, P, P, P, P, P, P]
    lib.tree_attention_workspace_bytes.restype = SZ
    lib.tree_attention_workspace_bytes.argtypes = [BP, CP, I32]
    lib.tree_attention_verify.restype = ctypes.c_int
    lib.tree_attention_verify.argtypes = [BP, P, P, P, P, I32, P, CP, I32, F32, F32, P, P, SZ, P, P]
    lib.tree_greedy_accept_workspace_bytes.restype = SZ
    lib.tree_greedy_accept_workspace_bytes.argtypes = [BP, I64]
    lib.tree_greedy_accept.restype = ctypes.c_int
    lib.tree_greedy_accept.argtypes = [BP, P, I32, I64, P, P, P, I32, P, P, P, P, P, SZ, P, P]
    lib.tree_greedy_accept_noalloc.restype = ctypes.c_int
    lib.tree_greedy_accept_noalloc.argtypes = [BP, P, I32, I64, P, P, P, I32, P, P, P, P, P, P]
    lib.tree_sample_accept.restype = ctypes.c_int
    lib.tree_sample_accept.argtypes = [BP, P, I32, I64, F32, P, P, P, P, I32, P, P, P, P, P, SZ, P, P]
    lib.tree_stochastic_accept_workspace_bytes.restype = SZ
    lib.tree_stochastic_accept_workspace_bytes.argtypes = [BP, I64]
    lib.tree_stochastic_accept.restype = ctypes.c_int
    lib.tree_stochastic_accept.argtypes = [BP, P, I32, I64, F32, P, P, P, P, P, P, I32, P, P, P, P, SZ, P, P]
    lib.tree_expand_mask.restype = ctypes.c_int
    lib.tree_expand_mask.argtypes = [BP, P, I32, I32, P, I64, P, P]
    lib.tree_pack_mask.restype = ctypes.c_int
    lib.tree_pack_mask.argtypes = [BP, P, I64, I32, P, I32, P, P]
    lib.tree_ddtree_workspace_bytes.restype = SZ
    lib.tree_ddtree_workspace_bytes.argtypes = [I32, I32, I64, I32]
    lib.tree_ddtree_build.restype = ctypes.c_int
    lib.tree_ddtree_build.argtypes = [I32, I32, I64, I32, P, P, P, P, P, SZ, P]
    lib.tree_merge_sequences.restype = ctypes.c_int
    lib.tree_merge_sequences.argtypes = [I32, I32, I32, P, I32, P, P, P, P, P]
    lib.tree_eagle_grow.restype = ctypes.c_int
    lib.tree_eagle_grow.argtypes = [I32, I32, I32, P, P, P, P, I32, P, P, P, P]
    lib.tree_kv_commit.restype = ctypes.c_int
    lib.tree_kv_commit.argtypes = [BP, CP, P, P, I32, P, P, P, P, P]
    _LIB = lib
    return lib


def ttv_version() -> int:
    return int(load_library().ttv_version())


def ttv_status_string(status: int) -> str:
    return load_library().ttv_status_string(int(status)).decode()


def ttv_debug_report(reset: bool = False):
    """(failed checks, first failing site) of the debug build on the current
    device (synchronise first), or None from a release build."""
    lib = load_library()
    count, site = ctypes.c_uint32(0), ctypes.c_int32(0)
    st = lib.ttv_debug_report(ctypes.addressof(count), ctypes.addressof(site), int(bool(reset)))
    if st == TTV_EINVAL:
        return None
    _check(st, "ttv_debug_report")
    return int(count.value), int(site.value)


def _check(status: int, what: str) -> None:
    if status != TTV_OK:
        raise RuntimeError(f"{what}: {ttv_status_string(status)} (status {status})")


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _dev(t, dtype, name, numel=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return t


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


class Batch:
    """Requests of one verify round: node_offsets [B+1] and ctx_lens [B] (int32, device)."""

    def __init__(self, node_offsets, ctx_lens, n_max: int, total_nodes: Optional[int] = None):
        torch = _torch()
        self.node_offsets = _dev(node_offsets, torch.int32, "node_offsets")
        self.ctx_lens = _dev(ctx_lens, torch.int32, "ctx_lens")
        self.batch = int(ctx_lens.numel())
        if node_offsets.numel() != self.batch + 1:
            raise ValueError("node_offsets must have batch + 1 entries")
        self.n_max = int(n_max)
        self.total_nodes = int(total_nodes) if total_nodes is not None else int(node_offsets[-1].item())
        self._c = _CBatch(self.batch, self.n_max, self.total_nodes,
                          _ptr(self.node_offsets), _ptr(self.ctx_lens))

    @property
    def mask_words(self) -> int:
        return max(1, (self.n_max + 31) // 32)


class KVCache:
    """bf16 K/V cache: contiguous [B, Hkv, capacity, D] or paged [num_blocks, Hkv, 16, D]."""

    def __init__(self, k, v, block_table=None):
        torch = _torch()
        self.k = _dev(k, torch.bfloat16, "k")
        self.v = _dev(v, torch.bfloat16, "v")
        if k.shape != v.shape or k.dim() != 4:
            raise ValueError("k and v must have the same 4-d shape")
        self.block_table = block_table
        if block_table is None:
            self.layout = KV_CONTIGUOUS
            _, hkv, cap, d = k.shape
            self._c = _CCache(_ptr(k), _ptr(v), KV_CONTIGUOUS, hkv, d, cap, None, 0, 0, 0)
        else:
            _dev(block_table, torch.int32, "block_table")
            if block_table.dim() != 2:
                raise ValueError("block_table must be [B, max_blocks]")
            self.layout = KV_PAGED
            nb, hkv, bs, d = k.shape
            if bs != BLOCK_SIZE:
                raise ValueError(f"paged blocks must hold {BLOCK_SIZE} tokens")
            self._c = _CCache(_ptr(k), _ptr(v), KV_PAGED, hkv, d, 0, _ptr(block_table),
                              block_table.shape[1], bs, nb)
        self.n_kv_heads = int(k.shape[1])
        self.head_dim = int(k.shape[3])

    @property
    def max_blocks(self) -> int:
        return 0 if self.block_table is None else int(self.block_table.shape[1])


def _check_cache_rows(bt: Batch, cache: "KVCache") -> None:
    """A contiguous cache holds B requests; a paged block table has B rows."""
    if cache.layout == KV_CONTIGUOUS:
        if int(cache.k.shape[0]) != bt.batch:
            raise ValueError(f"contiguous cache must be [B={bt.batch}, Hkv, capacity, D], "
                             f"got {tuple(cache.k.shape)}")
    elif int(cache.block_table.shape[0]) != bt.batch:
        raise ValueError(f"block_table must have B={bt.batch} rows, got {tuple(cache.block_table.shape)}")


def tree_build(bt: Batch, parents, out: Optional[Dict] = None, stream=None) -> Dict:
    """Masks, depths, positions and retrieve indices for every request's tree."""
    torch = _torch()
    lib = load_library()
    T = bt.total_nodes
    _dev(parents, torch.int32, "parents", T)
    dev = parents.device
    W = bt.mask_words
    if out is None:
        out = {"mask": torch.empty((T, W), dtype=torch.int32, device=dev)}
        for k in ("depth", "positions", "retrieve_index", "retrieve_next_token", "retrieve_next_sibling"):
            out[k] = torch.empty(T, dtype=torch.int32, device=dev)
        out["err"] = torch.empty(bt.batch, dtype=torch.int32, device=dev)
    st = lib.tree_build(ctypes.byref(bt._c), _ptr(parents), _ptr(out["mask"]), W, _ptr(out["depth"]),
                        _ptr(out["positions"]), _ptr(out["retrieve_index"]),
                        _ptr(out["retrieve_next_token"]), _ptr(out["retrieve_next_sibling"]),
                        _ptr(out["err"]), _stream(stream))
    _check(st, "tree_build")
    return out


def tree_attention_workspace_bytes(bt: Batch, cache: KVCache, n_heads: int) -> int:
    return int(load_library().tree_attention_workspace_bytes(ctypes.byref(bt._c), ctypes.byref(cache._c), int(n_heads)))


def tree_attention_verify(bt: Batch, q, k_new, v_new, mask, positions, cache: KVCache, err,
                          rope_base: float = 10000.0, softmax_scale: float = 0.0, out=None,
                          workspace=None, stream=None):
    """One layer of tree attention; writes rotated K / V into the tentative slots."""
    torch = _torch()
    lib = load_library()
    T = bt.total_nodes
    # Shapes first (they need no device), then dtype / device / layout.
    if q.dim() != 3 or q.shape[0] != T or q.shape[2] != cache.head_dim:
        raise ValueError(f"q must be [T={T}, n_heads, D={cache.head_dim}], got {tuple(q.shape)}")
    n_heads = int(q.shape[1])
    if mask.dim() != 2 or mask.shape[0] != T or not (bt.mask_words <= mask.shape[1] <= MAX_TREE_NODES // 32):
        raise ValueError(f"mask must be [T={T}, W] with {bt.mask_words} <= W <= {MAX_TREE_NODES // 32}, "
                         f"got {tuple(mask.shape)}")
    _check_cache_rows(bt, cache)
    if out is not None and tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out must have q's shape {tuple(q.shape)}, got {tuple(out.shape)}")
    _dev(q, torch.bfloat16, "q")
    _dev(k_new, torch.bfloat16, "k_new", T * cache.n_kv_heads * cache.head_dim)
    _dev(v_new, torch.bfloat16, "v_new", T * cache.n_kv_heads * cache.head_dim)
    _dev(mask, torch.int32, "mask")
    _dev(positions, torch.int32, "positions", T)
    _dev(err, torch.int32, "err", bt.batch)
    W = int(mask.shape[1])
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.bfloat16, "out")
    need = tree_attention_workspace_bytes(bt, cache, n_heads)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, torch.uint8, "workspace")
    st = lib.tree_attention_verify(ctypes.byref(bt._c), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(mask), W,
                                   _ptr(positions), ctypes.byref(cache._c), n_heads, float(rope_base),
                                   float(softmax_scale), _ptr(out), _ptr(workspace), workspace.numel(),
                                   _ptr(err), _stream(stream))
    _check(st, "tree_attention_verify")
    return out


def tree_greedy_accept_workspace_bytes(bt: Batch, vocab: int) -> int:
    return int(load_library().tree_greedy_accept_workspace_bytes(ctypes.byref(bt._c), int(vocab)))


def tree_greedy_accept(bt: Batch, logits, tokens, retrieve_next_token, retrieve_next_sibling,
                       max_accept: int, err, out: Optional[Dict] = None, workspace=None,
                       want_row_argmax: bool = True, stream=None) -> Dict:
    """Row argmax of every logits row and the greedy walk of every request."""
    torch = _torch()
    lib = load_library()
    T, B = bt.total_nodes, bt.batch
    if logits.dim() != 2 or logits.shape[0] != T + B:
        raise ValueError("logits must be [T + B, vocab]")
    if logits.dtype == torch.float32:
        dt = DTYPE_FP32
    elif logits.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    else:
        raise TypeError("logits must be float32 or bfloat16")
    _dev(logits, logits.dtype, "logits")
    vocab = int(logits.shape[1])
    _dev(tokens, torch.int32, "tokens", T)
    _dev(retrieve_next_token, torch.int32, "retrieve_next_token", T)
    _dev(retrieve_next_sibling, torch.int32, "retrieve_next_sibling", T)
    _dev(err, torch.int32, "err", B)
    dev = logits.device
    if out is None:
        out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
               "accepted_nodes": torch.empty((B, max_accept), dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((B, max_accept + 1), dtype=torch.int32, device=dev)}
        if want_row_argmax:
            out["row_argmax"] = torch.empty(T + B, dtype=torch.int32, device=dev)
    need = tree_greedy_accept_workspace_bytes(bt, vocab)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _dev(workspace, torch.uint8, "workspace")
    _check_accept_outputs(out, B, int(max_accept), T)
    st = lib.tree_greedy_accept(ctypes.byref(bt._c), _ptr(logits), dt, vocab, _ptr(tokens),
                                _ptr(retrieve_next_token), _ptr(retrieve_next_sibling), int(max_accept),
                                _ptr(out["accept_len"]), _ptr(out["accepted_nodes"]), _ptr(out["out_tokens"]),
                                _ptr(out.get("row_argmax")), _ptr(workspace), workspace.numel(), _ptr(err),
                                _stream(stream))
    _check(st, "tree_greedy_accept")
    return out


def tree_greedy_accept_noalloc(bt: Batch, logits, tokens, retrieve_next_token, retrieve_next_sibling,
                               max_accept: int, err, out: Dict, stream=None) -> Dict:
    """tree_greedy_accept without a workspace (the library's static device
    scratch holds the argmax keys); ``out`` must be preallocated, since this
    entry point exists for callers that cannot allocate."""
    torch = _torch()
    lib = load_library()
    T, B = bt.total_nodes, bt.batch
    if logits.dim() != 2 or logits.shape[0] != T + B:
        raise ValueError("logits must be [T + B, vocab]")
    if logits.dtype == torch.float32:
        dt = DTYPE_FP32
    elif logits.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    else:
        raise TypeError("logits must be float32 or bfloat16")
    _dev(logits, logits.dtype, "logits")
    _dev(tokens, torch.int32, "tokens", T)
    _dev(retrieve_next_token, torch.int32, "retrieve_next_token", T)
    _dev(retrieve_next_sibling, torch.int32, "retrieve_next_sibling", T)
    _dev(err, torch.int32, "err", B)
    _check_accept_outputs(out, B, int(max_accept), T)
    st = lib.tree_greedy_accept_noalloc(ctypes.byref(bt._c), _ptr(logits), dt, int(logits.shape[1]), _ptr(tokens),
                                        _ptr(retrieve_next_token), _ptr(retrieve_next_sibling), int(max_accept),
                                        _ptr(out["accept_len"]), _ptr(out["accepted_nodes"]),
                                        _ptr(out["out_tokens"]), _ptr(out.get("row_argmax")), _ptr(err),
                                        _stream(stream))
    _check(st, "tree_greedy_accept_noalloc")
    return out


def _logits_dtype(logits, T: int, B: int) -> int:
    torch = _torch()
    if logits.dim() != 2 or logits.shape[0] != T + B:
        raise ValueError("logits must be [T + B, vocab]")
    if logits.dtype == torch.float32:
        return DTYPE_FP32
    if logits.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError("logits must be float32 or bfloat16")


def _accept_outputs(out, B: int, max_accept: int, T: int, dev, want_rows: bool) -> Dict:
    torch = _torch()
    if out is None:
        out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
               "accepted_nodes": torch.empty((B, max_accept), dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((B, max_accept + 1), dtype=torch.int32, device=dev)}
        if want_rows:
            out["row_argmax"] = torch.empty(T + B, dtype=torch.int32, device=dev)
    return out


def tree_sample_accept(bt: Batch, logits, gumbel, temperature: float, tokens, retrieve_next_token,
                       retrieve_next_sibling, max_accept: int, err, out: Optional[Dict] = None,
                       workspace=None, want_row_choice: bool = True, stream=None) -> Dict:
    """The verifier walk with temperature-sampled choices: argmax of logits / T +
    Gumbel noise per row (``out["row_argmax"]`` holds the choices)."""
    torch = _torch()
    lib = load_library()
    T, B = bt.total_nodes, bt.batch
    dt = _logits_dtype(logits, T, B)
    _dev(logits, logits.dtype, "logits")
    vocab = int(logits.shape[1])
    _dev(gumbel, torch.float32, "gumbel", (T + B) * vocab)
    _dev(tokens, torch.int32, "tokens", T)
    _dev(retrieve_next_token, torch.int32, "retrieve_next_token", T)
    _dev(retrieve_next_sibling, torch.int32, "retrieve_next_sibling", T)
    _dev(err, torch.int32, "err", B)
    out = _accept_outputs(out, B, int(max_accept), T, logits.device, want_row_choice)
    _check_accept_outputs(out, B, int(max_accept), T)
    if workspace is None:
        workspace = torch.empty(max(tree_greedy_accept_workspace_bytes(bt, vocab), 256), dtype=torch.uint8,
                                device=logits.device)
    _dev(workspace, torch.uint8, "workspace")
    st = lib.tree_sample_accept(ctypes.byref(bt._c), _ptr(logits), dt, vocab, float(temperature), _ptr(gumbel),
                                _ptr(tokens), _ptr(retrieve_next_token), _ptr(retrieve_next_sibling),
                                int(max_accept), _ptr(out["accept_len"]), _ptr(out["accepted_nodes"]),
                                _ptr(out["out_tokens"]), _ptr(out.get("row_argmax")), _ptr(workspace),
                                workspace.numel(), _ptr(err), _stream(stream))
    _check(st, "tree_sample_accept")
    return out


def tree_stochastic_accept_workspace_bytes(bt: Batch, vocab: int) -> int:
    return int(load_library().tree_stochastic_accept_workspace_bytes(ctypes.byref(bt._c), int(vocab)))


def tree_stochastic_accept(bt: Batch, logits, temperature: float, draft_probs, uniforms, gumbel, tokens,
                           retrieve_next_token, retrieve_next_sibling, max_accept: int, err,
                           out: Optional[Dict] = None, workspace=None, stream=None) -> Dict:
    """The stochastic min(1, p/q) walk: draft_probs [T + B, V] (the draft
    distribution of each row's children), uniforms [T], gumbel [T + B, V]."""
    torch = _torch()
    lib = load_library()
    T, B = bt.total_nodes, bt.batch
    dt = _logits_dtype(logits, T, B)
    _dev(logits, logits.dtype, "logits")
    vocab = int(logits.shape[1])
    _dev(draft_probs, torch.float32, "draft_probs", (T + B) * vocab)
    _dev(uniforms, torch.float32, "uniforms", T)
    _dev(gumbel, torch.float32, "gumbel", (T + B) * vocab)
    _dev(tokens, torch.int32, "tokens", T)
    _dev(retrieve_next_token, torch.int32, "retrieve_next_token", T)
    _dev(retrieve_next_sibling, torch.int32, "retrieve_next_sibling", T)
    _dev(err, torch.int32, "err", B)
    out = _accept_outputs(out, B, int(max_accept), T, logits.device, False)
    _check_accept_outputs(out, B, int(max_accept), T)
    if workspace is None:
        workspace = torch.empty(max(tree_stochastic_accept_workspace_bytes(bt, vocab), 256), dtype=torch.uint8,
                                device=logits.device)
    _dev(workspace, torch.uint8, "workspace")
    st = lib.tree_stochastic_accept(ctypes.byref(bt._c), _ptr(logits), dt, vocab, float(temperature),
                                    _ptr(draft_probs), _ptr(uniforms), _ptr(gumbel), _ptr(tokens),
                                    _ptr(retrieve_next_token), _ptr(retrieve_next_sibling), int(max_accept),
                                    _ptr(out["accept_len"]), _ptr(out["accepted_nodes"]), _ptr(out["out_tokens"]),
                                    _ptr(workspace), workspace.numel(), _ptr(err), _stream(stream))
    _check(st, "tree_stochastic_accept")
    return out


def _check_accept_outputs(out: Dict, B: int, max_accept: int, T: int) -> None:
    torch = _torch()
    _dev(out["accept_len"], torch.int32, "accept_len", B)
    _dev(out["accepted_nodes"], torch.int32, "accepted_nodes", B * max_accept)
    _dev(out["out_tokens"], torch.int32, "out_tokens", B * (max_accept + 1))
    if out.get("row_argmax") is not None:
        _dev(out["row_argmax"], torch.int32, "row_argmax", T + B)


def tree_kv_commit(bt: Batch, cache: KVCache, accept_len, accepted_nodes, err,
                   out: Optional[Dict] = None, stream=None) -> Dict:
    """Move the accepted nodes' K/V into place; paged caches also release blocks."""
    torch = _torch()
    lib = load_library()
    B = bt.batch
    if accepted_nodes.dim() != 2 or accepted_nodes.shape[0] != B:
        raise ValueError(f"accepted_nodes must be [B={B}, max_accept], got {tuple(accepted_nodes.shape)}")
    _check_cache_rows(bt, cache)
    _dev(accept_len, torch.int32, "accept_len", B)
    _dev(accepted_nodes, torch.int32, "accepted_nodes")
    max_accept = int(accepted_nodes.shape[1])
    _dev(err, torch.int32, "err", B)
    dev = accept_len.device
    if out is None:
        out = {"new_lens": torch.empty(B, dtype=torch.int32, device=dev)}
        if cache.layout == KV_PAGED:
            out["released_blocks"] = torch.empty((B, cache.max_blocks), dtype=torch.int32, device=dev)
            out["num_released"] = torch.empty(B, dtype=torch.int32, device=dev)
    st = lib.tree_kv_commit(ctypes.byref(bt._c), ctypes.byref(cache._c), _ptr(accept_len),
                            _ptr(accepted_nodes), max_accept, _ptr(out["new_lens"]),
                            _ptr(out.get("released_blocks")), _ptr(out.get("num_released")),
                            _ptr(err), _stream(stream))
    _check(st, "tree_kv_commit")
    return out


def tree_expand_mask(bt: Batch, mask, mode: int, row_stride: int, err, out=None, stream=None):
    """Dense uint8 [T, row_stride] mask (MASK_QLEN_ONLY or MASK_FULL) from tree_build's packed rows."""
    torch = _torch()
    lib = load_library()
    T = bt.total_nodes
    if mask.dim() != 2 or mask.shape[0] != T:
        raise ValueError(f"mask must be [T={T}, W]")
    _dev(mask, torch.int32, "mask")
    _dev(err, torch.int32, "err", bt.batch)
    if out is None:
        out = torch.empty((T, int(row_stride)), dtype=torch.uint8, device=mask.device)
    _dev(out, torch.uint8, "dense", T * int(row_stride))
    st = lib.tree_expand_mask(ctypes.byref(bt._c), _ptr(mask), int(mask.shape[1]), int(mode), _ptr(out),
                              int(row_stride), _ptr(err), _stream(stream))
    _check(st, "tree_expand_mask")
    return out


def tree_pack_mask(bt: Batch, dense, mode: int, err, mask_words: Optional[int] = None, out=None, stream=None):
    """Bit-packed int32 [T, W] rows (the attention's input) from a dense uint8 [T, row_stride] mask."""
    torch = _torch()
    lib = load_library()
    T = bt.total_nodes
    if dense.dim() != 2 or dense.shape[0] != T:
        raise ValueError(f"dense must be [T={T}, row_stride]")
    _dev(dense, torch.uint8, "dense")
    _dev(err, torch.int32, "err", bt.batch)
    W = bt.mask_words if mask_words is None else int(mask_words)
    if out is None:
        out = torch.empty((T, W), dtype=torch.int32, device=dense.device)
    _dev(out, torch.int32, "mask", T * W)
    st = lib.tree_pack_mask(ctypes.byref(bt._c), _ptr(dense), int(dense.shape[1]), int(mode), _ptr(out), W,
                            _ptr(err), _stream(stream))
    _check(st, "tree_pack_mask")
    return out


def tree_ddtree_workspace_bytes(requests: int, depths: int, vocab: int, budget: int) -> int:
    return int(load_library().tree_ddtree_workspace_bytes(int(requests), int(depths), int(vocab), int(budget)))


def tree_ddtree_build(draft_logits, budget: int, out: Optional[Dict] = None, workspace=None, stream=None) -> Dict:
    """DDTree draft trees from float32 draft logits [R, L, V]: parents / tokens
    [R, budget] (pop order) and n_nodes [R]."""
    torch = _torch()
    lib = load_library()
    if draft_logits.dim() != 3:
        raise ValueError("draft_logits must be [requests, depths, vocab]")
    _dev(draft_logits, torch.float32, "draft_logits")
    R, L, V = (int(x) for x in draft_logits.shape)
    dev = draft_logits.device
    if out is None:
        out = {"parents": torch.empty((R, budget), dtype=torch.int32, device=dev),
               "tokens": torch.empty((R, budget), dtype=torch.int32, device=dev),
               "n_nodes": torch.empty(R, dtype=torch.int32, device=dev)}
    _dev(out["parents"], torch.int32, "parents", R * budget)
    _dev(out["tokens"], torch.int32, "tokens", R * budget)
    _dev(out["n_nodes"], torch.int32, "n_nodes", R)
    need = tree_ddtree_workspace_bytes(R, L, V, budget)
    if need == 0:
        raise ValueError("unsupported DDTree sizes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _dev(workspace, torch.uint8, "workspace")
    st = lib.tree_ddtree_build(R, L, V, int(budget), _ptr(draft_logits), _ptr(out["parents"]), _ptr(out["tokens"]),
                               _ptr(out["n_nodes"]), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "tree_ddtree_build")
    return out


def tree_merge_sequences(seqs, max_nodes: int, err=None, out: Optional[Dict] = None, stream=None) -> Dict:
    """SpecInfer's merged tree of int32 draft sequences [R, M, L] (negative = ended):
    parents / tokens [R, max_nodes] in level order, n_nodes [R], err [R]."""
    torch = _torch()
    lib = load_library()
    if seqs.dim() != 3:
        raise ValueError("seqs must be [requests, n_seqs, seq_len]")
    _dev(seqs, torch.int32, "seqs")
    R, M, L = (int(x) for x in seqs.shape)
    dev = seqs.device
    if out is None:
        out = {"parents": torch.empty((R, max_nodes), dtype=torch.int32, device=dev),
               "tokens": torch.empty((R, max_nodes), dtype=torch.int32, device=dev),
               "n_nodes": torch.empty(R, dtype=torch.int32, device=dev)}
    if err is None:
        err = torch.zeros(R, dtype=torch.int32, device=dev)
    out["err"] = _dev(err, torch.int32, "err", R)
    for k in ("parents", "tokens"):
        _dev(out[k], torch.int32, k, R * max_nodes)
    _dev(out["n_nodes"], torch.int32, "n_nodes", R)
    st = lib.tree_merge_sequences(R, M, L, _ptr(seqs), int(max_nodes), _ptr(out["parents"]), _ptr(out["tokens"]),
                                  _ptr(out["n_nodes"]), _ptr(err), _stream(stream))
    _check(st, "tree_merge_sequences")
    return out


def tree_eagle_grow(root_tokens, root_conf, child_tokens, child_conf, budget: int, out: Optional[Dict] = None,
                    stream=None) -> Dict:
    """EAGLE's layer-by-layer tree: root_tokens / root_conf [R, k], child_tokens /
    child_conf [R, L-1, k, k] -> parents / tokens [R, budget], n_nodes [R]."""
    torch = _torch()
    lib = load_library()
    if root_tokens.dim() != 2 or child_tokens.dim() != 4:
        raise ValueError("root_tokens must be [R, k] and child_tokens [R, L-1, k, k]")
    R, k = (int(x) for x in root_tokens.shape)
    L = int(child_tokens.shape[1]) + 1
    if tuple(child_tokens.shape) != (R, L - 1, k, k) or tuple(child_conf.shape) != tuple(child_tokens.shape):
        raise ValueError("child_tokens and child_conf must be [R, L-1, k, k]")
    _dev(root_tokens, torch.int32, "root_tokens")
    _dev(root_conf, torch.float32, "root_conf", R * k)
    _dev(child_tokens, torch.int32, "child_tokens")
    _dev(child_conf, torch.float32, "child_conf")
    dev = root_tokens.device
    if out is None:
        out = {"parents": torch.empty((R, budget), dtype=torch.int32, device=dev),
               "tokens": torch.empty((R, budget), dtype=torch.int32, device=dev),
               "n_nodes": torch.empty(R, dtype=torch.int32, device=dev)}
    for key in ("parents", "tokens"):
        _dev(out[key], torch.int32, key, R * budget)
    _dev(out["n_nodes"], torch.int32, "n_nodes", R)
    st = lib.tree_eagle_grow(R, k, L, _ptr(root_tokens), _ptr(root_conf), _ptr(child_tokens), _ptr(child_conf),
                             int(budget), _ptr(out["parents"]), _ptr(out["tokens"]), _ptr(out["n_nodes"]),
                             _stream(stream))
    _check(st, "tree_eagle_grow")
    return out
