"""Move a synthetic Workload onto a torch device (input plumbing only)."""

import numpy as np
import torch


def _bf16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def _i32(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def to_device(wl, device="cuda") -> dict:
    """Device tensors of a Workload: bf16 as torch.bfloat16, ints as int32."""
    d = dict(
        parents=_i32(wl.parents, device), tokens=_i32(wl.tokens, device),
        node_offsets=_i32(wl.node_offsets, device), ctx_lens=_i32(wl.ctx_lens, device),
        q=_bf16(wl.q, device), k_new=_bf16(wl.k_new, device), v_new=_bf16(wl.v_new, device),
        k_cache=_bf16(wl.k_cache, device), v_cache=_bf16(wl.v_cache, device),
        block_table=None if wl.block_table is None else _i32(wl.block_table, device),
    )
    if wl.logits_dtype == "fp32":
        d["logits"] = torch.from_numpy(np.ascontiguousarray(wl.logits)).to(device)
    else:
        d["logits"] = _bf16(wl.logits, device)
    return d


def bits_of(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
