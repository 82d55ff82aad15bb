"""Helpers for the GPU tests: device checks, host copies, cache regions."""

import os
import sys

import numpy as np
import pytest

import token_tree_attention_amd as tta


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no ROCm device visible: the gpu-marked tests need an MI355X")
    if not os.path.exists(tta.library_path()):
        pytest.fail("libtreeverify.so is not built")
    tta.load_library()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def bits(t) -> np.ndarray:
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def region_bits(d, wl, b, start, count, which="k", table=None):
    """[Hkv, count, D] bf16 bits of slots start..start+count-1 of request b on the device cache."""
    import torch
    cache = d["k_cache"] if which == "k" else d["v_cache"]
    if wl.layout == "contiguous":
        return bits(cache[b, :, start:start + count])
    tab = d["block_table"] if table is None else table
    slots = torch.arange(start, start + count, device=cache.device)
    blk = tab[b, slots // 16].long()
    t = cache[blk, :, slots % 16]          # [count, Hkv, D]
    return bits(t.permute(1, 0, 2))
