"""bench.py's roofline entry: the bound follows the arithmetic intensity."""

import bench


class _Wl:
    name = "no_such_workload"  # no stored counter summary: traffic is None


def test_low_intensity_is_hbm_bound():
    # 100 flop per byte is below the ridge 2500e12 / 8000e9 = 312.5
    r = bench.roofline_entry(_Wl(), attn_bytes=1e9, flops=1e11, attn_ms=1.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["achieved"] - 1000.0) < 1e-9          # 1 GB in 1 ms
    assert abs(r["frac"] - 1000.0 / bench.HBM_PEAK_GBS) < 1e-12
    assert r["traffic"] is None


def test_high_intensity_is_mfma_bound():
    # 1000 flop per byte is above the ridge
    r = bench.roofline_entry(_Wl(), attn_bytes=1e9, flops=1e12, attn_ms=1.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["achieved"] - 1000.0) < 1e-9          # 1 TFLOP in 1 ms
    assert abs(r["frac"] - 1000.0 / bench.BF16_PEAK_TFLOPS) < 1e-12
    assert abs(r["hbm_frac"] - 1000.0 / bench.HBM_PEAK_GBS) < 1e-12


class _Chain:
    """One request: a 3-node chain (depths 0, 1, 2) over a 5-token context."""
    import numpy as _np
    batch, n_max, total_nodes = 1, 3, 3
    head_dim, n_heads, n_kv_heads = 64, 4, 2
    node_offsets = _np.array([0, 3])
    ctx_lens = _np.array([5])
    parents = _np.array([-1, 0, 1])
    logits_dtype, vocab = "fp32", 10


def test_algorithmic_bytes_and_flops_closed_form():
    attn_bytes, flops, accept_bytes = bench.algorithmic(_Chain())
    D, Hq, Hkv, n, ctx, W = 64, 4, 2, 3, 5, 1
    assert attn_bytes == ctx * Hkv * D * 4 + n * Hq * D * 4 + n * Hkv * D * 8 + n * W * 4 + n * 4
    # each node attends to the context plus its depth + 1 tree keys
    assert flops == 4 * D * Hq * ((ctx + 1) + (ctx + 2) + (ctx + 3))
    assert accept_bytes == (n + 1) * 10 * 4
