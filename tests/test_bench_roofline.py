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
