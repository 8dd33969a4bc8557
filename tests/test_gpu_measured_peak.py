"""The measured ceilings the benchmark reports beside the datasheet peaks: a
pure MFMA loop and a 1 GiB device copy must land between a loose floor and
the datasheet figure (a probe that measured more than the datasheet, or far
less, would make every 'fraction of measured peak' meaningless)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_mfma_loop_is_below_the_datasheet_and_near_it(dtype):
    import torch
    import bench
    dev = torch.device("cuda:0")
    mp = bench.measured_peak(dev, "mfma", dtype)
    assert mp is not None and mp["unit"] == "TFLOP/s"
    peak = bench.PEAK[f"mfma_{dtype}"]
    print(f"{dtype}: MFMA loop {mp['peak']} TFLOP/s, {100 * mp['peak'] / peak:.1f}% of the datasheet {peak}")
    assert 0.5 * peak < mp["peak"] <= 1.02 * peak


def test_device_copy_is_below_the_datasheet_bandwidth():
    import torch
    import bench
    mp = bench.measured_peak(torch.device("cuda:0"), "hbm", "bf16")
    assert mp is not None and mp["unit"] == "GB/s"
    print(f"copy: {mp['peak']} GB/s, {100 * mp['peak'] / bench.PEAK['hbm']:.1f}% of the datasheet")
    assert 0.3 * bench.PEAK["hbm"] < mp["peak"] <= 1.02 * bench.PEAK["hbm"]
