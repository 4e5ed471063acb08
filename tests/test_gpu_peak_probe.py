"""The bench's matrix-core rate probe on the GPU: the rates it measures are
positive, below MI355X's published dense peaks scaled by the 2:4 factor where it
applies (with 10 % margin, since the peaks assume the nominal clock and a
measurement has noise), and the 2:4 instructions run faster than the dense
ones of the same data type (their dense-equivalent rate is up to 2x)."""

import pytest

pytestmark = pytest.mark.gpu


def test_measured_mfma_rates_are_plausible(gpu):
    import torch
    import bench
    bench._PEAK.clear()
    peak = bench.mfma_peak_measured(torch, iters=200, reps=3, warm_s=0.05)
    bench._PEAK.clear()
    assert peak is not None, "libssg_peak.so missing or failed"
    published = {"dense_f16": 2500.0, "w24_f16": 5000.0, "dense_i8": 5000.0, "w24_i8": 10000.0}
    for k, p in published.items():
        assert 0.1 * p < peak[k] <= 1.1 * p, (k, peak[k])
    assert peak["w24_f16"] > 1.2 * peak["dense_f16"]
    assert peak["w24_i8"] > 1.2 * peak["dense_i8"]
