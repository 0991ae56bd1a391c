"""Reference-rate kernels (measurement support): they run, reject bad sizes, and
report plausible rates for one MI355X (below the published peaks, far above
what a broken launch would give)."""

import ctypes

import pytest
import torch

from lossless_rejection_sampling_amd import dspark as ds

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def _time(fn):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3


def test_stream_read_rate():
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    gbs = buf.numel() / _time(lambda: ds.dspark_peak_stream_read(buf, sink)) / 1e9
    print(f"stream read {gbs:.0f} GB/s")
    assert 1000 < gbs < 8000 * 1.2   # the published HBM peak is 8 TB/s (the Infinity Cache may add a little)
    assert sink.item() == 0


def test_mfma_rate():
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    blocks, iters = 1024, 1024
    t = _time(lambda: ds.dspark_peak_mfma_bf16(blocks, iters, sink))
    tf = blocks * 4 * iters * 4 * 32768 / t / 1e12
    print(f"bf16 MFMA {tf:.0f} TFLOP/s")
    assert 200 < tf < 2500 * 1.05   # dense bf16 peak 2.5 PFLOP/s
    assert sink.item() == 0


def test_bad_sizes_rejected():
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    buf = torch.ones(1024, dtype=torch.uint8, device="cuda")
    L = ds.lib()
    assert L.dspark_peak_stream_read(ctypes.c_void_p(buf.data_ptr()), 1000, ctypes.c_void_p(sink.data_ptr()),
                                     None) == ds.DSPARK_EINVAL
    assert L.dspark_peak_stream_read(ctypes.c_void_p(buf.data_ptr()), 0, ctypes.c_void_p(sink.data_ptr()),
                                     None) == ds.DSPARK_EINVAL
    assert L.dspark_peak_mfma_bf16(0, 10, ctypes.c_void_p(sink.data_ptr()), None) == ds.DSPARK_EINVAL
    assert L.dspark_peak_mfma_bf16(4, 0, ctypes.c_void_p(sink.data_ptr()), None) == ds.DSPARK_EINVAL
