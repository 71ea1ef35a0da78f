"""The measured-peak microbenchmarks (libkda_peaks.so) compute what they claim,
so the peaks the benchmark reports come from real work."""
from __future__ import annotations

import ctypes
import os

import pytest

from gpu_util import need_gpu

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gated_delta_rule_28_amd",
                   "libkda_peaks.so")


def test_peak_kernels_compute():
    torch, _ = need_gpu()
    L = ctypes.CDLL(LIB)
    L.kda_peak_fmw.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    L.kda_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    x = torch.randn(4 * 16384, dtype=torch.float32, device="cuda")  # four 64 KiB blocks
    want = x * 1.0000001 + 1e-7
    assert L.kda_peak_fmw(ctypes.c_void_p(x.data_ptr()), x.numel() * 4, 32 << 10, stream) == 0
    torch.cuda.synchronize()
    assert torch.allclose(x, want, rtol=1e-6, atol=1e-6)
    L.kda_peak_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    assert L.kda_peak_stream(ctypes.c_void_p(x.data_ptr()), x.numel() * 4, 1, stream) == 0  # write zeros
    torch.cuda.synchronize()
    assert int((x != 0).sum()) == 0
    assert L.kda_peak_stream(ctypes.c_void_p(x.data_ptr()), x.numel() * 4, 0, stream) == 0  # read: no store
    torch.cuda.synchronize()
    assert int((x != 0).sum()) == 0
    L.kda_peak_rw.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    for threads in (256, 512, 1024):
        src = torch.randn(4 * 16384, dtype=torch.float32, device="cuda")
        dst = torch.zeros_like(src)
        assert L.kda_peak_rw(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), src.numel() * 4,
                             threads, stream) == 0  # copy
        torch.cuda.synchronize()
        assert torch.equal(dst, src)
        want = src * 1.0000001 + 1e-7
        assert L.kda_peak_rw(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(src.data_ptr()), src.numel() * 4,
                             threads, stream) == 0  # in place
        torch.cuda.synchronize()
        assert torch.allclose(src, want, rtol=1e-6, atol=1e-6)
    # rejected before any launch: bad workgroup size, partial overlap, ragged size
    assert L.kda_peak_rw(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), 65536, 384, stream) == -2
    assert L.kda_peak_rw(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(src.data_ptr() + 65536), 131072, 256,
                         stream) == -2
    assert L.kda_peak_rw(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), 1000, 256, stream) == -2
    out = torch.zeros(8 * 256, dtype=torch.float32, device="cuda")
    for chains in (4, 8):
        out.zero_()
        assert L.kda_peak_mfma(ctypes.c_void_p(out.data_ptr()), 8, 10, chains, stream) == 0
        torch.cuda.synchronize()
        assert torch.isfinite(out).all() and out.abs().sum() > 0
