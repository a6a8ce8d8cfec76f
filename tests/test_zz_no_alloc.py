"""The allocation-free calibration entry point, fp8_act_scale_noalloc, through
the raw C ABI: bitwise the s_act of fp8_act_scale (the workspace variant that
shares its kernels) on two calls in a row, the second with a smaller input, on
both the plain path (per-workgroup partials) and the RMSNorm path (one partial
per row); and the size limit of its static scratch refused before any launch."""
import ctypes

import numpy as np
import pytest

import workloads as wl
from helpers import bf16_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import fp8_w8a8_scaled_amd as m
    return m


def _raw_noalloc(fp8, x, gamma, eps, s_out):
    import torch
    L = fp8.raw_lib()
    f = L.fp8_act_scale_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    M, K = x.shape
    st = f(ctypes.c_void_p(x.data_ptr()), x.stride(0),
           None if gamma is None else ctypes.c_void_p(gamma.data_ptr()), float(eps), M, K,
           ctypes.c_void_p(s_out.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def _bits(t):
    return np.float32(t.item()).view(np.uint32)


@pytest.mark.parametrize("rms", [False, True])
def test_noalloc_matches_workspace_variant_twice(fp8, rms):
    import torch
    # first call: the decode-MLP input at M = 32 (rms) or a 6576 x 5120 prefill-sized input (plain: 4096 partials)
    shapes = [(32, 5120), (3, 5120)] if rms else [(6576, 5120), (5, 2048)]
    g = bf16_dev(wl.gamma_bf16(3, 5120)) if rms else None
    s_out = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    for i, (M, K) in enumerate(shapes):
        x = bf16_dev(wl.activation_bf16(3 if rms else 5, M, K, outliers=True, tensor=wl.T_X + 40 + i))
        gm = g[:K] if rms else None
        want = fp8.act_scale(x, gm, wl.EPS)
        s_out.fill_(-1.0)
        assert _raw_noalloc(fp8, x, gm, wl.EPS, s_out) == fp8.OK
        torch.cuda.synchronize()
        assert _bits(s_out) == _bits(want), (i, M, K, s_out.item(), want.item())
        # the binding's wrapper of the same entry point
        assert _bits(fp8.act_scale_noalloc(x, gm, wl.EPS)) == _bits(want)


def test_noalloc_refuses_inputs_past_its_scratch(fp8):
    import torch
    M, K = fp8.NOALLOC_SCRATCH_FLOATS + 1, 16               # the RMSNorm path needs one partial per row
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(K, dtype=torch.bfloat16, device="cuda")
    s_out = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    assert _raw_noalloc(fp8, x, g, wl.EPS, s_out) == fp8.ESCRATCH
    torch.cuda.synchronize()
    assert s_out.item() == -1.0                              # nothing was launched
    # the plain path never needs more than 4096 partials: the same tensor is fine
    assert _raw_noalloc(fp8, x, None, 0.0, s_out) == fp8.OK
    torch.cuda.synchronize()
    assert s_out.item() == 1.0                               # amax 0 -> scale 1
