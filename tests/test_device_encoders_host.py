"""The HIP path's number-format helpers, compiled for the host (CPU only).

fp8_w8a8_scaled_amd/csrc/device_common.h holds the GPU's own saturating RNE
E4M3 encoder (integer bit manipulation) and bf16 rounding, written separately
from the oracle's (binary search / frexp).  Both are __host__ __device__, so
this test builds them into a small host library with hipcc and compares them
with the oracle on random fp32 values, on every E4M3 rounding midpoint and its
fp32 neighbours, and on the special values.
"""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = r"""
#include "device_common.h"
extern "C" void enc(const float* t, long n, unsigned char* o) {
    for (long i = 0; i < n; ++i) o[i] = (unsigned char)fp8mm::f32_to_e4m3_sat(t[i]);
}
extern "C" void bf(const float* t, long n, unsigned short* o) {
    for (long i = 0; i < n; ++i) o[i] = (unsigned short)fp8mm::f32_to_bf16_rne(t[i]);
}
"""


@pytest.fixture(scope="module")
def dev():
    d = tempfile.mkdtemp()
    src = os.path.join(d, "drv.hip")
    so = os.path.join(d, "libdrv.so")
    with open(src, "w") as f:
        f.write(DRIVER)
    subprocess.check_call(["/opt/rocm/bin/hipcc", "--cuda-host-only", "-O2", "-fPIC", "-shared",
                           "-I", os.path.join(ROOT, "fp8_w8a8_scaled_amd", "csrc"), src, "-o", so],
                          stderr=subprocess.DEVNULL)
    lib = ctypes.CDLL(so)
    lib.enc.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p]
    lib.bf.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p]
    return lib


def _enc(lib, t):
    t = np.ascontiguousarray(t, np.float32)
    o = np.empty(t.size, np.uint8)
    lib.enc(t.ctypes.data, t.size, o.ctypes.data)
    return o


def _test_values():
    g = np.random.Generator(np.random.PCG64(2024))
    rand_bits = g.integers(0, 2 ** 32, 1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    # dense sampling of the interesting exponent range [2^-12, 2^10)
    e = g.integers(-12, 10, 1_000_000)
    m = g.random(1_000_000) + 1.0
    s = np.where(g.random(1_000_000) < 0.5, -1.0, 1.0)
    dense = (s * m * 2.0 ** e).astype(np.float32)
    # every midpoint between adjacent E4M3 magnitudes, and its fp32 neighbours
    tab = oracle.e4m3_table()[:0x7F]
    mids = ((tab[:-1] + tab[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                           tab.astype(np.float32), np.float32(464.0)[None], np.float32(448.0 + 1 / 64)[None]])
    near = np.concatenate([near, -near])
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan, 3.0e38, -3.0e38, 1e-45, -1e-45,
                        2.0 ** -10, -(2.0 ** -10), 2.0 ** -6, 2.0 ** -7 * 1.9375], np.float32)
    return np.concatenate([rand_bits, dense, near, special])


def test_gpu_e4m3_encoder_matches_oracle(dev):
    t = _test_values()
    got = _enc(dev, t)
    want = oracle.e4m3_encode(t)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(t[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_gpu_bf16_rounding_matches_oracle(dev):
    g = np.random.Generator(np.random.PCG64(77))
    f = g.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    f = f[(f & 0x7FFFFFFF) <= 0x7F800000].view(np.float32)        # NaN payloads are canonicalized
    ties = (np.arange(1, 50000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    f = np.concatenate([f, ties, -ties])
    o = np.empty(f.size, np.uint16)
    dev.bf(np.ascontiguousarray(f).ctypes.data, f.size, o.ctypes.data)
    want = np.array([oracle.f32_to_bf16(v) for v in f], np.uint16)
    assert np.array_equal(o, want)
