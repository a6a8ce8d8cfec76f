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
#include "act_tables.h"
extern "C" void enc(const float* t, long n, unsigned char* o) {
    for (long i = 0; i < n; ++i) o[i] = (unsigned char)fp8mm::f32_to_e4m3_sat(t[i]);
}
extern "C" void bf(const float* t, long n, unsigned short* o) {
    for (long i = 0; i < n; ++i) o[i] = (unsigned short)fp8mm::f32_to_bf16_rne(t[i]);
}
extern "C" long bf_sel_mismatches_all(void) {
    long bad = 0;
    for (unsigned long long i = 0; i < (1ull << 32); ++i) {
        const unsigned u = (unsigned)i;
        float f;
        __builtin_memcpy(&f, &u, 4);
        bad += fp8mm::f32_to_bf16_rne_sel(f) != fp8mm::f32_to_bf16_rne(f);
    }
    return bad;
}
static constexpr fp8mm::SiluBandTable g_tab = fp8mm::make_silu_band_table();
static const float* g_stab = g_tab.t;
extern "C" int silu_lut_build(void) { return fp8mm::kSiluTableSize; }
extern "C" void silu_both(const unsigned short* b, long n, float* from_lut, float* direct) {
    for (long i = 0; i < n; ++i) {
        from_lut[i] = fp8mm::silu_from_table(b[i], g_stab);
        direct[i] = fp8mm::silu_f64(fp8mm::bf16_to_f32(b[i]));
    }
}
static unsigned char g_codes[65536];
extern "C" int code_table_build(float s) {
    if (!fp8mm::code_table_ok(s)) return -1;
    const unsigned lo = fp8mm::code_band_lo(s);
    for (unsigned h = 0; h < 65536; ++h) g_codes[h] = (unsigned char)fp8mm::code_table_entry(h, lo, s);
    return (int)lo;
}
extern "C" void codes_from_table(const unsigned short* h, long n, unsigned char* o) {
    for (long i = 0; i < n; ++i) o[i] = g_codes[h[i]];
}
// The fused GEMM's encoder on the host: quant_quotient (multiply and fused
// multiply-add instead of a division), the software encoder standing in for
// the hardware conversion (the same codes on [0, 464], the quotients' range),
// the NaN mask and the sign byte; against code_table_entry for every bf16.
extern "C" long quotient_code_mismatches(float s) {
    if (!fp8mm::code_table_ok(s)) return -1;
    const unsigned lo = fp8mm::code_band_lo(s);
    const float rcp = 1.0f / s, sat = 448.0f * s;
    long bad = 0;
    for (unsigned h = 0; h < 65536; ++h) {
        const unsigned bits = (h << 16) & 0x7fffffffu;
        float a;
        __builtin_memcpy(&a, &bits, 4);
        const float q = fp8mm::quant_quotient(a, s, rcp, sat);
        const unsigned c = (fp8mm::f32_to_e4m3_sat(q) & 0x7fu) | ((h >> 8) & 0x80u);
        bad += c != fp8mm::code_table_entry(h, lo, s);
    }
    return bad;
}
extern "C" long band_code_mismatches(void) {
    long bad = 0;
    for (unsigned u = 0x39800000u; u < 0x44800000u; ++u) {     // every fp32 in [2^-12, 2^10)
        float f;
        __builtin_memcpy(&f, &u, 4);
        bad += fp8mm::e4m3_code_band(f) != fp8mm::f32_to_e4m3_sat(f);
    }
    return bad;
}
extern "C" long band_table_mismatches(float s, int nthreads) {
    if (!fp8mm::code_table_ok(s)) return -1;
    const unsigned lo = fp8mm::code_band_lo(s);
    static unsigned char tab[fp8mm::kCodeBand + 2];
    for (int t = 0; t < nthreads; ++t) fp8mm::fill_band_table(tab, lo, s, t, nthreads);
    long bad = 0;
    for (unsigned e = 0; e < fp8mm::kCodeBand; ++e) bad += tab[1 + e] != fp8mm::code_table_entry(lo + e, lo, s);
    return bad;
}
extern "C" void silu_mul_codes(const unsigned short* g, const unsigned short* u, long n, float s, unsigned char* o) {
    code_table_build(s);
    for (long i = 0; i < n; ++i)
        o[i] = g_codes[fp8mm::f32_to_bf16_cvt(fp8mm::silu_from_table(g[i], g_stab) * fp8mm::bf16_to_f32(u[i]))];
}
// The table kernel's per-piece logic (n a multiple of 8): the common-case
// codes where silu_mul_codes8_fast accepts the piece (fast[i / 8] = 1), else
// silu_mul_codes8_exact.
extern "C" void silu_mul_codes_pieces(const unsigned short* g, const unsigned short* u, long n, float s,
                                      unsigned char* o, unsigned char* fast) {
    static unsigned char tab[fp8mm::kBandTableBytes];
    const unsigned lo = fp8mm::code_band_lo(s);
    for (int t = 0; t < 1024; ++t) fp8mm::fill_band_table(tab, lo, s, t, 1024);
    tab[0] = 0u, tab[fp8mm::kCodeBand + 1] = 0x7eu, tab[fp8mm::kCodeBand + 2] = 0x7eu;
    for (long i = 0; i < n; i += 8) {
        uint32_t gw[4], uw[4];
        for (int k = 0; k < 4; ++k) {
            gw[k] = g[i + 2 * k] | ((uint32_t)g[i + 2 * k + 1] << 16);
            uw[k] = u[i + 2 * k] | ((uint32_t)u[i + 2 * k + 1] << 16);
        }
        float t[8];
        uint2 c;
        fast[i / 8] = fp8mm::silu_mul_codes8_fast(gw, uw, g_stab, tab, lo - 1u, t, c);
        if (!fast[i / 8]) c = fp8mm::silu_mul_codes8_exact(gw, uw, t, tab, lo - 1u);
        for (int k = 0; k < 4; ++k) o[i + k] = (c.x >> (8 * k)) & 0xffu, o[i + 4 + k] = (c.y >> (8 * k)) & 0xffu;
    }
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
    lib.silu_both.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p]
    lib.silu_mul_codes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long, ctypes.c_float, ctypes.c_void_p]
    lib.silu_mul_codes_pieces.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long, ctypes.c_float,
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.bf_sel_mismatches_all.restype = ctypes.c_long
    lib.band_code_mismatches.restype = ctypes.c_long
    lib.quotient_code_mismatches.argtypes = [ctypes.c_float]
    lib.quotient_code_mismatches.restype = ctypes.c_long
    lib.band_table_mismatches.argtypes = [ctypes.c_float, ctypes.c_int]
    lib.band_table_mismatches.restype = ctypes.c_long
    lib.code_table_build.argtypes = [ctypes.c_float]
    lib.codes_from_table.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p]
    lib.silu_lut_build()
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


@pytest.mark.parametrize("s", [1.0, 0.37, 1.0 / 448.0, 0.0137, 3.0e-5, 1234.5, 2.0 ** -100, 2.0 ** 100,
                               float(np.nextafter(np.float32(2.0 ** -100), np.float32(1))), 1.0e-30, 7.0e29])
def test_code_table_equals_plain_quant_for_every_bf16(dev, s):
    """The GPU's E4M3 code table (divisions only for one band of bf16
    magnitudes, signed zero below it, saturation above) against the oracle's
    static quant of all 65,536 bf16 patterns: bit-exact, NaN signs included."""
    s = np.float32(s)
    assert dev.code_table_build(s) > 0
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = np.empty(65536, np.uint8)
    dev.codes_from_table(h.ctypes.data, h.size, got.ctypes.data)
    want = oracle.quant_act(h[None], s)[0]
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(hex(h[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_code_table_refuses_scales_outside_its_range(dev):
    for s in (2.0 ** -101, 2.0 ** 101, 1e-40):
        assert dev.code_table_build(np.float32(s)) == -1


def bf16_value(b):
    return float(np.array([b << 16], np.uint32).view(np.float32)[0])


def test_silu_table_equals_direct_fp64_for_every_bf16_gate(dev):
    """The GPU's SiLU table, s = fma(g, m, t) with (m, t) from the table, gives
    the same fp32 bits as the direct fp64 evaluation for all 65,536 gates."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lut, direct = np.empty(65536, np.float32), np.empty(65536, np.float32)
    dev.silu_both(b.ctypes.data, b.size, lut.ctypes.data, direct.ctypes.data)
    nan = np.isnan(direct)
    assert np.array_equal(nan, np.isnan(lut))
    assert np.array_equal(lut.view(np.uint32)[~nan], direct.view(np.uint32)[~nan])
    # the closed-form regions are exercised: -0 from -109 down, g itself from 109
    # on, g/2 below 2^-25 (signed zeros kept)
    assert lut[0xC2DA].view(np.uint32) == 0x80000000 and lut[0x42DA] == np.float32(109.0)
    assert np.isnan(lut[0xFF80]) and lut[0x7F80] == np.inf
    assert lut[0x8000].view(np.uint32) == 0x80000000 and lut[0x0000].view(np.uint32) == 0
    assert lut[0x32FF] == np.float32(bf16_value(0x32FF) / 2)


def test_silu_mul_quant_device_logic_matches_oracle(dev):
    """The table-based SiLU*mul -> E4M3 of the GPU, run on the host, against the
    oracle's fused function for every gate pattern times unit, random and every
    up pattern (NaN codes compared up to their sign)."""
    every = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rnd = np.random.Generator(np.random.PCG64(11)).standard_normal(65536).astype(np.float32)
    rnd_b = (rnd.view(np.uint32) >> 16).astype(np.uint16)        # truncation is fine: any bf16 pattern will do
    gate = np.concatenate([every, every, every, rnd_b])
    up = np.concatenate([np.full(65536, 0x3F80, np.uint16), rnd_b, every[::-1].copy(), every])
    for s in (1.0, 0.37, 1.0 / 448.0):
        got = np.empty(gate.size, np.uint8)
        dev.silu_mul_codes(gate.ctypes.data, up.ctypes.data, gate.size, s, got.ctypes.data)
        want = oracle.silu_mul_quant(gate[None], up[None], np.float32(s))[0]
        nan_w = (want & 0x7F) == 0x7F
        assert np.array_equal(nan_w, (got & 0x7F) == 0x7F)
        bad = np.flatnonzero((got != want) & ~nan_w)
        assert bad.size == 0, [(hex(gate[i]), hex(up[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_silu_mul_piece_logic_matches_oracle(dev):
    """The table kernel's per-piece logic (the common-case fast path with its
    fallback to the exact path), run on the host, against the oracle: every
    gate pattern times unit, random and every up pattern, and N(0, 2) gates
    and ups, where every piece must take the fast path.  Pieces holding a gate
    outside the SiLU band or a NaN product must not."""
    every = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.Generator(np.random.PCG64(12))
    rnd_b = (rng.standard_normal(65536).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nrm_g = ((rng.standard_normal(1 << 16) * 2).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nrm_u = ((rng.standard_normal(1 << 16) * 2).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    gate = np.concatenate([every, every, every, rnd_b, nrm_g])
    up = np.concatenate([np.full(65536, 0x3F80, np.uint16), rnd_b, every[::-1].copy(), every, nrm_u])
    for s in (1.0, 0.37, 1.0 / 448.0):
        got = np.empty(gate.size, np.uint8)
        fast = np.empty(gate.size // 8, np.uint8)
        dev.silu_mul_codes_pieces(gate.ctypes.data, up.ctypes.data, gate.size, s, got.ctypes.data, fast.ctypes.data)
        want = oracle.silu_mul_quant(gate[None], up[None], np.float32(s))[0]
        nan_w = (want & 0x7F) == 0x7F
        assert np.array_equal(nan_w, (got & 0x7F) == 0x7F)
        bad = np.flatnonzero((got != want) & ~nan_w)
        assert bad.size == 0, [(hex(gate[i]), hex(up[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]
        # which pieces the fast path may take: every gate magnitude in the band, no NaN product
        mag = (gate & 0x7FFF).reshape(-1, 8)
        in_band = ((mag >= 0x3300) & (mag < 0x42DA)).all(axis=1)
        no_nan = ~nan_w.reshape(-1, 8).any(axis=1)
        assert np.array_equal(fast.astype(bool), in_band & no_nan)
        assert fast[-(1 << 13):].all()                  # the N(0, 2) pieces


def test_branch_free_bf16_rounding_equals_the_plain_one_on_every_fp32(dev):
    """f32_to_bf16_rne_sel (the select form the table kernel uses) against
    f32_to_bf16_rne on all 2^32 fp32 patterns."""
    assert dev.bf_sel_mismatches_all() == 0


def test_band_table_fill_equals_per_entry_division(dev):
    """fill_band_table (one division per mantissa, scaled by powers of two
    across the 20 binades, the work split over nthreads) against
    code_table_entry (one division per entry) over 3000 log-uniform scales in
    [2^-100, 2^100], both edges and the decode / prefill scales, for the
    thread counts the kernels launch with."""
    g = np.random.Generator(np.random.PCG64(1234))
    scales = np.exp2(g.uniform(-100.0, 100.0, 3000)).astype(np.float32)
    scales = np.concatenate([scales, np.float32([2.0 ** -100, 2.0 ** 100, 1.0, 1.0 / 448.0, 0.0137,
                                                 np.nextafter(np.float32(2.0 ** -100), np.float32(1.0)),
                                                 np.nextafter(np.float32(2.0 ** 100), np.float32(0.0))])])
    for n in (128, 256, 512, 640, 768, 1024):
        for s in scales:
            assert dev.band_table_mismatches(float(s), n) == 0, (float(s), n)
    assert dev.band_table_mismatches(2.0 ** -101, 128) == -1


def test_branch_free_band_encoder_equals_the_plain_one(dev):
    """e4m3_code_band (the band table fill's encoder: a select between the
    subnormal grid and the rounded mantissa) against f32_to_e4m3_sat on every
    positive fp32 in [2^-12, 2^10), the range of a band table's quotients."""
    assert dev.band_code_mismatches() == 0


def test_division_free_quotient_codes_equal_the_plain_quant(dev):
    """The fused quant + GEMM's encoder (quotient from the reciprocal and two
    fused multiply-adds, magnitude clamped at 448 s, NaN kept by the mask,
    sign from the bf16 bit) against the per-entry division, for every bf16
    pattern, over 1500 log-uniform scales in [2^-100, 2^100], scales with
    random low mantissa bits, both edges and the decode / prefill scales."""
    g = np.random.Generator(np.random.PCG64(77))
    scales = np.exp2(g.uniform(-100.0, 100.0, 1000)).astype(np.float32)
    jitter = (scales.view(np.uint32) ^ g.integers(0, 1 << 12, scales.size, dtype=np.uint32)).view(np.float32)
    scales = np.concatenate([scales, jitter[:500], np.float32([2.0 ** -100, 2.0 ** 100, 1.0, 1.0 / 448.0, 0.0137,
                                                               3.0, 1.0 / 7.0, 448.0])])
    scales = scales[(scales >= 2.0 ** -100) & (scales <= 2.0 ** 100)]
    bad = [(float(s), n) for s in scales if (n := dev.quotient_code_mismatches(float(s))) != 0]
    assert not bad, bad[:5]
