// act_tables.h -- small per-workgroup tables that replace per-element fp64 and
// IEEE-division work in the activation quant kernels, with results identical
// to the per-element evaluation (host-checked over every bf16 input).
//
// Both tables exist because the quantities are functions of one bf16 value:
// SiLU of a bf16 gate, and the E4M3 code of a bf16 activation h under a fixed
// static scale.  Building them costs a few thousand evaluations per
// workgroup; the per-element path then needs one LDS read each.  Where that
// fill does not pay (few rows per workgroup, or a GEMM's own launch), the code
// comes from the table-free encoder here instead: the exact quotient by
// multiply and fused multiply-add, then the hardware E4M3 conversion.
#pragma once

#include "device_common.h"

namespace fp8mm {

// Two 16-bit lanes of one 32-bit word (a pair of bf16 values): the packed
// 16-bit integer operations of gfx9 (v_pk_sub_u16, v_pk_min_u16, ...).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __host__ __forceinline__ u16x2_t as_u16x2(uint32_t w) { return __builtin_bit_cast(u16x2_t, w); }
__device__ __host__ __forceinline__ uint32_t as_u32(u16x2_t v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __host__ __forceinline__ u16x2_t splat_u16x2(uint32_t v)
{
    return u16x2_t{(unsigned short)v, (unsigned short)v};
}


// SiLU of a gate value, s = fl32( g / (1 + exp(-g)) ) with the expression in
// fp64 (the same reading as the RMSNorm scale: wide arithmetic, one rounding).
__device__ __host__ __forceinline__ float silu_f64(float g)
{
    const double d = (double)g;
    return (float)(d / (1.0 + exp(-d)));
}

// silu_f64 of every bf16 gate as s = fma(g, m, t).  Outside a band of
// magnitudes s is exact in closed form:
//   |g| < 2^-25           s = g / 2  (g^2/4 is below half an fp32 ulp of g/2)
//   g >= 109, +inf, +NaN  s = g      (exp(-g) < 2^-157)
//   g <= -109, -inf, -NaN s = g * 0  (-0: |g| e^g is below half the least fp32
//                                     subnormal; -inf / inf and NaN give NaN)
// so only the band entries silu_f64(g), for magnitudes [2^-25, 109) (bf16
// patterns 0x3300 .. 0x42D9) of both signs, come from a table (t, with m = 0);
// outside it t = -0 and m = 0.5 below the band, 1 above it for g > 0 and 0
// above it for g < 0.  fma(g, 0, t) = t exactly (no band value is zero) and
// fma(g, m, -0) = g * m exactly.
constexpr uint32_t kSiluLo = 0x3300u, kSiluBand = 0x42DAu - 0x3300u;
// Table layout: entry sign * kSiluSignStride + (|g| bits - kSiluLo).  The
// stride is a power of two, so the gate's sign bit moves into the index with
// one shift and mask.
constexpr int kSiluSignStride = 4096;
constexpr int kSiluTableSize = 2 * kSiluSignStride;

// exp(x) for |x| < 128, evaluated by the compiler to build the table below:
// x = k ln2 + r with |r| <= ln2 / 2 (Cody-Waite reduction; the high part of
// ln2 has trailing zero bits, so k ln2_hi is exact), exp(r) from its Taylor
// series to degree 18 by Horner's rule (the truncation error is below 2^-60
// of the result), times 2^k built from its exponent bits.  The host tests
// compare every table entry with silu_f64 (the C library's exp).
constexpr double silu_cx_exp(double x)
{
    constexpr double ln2_hi = 6.93147180369123816490e-01, ln2_lo = 1.90821492927058770002e-10;
    const double kd = x * 1.44269504088896338700e+00;
    const int k = (int)(kd < 0.0 ? kd - 0.5 : kd + 0.5);
    const double r = (x - k * ln2_hi) - k * ln2_lo;
    double c[19] = {};
    c[0] = 1.0;
    for (int n = 1; n < 19; ++n) c[n] = c[n - 1] / n;
    double p = c[18];
    for (int n = 17; n >= 0; --n) p = p * r + c[n];
    return p * __builtin_bit_cast(double, (uint64_t)(1023 + k) << 52);
}

// silu_f64 of a band gate, at compile time.
constexpr float silu_cx(uint32_t b)
{
    const double d = (double)__builtin_bit_cast(float, b << 16);
    return (float)(d / (1.0 + silu_cx_exp(-d)));
}

struct SiluBandTable {
    float t[kSiluTableSize];
};

// The band values of both signs (entries past the band in each half are 0 and
// never read).
constexpr SiluBandTable make_silu_band_table()
{
    SiluBandTable tab{};
    for (int sg = 0; sg < 2; ++sg)
        for (int j = 0; j < (int)kSiluBand; ++j)
            tab.t[sg * kSiluSignStride + j] = silu_cx(((uint32_t)sg << 15) | (kSiluLo + (uint32_t)j));
    return tab;
}

// Table index of gate bits b (clamped into the band; out-of-band gates do not
// use the value read there).
__device__ __host__ __forceinline__ uint32_t silu_table_index(uint32_t b)
{
    const int d = (int)(b & 0x7fffu) - (int)kSiluLo;
    const int k = d < 0 ? 0 : (d >= (int)kSiluBand ? (int)kSiluBand - 1 : d);   // a med3
    return (uint32_t)k + (b >> 15) * (uint32_t)kSiluSignStride;
}

__device__ __host__ __forceinline__ float silu_finish(uint32_t b, float t_band)
{
    const int d = (int)(b & 0x7fffu) - (int)kSiluLo;
    const bool below = d < 0, above = d >= (int)kSiluBand;
    const float m = below ? 0.5f : (above ? ((b >> 15) ? 0.0f : 1.0f) : 0.0f);
    const float t = below || above ? -0.0f : t_band;
    return __builtin_fmaf(bf16_to_f32(b), m, t);
}

__device__ __host__ __forceinline__ float silu_from_table(uint32_t b, const float* tab)
{
    return silu_finish(b, tab[silu_table_index(b)]);
}

// One E4M3 code of the bf16-valued h / s; a NaN h is encoded with its own sign
// (it is not divided: the sign of a NaN out of a division is not fixed).
__device__ __host__ __forceinline__ uint32_t quant_value(float h, float s_act)
{
    return f32_to_e4m3_sat(h != h ? h : h / s_act);
}

// E4M3 code of h / s_act for every bf16 pattern h: a 65,536-byte table.  Only
// the 2 x 2560 patterns of one band of magnitudes need the division: with lo
// the smallest bf16 magnitude >= s * 2^-11, |h| < lo gives |h/s| < 2^-11, a
// signed zero, and |h| >= 2^20 lo (pattern lo + 2560) gives |h/s| >= 512,
// saturated (inf too); NaN -> 0x7F | sign.  Valid for 2^-100 <= s <= 2^100
// (lo normal, the band below inf).
constexpr uint32_t kCodeBand = 20u * 128u;

__device__ __host__ __forceinline__ bool code_table_ok(float s_act)
{
    return s_act >= 0x1p-100f && s_act <= 0x1p100f;
}

__device__ __host__ __forceinline__ uint32_t code_band_lo(float s_act)
{
    const float f = s_act * 0x1p-11f;              // exact for s >= 2^-100
    uint32_t u;
    __builtin_memcpy(&u, &f, 4);
    return (u + 0xffffu) >> 16;                    // round the magnitude up to bf16
}

// E4M3 code of a positive fp32 q in [2^-12, 2^10) (the quotients of a band
// table), rounded to nearest even and saturating as f32_to_e4m3_sat does, with
// no branches: below 2^-6 the subnormal grid m 2^-9 (q 2^9, an exact scaling,
// rounded to the nearest even integer), else the fp32 mantissa rounded to 3
// bits at bit 20 and rebiased, clamped to the largest finite code.
__device__ __host__ __forceinline__ uint32_t e4m3_code_band(float q)
{
    uint32_t a;
    __builtin_memcpy(&a, &q, 4);
    const uint32_t cn = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
    const uint32_t cs = (uint32_t)__builtin_rintf(q * 512.0f);
    return a < 0x3c800000u ? cs : (cn < 0x7eu ? cn : 0x7eu);
}

__device__ __host__ __forceinline__ uint32_t code_table_entry(uint32_t h, uint32_t lo, float s_act)
{
    const uint32_t a = h & 0x7fffu, sg = (h >> 8) & 0x80u;
    if (a < lo) return sg;
    if (a - lo < kCodeBand) return quant_value(bf16_to_f32(h), s_act);
    return sg | (a > 0x7f80u ? 0x7fu : 0x7eu);
}

// Entries 1 .. kCodeBand of a band table (entry 1 + e: the code of the bf16
// magnitude lo + e; entries 0 and kCodeBand + 1 are the caller's), the share
// of thread `tid` of `nthreads` (a multiple of 128).  Adding 128 to a finite
// bf16 pattern doubles its value, and every quotient here is an fp32 normal
// in [2^-11, 2^9), where the rounded quotient doubles with it: fl32(h 2^k / s)
// = 2^k fl32(h / s).  So each thread divides once, for the mantissa lo +
// tid % 128, and scales that quotient by 2^k for each of its entries (all of
// the same mantissa, since nthreads is a multiple of 128).  Same bytes as
// code_table_entry for 2^-100 <= s_act <= 2^100.
__device__ __host__ __forceinline__ void fill_band_table(uint8_t* tab, uint32_t lo, float s_act, int tid,
                                                         int nthreads)
{
    const float q0 = bf16_to_f32(lo + ((uint32_t)tid & 127u)) / s_act;
    for (int e = tid; e < (int)kCodeBand; e += nthreads) {
        const uint32_t pw = (127u + (uint32_t)(e >> 7)) << 23;   // 2^(e / 128)
        float p2;
        __builtin_memcpy(&p2, &pw, 4);
        tab[1 + e] = (uint8_t)e4m3_code_band(q0 * p2);
    }
}

// The 8 E4M3 codes of 8 bf16 values (one 16-byte piece, words w0..w3, value i
// in bits 16 (i % 2) of word i / 2) under the band table `tab` of the plain
// static quant: entry 0 below the band (a signed zero), entries 1 ..
// kCodeBand the band (filled by fill_band_table), kCodeBand + 1 and + 2 the
// saturated code; a NaN keeps its sign (0x7F | sign).  lo1 = code_band_lo - 1.
__device__ __forceinline__ uint2 quant8_band(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                             const uint8_t* tab, int lo1)
{
    const uint32_t w[4] = {w0, w1, w2, w3};
    uint32_t o[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        uint32_t c = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t a = (w[2 * q + (e >> 1)] >> ((e & 1) * 16)) & 0x7fffu;
            const uint32_t t = tab[min(max((int)a - lo1, 0), (int)kCodeBand + 1)];
            c |= (a > 0x7f80u ? 0x7fu : t) << (8 * e);
        }
        // the four sign bits: bit 15 and bit 31 of each pair of values
        o[q] = c | (__builtin_amdgcn_perm(w[2 * q + 1], w[2 * q], 0x07050301u) & 0x80808080u);
    }
    return make_uint2(o[0], o[1]);
}

// The quotient a / s, a = |h| of a bf16 value, as the plain static quant
// rounds it (fp32, to nearest even), without a division: r = fl32(1 / s), the
// estimate q0 = fl32(a r), its remainder a - q0 s exact through one fused
// multiply-add, and one correction fl32(q0 + rem r).  With r correctly
// rounded and q0 within an ulp of a / s, that correction is the correctly
// rounded quotient (Markstein's theorem on division by fused multiply-add,
// valid while nothing overflows or underflows; exhaustively compared with the
// division for every bf16 a and thousands of scales in [2^-100, 2^100]).
// Magnitudes above F = fl32(448 s) are clamped to F first: their codes
// saturate either way (the quotient of F stays below 464, which rounds to
// 448), and no product overflows.  A NaN a compares false and stays NaN.
// Quotients that underflow are below 2^-26 here (s >= 2^-100), code 0 either way.
__device__ __host__ __forceinline__ float quant_quotient(float a, float s, float r, float F)
{
    const float c = a > F ? F : a;
    const float q0 = c * r;
    return __builtin_fmaf(__builtin_fmaf(-q0, s, c), r, q0);
}

// The 4 E4M3 codes (bytes 0..3) of the bf16 values in words w0 (values 0, 1)
// and w1 (values 2, 3) under the static quant, without a table: quant_quotient
// of each magnitude (rcp = fl32(1 / s), sat = fl32(448 s)), encoded two at a
// time by gfx950's conversion to E4M3 (round to nearest even like the
// software encoder on every magnitude up to 464, which bounds the quotients
// here), the signs from the bf16 sign bits.  A NaN gives a NaN quotient, whose
// code has its 7 low bits set: 0x7F after the mask, with the value's sign;
// inf takes sat and saturates.  Valid for 2^-100 <= s <= 2^100.
__device__ __forceinline__ uint32_t quant4_cvt(uint32_t w0, uint32_t w1, float s, float rcp, float sat)
{
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t h = i < 2 ? w0 : w1;
        q[i] = quant_quotient(__builtin_fabsf(__builtin_bit_cast(float, i & 1 ? h & 0xffff0000u : h << 16)), s, rcp,
                              sat);
    }
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], c, true);
    return ((uint32_t)c & 0x7f7f7f7fu) | (__builtin_amdgcn_perm(w1, w0, 0x07050301u) & 0x80808080u);
}

// quant4_cvt of the two bf16 values of one word: codes in bytes 0 and 1.
__device__ __forceinline__ uint32_t quant2_cvt(uint32_t w, float s, float rcp, float sat)
{
    const float q0 = quant_quotient(__builtin_fabsf(__builtin_bit_cast(float, w << 16)), s, rcp, sat);
    const float q1 = quant_quotient(__builtin_fabsf(__builtin_bit_cast(float, w & 0xffff0000u)), s, rcp, sat);
    const int c = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
    return ((uint32_t)c & 0x7f7fu) | (__builtin_amdgcn_perm(0u, w, 0x0c0c0301u) & 0x8080u);
}

// The band-table codes (without sign) of the two bf16 magnitudes in word h:
// entry clamp(|h| - lo1, 0, kCodeBand + 1) each, as bytes 0 and 1.  For
// values that are not NaN (a NaN takes the saturated entry).
__device__ __host__ __forceinline__ uint32_t band_codes2(uint32_t h, const uint8_t* tab, uint32_t lo1)
{
    const u16x2_t j = __builtin_elementwise_min(__builtin_elementwise_sub_sat(as_u16x2(h & 0x7fff7fffu), splat_u16x2(lo1)),
                                                splat_u16x2(kCodeBand + 1u));
    return (uint32_t)tab[as_u32(j) & 0xffffu] | ((uint32_t)tab[as_u32(j) >> 16] << 8);
}

// The 8 E4M3 codes of the RMSNorm output y_b = bf16(fl32(fl32(x r) gamma)) of
// one piece (x words w0..w3, gamma as fp32 gf[0..7]) by quant4_cvt, for any r
// and gamma (a NaN y_b takes 0x7F with its sign, +-inf saturates).
__device__ __forceinline__ uint2 rms_codes8_cvt(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, const float* gf,
                                                float r, float s, float rcp, float sat)
{
    const uint32_t w[4] = {w0, w1, w2, w3};
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        h[i] = pack_bf16x2(bf16_to_f32(w[i] & 0xffffu) * r * gf[2 * i], bf16_to_f32(w[i] >> 16) * r * gf[2 * i + 1]);
    return make_uint2(quant4_cvt(h[0], h[1], s, rcp, sat), quant4_cvt(h[2], h[3], s, rcp, sat));
}

// Bytes of a plain-quant band table: entries 0 .. kCodeBand + 2, padded.
constexpr int kBandTableBytes = ((int)kCodeBand + 3 + 15) & ~15;

// Fill a whole band table (entries 0, 1 .. kCodeBand, kCodeBand + 1, + 2) for
// s_act, the share of thread `tid` of `nthreads` (a multiple of 128).
__device__ __forceinline__ void fill_plain_band_table(uint8_t* tab, float s_act, int tid, int nthreads)
{
    fill_band_table(tab, code_band_lo(s_act), s_act, tid, nthreads);
    if (tid == 0) tab[0] = 0u, tab[kCodeBand + 1] = 0x7eu, tab[kCodeBand + 2] = 0x7eu;
}

// fp32 -> bf16 bits, round to nearest even, NaN -> quiet NaN with its sign,
// written without branches (same results as f32_to_bf16_rne).
__device__ __host__ __forceinline__ uint32_t f32_to_bf16_rne_sel(float f)
{
    uint32_t u;
    __builtin_memcpy(&u, &f, 4);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t q = ((u >> 16) & 0x8000u) | 0x7fc0u;
    return (u & 0x7fffffffu) > 0x7f800000u ? q : r;
}

// fp32 -> bf16 bits, round to nearest even, NaN stays NaN: gfx950's
// v_cvt_pk_bf16_f32 on the device, the integer form above on the host.
__device__ __host__ __forceinline__ uint32_t f32_to_bf16_cvt(float f)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(uint16_t, (__bf16)f);
#else
    return f32_to_bf16_rne_sel(f);
#endif
}

// Two fp32 -> packed bf16 bits (lo in bits 0-15), round to nearest even:
// v_cvt_pk_bf16_f32 on the device, the integer form on the host.
__device__ __host__ __forceinline__ uint32_t pack_bf16x2_hd(float lo, float hi)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return pack_bf16x2(lo, hi);
#else
    return f32_to_bf16_rne_sel(lo) | (f32_to_bf16_rne_sel(hi) << 16);
#endif
}

// The sign bits of the four bf16 values in words w0 (values 0, 1) and w1
// (values 2, 3) as bit 7 of bytes 0..3 (one byte permute on the device).
__device__ __host__ __forceinline__ uint32_t sign_bytes4(uint32_t w0, uint32_t w1)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_perm(w1, w0, 0x07050301u) & 0x80808080u;
#else
    return ((w0 >> 8) & 0x80u) | ((w0 >> 16) & 0x8000u) | ((w1 << 8) & 0x800000u) | (w1 & 0x80000000u);
#endif
}

// E4M3 codes of h = bf16(fl32(silu(g) * u)) under s_act for the 8 gate and up
// values of one 16-byte piece each (gate words gw, up words uw: value 2i in
// the low half of word i), the common case only: every gate inside the SiLU
// band (s = its table entry t) and no h a NaN.  Then h's code is the band
// table's entry of its magnitude (below the band a zero, above it 448, inf
// included) with h's sign.  Two values are handled per 32-bit word with
// packed 16-bit integer operations.  Writes the 8 table values of the gates
// (for the exact path) and returns false if some value is outside the common
// case; the codes are then not valid.  stab: the SiLU band table;
// ctab: the plain quant's band table; lo1 = code_band_lo(s_act) - 1.
__device__ __host__ __forceinline__ bool silu_mul_codes8_fast(const uint32_t (&gw)[4], const uint32_t (&uw)[4],
                                                              const float* stab, const uint8_t* ctab, uint32_t lo1,
                                                              float (&t)[8], uint2& out)
{
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // band offset |g| - kSiluLo of both halves; below the band it wraps past the band's end
        const u16x2_t d = as_u16x2(gw[i] & 0x7fff7fffu) - splat_u16x2(kSiluLo);
        const u16x2_t k = __builtin_elementwise_min(d, splat_u16x2(kSiluBand - 1u));
        ok = ok && as_u32(k) == as_u32(d);
        const uint32_t idx = as_u32(k) | ((gw[i] >> 3) & 0x10001000u);   // + sign * 4096
        t[2 * i] = stab[idx & 0xffffu];
        t[2 * i + 1] = stab[idx >> 16];
    }
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        h[i] = pack_bf16x2_hd(t[2 * i] * __builtin_bit_cast(float, uw[i] << 16),
                              t[2 * i + 1] * __builtin_bit_cast(float, uw[i] & 0xffff0000u));
    uint32_t c[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        uint32_t cc = 0u;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const u16x2_t a = as_u16x2(h[2 * q + e] & 0x7fff7fffu);
            ok = ok && as_u32(__builtin_elementwise_max(a, splat_u16x2(0x7f80u))) == 0x7f807f80u;   // no NaN
            cc |= band_codes2(h[2 * q + e], ctab, lo1) << (16 * e);
        }
        c[q] = cc | sign_bytes4(h[2 * q], h[2 * q + 1]);
    }
    out = make_uint2(c[0], c[1]);
    return ok;
}

// The same codes for any inputs, from the gates' table values t (as
// silu_mul_codes8_fast wrote them): s = silu_finish(g, t) (the closed forms
// outside the band), a NaN h encoded with its own sign.
__device__ __host__ __forceinline__ uint2 silu_mul_codes8_exact(const uint32_t (&gw)[4], const uint32_t (&uw)[4],
                                                                const float (&t)[8], const uint8_t* ctab,
                                                                uint32_t lo1)
{
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        h[i] = pack_bf16x2_hd(silu_finish(gw[i] & 0xffffu, t[2 * i]) * __builtin_bit_cast(float, uw[i] << 16),
                              silu_finish(gw[i] >> 16, t[2 * i + 1]) * __builtin_bit_cast(float, uw[i] & 0xffff0000u));
    uint32_t c[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        uint32_t cc = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t a = (h[2 * q + (e >> 1)] >> ((e & 1) * 16)) & 0x7fffu;
            const int j = (int)a - (int)lo1;
            const uint32_t code = ctab[j < 0 ? 0 : (j > (int)kCodeBand + 1 ? (int)kCodeBand + 1 : j)];
            cc |= (a > 0x7f80u ? 0x7fu : code) << (8 * e);
        }
        c[q] = cc | sign_bytes4(h[2 * q], h[2 * q + 1]);
    }
    return make_uint2(c[0], c[1]);
}

}  // namespace fp8mm
