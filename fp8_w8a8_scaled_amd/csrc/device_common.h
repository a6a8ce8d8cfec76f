// device_common.h -- number formats and small vector helpers for the gfx950
// kernels of the FP8 E4M3 W8A8 scaled-matmul layer.
//
// E4M3 here is OCP E4M3FN (gfx950's native FP8): bias 7, 3 mantissa bits, max
// 448, S.1111.111 = NaN, no infinity.  The pages name the dtype F8_E4M3 /
// torch.float8_e4m3fn (vllm.cpp #252 original post; vllm.cpp #417 Finding 2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mm {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Saturating round-to-nearest-even fp32 -> E4M3FN, integer bit manipulation.
//  |t| >= 448 or inf -> +-448 (0x7E); NaN -> 0x7F (sign kept); otherwise the
//  nearest E4M3 value with ties to the even mantissa; the sign bit is always
//  copied, so a negative value that rounds to zero gives 0x80.
__device__ __host__ __forceinline__ uint32_t f32_to_e4m3_sat(float t)
{
    uint32_t u;
    __builtin_memcpy(&u, &t, 4);
    const uint32_t s = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    uint32_t code;
    if (a > 0x7f800000u) {
        code = 0x7fu;                                  // NaN
    } else if (a >= 0x43e00000u) {
        code = 0x7eu;                                  // >= 448, inf: saturate
    } else if (a >= 0x3c800000u) {
        // >= 2^-6: normal E4M3.  Round the 23-bit fp32 mantissa to 3 bits
        // (RNE at bit 20); a carry moves into the exponent by itself.
        const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
        code = (r >> 20) - (120u << 3);                // rebias 127 -> 7
    } else if (a < 0x3a800000u) {
        code = 0u;                                     // below 2^-10: rounds to 0
    } else {
        // [2^-10, 2^-6): the subnormal grid m * 2^-9, m in 0..8 (8 = 2^-6).
        const uint32_t e = a >> 23;                    // 117..120
        const uint32_t mant = (a & 0x7fffffu) | 0x800000u;
        const uint32_t sh = 141u - e;                  // value * 2^9 = mant >> sh
        code = (mant + (1u << (sh - 1u)) - 1u + ((mant >> sh) & 1u)) >> sh;
    }
    return s | code;
}

__device__ __host__ __forceinline__ float bf16_to_f32(uint32_t b)
{
    uint32_t u = b << 16;
    float f;
    __builtin_memcpy(&f, &u, 4);
    return f;
}

// fp32 -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN.
__device__ __host__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    __builtin_memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> packed bf16 bits (lo in bits 0-15), round to nearest even, with
// one gfx950 v_cvt_pk_bf16_f32.  Same bits as f32_to_bf16_rne for every
// non-NaN input (a NaN stays a NaN of its sign).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// 8 bf16 values (one 16-byte load) -> 8 E4M3 codes of x / s (one 8-byte store).
// A NaN input is encoded with its own sign bit (the sign of a NaN produced by a
// division is not fixed by IEEE 754).
__device__ __forceinline__ uint2 quant8(const uint4 in, float s_act)
{
    const uint32_t w[4] = {in.x, in.y, in.z, in.w};
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t b = (w[i >> 1] >> ((i & 1) * 16)) & 0xffffu;
        const uint32_t c = ((b & 0x7fffu) > 0x7f80u) ? (0x7fu | ((b >> 8) & 0x80u))
                                                     : f32_to_e4m3_sat(bf16_to_f32(b) / s_act);
        o[i >> 2] |= c << ((i & 3) * 8);
    }
    return make_uint2(o[0], o[1]);
}

}  // namespace fp8mm
