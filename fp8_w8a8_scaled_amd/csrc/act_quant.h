// act_quant.h -- per-piece steps of the activation quant (16-byte pieces of 8
// bf16 values), shared by the activation quant kernels so that every one of
// them produces the same bytes.
//
// Fused RMSNorm -> FP8 (vllm.cpp issue #417, ranked follow-ons:
// InputLayernormFp8, byte-exact against QuantFp8Static), per row:
//   r   = fl32(1 / sqrt(sum(x^2) / K + eps))    (sum and sqrt in fp64)
//   y   = bf16_RNE(fl32(fl32(x * r) * gamma))
//   x_q = satRNE_E4M3(fl32(y / s_act))
#pragma once

#include "device_common.h"

namespace fp8mm {

// Threads that sum one row's squares in the standalone RMSNorm quant (4
// waves): thread t adds pieces t, t + 256, ... in order, each wave sums its
// threads' values by an xor butterfly, and the 4 wave sums are added in wave
// order.  A kernel that computes the same r must take the same order.
constexpr int kRmsRowThreads = 256;

// ss + the squares of the 8 values of a piece, added in element order.  The
// square of a bf16 value (8 significant bits) is exact in fp64, so the fused
// multiply-add rounds exactly as the product followed by the sum would.
__device__ __forceinline__ double sumsq8(const uint4 in, double ss)
{
    const uint32_t w[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double f = (double)bf16_to_f32((w[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
        ss = __builtin_fma(f, f, ss);
    }
    return ss;
}

// r from the row's sum of squares.
__device__ __forceinline__ float rms_inv(double ss, int64_t K, float eps)
{
    return (float)(1.0 / sqrt(ss / (double)K + (double)eps));
}

// y_b = bf16(fl32(fl32(x * r) * gamma)) for 8 values; returns them as fp32.
__device__ __forceinline__ void rms_apply8(const uint4 in, const uint4 g, float r, float y[8])
{
    const uint32_t w[4] = {in.x, in.y, in.z, in.w};
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float xv = bf16_to_f32((w[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
        const float gv = bf16_to_f32((gw[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
        const float xn = xv * r;
        const float yf = xn * gv;
        y[i] = bf16_to_f32(f32_to_bf16_rne(yf));
    }
}

// The 8 E4M3 codes of the RMSNorm output of a piece (gamma piece g).
__device__ __forceinline__ uint2 rms_quant8(const uint4 in, const uint4 g, float r, float s_act)
{
    float y[8];
    rms_apply8(in, g, r, y);
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i >> 2] |= f32_to_e4m3_sat(y[i] / s_act) << ((i & 3) * 8);
    return make_uint2(o[0], o[1]);
}

}  // namespace fp8mm
