// quant.hip -- activation quantize-once kernels (fused RMSNorm -> E4M3 and
// plain static quant), static-scale calibration, and load-time per-channel
// weight quantization, for gfx950.
//
// Sources: the static per-tensor quant (QuantFp8Static) and the fused
// RMSNorm->fp8 quant that is byte-exact against it (InputLayernormFp8, "112 ->
// 16 QuantFp8Static launches/step"): vllm.cpp issue #417, ranked follow-ons.
// Per-channel ("FP8 channelwise") weight scales: vLLM PR #53014, Marlin large-M
// commit message.
//
// All kernels are memory-bound streaming passes: 16-byte bf16 loads, 8-byte
// E4M3 stores, no LDS except for block reductions.
#include "device_common.h"
#include "internal.h"

namespace fp8mm {

namespace {

constexpr int kQuantThreads = 256;

// Fixed-order block reduction of a double (wave butterfly, then waves in order).
__device__ double block_sum_f64(double v, double* lds)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) lds[wave] = v;
    __syncthreads();
    double s = 0.0;
    const int nw = blockDim.x >> 6;
    for (int w = 0; w < nw; ++w) s += lds[w];
    __syncthreads();
    return s;
}

__device__ float block_max_f32(float v, float* lds)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) lds[wave] = v;
    __syncthreads();
    float s = 0.0f;
    const int nw = blockDim.x >> 6;
    for (int w = 0; w < nw; ++w) s = fmaxf(s, lds[w]);
    __syncthreads();
    return s;
}

// r = fl32(1 / sqrt(sum(x^2) / K + eps)) with the sum and the sqrt in fp64.
__device__ float row_rms_inv(const uint16_t* __restrict__ row, int64_t K, float eps, double* lds)
{
    const int64_t nv = K >> 3;
    double ss = 0.0;
    for (int64_t v = threadIdx.x; v < nv; v += blockDim.x) {
        const uint4 in = *reinterpret_cast<const uint4*>(row + v * 8);
        const uint32_t w[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double f = (double)bf16_to_f32((w[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
            ss += f * f;                      // exact: a bf16 square has <= 16 bits
        }
    }
    ss = block_sum_f64(ss, lds);
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

__global__ __launch_bounds__(kQuantThreads) void k_quant_plain(
    const uint16_t* __restrict__ x, int64_t ldx, float s_act,
    uint8_t* __restrict__ xq, int64_t M, int64_t K)
{
    const int64_t nv = K >> 3, total = M * nv;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / nv, v = i - m * nv;
        const uint4 in = *reinterpret_cast<const uint4*>(x + m * ldx + v * 8);
        *reinterpret_cast<uint2*>(xq + m * K + v * 8) = quant8(in, s_act);
    }
}

__global__ __launch_bounds__(kQuantThreads) void k_quant_rmsnorm(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ gamma, float eps,
    float s_act, uint8_t* __restrict__ xq, int64_t K)
{
    __shared__ double lds[kQuantThreads / 64];
    const int64_t m = blockIdx.x;
    const uint16_t* row = x + m * ldx;
    const float r = row_rms_inv(row, K, eps, lds);
    const int64_t nv = K >> 3;
    for (int64_t v = threadIdx.x; v < nv; v += blockDim.x) {
        const uint4 in = *reinterpret_cast<const uint4*>(row + v * 8);
        const uint4 g = *reinterpret_cast<const uint4*>(gamma + v * 8);
        float y[8];
        rms_apply8(in, g, r, y);
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i >> 2] |= f32_to_e4m3_sat(y[i] / s_act) << ((i & 3) * 8);
        *reinterpret_cast<uint2*>(xq + m * K + v * 8) = make_uint2(o[0], o[1]);
    }
}

// ---- calibration: amax of the tensor that gets quantized -> s_act ----------

__device__ __forceinline__ float finite_abs_max(float acc, float v)
{
    const float a = fabsf(v);
    return (a < INFINITY && a > acc) ? a : acc;   // NaN and inf are skipped
}

__global__ __launch_bounds__(kQuantThreads) void k_absmax_plain(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t M, int64_t K, float* __restrict__ partial)
{
    __shared__ float lds[kQuantThreads / 64];
    const int64_t nv = K >> 3, total = M * nv;
    float amax = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / nv, v = i - m * nv;
        const uint4 in = *reinterpret_cast<const uint4*>(x + m * ldx + v * 8);
        const uint32_t w[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = finite_abs_max(amax, bf16_to_f32((w[j >> 1] >> ((j & 1) * 16)) & 0xffffu));
    }
    amax = block_max_f32(amax, lds);
    if (threadIdx.x == 0) partial[blockIdx.x] = amax;
}

__global__ __launch_bounds__(kQuantThreads) void k_absmax_rmsnorm(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ gamma, float eps,
    int64_t K, float* __restrict__ partial)
{
    __shared__ double lds[kQuantThreads / 64];
    __shared__ float ldsf[kQuantThreads / 64];
    const int64_t m = blockIdx.x;
    const uint16_t* row = x + m * ldx;
    const float r = row_rms_inv(row, K, eps, lds);
    const int64_t nv = K >> 3;
    float amax = 0.0f;
    for (int64_t v = threadIdx.x; v < nv; v += blockDim.x) {
        const uint4 in = *reinterpret_cast<const uint4*>(row + v * 8);
        const uint4 g = *reinterpret_cast<const uint4*>(gamma + v * 8);
        float y[8];
        rms_apply8(in, g, r, y);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = finite_abs_max(amax, y[j]);
    }
    amax = block_max_f32(amax, ldsf);
    if (threadIdx.x == 0) partial[m] = amax;
}

__global__ __launch_bounds__(kQuantThreads) void k_absmax_final(
    const float* __restrict__ partial, int64_t n, float* __restrict__ s_act)
{
    __shared__ float lds[kQuantThreads / 64];
    float amax = 0.0f;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) amax = fmaxf(amax, partial[i]);
    amax = block_max_f32(amax, lds);
    if (threadIdx.x == 0) *s_act = (amax == 0.0f) ? 1.0f : amax / 448.0f;
}

// ---- SiLU*mul -> E4M3 (the MLP activation feeding the down projection) -----

// h_b = bf16(fl32(silu(g) * u)) for 8 values (silu(g) = g / (1 + exp(-g)) in
// fp64, rounded once to fp32), returned as fp32.
__device__ __forceinline__ void silu_mul8(const uint4 g, const uint4 u, float h[8])
{
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double d = (double)bf16_to_f32((gw[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
        const float s = (float)(d / (1.0 + exp(-d)));
        const float uv = bf16_to_f32((uw[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
        h[i] = bf16_to_f32(f32_to_bf16_rne(s * uv));
    }
}

__global__ __launch_bounds__(kQuantThreads) void k_silu_mul_quant(
    const uint16_t* __restrict__ gate, int64_t ldg, const uint16_t* __restrict__ up, int64_t ldu, float s_act,
    uint8_t* __restrict__ xq, int64_t M, int64_t I)
{
    const int64_t nv = I >> 3, total = M * nv;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / nv, v = i - m * nv;
        const uint4 g = *reinterpret_cast<const uint4*>(gate + m * ldg + v * 8);
        const uint4 u = *reinterpret_cast<const uint4*>(up + m * ldu + v * 8);
        float h[8];
        silu_mul8(g, u, h);
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t hb;
            __builtin_memcpy(&hb, &h[j], 4);
            // a NaN is encoded with its own sign (as the plain quant does)
            const uint32_t c = isnan(h[j]) ? (0x7fu | ((hb >> 24) & 0x80u)) : f32_to_e4m3_sat(h[j] / s_act);
            o[j >> 2] |= c << ((j & 3) * 8);
        }
        *reinterpret_cast<uint2*>(xq + m * I + v * 8) = make_uint2(o[0], o[1]);
    }
}

__global__ __launch_bounds__(kQuantThreads) void k_absmax_silu_mul(
    const uint16_t* __restrict__ gate, int64_t ldg, const uint16_t* __restrict__ up, int64_t ldu, int64_t M,
    int64_t I, float* __restrict__ partial)
{
    __shared__ float lds[kQuantThreads / 64];
    const int64_t nv = I >> 3, total = M * nv;
    float amax = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / nv, v = i - m * nv;
        float h[8];
        silu_mul8(*reinterpret_cast<const uint4*>(gate + m * ldg + v * 8),
                  *reinterpret_cast<const uint4*>(up + m * ldu + v * 8), h);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = finite_abs_max(amax, h[j]);
    }
    amax = block_max_f32(amax, lds);
    if (threadIdx.x == 0) partial[blockIdx.x] = amax;
}

// ---- load-time per-output-channel weight quant ----------------------------

__global__ __launch_bounds__(kQuantThreads) void k_quant_weight(
    const float* __restrict__ w, int64_t K, uint8_t* __restrict__ wq, float* __restrict__ s_w)
{
    __shared__ float lds[kQuantThreads / 64];
    const int64_t n = blockIdx.x;
    const float* row = w + n * K;
    const int64_t nv = K >> 3;
    float amax = 0.0f;
    for (int64_t v = threadIdx.x; v < nv; v += blockDim.x) {
        const float4 a = *reinterpret_cast<const float4*>(row + v * 8);
        const float4 b = *reinterpret_cast<const float4*>(row + v * 8 + 4);
        const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float av = fabsf(f[j]);
            amax = av > amax ? av : amax;
        }
    }
    amax = block_max_f32(amax, lds);
    const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    if (threadIdx.x == 0) s_w[n] = s;
    for (int64_t v = threadIdx.x; v < nv; v += blockDim.x) {
        const float4 a = *reinterpret_cast<const float4*>(row + v * 8);
        const float4 b = *reinterpret_cast<const float4*>(row + v * 8 + 4);
        const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j >> 2] |= f32_to_e4m3_sat(f[j] / s) << ((j & 3) * 8);
        *reinterpret_cast<uint2*>(wq + n * K + v * 8) = make_uint2(o[0], o[1]);
    }
}

int64_t plain_grid(int64_t M, int64_t K)
{
    const int64_t total = M * (K >> 3);
    int64_t blocks = (total + kQuantThreads - 1) / kQuantThreads;
    return blocks < 4096 ? (blocks < 1 ? 1 : blocks) : 4096;
}

}  // namespace

void launch_quant(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, float s_act,
                  uint8_t* xq, int64_t M, int64_t K, hipStream_t stream)
{
    if (gamma) {
        hipLaunchKernelGGL(k_quant_rmsnorm, dim3((uint32_t)M), dim3(kQuantThreads), 0, stream,
                           x, ldx, gamma, eps, s_act, xq, K);
    } else {
        hipLaunchKernelGGL(k_quant_plain, dim3((uint32_t)plain_grid(M, K)), dim3(kQuantThreads), 0, stream,
                           x, ldx, s_act, xq, M, K);
    }
}

size_t act_scale_partials(int64_t M, int64_t K, bool rms)
{
    return rms ? (size_t)M : (size_t)plain_grid(M, K);
}

void launch_act_scale(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps,
                      int64_t M, int64_t K, float* s_act, float* partial, hipStream_t stream)
{
    const int64_t np = (int64_t)act_scale_partials(M, K, gamma != nullptr);
    if (gamma) {
        hipLaunchKernelGGL(k_absmax_rmsnorm, dim3((uint32_t)M), dim3(kQuantThreads), 0, stream,
                           x, ldx, gamma, eps, K, partial);
    } else {
        hipLaunchKernelGGL(k_absmax_plain, dim3((uint32_t)np), dim3(kQuantThreads), 0, stream,
                           x, ldx, M, K, partial);
    }
    hipLaunchKernelGGL(k_absmax_final, dim3(1), dim3(kQuantThreads), 0, stream, partial, np, s_act);
}

void launch_silu_mul_quant(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu, float s_act,
                           uint8_t* xq, int64_t M, int64_t I, hipStream_t stream)
{
    hipLaunchKernelGGL(k_silu_mul_quant, dim3((uint32_t)plain_grid(M, I)), dim3(kQuantThreads), 0, stream, gate, ldg,
                       up, ldu, s_act, xq, M, I);
}

void launch_act_scale_silu_mul(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu, int64_t M,
                               int64_t I, float* s_act, float* partial, hipStream_t stream)
{
    const int64_t np = plain_grid(M, I);
    hipLaunchKernelGGL(k_absmax_silu_mul, dim3((uint32_t)np), dim3(kQuantThreads), 0, stream, gate, ldg, up, ldu, M,
                       I, partial);
    hipLaunchKernelGGL(k_absmax_final, dim3(1), dim3(kQuantThreads), 0, stream, partial, np, s_act);
}

void launch_quant_weight(const float* w, int64_t N, int64_t K, uint8_t* wq, float* s_w, hipStream_t stream)
{
    hipLaunchKernelGGL(k_quant_weight, dim3((uint32_t)N), dim3(kQuantThreads), 0, stream, w, K, wq, s_w);
}

}  // namespace fp8mm
