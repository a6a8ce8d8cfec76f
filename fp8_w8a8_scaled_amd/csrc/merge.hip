// merge.hip -- load-time weight preparation for merged projections whose
// shards carry one per-tensor weight scale each (the q/k/v or qkv/z shards of a
// checkpoint), for gfx950.
//
// Source: vllm.cpp issue #417, ranked follow-ons -- one implementation keeps
// the three q/k/v GEMMs apart unless their input scales are bitwise equal,
// another always merges and requantizes shards with mismatched scales to the
// largest weight scale, which loses precision where the first stays exact;
// vllm.cpp issue #213, "The GDN fp8 merge predicate FIRES" -- the merge only
// fires on bitwise-equal input scales.
//
// Two exact ways and one lossy way are provided:
//   - per-tensor weight quant (one scale for a whole shard);
//   - expanding each shard's per-tensor scale into the per-channel scale vector
//     the GEMMs take (exact: the merged product equals the split products);
//   - requantizing every shard to the largest shard scale (lossy: one scale
//     for the merged weight).
// All three are streaming passes over the weight with 16-byte accesses; none is
// on the per-step path.
#include "device_common.h"
#include "internal.h"

namespace fp8mm {

namespace {

constexpr int kThreads = 256;
constexpr int64_t kMaxGrid = 4096;

// Value of an E4M3FN code as fp32 (exact).  e == 0: m * 2^-9; otherwise
// (1 + m/8) * 2^(e-7), built directly as fp32 bits.  NaN codes are handled by
// the callers before they get here.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c)
{
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float mag;
    if (e == 0u) {
        mag = (float)m * 0x1p-9f;
    } else {
        const uint32_t u = ((e + 120u) << 23) | (m << 20);
        __builtin_memcpy(&mag, &u, 4);
    }
    return (c & 0x80u) ? -mag : mag;
}

int64_t grid_for(int64_t chunks)
{
    int64_t g = (chunks + kThreads - 1) / kThreads;
    return g < 1 ? 1 : (g > kMaxGrid ? kMaxGrid : g);
}

// ---- per-tensor weight quant ----------------------------------------------

// partial[b] = largest |w| this workgroup saw (a NaN is skipped, inf kept: the
// plain `a > amax` rule of the per-channel weight quant).
__global__ __launch_bounds__(kThreads) void k_absmax_weight(const float* __restrict__ w, int64_t chunks,
                                                            float* __restrict__ partial)
{
    __shared__ float lds[kThreads / 64];
    float amax = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < chunks; i += (int64_t)gridDim.x * kThreads) {
        const float4 v = reinterpret_cast<const float4*>(w)[i];
        const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float a = fabsf(f[j]);
            amax = a > amax ? a : amax;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = amax;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = 0.0f;
        for (int i = 0; i < kThreads / 64; ++i) m = fmaxf(m, lds[i]);
        partial[blockIdx.x] = m;
    }
}

// *s = fl32(max(partial) / 448), 1 when the weight is all zero.
__global__ __launch_bounds__(kThreads) void k_weight_scale(const float* __restrict__ partial, int64_t n,
                                                           float* __restrict__ s)
{
    __shared__ float lds[kThreads / 64];
    float amax = 0.0f;
    for (int64_t i = threadIdx.x; i < n; i += kThreads) amax = fmaxf(amax, partial[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = amax;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = 0.0f;
        for (int i = 0; i < kThreads / 64; ++i) m = fmaxf(m, lds[i]);
        *s = (m == 0.0f) ? 1.0f : m / 448.0f;
    }
}

// w_q = satRNE_E4M3(fl32(w / s)) with the device scale *s; 8 values per step.
__global__ __launch_bounds__(kThreads) void k_quant_weight_tensor(const float* __restrict__ w, int64_t chunks8,
                                                                  const float* __restrict__ s_dev,
                                                                  uint8_t* __restrict__ wq)
{
    const float s = *s_dev;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < chunks8; i += (int64_t)gridDim.x * kThreads) {
        const float4 a = reinterpret_cast<const float4*>(w)[2 * i];
        const float4 b = reinterpret_cast<const float4*>(w)[2 * i + 1];
        const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j >> 2] |= f32_to_e4m3_sat(f[j] / s) << ((j & 3) * 8);
        reinterpret_cast<uint2*>(wq)[i] = make_uint2(o[0], o[1]);
    }
}

// ---- shard scales -----------------------------------------------------------

// s_w[r] = scale of the shard that holds weight row r.
__global__ __launch_bounds__(kThreads) void k_expand_shard_scales(ShardScales tab, float* __restrict__ s_w)
{
    const int64_t rows = tab.start[tab.num];
    for (int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x; r < rows; r += (int64_t)gridDim.x * kThreads) {
        int i = 0;
        while (i + 1 < tab.num && r >= tab.start[i + 1]) ++i;
        s_w[r] = tab.scale[i];
    }
}

// out = satRNE_E4M3(fl32(fl32(dec(c) * s_i) / s_max)) per byte, 16 bytes per
// step (K % 16 == 0, so a step never straddles two rows or two shards); NaN
// codes are copied.  Every s_w[r] becomes s_max.  in == out is allowed: each
// byte is read and written by the same thread.
__global__ __launch_bounds__(kThreads) void k_requant_max_scale(const uint8_t* in, uint8_t* out, ShardScales tab,
                                                                float s_max, int64_t K, float* __restrict__ s_w)
{
    const int64_t rows = tab.start[tab.num];
    const int64_t chunks = rows * (K >> 4);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < chunks; i += stride) {
        const int64_t r = (i << 4) / K;
        int sh = 0;
        while (sh + 1 < tab.num && r >= tab.start[sh + 1]) ++sh;
        const float si = tab.scale[sh];
        const uint4 v = reinterpret_cast<const uint4*>(in)[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t acc = 0u;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t c = (w[q] >> (8 * b)) & 0xffu;
                uint32_t code;
                if ((c & 0x7fu) == 0x7fu) {
                    code = c;                                  // NaN kept as it is
                } else {
                    const float wv = e4m3_to_f32(c) * si;      // the shard's f32 weight value
                    code = f32_to_e4m3_sat(wv / s_max);
                }
                acc |= code << (8 * b);
            }
            o[q] = acc;
        }
        reinterpret_cast<uint4*>(out)[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    for (int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x; r < rows; r += stride) s_w[r] = s_max;
}

}  // namespace

size_t weight_absmax_partials(int64_t N, int64_t K) { return (size_t)grid_for((N * K) >> 2); }

void launch_quant_weight_per_tensor(const float* w, int64_t N, int64_t K, uint8_t* wq, float* s,
                                    float* partial, hipStream_t stream)
{
    const int64_t chunks4 = (N * K) >> 2, chunks8 = (N * K) >> 3;
    const int64_t np = grid_for(chunks4);
    hipLaunchKernelGGL(k_absmax_weight, dim3((uint32_t)np), dim3(kThreads), 0, stream, w, chunks4, partial);
    hipLaunchKernelGGL(k_weight_scale, dim3(1), dim3(kThreads), 0, stream, partial, np, s);
    hipLaunchKernelGGL(k_quant_weight_tensor, dim3((uint32_t)grid_for(chunks8)), dim3(kThreads), 0, stream, w,
                       chunks8, s, wq);
}

void launch_expand_shard_scales(const ShardScales& tab, float* s_w, hipStream_t stream)
{
    hipLaunchKernelGGL(k_expand_shard_scales, dim3((uint32_t)grid_for(tab.start[tab.num])), dim3(kThreads), 0,
                       stream, tab, s_w);
}

void launch_requant_max_scale(const uint8_t* in, uint8_t* out, const ShardScales& tab, float s_max, int64_t K,
                              float* s_w, hipStream_t stream)
{
    const int64_t chunks = tab.start[tab.num] * (K >> 4);
    hipLaunchKernelGGL(k_requant_max_scale, dim3((uint32_t)grid_for(chunks)), dim3(kThreads), 0, stream, in, out,
                       tab, s_max, K, s_w);
}

}  // namespace fp8mm
