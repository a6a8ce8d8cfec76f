// gemm_small_m.hip -- memory-bound FP8 E4M3 GEMM for decode-sized M (1..64) on
// gfx950: out[m,n] = bf16((sum_k x_q[m,k] w_q[n,k]) * s_act * s_w[n]).
//
// At decode M the layer streams the whole weight once per call, so the
// kernel is bound by HBM bandwidth, not by math: the pages measure the FP8
// tower at a quarter of a 27B decode step, its rate set by shape and merging
// (vllm.cpp #252 "SETTLED BY PAIRED TRACE"; 129.3 vs 213.6 GiB/s on GB10), and
// name the missing small-M tiles and the split-K reduce of the cuBLASLt path
// (vllm.cpp #252 original post item 3, "SETTLED BY PAIRED TRACE" table;
// vllm.cpp #213 "+0.0532 splitK reduce").
//
// Design (MI355X-first, not a port of those tiles):
//  * one workgroup owns a 16-row slice of W (one MFMA A tile) and the whole K;
//    its W waves split K into 128-byte chunks, wave w taking chunks w, w+W, ...
//    so that the workgroup sweeps each weight row front to back;
//  * every lane streams its 2 x 16 B of W per chunk straight from HBM into
//    registers (each weight byte is used by one MFMA only, so no LDS staging),
//    batched four chunks deep (fewer when x_q needs two or four M tiles);
//    x_q (at most 64 x K bytes) is re-read from L2;
//  * v_mfma_f32_16x16x128_f8f6f4 with x_q as the B operand, M padded to 16 (or
//    two / four M tiles for M <= 32 / 64): MFMA keeps the fp32 work off the VALU;
//  * the W partial sums are reduced in LDS in a fixed order (no atomics), then
//    the scale epilogue and the bf16 store happen in registers.
//  W depends on K only, so every column's summation order is the same for a
//  merged call and a per-shard call: results are bitwise identical.
#include "device_common.h"
#include "internal.h"

namespace fp8mm {

namespace {

constexpr int kChunk = 128;     // K bytes per MFMA (16x16x128)
constexpr int kBatchRegs = 4;   // chunk x M-tile fragments in flight per wave per batch
constexpr int kMaxWaves = 16;

__device__ __forceinline__ uint4 ld16(const uint8_t* p)
{
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ v8i pack(const uint4 lo, const uint4 hi)
{
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

template <int MT>
__global__ __launch_bounds__(64 * kMaxWaves) void k_gemm_small_m(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ wq, float s_act,
    const float* __restrict__ s_w, ShardTable sh, int M, int64_t K, int nchunks)
{
    extern __shared__ v4f red[];                       // [W][MT][64]
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;

    const uint8_t* wrow = wq + (n0 + r) * K + g * 32;
    const uint8_t* xrow[MT];
    bool xv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r;
        xv[mt] = m < M;
        xrow[mt] = xq + (int64_t)(xv[mt] ? m : 0) * K + g * 32;
    }

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};

    constexpr int kBatch = kBatchRegs / MT > 0 ? kBatchRegs / MT : 1;   // chunks per batch
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    const int nc = (nchunks - wave + W - 1) / W;       // chunks owned by this wave
    for (int i0 = 0; i0 < nc; i0 += kBatch) {
        uint4 a[kBatch][2];
        uint4 b[kBatch][MT][2];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t c = (int64_t)wave + (int64_t)(i0 + j) * W;
            const int64_t kb = c * kChunk + g * 32;    // this lane's first K byte
            const bool cv = (i0 + j) < nc;
            const bool v0 = cv && kb < K, v1 = cv && kb + 16 < K;
            a[j][0] = v0 ? ld16(wrow + c * kChunk) : z;
            a[j][1] = v1 ? ld16(wrow + c * kChunk + 16) : z;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                b[j][mt][0] = (v0 && xv[mt]) ? ld16(xrow[mt] + c * kChunk) : z;
                b[j][mt][1] = (v1 && xv[mt]) ? ld16(xrow[mt] + c * kChunk + 16) : z;
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const v8i A = pack(a[j][0], a[j][1]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    A, pack(b[j][mt][0], b[j][mt][1]), acc[mt], 0, 0, 0, 0, 0, 0);
        }
    }

    // Fixed-order reduction of the W per-wave partials.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * 64 + lane] = acc[mt];
    __syncthreads();
    for (int idx = threadIdx.x; idx < MT * 64; idx += blockDim.x) {   // blocks may be narrower than MT*64
        const int mt = idx >> 6, l = idx & 63;
        v4f s = red[mt * 64 + l];
        for (int w = 1; w < W; ++w) {
            const v4f p = red[(w * MT + mt) * 64 + l];
            s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
        }
        // C layout of 16x16 MFMA: lane l holds rows 4*(l/16)+v (= n) of column l%16 (= m).
        const int m = mt * 16 + (l & 15);
        if (m < M) {
            const int64_t n = n0 + 4 * (l >> 4);
            int i = 0;
            while (i + 1 < sh.num && n0 >= sh.start[i + 1]) ++i;
            const float4 sw = *reinterpret_cast<const float4*>(s_w + n);
            const uint32_t o0 = f32_to_bf16_rne((s.x * s_act) * sw.x) | (f32_to_bf16_rne((s.y * s_act) * sw.y) << 16);
            const uint32_t o1 = f32_to_bf16_rne((s.z * s_act) * sw.z) | (f32_to_bf16_rne((s.w * s_act) * sw.w) << 16);
            *reinterpret_cast<uint2*>(sh.out[i] + (int64_t)m * sh.ldo[i] + (n - sh.start[i])) = make_uint2(o0, o1);
        }
    }
}

}  // namespace

// Waves per workgroup: a function of K only (it fixes the summation order).
int small_m_waves(int64_t K)
{
    const int64_t nchunks = (K + kChunk - 1) / kChunk;
    int64_t w = (nchunks + 7) / 8;
    if (w < 1) w = 1;
    if (w > kMaxWaves) w = kMaxWaves;
    return (int)w;
}

void launch_gemm_small_m(const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w,
                         const ShardTable& shards, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    const int W = small_m_waves(K);
    const int nchunks = (int)((K + kChunk - 1) / kChunk);
    const dim3 grid((uint32_t)(N / 16)), block(64 * W);
    const int MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    const size_t lds = (size_t)W * MT * 64 * sizeof(v4f);
    if (MT == 1)
        hipLaunchKernelGGL(k_gemm_small_m<1>, grid, block, lds, stream, xq, wq, s_act, s_w, shards, (int)M, K, nchunks);
    else if (MT == 2)
        hipLaunchKernelGGL(k_gemm_small_m<2>, grid, block, lds, stream, xq, wq, s_act, s_w, shards, (int)M, K, nchunks);
    else
        hipLaunchKernelGGL(k_gemm_small_m<4>, grid, block, lds, stream, xq, wq, s_act, s_w, shards, (int)M, K, nchunks);
}

}  // namespace fp8mm
