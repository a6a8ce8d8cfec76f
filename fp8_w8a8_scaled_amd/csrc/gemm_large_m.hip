// gemm_large_m.hip -- compute-bound FP8 E4M3 GEMM for prefill-sized M on gfx950
// FP8 MFMA: out[m,n] = bf16((sum_k x_q[m,k] w_q[n,k]) * s_act * s_w[n]).
//
// At chunked-prefill M the layer is compute-bound (vLLM PR #53014, Marlin
// large-M commit message: a 6576-token chunk spends 96.5% of its GPU time in
// GEMM).  W8A8 needs no weight dequantization there: both operands are already
// E4M3, so the large-M arm runs the FP8 matrix cores directly.
//
// Design: 128x128 output tile per 256-thread workgroup (2x2 waves, 64x64 per
// wave as 2x2 v_mfma_f32_32x32x64_f8f6f4 tiles), K stepped 128 bytes at a
// time through a double-buffered LDS stage (global -> registers -> LDS while
// the previous stage feeds the MFMAs, one barrier per step).  LDS rows are
// padded to 144 B so the 16-byte fragment reads of 16 consecutive rows hit
// distinct banks.  Ragged M, N and K edges are zero-filled on load and masked
// on store.  The epilogue scales in fp32 and stores bf16.
#include "device_common.h"
#include "internal.h"

namespace fp8mm {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDS_ROW = BK + 16;                  // padded row stride, bytes
constexpr int kThreads = 256;

__device__ __forceinline__ v8i pack(const uint4 lo, const uint4 hi)
{
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

__global__ __launch_bounds__(kThreads) void k_gemm_large_m(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ wq, float s_act,
    const float* __restrict__ s_w, ShardTable sh, int64_t M, int64_t N, int64_t K)
{
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * LDS_ROW];   // x_q tile, m rows
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * LDS_ROW];   // w_q tile, n rows

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;

    // Each thread moves 4 16-byte pieces of each operand tile per K step.
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    uint4 ra[4], rb[4];
    auto load_tile = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = t + i * kThreads;
            const int row = p >> 3, c16 = (p & 7) * 16;
            const int64_t k = k0 + c16;
            const int64_t gm = m0 + row, gn = n0 + row;
            ra[i] = (gm < M && k < K) ? *reinterpret_cast<const uint4*>(xq + gm * K + k) : z;
            rb[i] = (gn < N && k < K) ? *reinterpret_cast<const uint4*>(wq + gn * K + k) : z;
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = t + i * kThreads;
            const int row = p >> 3, c16 = (p & 7) * 16;
            *reinterpret_cast<uint4*>(&sA[buf][row * LDS_ROW + c16]) = ra[i];
            *reinterpret_cast<uint4*>(&sB[buf][row * LDS_ROW + c16]) = rb[i];
        }
    };

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int64_t nk = (K + BK - 1) / BK;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    const int fr = lane & 31, fk = (lane >> 5) * 32;   // fragment row, K byte offset
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int buf = (int)(kt & 1);
        if (kt + 1 < nk) load_tile((kt + 1) * BK);
#pragma unroll
        for (int s = 0; s < 2; ++s) {                 // two 64-byte K sub-steps
            v8i a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint8_t* pa = &sA[buf][(wm * 64 + i * 32 + fr) * LDS_ROW + s * 64 + fk];
                a[i] = pack(*reinterpret_cast<const uint4*>(pa), *reinterpret_cast<const uint4*>(pa + 16));
                const uint8_t* pb = &sB[buf][(wn * 64 + i * 32 + fr) * LDS_ROW + s * 64 + fk];
                b[i] = pack(*reinterpret_cast<const uint4*>(pb), *reinterpret_cast<const uint4*>(pb + 16));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        a[i], b[j], acc[i][j], 0, 0, 0, 0, 0, 0);
        }
        if (kt + 1 < nk) store_tile(buf ^ 1);
        __syncthreads();
    }

    // Epilogue.  32x32 MFMA C layout: lane l holds column l%32 (= n) and rows
    // 8*(v/4) + 4*(l/32) + v%4 (= m) for v = 0..15.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (n >= N) continue;
        int si = 0;
        while (si + 1 < sh.num && n >= sh.start[si + 1]) ++si;
        uint16_t* o = sh.out[si] + (n - sh.start[si]);
        const int64_t ldo = sh.ldo[si];
        const float swn = s_w[n];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < M) o[m * ldo] = (uint16_t)f32_to_bf16_rne((acc[i][j][v] * s_act) * swn);
            }
    }
}

}  // namespace

void launch_gemm_large_m(const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w,
                         const ShardTable& shards, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    const dim3 grid((uint32_t)((N + BN - 1) / BN), (uint32_t)((M + BM - 1) / BM));
    hipLaunchKernelGGL(k_gemm_large_m, grid, dim3(kThreads), 0, stream, xq, wq, s_act, s_w, shards, M, N, K);
}

}  // namespace fp8mm
