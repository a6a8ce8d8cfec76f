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
//  * a workgroup owns NT x 16 rows of W (NT MFMA A tiles) and the whole K; its
//    W waves split K into 128-byte chunks, wave w taking chunks w, w+W, ..., so
//    the workgroup sweeps each weight row front to back;
//  * every lane streams 2 x 16 B of each of its rows per chunk straight from
//    HBM into registers: bytes [16g, 16g+16) and [64+16g, 80+16g) of the chunk
//    for lane group g, so one load instruction covers 64 contiguous bytes of
//    each of 16 rows.  Each weight byte feeds one MFMA only, so there is no LDS
//    staging.  Loads run a batch of chunks ahead of the MFMAs (double buffer);
//  * v_mfma_f32_16x16x128_f8f6f4 with x_q as the B operand, M padded to 16
//    (MT = 2 or 4 M tiles for M <= 32 / 64).  x_q (at most 64 x K bytes) is read
//    from L2 with the same K mapping as W, which is all the MFMA needs;
//  * the W per-wave partial sums are reduced in LDS in a fixed order (no
//    atomics), then the scale epilogue and the bf16 store happen in registers.
//  W and the chunk assignment depend on K only, so every column's summation
//  order is the same for a merged call and a per-shard call: bitwise identical.
#include "device_common.h"
#include "internal.h"
#include "out_store.h"

// Tuning knobs (build-time).  Target chunks per wave -> waves per workgroup.
#ifndef FP8MM_SMALLM_CPW
#define FP8MM_SMALLM_CPW 5
#endif
// Chunk fragments (x N tiles x M tiles) in flight per wave per batch.
#ifndef FP8MM_SMALLM_BATCH
#define FP8MM_SMALLM_BATCH 2
#endif
// 1: issue the next batch's loads before the current batch's MFMAs.
#ifndef FP8MM_SMALLM_PIPE
#define FP8MM_SMALLM_PIPE 1
#endif
// 16-row N tiles per workgroup (each wave covers all of them; x_q is reused).
#ifndef FP8MM_SMALLM_NT
#define FP8MM_SMALLM_NT 1
#endif
// 1: weight loads marked non-temporal (streamed once).
#ifndef FP8MM_SMALLM_NTLOAD
#define FP8MM_SMALLM_NTLOAD 0
#endif

// Largest LDS footprint (x_q rows + reduction) of the all-in-flight variant;
// 0 disables it.  Three workgroups of this size fit in a 160 KB CU.
#ifndef FP8MM_SMALLM_XLDS_MAX
#define FP8MM_SMALLM_XLDS_MAX (52 * 1024)
#endif
// 16-row weight tiles per workgroup of the all-in-flight variant (x_q reuse).
#ifndef FP8MM_SMALLM_XLDS_NT
#define FP8MM_SMALLM_XLDS_NT 1
#endif

// Persistent variant (one workgroup per CU walking its weight tiles): 1 = on.
#ifndef FP8MM_SMALLM_PERSIST
#define FP8MM_SMALLM_PERSIST 1
#endif

// Cache-policy bits of the streamed weight loads: 2 = nt (streamed once,
// non-temporal; measured faster than the default on every decode shape).
#ifndef FP8MM_SMALLM_CPOL
#define FP8MM_SMALLM_CPOL 2
#endif

// Ring kernel: row-balanced last round where whole tiles are badly
// unbalanced over the CUs (see k_gemm_small_m_ring): 1 = on.
#ifndef FP8MM_SMALLM_BAL
#define FP8MM_SMALLM_BAL 1
#endif

// Persistent variant with the weight staged through per-wave LDS rings: 1 = on.
#ifndef FP8MM_SMALLM_RING
#define FP8MM_SMALLM_RING 1
#endif

// Persistent variant: reduce every tile once, at the end (1), when the
// partials of all of a workgroup's tiles fit in LDS; else tile by tile.
#ifndef FP8MM_SMALLM_DEFER
#define FP8MM_SMALLM_DEFER 1
#endif

// s_waitcnt with only vmcnt constrained (expcnt = 7, lgkmcnt = 15: no wait);
// a compile-time count.
#define FP8MM_SM_VMCNT(n) ((((n) & 15) | ((((n) >> 4) & 3) << 14)) | (7 << 4) | (15 << 8))
// lgkmcnt(0) only (vmcnt = 63, expcnt = 7: no wait)
#define FP8MM_SM_LGKM0 (15 | (3 << 14) | (7 << 4))

namespace fp8mm {

namespace {

constexpr int kXldsMaxCpw = 8;   // weight chunks per wave held in registers
constexpr int kXldsNT = FP8MM_SMALLM_XLDS_NT;   // 16-row tiles per workgroup
constexpr int kChunk = 128;     // K bytes per MFMA (16x16x128)
constexpr int kMaxWaves = 16;
constexpr int kNT = FP8MM_SMALLM_NT;

__device__ __forceinline__ uint4 ld16_stream(const uint8_t* p)
{
#if FP8MM_SMALLM_NTLOAD
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
#else
    return *reinterpret_cast<const uint4*>(p);
#endif
}

// Branch-free masked 16-byte load: the address is always an in-bounds one (the
// caller passes a fallback), and invalid lanes get zeros through a select.  A
// conditional load would become a branch, after which the compiler waits for
// all outstanding loads -- serializing the stream.
__device__ __forceinline__ uint4 ld16_masked(const uint8_t* p, const uint8_t* safe, bool ok)
{
    const uint4 v = *reinterpret_cast<const uint4*>(ok ? p : safe);
    return ok ? v : make_uint4(0u, 0u, 0u, 0u);
}

__device__ __forceinline__ uint4 ld16_stream_masked(const uint8_t* p, const uint8_t* safe, bool ok)
{
    const uint4 v = ld16_stream(ok ? p : safe);
    return ok ? v : make_uint4(0u, 0u, 0u, 0u);
}

__device__ __forceinline__ v8i pack(const uint4 lo, const uint4 hi)
{
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

template <int MT, int B>
struct Frags {
    uint4 a[B][kNT][2];
    uint4 b[B][MT][2];
};

template <int MT, int B>
__device__ __forceinline__ void load_batch(Frags<MT, B>& f, int i0, int nc, int wave, int W, int g, int64_t K,
                                           const uint8_t* const (&wrow)[kNT], const bool (&wv)[kNT],
                                           const uint8_t* const (&xrow)[MT], const bool (&xv)[MT])
{
#pragma unroll
    for (int j = 0; j < B; ++j) {
        const int64_t c = (int64_t)wave + (int64_t)(i0 + j) * W;
        const int64_t k0 = c * kChunk + g * 16;          // this lane's two 16-byte pieces
        const bool cv = (i0 + j) < nc;
        const bool v0 = cv && k0 < K, v1 = cv && k0 + 64 < K;
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            f.a[j][t][0] = ld16_stream_masked(wrow[t] + k0, wrow[t], v0 && wv[t]);
            f.a[j][t][1] = ld16_stream_masked(wrow[t] + k0 + 64, wrow[t], v1 && wv[t]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f.b[j][mt][0] = ld16_masked(xrow[mt] + k0, xrow[mt], v0 && xv[mt]);
            f.b[j][mt][1] = ld16_masked(xrow[mt] + k0 + 64, xrow[mt], v1 && xv[mt]);
        }
    }
}

template <int MT, int B>
__device__ __forceinline__ void mfma_batch(const Frags<MT, B>& f, v4f (&acc)[kNT][MT])
{
#pragma unroll
    for (int j = 0; j < B; ++j)
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            const v8i A = pack(f.a[j][t][0], f.a[j][t][1]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[t][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    A, pack(f.b[j][mt][0], f.b[j][mt][1]), acc[t][mt], 0, 0, 0, 0, 0, 0);
        }
}

// Sum the W per-wave partials red[W][NTt][MT][64] in wave order (fixed, no
// atomics), apply the scales in fp32 and store bf16.  16x16 MFMA C layout:
// lane l holds rows 4*(l/16)+v (= n) of column l%16 (= m).
template <int MT, int NTt>
__device__ __forceinline__ void reduce_store(const v4f* red, int W, int64_t n0, float s_act,
                                             const float* __restrict__ s_w, const ShardTable& sh,
                                             int M, int64_t N)
{
    for (int idx = threadIdx.x; idx < NTt * MT * 64; idx += blockDim.x) {   // blocks may be narrower
        const int t = idx / (MT * 64), mt = (idx >> 6) % MT, l = idx & 63;
        const int64_t nt0 = n0 + 16 * t;
        const int m = mt * 16 + (l & 15);
        if (nt0 >= N || m >= M) continue;
        v4f s = red[(t * MT + mt) * 64 + l];
        for (int w = 1; w < W; ++w) {
            const v4f p = red[((w * NTt + t) * MT + mt) * 64 + l];
            s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
        }
        const int64_t n = nt0 + 4 * (l >> 4);
        const float4 sw = *reinterpret_cast<const float4*>(s_w + n);
        const float sa = row_scale(sh, m, s_act);
        store_out4(sh, shard_of(sh, nt0), m, n, (s.x * sa) * sw.x, (s.y * sa) * sw.y, (s.z * sa) * sw.z,
                   (s.w * sa) * sw.w);
    }
}

template <int MT>
__global__ __launch_bounds__(64 * kMaxWaves) void k_gemm_small_m(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ wq, float s_act,
    const float* __restrict__ s_w, ShardTable sh, int M, int64_t N, int64_t K, int nchunks)
{
    extern __shared__ v4f red[];                       // [W][kNT][MT][64]
    constexpr int B = FP8MM_SMALLM_BATCH / (MT * kNT) > 0 ? FP8MM_SMALLM_BATCH / (MT * kNT) : 1;
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * kNT);

    const uint8_t* wrow[kNT];
    bool wv[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
        wv[t] = n0 + 16 * t < N;                        // a ragged last workgroup may hold fewer tiles
        wrow[t] = wq + (wv[t] ? n0 + 16 * t + r : r) * K;
    }
    const uint8_t* xrow[MT];
    bool xv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r;
        xv[mt] = m < M;
        xrow[mt] = xq + (int64_t)(xv[mt] ? m : 0) * K;
    }

    v4f acc[kNT][MT];
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nc = (nchunks - wave + W - 1) / W;       // chunks owned by this wave
#if FP8MM_SMALLM_PIPE
    Frags<MT, B> cur;
    load_batch<MT, B>(cur, 0, nc, wave, W, g, K, wrow, wv, xrow, xv);
    for (int i0 = 0; i0 < nc; i0 += B) {
        Frags<MT, B> nxt;
        const bool more = i0 + B < nc;
        if (more) load_batch<MT, B>(nxt, i0 + B, nc, wave, W, g, K, wrow, wv, xrow, xv);
        mfma_batch<MT, B>(cur, acc);
        if (more) cur = nxt;
    }
#else
    for (int i0 = 0; i0 < nc; i0 += B) {
        Frags<MT, B> cur;
        load_batch<MT, B>(cur, i0, nc, wave, W, g, K, wrow, wv, xrow, xv);
        mfma_batch<MT, B>(cur, acc);
    }
#endif

    // Fixed-order reduction of the W per-wave partials.
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[((wave * kNT + t) * MT + mt) * 64 + lane] = acc[t][mt];
    __syncthreads();
    reduce_store<MT, kNT>(red, W, n0, s_act, s_w, sh, M, N);
}


// All-in-flight variant for M <= 16 and K % 1024 == 0 when x_q fits in LDS:
// every wave issues the loads of ALL its weight chunks at once (CPW x 2 x 16 B
// per lane, into registers); the workgroup then copies x_q[0:M, :] into LDS
// with direct global->LDS loads (no registers; rows padded to K + 16 bytes so
// the 16 fragment rows of an MFMA fall in distinct banks), waits once, and the
// MFMAs read their B fragments from LDS.  With every workgroup resident, the
// whole weight is requested up front, which is what a 50-200 MB stream needs
// to reach the HBM rate.  Same chunk assignment and reduction order as
// k_gemm_small_m, so both kernels give identical bits.
typedef __attribute__((address_space(3))) void lds_void;

template <int CPW, int NTX>
__global__ __launch_bounds__(64 * kMaxWaves) void k_gemm_small_m_xlds(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ wq, float s_act,
    const float* __restrict__ s_w, ShardTable sh, int M, int64_t N, int64_t K, int nchunks)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * NTX);
    const int64_t ldsx = K + 16;
    uint8_t* xs = smem;
    v4f* red = reinterpret_cast<v4f*>(smem + ((M * ldsx + 15) & ~(int64_t)15));

    // every weight chunk of this wave (for each of its NTX row tiles), all in flight
    const uint8_t* wrow[NTX];
    bool wok[NTX];
#pragma unroll
    for (int t = 0; t < NTX; ++t) {
        wok[t] = n0 + 16 * t < N;                          // a ragged last workgroup holds fewer tiles
        wrow[t] = wq + (wok[t] ? n0 + 16 * t + r : r) * K;
    }
    uint4 a[CPW][NTX][2];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int64_t c = (int64_t)wave + (int64_t)i * W;
        const int64_t k0 = c * kChunk + g * 16;
        const bool cv = c < nchunks;
#pragma unroll
        for (int t = 0; t < NTX; ++t) {
            a[i][t][0] = ld16_stream_masked(wrow[t] + k0, wrow[t], wok[t] && cv && k0 < K);
            a[i][t][1] = ld16_stream_masked(wrow[t] + k0 + 64, wrow[t], wok[t] && cv && k0 + 64 < K);
        }
    }
    // x_q -> LDS: each wave moves 64 consecutive 16-byte pieces (1 KB, inside
    // one row because K/16 is a multiple of 64) per instruction.
    const int64_t kp = K >> 4, np = (int64_t)M * kp;
    for (int64_t p0 = (int64_t)wave * 64; p0 < np; p0 += blockDim.x) {
        const int64_t row = p0 / kp, col0 = p0 - row * kp;
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(xq + (p0 + lane) * 16),
                                         (lds_void*)(xs + row * ldsx + col0 * 16), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);                      // all loads, weight and x_q, have landed
    __syncthreads();

    v4f acc[NTX];
#pragma unroll
    for (int t = 0; t < NTX; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    const bool xr = r < M;
    const uint8_t* xrow = xs + (xr ? r : 0) * ldsx;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int64_t c = (int64_t)wave + (int64_t)i * W;
        if (c >= nchunks) break;                          // wave-uniform
        const int64_t k0 = c * kChunk + g * 16;
        const v8i B = pack(ld16_masked(xrow + k0, xrow, xr && k0 < K), ld16_masked(xrow + k0 + 64, xrow, xr && k0 + 64 < K));
#pragma unroll
        for (int t = 0; t < NTX; ++t)
            acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pack(a[i][t][0], a[i][t][1]), B, acc[t],
                                                                     0, 0, 0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NTX; ++t) red[(wave * NTX + t) * 64 + lane] = acc[t];
    __syncthreads();
    reduce_store<1, NTX>(red, W, n0, s_act, s_w, sh, M, N);
}

// Persistent variant for M <= 16 and K % 1024 == 0 when x_q fits in LDS next
// to the reduction buffers: one workgroup per CU walks the 16-row weight
// tiles bid, bid + G, bid + 2G, ... (G workgroups).  x_q[0:M, :] is copied
// into LDS once per workgroup (not once per tile), and the weight loads of
// the next D tiles are always in flight: each wave keeps a ring of D tiles x
// CPW chunks of registers, refilling a slot as soon as its MFMAs have read
// it.  Weight loads are raw buffer loads over the whole weight; a chunk or
// tile that does not exist loads from an offset past the end of the buffer,
// which returns zeros without a memory access, so every wave issues the same
// instruction stream and the wait counts stay static.  The per-tile
// reduction of the W wave partials is the fixed-order one of the other two
// kernels (same chunk -> wave assignment), so all three give identical bits.
constexpr uint32_t kOob = 0x80000000u;   // > any weight byte offset served here (N*K < 2^31)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const uint8_t* p, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// The CPW chunks of one weight tile this wave owns: 2 x 16 bytes per lane and
// chunk ([16g, 16g+16) and [64+16g, 80+16g) of the chunk, row r of the tile).
template <int CPW>
__device__ __forceinline__ void issue_tile(u32x4_t (&a)[CPW][2], __amdgpu_buffer_rsrc_t rw, uint32_t tile_off,
                                           bool tile_ok, int wave, int W, int nchunks)
{
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int chunk = wave + c * W;
        const uint32_t v = (tile_ok && chunk < nchunks) ? tile_off + (uint32_t)chunk * kChunk : kOob;
        a[c][0] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)v, 0, 0);
        a[c][1] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(v + 64), 0, 0);
    }
}

// MFMAs of one tile; B fragments (x_q) from LDS.  A chunk past K reads the
// last real chunk of x_q (its weight fragment is zero, and x_q is finite
// there, so it adds exact zeros).
template <int CPW>
__device__ __forceinline__ v4f tile_mfma(const u32x4_t (&a)[CPW][2], const uint8_t* __restrict__ xrow, int wave,
                                         int W, int nchunks, int g)
{
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        int chunk = wave + c * W;
        chunk = chunk < nchunks ? chunk : nchunks - 1;
        const uint8_t* p = xrow + chunk * kChunk + g * 16;
        const uint4 b0 = *reinterpret_cast<const uint4*>(p), b1 = *reinterpret_cast<const uint4*>(p + 64);
        v8i A, B;
        A[0] = (int)a[c][0][0]; A[1] = (int)a[c][0][1]; A[2] = (int)a[c][0][2]; A[3] = (int)a[c][0][3];
        A[4] = (int)a[c][1][0]; A[5] = (int)a[c][1][1]; A[6] = (int)a[c][1][2]; A[7] = (int)a[c][1][3];
        B = pack(b0, b1);
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 0, 0, 0, 0, 0, 0);
    }
    return acc;
}

// Sum the W partials of one tile in wave order (partial of wave w for MFMA
// lane `lane` at red[w * stride + slot]), scale (weight scales in sw: n = n0 +
// 4*(lane/16) .. +3) and store bf16.  Rows n >= nend belong to another
// workgroup (or do not exist) and are not stored.  The shard is that of n0
// (one lookup for the tile: a tile starting at a multiple of 16 lies in one
// shard), or with lane_shard that of each 4-row group (such a group never
// straddles two shards: shard starts are multiples of 16).
__device__ __forceinline__ void reduce_tile(const v4f* red, int stride, int slot, int W, int64_t n0, int64_t nend,
                                            float s_act, const float4 sw, const ShardTable& sh, int M, int lane,
                                            bool lane_shard = false)
{
    const int m = lane & 15;
    const int64_t n = n0 + 4 * (lane >> 4);
    if (m >= M || n >= nend) return;
    v4f s = red[slot];
    for (int w = 1; w < W; ++w) {
        const v4f p = red[w * stride + slot];
        s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
    }
    const float sa = row_scale(sh, m, s_act);
    store_out4(sh, shard_of(sh, lane_shard ? n : n0), m, n, (s.x * sa) * sw.x, (s.y * sa) * sw.y, (s.z * sa) * sw.z,
               (s.w * sa) * sw.w);
}

template <int CPW, int D, int WMAX, bool DEFER>
__global__ __launch_bounds__(64 * WMAX) void k_gemm_small_m_persist(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ wq, float s_act,
    const float* __restrict__ s_w, ShardTable sh, int M, int64_t N, int64_t K, int nchunks)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int G = gridDim.x, bid = blockIdx.x;
    const int ntiles = (int)(N >> 4);
    const int my_tiles = (ntiles - bid + G - 1) / G;
    __builtin_assume(my_tiles >= 1);                    // G <= ntiles
    const int64_t ldsx = K + 16;
    uint8_t* xs = smem;
    // W partials: [2][W][64], or with DEFER [my_tiles][W][64] (reduced once, at the end)
    v4f* red = reinterpret_cast<v4f*>(smem + ((M * ldsx + 15) & ~(int64_t)15));
    const __amdgpu_buffer_rsrc_t rw = weight_rsrc(wq, N * K);
    const __amdgpu_buffer_rsrc_t rs = weight_rsrc(reinterpret_cast<const uint8_t*>(s_w), N * 4);
    const uint32_t lane_off = (uint32_t)(r * K + g * 16);
    auto tile_off = [&](int u) { return (uint32_t)((int64_t)(bid + u * G) * 16 * K) + lane_off; };
    // weight scales of tile u for this lane's four rows (zeros past the last tile)
    auto tile_sw = [&](int u) {
        const uint32_t o = u < my_tiles ? (uint32_t)((bid + u * G) * 64 + g * 16) : kOob;
        return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)o, 0, 0);
    };

    // x_q -> LDS first: each wave moves 64 consecutive 16-byte pieces (1 KB,
    // inside one row because K/16 is a multiple of 64) per instruction.
    const int64_t kp = K >> 4, np = (int64_t)M * kp;
    for (int64_t p0 = (int64_t)wave * 64; p0 < np; p0 += blockDim.x) {
        const int64_t row = p0 / kp, col0 = p0 - row * kp;
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(xq + (p0 + lane) * 16),
                                         (lds_void*)(xs + row * ldsx + col0 * 16), 16, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4_t a[D][CPW][2], sws[D];
#pragma unroll
    for (int s = 0; s < D; ++s) {
        issue_tile<CPW>(a[s], rw, tile_off(s), s < my_tiles, wave, W, nchunks);
        if constexpr (!DEFER) sws[s] = tile_sw(s);
    }
    __builtin_amdgcn_sched_barrier(0);
    // x_q landed: only the D tiles' weight (and scale) loads, issued after it,
    // may be in flight (for this wave; the barrier extends it to the workgroup)
    __builtin_amdgcn_s_waitcnt(FP8MM_SM_VMCNT(D * (2 * CPW + (DEFER ? 0 : 1))));
    __builtin_amdgcn_s_barrier();

    const uint8_t* xrow = xs + (r < M ? r : M - 1) * ldsx;
    for (int u0 = 0; u0 < my_tiles; u0 += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            const int u = u0 + s;
            if (u >= my_tiles) break;                    // workgroup-uniform
            const v4f acc = tile_mfma<CPW>(a[s], xrow, wave, W, nchunks, g);
            issue_tile<CPW>(a[s], rw, tile_off(u + D), u + D < my_tiles, wave, W, nchunks);
            if constexpr (DEFER) {
                red[(u * W + wave) * 64 + lane] = acc;
            } else {
                const u32x4_t swu = sws[s];
                sws[s] = tile_sw(u + D);
                v4f* rb = red + (u & 1) * W * 64;
                rb[wave * 64 + lane] = acc;
                __syncthreads();
                if (wave == 0)
                    reduce_tile(rb, 64, lane, W, (int64_t)(bid + u * G) * 16, N, s_act,
                                make_float4(__uint_as_float(swu[0]), __uint_as_float(swu[1]),
                                            __uint_as_float(swu[2]), __uint_as_float(swu[3])),
                                sh, M, lane);
            }
        }
    }
    if constexpr (DEFER) {                               // one barrier, then every wave reduces
        __syncthreads();
        for (int idx = threadIdx.x; idx < my_tiles * 64; idx += blockDim.x) {
            const int u = idx >> 6, l = idx & 63;
            const int64_t n0 = (int64_t)(bid + u * G) * 16;
            reduce_tile(red + u * W * 64, 64, l, W, n0, N, s_act,
                        *reinterpret_cast<const float4*>(s_w + n0 + 4 * (l >> 4)), sh, M, l);
        }
    }
}

// Weight staging through LDS for the persistent variant.  A weight load
// instruction in which each lane takes 16 bytes of a 16-row fragment in the
// MFMA operand layout (lane -> row) touches 16 half cache lines; one in which 8
// lanes cover a row's 128-byte chunk (8 rows per instruction) touches 8 whole
// lines, and the memory pipeline streams the latter markedly faster at decode
// sizes.  So each wave moves its chunks with whole-line direct-to-LDS loads
// into a private ring of S 2 KB slots and reads its A fragments back from
// there (no barrier: the wave that loads a slot is the only one reading it).
// Within a slot row n holds its 16-byte pieces XOR-swizzled by row (skipping
// one row bit), so the fragment reads are bank-conflict free.
__device__ __forceinline__ int wswz(int row, int piece) { return piece ^ ((row >> 1) & 7); }

// Chunk `chunk` of tile rows n0..n0+15 into an LDS slot: instruction i covers
// rows 8i..8i+7; lane -> row 8i + lane/8, physical piece lane%8.  `ok` false:
// an offset past the end of the buffer (zeros, no memory access).
__device__ __forceinline__ void dma_wchunk(__amdgpu_buffer_rsrc_t rw, uint8_t* slot, uint32_t row_off0,
                                           uint32_t row_off1, int chunk, bool ok)
{
    const uint32_t c = (uint32_t)chunk * kChunk;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)slot, 16, (int)(ok ? row_off0 + c : kOob), 0, 0,
                                             FP8MM_SMALLM_CPOL);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(slot + 1024), 16, (int)(ok ? row_off1 + c : kOob), 0,
                                             0, FP8MM_SMALLM_CPOL);
}

// The A fragment (row r, logical pieces g and g+4) of a staged chunk, and the
// matching B fragment of x_q.  Both pointers are restrict-qualified: these LDS
// reads never touch a slot with loads in flight (the explicit waits order
// them), which keeps the compiler from waiting for every outstanding load.
__device__ __forceinline__ v4f chunk_mfma(const uint8_t* __restrict__ slot, const uint8_t* __restrict__ xrow,
                                          int chunk, int r, int g, v4f acc)
{
    const uint8_t* ws = slot + r * kChunk;
    const v8i A = pack(*reinterpret_cast<const uint4*>(ws + wswz(r, g) * 16),
                       *reinterpret_cast<const uint4*>(ws + wswz(r, g + 4) * 16));
    const uint8_t* xp = xrow + chunk * kChunk + g * 16;
    const v8i B = pack(*reinterpret_cast<const uint4*>(xp), *reinterpret_cast<const uint4*>(xp + 64));
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 0, 0, 0, 0, 0, 0);
}

// Same, with the x_q chunk staged in the slot too (at +2048, rows swizzled
// like the weight's).  A missing chunk is all zeros in both operands.
__device__ __forceinline__ v4f chunk_mfma_x(const uint8_t* __restrict__ slot, int r, int g, int xr, v4f acc)
{
    const uint8_t* ws = slot + r * kChunk;
    const v8i A = pack(*reinterpret_cast<const uint4*>(ws + wswz(r, g) * 16),
                       *reinterpret_cast<const uint4*>(ws + wswz(r, g + 4) * 16));
    const uint8_t* xs = slot + 2048 + xr * kChunk;
    const v8i B = pack(*reinterpret_cast<const uint4*>(xs + wswz(xr, g) * 16),
                       *reinterpret_cast<const uint4*>(xs + wswz(xr, g + 4) * 16));
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 0, 0, 0, 0, 0, 0);
}

// BAL (row-balanced last round): taken where whole tiles would leave the
// busiest workgroup with much more weight than the average (e.g. N = 5120: 320
// tiles on 256 CUs, 2 against 1.25).  A workgroup then runs FR full rounds of
// 16-row tiles bid, bid + G, ... and a share of the rows left over, [R + q0,
// R + q1): their 4-row groups split evenly (+-1 group) over the G workgroups.
// Rows of that last tile past its end load as zeros and are not stored.  The
// chunk -> wave assignment and the reduction order do not change: the same
// bits.  Its refill offsets come from an incremental cursor, computed before
// the wait for the chunk whose slot they refill.
template <int S, bool DEFER, int XI, bool BAL>
__global__ __launch_bounds__(64 * kMaxWaves) void k_gemm_small_m_ring(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ wq, float s_act,
    const float* __restrict__ s_w, ShardTable sh, int M, int64_t N, int64_t K, int nchunks, int cpw)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int G = gridDim.x, bid = blockIdx.x;
    const int ntiles = (int)(N >> 4);
    const int FR = BAL ? ntiles / G : 0;                // >= 1 with BAL: G <= N / 16
    const int R = FR * G * 16, ngr = BAL ? ((int)N - R) >> 2 : 0;
    const int q0 = 4 * (int)((int64_t)ngr * bid / G), q1 = 4 * (int)((int64_t)ngr * (bid + 1) / G);
    const int my_tiles = BAL ? FR + (q1 > q0 ? 1 : 0) : (ntiles - bid + G - 1) / G;
    __builtin_assume(my_tiles >= 1);                    // G <= ntiles
    const int tiles_max = BAL ? FR + (ngr > 0 ? 1 : 0) : (ntiles + G - 1) / G;
    auto tile_rows = [&](int u, int& rt, int& re) {     // rows [rt, re) of tile u
        if (!BAL || u < FR) {
            rt = (bid + u * G) * 16;
            re = rt + 16;
        } else {
            rt = R + q0;
            re = R + q1;
        }
    };
    constexpr int SB = 2048 + 1024 * XI;                // ring slot: W chunk (+ x_q chunk)
    constexpr int LPC = 2 + XI;                          // direct-to-LDS loads per chunk
    const int64_t ldsx = K + 16;
    uint8_t* xs = smem;
    const int64_t xbytes = XI ? 0 : (M * ldsx + 15) & ~(int64_t)15;
    // W partials: [2][W][64], or with DEFER [tiles_max][W][mp] (reduced once, at
    // the end; for M <= 8 only the 32 lanes holding columns m < 8 are kept)
    const int mp = M <= 8 ? 32 : 64;
    const int pslot = mp == 64 ? lane : (lane >> 4) * 8 + (lane & 7);
    v4f* red = reinterpret_cast<v4f*>(smem + xbytes);
    uint8_t* ring = smem + xbytes + (DEFER ? (int64_t)tiles_max * W * mp : (int64_t)2 * W * 64) * sizeof(v4f) +
                    wave * S * SB;
    const __amdgpu_buffer_rsrc_t rw = weight_rsrc(wq, N * K);
    const __amdgpu_buffer_rsrc_t rx = weight_rsrc(xq, M * K);
    // this lane's two rows of a chunk (instruction i: row 8i + lane/8), logical piece
    const int lrow = lane >> 3;
    const uint32_t pieceoff0 = (uint32_t)(lrow * K + wswz(lrow, lane & 7) * 16);
    const uint32_t pieceoff1 = (uint32_t)((lrow + 8) * K + wswz(lrow + 8, lane & 7) * 16);
    // streamed x_q: rows past M repeat row M-1 (their columns are never stored)
    const int xr0 = lrow < M ? lrow : M - 1, xr1 = lrow + 8 < M ? lrow + 8 : M - 1;
    const uint32_t xoff0 = (uint32_t)(xr0 * K + wswz(lrow, lane & 7) * 16);
    const uint32_t xoff1 = (uint32_t)(xr1 * K + wswz(lrow + 8, lane & 7) * 16);
    const int total = my_tiles * cpw;                   // this wave's chunks, tile-major
    // BAL issue cursor: sequence position iq, its tile iu and chunk index ic,
    // and the rows [irt, ire) of tile iu.  prep() returns the buffer offsets of
    // the chunk at the cursor (past the buffer, i.e. zeros, where nothing is
    // loaded) and advances it; fire() issues those loads into a ring slot.
    int iq = 0, iu = 0, ic = 0, irt, ire;
    tile_rows(0, irt, ire);
    struct Pend {
        uint32_t w0, w1, x0, x1;
    };
    [[maybe_unused]] auto prep = [&]() {
        const int chunk = wave + ic * W;
        const bool ok = iq < total && chunk < nchunks;
        const uint32_t t0 = (uint32_t)((int64_t)irt * K) + (uint32_t)chunk * kChunk;
        const uint32_t cx = (uint32_t)chunk * kChunk;
        Pend pd;
        pd.w0 = ok && irt + lrow < ire ? t0 + pieceoff0 : kOob;
        pd.w1 = ok && irt + lrow + 8 < ire ? t0 + pieceoff1 : kOob;
        pd.x0 = ok ? xoff0 + cx : kOob;
        pd.x1 = ok ? xoff1 + cx : kOob;
        ++iq;
        if (++ic == cpw) {
            ic = 0;
            ++iu;
            tile_rows(iu, irt, ire);
        }
        return pd;
    };
    [[maybe_unused]] auto fire = [&](const Pend& pd, int slot) {
        uint8_t* sl = ring + slot * SB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)sl, 16, (int)pd.w0, 0, 0, FP8MM_SMALLM_CPOL);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(sl + 1024), 16, (int)pd.w1, 0, 0, FP8MM_SMALLM_CPOL);
        if (XI >= 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(sl + 2048), 16, (int)pd.x0, 0, 0, 0);
        if (XI >= 2)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(sl + 3072), 16, (int)pd.x1, 0, 0, 0);
    };
    [[maybe_unused]] auto issue = [&](int j, int slot) {   // chunk j of the sequence into a ring slot (not BAL)
        const int u = j / cpw, c = j - u * cpw;
        const int chunk = wave + c * W;
        const bool ok = j < total && chunk < nchunks;
        const uint32_t t0 = (uint32_t)((int64_t)(bid + u * G) * 16 * K);
        uint8_t* sl = ring + slot * SB;
        dma_wchunk(rw, sl, t0 + pieceoff0, t0 + pieceoff1, chunk, ok);
        const uint32_t cx = (uint32_t)chunk * kChunk;
        if (XI >= 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(sl + 2048), 16, (int)(ok ? xoff0 + cx : kOob),
                                                     0, 0, 0);
        if (XI >= 2)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(sl + 3072), 16, (int)(ok ? xoff1 + cx : kOob),
                                                     0, 0, 0);
    };

    if (XI == 0) {
        // x_q -> LDS first: each wave moves 64 consecutive 16-byte pieces (1 KB,
        // inside one row because K/16 is a multiple of 64) per instruction.
        const int64_t kp = K >> 4, np = (int64_t)M * kp;
        for (int64_t p0 = (int64_t)wave * 64; p0 < np; p0 += blockDim.x) {
            const int64_t row = p0 / kp, col0 = p0 - row * kp;
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(xq + (p0 + lane) * 16),
                                             (lds_void*)(xs + row * ldsx + col0 * 16), 16, 0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < S; ++s) {
        if constexpr (BAL) fire(prep(), s);
        else issue(s, s);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (XI == 0) {
        // x_q landed: only the S chunks issued after it may be in flight (for
        // this wave; the barrier extends it to the workgroup)
        __builtin_amdgcn_s_waitcnt(FP8MM_SM_VMCNT(LPC * S));
        __builtin_amdgcn_s_barrier();
    }

    const uint8_t* xrow = xs + (r < M ? r : M - 1) * ldsx;
    const int xsr = XI == 1 ? (r < 8 ? r : 7) : r;      // streamed x_q: row of the slot's x part
    // weight scales of tile u for this lane's four rows (tile-by-tile reduction only)
    const __amdgpu_buffer_rsrc_t rs = weight_rsrc(reinterpret_cast<const uint8_t*>(s_w), N * 4);
    auto tile_sw = [&](int t) {
        int rt, re;
        tile_rows(t, rt, re);
        const int n = rt + 4 * g;
        const uint32_t o = t < my_tiles && n < re ? (uint32_t)n * 4 : kOob;
        return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)o, 0, 0);
    };
    u32x4_t swu{0u, 0u, 0u, 0u};
    if constexpr (!DEFER) swu = tile_sw(0);
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    int u = 0, c = 0;                                   // tile and chunk of sequence position j
    for (int j0 = 0; j0 < total; j0 += S) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int j = j0 + s;
            if (j >= total) break;                       // wave-uniform
            [[maybe_unused]] Pend refill;
            if constexpr (BAL) refill = prep();          // chunk j + S, into this slot once it is read
            // chunk j landed: only the S-1 chunks after it may be in flight
            __builtin_amdgcn_s_waitcnt(FP8MM_SM_VMCNT(LPC * (S - 1)));
            if (XI == 0) {
                int chunk = wave + c * W;
                chunk = chunk < nchunks ? chunk : nchunks - 1;   // (a zero slot: adds exact zeros)
                acc = chunk_mfma(ring + s * SB, xrow, chunk, r, g, acc);
            } else {
                acc = chunk_mfma_x(ring + s * SB, r, g, xsr, acc);
            }
            __builtin_amdgcn_s_waitcnt(FP8MM_SM_LGKM0);  // the slot's reads have returned
            if constexpr (BAL) fire(refill, s);
            else issue(j + S, s);
            if (++c == cpw) {                            // tile u complete
                if constexpr (DEFER) {
                    if (mp == 64 || (lane & 15) < 8) red[(u * W + wave) * mp + pslot] = acc;
                } else {
                    v4f* rb = red + (u & 1) * W * 64;
                    rb[wave * 64 + lane] = acc;
                    __syncthreads();
                    int rt, re;
                    tile_rows(u, rt, re);
                    if (wave == 0)
                        reduce_tile(rb, 64, lane, W, rt, re, s_act,
                                    make_float4(__uint_as_float(swu[0]), __uint_as_float(swu[1]),
                                                __uint_as_float(swu[2]), __uint_as_float(swu[3])),
                                    sh, M, lane, BAL && u >= FR);
                    swu = tile_sw(u + 1);                // scales of the next tile
                }
                acc = v4f{0.f, 0.f, 0.f, 0.f};
                c = 0;
                ++u;
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);                      // no direct-to-LDS load outlives the workgroup
    if constexpr (DEFER) {                               // one barrier, then every wave reduces
        __syncthreads();
        for (int idx = threadIdx.x; idx < my_tiles * mp; idx += blockDim.x) {
            const int uu = idx / mp, ps = idx - uu * mp;
            const int l = mp == 64 ? ps : (ps >> 3) * 16 + (ps & 7);
            int n0, re;
            tile_rows(uu, n0, re);
            if (n0 + 4 * (l >> 4) >= re) continue;       // another workgroup's rows
            reduce_tile(red + uu * W * mp, mp, ps, W, n0, re, s_act,
                        *reinterpret_cast<const float4*>(s_w + n0 + 4 * (l >> 4)), sh, M, l, BAL);
        }
    }
}

// Waves per workgroup: a function of K only (it fixes the summation order).
int small_m_waves(int64_t K)
{
    const int64_t nchunks = (K + kChunk - 1) / kChunk;
    int64_t w = (nchunks + FP8MM_SMALLM_CPW - 1) / FP8MM_SMALLM_CPW;
    if (w < 1) w = 1;
    if (w > kMaxWaves) w = kMaxWaves;
    return (int)w;
}

}  // namespace

// The reduction buffer can exceed the default 64 KB dynamic-LDS limit (W = 16
// waves x 4 M tiles x NT tiles); allow up to the 160 KB a gfx950 CU has.
template <int MT>
void allow_large_lds()
{
    static const bool done = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_small_m<MT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        return true;
    }();
    (void)done;
}

// LDS bytes of the all-in-flight variant, or 0 if it does not apply.
size_t xlds_bytes(int64_t M, int64_t K, int W)
{
    if (M > 16 || K % 1024 != 0 || K > (int64_t)kChunk * kXldsMaxCpw * W) return 0;
    const size_t b = (size_t)((M * (K + 16) + 15) & ~(int64_t)15) + (size_t)W * kXldsNT * 64 * sizeof(v4f);
    return b <= (size_t)FP8MM_SMALLM_XLDS_MAX ? b : 0;
}

template <int CPW>
void launch_xlds(const dim3& grid, const dim3& block, size_t lds, hipStream_t stream, const uint8_t* xq,
                 const uint8_t* wq, float s_act, const float* s_w, const ShardTable& sh, int M, int64_t N,
                 int64_t K, int nchunks)
{
    static const bool attr = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_small_m_xlds<CPW, kXldsNT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        return true;
    }();
    (void)attr;
    hipLaunchKernelGGL((k_gemm_small_m_xlds<CPW, kXldsNT>), grid, block, lds, stream, xq, wq, s_act, s_w, sh,
                       M, N, K, nchunks);
}

// LDS bytes of the persistent variant (x_q rows + reduction buffers for
// `tiles` tiles), or 0 if it does not apply.
size_t persist_bytes(int64_t M, int64_t N, int64_t K, int W, int64_t tiles)
{
    if (!FP8MM_SMALLM_PERSIST || M > 16 || K % 1024 != 0 || N * K >= ((int64_t)1 << 31)) return 0;
    const size_t b = (size_t)((M * (K + 16) + 15) & ~(int64_t)15) + (size_t)tiles * W * 64 * sizeof(v4f);
    return b <= (size_t)160 * 1024 ? b : 0;
}

template <int CPW, int D, int WMAX, bool DEFER>
void launch_persist(const dim3& grid, const dim3& block, size_t lds, hipStream_t stream, const uint8_t* xq,
                    const uint8_t* wq, float s_act, const float* s_w, const ShardTable& sh, int M, int64_t N,
                    int64_t K, int nchunks)
{
    static const bool attr = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_small_m_persist<CPW, D, WMAX, DEFER>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        return true;
    }();
    (void)attr;
    hipLaunchKernelGGL((k_gemm_small_m_persist<CPW, D, WMAX, DEFER>), grid, block, lds, stream, xq, wq, s_act, s_w, sh,
                       M, N, K, nchunks);
}

template <int S, bool DEFER, int XI, bool BAL>
void launch_ring(const dim3& grid, const dim3& block, size_t lds, hipStream_t stream, const uint8_t* xq,
                 const uint8_t* wq, float s_act, const float* s_w, const ShardTable& sh, int M, int64_t N, int64_t K,
                 int nchunks, int cpw)
{
    static const bool attr = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_small_m_ring<S, DEFER, XI, BAL>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        return true;
    }();
    (void)attr;
    hipLaunchKernelGGL((k_gemm_small_m_ring<S, DEFER, XI, BAL>), grid, block, lds, stream, xq, wq, s_act, s_w, sh, M, N, K,
                       nchunks, cpw);
}

// The LDS-ring persistent kernel, if it applies (M <= 16, K % 1024 == 0,
// x_q + partials + rings within 160 KB): deepest ring that fits, deferred
// reduction preferred.
bool try_ring(const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w, const ShardTable& sh,
              int64_t M, int64_t N, int64_t K, int W, int nchunks, hipStream_t stream)
{
    if (!FP8MM_SMALLM_RING || M > 16 || K % 1024 != 0 || N * K >= ((int64_t)1 << 31)) return false;
    const int64_t G = N / 16 < num_cus() ? N / 16 : num_cus();
    const int64_t tiles_max = (N / 16 + G - 1) / G;      // whole tiles, or FR + 1 with the balanced last round
    // Balanced last round when whole tiles leave the busiest workgroup at least
    // 1.3x the average weight bytes.
    const bool bal = FP8MM_SMALLM_BAL && 10 * tiles_max * G >= 13 * (N / 16);
    const size_t xb = (size_t)((M * (K + 16) + 15) & ~(int64_t)15);
    const size_t part = (size_t)W * 64 * sizeof(v4f);               // one tile's partials
    const size_t dpart = (size_t)W * (M <= 8 ? 32 : 64) * sizeof(v4f);   // ... as the deferred buffer keeps them
    const int cpw = (nchunks + W - 1) / W;
    const dim3 grid((uint32_t)G), block(64 * W);
    // x_q in LDS (XI = 0), else streamed with each chunk (1 KB for M <= 8, 2 KB for M <= 16)
    auto bytes = [&](int S, bool df, int xi) {
        return (xi ? 0 : xb) + (df ? tiles_max * dpart : 2 * part) + (size_t)W * S * (2048 + 1024 * xi);
    };
#define FP8MM_RING_TRY(S, DF, XI)                                                                      \
    if (bytes(S, DF, XI) <= 160 * 1024) {                                                              \
        if (bal)                                                                                       \
            launch_ring<S, DF, XI, true>(grid, block, bytes(S, DF, XI), stream, xq, wq, s_act, s_w, sh, (int)M, N, K, \
                                         nchunks, cpw);                                                \
        else                                                                                           \
            launch_ring<S, DF, XI, false>(grid, block, bytes(S, DF, XI), stream, xq, wq, s_act, s_w, sh, (int)M, N, K, \
                                          nchunks, cpw);                                               \
        return true;                                                                                   \
    }
    FP8MM_RING_TRY(6, true, 0)
    FP8MM_RING_TRY(5, true, 0)
    FP8MM_RING_TRY(6, false, 0)
    FP8MM_RING_TRY(4, true, 0)
    FP8MM_RING_TRY(4, false, 0)
    FP8MM_RING_TRY(3, false, 0)
    if (M <= 8) {
        FP8MM_RING_TRY(4, true, 1)
        FP8MM_RING_TRY(3, true, 1)
        FP8MM_RING_TRY(2, true, 1)
    } else {
        FP8MM_RING_TRY(3, true, 2)
        FP8MM_RING_TRY(2, true, 2)
    }
#undef FP8MM_RING_TRY
    return false;
}

void launch_gemm_small_m(const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w,
                         const ShardTable& shards, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    const int W = small_m_waves(K);
    const int nchunks = (int)((K + kChunk - 1) / kChunk);
    if (try_ring(xq, wq, s_act, s_w, shards, M, N, K, W, nchunks, stream)) return;
    const int64_t G = N / 16 < num_cus() ? N / 16 : num_cus();
    const int64_t tiles_max = (N / 16 + G - 1) / G;            // tiles of the busiest workgroup
    // (deferring needs registers too: only with up to 8 waves, 256 VGPRs each)
    const size_t pl_defer = FP8MM_SMALLM_DEFER && W <= 8 ? persist_bytes(M, N, K, W, tiles_max) : 0;
    const size_t pl = pl_defer ? pl_defer : persist_bytes(M, N, K, W, 2);
    const bool defer = pl_defer != 0;
    if (pl) {
        // Ring depth: as many tiles in flight as the registers allow (<= 3).
        // Up to 8 waves: 2 waves per SIMD, 256 VGPRs each; more: 4, 128 VGPRs.
        const int cpw = (nchunks + W - 1) / W;
        const dim3 grid((uint32_t)G), block(64 * W);
        const int budget = (W <= 8 ? 256 : 128) - 72;
        int d = budget / (cpw * 8);
        d = d < 1 ? 1 : (d > 3 ? 3 : d);
#define FP8MM_PERSIST_ARGS grid, block, pl, stream, xq, wq, s_act, s_w, shards, (int)M, N, K, nchunks
#define FP8MM_PERSIST_DISPATCH(C, DF)                                                         \
        if (W > 8) launch_persist<C, 1, 16, DF>(FP8MM_PERSIST_ARGS);                           \
        else if (d == 1) launch_persist<C, 1, 8, DF>(FP8MM_PERSIST_ARGS);                      \
        else if (d == 2) launch_persist<C, 2, 8, DF>(FP8MM_PERSIST_ARGS);                      \
        else launch_persist<C, 3, 8, DF>(FP8MM_PERSIST_ARGS);
#define FP8MM_PERSIST_CASE(C)                                                                 \
    case C:                                                                                   \
        if (defer) { FP8MM_PERSIST_DISPATCH(C, true) } else { FP8MM_PERSIST_DISPATCH(C, false) } \
        return;
        switch (cpw) {
            FP8MM_PERSIST_CASE(1)
            FP8MM_PERSIST_CASE(2)
            FP8MM_PERSIST_CASE(3)
            FP8MM_PERSIST_CASE(4)
            FP8MM_PERSIST_CASE(5)
            FP8MM_PERSIST_CASE(6)
            FP8MM_PERSIST_CASE(7)
            FP8MM_PERSIST_CASE(8)
            FP8MM_PERSIST_CASE(9)
        default: break;                                  // more chunks per wave: the kernels below
        }
#undef FP8MM_PERSIST_ARGS
#undef FP8MM_PERSIST_DISPATCH
#undef FP8MM_PERSIST_CASE
    }
    const size_t xl = xlds_bytes(M, K, W);
    if (xl) {
        const int cpw = (nchunks + W - 1) / W;
        const dim3 grid((uint32_t)((N + 16 * kXldsNT - 1) / (16 * kXldsNT))), block(64 * W);
        switch (cpw) {
        case 1: launch_xlds<1>(grid, block, xl, stream, xq, wq, s_act, s_w, shards, (int)M, N, K, nchunks); return;
        case 2: launch_xlds<2>(grid, block, xl, stream, xq, wq, s_act, s_w, shards, (int)M, N, K, nchunks); return;
        case 3: launch_xlds<3>(grid, block, xl, stream, xq, wq, s_act, s_w, shards, (int)M, N, K, nchunks); return;
        case 4: launch_xlds<4>(grid, block, xl, stream, xq, wq, s_act, s_w, shards, (int)M, N, K, nchunks); return;
        case 5: launch_xlds<5>(grid, block, xl, stream, xq, wq, s_act, s_w, shards, (int)M, N, K, nchunks); return;
        case 6: launch_xlds<6>(grid, block, xl, stream, xq, wq, s_act, s_w, shards, (int)M, N, K, nchunks); return;
        case 7: launch_xlds<7>(grid, block, xl, stream, xq, wq, s_act, s_w, shards, (int)M, N, K, nchunks); return;
        default: launch_xlds<8>(grid, block, xl, stream, xq, wq, s_act, s_w, shards, (int)M, N, K, nchunks); return;
        }
    }
    const int MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    const size_t lds = (size_t)W * kNT * MT * 64 * sizeof(v4f);
    const dim3 grid((uint32_t)((N + 16 * kNT - 1) / (16 * kNT))), block(64 * W);
    if (lds > 64 * 1024) {
        if (MT == 1) allow_large_lds<1>();
        else if (MT == 2) allow_large_lds<2>();
        else allow_large_lds<4>();
    }
    if (MT == 1)
        hipLaunchKernelGGL(k_gemm_small_m<1>, grid, block, lds, stream, xq, wq, s_act, s_w, shards, (int)M, N, K, nchunks);
    else if (MT == 2)
        hipLaunchKernelGGL(k_gemm_small_m<2>, grid, block, lds, stream, xq, wq, s_act, s_w, shards, (int)M, N, K, nchunks);
    else
        hipLaunchKernelGGL(k_gemm_small_m<4>, grid, block, lds, stream, xq, wq, s_act, s_w, shards, (int)M, N, K, nchunks);
}

}  // namespace fp8mm
