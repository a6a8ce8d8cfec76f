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
//  * a 16-row weight tile is reduced over K by W waves of one workgroup: K is
//    cut into 128-byte chunks and wave w takes chunks w, w+W, ... (W = a
//    function of K only);
//  * every weight byte feeds exactly one v_mfma_f32_16x16x128_f8f6f4, with
//    x_q as the B operand (M padded to 16; MT = 2 or 4 B tiles for M <= 32 /
//    64);
//  * the W per-wave partial sums are reduced in LDS in a fixed order (no
//    atomics, no workspace), then the scale epilogue and the store happen in
//    registers.
// Four kernels share that work split, so they give the same bits:
//  * k_gemm_small_m_pair (M <= 32, rows longer than 5 chunks per wave, at
//    most two tiles per workgroup): the two tiles' chunks in one slot (3 KB
//    when the second tile is a share of at most 8 rows), against fragments
//    streamed with each chunk, so x_q is read once per workgroup;
//  * k_gemm_small_m_rx (M <= 32, K % 128 == 0 with 4-5 chunks per wave, and
//    M 17-32 beyond): persistent, one workgroup per CU walking its weight
//    tiles; each wave streams its weight chunks with whole-line direct-to-LDS
//    loads into a private ring of LDS slots and keeps its x_q B fragments in
//    registers (loaded once, or with each chunk); for M <= 8 it can also
//    quantize the bf16 activation itself (the static or the fused RMSNorm
//    quant in its launch), and on an interleaved gate_up weight it can end
//    with the SiLU*mul -> E4M3 quant instead of the bf16 store;
//  * k_gemm_small_m_ring (M <= 16, K % 1024 == 0, the longer rows): the same
//    stream, with x_q staged in LDS once (or streamed with each chunk when it
//    does not fit);
//  * k_gemm_small_m (anything else up to M = 64): one workgroup per tile, the
//    fragments loaded straight into registers.
// W and the chunk assignment depend on K only, so every column's summation
// order is the same for a merged call and a per-shard call: bitwise identical.
#include "act_quant.h"
#include "act_tables.h"
#include "device_common.h"
#include "internal.h"
#include "out_store.h"

// s_waitcnt with only vmcnt constrained (expcnt = 7, lgkmcnt = 15: no wait);
// a compile-time count.
#define FP8MM_SM_VMCNT(n) ((((n) & 15) | ((((n) >> 4) & 3) << 14)) | (7 << 4) | (15 << 8))
// lgkmcnt(0) only (vmcnt = 63, expcnt = 7: no wait)
#define FP8MM_SM_LGKM0 (15 | (3 << 14) | (7 << 4))

namespace fp8mm {

namespace {

constexpr int kChunk = 128;     // K bytes per MFMA (16x16x128)
constexpr int kMaxWaves = 16;
constexpr int kCpw = 5;         // target 128-byte chunks per wave: fixes the waves per workgroup
constexpr int kBatch = 2;       // chunk fragments (x M tiles) in flight per wave, generic kernel
// Cache-policy bits of the streamed weight loads of the ring kernel: 2 = nt
// (non-temporal: the weight is read once; measured faster than the default on
// every decode shape).
constexpr int kWeightCpol = 2;

// Branch-free masked 16-byte load: the address is always an in-bounds one (the
// caller passes a fallback), and invalid lanes get zeros through a select.  A
// conditional load would become a branch, after which the compiler waits for
// all outstanding loads -- serializing the stream.
__device__ __forceinline__ uint4 ld16_masked(const uint8_t* p, const uint8_t* safe, bool ok)
{
    const uint4 v = *reinterpret_cast<const uint4*>(ok ? p : safe);
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
    uint4 a[B][2];
    uint4 b[B][MT][2];
};

// Chunks i0 .. i0+B-1 of this wave (chunk c = wave + i W): the weight row's
// and the MT x_q rows' two 16-byte pieces each, zeros where a chunk, row or
// piece does not exist.
template <int MT, int B>
__device__ __forceinline__ void load_batch(Frags<MT, B>& f, int i0, int nc, int wave, int W, int g, int64_t K,
                                           const uint8_t* wrow, bool wv, const uint8_t* const (&xrow)[MT],
                                           const bool (&xv)[MT])
{
#pragma unroll
    for (int j = 0; j < B; ++j) {
        const int64_t c = (int64_t)wave + (int64_t)(i0 + j) * W;
        const int64_t k0 = c * kChunk + g * 16;          // this lane's two 16-byte pieces
        const bool cv = (i0 + j) < nc;
        const bool v0 = cv && k0 < K, v1 = cv && k0 + 64 < K;
        f.a[j][0] = ld16_masked(wrow + k0, wrow, v0 && wv);
        f.a[j][1] = ld16_masked(wrow + k0 + 64, wrow, v1 && wv);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f.b[j][mt][0] = ld16_masked(xrow[mt] + k0, xrow[mt], v0 && xv[mt]);
            f.b[j][mt][1] = ld16_masked(xrow[mt] + k0 + 64, xrow[mt], v1 && xv[mt]);
        }
    }
}

template <int MT, int B>
__device__ __forceinline__ void mfma_batch(const Frags<MT, B>& f, v4f (&acc)[MT])
{
#pragma unroll
    for (int j = 0; j < B; ++j) {
        const v8i A = pack(f.a[j][0], f.a[j][1]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, pack(f.b[j][mt][0], f.b[j][mt][1]), acc[mt],
                                                                      0, 0, 0, 0, 0, 0);
    }
}

// Sum the W per-wave partials red[W][MT][64] in wave order (fixed, no
// atomics), apply the scales in fp32 and store.  16x16 MFMA C layout: lane l
// holds rows 4*(l/16)+v (= n) of column l%16 (= m).
template <int MT>
__device__ __forceinline__ void reduce_store(const v4f* red, int W, int64_t n0, float s_act,
                                             const float* __restrict__ s_w, const ShardTable& sh, int M, int64_t N)
{
    for (int idx = threadIdx.x; idx < MT * 64; idx += blockDim.x) {   // blocks may be narrower
        const int mt = idx >> 6, l = idx & 63;
        const int m = mt * 16 + (l & 15);
        if (n0 >= N || m >= M) continue;
        v4f s = red[mt * 64 + l];
        for (int w = 1; w < W; ++w) {
            const v4f p = red[(w * MT + mt) * 64 + l];
            s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
        }
        const int64_t n = n0 + 4 * (l >> 4);
        const float4 sw = *reinterpret_cast<const float4*>(s_w + n);
        const float sa = row_scale(sh, m, s_act);
        store_out4(sh, shard_of(sh, n0), m, n, (s.x * sa) * sw.x, (s.y * sa) * sw.y, (s.z * sa) * sw.z,
                   (s.w * sa) * sw.w);
    }
}

// Generic kernel (any M <= 64, any K % 16 == 0): one workgroup per 16-row
// weight tile, the weight and x_q fragments loaded straight into registers
// (MFMA operand layout), a batch of chunks ahead of the MFMAs.
template <int MT>
__global__ __launch_bounds__(64 * kMaxWaves) void k_gemm_small_m(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ wq, float s_act,
    const float* __restrict__ s_w, ShardTable sh, int M, int64_t N, int64_t K, int nchunks)
{
    extern __shared__ v4f red[];                       // [W][MT][64]
    constexpr int B = kBatch / MT > 0 ? kBatch / MT : 1;
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const bool wv = n0 < N;
    const uint8_t* wrow = wq + (wv ? n0 + r : r) * K;
    const uint8_t* xrow[MT];
    bool xv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r;
        xv[mt] = m < M;
        xrow[mt] = xq + (int64_t)(xv[mt] ? m : 0) * K;
    }

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nc = (nchunks - wave + W - 1) / W;       // chunks owned by this wave
    Frags<MT, B> cur;
    load_batch<MT, B>(cur, 0, nc, wave, W, g, K, wrow, wv, xrow, xv);
    for (int i0 = 0; i0 < nc; i0 += B) {
        Frags<MT, B> nxt;
        const bool more = i0 + B < nc;
        if (more) load_batch<MT, B>(nxt, i0 + B, nc, wave, W, g, K, wrow, wv, xrow, xv);
        mfma_batch<MT, B>(cur, acc);
        if (more) cur = nxt;
    }

    // Fixed-order reduction of the W per-wave partials.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * 64 + lane] = acc[mt];
    __syncthreads();
    reduce_store<MT>(red, W, n0, s_act, s_w, sh, M, N);
}

// Weight staging through LDS for the persistent ring kernel.  A weight load
// instruction in which each lane takes 16 bytes of a 16-row fragment in the
// MFMA operand layout (lane -> row) touches 16 half cache lines; one in which 8
// lanes cover a row's 128-byte chunk (8 rows per instruction) touches 8 whole
// lines, and the memory pipeline streams the latter markedly faster at decode
// sizes.  So each wave moves its chunks with whole-line direct-to-LDS loads
// into a private ring of S 2 KB slots and reads its A fragments back from
// there (no barrier: the wave that loads a slot is the only one reading it).
// Within a slot row n holds its 16-byte pieces XOR-swizzled by row (skipping
// one row bit), so the fragment reads are bank-conflict free.
typedef __attribute__((address_space(3))) void lds_void;

// A tile or chunk that does not exist loads from this offset, past the end of
// the buffer resource: zeros without a memory access (N*K < 2^31 here).
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const uint8_t* p, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Sum the W partials of one tile in wave order (partial of wave w for MFMA
// lane `lane` at red[w * stride + slot]), scale (weight scales in sw: n = n0 +
// 4*(lane/16) .. +3) and store.  Rows n >= nend belong to another workgroup
// (or do not exist) and are not stored.  The shard is that of n0 (one lookup
// for the tile: a tile starting at a multiple of 16 lies in one shard), or
// with lane_shard that of each 4-row group (such a group never straddles two
// shards: shard starts are multiples of 16).  m_off: the first output row of
// the MFMA B tile (16 for the second of two).  srl: the activation scales of
// the output rows in LDS, or null (per-tensor s_act, or sh's per-row scales
// read from memory).
__device__ __forceinline__ void reduce_tile(const v4f* __restrict__ red, int stride, int slot, int W, int64_t n0,
                                            int64_t nend,
                                            float s_act, const float4 sw, const ShardTable& sh, int M, int lane,
                                            bool lane_shard = false, int m_off = 0,
                                            const float* __restrict__ srl = nullptr)
{
    const int m = m_off + (lane & 15);
    const int64_t n = n0 + 4 * (lane >> 4);
    if (m >= M || n >= nend) return;
    v4f s = red[slot];
    for (int w = 1; w < W; ++w) {
        const v4f p = red[w * stride + slot];
        s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
    }
    const float sa = srl ? srl[m] : row_scale(sh, m, s_act);
    store_out4_any(sh, lane_shard ? n : n0, m, n, (s.x * sa) * sw.x, (s.y * sa) * sw.y, (s.z * sa) * sw.z,
                   (s.w * sa) * sw.w);
}

__device__ __forceinline__ int wswz(int row, int piece) { return piece ^ ((row >> 1) & 7); }

// The weight scales of rows n..n+3 through the buffer resource of s_w (a
// buffer load, which the compiler cannot fold with an LDS read of the same
// values into one flat load).
__device__ __forceinline__ float4 tile_scales(__amdgpu_buffer_rsrc_t rs, int n)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, n * 4, 0, 0);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

// Chunk `chunk` of tile rows n0..n0+15 into an LDS slot: instruction i covers
// rows 8i..8i+7; lane -> row 8i + lane/8, physical piece lane%8.  `ok` false:
// an offset past the end of the buffer (zeros, no memory access).
__device__ __forceinline__ void dma_wchunk(__amdgpu_buffer_rsrc_t rw, uint8_t* slot, uint32_t row_off0,
                                           uint32_t row_off1, int chunk, bool ok)
{
    const uint32_t c = (uint32_t)chunk * kChunk;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)slot, 16, (int)(ok ? row_off0 + c : kOob), 0, 0,
                                             kWeightCpol);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(slot + 1024), 16, (int)(ok ? row_off1 + c : kOob), 0,
                                             0, kWeightCpol);
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
    const float* __restrict__ s_w, ShardTable sh, int M, int64_t N, int64_t K, int nchunks, int cpw, int sw_lds)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int G = gridDim.x, bid = blockIdx.x;
    const int ntiles = (int)(N >> 4);
    const int FR = BAL ? ntiles / G : 0;                // >= 1 with BAL: G <= N / 16
    const int R = FR * G * 16, ngr = BAL ? ((int)N - R) >> 2 : 0;
    // 32-bit: ngr (bid + 1) <= (N / 4) G < 2^30 (N < 2^24: N K < 2^31 here; G <= 256 CUs)
    const int q0 = 4 * (int)((uint32_t)ngr * (uint32_t)bid / (uint32_t)G),
              q1 = 4 * (int)((uint32_t)ngr * (uint32_t)(bid + 1) / (uint32_t)G);
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
    uint8_t* ring0 = smem + xbytes + (DEFER ? (int64_t)tiles_max * W * mp : (int64_t)2 * W * 64) * sizeof(v4f);
    uint8_t* ring = ring0 + wave * S * SB;
    float* swl = reinterpret_cast<float*>(ring0 + W * S * SB);   // DEFER, sw_lds: the tiles' weight scales
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
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)sl, 16, (int)pd.w0, 0, 0, kWeightCpol);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(sl + 1024), 16, (int)pd.w1, 0, 0, kWeightCpol);
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

    const __amdgpu_buffer_rsrc_t rs = weight_rsrc(reinterpret_cast<const uint8_t*>(s_w), N * 4);
    if (DEFER && sw_lds) {
        // The weight scales of this workgroup's tiles into LDS, 16 per tile
        // (zeros past a tile's rows), ahead of everything else: the final
        // reduction reads them from LDS instead of waiting on memory (where
        // the LDS has room for them).
        for (int t0 = 4 * wave; t0 < tiles_max; t0 += 4 * W) {
            const int t = t0 + (lane >> 4);
            int rt, re;
            tile_rows(t, rt, re);
            const int n = rt + (lane & 15);
            const uint32_t o = t < my_tiles && n < re ? (uint32_t)n * 4 : kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(swl + t0 * 16), 4, (int)o, 0, 0, 0);
        }
    }
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
            const float4 sw4 = sw_lds ? *reinterpret_cast<const float4*>(swl + uu * 16 + 4 * (l >> 4))
                                      : tile_scales(rs, n0 + 4 * (l >> 4));
            reduce_tile(red + uu * W * mp, mp, ps, W, n0, re, s_act, sw4, sh, M, l, BAL);
        }
    }
}

// ---------------------------------------------------------------------------
// k_gemm_small_m_rx: the ring kernel's weight stream with the x_q B fragments
// in registers.
//
// A wave works on the same chunks (w, w + W, ...) of every weight tile, so it
// multiplies every tile by the same B fragments.  XM_RES loads them once,
// before the weight stream starts, and keeps them in registers (CPW chunks x
// MT B tiles x 8 VGPRs), so all of the LDS holds weight rings and partial
// sums.  Where they would not fit (more than 5 chunks per wave, e.g. K =
// 17408), XM_STREAM loads each chunk's fragments from L2 (x_q is at most 32 x
// K bytes) together with that chunk's weight, into a register ring as deep as
// the weight ring.
// MT = 1 or 2 B tiles (M <= 16 or M <= 32).  The chunk -> wave assignment (W
// depends on K only), the MFMA sequence and the fixed-order reduction are
// those of the other kernels of this file, so for a given M every kernel
// choice gives the same bits.
// XM_LDS (M <= 16): the resident fragments come through LDS: per chunk one
// 1 KB direct-to-LDS load per 8 x_q rows (8 rows at M <= 8, else 16) issued
// before the weight stream, read into registers once the first chunk has
// landed.  Register loads issued before the stream made the compiler wait
// for every outstanding load (the whole first ring fill) before the first
// chunk.
// XM_QLDS (M <= 8): XM_LDS with the fragments quantized in the kernel from the
// bf16 activation (the static quant fused into the GEMM launch): each wave
// loads the bf16 values of its own chunks interleaved with the ring fill, one
// chunk ahead of the weights (activation c + 1 before weight chunk c), and
// encodes each chunk inside the fill, where issuing stalls on the full memory
// pipe anyway: quotients by multiply and fused multiply-add, codes by the
// hardware conversion, no table and no barrier.  Each wave stages its own
// codes in LDS (read back by the same wave only); workgroup 0 also stores them
// (x_q).
// XM_QRMS (M <= 8, 8 waves: K of 4608..5120): XM_QLDS for the fused RMSNorm
// quant.  r of each row takes the standalone kernel's summation order: its
// thread t holds pieces t, t + 256, ... (8 values each), which are all in one
// lane here (chunk c's pieces 16c .. 16c + 15 sit in wave c % 8, and 256
// pieces are 16 chunks apart), so each lane sums its 4 threads' squares,
// stages them in LDS (one barrier), and wave m does row m's 4 xor butterflies
// and adds the 4 sums in order (a second barrier) before any chunk is encoded.
constexpr int XM_RES = 0, XM_STREAM = 1, XM_LDS = 2, XM_QLDS = 3, XM_QRMS = 4;

// The bf16 activation of a fused quant + GEMM launch (XM_QLDS): rows of ldx
// elements, and where workgroup 0 stores its E4M3 codes ([M, K], contiguous).
// rcp = fl32(1 / s_act), sat = fl32(448 s_act): the quotient's operands;
// gamma (bf16 [K]) and eps for XM_QRMS.
struct XSrc {
    const uint16_t* x;
    int64_t ldx;
    uint8_t* xq_out;
    float rcp, sat;
    const uint16_t* gamma;
    float eps;
};

// The SiLU*mul -> E4M3 epilogue of a gate_up launch.  The weight rows come
// interleaved: 16-row tile t holds gate rows 8t .. 8t + 7, then the up rows of
// the same 8 columns.  Instead of the bf16 gate_up output the kernel stores
// h_q[m, j] = E4M3 code of fl32(h / s) for h = bf16(fl32(silu(g) u)), with g
// and u the bf16 values the gate_up output would hold: E4M3 [M, I],
// contiguous.  rcp = fl32(1 / s), sat = fl32(448 s).
struct SiluOut {
    uint8_t* hq;
    int64_t I;
    float s, rcp, sat;
};

// The 16 E4M3 codes of 16 bf16 values (words of a then b; value i in bits
// 16 (i % 2) of word i / 2) under the plain static quant, four at a time by
// quant4_cvt (exact quotients, the hardware conversion, no table).
__device__ __forceinline__ uint4 quant16_div(uint4 a, uint4 b, float s, float rcp, float sat)
{
    return make_uint4(quant4_cvt(a.x, a.y, s, rcp, sat), quant4_cvt(a.z, a.w, s, rcp, sat),
                      quant4_cvt(b.x, b.y, s, rcp, sat), quant4_cvt(b.z, b.w, s, rcp, sat));
}


// The A fragment (row r, logical pieces g and g + 4) of a staged weight chunk.
// The pointer is restrict-qualified: this read never touches a slot with
// loads in flight (the explicit waits order it), which keeps the compiler from
// waiting for every outstanding direct-to-LDS load first.
__device__ __forceinline__ v8i slot_afrag(const uint8_t* __restrict__ slot, int r, int g)
{
    const uint8_t* ws = slot + r * kChunk;
    return pack(*reinterpret_cast<const uint4*>(ws + wswz(r, g) * 16),
                *reinterpret_cast<const uint4*>(ws + wswz(r, g + 4) * 16));
}

// The B fragment (x_q row `row`, pieces g and g + 4) of a chunk staged in LDS
// as 8 rows x 128 bytes (restrict, as slot_afrag).
__device__ __forceinline__ v8i lds_bfrag(const uint8_t* __restrict__ base, int row, int g)
{
    return pack(*reinterpret_cast<const uint4*>(base + row * kChunk + g * 16),
                *reinterpret_cast<const uint4*>(base + row * kChunk + (g + 4) * 16));
}

// Staged values of the fused RMSNorm's row sums (restrict: these LDS areas are
// never targets of the in-flight direct-to-LDS loads, so the compiler need not
// wait for them).
__device__ __forceinline__ void lds_put_f64(double* __restrict__ p, double v) { *p = v; }
__device__ __forceinline__ double lds_get_f64(const double* __restrict__ p) { return *p; }
__device__ __forceinline__ void lds_put_f32(float* __restrict__ p, float v) { *p = v; }
__device__ __forceinline__ float lds_get_f32(const float* __restrict__ p) { return *p; }

// 16 codes into the fragment staging area (restrict: this area is never a
// target of the in-flight direct-to-LDS loads).
__device__ __forceinline__ void put_codes(uint8_t* __restrict__ dst, uint4 q) { *reinterpret_cast<uint4*>(dst) = q; }

// Four weight scales staged in LDS (restrict, as slot_afrag).
__device__ __forceinline__ float4 lds_f4(const float* __restrict__ p) { return *reinterpret_cast<const float4*>(p); }

// B fragments of chunk `chunk` for the MT B tiles (rows mt*16 + r, bytes 16g
// and 64 + 16g of the chunk); zeros for rows past M or a chunk that does not
// exist (an offset past the end of the buffer).
template <int MT>
__device__ __forceinline__ void load_bfrag(v8i (&b)[MT], __amdgpu_buffer_rsrc_t rx, int chunk, bool cok, int r, int g,
                                           int M, int64_t K)
{
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r;
        const uint32_t o = cok && m < M ? (uint32_t)((int64_t)m * K + chunk * kChunk + g * 16) : kOob;
        const u32x4_t lo = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)o, 0, 0);
        const u32x4_t hi = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(o + 64), 0, 0);
        b[mt] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
}

// reduce_tile for the SiLU*mul epilogue (a whole tile of the interleaved
// gate_up weight, activation scales in LDS): every lane sums its W partials
// in wave order, scales its 4 columns and rounds them to bf16 as the gate_up
// output would hold them.  Lanes l and l + 32 hold the gate and the up values
// of the same 4 columns of one row and swap them; lane l < 32 then takes
// columns 0, 1 and lane l + 32 columns 2, 3, and where the B tile has at most
// 8 live rows (lanes with l % 16 >= 8 idle) a second swap leaves one column
// per lane.  Each column: h = bf16(fl32(silu(g) u)) with silu in fp64, as in
// the standalone SiLU*mul kernel, and its E4M3 code under so.s.  Every lane
// takes part in the swaps.
__device__ __forceinline__ void reduce_tile_silu(const v4f* __restrict__ red, int stride, int slot, int W, int64_t n0,
                                                 const float4 sw, int M, int lane, int m_off,
                                                 const float* __restrict__ srl, const SiluOut& so)
{
    const int r = lane & 15;
    v4f s = red[slot];
    for (int w = 1; w < W; ++w) {
        const v4f p = red[w * stride + slot];
        s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
    }
    const float sa = srl[m_off + r];
    const uint32_t v0 = f32_to_bf16_rne((s.x * sa) * sw.x) | (f32_to_bf16_rne((s.y * sa) * sw.y) << 16);
    const uint32_t v1 = f32_to_bf16_rne((s.z * sa) * sw.z) | (f32_to_bf16_rne((s.w * sa) * sw.w) << 16);
    const uint32_t o0 = (uint32_t)__shfl_xor((int)v0, 32, 64), o1 = (uint32_t)__shfl_xor((int)v1, 32, 64);
    const bool hi = lane >= 32;
    const uint32_t gw = hi ? o1 : v0, uw = hi ? v1 : o0;   // columns 2 hi, 2 hi + 1: gate, up
    // h_q column of this lane's first value
    const int64_t j = (n0 >> 1) + 4 * ((lane >> 4) & 1) + 2 * (hi ? 1 : 0);
    if (M - m_off <= 8) {
        // rows 0..7 only: lane l + 8 takes the second column of lane l's pair
        const uint32_t g2 = (uint32_t)__shfl_xor((int)gw, 8, 64), u2 = (uint32_t)__shfl_xor((int)uw, 8, 64);
        const bool second = (lane & 8) != 0;
        const int m = m_off + (lane & 7);
        if (m >= M) return;
        const uint32_t gb = second ? g2 >> 16 : gw & 0xffffu, ub = second ? u2 >> 16 : uw & 0xffffu;
        const uint32_t h = f32_to_bf16_rne(silu_f64(bf16_to_f32(gb)) * bf16_to_f32(ub));
        so.hq[(int64_t)m * so.I + j + (second ? 1 : 0)] = (uint8_t)quant2_cvt(h, so.s, so.rcp, so.sat);
    } else {
        const int m = m_off + r;
        if (m >= M) return;
        const uint32_t h = f32_to_bf16_rne(silu_f64(bf16_to_f32(gw & 0xffffu)) * bf16_to_f32(uw & 0xffffu)) |
                           (f32_to_bf16_rne(silu_f64(bf16_to_f32(gw >> 16)) * bf16_to_f32(uw >> 16)) << 16);
        *reinterpret_cast<uint16_t*>(so.hq + (int64_t)m * so.I + j) = (uint16_t)quant2_cvt(h, so.s, so.rcp, so.sat);
    }
}

// Workgroup barrier for LDS data written by the waves' own stores: wait for
// this wave's LDS stores (lgkmcnt), then s_barrier; the empty asm statements
// keep the compiler from moving memory accesses across it.  __syncthreads()
// (and any LDS fence) would also wait for every outstanding direct-to-LDS
// load, i.e. drain the weight ring.
__device__ __forceinline__ void lds_barrier()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(FP8MM_SM_LGKM0);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Partial sums of a finished tile into LDS (restrict: the partials area is
// never a target of the in-flight direct-to-LDS loads).
__device__ __forceinline__ void put_partial(v4f* __restrict__ dst, v4f v) { *dst = v; }

// (XM_QRMS and the SiLU*mul epilogue run at most 8 waves: the bound leaves
// each lane 256 registers, which the activation, gamma and fragments of 5
// chunks, or 2 B tiles' fragments and the epilogue's fp64 work, need.)
template <int S, int MT, int XM, int CPW, bool BAL, bool DEFER, bool SILU>
__global__ __launch_bounds__(XM == XM_QRMS || SILU ? 64 * 8 : 64 * kMaxWaves) void k_gemm_small_m_rx(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ wq, float s_act, const float* __restrict__ s_w,
    ShardTable sh, int M, int64_t N, int64_t K, int nchunks, int cpw, XSrc xs, SiluOut so)
{
    static_assert(XM == XM_STREAM || CPW > 0, "resident fragments need a compile-time chunk count");
    static_assert(!SILU || (!BAL && !DEFER), "the SiLU*mul epilogue: whole tiles, reduced one at a time");
    static_assert((XM != XM_LDS && XM != XM_QLDS && XM != XM_QRMS) || MT == 1, "fragments through LDS: M <= 16");
    constexpr bool kQ = XM == XM_QLDS || XM == XM_QRMS;   // the activation quantized in the kernel
    constexpr bool kLds = XM == XM_LDS || kQ;            // fragments staged in LDS
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int G = gridDim.x, bid = blockIdx.x;
    const int ntiles = (int)(N >> 4);
    const int FR = BAL ? ntiles / G : 0;                // >= 1 with BAL: G <= N / 16
    const int R = FR * G * 16, ngr = BAL ? ((int)N - R) >> 2 : 0;
    // 32-bit: ngr (bid + 1) <= (N / 4) G < 2^30 (N < 2^24: N K < 2^31 here; G <= 256 CUs)
    const int q0 = 4 * (int)((uint32_t)ngr * (uint32_t)bid / (uint32_t)G),
              q1 = 4 * (int)((uint32_t)ngr * (uint32_t)(bid + 1) / (uint32_t)G);
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
    const int cw = XM == XM_STREAM ? cpw : CPW;         // chunks per wave and tile
    // LDS: [partials] [W rings of S 2 KB slots] [XM_LDS: W x CPW chunks of xr x_q rows]
    // [activation scales of the 64 output rows] [weight scales of the
    // workgroup's tiles, 16 per tile].
    // partials: [2][W][MT][64], or with DEFER [tiles_max][W][MT][mp] (reduced
    // once, at the end; for M <= 8 only the 32 lanes holding columns m < 8).
    const int mp = MT == 1 && M <= 8 ? 32 : 64;
    const int pslot = mp == 64 ? lane : (lane >> 4) * 8 + (lane & 7);
    v4f* red = reinterpret_cast<v4f*>(smem);
    const int64_t red_elems = DEFER ? (int64_t)tiles_max * W * MT * mp : (int64_t)2 * W * MT * 64;
    uint8_t* ring = reinterpret_cast<uint8_t*>(red + red_elems) + wave * S * 2048;
    const int xr = M <= 8 ? 8 : 16;                     // XM_LDS, XM_QLDS (8): x_q rows staged per chunk
    uint8_t* bxl = reinterpret_cast<uint8_t*>(red + red_elems) + W * S * 2048;
    float* srl = reinterpret_cast<float*>(bxl + (kLds ? W * CPW * xr * kChunk : 0));
    float* swl = srl + 64;
    const __amdgpu_buffer_rsrc_t rw = weight_rsrc(wq, N * K);
    // this lane's two rows of a weight chunk (instruction i: row 8i + lane/8), logical piece
    const int lrow = lane >> 3;
    const uint32_t pieceoff0 = (uint32_t)(lrow * K + wswz(lrow, lane & 7) * 16);
    const uint32_t pieceoff1 = (uint32_t)((lrow + 8) * K + wswz(lrow + 8, lane & 7) * 16);
    const int total = my_tiles * cw;                    // this wave's chunks, tile-major
    // Issue cursor: sequence position iq, its tile iu and chunk index ic, and
    // the rows [irt, ire) of tile iu.  prep() returns the weight offsets of the
    // chunk at the cursor (past the buffer, i.e. zeros, where nothing is loaded)
    // and its chunk, and advances; fire() issues the weight loads into a slot.
    int iq = 0, iu = 0, ic = 0, irt, ire;
    tile_rows(0, irt, ire);
    struct Pend {
        uint32_t w0, w1;
        int chunk;
        bool ok;
    };
    auto prep = [&]() {
        const int chunk = wave + ic * W;
        const bool ok = iq < total && chunk < nchunks;
        const uint32_t t0 = (uint32_t)((int64_t)irt * K) + (uint32_t)chunk * kChunk;
        Pend pd;
        pd.w0 = ok && irt + lrow < ire ? t0 + pieceoff0 : kOob;
        pd.w1 = ok && irt + lrow + 8 < ire ? t0 + pieceoff1 : kOob;
        pd.chunk = chunk;
        pd.ok = ok;
        ++iq;
        if (++ic == cw) {
            ic = 0;
            ++iu;
            tile_rows(iu, irt, ire);
        }
        return pd;
    };
    auto fire = [&](const Pend& pd, int slot) {
        uint8_t* sl = ring + slot * 2048;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)sl, 16, (int)pd.w0, 0, 0, kWeightCpol);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(sl + 1024), 16, (int)pd.w1, 0, 0, kWeightCpol);
    };
    auto a_frag = [&](int slot) { return slot_afrag(ring + slot * 2048, r, g); };

    // XM_QLDS: this lane's bf16 values of each of the wave's chunks (x row
    // lane / 8, values 16 (lane % 8) .. + 15; zeros past M or past the last
    // chunk), loaded by load_xv inside the ring fill
    [[maybe_unused]] uint4 xv[kQ ? CPW : 1][2];
    [[maybe_unused]] const __amdgpu_buffer_rsrc_t rxb =
        weight_rsrc(reinterpret_cast<const uint8_t*>(xs.x), kQ ? ((int64_t)(M - 1) * xs.ldx + K) * 2 : 0);
    auto load_xv = [&](int c) {
        const int chunk = wave + c * W, xrow = lane >> 3;
        const uint32_t o = chunk < nchunks && xrow < M
                               ? (uint32_t)((xrow * xs.ldx + chunk * kChunk + (lane & 7) * 16) * 2) : kOob;
        const u32x4_t lo = __builtin_amdgcn_raw_buffer_load_b128(rxb, (int)o, 0, 0);
        const u32x4_t hi = __builtin_amdgcn_raw_buffer_load_b128(rxb, (int)(o + 16), 0, 0);
        xv[c][0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        xv[c][1] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    };
    // XM_QRMS: gamma of this lane's 16 columns of each chunk (the same for the
    // 8 rows), and each row's r (LDS, after the swl scales)
    [[maybe_unused]] uint4 gv[XM == XM_QRMS ? CPW : 1][2];
    [[maybe_unused]] const __amdgpu_buffer_rsrc_t rgb =
        weight_rsrc(reinterpret_cast<const uint8_t*>(xs.gamma), XM == XM_QRMS ? K * 2 : 0);
    auto load_g = [&](int c) {
        const int chunk = wave + c * W;
        const uint32_t o = chunk < nchunks ? (uint32_t)((chunk * kChunk + (lane & 7) * 16) * 2) : kOob;
        const u32x4_t lo = __builtin_amdgcn_raw_buffer_load_b128(rgb, (int)o, 0, 0);
        const u32x4_t hi = __builtin_amdgcn_raw_buffer_load_b128(rgb, (int)(o + 16), 0, 0);
        gv[c][0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        gv[c][1] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    };
    float* rrow = swl + (tiles_max + 3) / 4 * 64;       // XM_QRMS: r of rows 0..7

    const __amdgpu_buffer_rsrc_t rs = weight_rsrc(reinterpret_cast<const uint8_t*>(s_w), N * 4);
    // The activation scale of each output row into LDS: the per-row scales
    // with one direct-to-LDS load (wave 0), else s_act.  A global load of them
    // inside the stream would make the compiler drain the ring around it.
    if (sh.s_rows) {
        if (wave == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                weight_rsrc(reinterpret_cast<const uint8_t*>(sh.s_rows), (int64_t)M * 4), (lds_void*)srl, 4,
                lane < M ? lane * 4 : (int)kOob, 0, 0, 0);
    } else if (threadIdx.x < 64) {
        srl[threadIdx.x] = s_act;
    }
    {
        // The weight scales of this workgroup's tiles into LDS, 16 per tile
        // (zeros past a tile's rows), one 4-byte direct-to-LDS load per lane,
        // issued ahead of the stream: the reductions then read them from LDS
        // (a global load inside the stream made the compiler drain the ring
        // around it).
        for (int t0 = 4 * wave; t0 < tiles_max; t0 += 4 * W) {
            const int t = t0 + (lane >> 4);
            int rt, re;
            tile_rows(t, rt, re);
            const int n = rt + (lane & 15);
            const uint32_t o = t < my_tiles && n < re ? (uint32_t)n * 4 : kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(swl + t0 * 16), 4, (int)o, 0, 0, 0);
        }
    }
    constexpr int NB = XM == XM_STREAM ? S : CPW;
    v8i bx[NB][MT];
    const __amdgpu_buffer_rsrc_t rx = weight_rsrc(xq, (int64_t)M * K);
    if constexpr (XM == XM_RES) {
#pragma unroll
        for (int c = 0; c < CPW; ++c) load_bfrag<MT>(bx[c], rx, wave + c * W, wave + c * W < nchunks, r, g, M, K);
    } else if constexpr (XM == XM_LDS) {
        // chunk c of this wave, x_q rows 8h .. 8h + 7: lane -> row 8h + lane / 8, piece lane % 8
#pragma unroll
        for (int c = 0; c < CPW; ++c)
            for (int h = 0; h < xr / 8; ++h) {
                const int chunk = wave + c * W, xrow = 8 * h + (lane >> 3);
                const uint32_t o = chunk < nchunks && xrow < M
                                       ? (uint32_t)(xrow * K + chunk * kChunk + (lane & 7) * 16) : kOob;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (lds_void*)(bxl + (wave * CPW + c) * xr * kChunk + h * 1024), 16, (int)o, 0, 0, 0);
            }
    }
    // XM_QLDS: chunk c's codes into the wave's own staging area (read back
    // by the same wave only), then into its fragment; workgroup 0 also stores
    // them to x_q
    auto quant_chunk = [&](int c) {
        uint4 a = xv[c][0], b = xv[c][1];
        if constexpr (XM == XM_QRMS) {
            // y = bf16(fl32(fl32(x r) gamma)), the values the plain quant then takes
            const float rr = lds_get_f32(rrow + (lane >> 3));
            const uint32_t xw[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            const uint32_t gw[8] = {gv[c][0].x, gv[c][0].y, gv[c][0].z, gv[c][0].w,
                                    gv[c][1].x, gv[c][1].y, gv[c][1].z, gv[c][1].w};
            uint32_t yw[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                yw[i] = pack_bf16x2((bf16_to_f32(xw[i] & 0xffffu) * rr) * bf16_to_f32(gw[i] & 0xffffu),
                                    (bf16_to_f32(xw[i] >> 16) * rr) * bf16_to_f32(gw[i] >> 16));
            a = make_uint4(yw[0], yw[1], yw[2], yw[3]);
            b = make_uint4(yw[4], yw[5], yw[6], yw[7]);
        }
        const uint4 q = quant16_div(a, b, s_act, xs.rcp, xs.sat);
        put_codes(bxl + (wave * CPW + c) * 1024 + lane * 16, q);
        const int chunk = wave + c * W, xrow = lane >> 3;
        if (bid == 0 && xs.xq_out && chunk < nchunks && xrow < M)
            *reinterpret_cast<uint4*>(xs.xq_out + (int64_t)xrow * K + chunk * kChunk + (lane & 7) * 16) = q;
        __builtin_amdgcn_s_waitcnt(FP8MM_SM_LGKM0);
        bx[c][0] = lds_bfrag(bxl + (wave * CPW + c) * 1024, r & 7, g);
    };
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (XM == XM_QRMS) {
        // activation and gamma first, two ring slots, then r (two barriers),
        // then the rest of the fill with the chunks encoded between its slots
#pragma unroll
        for (int c = 0; c < CPW; ++c) load_xv(c);
#pragma unroll
        for (int c = 0; c < CPW; ++c) load_g(c);
        constexpr int S0 = S < 2 ? S : 2;
#pragma unroll
        for (int s = 0; s < S0; ++s) fire(prep(), s);
        __builtin_amdgcn_sched_barrier(0);              // every load above issued before the sums wait for any
        // this lane's 4 threads of the standalone order (W = 8): t = 16 (wave +
        // 8 gg) + 2 (lane % 8) + h holds the chunks at positions gg, gg + 2, ...
        double ss[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            ss[c & 1][0] = sumsq8(xv[c][0], ss[c & 1][0]);
            ss[c & 1][1] = sumsq8(xv[c][1], ss[c & 1][1]);
        }
        double* part = reinterpret_cast<double*>(bxl);  // [8 rows][256 threads], free until the encoding
#pragma unroll
        for (int gg = 0; gg < 2; ++gg)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                lds_put_f64(part + (lane >> 3) * kRmsRowThreads + 16 * (wave + 8 * gg) + 2 * (lane & 7) + h, ss[gg][h]);
        lds_barrier();
        if (wave < M) {
            double tot = 0.0;                            // the 4 wave sums in order, each an xor butterfly
#pragma unroll
            for (int k = 0; k < kRmsRowThreads / 64; ++k) {
                double v = lds_get_f64(part + wave * kRmsRowThreads + 64 * k + lane);
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
                tot += v;
            }
            if (lane == 0) lds_put_f32(rrow + wave, rms_inv(tot, K, xs.eps));
        } else if (lane == 0) {
            lds_put_f32(rrow + wave, 0.0f);              // rows past M: never kept
        }
        lds_barrier();
#pragma unroll
        for (int s = S0; s < S; ++s) {
            fire(prep(), s);
            if (s - S0 < CPW) {
                __builtin_amdgcn_sched_barrier(0);
                quant_chunk(s - S0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int c = S - S0; c < CPW; ++c) quant_chunk(c);
    } else if constexpr (XM == XM_QLDS) {
        // Issuing the fill stalls on a full memory pipe for microseconds:
        // chunk c is encoded there, two ring slots after its activation was
        // requested, instead of in the first tile (the weights have landed
        // by then, and the encoding would only add to the wait).
        if (M > 4) {
            // Past 4 rows the 32 workgroups of an XCD asking for the same
            // activation lines at once cost more than the interleaving saves:
            // every activation load goes first, the wave's chunks in an order
            // rotated by the workgroup's place within its XCD (workgroups go
            // round-robin over the 8 XCDs).  Each unrolled order keeps the
            // register indices compile-time constants.
            const int rot = (int)((blockIdx.x >> 3) % CPW);
#pragma unroll
            for (int rr = 0; rr < CPW; ++rr)
                if (rr == rot) {
#pragma unroll
                    for (int c = 0; c < CPW; ++c) load_xv((c + rr) % CPW);
                }
        } else {
            load_xv(0);
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
            if (M <= 4 && s + 1 < CPW) load_xv(s + 1);
            fire(prep(), s);
            if (s >= 2 && s - 2 < CPW) {
                __builtin_amdgcn_sched_barrier(0);
                quant_chunk(s - 2);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (M <= 4)
#pragma unroll
            for (int c = S + 1; c < CPW; ++c) load_xv(c);
#pragma unroll
        for (int c = S - 2 > 0 ? S - 2 : 0; c < CPW; ++c) quant_chunk(c);
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const Pend pd = prep();
            fire(pd, s);
            if constexpr (XM == XM_STREAM) load_bfrag<MT>(bx[s], rx, pd.chunk, pd.ok, r, g, M, K);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
    // end of tile u: keep its partials (DEFER) or reduce it now
    auto tile_done = [&](int u) {
        if constexpr (DEFER) {
            if (mp == 64 || (lane & 15) < 8)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) put_partial(red + ((u * W + wave) * MT + mt) * mp + pslot, acc[mt]);
        } else {
            v4f* rb = red + (u & 1) * W * MT * 64;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) put_partial(rb + (wave * MT + mt) * 64 + lane, acc[mt]);
            lds_barrier();
            int rt, re;
            tile_rows(u, rt, re);
            // the SiLU*mul epilogue's fp64 work goes round the waves, one tile each
            if (wave == (SILU ? u % W : 0)) {
                const float4 sw4 = lds_f4(swl + u * 16 + 4 * g);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if constexpr (SILU)
                        reduce_tile_silu(rb + mt * 64, MT * 64, lane, W, rt, sw4, M, lane, 16 * mt, srl, so);
                    else
                        reduce_tile(rb + mt * 64, MT * 64, lane, W, rt, re, s_act, sw4, sh, M, lane, BAL && u >= FR,
                                    16 * mt, srl);
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
    };

    if constexpr (XM == XM_LDS) {
        // the fragments landed (only the ring fill may be in flight); at
        // M <= 8 rows 8..15 of the B tile repeat rows 0..7 (their columns are
        // never kept)
        __builtin_amdgcn_s_waitcnt(FP8MM_SM_VMCNT(2 * S));
#pragma unroll
        for (int c = 0; c < CPW; ++c) bx[c][0] = lds_bfrag(bxl + (wave * CPW + c) * xr * kChunk, r & (xr - 1), g);
    }
    if constexpr (XM == XM_STREAM) {
        // Whole ring cycles: positions past `total` load zeros and add zeros, and
        // a tile past my_tiles is not kept (an early exit from the cycle would
        // join the loop's back edge with other load counts, and the compiler
        // would then wait for every outstanding load).  DEFER only.
        static_assert(XM != XM_STREAM || DEFER, "streamed fragments keep the scales out of the loop");
        int c = 0, u = 0;
        for (int j0 = 0; j0 < total; j0 += S) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const Pend nx = prep();                  // chunk j + S, into this slot once it is read
                // chunk j's weight and fragments landed: the S-1 chunks after it may be in flight
                __builtin_amdgcn_s_waitcnt(FP8MM_SM_VMCNT((2 + 2 * MT) * (S - 1)));
                const v8i A = a_frag(s);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, bx[s][mt], acc[mt], 0, 0, 0, 0, 0,
                                                                              0);
                __builtin_amdgcn_s_waitcnt(FP8MM_SM_LGKM0);   // the slot's reads have returned
                fire(nx, s);
                load_bfrag<MT>(bx[s], rx, nx.chunk, nx.ok, r, g, M, K);
                if (++c == cw) {
                    if (u < my_tiles) tile_done(u);
                    c = 0;
                    ++u;
                }
            }
        }
    } else {
        int slot = 0;
        auto tile_body = [&](int u) {
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                const Pend nx = prep();
                // chunk landed: only the S-1 chunks after it may be in flight
                __builtin_amdgcn_s_waitcnt(FP8MM_SM_VMCNT(2 * (S - 1)));
                const v8i A = a_frag(slot);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, bx[c][mt], acc[mt], 0, 0, 0, 0, 0,
                                                                              0);
                __builtin_amdgcn_s_waitcnt(FP8MM_SM_LGKM0);
                fire(nx, slot);
                slot = slot + 1 == S ? 0 : slot + 1;
            }
            tile_done(u);
        };
        // Register fragments: the first tile outside the loop.  Their first
        // uses are then straight-line code, where the compiler counts the
        // loads issued after them; at the head of a loop that uses them it
        // waited for every outstanding load (the whole first ring fill).
        int u0 = 0;
        if constexpr (XM == XM_RES) {
            tile_body(0);
            u0 = 1;
        }
        for (int u = u0; u < my_tiles; ++u) tile_body(u);
    }
    __builtin_amdgcn_s_waitcnt(0);                      // no load outlives the workgroup
    if constexpr (DEFER) {                               // one barrier, then every wave reduces
        __syncthreads();
        for (int idx = threadIdx.x; idx < my_tiles * MT * mp; idx += blockDim.x) {
            const int uu = idx / (MT * mp), rem = idx - uu * MT * mp;
            const int mt = rem / mp, ps = rem - mt * mp;
            const int l = mp == 64 ? ps : (ps >> 3) * 16 + (ps & 7);
            int n0, re;
            tile_rows(uu, n0, re);
            if (n0 + 4 * (l >> 4) >= re) continue;       // another workgroup's rows
            reduce_tile(red + (uu * W * MT + mt) * mp, MT * mp, ps, W, n0, re, s_act, lds_f4(swl + uu * 16 + 4 * (l >> 4)),
                        sh, M, l, BAL, 16 * mt, srl);
        }
    }
}

// Two-tile kernel for long rows (more chunks per wave than stay resident: the
// x_q fragments streamed from L2 with every chunk, MT B tiles of 16 rows) when
// no workgroup has more than two tiles: both tiles' weight chunks travel in
// one 4 KB ring slot and multiply the same fragments, so each workgroup reads
// x_q once instead of once per tile (the balanced last round gives every
// workgroup a whole tile and a few rows, and the fragments of those rows cost
// as much as a whole tile's).  Chunks, their order per wave, the MFMAs and the
// reduction are those of the other kernels: the same bits.  At the end each
// wave writes its partial sums into its own ring area (its loads have all
// landed) and the workgroup reduces them.
// SHORT (balanced, at most 8 rows in every workgroup's second tile): that
// tile's chunk takes 1 KB of the slot (rows 0..7, one load), so a slot is
// 3 KB and a third slot fits in LDS.  Its A fragment rows 8..15 then read
// whatever follows (the next slot, or the 1 KB of padding after the rings):
// they only reach output rows past the tile's end, which are never stored.
template <int S, int MT, bool BAL, bool SHORT>
__global__ __launch_bounds__(64 * kMaxWaves) void k_gemm_small_m_pair(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ wq, float s_act, const float* __restrict__ s_w,
    ShardTable sh, int M, int64_t N, int64_t K, int nchunks, int cpw)
{
    static_assert(!SHORT || BAL, "a short second tile is a balanced share");
    constexpr int SB = SHORT ? 3072 : 4096;             // slot bytes
    constexpr int NW = SHORT ? 3 : 4;                   // weight loads per position
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int W = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int G = gridDim.x, bid = blockIdx.x;
    const int ntiles = (int)(N >> 4);
    // tile 0: rows bid*16 .. (BAL: FR = 1 whole tile per workgroup); tile 1:
    // the balanced share of the leftover rows (BAL) or tile bid + G
    const int R = BAL ? G * 16 : 0, ngr = BAL ? ((int)N - R) >> 2 : 0;
    // 32-bit: ngr (bid + 1) <= (N / 4) G < 2^30 (N < 2^24: N K < 2^31 here; G <= 256 CUs)
    const int q0 = 4 * (int)((uint32_t)ngr * (uint32_t)bid / (uint32_t)G),
              q1 = 4 * (int)((uint32_t)ngr * (uint32_t)(bid + 1) / (uint32_t)G);
    int rt[2], re[2];
    rt[0] = bid * 16;
    re[0] = rt[0] + 16;
    if (BAL) {
        rt[1] = R + q0;
        re[1] = R + q1;
    } else {
        rt[1] = (bid + G) * 16;
        re[1] = bid + G < ntiles ? rt[1] + 16 : rt[1];
    }
    const int my_tiles = re[1] > rt[1] ? 2 : 1;
    // LDS: [W rings of S slots of SB bytes (two tiles' chunks); at the end each
    // wave's partial sums in its own ring area] [SHORT: 1 KB of padding]
    // [activation scales of 64 rows] [the two tiles' weight scales]
    uint8_t* ring = smem + wave * S * SB;
    float* srl = reinterpret_cast<float*>(smem + W * S * SB + (SHORT ? 1024 : 0));
    float* swl = srl + 64;
    const __amdgpu_buffer_rsrc_t rw = weight_rsrc(wq, N * K);
    const __amdgpu_buffer_rsrc_t rx = weight_rsrc(xq, (int64_t)M * K);
    const __amdgpu_buffer_rsrc_t rs = weight_rsrc(reinterpret_cast<const uint8_t*>(s_w), N * 4);
    if (sh.s_rows) {
        if (wave == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                weight_rsrc(reinterpret_cast<const uint8_t*>(sh.s_rows), (int64_t)M * 4), (lds_void*)srl, 4,
                lane < M ? lane * 4 : (int)kOob, 0, 0, 0);
    } else if (threadIdx.x < 64) {
        srl[threadIdx.x] = s_act;
    }
    if (wave == 0) {
        // the two tiles' 16 weight scales each (zeros past a tile's rows)
        const int t = lane >> 4, n = rt[t & 1] + (lane & 15);
        const uint32_t o = t < 2 && n < re[t & 1] ? (uint32_t)n * 4 : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)swl, 4, (int)o, 0, 0, 0);
    }
    // this lane's two rows of a tile's chunk (instruction i: row 8i + lane/8), logical piece
    const int lrow = lane >> 3;
    const uint32_t pieceoff0 = (uint32_t)(lrow * K + wswz(lrow, lane & 7) * 16);
    const uint32_t pieceoff1 = (uint32_t)((lrow + 8) * K + wswz(lrow + 8, lane & 7) * 16);
    // position i of this wave's stream: chunk wave + i W of both tiles, into a slot
    auto fire = [&](int i, int slot) {
        const int chunk = wave + i * W;
        const bool ok = i < cpw && chunk < nchunks;
        uint8_t* sl = ring + slot * SB;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t t0 = (uint32_t)((int64_t)rt[t] * K) + (uint32_t)chunk * kChunk;
            const uint32_t w0 = ok && rt[t] + lrow < re[t] ? t0 + pieceoff0 : kOob;
            const uint32_t w1 = ok && rt[t] + lrow + 8 < re[t] ? t0 + pieceoff1 : kOob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(sl + t * 2048), 16, (int)w0, 0, 0, kWeightCpol);
            if (!SHORT || t == 0)                        // SHORT: rows 8..15 of the second tile are never loaded
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(sl + t * 2048 + 1024), 16, (int)w1, 0, 0,
                                                         kWeightCpol);
        }
    };
    v8i bx[S][MT];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < S; ++s) {
        fire(s, s);
        load_bfrag<MT>(bx[s], rx, wave + s * W, s < cpw && wave + s * W < nchunks, r, g, M, K);
    }
    __builtin_amdgcn_sched_barrier(0);
    v4f acc[2][MT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = v4f{0.f, 0.f, 0.f, 0.f};
    // whole ring cycles: positions past cpw load zeros and add zeros
    for (int j0 = 0; j0 < cpw; j0 += S) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int nx = j0 + s + S;
            // position j0 + s landed (NW weight + 2 MT fragment loads per position): the S - 1 after it may be in flight
            __builtin_amdgcn_s_waitcnt(FP8MM_SM_VMCNT((NW + 2 * MT) * (S - 1)));
            const v8i A0 = slot_afrag(ring + s * SB, r, g);
            const v8i A1 = slot_afrag(ring + s * SB + 2048, r, g);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                acc[0][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A0, bx[s][mt], acc[0][mt], 0, 0, 0, 0,
                                                                             0, 0);
                acc[1][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, bx[s][mt], acc[1][mt], 0, 0, 0, 0,
                                                                             0, 0);
            }
            __builtin_amdgcn_s_waitcnt(FP8MM_SM_LGKM0);   // the slot's reads have returned
            fire(nx, s);
            load_bfrag<MT>(bx[s], rx, wave + nx * W, nx < cpw && wave + nx * W < nchunks, r, g, M, K);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);                      // no load outlives the workgroup; the ring area is free
    v4f* mine = reinterpret_cast<v4f*>(ring);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) put_partial(mine + (t * MT + mt) * 64 + lane, acc[t][mt]);
    __syncthreads();
    const int stride = S * SB / (int)sizeof(v4f);       // v4f per wave's ring area
    for (int idx = threadIdx.x; idx < my_tiles * MT * 64; idx += blockDim.x) {
        const int t = idx / (MT * 64), rem = idx - t * MT * 64;
        const int mt = rem / 64, l = rem - mt * 64;
        if (rt[t] + 4 * (l >> 4) >= re[t]) continue;     // rows of another workgroup
        reduce_tile(reinterpret_cast<const v4f*>(smem) + (t * MT + mt) * 64, stride, l, W, rt[t], re[t], s_act,
                    lds_f4(swl + t * 16 + 4 * (l >> 4)), sh, M, l, t == 1 && BAL, 16 * mt, srl);
    }
}

// Waves per workgroup: a function of K only (it fixes the summation order).
int small_m_waves(int64_t K)
{
    const int64_t nchunks = (K + kChunk - 1) / kChunk;
    int64_t w = (nchunks + kCpw - 1) / kCpw;
    if (w < 1) w = 1;
    if (w > kMaxWaves) w = kMaxWaves;
    return (int)w;
}

}  // namespace

// The reduction buffer can exceed the default 64 KB dynamic-LDS limit (W = 16
// waves x 4 M tiles); allow up to the 160 KB a gfx950 CU has.
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

template <int S, bool DEFER, int XI, bool BAL>
void launch_ring(const dim3& grid, const dim3& block, size_t lds, hipStream_t stream, const uint8_t* xq,
                 const uint8_t* wq, float s_act, const float* s_w, const ShardTable& sh, int M, int64_t N, int64_t K,
                 int nchunks, int cpw, int sw_lds)
{
    static const bool attr = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_small_m_ring<S, DEFER, XI, BAL>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        return true;
    }();
    (void)attr;
    hipLaunchKernelGGL((k_gemm_small_m_ring<S, DEFER, XI, BAL>), grid, block, lds, stream, xq, wq, s_act, s_w, sh, M, N, K,
                       nchunks, cpw, sw_lds);
}

// The LDS-ring persistent kernel, if it applies (M <= 16, K % 1024 == 0,
// x_q + partials + rings within 160 KB): deepest ring that fits, deferred
// reduction preferred.
bool try_ring(const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w, const ShardTable& sh,
              int64_t M, int64_t N, int64_t K, int W, int nchunks, hipStream_t stream)
{
    if (M > 16 || K % 1024 != 0 || N * K >= ((int64_t)1 << 31)) return false;
    const int64_t G = N / 16 < num_cus() ? N / 16 : num_cus();
    const int64_t tiles_max = (N / 16 + G - 1) / G;      // whole tiles, or FR + 1 with the balanced last round
    // Balanced last round when whole tiles leave the busiest workgroup at least
    // 1.3x the average weight bytes.
    const bool bal = 10 * tiles_max * G >= 13 * (N / 16);
    const size_t xb = (size_t)((M * (K + 16) + 15) & ~(int64_t)15);
    const size_t part = (size_t)W * 64 * sizeof(v4f);               // one tile's partials
    const size_t dpart = (size_t)W * (M <= 8 ? 32 : 64) * sizeof(v4f);   // ... as the deferred buffer keeps them
    const int cpw = (nchunks + W - 1) / W;
    const dim3 grid((uint32_t)G), block(64 * W);
    // x_q in LDS (XI = 0), else streamed with each chunk (1 KB for M <= 8, 2 KB for M <= 16)
    auto bytes = [&](int S, bool df, int xi) {
        return (xi ? 0 : xb) + (df ? tiles_max * dpart : 2 * part) + (size_t)W * S * (2048 + 1024 * xi);
    };
    // with DEFER, the tiles' weight scales in LDS too where they fit
    const size_t swb = (size_t)(tiles_max + 3) / 4 * 256;
#define FP8MM_RING_TRY(S, DF, XI)                                                                      \
    if (bytes(S, DF, XI) <= 160 * 1024) {                                                              \
        const int swl = DF && bytes(S, DF, XI) + swb <= 160 * 1024;                                    \
        const size_t lds = bytes(S, DF, XI) + (swl ? swb : 0);                                         \
        if (bal)                                                                                       \
            launch_ring<S, DF, XI, true>(grid, block, lds, stream, xq, wq, s_act, s_w, sh, (int)M, N, K, nchunks, \
                                         cpw, swl);                                                    \
        else                                                                                           \
            launch_ring<S, DF, XI, false>(grid, block, lds, stream, xq, wq, s_act, s_w, sh, (int)M, N, K, nchunks, \
                                          cpw, swl);                                                   \
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

// Mode, ring depth and reduction of the register-fragment kernel for a shape
// it takes: fragments resident for 4..5 chunks per wave, streamed beyond that
// (M > 16 only: at M <= 16 the ring kernel's LDS streaming is faster); the
// deepest ring that fits, deferred reduction preferred.
struct RxPlan {
    int xm, mt, cpw, S;
    bool bal, defer;
    size_t lds;
    unsigned G, W;
};

bool plan_rx(int64_t M, int64_t N, int64_t K, RxPlan* p, size_t extra = 0, bool no_defer = false)
{
    if (M < 1 || M > 32 || K % kChunk != 0 || N * K >= ((int64_t)1 << 31) || M * K >= ((int64_t)1 << 31)) return false;
    const int W = small_m_waves(K);
    const int nchunks = (int)(K / kChunk);
    const int cpw = (nchunks + W - 1) / W;
    const bool res = cpw >= 4 && cpw <= kCpw;
    if (cpw < 4 || (!res && M <= 16)) return false;      // short rows, or streamed at M <= 16: the ring kernel
    const int64_t G = N / 16 < num_cus() ? N / 16 : num_cus();
    const int64_t tiles_max = (N / 16 + G - 1) / G;
    p->bal = 10 * tiles_max * G >= 13 * (N / 16);
    p->xm = res ? XM_RES : XM_STREAM;
    p->mt = M <= 16 ? 1 : 2;
    p->cpw = cpw;
    p->G = (unsigned)G;
    p->W = (unsigned)W;
    const size_t mp = p->mt == 1 && M <= 8 ? 32 : 64;
    auto bytes = [&](int S, bool df) {
        return (df ? (size_t)tiles_max * W * p->mt * mp : (size_t)2 * W * p->mt * 64) * sizeof(v4f) +
               (size_t)W * S * 2048;
    };
    static const struct { int S; bool df; } order[] = {{6, true}, {6, false}, {4, true}, {4, false}, {3, true},
                                                       {3, false}, {2, true}, {2, false}};
    // M <= 16 with resident fragments: through LDS (XM_LDS) where they fit
    // beside some ring, even one shallower than the register path's (measured
    // faster on every decode shape); else in registers
    const size_t xl = res && M <= 16 ? (size_t)W * cpw * (M <= 8 ? 8 : 16) * kChunk : 0;
    const size_t swb = 256 + (size_t)(tiles_max + 3) / 4 * 256 + extra;   // the rows' and the tiles' scales
    for (const size_t xlb : {xl, (size_t)0})
        for (const auto& o : order)
            if (bytes(o.S, o.df) + xlb + swb <= 160 * 1024 && (o.df || p->xm != XM_STREAM) && !(o.df && no_defer)) {
                if (xlb) p->xm = XM_LDS;
                p->S = o.S;
                p->defer = o.df;
                p->lds = bytes(o.S, o.df) + xlb + swb;
                return true;
            }
    return false;
}

#define FP8MM_RX_ARGS p, xq, wq, s_act, s_w, sh, M, N, K, nchunks, xs, so, stream
template <int S, int MT, int XM, int CPW, bool BAL, bool DEFER, bool SILU = false>
void launch_rx(const RxPlan& p, const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w,
               const ShardTable& sh, int M, int64_t N, int64_t K, int nchunks, const XSrc& xs, const SiluOut& so,
               hipStream_t stream)
{
    static const bool attr = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_small_m_rx<S, MT, XM, CPW, BAL, DEFER, SILU>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        return true;
    }();
    (void)attr;
    hipLaunchKernelGGL((k_gemm_small_m_rx<S, MT, XM, CPW, BAL, DEFER, SILU>), dim3(p.G), dim3(64 * p.W), p.lds, stream,
                       xq, wq, s_act, s_w, sh, M, N, K, nchunks, p.cpw, xs, so);
}

template <int MT, int XM, int CPW, bool BAL>
void dispatch_rx_sd(const RxPlan& p, const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w,
                    const ShardTable& sh, int M, int64_t N, int64_t K, int nchunks, const XSrc& xs,
                    const SiluOut& so, hipStream_t stream)
{
    constexpr bool kStream = XM == XM_STREAM;   // streamed fragments: deferred reduction only
    if (p.S == 6 && p.defer) launch_rx<6, MT, XM, CPW, BAL, true>(FP8MM_RX_ARGS);
    else if (p.S == 4 && p.defer) launch_rx<4, MT, XM, CPW, BAL, true>(FP8MM_RX_ARGS);
    else if (p.S == 3 && p.defer) launch_rx<3, MT, XM, CPW, BAL, true>(FP8MM_RX_ARGS);
    else if (p.S == 2 && p.defer) launch_rx<2, MT, XM, CPW, BAL, true>(FP8MM_RX_ARGS);
    else if constexpr (!kStream) {
        if (p.S == 6) launch_rx<6, MT, XM, CPW, BAL, false>(FP8MM_RX_ARGS);
        else if (p.S == 4) launch_rx<4, MT, XM, CPW, BAL, false>(FP8MM_RX_ARGS);
        else if (p.S == 3) launch_rx<3, MT, XM, CPW, BAL, false>(FP8MM_RX_ARGS);
        else launch_rx<2, MT, XM, CPW, BAL, false>(FP8MM_RX_ARGS);
    }
}

template <int MT, int XM, int CPW>
void dispatch_rx(const RxPlan& p, const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w,
                 const ShardTable& sh, int M, int64_t N, int64_t K, int nchunks, const XSrc& xs, const SiluOut& so,
                 hipStream_t stream)
{
    if (so.hq) {                                         // the SiLU*mul epilogue: whole tiles, no deferral
        if constexpr (XM != XM_STREAM) {                 // (streamed fragments need the deferral)
            if (p.S == 6) launch_rx<6, MT, XM, CPW, false, false, true>(FP8MM_RX_ARGS);
            else if (p.S == 4) launch_rx<4, MT, XM, CPW, false, false, true>(FP8MM_RX_ARGS);
            else if (p.S == 3) launch_rx<3, MT, XM, CPW, false, false, true>(FP8MM_RX_ARGS);
            else launch_rx<2, MT, XM, CPW, false, false, true>(FP8MM_RX_ARGS);
        }
    } else if (p.bal) {
        dispatch_rx_sd<MT, XM, CPW, true>(FP8MM_RX_ARGS);
    } else {
        dispatch_rx_sd<MT, XM, CPW, false>(FP8MM_RX_ARGS);
    }
}

// Launch the register-fragment kernel if it takes this shape.  With xsrc, the
// fused static quant: only the XM_QLDS plan (M <= 8, fragments staged in LDS),
// else false.
bool try_rx(const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w, const ShardTable& sh, int64_t M64,
            int64_t N, int64_t K, hipStream_t stream, const XSrc* xsrc = nullptr, const SiluOut* silu = nullptr)
{
    RxPlan p;
    const bool rms = xsrc && xsrc->gamma;
    // XM_QRMS: the rows' r after the scales; the SiLU*mul epilogue: whole tiles
    if (!plan_rx(M64, N, K, &p, rms ? 32 : 0, silu != nullptr) || (silu && p.bal)) return false;
    const int M = (int)M64, nchunks = (int)(K / kChunk);
    const XSrc xs = xsrc ? *xsrc : XSrc{nullptr, 0, nullptr, 0.0f, 0.0f, nullptr, 0.0f};
    const SiluOut so = silu ? *silu : SiluOut{nullptr, 0, 0.0f, 0.0f, 0.0f};
    if (rms) {
        if (p.xm != XM_LDS || M > 8 || p.W != 8 || p.cpw != 5) return false;
        dispatch_rx<1, XM_QRMS, 5>(FP8MM_RX_ARGS);
    } else if (xsrc) {
        if (p.xm != XM_LDS || M > 8) return false;
        if (p.cpw == 4) dispatch_rx<1, XM_QLDS, 4>(FP8MM_RX_ARGS);
        else dispatch_rx<1, XM_QLDS, 5>(FP8MM_RX_ARGS);
    } else if (p.xm == XM_LDS) {
        if (p.cpw == 4) dispatch_rx<1, XM_LDS, 4>(FP8MM_RX_ARGS);
        else dispatch_rx<1, XM_LDS, 5>(FP8MM_RX_ARGS);
    } else if (p.xm == XM_RES) {
        if (p.mt == 1 && p.cpw == 4) dispatch_rx<1, XM_RES, 4>(FP8MM_RX_ARGS);
        else if (p.mt == 1) dispatch_rx<1, XM_RES, 5>(FP8MM_RX_ARGS);
        else if (p.cpw == 4) dispatch_rx<2, XM_RES, 4>(FP8MM_RX_ARGS);
        else dispatch_rx<2, XM_RES, 5>(FP8MM_RX_ARGS);
    } else {
        dispatch_rx<2, XM_STREAM, 0>(FP8MM_RX_ARGS);
    }
    return true;
}
#undef FP8MM_RX_ARGS

template <int S, int MT, bool BAL, bool SHORT = false>
void launch_pair(unsigned G, unsigned W, size_t lds, const uint8_t* xq, const uint8_t* wq, float s_act,
                 const float* s_w, const ShardTable& sh, int M, int64_t N, int64_t K, int nchunks, int cpw,
                 hipStream_t stream)
{
    static const bool attr = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_small_m_pair<S, MT, BAL, SHORT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        return true;
    }();
    (void)attr;
    hipLaunchKernelGGL((k_gemm_small_m_pair<S, MT, BAL, SHORT>), dim3(G), dim3(64 * W), lds, stream, xq, wq, s_act,
                       s_w, sh, M, N, K, nchunks, cpw);
}

// The two-tile kernel, if it takes the shape: M <= 32, more chunks per wave
// than stay resident (the fragments streamed), and at most two tiles per
// workgroup (one whole tile and a balanced share of the rest, or two whole).
// Measured against the kernels it replaces there (5120 x 17408, the decode
// MLP's down projection): M = 32 42.4 -> 29.0 us, M = 16 23.6 -> 21.1 us,
// M = 8 19.7 -> 19.2 us, M = 1 unchanged.
bool try_pair(const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w, const ShardTable& sh, int64_t M,
              int64_t N, int64_t K, hipStream_t stream)
{
    if (M < 1 || M > 32 || K % kChunk != 0 || N * K >= ((int64_t)1 << 31) || M * K >= ((int64_t)1 << 31))
        return false;
    const int W = small_m_waves(K);
    const int nchunks = (int)(K / kChunk);
    const int cpw = (nchunks + W - 1) / W;
    if (cpw <= kCpw) return false;                      // resident fragments: the register kernel
    const int64_t ntiles = N / 16;
    const int64_t G = ntiles < num_cus() ? ntiles : num_cus();
    const int64_t tiles_max = (ntiles + G - 1) / G;
    const bool bal = 10 * tiles_max * G >= 13 * ntiles;  // the register kernel's rule
    if (bal ? ntiles / G != 1 : tiles_max != 2) return false;
#define FP8MM_PAIR_LAUNCH(S, MT) \
    (bal ? launch_pair<S, MT, true>((unsigned)G, (unsigned)W, lds, xq, wq, s_act, s_w, sh, (int)M, N, K, nchunks, cpw, stream) \
         : launch_pair<S, MT, false>((unsigned)G, (unsigned)W, lds, xq, wq, s_act, s_w, sh, (int)M, N, K, nchunks, cpw, stream))
    // a short second tile (every balanced share <= 8 rows: ceil(share groups / G) <= 2): 3 KB slots, 3 of them
    const int64_t ngr = (N - G * 16) / 4;
    if (bal && (ngr + G - 1) / G <= 2 && (size_t)W * 3 * 3072 + 1024 + 512 <= 160 * 1024) {
        const size_t lds = (size_t)W * 3 * 3072 + 1024 + 512;
        if (M <= 16)
            launch_pair<3, 1, true, true>((unsigned)G, (unsigned)W, lds, xq, wq, s_act, s_w, sh, (int)M, N, K, nchunks,
                                          cpw, stream);
        else
            launch_pair<3, 2, true, true>((unsigned)G, (unsigned)W, lds, xq, wq, s_act, s_w, sh, (int)M, N, K, nchunks,
                                          cpw, stream);
        return true;
    }
    for (const int S : {3, 2}) {
        const size_t lds = (size_t)W * S * 4096 + 512;
        if (lds > 160 * 1024) continue;
        if (M <= 16) {
            if (S == 3) FP8MM_PAIR_LAUNCH(3, 1);
            else FP8MM_PAIR_LAUNCH(2, 1);
        } else {
            if (S == 3) FP8MM_PAIR_LAUNCH(3, 2);
            else FP8MM_PAIR_LAUNCH(2, 2);
        }
        return true;
    }
#undef FP8MM_PAIR_LAUNCH
    return false;
}

bool quant_gemm_small_m_fits(int64_t M, int64_t N, int64_t K, int64_t ldx, float s_act, bool rmsnorm)
{
    // 32-bit buffer offsets into the activation; the range where the
    // quotient by multiply and fused multiply-add is exact
    if (M < 1 || M > 8 || ldx < K || !code_table_ok(s_act) || ((M - 1) * ldx + K) * 2 >= ((int64_t)1 << 31))
        return false;
    RxPlan p;
    if (!plan_rx(M, N, K, &p, rmsnorm ? 32 : 0) || p.xm != XM_LDS) return false;
    return !rmsnorm || (p.W == 8 && p.cpw == 5);         // the RMSNorm's summation order needs 8 waves
}

bool launch_quant_gemm_small_m(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, uint8_t* xq_out,
                               const uint8_t* wq, float s_act, const float* s_w, const ShardTable& shards, int64_t M,
                               int64_t N, int64_t K, hipStream_t stream)
{
    if (!quant_gemm_small_m_fits(M, N, K, ldx, s_act, gamma != nullptr)) return false;
    // the quotient's operands, rounded once here (IEEE single on the host)
    const XSrc xs{x, ldx, xq_out, 1.0f / s_act, 448.0f * s_act, gamma, eps};
    return try_rx(nullptr, wq, s_act, s_w, shards, M, N, K, stream, &xs);
}

bool gate_up_silu_fits(int64_t M, int64_t I, int64_t K, int64_t ldx, float s_act, float s_down, int quant)
{
    if (M < 1 || M > 32 || I < 8 || I % 8 != 0 || !code_table_ok(s_down)) return false;
    // with the quant in the launch: as quant_gemm_small_m_fits
    if (quant && (M > 8 || ldx < K || !code_table_ok(s_act) || ((M - 1) * ldx + K) * 2 >= ((int64_t)1 << 31)))
        return false;
    RxPlan p;
    if (!plan_rx(M, 2 * I, K, &p, quant == 2 ? 32 : 0, true) || p.bal || p.W > 8) return false;
    if (quant && p.xm != XM_LDS) return false;
    return quant != 2 || (p.W == 8 && p.cpw == 5);
}

bool launch_gate_up_silu(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, uint8_t* xq,
                         const uint8_t* wq, float s_act, const float* s_w, int64_t M, int64_t I, int64_t K,
                         float s_down, uint8_t* hq, hipStream_t stream)
{
    const int quant = x ? (gamma ? 2 : 1) : 0;
    if (!gate_up_silu_fits(M, I, K, ldx, s_act, s_down, quant)) return false;
    // one shard over the interleaved rows; the epilogue stores h_q instead
    ShardTable sh{};
    sh.num = 1;
    sh.start[1] = 2 * I;
    sh.out[0] = hq;
    sh.ldo[0] = I;
    // the quotients' operands, rounded once here (IEEE single on the host)
    const SiluOut so{hq, I, s_down, 1.0f / s_down, 448.0f * s_down};
    if (quant) {
        const XSrc xs{x, ldx, xq, 1.0f / s_act, 448.0f * s_act, gamma, eps};
        return try_rx(nullptr, wq, s_act, s_w, sh, M, 2 * I, K, stream, &xs, &so);
    }
    return try_rx(xq, wq, s_act, s_w, sh, M, 2 * I, K, stream, nullptr, &so);
}

void launch_gemm_small_m(const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w,
                         const ShardTable& shards, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    const int W = small_m_waves(K);
    const int nchunks = (int)((K + kChunk - 1) / kChunk);
    if (try_pair(xq, wq, s_act, s_w, shards, M, N, K, stream)) return;
    if (try_rx(xq, wq, s_act, s_w, shards, M, N, K, stream)) return;
    if (try_ring(xq, wq, s_act, s_w, shards, M, N, K, W, nchunks, stream)) return;
    const int MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    const size_t lds = (size_t)W * MT * 64 * sizeof(v4f);
    const dim3 grid((uint32_t)((N + 15) / 16)), block(64 * W);
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
