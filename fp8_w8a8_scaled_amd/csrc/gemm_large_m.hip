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
#include "out_store.h"

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
        const int si = shard_of(sh, n);
        const float swn = s_w[n];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < M) store_out1(sh, si, m, n, (acc[i][j][v] * row_scale(sh, m, s_act)) * swn);
            }
    }
}


// ---------------------------------------------------------------------------
// Tiled kernel for K % 128 == 0 (every prefill shape of the layer).
//
// 256x256 output tile per 256-thread workgroup; wave (wn, wm) owns 128 rows of
// W (n) x 128 rows of x_q (m) as 4x4 v_mfma_f32_32x32x64_f8f6f4 tiles with W
// as the A operand (accumulators live in AGPRs).  K advances 128 bytes per
// stage through two LDS stages of 64 KB filled by direct global->LDS loads
// (global_load_lds_dwordx4: whole 128-byte lines, no staging registers).  A
// stage is two sub-steps of 16 MFMAs (one 64-byte MFMA depth each); fragment
// registers are double-buffered, so the 16 ds_read_b128 of the next sub-step
// are interleaved with the first 8 MFMAs of the current one.
// Stage boundary (before the last sub-step of stage kt reads stage kt+1):
// wait until stage kt+1 has landed and this wave's reads of stage kt are
// done, then a bare barrier; stage kt's buffer then takes stage kt+2, whose
// 16 loads are issued one per MFMA of the following sub-step.  Issued as one
// burst, those loads queue on the CU's one address unit and hold up every
// wave's matrix pipe behind them (in-order issue); spread out they overlap
// the MFMAs (measured 10% faster on the prefill gate_up shape).
// sched_barrier fences keep each MFMA with its fragment read and its load.
// LDS rows are 128 bytes with their eight 16-byte pieces XOR-swizzled by row
// (skipping one row bit: gfx950 LDS serves 16 lanes x 16 B per cycle) so the
// fragment reads are bank-conflict free.
// Workgroups are renumbered so that each XCD (blocks are dealt to the 8 XCDs
// round-robin) walks a contiguous range of tiles, in groups of GM row-tiles
// that share W column tiles through L2.  The epilogue scales in fp32, rounds
// pairs to bf16 with v_cvt_pk_bf16_f32, stages the tile in LDS and writes it
// with row-contiguous 16-byte stores.
// Rows past M or N load a clamped (real) row and are never stored.
// ---------------------------------------------------------------------------
// x_q row-tiles per tile group (L2 sharing).  A round of an XCD's 32
// workgroups then spans GM x_q panels and 32 / GM weight panels, fewest near
// GM = sqrt(32); measured at prefill M (same bits): GM = 8 924 / 467 us
// (gate_up / down), 4-6 901-915 / 445-454 us, 12 972 / 474 us.
constexpr int kGroupM = 6;

// The C tile stores are non-temporal.  The workgroups finish their tiles at
// about the same time, and the C tiles they write (4 MB per XCD per round)
// would otherwise displace from L2 the operand panels the next round reads;
// measured 13% faster on the prefill gate_up shape.
__device__ __forceinline__ void store_c16(void* dst, const uint4 v)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
}

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int TW = 256;                      // tile rows of W (2 waves x 128)
constexpr int TK = 128;                      // K bytes per stage (two MFMA depths)
constexpr int NSTAGE = 2;
constexpr int PPR = TK / 16;                 // 16-byte pieces per LDS row
constexpr int ROWS_PER_INST = 64 / PPR;      // rows one direct-to-LDS instruction fills
constexpr int WQ = TW / ROWS_PER_INST / 4;   // W loads per wave and stage

// Tile shapes: NJ 32-row blocks of x_q per wave, so TX = 64 NJ rows of x_q per
// tile (NJ = 4: 256x256 tiles; NJ = 3: 256x192, for shapes whose 256x256 tile
// count leaves the last round of the persistent grid nearly empty).
template <int NJ>
struct Cfg {
    static constexpr int TX = 64 * NJ;                        // tile rows of x_q
    static constexpr int XQ = TX / ROWS_PER_INST / 4;         // x_q loads per wave and stage
    static constexpr int LOADS = WQ + XQ;                     // loads per wave and stage
    static constexpr int MF = 4 * NJ;                         // MFMAs per sub-step
    static constexpr int NF = 4 + NJ;                         // fragments per sub-step
    static constexpr int STAGE_BYTES = (TW + TX) * TK;        // W tile + x_q tile
    static constexpr int C_ROW = TW * 2 + 16;                 // padded bf16 C row (one m), bytes
    static constexpr int C_ROW32 = TW * 4 + 16;               // padded f32 C row, bytes
    static constexpr int A = NSTAGE * STAGE_BYTES, B = TX * C_ROW, C = TX / 2 * C_ROW32;
    static constexpr int LDS_MAIN = A > B ? (A > C ? A : C) : (B > C ? B : C);
    static constexpr int SW_OFF = LDS_MAIN;                   // the tile's TW weight scales (f32), after the rest
    static constexpr int LDS = LDS_MAIN + TW * 4;
    static_assert(NF <= MF && LOADS <= 2 * MF, "reads and loads fit the sub-step's MFMA slots");
    static_assert((TX / 8) % 4 == 0 && (TX / 2 / 4) % 4 == 0, "epilogue rows per thread come in groups of 4");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int swz(int row, int piece)
{
    return piece ^ ((row >> 1) & (PPR - 1));
}

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// s_waitcnt with only vmcnt constrained (expcnt = 7, lgkmcnt = 15: no wait).
// The count must be a compile-time constant.
#define FP8MM_VMCNT_IMM(n) ((((n) & 15) | ((((n) >> 4) & 3) << 14)) | (7 << 4) | (15 << 8))
// same, and lgkmcnt(0): every LDS read of this wave has returned
#define FP8MM_VMCNT_LGKM0_IMM(n) ((((n) & 15) | ((((n) >> 4) & 3) << 14)) | (7 << 4))

// Operand addressing of one tile.  The lane's load i of an operand moves
// LDS row (wave + 4 i) * ROWS_PER_INST + lane / PPR, i.e. global row
// row0 + 32 i: byte offset w0 (x0) + i * step in the operand's buffer, plus the
// stage's K offset.  The XOR swizzle of the piece uses row bits 1..3 only, so
// it is the same for all i.  Rows past N (M) fall past the end of the buffer
// resource and load zeros; their results are never stored.  Offsets are
// 32-bit (N K, M K < 2^32); an offset that wraps around for such a row stays
// inside the buffer, so no load leaves its buffer.
template <int NJ>
struct RowOffsets {
    uint32_t w0, x0, step;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const uint8_t* p, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

template <int NJ>
__device__ __forceinline__ void row_offsets(RowOffsets<NJ>& o, int64_t n0, int64_t m0, int64_t K, int wave, int lane)
{
    const int lr = lane / PPR, lp = lane % PPR;       // row within instruction, physical piece
    const int row = wave * ROWS_PER_INST + lr;
    o.w0 = (uint32_t)((n0 + row) * K + swz(row, lp) * 16);   // logical piece stored at physical lp
    o.x0 = (uint32_t)((m0 + row) * K + swz(row, lp) * 16);
    o.step = (uint32_t)(4 * ROWS_PER_INST * K);
}

// Load li of the stage at K offset k: li < WQ fill W rows, the rest x_q rows;
// instruction q = wave + 4 i fills the LDS rows q * ROWS_PER_INST.. of its
// operand tile.
template <int NJ>
__device__ __forceinline__ void stage_load(int li, uint8_t* st, uint32_t k, __amdgpu_buffer_rsrc_t rw,
                                           __amdgpu_buffer_rsrc_t rx, const RowOffsets<NJ>& o, int wave)
{
    if (li < WQ) {
        const int q = wave + 4 * li;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(st + q * 1024), 16,
                                                 (int)(o.w0 + (uint32_t)li * o.step + k), 0, 0, 0);
    } else {
        const int i = li - WQ, q = wave + 4 * i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)(st + TW * TK + q * 1024), 16,
                                                 (int)(o.x0 + (uint32_t)i * o.step + k), 0, 0, 0);
    }
}

template <int NJ>
struct Frags {
    v8i a[4], b[NJ];
};

// Fragment half h of MFMA operand f (0-3: W rows, 4..: x_q rows) for sub-step
// `sub` of a stage: lane l supplies row l % 32 and K bytes [32 (l / 32),
// 32 (l / 32) + 32) of the 64-byte depth.
template <int NJ>
__device__ __forceinline__ uint4 frag_half(const uint8_t* __restrict__ st, int f, int h, int sub, int lane, int wn,
                                           int wm)
{
    const int fr = lane & 31, p = sub * 4 + (lane >> 5) * 2 + h;
    const int row = f < 4 ? wn * 128 + f * 32 + fr : wm * (32 * NJ) + (f - 4) * 32 + fr;
    const uint8_t* base = f < 4 ? st : st + TW * TK;
    return lds16(base + row * TK + swz(row, p) * 16);
}

// One sub-step: the MF MFMAs of `fc`; the first NF are each followed by the
// two 16-byte reads of one fragment of the next sub-step (into `fn`), so the
// reads have landed before the sub-step ends, and, when LD is set, the
// stage's LOADS loads (into `fill`) are spread over all MF MFMAs.  With Z the
// MFMAs start from zero (the tile's first sub-step): the accumulators need no
// clearing (256 register writes per lane and tile).
template <int NJ, bool LD, bool Z = false>
__device__ __forceinline__ void substep(const uint8_t* __restrict__ frag_src, int sub_next, int lane, int wn, int wm,
                                        const Frags<NJ>& fc, Frags<NJ>& fn, v16f (&acc)[4][NJ], uint8_t* fill,
                                        uint32_t k, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx,
                                        const RowOffsets<NJ>& ro, int wave)
{
    using C = Cfg<NJ>;
    uint4 t[2 * C::NF];
#pragma unroll
    for (int s = 0; s < C::MF; ++s) {
        const int i = s / NJ, j = s % NJ;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fc.a[i], fc.b[j], Z ? v16f{} : acc[i][j], 0, 0, 0,
                                                                    0, 0, 0);
        if (s < C::NF) {
            t[2 * s] = frag_half<NJ>(frag_src, s, 0, sub_next, lane, wn, wm);
            t[2 * s + 1] = frag_half<NJ>(frag_src, s, 1, sub_next, lane, wn, wm);
        }
        if (LD) {
#pragma unroll
            for (int li = s * C::LOADS / C::MF; li < (s + 1) * C::LOADS / C::MF; ++li)
                stage_load<NJ>(li, fill, k, rw, rx, ro, wave);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) fn.a[f] = pack(t[2 * f], t[2 * f + 1]);
#pragma unroll
    for (int f = 0; f < NJ; ++f) fn.b[f] = pack(t[8 + 2 * f], t[8 + 2 * f + 1]);
}

template <int NJ>
__global__ __launch_bounds__(256) void k_gemm_large_m_tiled(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ wq, float s_act,
    const float* __restrict__ s_w, ShardTable sh, int64_t M, int64_t N, int64_t K)
{
    using C = Cfg<NJ>;
    constexpr int TX = C::TX, HX = TX / 2;             // x_q rows per tile and per wave
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar registers
    const int wn = wave & 1, wm = wave >> 1;

    // Persistent schedule.  Workgroups are dealt to the 8 XCDs round-robin, so
    // the ones with bid % 8 == x share XCD x's L2: give that XCD a contiguous
    // range of tiles and let its workgroups walk it in lockstep rounds (round
    // r = tiles r*nbx .. r*nbx+nbx-1 of the range).  Tiles are numbered in
    // groups of GM row-tiles per W column-tile, so one round covers a few
    // x_q row-tiles and W column-tiles whose K slices the concurrent
    // workgroups fetch at about the same time -- they meet in L2.
    const int nb = gridDim.x, bid = blockIdx.x;
    const int num_m = (int)((M + TX - 1) / TX), num_n = (int)((N + TW - 1) / TW);
    const int ntiles = num_m * num_n;
    const int xcd = bid & 7;
    const int nbx = (nb >> 3) + (xcd < (nb & 7) ? 1 : 0);
    const int tiles_x = (ntiles >> 3) + (xcd < (ntiles & 7) ? 1 : 0);
    const int start_x = xcd * (ntiles >> 3) + (xcd < (ntiles & 7) ? xcd : (ntiles & 7));
    const int GM = kGroupM;
    const int in_group = GM * num_n;
    // operand buffers: rows past N or M load zeros
    const __amdgpu_buffer_rsrc_t rw = operand_rsrc(wq, N * K), rx = operand_rsrc(xq, M * K);
    const __amdgpu_buffer_rsrc_t rsw = operand_rsrc(reinterpret_cast<const uint8_t*>(s_w), N * 4);
    float* swl = reinterpret_cast<float*>(smem + C::SW_OFF);
    for (int u = bid >> 3; u < tiles_x; u += nbx) {
    const int t = start_x + u;
    const int first_m = (t / in_group) * GM;
    const int gsz = (num_m - first_m) < GM ? (num_m - first_m) : GM;
    const int tm = first_m + (t % in_group) % gsz;
    const int tn = (t % in_group) / gsz;
    const int64_t m0 = (int64_t)tm * TX, n0 = (int64_t)tn * TW;

    v16f acc[4][NJ];                                   // set by the first sub-step (Z)

    const int nk = (int)(K / TK);
    // K offset of stage st; the stages past the end (the pipeline's trailing
    // loads) load from past the end of the buffers: zeros, no memory traffic
    auto kof = [&](int st) { return st < nk ? (int64_t)st * TK : (int64_t)0x80000000u; };
    RowOffsets<NJ> ro;
    // The lane index passes through an empty asm statement, so the offsets'
    // lane arithmetic is redone per tile rather than hoisted out of the tile
    // loop: hoisted, its values live across the main loop and get spilled
    // (and reloaded from scratch on every tile's critical path).
    int rlane = lane;
    __asm__ volatile("" : "+v"(rlane));
    row_offsets<NJ>(ro, n0, m0, K, wave, rlane);
#pragma unroll
    for (int s = 0; s < NSTAGE; ++s)
#pragma unroll
        for (int li = 0; li < C::LOADS; ++li)
            stage_load<NJ>(li, smem + s * C::STAGE_BYTES, (uint32_t)kof(s), rw, rx, ro, wave);
    __builtin_amdgcn_s_waitcnt(FP8MM_VMCNT_IMM(C::LOADS));   // stage 0 landed for this wave
    __builtin_amdgcn_s_barrier();

    // Sub-steps run in order (stage kt: sub-step 0, boundary, sub-step 1);
    // fragments alternate between fa and fb.
    Frags<NJ> fa, fb;
#pragma unroll
    for (int f = 0; f < 4; ++f)
        fa.a[f] = pack(frag_half<NJ>(smem, f, 0, 0, lane, wn, wm), frag_half<NJ>(smem, f, 1, 0, lane, wn, wm));
#pragma unroll
    for (int f = 0; f < NJ; ++f)
        fa.b[f] = pack(frag_half<NJ>(smem, 4 + f, 0, 0, lane, wn, wm), frag_half<NJ>(smem, 4 + f, 1, 0, lane, wn, wm));
    // stage kt (kt < nk): sub-step 0 (its sub-step 1 fragments come from the
    // same stage); boundary: stage kt+1 landed (the only stage in flight),
    // stage kt fully read; sub-step 1: fragments of stage kt+1, and the loads
    // of stage kt+2 into stage kt's buffer.  Stage 0 starts the accumulators;
    // the last stage also fetches the tile's weight scales into LDS (one
    // direct-to-LDS load per wave, past the boundary's wait: it lands during
    // the last sub-step instead of in front of the epilogue).
    auto stage = [&](int kt, auto first, auto last) {
        uint8_t* cur = smem + (kt & 1) * C::STAGE_BYTES;
        uint8_t* nxt = smem + ((kt + 1) & 1) * C::STAGE_BYTES;
        substep<NJ, false, decltype(first)::value>(cur, 1, lane, wn, wm, fa, fb, acc, nullptr, 0u, rw, rx, ro, wave);
        __builtin_amdgcn_s_waitcnt(FP8MM_VMCNT_LGKM0_IMM(0));
        __builtin_amdgcn_s_barrier();
        if constexpr (decltype(last)::value) {
            const int64_t n = n0 + wave * 64 + lane;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void_t*)(swl + wave * 64), 4,
                                                     n < N ? (int)(n * 4) : (int)0x80000000u, 0, 0, 0);
        }
        const int64_t k2 = kof(kt + 2);
        substep<NJ, true>(nxt, 0, lane, wn, wm, fb, fa, acc, cur, (uint32_t)k2, rw, rx, ro, wave);
    };
    if (nk == 1) {
        stage(0, std::true_type{}, std::true_type{});
    } else {
        stage(0, std::true_type{}, std::false_type{});
        for (int kt = 1; kt < nk - 1; ++kt) stage(kt, std::false_type{}, std::false_type{});
        stage(nk - 1, std::false_type{}, std::true_type{});
    }

    // Epilogue: scale, round to bf16, stage the TX x 256 tile in LDS (rows of
    // m, padded), then store rows with 16-byte, row-contiguous writes (an f32
    // output in two halves: a whole f32 tile would not fit in LDS).
    __builtin_amdgcn_s_waitcnt(0);                     // retire the trailing (zero) stage loads
    __syncthreads();                                   // every stage read by every wave
    // The same for the epilogue's thread-index arithmetic (row and column
    // indices, LDS addresses).
    int tid = threadIdx.x;
    __asm__ volatile("" : "+v"(tid));
    const int fr = tid & 31, fh = (tid & 63) >> 5;
    const int ewn = (tid >> 6) & 1, ewm = tid >> 7;    // this wave's wn, wm
    // 32x32 C layout with W as A: lane l holds column l%32 (= m) and rows
    // 8*(v/4) + 4*(l/32) + v%4 (= n): four consecutive n per v/4.
    float4 swv[4][4];                                  // the weight scales, staged by the last stage (zeros past N)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            swv[i][q] = *reinterpret_cast<const float4*>(swl + ewn * 128 + i * 32 + 8 * q + 4 * fh);
    // The loops below run row group j outermost, so only one activation scale
    // (per-tensor, or this lane's row's) is live at a time.
    if (sh.f32) {
        // f32: the tile in two halves of HX rows (the waves with wm == h hold
        // half h), each staged in LDS and stored with row-contiguous 16-byte writes
        for (int h = 0; h < 2; ++h) {
            if (ewm == h) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const float sa = row_scale(sh, min(m0 + ewm * HX + j * 32 + fr, M - 1), s_act);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int nl = ewn * 128 + i * 32 + 8 * q + 4 * fh;
                            const float4 sw = swv[i][q];
                            const v16f& c = acc[i][j];
                            *reinterpret_cast<float4*>(smem + (j * 32 + fr) * C::C_ROW32 + nl * 4) =
                                make_float4((c[4 * q + 0] * sa) * sw.x, (c[4 * q + 1] * sa) * sw.y,
                                            (c[4 * q + 2] * sa) * sw.z, (c[4 * q + 3] * sa) * sw.w);
                        }
                }
            }
            __syncthreads();
            // This thread's 4 columns are the same in every row it stores:
            // shard, destination column and row stride are fixed per tile.
            const int nl = (tid & 63) * 4;
            const int64_t n = n0 + nl;
            if (n < N) {
                void* o;
                int64_t ldo, st;
                shard_fields(sh, n, o, ldo, st);
                float* col = static_cast<float*>(o) + (n - st);
                // rows ml = threadIdx/64 + 4 r: four LDS reads, then their stores
                // (rows past M are read but not stored)
#pragma unroll
                for (int g = 0; g < HX / 4; g += 4) {
                    uint4 v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = *reinterpret_cast<const uint4*>(smem + ((tid >> 6) + 4 * (g + r)) * C::C_ROW32 +
                                                               nl * 4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int64_t m = m0 + h * HX + (tid >> 6) + 4 * (g + r);
                        if (m < M) {
                            store_c16(col + m * ldo, v[r]);
                        }
                    }
                }
            }
            __syncthreads();                           // the LDS is reused (next half, next tile)
        }
        continue;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const float sa = row_scale(sh, min(m0 + ewm * HX + j * 32 + fr, M - 1), s_act);
        const int ml = ewm * HX + j * 32 + fr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = ewn * 128 + i * 32 + 8 * q + 4 * fh;
                const float4 sw = swv[i][q];
                const v16f& c = acc[i][j];
                const uint32_t lo = pack_bf16x2((c[4 * q + 0] * sa) * sw.x, (c[4 * q + 1] * sa) * sw.y);
                const uint32_t hi = pack_bf16x2((c[4 * q + 2] * sa) * sw.z, (c[4 * q + 3] * sa) * sw.w);
                *reinterpret_cast<uint2*>(smem + ml * C::C_ROW + nl * 2) = make_uint2(lo, hi);
            }
    }
    __syncthreads();
    {
        // This thread's 8 columns are the same in every row it stores (rows
        // advance by 8 per 256 threads): shard, destination column and row
        // stride are fixed per tile, so the store loop carries no table lookup.
        const int nl = (tid & 31) * 8;
        const int64_t n = n0 + nl;
        if (n < N) {
            void* o;
            int64_t ldo, st;
            shard_fields(sh, n, o, ldo, st);
            uint16_t* col = static_cast<uint16_t*>(o) + (n - st);
            // rows ml = threadIdx/32 + 8 r: four LDS reads, then their stores
            // (rows past M are read but not stored)
#pragma unroll
            for (int g = 0; g < TX / 8; g += 4) {
                uint4 v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[r] = *reinterpret_cast<const uint4*>(smem + ((tid >> 5) + 8 * (g + r)) * C::C_ROW + nl * 2);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t m = m0 + (tid >> 5) + 8 * (g + r);
                    if (m < M) {
                        store_c16(col + m * ldo, v[r]);
                    }
                }
            }
        }
    }
    __syncthreads();                                   // the next tile reuses the LDS
    }
}


}  // namespace

// Compute units of the current device (cached per device ordinal).
int num_cus()
{
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// Rounds of the persistent grid times x_q rows per tile, for a tile of 64 nj
// rows of x_q: the time the grid takes, in units of one 256x64 strip.
static int64_t tiled_cost(int64_t M, int64_t N, int nj, int64_t cus)
{
    const int64_t tiles = ((M + 64 * nj - 1) / (64 * nj)) * ((N + TW - 1) / TW);
    const int64_t grid = tiles < cus ? tiles : cus;
    return ((tiles + grid - 1) / grid) * nj;
}

template <int NJ>
static void launch_tiled(const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w,
                         const ShardTable& shards, int64_t M, int64_t N, int64_t K, int64_t cus, hipStream_t stream)
{
    static const bool attr = [] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_large_m_tiled<NJ>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        return true;
    }();
    (void)attr;
    const int64_t tiles = ((M + Cfg<NJ>::TX - 1) / Cfg<NJ>::TX) * ((N + TW - 1) / TW);
    const int64_t grid = tiles < cus ? tiles : cus;   // one resident workgroup per CU
    hipLaunchKernelGGL(k_gemm_large_m_tiled<NJ>, dim3((uint32_t)grid), dim3(256), (size_t)Cfg<NJ>::LDS, stream, xq,
                       wq, s_act, s_w, shards, M, N, K);
}

void launch_gemm_large_m(const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w,
                         const ShardTable& shards, int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    // the tiled kernel addresses operands with 32-bit row offsets
    if (K % TK == 0 && N * K < ((int64_t)1 << 32) && M * K < ((int64_t)1 << 32)) {
        // 256x192 tiles when they cut the grid's time by at least 10% (their
        // operand traffic per flop is about 17% higher): e.g. the prefill down
        // projection, 26 x 20 = 520 tiles of 256x256 (2 full rounds and 8
        // tiles on 256 CUs) against 35 x 20 = 700 of 256x192 (3 rounds of
        // three-quarter tiles).
        const int64_t cus = num_cus();
        if (10 * tiled_cost(M, N, 3, cus) <= 9 * tiled_cost(M, N, 4, cus))
            launch_tiled<3>(xq, wq, s_act, s_w, shards, M, N, K, cus, stream);
        else
            launch_tiled<4>(xq, wq, s_act, s_w, shards, M, N, K, cus, stream);
        return;
    }
    const dim3 grid((uint32_t)((N + BN - 1) / BN), (uint32_t)((M + BM - 1) / BM));
    hipLaunchKernelGGL(k_gemm_large_m, grid, dim3(kThreads), 0, stream, xq, wq, s_act, s_w, shards, M, N, K);
}

}  // namespace fp8mm
