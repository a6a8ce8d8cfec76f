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
// E4M3 stores; LDS holds block reductions and the lookup tables that replace
// the per-element division and encode (the fused RMSNorm quant instead takes
// the exact quotient by multiply and fused multiply-add and the hardware E4M3
// conversion).  Also here: the load-time interleave of a gate_up weight for
// the SiLU*mul epilogue of the small-M GEMM.
#include <mutex>

#include "act_quant.h"
#include "act_tables.h"
#include "device_common.h"
#include "internal.h"

namespace fp8mm {

namespace {

constexpr int kQuantThreads = kRmsRowThreads;

typedef __attribute__((address_space(3))) void lds_void;

// Launch choices of the table-based kernels (measured on MI355X; the bytes do
// not depend on them).
constexpr int kSiluLutPerCu = 2;                  // SiLU*mul quant: workgroups per CU
constexpr int kSiluLutPieces = 2;                 // ... 16-byte pieces per thread and step
constexpr int64_t kPlainLutMinElems = 1LL << 20;  // plain quant: table path from this many elements
constexpr int kPlainLutPerCu = 2;
constexpr int kPlainLutPieces = 2;
constexpr int64_t kPlainHalfMaxElems = (1LL << 20) - 1;   // plain quant: 4 values per thread below this
constexpr int kRmsRowsGroups = 2;                 // fused RMSNorm quant: 256-thread row groups per workgroup
constexpr int kRmsRowsPerCu = 2;                  // ... workgroups per CU

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
    for (int64_t v = threadIdx.x; v < nv; v += blockDim.x)
        ss = sumsq8(*reinterpret_cast<const uint4*>(row + v * 8), ss);
    ss = block_sum_f64(ss, lds);
    return rms_inv(ss, K, eps);
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

// Few elements (decode): the same codes with 4 values (8 bytes) per thread, so
// the per-element division and encode that follow the load are half as long.
__global__ __launch_bounds__(kQuantThreads) void k_quant_plain_half(
    const uint16_t* __restrict__ x, int64_t ldx, float s_act, uint8_t* __restrict__ xq, int64_t M, int64_t K)
{
    const int64_t nh = K >> 2, total = M * nh;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / nh, h = i - m * nh;
        const uint2 in = *reinterpret_cast<const uint2*>(x + m * ldx + h * 4);
        const uint32_t w[2] = {in.x, in.y};
        uint32_t o = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t b = (w[j >> 1] >> ((j & 1) * 16)) & 0xffffu;
            const uint32_t c = ((b & 0x7fffu) > 0x7f80u) ? (0x7fu | ((b >> 8) & 0x80u))
                                                         : f32_to_e4m3_sat(bf16_to_f32(b) / s_act);
            o |= c << (8 * j);
        }
        *reinterpret_cast<uint32_t*>(xq + m * K + h * 4) = o;
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
        *reinterpret_cast<uint2*>(xq + m * K + v * 8) = rms_quant8(in, g, r, s_act);
    }
}

// The same bytes as k_quant_rmsnorm with the division and the encode replaced
// by rms_codes8_cvt (exact quotients by multiply and fused multiply-add, the
// hardware E4M3 conversion; K <= 2048 * PPT, 2^-100 <= s_act <= 2^100, with
// rcp = fl32(1 / s_act) and sat = fl32(448 s_act) from the host).  Every
// value, inf and NaN included, takes the same path: no table, no fallback.
//
// A workgroup is G groups of 256 threads, persistent over rows: each group
// takes one row at a time and sums its squares in k_quant_rmsnorm's order
// (thread t: pieces t, t + 256, ...; xor butterfly per wave; the 4 wave sums
// in order), so r is bitwise the same.  A thread holds its pieces of the row
// and of gamma in registers and loads its pieces of the group's next row
// before the row's barrier.
template <int G>
struct RmsRowsShared {
    double part[2][G][kRmsRowThreads / 64];
};

// A thread's PPT pieces of row m (pieces t, t + 256, ...) through a buffer
// resource over that row: pieces past the row, and every piece of a row past
// M (a resource of 0 bytes), read as zeros without a branch, so the loads of a
// prefetched row stay in flight past the uses of the current one.  m is the
// same across the wave (one group is 4 whole waves).
template <int PPT>
__device__ __forceinline__ void load_row_pieces(const uint16_t* __restrict__ x, int64_t ldx, int m, int64_t M,
                                                int64_t K, int t, uint4 (&in)[PPT])
{
    const int mu = __builtin_amdgcn_readfirstlane(m);
    const bool live = mu < M;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(live ? x + (int64_t)mu * ldx : x), (short)0, live ? (int)(K * 2) : 0, 0x00020000);
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(rs, (t + p * kRmsRowThreads) * 16, 0, 0);
        in[p] = make_uint4(r.x, r.y, r.z, r.w);
    }
}

template <int PPT, int G>
__global__ __launch_bounds__(G * kRmsRowThreads) void k_quant_rmsnorm_rows(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ gamma, float eps,
    float s_act, float rcp, float sat, uint8_t* __restrict__ xq, int64_t M, int64_t K)
{
    __shared__ RmsRowsShared<G> sh;
    const int grp = threadIdx.x / kRmsRowThreads, t = threadIdx.x % kRmsRowThreads;
    const int wave = t >> 6, lane = t & 63;
    const int nv = (int)(K >> 3);
    const int64_t stride = (int64_t)gridDim.x * G;
    int64_t m = (int64_t)blockIdx.x * G + grp;
    // the group's rows m, m + stride, ... alternate between two buffers, so a
    // prefetched row is never copied (a copy would wait for its loads)
    uint4 buf[2][PPT];
    load_row_pieces<PPT>(x, ldx, (int)m, M, K, t, buf[0]);

    // gamma as fp32, fixed per thread
    float gf[PPT][8];
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
        const int v = t + p * kRmsRowThreads;
        const uint4 g = v < nv ? *reinterpret_cast<const uint4*>(gamma + (int64_t)v * 8) : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) gf[p][i] = bf16_to_f32((gw[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
    }

    // one row of the group: `in` holds it, `nx` receives the group's next row
    auto row_step = [&](const uint4 (&in)[PPT], uint4 (&nx)[PPT], int it) {
        double ss = 0.0;
#pragma unroll
        for (int p = 0; p < PPT; ++p) ss = sumsq8(in[p], ss);           // zero pieces add exact zeros
        load_row_pieces<PPT>(x, ldx, (int)(m + stride), M, K, t, nx);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
        if (lane == 0) sh.part[it & 1][grp][wave] = ss;
        __syncthreads();
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < kRmsRowThreads / 64; ++w) tot += sh.part[it & 1][grp][w];
        const float r = rms_inv(tot, K, eps);
        uint8_t* out = xq + m * K;
        if (m >= M) return;
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int v = t + p * kRmsRowThreads;
            const uint2 o = rms_codes8_cvt(in[p].x, in[p].y, in[p].z, in[p].w, gf[p], r, s_act, rcp, sat);
            if (v < nv) *reinterpret_cast<uint2*>(out + (int64_t)v * 8) = o;
        }
    };
    const int64_t first = (int64_t)blockIdx.x * G;       // the workgroup runs while its first group has a row
    for (int it = 0; first + it * stride < M;) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (first + it * stride >= M) break;
            row_step(buf[j], buf[j ^ 1], it);
            m += stride;
            ++it;
        }
    }
}

// ---- per-token dynamic quant: every row with its own scale ------------------

__device__ __forceinline__ float finite_abs_max(float acc, float v);

// The 8 values of piece v of a row that get quantized: x itself, or the bf16
// RMSNorm output (r the row's scale).
__device__ __forceinline__ void row_values8(const uint16_t* __restrict__ row, const uint16_t* __restrict__ gamma,
                                           float r, int64_t v, float y[8])
{
    const uint4 in = *reinterpret_cast<const uint4*>(row + v * 8);
    if (gamma) {
        rms_apply8(in, *reinterpret_cast<const uint4*>(gamma + v * 8), r, y);
    } else {
        const uint32_t w[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = bf16_to_f32((w[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
    }
}

// One workgroup per row: s_rows[m] = fl32(amax / 448) over the row's finite
// values (1 when 0), then the codes of fl32(y / s_rows[m]) (a NaN keeps its own
// sign, as in the static quant).  The row is re-read from L2 for each pass.
__global__ __launch_bounds__(kQuantThreads) void k_quant_per_token(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ gamma, float eps,
    uint8_t* __restrict__ xq, float* __restrict__ s_rows, int64_t K)
{
    __shared__ double lds[kQuantThreads / 64];
    __shared__ float ldsf[kQuantThreads / 64];
    const int64_t m = blockIdx.x;
    const uint16_t* row = x + m * ldx;
    const float r = gamma ? row_rms_inv(row, K, eps, lds) : 1.0f;
    const int64_t nv = K >> 3;
    float amax = 0.0f;
    for (int64_t v = threadIdx.x; v < nv; v += blockDim.x) {
        float y[8];
        row_values8(row, gamma, r, v, y);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = finite_abs_max(amax, y[j]);
    }
    amax = block_max_f32(amax, ldsf);
    const float s = amax == 0.0f ? 1.0f : amax / 448.0f;
    if (threadIdx.x == 0) s_rows[m] = s;
    for (int64_t v = threadIdx.x; v < nv; v += blockDim.x) {
        float y[8];
        row_values8(row, gamma, r, v, y);
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j >> 2] |= quant_value(y[j], s) << ((j & 3) * 8);
        *reinterpret_cast<uint2*>(xq + m * K + v * 8) = make_uint2(o[0], o[1]);
    }
}

// The same with the row held in registers (K <= 8 * 256 * PPT): one read of
// x, and the fp64 sum of squares taken in the generic kernel's order (each
// thread's pieces in turn, then the block reduction).
template <int PPT>
__global__ __launch_bounds__(kQuantThreads) void k_quant_per_token_reg(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ gamma, float eps,
    uint8_t* __restrict__ xq, float* __restrict__ s_rows, int64_t K)
{
    __shared__ double lds[kQuantThreads / 64];
    __shared__ float ldsf[kQuantThreads / 64];
    const int64_t m = blockIdx.x;
    const uint16_t* row = x + m * ldx;
    const int nv = (int)(K >> 3);
    uint4 in[PPT], gm[PPT];                             // gamma too: both loads in flight together
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
        const int v = threadIdx.x + p * kQuantThreads;
        in[p] = v < nv ? *reinterpret_cast<const uint4*>(row + (int64_t)v * 8) : make_uint4(0u, 0u, 0u, 0u);
        gm[p] = gamma && v < nv ? *reinterpret_cast<const uint4*>(gamma + (int64_t)v * 8)
                                : make_uint4(0u, 0u, 0u, 0u);
    }
    float r = 1.0f;
    if (gamma) {
        double ss = 0.0;
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const uint32_t w[4] = {in[p].x, in[p].y, in[p].z, in[p].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double f = (double)bf16_to_f32((w[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
                ss += f * f;                  // zero pieces past the row add exact zeros
            }
        }
        ss = block_sum_f64(ss, lds);
        r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
    }
    float y[PPT][8];
    float amax = 0.0f;
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
        if (gamma) {
            rms_apply8(in[p], gm[p], r, y[p]);
        } else {
            const uint32_t w[4] = {in[p].x, in[p].y, in[p].z, in[p].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) y[p][i] = bf16_to_f32((w[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = finite_abs_max(amax, y[p][j]);   // zero pieces: no effect
    }
    amax = block_max_f32(amax, ldsf);
    const float s = amax == 0.0f ? 1.0f : amax / 448.0f;
    if (threadIdx.x == 0) s_rows[m] = s;
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
        const int v = threadIdx.x + p * kQuantThreads;
        if (v >= nv) break;
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j >> 2] |= quant_value(y[p][j], s) << ((j & 3) * 8);
        *reinterpret_cast<uint2*>(xq + m * K + (int64_t)v * 8) = make_uint2(o[0], o[1]);
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

// h_b = bf16(fl32(s * u)) (bits) for one gate / up pair of bf16 bits, with
// s = silu(g) from `silu` (silu_f64 itself, or its table).
template <class Silu>
__device__ __forceinline__ uint32_t silu_mul1(uint32_t g, uint32_t u, Silu silu)
{
    return f32_to_bf16_rne(silu(g) * bf16_to_f32(u));
}

// silu_mul1 of the 8 gate / up values of one 16-byte load each.
template <class Silu>
__device__ __forceinline__ void silu_mul8(const uint4 g, const uint4 u, uint32_t hb[8], Silu silu)
{
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
        hb[i] = silu_mul1((gw[i >> 1] >> ((i & 1) * 16)) & 0xffffu, (uw[i >> 1] >> ((i & 1) * 16)) & 0xffffu, silu);
}

struct SiluDirect {
    __device__ float operator()(uint32_t b) const { return silu_f64(bf16_to_f32(b)); }
};

struct CodeDirect {
    float s_act;
    __device__ uint32_t operator()(uint32_t hb) const { return quant_value(bf16_to_f32(hb), s_act); }
};

// Few rows (decode): silu in fp64 and the IEEE division per element.  Each
// thread takes two elements (4-byte loads, a 2-byte store), so a decode step's
// M x I (8 x 17408: 70K threads) still spreads over every CU and each wave's
// serial fp64 work stays short.
__global__ __launch_bounds__(kQuantThreads) void k_silu_mul_quant(
    const uint16_t* __restrict__ gate, int64_t ldg, const uint16_t* __restrict__ up, int64_t ldu, float s_act,
    uint8_t* __restrict__ xq, int64_t M, int64_t I)
{
    const int64_t np = I >> 1, total = M * np;
    const CodeDirect code{s_act};
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = i / np, v = i - m * np;
        const uint32_t g = *reinterpret_cast<const uint32_t*>(gate + m * ldg + v * 2);
        const uint32_t u = *reinterpret_cast<const uint32_t*>(up + m * ldu + v * 2);
        const uint32_t lo = code(silu_mul1(g & 0xffffu, u & 0xffffu, SiluDirect{}));
        const uint32_t hi = code(silu_mul1(g >> 16, u >> 16, SiluDirect{}));
        *reinterpret_cast<uint16_t*>(xq + m * I + v * 2) = (uint16_t)(lo | (hi << 8));
    }
}

// The SiLU band table (silu_f64 of every band gate, both signs), evaluated by
// the compiler: each workgroup copies it into LDS instead of evaluating 8116
// fp64 SiLUs.
__device__ const SiluBandTable kSiluBandTableDev = make_silu_band_table();

// Many rows (prefill).  Each workgroup first copies the SiLU band table into
// LDS (32 KB: two 16-byte direct-to-LDS loads per thread) and fills the band
// code table of the plain quant under s_act (2.5 KB, one division per
// mantissa), 35 KB in all: two 1024-thread workgroups per CU (fewer
// workgroups when the pieces do not fill them), with its first step's loads
// already in flight.  The grid then
// sweeps the [M, I] pieces together, NP per thread per step (kSiluLutThreads
// apart, so each load instruction of a wave covers 1 KB), with one step of
// the whole grid between a thread's steps.  A piece past the end is loaded
// from the thread's first piece of the step and stores that piece's codes
// there again, so nothing branches around a load or a store.  Per piece the
// common case (silu_mul_codes8_fast) runs first; a piece with a gate outside
// the SiLU band or a NaN product takes the exact path.  total = M * I / 8 <
// 2^31.
constexpr int kSiluLutThreads = 1024;

// Non-temporal: the activation is read once.
__device__ __forceinline__ uint4 load_piece(const uint16_t* p)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(r.x, r.y, r.z, r.w);
}

template <int NP>
__global__ __launch_bounds__(kSiluLutThreads) void k_silu_mul_quant_lut(
    const uint16_t* __restrict__ gate, int64_t ldg, const uint16_t* __restrict__ up, int64_t ldu, float s_act,
    uint8_t* __restrict__ xq, uint32_t nv, uint32_t total, int64_t I)
{
    __shared__ __attribute__((aligned(16))) float stab[kSiluTableSize];
    __shared__ uint8_t ctab[kBandTableBytes];
    const uint32_t stride = gridDim.x * (uint32_t)(NP * kSiluLutThreads);
    uint32_t i = blockIdx.x * (uint32_t)(NP * kSiluLutThreads) + threadIdx.x;
    const bool live = i < total;
    // the pieces' rows and columns, stepped instead of divided: piece
    // ip + stride is dm rows and dv pieces further
    const uint32_t dm = stride / nv, dv = stride - dm * nv;
    uint32_t m[NP], v[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const uint32_t ip = live ? i + (uint32_t)p * kSiluLutThreads : 0u;
        m[p] = ip / nv;
        v[p] = ip - m[p] * nv;
    }
    uint4 g[NP], u[NP];
    auto load_step = [&]() {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const bool in = i + (uint32_t)p * kSiluLutThreads < total;
            const uint32_t mm = in ? m[p] : m[0], vv = in ? v[p] : v[0];
            g[p] = load_piece(gate + mm * ldg + vv * 8);
            u[p] = load_piece(up + mm * ldu + vv * 8);
        }
    };
    load_step();                                        // the first step's loads fly while the tables are built
    {
        // the SiLU table: 32 chunks of 1 KB, a wave's 64 lanes x 16 bytes each
        const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<SiluBandTable*>(&kSiluBandTableDev), (short)0, (int)sizeof(SiluBandTable), 0x00020000);
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
        for (int c = wave; c < (int)(sizeof(SiluBandTable) / 1024); c += kSiluLutThreads / 64)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, (lds_void*)(reinterpret_cast<uint8_t*>(stab) + c * 1024), 16,
                                                     c * 1024 + lane * 16, 0, 0, 0);
    }
    fill_plain_band_table(ctab, s_act, threadIdx.x, blockDim.x);
    const uint32_t lo1 = code_band_lo(s_act) - 1u;
    __syncthreads();                                    // both tables in LDS
    if (!live) return;
    for (;;) {
        __builtin_amdgcn_sched_barrier(0);              // every load of the step in flight before any use
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const bool in = i + (uint32_t)p * kSiluLutThreads < total;
            const uint32_t gw[4] = {g[p].x, g[p].y, g[p].z, g[p].w};
            const uint32_t uw[4] = {u[p].x, u[p].y, u[p].z, u[p].w};
            float t[8];
            uint2 o;
            if (!silu_mul_codes8_fast(gw, uw, stab, ctab, lo1, t, o)) o = silu_mul_codes8_exact(gw, uw, t, ctab, lo1);
            *reinterpret_cast<uint2*>(xq + (int64_t)(in ? m[p] : m[0]) * I + (in ? v[p] : v[0]) * 8) = o;
        }
        i += stride;
        if (i >= total) break;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            v[p] += dv;
            m[p] += dm + (v[p] >= nv ? 1u : 0u);
            v[p] -= v[p] >= nv ? nv : 0u;
        }
        load_step();
    }
}

// Plain static quant of many elements: the codes of quant8 from a 2563-byte
// table of the band of magnitudes whose code needs the division (entry
// kCodeBand + 2 is unused padding), a NaN keeping
// its sign.  Each workgroup issues its first step's loads, fills the table,
// then the grid sweeps the [M, K] pieces together, NP per thread per step (one
// grid step between a thread's steps), without branches: a piece past the end
// is loaded from the thread's first piece of the step and stores that piece's
// codes there again.  total = M * K / 8 < 2^31.
constexpr int kPlainLutThreads = 1024;
static_assert(kPlainLutThreads % 128 == 0 && kSiluLutThreads % 128 == 0,
              "fill_band_table: one mantissa per thread across the binades");

template <int NP>
__global__ __launch_bounds__(kPlainLutThreads) void k_quant_plain_lut(
    const uint16_t* __restrict__ x, int64_t ldx, float s_act, uint8_t* __restrict__ xq, uint32_t nv,
    uint32_t total, int64_t K)
{
    __shared__ uint8_t tab[kBandTableBytes];
    const uint32_t stride = gridDim.x * (uint32_t)(NP * kPlainLutThreads);
    uint32_t i = blockIdx.x * (uint32_t)(NP * kPlainLutThreads) + threadIdx.x;
    const bool live = i < total;
    const uint32_t dm = stride / nv, dv = stride - dm * nv;     // one grid step = dm rows + dv pieces
    uint32_t m[NP], v[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const uint32_t ip = live ? i + (uint32_t)p * kPlainLutThreads : 0u;
        m[p] = ip / nv;
        v[p] = ip - m[p] * nv;
    }
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    uint4 in[NP];
    auto load_step = [&]() {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const bool in_range = i + (uint32_t)p * kPlainLutThreads < total;
            const u32x4 r = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(x + (in_range ? m[p] : m[0]) * ldx + (in_range ? v[p] : v[0]) * 8));
            in[p] = make_uint4(r.x, r.y, r.z, r.w);
        }
    };
    load_step();                                        // the first step's loads fly while the table is built
    const int lo1 = (int)code_band_lo(s_act) - 1;
    fill_plain_band_table(tab, s_act, threadIdx.x, blockDim.x);
    __syncthreads();
    if (!live) return;
    for (;;) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const bool in_range = i + (uint32_t)p * kPlainLutThreads < total;
            *reinterpret_cast<uint2*>(xq + (int64_t)(in_range ? m[p] : m[0]) * K + (in_range ? v[p] : v[0]) * 8) =
                quant8_band(in[p].x, in[p].y, in[p].z, in[p].w, tab, lo1);
        }
        i += stride;
        if (i >= total) break;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            v[p] += dv;
            m[p] += dm + (v[p] >= nv ? 1u : 0u);
            v[p] -= v[p] >= nv ? nv : 0u;
        }
        load_step();
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
        uint32_t hb[8];
        silu_mul8(*reinterpret_cast<const uint4*>(gate + m * ldg + v * 8),
                  *reinterpret_cast<const uint4*>(up + m * ldu + v * 8), hb, SiluDirect{});
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = finite_abs_max(amax, bf16_to_f32(hb[j]));
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

// Load-time layout of a merged gate_up weight for the SiLU*mul epilogue: row
// 16t + i of w_il is gate row 8t + i (i < 8) or up row 8t + i - 8 (rows I +
// 8t + i - 8 of the merged [gate; up] weight), and s_il follows the rows.
// One thread per 16-byte piece.
__global__ __launch_bounds__(kQuantThreads) void k_interleave_gate_up(
    const uint8_t* __restrict__ wq, const float* __restrict__ s_w, uint8_t* __restrict__ w_il,
    float* __restrict__ s_il, int64_t I, int64_t K)
{
    const int64_t nv = K >> 4, total = 2 * I * nv;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / nv, v = i - row * nv;
        const int64_t t = row >> 4, k = row & 15;
        const int64_t src = k < 8 ? 8 * t + k : I + 8 * t + (k - 8);
        *reinterpret_cast<uint4*>(w_il + row * K + v * 16) = *reinterpret_cast<const uint4*>(wq + src * K + v * 16);
        if (v == 0) s_il[row] = s_w[src];
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
    const int64_t ppt = ((K >> 3) + kRmsRowThreads - 1) / kRmsRowThreads;   // 16-byte pieces per thread
    if (gamma && M < ((int64_t)1 << 30) && ppt <= 4 && code_table_ok(s_act)) {
        constexpr int G = kRmsRowsGroups;
        const int64_t want = (M + G - 1) / G, cap = (int64_t)num_cus() * kRmsRowsPerCu;
        const dim3 grid((uint32_t)(want < cap ? want : cap)), block(G * kRmsRowThreads);
        const float rcp = 1.0f / s_act, sat = 448.0f * s_act;     // the quotient's operands, rounded once
#define FP8MM_RMS_ROWS(PPT)                                                                                    \
    hipLaunchKernelGGL((k_quant_rmsnorm_rows<PPT, G>), grid, block, 0, stream, x, ldx, gamma, eps, s_act, rcp, sat, \
                       xq, M, K)
        if (ppt <= 1) FP8MM_RMS_ROWS(1);
        else if (ppt <= 2) FP8MM_RMS_ROWS(2);
        else if (ppt <= 3) FP8MM_RMS_ROWS(3);
        else FP8MM_RMS_ROWS(4);
#undef FP8MM_RMS_ROWS
    } else if (gamma) {
        hipLaunchKernelGGL(k_quant_rmsnorm, dim3((uint32_t)M), dim3(kQuantThreads), 0, stream,
                           x, ldx, gamma, eps, s_act, xq, K);
    } else if (M * (K >> 3) >= kPlainLutMinElems / 8 && M * (K >> 3) < ((int64_t)1 << 31) &&
               code_table_ok(s_act)) {
        const int64_t total = M * (K >> 3);
        const int64_t cap = (int64_t)num_cus() * kPlainLutPerCu;
        const int64_t need = (total + kPlainLutPieces * kPlainLutThreads - 1) / (kPlainLutPieces * kPlainLutThreads);
        hipLaunchKernelGGL((k_quant_plain_lut<kPlainLutPieces>), dim3((uint32_t)(need < cap ? need : cap)),
                           dim3(kPlainLutThreads), 0, stream, x, ldx, s_act, xq, (uint32_t)(K >> 3), (uint32_t)total, K);
    } else if (M * K <= kPlainHalfMaxElems) {
        const int64_t blocks = (M * (K >> 2) + kQuantThreads - 1) / kQuantThreads;
        hipLaunchKernelGGL(k_quant_plain_half, dim3((uint32_t)(blocks < 1 ? 1 : blocks)), dim3(kQuantThreads), 0,
                           stream, x, ldx, s_act, xq, M, K);
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

void launch_quant_per_token(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, uint8_t* xq,
                            float* s_rows, int64_t M, int64_t K, hipStream_t stream)
{
    const int64_t ppt = ((K >> 3) + kQuantThreads - 1) / kQuantThreads;   // 16-byte pieces per thread
    const dim3 grid((uint32_t)M), block(kQuantThreads);
    if (ppt <= 1)
        hipLaunchKernelGGL(k_quant_per_token_reg<1>, grid, block, 0, stream, x, ldx, gamma, eps, xq, s_rows, K);
    else if (ppt <= 2)
        hipLaunchKernelGGL(k_quant_per_token_reg<2>, grid, block, 0, stream, x, ldx, gamma, eps, xq, s_rows, K);
    else if (ppt <= 4)
        hipLaunchKernelGGL(k_quant_per_token_reg<4>, grid, block, 0, stream, x, ldx, gamma, eps, xq, s_rows, K);
    else if (ppt <= 9)
        hipLaunchKernelGGL(k_quant_per_token_reg<9>, grid, block, 0, stream, x, ldx, gamma, eps, xq, s_rows, K);
    else
        hipLaunchKernelGGL(k_quant_per_token, grid, block, 0, stream, x, ldx, gamma, eps, xq, s_rows, K);
}

static bool silu_mul_uses_table(int64_t M, int64_t I, float s_act)
{
    const int64_t total = M * (I >> 3);
    return total >= FP8MM_SILU_TABLE_MIN_ELEMS / 8 && total < ((int64_t)1 << 31) && code_table_ok(s_act);
}

void launch_silu_mul_quant(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu, float s_act,
                           uint8_t* xq, int64_t M, int64_t I, hipStream_t stream)
{
    const int64_t total = M * (I >> 3);
    if (silu_mul_uses_table(M, I, s_act)) {
        // up to two workgroups per CU, fewer when the pieces do not fill them
        const int64_t cap = (int64_t)num_cus() * kSiluLutPerCu;
        const int64_t need = (total + kSiluLutPieces * kSiluLutThreads - 1) / (kSiluLutPieces * kSiluLutThreads);
        const int64_t grid = need < cap ? need : cap;
        hipLaunchKernelGGL((k_silu_mul_quant_lut<kSiluLutPieces>), dim3((uint32_t)grid),
                           dim3(kSiluLutThreads), 0, stream, gate, ldg,
                           up, ldu, s_act, xq, (uint32_t)(I >> 3), (uint32_t)total, I);
    } else {
        // two elements per thread, at most 4096 workgroups (grid-stride beyond)
        const int64_t blocks = (M * (I >> 1) + kQuantThreads - 1) / kQuantThreads;
        hipLaunchKernelGGL(k_silu_mul_quant, dim3((uint32_t)(blocks < 4096 ? blocks : 4096)), dim3(kQuantThreads),
                           0, stream, gate, ldg, up, ldu, s_act, xq, M, I);
    }
}


void launch_act_scale_silu_mul(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu, int64_t M,
                               int64_t I, float* s_act, float* partial, hipStream_t stream)
{
    const int64_t np = plain_grid(M, I);
    hipLaunchKernelGGL(k_absmax_silu_mul, dim3((uint32_t)np), dim3(kQuantThreads), 0, stream, gate, ldg, up, ldu, M,
                       I, partial);
    hipLaunchKernelGGL(k_absmax_final, dim3(1), dim3(kQuantThreads), 0, stream, partial, np, s_act);
}

// Scratch of fp8_act_scale_noalloc: the partial maxima of k_absmax_plain /
// k_absmax_rmsnorm, read by k_absmax_final.  Each GPU holds its own copy at its
// own address; host code uses the address hipGetSymbolAddress returns for the
// current device, never the array's name (a host-side stand-in).
static __device__ __align__(256) float scratch[FP8MM_NOALLOC_SCRATCH_FLOATS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(float** ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<float*>(p);
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

void launch_quant_weight(const float* w, int64_t N, int64_t K, uint8_t* wq, float* s_w, hipStream_t stream)
{
    hipLaunchKernelGGL(k_quant_weight, dim3((uint32_t)N), dim3(kQuantThreads), 0, stream, w, K, wq, s_w);
}

void launch_interleave_gate_up(const uint8_t* wq, const float* s_w, uint8_t* w_il, float* s_il, int64_t I,
                               int64_t K, hipStream_t stream)
{
    const int64_t blocks = (2 * I * (K >> 4) + kQuantThreads - 1) / kQuantThreads;
    hipLaunchKernelGGL(k_interleave_gate_up, dim3((uint32_t)(blocks < 4096 ? blocks : 4096)), dim3(kQuantThreads), 0,
                       stream, wq, s_w, w_il, s_il, I, K);
}

}  // namespace fp8mm
