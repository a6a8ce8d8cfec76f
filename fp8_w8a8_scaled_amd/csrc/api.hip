// api.hip -- the C ABI of libfp8mm (declared in include/fp8mm.h): argument
// validation (fail closed), the M-threshold dispatcher, the merge predicate and
// the launches.  No call allocates, synchronizes or throws.
//
// Dispatcher: the small-M arm serves M <= T, the large-M arm M > T.  The branch
// is a pure function of M (and T), re-decided on every call, so a captured
// graph freezes the same branch an eager call takes; thresholds in [2,16) are
// rejected so that decode / speculative-verify batches (M <= 8) never leave the
// memory-bound arm (vLLM PR #53014, Marlin large-M commit message).
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "internal.h"

namespace {

// Default threshold: the largest M served by the small-M arm.  Measured on
// MI355X for the decode-MLP gate_up (34816 x 5120): the small-M arm takes 37 us
// at M = 32 against 65 us for the large-M arm, and 81 us at M = 40 against 66.
constexpr int64_t kDefaultThreshold = 32;

int64_t initial_threshold()
{
    const char* e = std::getenv("FP8MM_LARGE_M_THRESHOLD");
    if (e && *e) {
        char* end = nullptr;
        const long long v = std::strtoll(e, &end, 10);
        if (end && *end == '\0' && v >= FP8MM_THRESHOLD_MIN && v <= FP8MM_SMALL_M_MAX) return (int64_t)v;
    }
    return kDefaultThreshold;
}

std::atomic<int64_t> g_threshold{initial_threshold()};

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool good_scale(float s) { return std::isfinite(s) && s > 0.0f; }

int launch_status()
{
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? FP8MM_OK : FP8MM_ELAUNCH;
}

// One output shard of either output type.
struct OutShard {
    int64_t n;
    void* out;
    int64_t ldo;
};

// Shared validation of the GEMM operands; fills the shard table.  Rows of an
// output start 16-byte aligned: ldo a multiple of 8 (bf16) or 4 (f32).
int check_gemm(const uint8_t* x_q, const uint8_t* w_q, float s_act, const float* s_w,
               const OutShard* shards, int num_shards, bool f32, int64_t M, int64_t K,
               fp8mm::ShardTable* tab, int64_t* N_out)
{
    tab->s_rows = nullptr;
    // Sizes and scalars first; an empty product (M == 0 or N == 0) is a no-op
    // that may come with null pointers (empty tensors).
    if (!shards || M < 0 || K < 0 || num_shards < 1 || num_shards > FP8MM_MAX_SHARDS) return FP8MM_EINVAL;
    if (!good_scale(s_act)) return FP8MM_EINVAL;
    int64_t N = 0;
    tab->num = num_shards;
    tab->f32 = f32 ? 1 : 0;
    for (int i = 0; i < num_shards; ++i) {
        const OutShard& s = shards[i];
        if (s.n < 0 || s.ldo < s.n) return FP8MM_EINVAL;
        if (M > 0 && s.n > 0 && !s.out) return FP8MM_EINVAL;
        if (s.n % 16 != 0) return FP8MM_EUNSUPPORTED;
        // an empty shard is never written: its stride and pointer are not checked
        if (s.n > 0 && (s.ldo % (f32 ? 4 : 8) != 0 || !aligned16(s.out))) return FP8MM_EUNSUPPORTED;
        tab->start[i] = N;
        tab->out[i] = s.out;
        tab->ldo[i] = s.ldo;
        N += s.n;
    }
    tab->start[num_shards] = N;
    if (K % 16 != 0) return FP8MM_EUNSUPPORTED;
    *N_out = N;
    if (M == 0 || N == 0) return FP8MM_OK;
    if (!x_q || !w_q || !s_w) return FP8MM_EINVAL;
    if (K == 0) return FP8MM_EUNSUPPORTED;
    if (!aligned16(x_q) || !aligned16(w_q) || !aligned16(s_w)) return FP8MM_EUNSUPPORTED;
    if (M > (int64_t)65535 * 128 || N / 16 > (int64_t)0x7fffffff) return FP8MM_EUNSUPPORTED;
    *N_out = N;
    return FP8MM_OK;
}

int run_gemm(const uint8_t* x_q, const uint8_t* w_q, float s_act, const float* s_w,
             const OutShard* shards, int num_shards, bool f32, int64_t M, int64_t K, int arm,
             void* workspace, size_t workspace_bytes, hipStream_t stream, bool per_row = false,
             const float* s_rows = nullptr)
{
    fp8mm::ShardTable tab{};
    int64_t N = 0;
    int st = check_gemm(x_q, w_q, s_act, s_w, shards, num_shards, f32, M, K, &tab, &N);
    if (st != FP8MM_OK) return st;
    if (per_row) {                                       // s_act is unused: device per-row scales instead
        if (M > 0 && N > 0 && !s_rows) return FP8MM_EINVAL;
        if (reinterpret_cast<uintptr_t>(s_rows) & 3u) return FP8MM_EUNSUPPORTED;
        tab.s_rows = s_rows;
    }
    if (workspace_bytes < fp8_scaled_mm_workspace_bytes(M, N, K)) return FP8MM_EWORKSPACE;
    (void)workspace;
    if (M == 0 || N == 0) return FP8MM_OK;
    if (arm < 0) arm = fp8_scaled_mm_select(M, N, K);
    if (arm == 0) {
        if (M > FP8MM_SMALL_M_MAX) return FP8MM_EINVAL;
        fp8mm::launch_gemm_small_m(x_q, w_q, s_act, s_w, tab, M, N, K, stream);
    } else if (arm == 1) {
        fp8mm::launch_gemm_large_m(x_q, w_q, s_act, s_w, tab, M, N, K, stream);
    } else {
        return FP8MM_EINVAL;
    }
    return launch_status();
}

}  // namespace

extern "C" {

int fp8_quant_rmsnorm(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, float s_act,
                      uint8_t* x_q, int64_t M, int64_t K, hipStream_t stream)
{
    if (M < 0 || K < 0 || ldx < K) return FP8MM_EINVAL;
    if (!good_scale(s_act)) return FP8MM_EINVAL;
    if (gamma && !(std::isfinite(eps) && eps >= 0.0f)) return FP8MM_EINVAL;
    if (K % 16 != 0 || ldx % 8 != 0) return FP8MM_EUNSUPPORTED;
    if (M == 0 || K == 0) return FP8MM_OK;
    if (!x || !x_q) return FP8MM_EINVAL;
    if (!aligned16(x) || !aligned16(x_q) || (gamma && !aligned16(gamma))) return FP8MM_EUNSUPPORTED;
    if (gamma && M > (int64_t)0x7fffffff) return FP8MM_EUNSUPPORTED;
    // x_q must not overlap x
    const uintptr_t xb = reinterpret_cast<uintptr_t>(x), xe = xb + (uintptr_t)((M - 1) * ldx + K) * 2;
    const uintptr_t qb = reinterpret_cast<uintptr_t>(x_q), qe = qb + (uintptr_t)(M * K);
    if (qb < xe && xb < qe) return FP8MM_EINVAL;
    fp8mm::launch_quant(x, ldx, gamma, eps, s_act, x_q, M, K, stream);
    return launch_status();
}

int fp8_scaled_mm(const uint8_t* x_q, const uint8_t* w_q, float s_act, const float* s_w,
                  uint16_t* out, int64_t ldo, int64_t M, int64_t N, int64_t K,
                  void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (N < 0) return FP8MM_EINVAL;
    const OutShard one{N, out, ldo};
    return run_gemm(x_q, w_q, s_act, s_w, &one, 1, false, M, K, -1, workspace, workspace_bytes, stream);
}

int fp8_scaled_mm_arm(const uint8_t* x_q, const uint8_t* w_q, float s_act, const float* s_w,
                      uint16_t* out, int64_t ldo, int64_t M, int64_t N, int64_t K, int arm,
                      void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (N < 0 || (arm != 0 && arm != 1)) return FP8MM_EINVAL;
    if (arm == 0 && M > FP8MM_SMALL_M_MAX) return FP8MM_EINVAL;
    const OutShard one{N, out, ldo};
    return run_gemm(x_q, w_q, s_act, s_w, &one, 1, false, M, K, arm, workspace, workspace_bytes, stream);
}

int fp8_scaled_mm_merged(const uint8_t* x_q, const uint8_t* w_q, float s_act, const float* s_w,
                         const fp8_shard_t* shards, int num_shards, int64_t M, int64_t K,
                         void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!shards || num_shards < 1 || num_shards > FP8MM_MAX_SHARDS) return FP8MM_EINVAL;
    OutShard tab[FP8MM_MAX_SHARDS];
    for (int i = 0; i < num_shards; ++i) tab[i] = OutShard{shards[i].n, shards[i].out, shards[i].ldo};
    return run_gemm(x_q, w_q, s_act, s_w, tab, num_shards, false, M, K, -1, workspace, workspace_bytes, stream);
}

int fp8_quant_scaled_mm_fused(int64_t M, int64_t N, int64_t K, int64_t ldx, float s_act, int rmsnorm)
{
    if (M < 1 || N < 1 || K < 1 || N % 16 != 0 || K % 16 != 0 || ldx < K || ldx % 8 != 0 || !good_scale(s_act))
        return 0;
    return fp8_scaled_mm_select(M, N, K) == 0 && fp8mm::quant_gemm_small_m_fits(M, N, K, ldx, s_act, rmsnorm != 0)
               ? 1 : 0;
}

int fp8_quant_rmsnorm_scaled_mm_merged(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, float s_act,
                                       uint8_t* x_q, const uint8_t* w_q, const float* s_w,
                                       const fp8_shard_t* shards, int num_shards, int64_t M, int64_t K,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!shards || num_shards < 1 || num_shards > FP8MM_MAX_SHARDS) return FP8MM_EINVAL;
    // the quant's arguments (as fp8_quant_rmsnorm)
    if (M < 0 || K < 0 || ldx < K) return FP8MM_EINVAL;
    if (!good_scale(s_act)) return FP8MM_EINVAL;
    if (gamma && !(std::isfinite(eps) && eps >= 0.0f)) return FP8MM_EINVAL;
    if (K % 16 != 0 || ldx % 8 != 0) return FP8MM_EUNSUPPORTED;
    if (M > 0 && K > 0) {
        if (!x || !x_q) return FP8MM_EINVAL;
        if (!aligned16(x) || !aligned16(x_q) || (gamma && !aligned16(gamma))) return FP8MM_EUNSUPPORTED;
        if (gamma && M > (int64_t)0x7fffffff) return FP8MM_EUNSUPPORTED;
        const uintptr_t xb = reinterpret_cast<uintptr_t>(x), xe = xb + (uintptr_t)((M - 1) * ldx + K) * 2;
        const uintptr_t qb = reinterpret_cast<uintptr_t>(x_q), qe = qb + (uintptr_t)(M * K);
        if (qb < xe && xb < qe) return FP8MM_EINVAL;
    }
    // the GEMM's arguments
    OutShard tab[FP8MM_MAX_SHARDS];
    for (int i = 0; i < num_shards; ++i) tab[i] = OutShard{shards[i].n, shards[i].out, shards[i].ldo};
    fp8mm::ShardTable st{};
    int64_t N = 0;
    const int rc = check_gemm(x_q, w_q, s_act, s_w, tab, num_shards, false, M, K, &st, &N);
    if (rc != FP8MM_OK) return rc;
    if (workspace_bytes < fp8_scaled_mm_workspace_bytes(M, N, K)) return FP8MM_EWORKSPACE;
    if (M == 0 || K == 0) return FP8MM_OK;
    if (fp8_quant_scaled_mm_fused(M, N, K, ldx, s_act, gamma != nullptr) &&
        fp8mm::launch_quant_gemm_small_m(x, ldx, gamma, eps, x_q, w_q, s_act, s_w, st, M, N, K, stream))
        return launch_status();
    fp8mm::launch_quant(x, ldx, gamma, eps, s_act, x_q, M, K, stream);
    if (N == 0) return launch_status();
    const int qs = launch_status();
    if (qs != FP8MM_OK) return qs;
    return run_gemm(x_q, w_q, s_act, s_w, tab, num_shards, false, M, K, -1, workspace, workspace_bytes, stream);
}

int fp8_quant_scaled_mm_merged(const uint16_t* x, int64_t ldx, float s_act, uint8_t* x_q,
                               const uint8_t* w_q, const float* s_w, const fp8_shard_t* shards, int num_shards,
                               int64_t M, int64_t K, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    return fp8_quant_rmsnorm_scaled_mm_merged(x, ldx, nullptr, 0.0f, s_act, x_q, w_q, s_w, shards, num_shards, M, K,
                                              workspace, workspace_bytes, stream);
}

int fp8_scaled_mm_f32(const uint8_t* x_q, const uint8_t* w_q, float s_act, const float* s_w,
                      float* out, int64_t ldo, int64_t M, int64_t N, int64_t K,
                      void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (N < 0) return FP8MM_EINVAL;
    const OutShard one{N, out, ldo};
    return run_gemm(x_q, w_q, s_act, s_w, &one, 1, true, M, K, -1, workspace, workspace_bytes, stream);
}

int fp8_scaled_mm_merged_f32(const uint8_t* x_q, const uint8_t* w_q, float s_act, const float* s_w,
                             const fp8_shard_f32_t* shards, int num_shards, int64_t M, int64_t K,
                             void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!shards || num_shards < 1 || num_shards > FP8MM_MAX_SHARDS) return FP8MM_EINVAL;
    OutShard tab[FP8MM_MAX_SHARDS];
    for (int i = 0; i < num_shards; ++i) tab[i] = OutShard{shards[i].n, shards[i].out, shards[i].ldo};
    return run_gemm(x_q, w_q, s_act, s_w, tab, num_shards, true, M, K, -1, workspace, workspace_bytes, stream);
}

int fp8_quant_per_token(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, uint8_t* x_q,
                        float* s_rows, int64_t M, int64_t K, hipStream_t stream)
{
    if (M < 0 || K < 0 || ldx < K) return FP8MM_EINVAL;
    if (gamma && !(std::isfinite(eps) && eps >= 0.0f)) return FP8MM_EINVAL;
    if (K % 16 != 0 || ldx % 8 != 0) return FP8MM_EUNSUPPORTED;
    if (M == 0) return FP8MM_OK;
    if (!x || !x_q || !s_rows) return FP8MM_EINVAL;
    if (K == 0) return FP8MM_EUNSUPPORTED;               // a row with no values has no scale
    if (!aligned16(x) || !aligned16(x_q) || (gamma && !aligned16(gamma)) ||
        (reinterpret_cast<uintptr_t>(s_rows) & 3u))
        return FP8MM_EUNSUPPORTED;
    if (M > (int64_t)0x7fffffff) return FP8MM_EUNSUPPORTED;
    const uintptr_t xb = reinterpret_cast<uintptr_t>(x), xe = xb + (uintptr_t)((M - 1) * ldx + K) * 2;
    const uintptr_t qb = reinterpret_cast<uintptr_t>(x_q), qe = qb + (uintptr_t)(M * K);
    const uintptr_t sb = reinterpret_cast<uintptr_t>(s_rows), se = sb + (uintptr_t)M * 4;
    if ((qb < xe && xb < qe) || (sb < xe && xb < se) || (sb < qe && qb < se)) return FP8MM_EINVAL;
    fp8mm::launch_quant_per_token(x, ldx, gamma, eps, x_q, s_rows, M, K, stream);
    return launch_status();
}

int fp8_scaled_mm_per_token(const uint8_t* x_q, const uint8_t* w_q, const float* s_rows, const float* s_w,
                            uint16_t* out, int64_t ldo, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (N < 0) return FP8MM_EINVAL;
    const OutShard one{N, out, ldo};
    return run_gemm(x_q, w_q, 1.0f, s_w, &one, 1, false, M, K, -1, workspace, workspace_bytes, stream, true,
                    s_rows);
}

int fp8_scaled_mm_merged_per_token(const uint8_t* x_q, const uint8_t* w_q, const float* s_rows, const float* s_w,
                                   const fp8_shard_t* shards, int num_shards, int64_t M, int64_t K,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!shards || num_shards < 1 || num_shards > FP8MM_MAX_SHARDS) return FP8MM_EINVAL;
    OutShard tab[FP8MM_MAX_SHARDS];
    for (int i = 0; i < num_shards; ++i) tab[i] = OutShard{shards[i].n, shards[i].out, shards[i].ldo};
    return run_gemm(x_q, w_q, 1.0f, s_w, tab, num_shards, false, M, K, -1, workspace, workspace_bytes, stream, true,
                    s_rows);
}

size_t fp8_scaled_mm_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    (void)M; (void)N; (void)K;
    return 0;   // both arms reduce on chip: no split-K partials leave the workgroup
}

int fp8_scaled_mm_select(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0) return FP8MM_EINVAL;
    return M <= g_threshold.load(std::memory_order_relaxed) ? 0 : 1;
}

int fp8_set_large_m_threshold(int64_t t)
{
    if (t < FP8MM_THRESHOLD_MIN || t > FP8MM_SMALL_M_MAX) return FP8MM_EINVAL;
    g_threshold.store(t, std::memory_order_relaxed);
    return FP8MM_OK;
}

int64_t fp8_get_large_m_threshold(void) { return g_threshold.load(std::memory_order_relaxed); }

int fp8_scales_bitwise_equal(const float* s, int n)
{
    if (!s || n < 1) return FP8MM_EINVAL;
    uint32_t first;
    std::memcpy(&first, &s[0], 4);
    for (int i = 1; i < n; ++i) {
        uint32_t b;
        std::memcpy(&b, &s[i], 4);
        if (b != first) return 0;
    }
    return 1;
}

const char* fp8mm_strerror(int status)
{
    switch (status) {
    case FP8MM_OK: return "ok";
    case FP8MM_EINVAL: return "invalid argument (null pointer, negative size, bad scale or out-of-range value)";
    case FP8MM_EUNSUPPORTED: return "unsupported shape or alignment (K%16, N%16, ld%8, 16-byte pointers)";
    case FP8MM_EWORKSPACE: return "workspace too small";
    case FP8MM_ELAUNCH: return "HIP kernel launch failed";
    case FP8MM_ESCRATCH: return "input needs more scratch than the allocation-free entry point's static array holds";
    default: return "unknown status";
    }
}

int fp8_quant_weight(const float* w, int64_t N, int64_t K, uint8_t* w_q, float* s_w, hipStream_t stream)
{
    if (N < 0 || K < 0) return FP8MM_EINVAL;
    if (K % 16 != 0) return FP8MM_EUNSUPPORTED;
    if (N == 0) return FP8MM_OK;
    if (!s_w || (K > 0 && (!w || !w_q))) return FP8MM_EINVAL;
    if (!aligned16(w) || !aligned16(w_q) || !aligned16(s_w)) return FP8MM_EUNSUPPORTED;
    if (N > (int64_t)0x7fffffff) return FP8MM_EUNSUPPORTED;
    if (K == 0) return FP8MM_EUNSUPPORTED;   // no row to take a scale from
    fp8mm::launch_quant_weight(w, N, K, w_q, s_w, stream);
    return launch_status();
}

namespace {

// Validation shared by the SiLU*mul entry points.
int check_silu_mul(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu, int64_t M, int64_t I,
                   bool* empty)
{
    *empty = false;
    if (M < 0 || I < 0 || ldg < I || ldu < I) return FP8MM_EINVAL;
    if (I % 16 != 0 || ldg % 8 != 0 || ldu % 8 != 0) return FP8MM_EUNSUPPORTED;
    if (M == 0 || I == 0) {
        *empty = true;
        return FP8MM_OK;
    }
    if (!gate || !up) return FP8MM_EINVAL;
    if (!aligned16(gate) || !aligned16(up)) return FP8MM_EUNSUPPORTED;
    return FP8MM_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t ab = reinterpret_cast<uintptr_t>(a), bb = reinterpret_cast<uintptr_t>(b);
    return ab < bb + nb && bb < ab + na;
}

}  // namespace

int fp8_silu_mul_quant(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu, float s_act,
                       uint8_t* x_q, int64_t M, int64_t I, hipStream_t stream)
{
    bool empty = false;
    const int st = check_silu_mul(gate, ldg, up, ldu, M, I, &empty);
    if (st != FP8MM_OK) return st;
    if (!good_scale(s_act)) return FP8MM_EINVAL;
    if (empty) return FP8MM_OK;
    if (!x_q) return FP8MM_EINVAL;
    if (!aligned16(x_q)) return FP8MM_EUNSUPPORTED;
    const size_t gb = (size_t)((M - 1) * ldg + I) * 2, ub = (size_t)((M - 1) * ldu + I) * 2, qb = (size_t)(M * I);
    if (overlaps(x_q, qb, gate, gb) || overlaps(x_q, qb, up, ub)) return FP8MM_EINVAL;
    fp8mm::launch_silu_mul_quant(gate, ldg, up, ldu, s_act, x_q, M, I, stream);
    return launch_status();
}

int fp8_act_scale_silu_mul(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu, int64_t M,
                           int64_t I, float* s_act, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    bool empty = false;
    const int st = check_silu_mul(gate, ldg, up, ldu, M, I, &empty);
    if (st != FP8MM_OK) return st;
    if (empty || !s_act) return FP8MM_EINVAL;           // no tensor to calibrate on
    if (!workspace || workspace_bytes < fp8_act_scale_workspace_bytes(M, I)) return FP8MM_EWORKSPACE;
    if (!aligned16(workspace)) return FP8MM_EUNSUPPORTED;
    fp8mm::launch_act_scale_silu_mul(gate, ldg, up, ldu, M, I, s_act, static_cast<float*>(workspace), stream);
    return launch_status();
}

int fp8_interleave_gate_up(const uint8_t* w_q, const float* s_w, uint8_t* w_il, float* s_il, int64_t I, int64_t K,
                           hipStream_t stream)
{
    if (I < 0 || K < 0) return FP8MM_EINVAL;
    if (I % 16 != 0 || K % 16 != 0) return FP8MM_EUNSUPPORTED;
    if (I == 0) return FP8MM_OK;
    if (K == 0) return FP8MM_EUNSUPPORTED;
    if (!w_q || !s_w || !w_il || !s_il) return FP8MM_EINVAL;
    if (!aligned16(w_q) || !aligned16(w_il) || !aligned16(s_w) || !aligned16(s_il)) return FP8MM_EUNSUPPORTED;
    if (I > ((int64_t)1 << 40) / K) return FP8MM_EUNSUPPORTED;
    const size_t wb = (size_t)(2 * I * K), sb = (size_t)(2 * I) * 4;
    if (overlaps(w_il, wb, w_q, wb) || overlaps(w_il, wb, s_w, sb) || overlaps(s_il, sb, w_q, wb) ||
        overlaps(s_il, sb, s_w, sb) || overlaps(s_il, sb, w_il, wb))
        return FP8MM_EINVAL;
    fp8mm::launch_interleave_gate_up(w_q, s_w, w_il, s_il, I, K, stream);
    return launch_status();
}

int fp8_gate_up_silu_quant_fused(int64_t M, int64_t I, int64_t K, int64_t ldx, float s_act, float s_down, int quant)
{
    if (M < 1 || I < 1 || K < 1 || I % 16 != 0 || K % 16 != 0 || quant < 0 || quant > 2 || !good_scale(s_act) ||
        !good_scale(s_down))
        return 0;
    if (quant && (ldx < K || ldx % 8 != 0)) return 0;
    return fp8_scaled_mm_select(M, 2 * I, K) == 0 && fp8mm::gate_up_silu_fits(M, I, K, ldx, s_act, s_down, quant)
               ? 1 : 0;
}

int fp8_gate_up_silu_quant(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, float s_act,
                           uint8_t* x_q, const uint8_t* w_il, const float* s_il, float s_down, uint8_t* h_q,
                           int64_t M, int64_t I, int64_t K, hipStream_t stream)
{
    if (M < 0 || I < 0 || K < 0) return FP8MM_EINVAL;
    if (!good_scale(s_act) || !good_scale(s_down)) return FP8MM_EINVAL;
    if (gamma && (!x || !(std::isfinite(eps) && eps >= 0.0f))) return FP8MM_EINVAL;
    if (x && ldx < K) return FP8MM_EINVAL;
    if (I % 16 != 0 || K % 16 != 0 || (x && ldx % 8 != 0)) return FP8MM_EUNSUPPORTED;
    if (M == 0 || I == 0) return FP8MM_OK;
    if (K == 0) return FP8MM_EUNSUPPORTED;
    if (!w_il || !s_il || !h_q || (!x && !x_q)) return FP8MM_EINVAL;
    if (!aligned16(w_il) || !aligned16(s_il) || !aligned16(h_q) || (x_q && !aligned16(x_q)) || (x && !aligned16(x)) ||
        (gamma && !aligned16(gamma)))
        return FP8MM_EUNSUPPORTED;
    // h_q is written, and x_q too when the quant runs in the launch
    const size_t hb = (size_t)(M * I), qb = (size_t)(M * K), wb = (size_t)(2 * I * K), sb = (size_t)(2 * I) * 4;
    const size_t xb = x ? (size_t)((M - 1) * ldx + K) * 2 : 0;
    if (overlaps(h_q, hb, w_il, wb) || overlaps(h_q, hb, s_il, sb) || (x_q && overlaps(h_q, hb, x_q, qb)) ||
        (x && overlaps(h_q, hb, x, xb)) || (gamma && overlaps(h_q, hb, gamma, (size_t)K * 2)))
        return FP8MM_EINVAL;
    if (x && x_q && (overlaps(x_q, qb, x, xb) || overlaps(x_q, qb, w_il, wb) || overlaps(x_q, qb, s_il, sb) ||
                     (gamma && overlaps(x_q, qb, gamma, (size_t)K * 2))))
        return FP8MM_EINVAL;
    const int quant = x ? (gamma ? 2 : 1) : 0;
    if (!fp8_gate_up_silu_quant_fused(M, I, K, ldx, s_act, s_down, quant)) return FP8MM_EUNSUPPORTED;
    if (!fp8mm::launch_gate_up_silu(x, ldx, gamma, eps, x_q, w_il, s_act, s_il, M, I, K, s_down, h_q, stream))
        return FP8MM_EUNSUPPORTED;
    return launch_status();
}

size_t fp8_act_scale_workspace_bytes(int64_t M, int64_t K)
{
    if (M <= 0 || K <= 0) return 0;
    const size_t a = fp8mm::act_scale_partials(M, K, true), b = fp8mm::act_scale_partials(M, K, false);
    return (a > b ? a : b) * sizeof(float);
}

int fp8_act_scale(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, int64_t M, int64_t K,
                  float* s_act, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!x || !s_act || M < 0 || K < 0 || ldx < K) return FP8MM_EINVAL;
    if (gamma && !(std::isfinite(eps) && eps >= 0.0f)) return FP8MM_EINVAL;
    if (K % 16 != 0 || ldx % 8 != 0 || !aligned16(x) || (gamma && !aligned16(gamma))) return FP8MM_EUNSUPPORTED;
    if (gamma && M > (int64_t)0x7fffffff) return FP8MM_EUNSUPPORTED;
    if (M == 0 || K == 0) return FP8MM_EINVAL;   // no tensor to calibrate on
    if (!workspace || workspace_bytes < fp8_act_scale_workspace_bytes(M, K)) return FP8MM_EWORKSPACE;
    if (!aligned16(workspace)) return FP8MM_EUNSUPPORTED;
    fp8mm::launch_act_scale(x, ldx, gamma, eps, M, K, s_act, static_cast<float*>(workspace), stream);
    return launch_status();
}

int fp8_act_scale_noalloc(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, int64_t M, int64_t K,
                          float* s_act, hipStream_t stream)
{
    if (!x || !s_act || M < 0 || K < 0 || ldx < K) return FP8MM_EINVAL;
    if (gamma && !(std::isfinite(eps) && eps >= 0.0f)) return FP8MM_EINVAL;
    if (K % 16 != 0 || ldx % 8 != 0 || !aligned16(x) || (gamma && !aligned16(gamma))) return FP8MM_EUNSUPPORTED;
    if (gamma && M > (int64_t)0x7fffffff) return FP8MM_EUNSUPPORTED;
    if (M == 0 || K == 0) return FP8MM_EINVAL;   // no tensor to calibrate on
    if (fp8mm::act_scale_partials(M, K, gamma != nullptr) > (size_t)FP8MM_NOALLOC_SCRATCH_FLOATS) return FP8MM_ESCRATCH;
    float* partial = nullptr;
    if (fp8mm::noalloc_scratch(&partial) != hipSuccess || !partial) return FP8MM_ELAUNCH;
    fp8mm::launch_act_scale(x, ldx, gamma, eps, M, K, s_act, partial, stream);
    return launch_status();
}

size_t fp8_quant_weight_per_tensor_workspace_bytes(int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0) return 0;
    return fp8mm::weight_absmax_partials(N, K) * sizeof(float);
}

int fp8_quant_weight_per_tensor(const float* w, int64_t N, int64_t K, uint8_t* w_q, float* s_w, void* workspace,
                                size_t workspace_bytes, hipStream_t stream)
{
    if (N < 0 || K < 0) return FP8MM_EINVAL;
    if (K % 16 != 0) return FP8MM_EUNSUPPORTED;
    if (N == 0 || K == 0) return FP8MM_EINVAL;           // no value to take a scale from
    if (!w || !w_q || !s_w) return FP8MM_EINVAL;
    if (N > ((int64_t)1 << 40) / K) return FP8MM_EUNSUPPORTED;
    if (!workspace || workspace_bytes < fp8_quant_weight_per_tensor_workspace_bytes(N, K)) return FP8MM_EWORKSPACE;
    if (!aligned16(w) || !aligned16(w_q) || !aligned16(workspace) || (reinterpret_cast<uintptr_t>(s_w) & 3u))
        return FP8MM_EUNSUPPORTED;
    const size_t wb = (size_t)(N * K) * 4, qb = (size_t)(N * K), pb = workspace_bytes;
    if (overlaps(w_q, qb, w, wb) || overlaps(s_w, 4, w, wb) || overlaps(s_w, 4, w_q, qb) ||
        overlaps(workspace, pb, w, wb) || overlaps(workspace, pb, w_q, qb) || overlaps(workspace, pb, s_w, 4))
        return FP8MM_EINVAL;
    fp8mm::launch_quant_weight_per_tensor(w, N, K, w_q, s_w, static_cast<float*>(workspace), stream);
    return launch_status();
}

}  // extern "C"

namespace {

// Host shard table of per-tensor scales; rows and scales validated.
int shard_scales_table(const int64_t* shard_rows, const float* shard_scales, int num_shards,
                       fp8mm::ShardScales* tab)
{
    if (!shard_rows || !shard_scales || num_shards < 1 || num_shards > FP8MM_MAX_SHARDS) return FP8MM_EINVAL;
    tab->num = num_shards;
    int64_t r = 0;
    for (int i = 0; i < num_shards; ++i) {
        if (shard_rows[i] < 0 || !good_scale(shard_scales[i])) return FP8MM_EINVAL;
        if (shard_rows[i] > ((int64_t)1 << 40)) return FP8MM_EUNSUPPORTED;
        tab->start[i] = r;
        tab->scale[i] = shard_scales[i];
        r += shard_rows[i];
    }
    tab->start[num_shards] = r;
    return FP8MM_OK;
}

}  // namespace

extern "C" {

int fp8_expand_shard_scales(const int64_t* shard_rows, const float* shard_scales, int num_shards, float* s_w,
                            hipStream_t stream)
{
    fp8mm::ShardScales tab{};
    const int st = shard_scales_table(shard_rows, shard_scales, num_shards, &tab);
    if (st != FP8MM_OK) return st;
    if (tab.start[num_shards] == 0) return FP8MM_OK;
    if (!s_w) return FP8MM_EINVAL;
    if (reinterpret_cast<uintptr_t>(s_w) & 3u) return FP8MM_EUNSUPPORTED;
    fp8mm::launch_expand_shard_scales(tab, s_w, stream);
    return launch_status();
}

int fp8_requant_max_scale(const uint8_t* w_q, uint8_t* w_out, int64_t K, const int64_t* shard_rows,
                          const float* shard_scales, int num_shards, float* s_w, float* s_max_out,
                          hipStream_t stream)
{
    fp8mm::ShardScales tab{};
    const int st = shard_scales_table(shard_rows, shard_scales, num_shards, &tab);
    if (st != FP8MM_OK) return st;
    if (K < 0) return FP8MM_EINVAL;
    if (K % 16 != 0) return FP8MM_EUNSUPPORTED;
    float s_max = shard_scales[0];
    for (int i = 1; i < num_shards; ++i) s_max = shard_scales[i] > s_max ? shard_scales[i] : s_max;
    const int64_t rows = tab.start[num_shards];
    if (rows > ((int64_t)1 << 40) / (K > 0 ? K : 1)) return FP8MM_EUNSUPPORTED;
    if (rows > 0) {
        if (!s_w || (K > 0 && (!w_q || !w_out))) return FP8MM_EINVAL;
        if ((K > 0 && (!aligned16(w_q) || !aligned16(w_out))) || (reinterpret_cast<uintptr_t>(s_w) & 3u))
            return FP8MM_EUNSUPPORTED;
        const size_t wb = (size_t)(rows * K), sb = (size_t)rows * 4;
        if (K > 0 && w_out != w_q && overlaps(w_out, wb, w_q, wb)) return FP8MM_EINVAL;
        if (K > 0 && (overlaps(s_w, sb, w_q, wb) || overlaps(s_w, sb, w_out, wb))) return FP8MM_EINVAL;
        if (K > 0) {
            fp8mm::launch_requant_max_scale(w_q, w_out, tab, s_max, K, s_w, stream);
        } else {
            fp8mm::ShardScales one = tab;                  // no weight bytes: only the scale vector
            for (int i = 0; i < num_shards; ++i) one.scale[i] = s_max;
            fp8mm::launch_expand_shard_scales(one, s_w, stream);
        }
        const int ls = launch_status();
        if (ls != FP8MM_OK) return ls;
    }
    if (s_max_out) *s_max_out = s_max;
    return FP8MM_OK;
}

int fp8_merge_admit(const float* input_scales, int num_shards, int policy, float* s_act_out)
{
    if (!input_scales || !s_act_out || num_shards < 1 || num_shards > FP8MM_MAX_SHARDS) return FP8MM_EINVAL;
    if (policy != FP8MM_MERGE_EXACT && policy != FP8MM_MERGE_MAX_SCALE) return FP8MM_EINVAL;
    float s_max = input_scales[0];
    for (int i = 0; i < num_shards; ++i) {
        if (!good_scale(input_scales[i])) return FP8MM_EINVAL;
        s_max = input_scales[i] > s_max ? input_scales[i] : s_max;
    }
    if (policy == FP8MM_MERGE_MAX_SCALE) {
        *s_act_out = s_max;
        return 1;
    }
    if (fp8_scales_bitwise_equal(input_scales, num_shards) != 1) return 0;
    *s_act_out = input_scales[0];
    return 1;
}

}  // extern "C"
