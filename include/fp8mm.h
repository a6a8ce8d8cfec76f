/*
 * fp8mm.h -- C ABI of the MI355X (gfx950) FP8 E4M3 W8A8 scaled-matmul layer.
 *
 * The layer (one linear projection of a quantized LLM's decode or prefill step):
 *
 *     out[m,n] = bf16( (sum_k x_q[m,k] * W_q[n,k]) * s_act * s_w[n] )
 *     x_q      = saturating round-to-nearest-even E4M3( x / s_act )
 *
 * Sources (web pages):
 *   - bmm_fp8(a, b, scale_a, scale_b, out_dtype, backend): vllm.cpp issue #252
 *     ("FP8 tower's cuBLASLt default rests on a false premise"), "CORRECTION".
 *   - bf16 (model dtype) output instead of F32: vllm.cpp issue #417 ("We emit F32
 *     where vLLM emits bf16"), Finding 1; vllm.cpp issue #213 ("Qwen3.6 NVFP4
 *     baselines must reach vLLM speed parity"), original post, instance 2.
 *   - static per-tensor activation scale, quantize-once and the fused
 *     RMSNorm->fp8 quant (byte-exact against the unfused path): vllm.cpp #417,
 *     ranked follow-ons; vllm.cpp #213, "The GDN fp8 merge predicate FIRES".
 *   - merged projections (qkvz, qkv, gate_up) and merging only on bitwise-equal
 *     input scales: vllm.cpp #252, "SETTLED BY PAIRED TRACE"; vllm.cpp #213,
 *     "merge predicate FIRES"; vllm.cpp #417, ranked follow-ons.
 *   - an M-threshold dispatch between a memory-bound small-M kernel and a
 *     compute-bound large-M kernel, decided per call as a pure function of M,
 *     thresholds in [2,16) rejected, workspaces never allocated in the forward:
 *     vLLM PR #53014 ("[Kernel] add Flashinfer cutedsl w4a16 linear"), the
 *     Marlin large-M commit message.
 *   - per-output-channel weight scales ("FP8 channelwise"): same commit message.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns every
 *     buffer (inputs, outputs, weights, scales, workspaces); the library never
 *     calls hipMalloc/hipFree.  Its only device memory of its own is the fixed
 *     static scratch array of fp8_act_scale_noalloc (FP8MM_NOALLOC_SCRATCH_FLOATS
 *     floats per GPU, held until the process ends).
 *   - Every GPU call is asynchronous on `stream` (0 = the null stream), never
 *     synchronizes and returns an int status (enum below).  No C++ exception
 *     crosses the ABI.
 *   - M == 0 (or N == 0) is a no-op returning FP8MM_OK.
 *   - Layouts are row-major.  E4M3 is OCP E4M3FN (bias 7, max 448, S.1111.111 =
 *     NaN, no infinity), one byte per value.  bf16 is passed as uint16_t bits.
 *   - Fail closed: a shape or alignment the kernels do not cover returns
 *     FP8MM_EUNSUPPORTED (there is no silent slow path):
 *       K % 16 == 0, N % 16 == 0 (each merged shard too), ldx % 8 == 0,
 *       ldo % 8 == 0, and every pointer 16-byte aligned.
 *   - FP8MM_EINVAL: a null pointer, a negative size, a leading dimension smaller
 *     than the row, a non-finite or non-positive scale, an out-of-range
 *     argument.
 *   - FP8MM_ELAUNCH: the HIP runtime reported an error for the launch.
 *   - Kernel choice depends only on (M, N, K) and the threshold, so a stream
 *     capture into a HIP graph freezes exactly the branch an eager call takes.
 *   - Results are bitwise deterministic run to run (no floating-point atomics),
 *     and column n of a merged call is bitwise equal to the same column of a
 *     separate call on that shard.
 */
#ifndef FP8MM_H
#define FP8MM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fp8mm_status {
    FP8MM_OK = 0,
    FP8MM_EINVAL = -1,
    FP8MM_EUNSUPPORTED = -2,
    FP8MM_EWORKSPACE = -3,
    FP8MM_ELAUNCH = -4,
    FP8MM_ESCRATCH = -5
};

/* Largest M the small-M (memory-bound) kernel serves; the threshold may not
 * exceed it. */
#define FP8MM_SMALL_M_MAX 64
/* Smallest threshold accepted: M <= 8 (decode and speculative-verify batches)
 * must always stay on the small-M kernel. */
#define FP8MM_THRESHOLD_MIN 16
/* Most shards one merged call takes. */
#define FP8MM_MAX_SHARDS 8

/* ------------------------------------------------------------------------
 * Activation quantization (quantize-once): vllm.cpp #417, ranked follow-ons
 * (InputLayernormFp8 / QuantFp8Static, "byte-exact quant fusion").
 *
 * gamma != NULL -- fused RMSNorm -> FP8, per row m:
 *     r      = fl32( 1 / sqrt( (sum_k x[m,k]^2) / K + eps ) )   (sum and sqrt in fp64)
 *     y      = bf16_RNE( fl32( fl32(x[m,k] * r) * gamma[k] ) )
 *     x_q    = satRNE_E4M3( fl32( y / s_act ) )
 * gamma == NULL -- plain static quant: x_q = satRNE_E4M3( fl32( x / s_act ) );
 *     eps is ignored.
 * Division is IEEE fp32 division.  Values >= 448 in magnitude (inf included)
 * saturate to +-448, NaN gives 0x7F/0xFF, and a negative value that rounds to
 * zero gives 0x80.
 *
 * x     : bf16 [M, K], row stride ldx (elements, ldx >= K).
 * gamma : bf16 [K] or NULL.
 * s_act : static per-tensor scale, finite and > 0 (FP8MM_EINVAL otherwise).
 * x_q   : E4M3 [M, K], contiguous (row stride K); must not overlap x.
 * With 2^-100 <= s_act <= 2^100, the fused form for K <= 8192 computes each
 * quotient by multiply and fused multiply-add (exact: the same quotient as the
 * division) and encodes it with the hardware conversion, and the plain form
 * from 2^20 elements on takes each code from a per-workgroup table of the
 * same divisions (a NaN keeps the per-element rule); the bytes are the same.
 * ---------------------------------------------------------------------- */
int fp8_quant_rmsnorm(const uint16_t* x, int64_t ldx,
                      const uint16_t* gamma, float eps,
                      float s_act,
                      uint8_t* x_q,
                      int64_t M, int64_t K, hipStream_t stream);

/* ------------------------------------------------------------------------
 * SiLU*mul -> FP8: the MLP activation between the merged gate_up projection and
 * the down projection, quantized once for the down GEMM (the gate/up pair of
 * the tower: vllm.cpp #252, "SETTLED BY PAIRED TRACE"; quantize-once input of
 * the next GEMM: vllm.cpp #417, ranked follow-ons).  Per element:
 *     s    = fl32( g / (1 + exp(-g)) )            (evaluated in fp64)
 *     h    = bf16_RNE( fl32( s * u ) )             (the unfused activation's bf16)
 *     x_q  = satRNE_E4M3( fl32( h / s_act ) )      (NaN h: 0x7F/0xFF)
 * so the bytes equal fp8_quant_rmsnorm(gamma = NULL) applied to the bf16
 * activation an unfused silu_and_mul would write.  The sign of a NaN that the
 * arithmetic itself creates (g = -inf, 0 * inf) is not specified.
 *
 * gate, up : bf16 [M, I], row strides ldg, ldu (elements, >= I, multiples of
 *            8); typically the two halves of the gate_up output (up = gate + I,
 *            ldg = ldu = 2 I).
 * s_act    : static per-tensor scale of the down projection's input, finite > 0.
 * x_q      : E4M3 [M, I], contiguous; must not overlap gate or up.
 * I % 16 == 0 and 16-byte aligned pointers (FP8MM_EUNSUPPORTED otherwise).
 * From FP8MM_SILU_TABLE_MIN_ELEMS elements on (M * I below 2^34, and
 * 2^-100 <= s_act <= 2^100) the kernel takes silu and the E4M3 code from
 * per-workgroup tables of the same evaluations instead of evaluating them per
 * element; the bytes are the same.
 * ---------------------------------------------------------------------- */
#define FP8MM_SILU_TABLE_MIN_ELEMS (1LL << 19)
int fp8_silu_mul_quant(const uint16_t* gate, int64_t ldg,
                       const uint16_t* up, int64_t ldu,
                       float s_act, uint8_t* x_q,
                       int64_t M, int64_t I, hipStream_t stream);

/* Static scale calibration for fp8_silu_mul_quant: *s_act (DEVICE f32) =
 * fl32(amax / 448), amax the largest finite |h| over the [M, I] activation
 * (1 when amax == 0).  workspace: at least fp8_act_scale_workspace_bytes(M, I)
 * bytes.  M == 0 or I == 0 is FP8MM_EINVAL (nothing to calibrate on). */
int fp8_act_scale_silu_mul(const uint16_t* gate, int64_t ldg,
                           const uint16_t* up, int64_t ldu,
                           int64_t M, int64_t I, float* s_act,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Scaled FP8 GEMM with bf16 output (bmm_fp8 with scale_a = s_act, scale_b =
 * s_w, out_dtype = bf16): vllm.cpp #252 "CORRECTION"; vllm.cpp #417 Finding 1.
 *
 *     out[m,n] = bf16_RNE( fl32( fl32(acc[m,n] * s_act) * s_w[n] ) ),
 *     acc[m,n] = sum_k dec(x_q[m,k]) * dec(w_q[n,k])   (fp32 accumulation)
 *
 * x_q  : E4M3 [M, K], contiguous.
 * w_q  : E4M3 [N, K], row-major, K contiguous ([out, in], as checkpoints store it).
 * s_act: per-tensor activation scale (by value), finite and > 0.
 * s_w  : f32 [N] per-output-channel weight scales.
 * out  : bf16 [M, N], row stride ldo >= N.
 * workspace / workspace_bytes: caller-provided scratch of at least
 *     fp8_scaled_mm_workspace_bytes(M, N, K) bytes (may be NULL/0 when that is
 *     0); FP8MM_EWORKSPACE if too small.
 * The kernel is chosen by fp8_scaled_mm_select(M, N, K).
 * ---------------------------------------------------------------------- */
int fp8_scaled_mm(const uint8_t* x_q, const uint8_t* w_q,
                  float s_act, const float* s_w,
                  uint16_t* out, int64_t ldo,
                  int64_t M, int64_t N, int64_t K,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Same as fp8_scaled_mm but with the kernel forced: arm 0 = small-M
 * (memory-bound, M <= FP8MM_SMALL_M_MAX), arm 1 = large-M (MFMA-tiled, any M).
 * For tests of both arms against each other and for threshold sweeps.
 * FP8MM_EINVAL for another arm or for arm 0 with M > FP8MM_SMALL_M_MAX. */
int fp8_scaled_mm_arm(const uint8_t* x_q, const uint8_t* w_q,
                      float s_act, const float* s_w,
                      uint16_t* out, int64_t ldo,
                      int64_t M, int64_t N, int64_t K, int arm,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Merged projection: ONE launch over the physically concatenated weight of
 * several projections that share x_q and s_act (GDN qkv+z -> qkvz, attention
 * q/k/v -> qkv, MLP gate/up -> gate_up): vllm.cpp #252 "SETTLED BY PAIRED
 * TRACE" (merging is the lever: shape and fusion, not library).
 *
 * w_q  : E4M3 [sum n_i, K]; s_w: f32 [sum n_i].
 * shards (HOST array, read during the call only): shard i covers weight rows
 *     [sum_{j<i} n_j, sum_{j<=i} n_j) and writes bf16 [M, n_i] to out_i with
 *     row stride ldo_i >= n_i.  n_i % 16 == 0; an empty shard (n_i == 0)
 *     is never written and its out_i and ldo_i are not checked.
 *     1 <= num_shards <= 8.
 * Merge admission is the caller's: merge only shards whose input scales are
 * bitwise equal (fp8_scales_bitwise_equal); otherwise call fp8_scaled_mm per
 * shard.  Column n of shard i is bitwise equal to the same column of a
 * separate fp8_scaled_mm call on that shard.
 * ---------------------------------------------------------------------- */
typedef struct fp8_shard {
    int64_t n;        /* output columns (weight rows) of this shard */
    uint16_t* out;    /* device, bf16 [M, n] */
    int64_t ldo;      /* row stride of out, elements */
} fp8_shard_t;

int fp8_scaled_mm_merged(const uint8_t* x_q, const uint8_t* w_q,
                         float s_act, const float* s_w,
                         const fp8_shard_t* shards, int num_shards,
                         int64_t M, int64_t K,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Static quant and merged projection in one call: x_q = the codes of
 * fp8_quant_rmsnorm(x, gamma = NULL, s_act), then fp8_scaled_mm_merged on
 * them (the quantize-once follow-on of vllm.cpp #417, its ranked follow-ons:
 * one launch instead of a quant launch per projection).  For 1 <= M <= 8 on
 * the small-M arm, with 2^-100 <= s_act <= 2^100 and an LDS plan for the
 * shape, ONE kernel does both: every workgroup encodes the activation rows
 * it multiplies by (the correctly rounded fp32 quotient x / s_act from the
 * reciprocal and fused multiply-adds, then the hardware E4M3 conversion) and
 * workgroup 0 writes x_q.  Otherwise the two calls run back to back.  Either
 * way x_q and the outputs are bitwise those of the two separate calls.
 *
 * x      : bf16 [M, K] (DEVICE), row stride ldx >= K (a multiple of 8),
 *          16-byte aligned.
 * s_act  : static per-tensor scale, finite > 0.
 * x_q    : E4M3 [M, K] (DEVICE), contiguous, written; must not overlap x.
 * w_q, s_w, shards, num_shards, workspace: as fp8_scaled_mm_merged.
 * Errors: those of fp8_quant_rmsnorm and fp8_scaled_mm_merged; nothing is
 * launched on an error.
 * ---------------------------------------------------------------------- */
int fp8_quant_scaled_mm_merged(const uint16_t* x, int64_t ldx, float s_act, uint8_t* x_q,
                               const uint8_t* w_q, const float* s_w,
                               const fp8_shard_t* shards, int num_shards,
                               int64_t M, int64_t K,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same with the fused RMSNorm quant: x_q = fp8_quant_rmsnorm(x, gamma,
 * eps, s_act), then fp8_scaled_mm_merged (gamma == NULL: exactly
 * fp8_quant_scaled_mm_merged).  One kernel where the plain form takes one and
 * the rows are 36..40 chunks of 128 (K of 4608..5120: 8 waves, whose chunks
 * hold each of the standalone kernel's 256 summing threads in one lane, so the
 * row sums keep its order): the workgroups compute each row's r, then encode.
 * x_q and the outputs are bitwise those of the two separate calls.
 * gamma: bf16 [K] (DEVICE), 16-byte aligned, or NULL; eps finite >= 0.
 * Errors: those of fp8_quant_rmsnorm and fp8_scaled_mm_merged. */
int fp8_quant_rmsnorm_scaled_mm_merged(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps,
                                       float s_act, uint8_t* x_q, const uint8_t* w_q, const float* s_w,
                                       const fp8_shard_t* shards, int num_shards, int64_t M, int64_t K,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* 1 if fp8_quant_scaled_mm_merged (rmsnorm = 0) or
 * fp8_quant_rmsnorm_scaled_mm_merged with a gamma (rmsnorm != 0) runs as one
 * launch for an [M, K] activation of row stride ldx, N output columns in total
 * and scale s_act; else 0 (also for arguments it would reject).  Host-only:
 * launches nothing. */
int fp8_quant_scaled_mm_fused(int64_t M, int64_t N, int64_t K, int64_t ldx, float s_act, int rmsnorm);

/* ------------------------------------------------------------------------
 * Merged gate_up projection with the SiLU*mul -> FP8 quant as its epilogue
 * (the gate/up pair of the tower, vllm.cpp #252 "SETTLED BY PAIRED TRACE";
 * quantize once for the next GEMM, vllm.cpp #417, ranked follow-ons): for the
 * decode MLP, one launch computes
 *     h_q = fp8_silu_mul_quant(gate, up, s_down)
 * of [gate | up] = fp8_scaled_mm_merged(x_q, [W_gate; W_up], s_act, s_w)
 * without writing the bf16 gate_up output; with x != NULL the activation
 * quant runs in the same launch as in fp8_quant_rmsnorm_scaled_mm_merged
 * (gamma != NULL: the fused RMSNorm quant).  h_q (and x_q when written) are
 * bitwise those of the separate calls on the merged weight.
 *
 * The weight comes in the layout fp8_interleave_gate_up writes: each 16-row
 * tile holds 8 gate rows, then the up rows of the same 8 columns, so one
 * workgroup owns both halves of every column it reduces.
 *
 * x, ldx, gamma, eps: as fp8_quant_rmsnorm_scaled_mm_merged, or x == NULL
 *          (and gamma == NULL): x_q is the input.
 * s_act  : static scale of x_q, finite > 0.
 * x_q    : E4M3 [M, K] (DEVICE), contiguous: the input when x == NULL, else
 *          written when not NULL.
 * w_il   : E4M3 [2I, K] (DEVICE), interleaved; s_il: f32 [2I], interleaved.
 * s_down : static scale of h_q (the down projection's input), finite > 0.
 * h_q    : E4M3 [M, I] (DEVICE), contiguous, written; overlaps no input.
 * I % 16 == 0, K % 16 == 0, 16-byte aligned pointers.  FP8MM_EUNSUPPORTED
 * (nothing launched) unless fp8_gate_up_silu_quant_fused accepts the call:
 * the caller then runs the separate calls on the merged weight.
 * ---------------------------------------------------------------------- */
int fp8_gate_up_silu_quant(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, float s_act,
                           uint8_t* x_q, const uint8_t* w_il, const float* s_il, float s_down, uint8_t* h_q,
                           int64_t M, int64_t I, int64_t K, hipStream_t stream);

/* 1 if fp8_gate_up_silu_quant takes an [M, K] activation (row stride ldx),
 * I gate columns and the scales s_act, s_down, with quant = 0 (x_q given),
 * 1 (plain static quant of x) or 2 (fused RMSNorm quant); else 0.  It needs
 * the small-M arm (fp8_scaled_mm_select(M, 2I, K) == 0), M <= 32 (M <= 8 with
 * the quant in the launch), 2^-100 <= s_down <= 2^100 (and s_act with the
 * quant), and a plan of whole 16-row tiles per workgroup.  Host-only. */
int fp8_gate_up_silu_quant_fused(int64_t M, int64_t I, int64_t K, int64_t ldx, float s_act, float s_down, int quant);

/* Load-time layout for fp8_gate_up_silu_quant: from the merged gate_up
 * weight w_q = [W_gate; W_up] (E4M3 [2I, K]) and its scales s_w (f32 [2I]),
 * row 16t + i of w_il is gate row 8t + i for i < 8 and up row 8t + i - 8
 * (merged row I + 8t + i - 8) for i >= 8; s_il follows the rows.  A copy:
 * outputs must not overlap inputs.  I % 16 == 0, K % 16 == 0, 16-byte
 * aligned pointers. */
int fp8_interleave_gate_up(const uint8_t* w_q, const float* s_w, uint8_t* w_il, float* s_il, int64_t I, int64_t K,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * F32-output variants (the A/B of vllm.cpp #417 Finding 1: an F32 output
 * doubles the bytes of the largest activation buffers against the model's
 * bf16).  Same kernels, same arithmetic and kernel choice; the epilogue stores
 *
 *     out[m,n] = fl32( fl32(acc[m,n] * s_act) * s_w[n] )
 *
 * instead of its bf16 rounding, so bf16_RNE of an F32 result equals the bf16
 * entry point's result bit for bit.  out: f32 [M, N] (shard i: f32 [M, n_i]),
 * row stride ldo a multiple of 4 (16-byte rows), 16-byte aligned.
 * ---------------------------------------------------------------------- */
typedef struct fp8_shard_f32 {
    int64_t n;        /* output columns (weight rows) of this shard */
    float* out;       /* device, f32 [M, n] */
    int64_t ldo;      /* row stride of out, elements */
} fp8_shard_f32_t;

int fp8_scaled_mm_f32(const uint8_t* x_q, const uint8_t* w_q,
                      float s_act, const float* s_w,
                      float* out, int64_t ldo,
                      int64_t M, int64_t N, int64_t K,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

int fp8_scaled_mm_merged_f32(const uint8_t* x_q, const uint8_t* w_q,
                             float s_act, const float* s_w,
                             const fp8_shard_f32_t* shards, int num_shards,
                             int64_t M, int64_t K,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Per-token dynamic activation scales: the scale granularity vllm.cpp #252
 * leaves open ("What is owed", item 2: per-tensor vs per-channel vs
 * per-token).  Each row is quantized as a tensor of its own:
 *
 *     s_rows[m] = fl32( amax_k |y[m,k]| / 448 )   (finite values; 1 when 0)
 *     x_q[m,k]  = satRNE_E4M3( fl32( y[m,k] / s_rows[m] ) )
 *
 * with y = x (gamma == NULL) or the bf16 RMSNorm output of fp8_quant_rmsnorm.
 * s_rows: DEVICE f32 [M] (4-byte aligned), written by the quant; it must not
 * overlap x or x_q.  Other arguments and checks as fp8_quant_rmsnorm.
 * ---------------------------------------------------------------------- */
int fp8_quant_per_token(const uint16_t* x, int64_t ldx,
                        const uint16_t* gamma, float eps,
                        uint8_t* x_q, float* s_rows,
                        int64_t M, int64_t K, hipStream_t stream);

/* The GEMM with per-row activation scales (device s_rows [M], as written by
 * fp8_quant_per_token):
 *     out[m,n] = bf16_RNE( fl32( fl32(acc[m,n] * s_rows[m]) * s_w[n] ) )
 * Same kernels, dispatcher and checks as fp8_scaled_mm / _merged. */
int fp8_scaled_mm_per_token(const uint8_t* x_q, const uint8_t* w_q,
                            const float* s_rows, const float* s_w,
                            uint16_t* out, int64_t ldo,
                            int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

int fp8_scaled_mm_merged_per_token(const uint8_t* x_q, const uint8_t* w_q,
                                   const float* s_rows, const float* s_w,
                                   const fp8_shard_t* shards, int num_shards,
                                   int64_t M, int64_t K,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes fp8_scaled_mm / _merged need for (M, N, K) (N = sum n_i).
 * 0 when the chosen kernel needs none.  Pure host function. */
size_t fp8_scaled_mm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Dispatcher (pure host function of M and the threshold T):
 * returns 0 (small-M kernel) when M <= T, 1 (large-M kernel) otherwise.
 * M <= 8 always returns 0 because T >= 16.  Negative sizes -> FP8MM_EINVAL. */
int fp8_scaled_mm_select(int64_t M, int64_t N, int64_t K);

/* Set the threshold T.  Accepts FP8MM_THRESHOLD_MIN <= t <= FP8MM_SMALL_M_MAX;
 * anything else (including t in [2,16)) returns FP8MM_EINVAL and leaves T
 * unchanged.  The initial T is the built-in default unless the environment
 * variable FP8MM_LARGE_M_THRESHOLD holds a valid value when the library loads.
 * Set T at start-up: a call that races with a concurrent GEMM call on another
 * thread may take either value. */
int fp8_set_large_m_threshold(int64_t t);
int64_t fp8_get_large_m_threshold(void);

/* Merge predicate (host): 1 iff all n f32 values in the HOST array s have the
 * same bit pattern (so 0.0 != -0.0 and NaN == NaN only with equal payloads),
 * 0 otherwise, FP8MM_EINVAL for s == NULL or n < 1. */
int fp8_scales_bitwise_equal(const float* s, int n);

/* Static string for a status code. */
const char* fp8mm_strerror(int status);

/* ------------------------------------------------------------------------
 * Load-time helpers (not on the per-step path).
 * ---------------------------------------------------------------------- */

/* Per-output-channel weight quantization:
 *     s_w[n]   = fl32( max_k |w[n,k]| / 448 )   (1 for an all-zero row)
 *     w_q[n,k] = satRNE_E4M3( fl32( w[n,k] / s_w[n] ) )
 * w: f32 [N, K] row-major; w_q: E4M3 [N, K]; s_w: f32 [N]. */
int fp8_quant_weight(const float* w, int64_t N, int64_t K,
                     uint8_t* w_q, float* s_w, hipStream_t stream);

/* Static activation scale calibration: *s_act = fl32(amax / 448) where amax is
 * the largest finite |value| of the tensor that fp8_quant_rmsnorm with the same
 * (x, ldx, gamma, eps, M, K) would quantize (x itself when gamma == NULL, the
 * bf16 RMSNorm output otherwise); 1 when amax == 0.  s_act is a DEVICE f32.
 * workspace must hold fp8_act_scale_workspace_bytes(M, K) bytes. */
size_t fp8_act_scale_workspace_bytes(int64_t M, int64_t K);
int fp8_act_scale(const uint16_t* x, int64_t ldx,
                  const uint16_t* gamma, float eps,
                  int64_t M, int64_t K, float* s_act,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* fp8_act_scale without a workspace, for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same *s_act bits, with the partial
 * maxima kept in a static device array of FP8MM_NOALLOC_SCRATCH_FLOATS floats
 * (one copy per GPU, held until the process ends).  The first call on a device
 * looks up that device's copy (hipGetSymbolAddress); no call allocates.
 * The scratch needs fp8_act_scale_workspace_bytes(M, K) / 4 floats (at most
 * 4096 without gamma, M with gamma); more returns FP8MM_ESCRATCH before any
 * launch.  Every call on one GPU shares its array (each call writes all the
 * partials it reads, nothing needs clearing): calls that overlap on one GPU,
 * on different streams or host threads, race and must not be issued. */
#define FP8MM_NOALLOC_SCRATCH_FLOATS 65536
int fp8_act_scale_noalloc(const uint16_t* x, int64_t ldx,
                          const uint16_t* gamma, float eps,
                          int64_t M, int64_t K, float* s_act, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Merged projections whose shards carry per-tensor scales (the q/k/v shards
 * of an attention projection, or qkv and z): vllm.cpp #417, ranked follow-ons
 * (one implementation keeps q/k/v apart unless their input scales are bitwise
 * equal; another always merges and requantizes mismatched shards to the
 * largest weight scale, which is lossy); vllm.cpp #213, "The GDN fp8 merge
 * predicate FIRES".  All load-time calls except fp8_merge_admit (host only).
 * ---------------------------------------------------------------------- */

/* Per-tensor weight quantization (one scale for the whole weight):
 *     *s_w     = fl32( max |w| / 448 )   over all N*K values (1 when all zero;
 *                a NaN is skipped, an inf makes the scale inf)
 *     w_q[n,k] = satRNE_E4M3( fl32( w[n,k] / *s_w ) )
 * w: f32 [N, K]; w_q: E4M3 [N, K]; s_w: DEVICE f32 [1] (4-byte aligned).
 * workspace: at least fp8_quant_weight_per_tensor_workspace_bytes(N, K) bytes,
 * 16-byte aligned.  N == 0 or K == 0 is FP8MM_EINVAL (no value to take a scale
 * from); K % 16 != 0 is FP8MM_EUNSUPPORTED. */
size_t fp8_quant_weight_per_tensor_workspace_bytes(int64_t N, int64_t K);
int fp8_quant_weight_per_tensor(const float* w, int64_t N, int64_t K,
                                uint8_t* w_q, float* s_w,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Exact merge: expand per-tensor shard scales into the per-channel vector the
 * GEMMs take, s_w[r] = shard_scales[i] for every weight row r of shard i.  A
 * merged call with this s_w gives, column for column, the bits of a separate
 * call per shard with that shard's scale.
 * shard_rows, shard_scales: HOST arrays of num_shards (1..8) entries; rows >= 0,
 * scales finite and > 0.  s_w: DEVICE f32 [sum shard_rows], 4-byte aligned. */
int fp8_expand_shard_scales(const int64_t* shard_rows, const float* shard_scales, int num_shards,
                            float* s_w, hipStream_t stream);

/* Lossy merge: requantize every shard to the largest shard scale so that one
 * per-tensor scale serves the whole merged weight:
 *     s_max      = max_i shard_scales[i]
 *     w_out[r,k] = satRNE_E4M3( fl32( fl32( dec(w_q[r,k]) * shard_scales[i] ) / s_max ) )
 * for row r of shard i (NaN codes are copied).  Shards whose scale equals s_max
 * come out unchanged; the others lose the low bits their smaller scale held.
 * w_q, w_out: E4M3 [sum shard_rows, K] (w_out == w_q requantizes in place; any
 * other overlap is FP8MM_EINVAL).  s_w: DEVICE f32 [sum shard_rows], filled with
 * s_max (the per-channel form of the one scale).  *s_max_out (HOST, may be
 * NULL) receives s_max.  K % 16 == 0, 16-byte aligned w_q / w_out. */
int fp8_requant_max_scale(const uint8_t* w_q, uint8_t* w_out, int64_t K,
                          const int64_t* shard_rows, const float* shard_scales, int num_shards,
                          float* s_w, float* s_max_out, hipStream_t stream);

/* Merge admission (host).  Projections that share one input each carry a
 * static input scale; a merged launch quantizes the input once, so it needs one.
 *   FP8MM_MERGE_EXACT: merge only when all input scales are bitwise equal
 *     (returns 1, *s_act_out = that scale); otherwise returns 0: run each shard
 *     as its own quant + GEMM at its own scale (exact).
 *   FP8MM_MERGE_MAX_SCALE: always merge (returns 1) with *s_act_out = the
 *     largest input scale (lossy for the shards with smaller scales: their
 *     inputs are quantized on a coarser grid; none saturates).
 * input_scales: HOST array of num_shards (1..8) finite scales > 0.
 * FP8MM_EINVAL for a null pointer, a bad count or scale, another policy. */
#define FP8MM_MERGE_EXACT 0
#define FP8MM_MERGE_MAX_SCALE 1
int fp8_merge_admit(const float* input_scales, int num_shards, int policy, float* s_act_out);

#ifdef __cplusplus
}
#endif

#endif /* FP8MM_H */
