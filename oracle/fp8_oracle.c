/*
 * fp8_oracle.c -- plain, slow, obviously-correct CPU oracle for the FP8 (E4M3)
 * W8A8 scaled-matmul linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no code,
 * header, table or constant generator with the HIP path under
 * fp8_w8a8_scaled_amd/ and it never reads anything that path produced.
 *
 * What it computes (the layer the pages describe):
 *   out[m,n] = bf16( (sum_k q(x)[m,k] * W_q[n,k]) * s_act * s_w[n] ),
 *   q(x)     = saturating round-to-nearest-even E4M3 of x / s_act.
 * Sources (web pages; "vllm.cpp #252" = the issue "FP8 tower's cuBLASLt default
 * rests on a false premise", "vllm.cpp #213" = "Qwen3.6 NVFP4 baselines must
 * reach vLLM speed parity", "vllm.cpp #417" = "We emit F32 where vLLM emits
 * bf16", "vLLM #53014" = the PR "[Kernel] add Flashinfer cutedsl w4a16 linear"):
 *   - FP8 = F8_E4M3 / float8_e4m3fn weights and activations: vllm.cpp #252,
 *     original post, kernel table and byte total; vllm.cpp #417, Finding 2.
 *   - bmm_fp8(a, b, scale_a, scale_b, out_dtype): vllm.cpp #252, "CORRECTION".
 *   - static per-tensor activation scale (QuantFp8Static, input_scale) and the
 *     fused RMSNorm->fp8 quant that is byte-exact against the unfused path:
 *     vllm.cpp #417, ranked follow-ons; vllm.cpp #213, "merge predicate FIRES".
 *   - bf16 (model dtype) GEMM output: vllm.cpp #417, Finding 1.
 *   - per-channel ("FP8 channelwise") weight scales: vLLM #53014, the Marlin
 *     large-M commit message, last paragraph.
 * The pages fix no intermediate precision; the readings taken here (division,
 * fp64 sum of squares, bf16 rounding of the normalised row before quant, fp64
 * epilogue with one final rounding) are listed with the rest of the design.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared
 * (no fast-math: every float operation below must be an IEEE-754 operation in
 * the precision its type says).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_E4M3_MAX 448.0

/* ---------------------------------------------------------------- E4M3 ---- */

/* Value of one OCP E4M3FN code from its bit fields: sign s, exponent e (4 bits,
 * bias 7), mantissa m (3 bits).  e == 0 -> subnormal m * 2^-9; e in 1..15 ->
 * (1 + m/8) * 2^(e-7); S.1111.111 is NaN; there is no infinity. */
static double e4m3_value(unsigned code)
{
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double mag;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0u) mag = ldexp((double)m, -9);
    else mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* Decode table: tab[c] = value of code c (NaN for 0x7F and 0xFF). */
void oracle_e4m3_table(double tab[256])
{
    for (unsigned c = 0; c < 256u; ++c) tab[c] = e4m3_value(c);
}

/* Saturating round-to-nearest-even encode of one fp32 value.
 * |t| >= 448 (inf included) -> +-448; NaN -> 0x7F with t's sign; otherwise the
 * nearest representable magnitude, ties to the even code (mantissa LSB 0), and
 * the sign bit copied from t, so a negative value that rounds to zero gives 0x80.
 * Method: binary search over the 127 non-negative finite magnitudes, which the
 * codes 0x00..0x7E list in increasing order. */
unsigned char oracle_e4m3_encode(float t)
{
    unsigned sign = signbit(t) ? 0x80u : 0u;
    double a, lo_v, hi_v, dlo, dhi;
    int lo, hi;
    if (isnan(t)) return (unsigned char)(sign | 0x7Fu);
    a = fabs((double)t);
    if (a >= ORACLE_E4M3_MAX) return (unsigned char)(sign | 0x7Eu);
    /* find lo = largest code in [0, 0x7E] with value <= a */
    lo = 0; hi = 0x7E;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (e4m3_value((unsigned)mid) <= a) lo = mid; else hi = mid - 1;
    }
    if (lo == 0x7E) return (unsigned char)(sign | 0x7Eu);
    lo_v = e4m3_value((unsigned)lo);
    hi_v = e4m3_value((unsigned)lo + 1u);
    dlo = a - lo_v;            /* exact: both are short binary fractions */
    dhi = hi_v - a;
    if (dlo < dhi) return (unsigned char)(sign | (unsigned)lo);
    if (dhi < dlo) return (unsigned char)(sign | (unsigned)(lo + 1));
    return (unsigned char)(sign | (unsigned)((lo & 1) ? lo + 1 : lo));
}

void oracle_e4m3_encode_array(const float* t, int64_t n, unsigned char* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(t[i]);
}

/* ---------------------------------------------------------------- BF16 ---- */

float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a double to bf16 (8 significant bits, exponent range of fp32) with one
 * round-to-nearest-even step.  Written with frexp/nearbyint so that it never
 * rounds through fp32. */
uint16_t oracle_f64_to_bf16(double d)
{
    double a, q, r, res;
    int ex;
    uint32_t sign = signbit(d) ? 0x8000u : 0u, u;
    float f;
    if (isnan(d)) return (uint16_t)(sign | 0x7FC0u);
    a = fabs(d);
    if (a == 0.0) return (uint16_t)sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    (void)frexp(a, &ex);               /* a = f * 2^ex, f in [0.5, 1) */
    if (ex - 1 < -126) {               /* below the smallest normal: quantum 2^-133 */
        q = ldexp(a, 133);
        r = nearbyint(q);              /* default rounding mode: to nearest, ties even */
        res = ldexp(r, -133);
    } else {                           /* 8 significant bits: quantum 2^(ex-8) */
        q = ldexp(a, 8 - ex);          /* in [128, 256) exactly */
        r = nearbyint(q);
        res = ldexp(r, ex - 8);
    }
    if (res >= 0x1p128) return (uint16_t)(sign | 0x7F80u);      /* overflow -> inf */
    f = (float)res;                                              /* exact */
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

uint16_t oracle_f32_to_bf16(float f) { return oracle_f64_to_bf16((double)f); }

/* oracle_f64_to_bf16 applied to each of n doubles. */
void oracle_f64_to_bf16_array(const double* d, int64_t n, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(d[i]);
}

/* ------------------------------------------------------ activation quant --- */

/* Plain static per-tensor quant: x_q = satRNE_E4M3( fl32(f32(x) / s_act) ).
 * One IEEE fp32 division, then the E4M3 rounding (QuantFp8Static).  A NaN input
 * skips the division so that its own sign bit is the one encoded (IEEE leaves
 * the sign of a NaN result unspecified). */
void oracle_quant_act(const uint16_t* x, int64_t ldx, int64_t M, int64_t K,
                      float s_act, unsigned char* xq)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            float v = oracle_bf16_to_f32(x[m * ldx + k]);
            float t = isnan(v) ? v : v / s_act;
            xq[m * K + k] = oracle_e4m3_encode(t);
        }
}

/* RMSNorm to the model dtype (bf16), the unfused producer:
 *   ss = sum_k x_k^2 (fp64, k ascending)
 *   r  = fl32( 1 / sqrt(ss / K + eps) )   (fp64 inside, one rounding to fp32)
 *   y  = bf16_RNE( fl32( fl32(x_k * r) * gamma_k ) ) */
static float rms_inv(const uint16_t* row, int64_t K, float eps)
{
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double v = (double)oracle_bf16_to_f32(row[k]);
        ss += v * v;
    }
    return (float)(1.0 / sqrt(ss / (double)K + (double)eps));
}

void oracle_rmsnorm(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps,
                    int64_t M, int64_t K, uint16_t* y)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = x + m * ldx;
        float r = rms_inv(row, K, eps);
        for (int64_t k = 0; k < K; ++k) {
            float xn = oracle_bf16_to_f32(row[k]) * r;
            float yk = xn * oracle_bf16_to_f32(gamma[k]);
            y[m * K + k] = oracle_f32_to_bf16(yk);
        }
    }
}

/* Fused RMSNorm -> static FP8 quant, written as one pass over each row (the
 * quantize-once input-layernorm).  Its bytes must equal quant(rmsnorm(x)). */
void oracle_quant_rmsnorm(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps,
                          float s_act, int64_t M, int64_t K, unsigned char* xq)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = x + m * ldx;
        double ss = 0.0;
        float r;
        for (int64_t k = 0; k < K; ++k) {
            double v = (double)oracle_bf16_to_f32(row[k]);
            ss += v * v;
        }
        r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
        for (int64_t k = 0; k < K; ++k) {
            float g = oracle_bf16_to_f32(gamma[k]);
            float xn = oracle_bf16_to_f32(row[k]) * r;
            float yf = xn * g;
            float yb = oracle_bf16_to_f32(oracle_f32_to_bf16(yf));
            xq[m * K + k] = oracle_e4m3_encode(yb / s_act);
        }
    }
}

/* Static activation scale calibration: s_act = fl32(amax / 448), amax = max |.|
 * over the whole tensor that is quantized (x itself, or the bf16 RMSNorm output
 * when gamma != NULL).  amax == 0 gives 1.  Non-finite entries are ignored. */
float oracle_act_scale(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps,
                       int64_t M, int64_t K)
{
    float amax = 0.0f;
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = x + m * ldx;
        float r = gamma ? rms_inv(row, K, eps) : 1.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = oracle_bf16_to_f32(row[k]);
            if (gamma) v = oracle_bf16_to_f32(oracle_f32_to_bf16((v * r) * oracle_bf16_to_f32(gamma[k])));
            v = fabsf(v);
            if (isfinite(v) && v > amax) amax = v;
        }
    }
    if (amax == 0.0f) return 1.0f;
    return amax / 448.0f;                 /* one IEEE fp32 division */
}

/* ------------------------------------------------ SiLU*mul -> FP8 ------- */

/* The MLP activation between the merged gate_up projection and the down
 * projection, quantized once for the down GEMM: h = silu(gate) * up with
 * silu(g) = g * sigmoid(g) = g / (1 + exp(-g)).  The merged gate_up launch and
 * its two shards: vllm.cpp #252 "SETTLED BY PAIRED TRACE" (the MLP pair), the
 * quantize-once input of the next GEMM: vllm.cpp #417, ranked follow-ons.
 * The pages fix no precision; the reading taken (like the RMSNorm one): silu
 * evaluated in fp64 and rounded once to fp32, the product in fp32, the
 * unfused activation emitting the model dtype, h_b = bf16_RNE(h), and then the
 * static quant x_q = satRNE_E4M3(fl32(h_b / s_act)). */
static float silu_f32(float g)
{
    double d = (double)g;
    return (float)(d / (1.0 + exp(-d)));
}

/* Unfused: h_b[m,i] = bf16_RNE( fl32( silu(gate[m,i]) * up[m,i] ) ). */
void oracle_silu_mul(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu,
                     int64_t M, int64_t I, uint16_t* h)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t i = 0; i < I; ++i) {
            float s = silu_f32(oracle_bf16_to_f32(gate[m * ldg + i]));
            float hf = s * oracle_bf16_to_f32(up[m * ldu + i]);
            h[m * I + i] = oracle_f32_to_bf16(hf);
        }
}

/* Fused SiLU*mul -> static FP8 quant, written as one pass; its bytes must equal
 * quant(silu_mul(gate, up)). */
void oracle_silu_mul_quant(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu,
                           float s_act, int64_t M, int64_t I, unsigned char* xq)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t i = 0; i < I; ++i) {
            double g = (double)oracle_bf16_to_f32(gate[m * ldg + i]);
            float sig_g = (float)(g / (1.0 + exp(-g)));
            float u = oracle_bf16_to_f32(up[m * ldu + i]);
            float hb = oracle_bf16_to_f32(oracle_f32_to_bf16(sig_g * u));
            xq[m * I + i] = oracle_e4m3_encode(isnan(hb) ? hb : hb / s_act);
        }
}

/* ------------------------------------------------------- weight prep ------ */

/* Per-output-channel weight quant (load time): s_w[n] = fl32(amax_k |W[n,k]| / 448)
 * (1 for an all-zero row), W_q[n,k] = satRNE_E4M3( fl32(W[n,k] / s_w[n]) ). */
void oracle_quant_weight(const float* W, int64_t N, int64_t K, unsigned char* wq, float* s_w)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const float* row = W + n * K;
        float amax = 0.0f, s;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(row[k]);
            if (a > amax) amax = a;
        }
        s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
        s_w[n] = s;
        for (int64_t k = 0; k < K; ++k) wq[n * K + k] = oracle_e4m3_encode(row[k] / s);
    }
}

/* Per-tensor weight quant (one scale for the whole [N,K] weight, the scale
 * form a checkpoint's q/k/v shards carry one each): s = fl32(amax |W| / 448)
 * over every element (1 for an all-zero weight), W_q = satRNE_E4M3(fl32(W / s)).
 * The same rule as the per-channel quant above, applied to the whole tensor. */
void oracle_quant_weight_per_tensor(const float* W, int64_t N, int64_t K, unsigned char* wq, float* s_out)
{
    float amax = 0.0f, s;
    for (int64_t i = 0; i < N * K; ++i) {
        float a = fabsf(W[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) s = 1.0f; else s = amax / 448.0f;
    *s_out = s;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N * K; ++i) wq[i] = oracle_e4m3_encode(W[i] / s);
}

/* Requantize a merged weight whose shards carry different per-tensor scales to
 * the largest of them, so that one per-tensor scale serves the whole merged
 * projection (the lossy alternative to declining the merge that vllm.cpp #417,
 * ranked follow-ons, contrasts with the exact split path).  Shard i holds rows
 * [r_i, r_i + rows[i]) of the [sum rows, K] weight and has scale scales[i]:
 *     s_max = max_i scales[i]
 *     w     = fl32( dec(c) * scales[i] )          (the shard's f32 weight value)
 *     c'    = satRNE_E4M3( fl32( w / s_max ) )    (the per-tensor quant of w at s_max)
 * A NaN code is kept as it is.  Scales are finite and > 0. */
void oracle_requant_max_scale(const unsigned char* wq, const int64_t* rows, const float* scales,
                              int num_shards, int64_t K, unsigned char* out, float* s_max_out)
{
    float s_max = scales[0];
    int64_t r0 = 0;
    for (int i = 1; i < num_shards; ++i)
        if (scales[i] > s_max) s_max = scales[i];
    *s_max_out = s_max;
    for (int i = 0; i < num_shards; ++i) {
#pragma omp parallel for schedule(static)
        for (int64_t e = r0 * K; e < (r0 + rows[i]) * K; ++e) {
            double d = e4m3_value(wq[e]);
            float w;
            if (isnan(d)) { out[e] = wq[e]; continue; }
            w = (float)d * scales[i];
            out[e] = oracle_e4m3_encode(w / s_max);
        }
        r0 += rows[i];
    }
}

/* ------------------------------------------------------------- GEMM ------- */

/* out[m,n] = bf16_RNE( (acc * s_act) * s_w[n] ) with
 * acc = sum_k dec(x_q[m,k]) * dec(W_q[n,k]) accumulated in fp64 (exact for these
 * operand sizes), the two scale multiplies in fp64 and one rounding to bf16.
 * If v != NULL the unrounded fp64 v[m,n] is stored too (the tolerance uses the
 * row norm of v).  out has row stride ldo. */
void oracle_scaled_mm(const unsigned char* xq, const unsigned char* wq, float s_act,
                      const float* s_w, int64_t M, int64_t N, int64_t K,
                      uint16_t* out, int64_t ldo, double* v)
{
    double tab[256];
    oracle_e4m3_table(tab);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            const unsigned char* a = xq + m * K;
            const unsigned char* b = wq + n * K;
            double acc = 0.0, val;
            for (int64_t k = 0; k < K; ++k) acc += tab[a[k]] * tab[b[k]];
            val = (acc * (double)s_act) * (double)s_w[n];
            out[m * ldo + n] = oracle_f64_to_bf16(val);
            if (v) v[m * N + n] = val;
        }
}

/* ------------------------------------------ per-token dynamic scales --- */

/* Per-token dynamic activation scales: the scale granularity vllm.cpp #252
 * leaves open ("What is owed", item 2: per-tensor vs per-channel vs per-token
 * scaling).  Reading taken: every row is quantized as a tensor of its own, with
 * the static quant's calibration rule applied to that row alone:
 *     s[m]     = fl32( amax_k |y[m,k]| / 448 )    (finite values; 1 when 0)
 *     x_q[m,k] = satRNE_E4M3( fl32( y[m,k] / s[m] ) )
 * y is x (gamma == NULL) or the bf16 RMSNorm output of the row. */
void oracle_quant_per_token(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps,
                            int64_t M, int64_t K, unsigned char* xq, float* s_rows)
{
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = x + m * ldx;
        const float s = oracle_act_scale(row, ldx, gamma, eps, 1, K);
        s_rows[m] = s;
        if (gamma)
            oracle_quant_rmsnorm(row, ldx, gamma, eps, s, 1, K, xq + m * K);
        else
            oracle_quant_act(row, ldx, 1, K, s, xq + m * K);
    }
}

/* The GEMM with a per-row activation scale: v[m,n] = (acc[m,n] * s[m]) * s_w[n]
 * in fp64, out = bf16_RNE(v) (the per-tensor epilogue with s_act -> s[m]). */
void oracle_scaled_mm_rows(const unsigned char* xq, const unsigned char* wq, const float* s_rows,
                           const float* s_w, int64_t M, int64_t N, int64_t K,
                           uint16_t* out, int64_t ldo, double* v)
{
    for (int64_t m = 0; m < M; ++m)
        oracle_scaled_mm(xq + m * K, wq, s_rows[m], s_w, 1, N, K, out + m * ldo, ldo, v ? v + m * N : NULL);
}

/* Only the exact accumulator (fp64), for the closed-form pins. */
void oracle_exact_acc(const unsigned char* xq, const unsigned char* wq,
                      int64_t M, int64_t N, int64_t K, double* acc)
{
    double tab[256];
    oracle_e4m3_table(tab);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += tab[xq[m * K + k]] * tab[wq[n * K + k]];
            acc[m * N + n] = s;
        }
}

/* Threads of the OpenMP loops above (the CPU baseline times 1 and all). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
