// internal.h -- launcher interface between the C ABI (api.hip) and the kernels.
// Callers have already validated shapes, strides and alignment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8mm.h"

namespace fp8mm {

// Output placement of a (possibly merged) projection, passed by value in the
// kernel arguments: weight rows [start[i], start[i+1]) go to out[i] with row
// stride ldo[i] (elements).  Every start[i] is a multiple of 16.  f32 selects
// the output type for every shard: 0 bf16 (RNE), 1 f32 (the scaled fp32 value
// itself).  s_rows, when not null, holds per-row activation scales (device f32
// [M]) that replace the per-tensor s_act in the epilogue.
struct ShardTable {
    int num;
    int f32;
    const float* s_rows;
    int64_t start[FP8MM_MAX_SHARDS + 1];
    void* out[FP8MM_MAX_SHARDS];
    int64_t ldo[FP8MM_MAX_SHARDS];
};

// quant.hip
void launch_quant(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, float s_act,
                  uint8_t* xq, int64_t M, int64_t K, hipStream_t stream);
size_t act_scale_partials(int64_t M, int64_t K, bool rms);
void launch_act_scale(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps,
                      int64_t M, int64_t K, float* s_act, float* partial, hipStream_t stream);
void launch_quant_weight(const float* w, int64_t N, int64_t K, uint8_t* wq, float* s_w,
                         hipStream_t stream);
// The current device's copy of the static scratch array of the allocation-free
// calibration (FP8MM_NOALLOC_SCRATCH_FLOATS floats), looked up once per device.
hipError_t noalloc_scratch(float** ptr);
void launch_quant_per_token(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, uint8_t* xq,
                            float* s_rows, int64_t M, int64_t K, hipStream_t stream);
void launch_silu_mul_quant(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu, float s_act,
                           uint8_t* xq, int64_t M, int64_t I, hipStream_t stream);
void launch_act_scale_silu_mul(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu, int64_t M,
                               int64_t I, float* s_act, float* partial, hipStream_t stream);

// merge.hip: load-time weight preparation for merged shards with per-tensor
// scales.  Shard i holds weight rows [start[i], start[i+1]) and has the
// per-tensor scale scale[i].
struct ShardScales {
    int num;
    float scale[FP8MM_MAX_SHARDS];
    int64_t start[FP8MM_MAX_SHARDS + 1];
};
size_t weight_absmax_partials(int64_t N, int64_t K);
void launch_quant_weight_per_tensor(const float* w, int64_t N, int64_t K, uint8_t* wq, float* s,
                                    float* partial, hipStream_t stream);
void launch_expand_shard_scales(const ShardScales& tab, float* s_w, hipStream_t stream);
void launch_requant_max_scale(const uint8_t* in, uint8_t* out, const ShardScales& tab, float s_max, int64_t K,
                              float* s_w, hipStream_t stream);

// gemm_small_m.hip: memory-bound arm, M <= FP8MM_SMALL_M_MAX.
void launch_gemm_small_m(const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w,
                         const ShardTable& shards, int64_t M, int64_t N, int64_t K,
                         hipStream_t stream);
// The static quant of bf16 x (with gamma: the fused RMSNorm quant) inside
// the small-M GEMM (one launch; x_q also written).  Returns false, launching
// nothing, where the fused kernel does not take the shape (M > 8, a scale
// outside 2^-100..2^100, no LDS plan; with gamma also W != 8): the caller then
// quantizes and multiplies separately.  quant_gemm_small_m_fits: whether it
// takes the shape (the host-side plan only).
bool quant_gemm_small_m_fits(int64_t M, int64_t N, int64_t K, int64_t ldx, float s_act, bool rmsnorm);
// The gate_up launch with the SiLU*mul -> E4M3 quant as its epilogue (weight
// rows interleaved 8 gate / 8 up per 16-row tile, N = 2I; h_q E4M3 [M, I]).
// quant: 0 = x_q given (x NULL), 1 = plain static quant of x in the launch,
// 2 = fused RMSNorm quant (gamma); x_q is then written when not NULL.
// gate_up_silu_fits: whether the launch takes the shape (else
// launch_gate_up_silu returns false and launches nothing).
bool gate_up_silu_fits(int64_t M, int64_t I, int64_t K, int64_t ldx, float s_act, float s_down, int quant);
bool launch_gate_up_silu(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, uint8_t* xq,
                         const uint8_t* wq, float s_act, const float* s_w, int64_t M, int64_t I, int64_t K,
                         float s_down, uint8_t* hq, hipStream_t stream);
void launch_interleave_gate_up(const uint8_t* wq, const float* s_w, uint8_t* w_il, float* s_il, int64_t I,
                               int64_t K, hipStream_t stream);
bool launch_quant_gemm_small_m(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, uint8_t* xq_out,
                               const uint8_t* wq, float s_act, const float* s_w, const ShardTable& shards, int64_t M,
                               int64_t N, int64_t K, hipStream_t stream);

// gemm_large_m.hip: compute units of the current device (cached).
int num_cus();

// gemm_large_m.hip: compute-bound MFMA-tiled arm, any M.
void launch_gemm_large_m(const uint8_t* xq, const uint8_t* wq, float s_act, const float* s_w,
                         const ShardTable& shards, int64_t M, int64_t N, int64_t K,
                         hipStream_t stream);

}  // namespace fp8mm
