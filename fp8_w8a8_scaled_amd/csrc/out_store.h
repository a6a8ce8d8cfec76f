// out_store.h -- the GEMM output stores: scaled fp32 values to bf16 (RNE) or
// to f32, for the output type a ShardTable selects.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace fp8mm {

// Shard of output column n (n0 of a 16-column tile works for the whole tile:
// shard boundaries are multiples of 16).
__device__ __forceinline__ int shard_of(const ShardTable& sh, int64_t n)
{
    int i = 0;
    while (i + 1 < sh.num && n >= sh.start[i + 1]) ++i;
    return i;
}

// Activation scale of output row m (m < M): per-row when the table has them.
__device__ __forceinline__ float row_scale(const ShardTable& sh, int64_t m, float s_act)
{
    return sh.s_rows ? sh.s_rows[m] : s_act;
}

// Four consecutive columns n..n+3 (n % 4 == 0) of row m in shard i: 8 bytes of
// bf16 or 16 bytes of f32.
__device__ __forceinline__ void store_out4(const ShardTable& sh, int i, int64_t m, int64_t n, float a, float b,
                                           float c, float d)
{
    const int64_t off = m * sh.ldo[i] + (n - sh.start[i]);
    if (sh.f32) {
        *reinterpret_cast<float4*>(static_cast<float*>(sh.out[i]) + off) = make_float4(a, b, c, d);
    } else {
        const uint32_t lo = f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
        const uint32_t hi = f32_to_bf16_rne(c) | (f32_to_bf16_rne(d) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(sh.out[i]) + off) = make_uint2(lo, hi);
    }
}

// The fields of the shard that holds column n (n may differ from lane to
// lane): picked with constant indices only, so they stay scalar kernel
// arguments.  A lane-dependent index into the table would read them from the
// argument buffer with vector loads, one memory round trip before the stores
// that need them.
__device__ __forceinline__ void shard_fields(const ShardTable& sh, int64_t n, void*& out, int64_t& ldo,
                                             int64_t& start)
{
    out = sh.out[0];
    ldo = sh.ldo[0];
    start = sh.start[0];
#pragma unroll
    for (int j = 1; j < FP8MM_MAX_SHARDS; ++j) {
        if (j >= sh.num) break;                          // uniform: only the table's shards are visited
        const bool in = n >= sh.start[j];
        out = in ? sh.out[j] : out;
        ldo = in ? sh.ldo[j] : ldo;
        start = in ? sh.start[j] : start;
    }
}

// Four consecutive columns n..n+3 of row m, in the shard that holds column ns
// (the same shard as n's; ns may differ from lane to lane).
__device__ __forceinline__ void store_out4_any(const ShardTable& sh, int64_t ns, int64_t m, int64_t n, float a,
                                               float b, float c, float d)
{
    void* o;
    int64_t ld, st;
    shard_fields(sh, ns, o, ld, st);
    const int64_t off = m * ld + (n - st);
    if (sh.f32) {
        *reinterpret_cast<float4*>(static_cast<float*>(o) + off) = make_float4(a, b, c, d);
    } else {
        const uint32_t lo = f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
        const uint32_t hi = f32_to_bf16_rne(c) | (f32_to_bf16_rne(d) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(o) + off) = make_uint2(lo, hi);
    }
}

// One element.
__device__ __forceinline__ void store_out1(const ShardTable& sh, int i, int64_t m, int64_t n, float v)
{
    const int64_t off = m * sh.ldo[i] + (n - sh.start[i]);
    if (sh.f32)
        static_cast<float*>(sh.out[i])[off] = v;
    else
        static_cast<uint16_t*>(sh.out[i])[off] = (uint16_t)f32_to_bf16_rne(v);
}

}  // namespace fp8mm
