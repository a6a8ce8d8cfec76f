"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds NO arithmetic of the method (no quantization, no scaling, no
norm, no GEMM): it only draws random numbers and converts them to the storage
dtypes the layer consumes (fp32 weights, bf16 activations and gamma, raw E4M3
codes for GEMM-only cases).  Both the oracle and the GPU path start from these
exact bytes.

Shapes follow the five workloads of the FP8 W8A8 scaled-MM layer (tiny check,
decode projection, decode MLP, full decode-step weight sweep, prefill chunk);
the per-layer shapes come from the layer projections the pages trace
(vllm.cpp #252 "SETTLED BY PAIRED TRACE": GDN in_proj_qkv 10240x5120 and the
merged qkvz, out_proj / o_proj 5120x6144; the MLP pair) and the prefill chunk
of 6576 tokens (vLLM #53014, the Marlin large-M commit message).

Generator: numpy PCG64 seeded with the entropy list
``[0x5EED0000, workload_id, tensor_id, M]`` so every tensor is reproducible on
its own.  Tensor ids: 0 weight, 1 activation, 2 gamma, 3 outlier positions,
4 down-projection weight, 5 down-projection activation, 6 random codes,
7 gate_up output (the SiLU*mul input), 32 + i for shard i of a merged weight
whose shards are quantized per tensor, 64 + layer for the decode-step sweep.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

SEED_BASE = 0x5EED0000
T_W, T_X, T_GAMMA, T_OUTLIER, T_DOWN_W, T_DOWN_X, T_CODES, T_GATE_UP = 0, 1, 2, 3, 4, 5, 6, 7
T_SHARD0 = 32
T_LAYER0 = 64

EPS = 1e-6
W_STD = 0.02
GAMMA_MEAN, GAMMA_STD = 1.0, 0.1
OUTLIER_FRAC, OUTLIER_MUL = 0.01, 20.0


def rng(workload: int, tensor: int, m: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([SEED_BASE, int(workload), int(tensor), int(m)]))


def to_bf16_bits(a_f32: np.ndarray) -> np.ndarray:
    """Storage conversion fp32 -> bf16 bit patterns (round to nearest even),
    done by torch's dtype cast so this module carries no rounding code."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def weight_f32(workload: int, N: int, K: int, tensor: int = T_W) -> np.ndarray:
    """W ~ N(0, 0.02) in fp32, [N, K] row-major (K contiguous)."""
    g = rng(workload, tensor)
    w = g.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(W_STD)
    return w


def activation_bf16(workload: int, M: int, K: int, outliers: bool, tensor: int = T_X) -> np.ndarray:
    """x ~ N(0, 1) drawn in fp32; if ``outliers``, exactly round(0.01*M*K)
    distinct positions (a seeded permutation) are multiplied by 20 in fp32;
    then stored as bf16 bits [M, K]."""
    g = rng(workload, tensor, M)
    x = g.standard_normal((M, K), dtype=np.float32)
    if outliers and M * K > 0:
        n_out = int(round(OUTLIER_FRAC * M * K))
        pos = rng(workload, T_OUTLIER if tensor == T_X else tensor + 100, M).permutation(M * K)[:n_out]
        flat = x.reshape(-1)
        flat[pos] *= np.float32(OUTLIER_MUL)
    return to_bf16_bits(x)


def gamma_bf16(workload: int, K: int) -> np.ndarray:
    """gamma ~ N(1, 0.1) stored as bf16 bits [K]."""
    g = rng(workload, T_GAMMA)
    v = g.standard_normal(K, dtype=np.float32) * np.float32(GAMMA_STD) + np.float32(GAMMA_MEAN)
    return to_bf16_bits(v)


# The 254 finite E4M3FN code values: every byte except S.1111.111 (NaN).
FINITE_CODE_VALUES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def random_codes(workload: int, rows: int, cols: int, tensor: int = T_CODES, m: int = 0) -> np.ndarray:
    """Uniformly random finite E4M3 codes [rows, cols] (for GEMM-only cases)."""
    g = rng(workload, tensor, m)
    return FINITE_CODE_VALUES[g.integers(0, FINITE_CODE_VALUES.size, size=(rows, cols))]


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# ---------------------------------------------------------------- workloads --

@dataclasses.dataclass(frozen=True)
class Projection:
    name: str
    N: int
    K: int
    shards: tuple = ()          # output split of a merged projection, sums to N


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    Ms: tuple
    projections: tuple
    rmsnorm_input: bool         # fused RMSNorm->quant feeds the first projection
    outliers: bool


TINY = Workload(1, "tiny_w8a8_M4_K256_N384", (4,),
                (Projection("proj", 384, 256),), False, False)
DECODE_PROJ = Workload(2, "decode_proj_K5120_N10240", (1, 2, 4, 8),
                       (Projection("qkv", 10240, 5120),), False, True)
DECODE_MLP = Workload(3, "decode_mlp_gateup_K5120_N34816_down_K17408_N5120", (1, 4, 8, 16, 32),
                      (Projection("gate_up", 34816, 5120, (17408, 17408)),
                       Projection("down", 5120, 17408)), True, True)
# Per layer of the decode-step sweep: merged qkvz, out-proj, and the MLP pair.
DECODE_STEP_LAYER = (Projection("qkvz", 12288, 5120),
                     Projection("out_proj", 5120, 6144),
                     Projection("gate_up", 34816, 5120, (17408, 17408)),
                     Projection("down", 5120, 17408))
DECODE_STEP = Workload(4, "decode_step_64_layers_M8", (8,), DECODE_STEP_LAYER, False, True)
DECODE_STEP_LAYERS = 64
# The pages' own tower (the 7.7 GiB of E4M3 a decode step reads), as (layers,
# projections): 48 GDN layers with a merged qkvz and out_proj, 16 attention
# layers with a merged qkv and o_proj, and the MLP pair; 136 launches.
DECODE_STEP_4B = ((48, (Projection("in_proj_qkvz", 16384, 5120), Projection("out_proj", 5120, 6144))),
                  (16, (Projection("qkv", 14336, 5120), Projection("o_proj", 5120, 6144))),
                  (4, (Projection("gate_up", 34816, 5120, (17408, 17408)), Projection("down", 5120, 17408))))
PREFILL = Workload(5, "prefill_M6576_gateup_K5120_N34816_down_K17408_N5120", (6576,),
                   (Projection("gate_up", 34816, 5120, (17408, 17408)),
                    Projection("down", 5120, 17408)), True, False)

WORKLOADS = {w.wid: w for w in (TINY, DECODE_PROJ, DECODE_MLP, DECODE_STEP, PREFILL)}
