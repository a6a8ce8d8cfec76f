"""CPU oracle for the FP8 (E4M3) W8A8 scaled-matmul linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP path in ``fp8_w8a8_scaled_amd/`` and never imports it.

The arithmetic lives in ``fp8_oracle.c`` (plain C, fp64 where the definition
allows, OpenMP over independent rows); this module only builds that file with
gcc and marshals numpy arrays into it.  ``exact.py`` is a second, independent
checker written with ``fractions.Fraction`` for tiny cases.

Every function here follows the definitions stated in ``fp8_oracle.c``'s
header, which cites the pages each step comes from.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = load(_LIB)
    return _lib


def load(path: str) -> ctypes.CDLL:
    """Load a compiled oracle library and declare its C signatures."""
    L = ctypes.CDLL(path)
    P, I64, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    L.oracle_e4m3_table.argtypes = [P]
    L.oracle_e4m3_encode.argtypes = [F32]
    L.oracle_e4m3_encode.restype = ctypes.c_ubyte
    L.oracle_e4m3_encode_array.argtypes = [P, I64, P]
    L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_bf16_to_f32.restype = F32
    L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
    L.oracle_f64_to_bf16.restype = ctypes.c_uint16
    L.oracle_f32_to_bf16.argtypes = [F32]
    L.oracle_f64_to_bf16_array.argtypes = [P, I64, P]
    L.oracle_f32_to_bf16.restype = ctypes.c_uint16
    L.oracle_quant_act.argtypes = [P, I64, I64, I64, F32, P]
    L.oracle_rmsnorm.argtypes = [P, I64, P, F32, I64, I64, P]
    L.oracle_quant_rmsnorm.argtypes = [P, I64, P, F32, F32, I64, I64, P]
    L.oracle_act_scale.argtypes = [P, I64, P, F32, I64, I64]
    L.oracle_act_scale.restype = F32
    L.oracle_quant_weight.argtypes = [P, I64, I64, P, P]
    L.oracle_scaled_mm.argtypes = [P, P, F32, P, I64, I64, I64, P, I64, P]
    L.oracle_exact_acc.argtypes = [P, P, I64, I64, I64, P]
    L.oracle_silu_mul.argtypes = [P, I64, P, I64, I64, I64, P]
    L.oracle_silu_mul_quant.argtypes = [P, I64, P, I64, F32, I64, I64, P]
    L.oracle_quant_per_token.argtypes = [P, I64, P, F32, I64, I64, P, P]
    L.oracle_scaled_mm_rows.argtypes = [P, P, P, P, I64, I64, I64, P, I64, P]
    L.oracle_quant_weight_per_tensor.argtypes = [P, I64, I64, P, P]
    L.oracle_requant_max_scale.argtypes = [P, P, P, ctypes.c_int, I64, P, P]
    L.oracle_num_threads.restype = ctypes.c_int
    L.oracle_set_num_threads.argtypes = [ctypes.c_int]
    return L


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# ---------------------------------------------------------------- scalars ---

def e4m3_table() -> np.ndarray:
    """float64[256]: value of every E4M3FN code (NaN for 0x7F, 0xFF)."""
    t = np.empty(256, np.float64)
    lib().oracle_e4m3_table(_ptr(t))
    return t


def e4m3_encode(t) -> np.ndarray:
    """Saturating RNE encode of fp32 values -> uint8 codes."""
    a = _c(np.asarray(t, np.float32).reshape(-1), np.float32)
    out = np.empty(a.size, np.uint8)
    lib().oracle_e4m3_encode_array(_ptr(a), a.size, _ptr(out))
    return out.reshape(np.shape(t))


def f64_to_bf16(d: float) -> int:
    return int(lib().oracle_f64_to_bf16(float(d)))


def f64_to_bf16_array(d: np.ndarray) -> np.ndarray:
    """bf16 bits (RNE, one rounding) of every double of d."""
    a = _c(d, np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_f64_to_bf16_array(_ptr(a), a.size, _ptr(out))
    return out


def f32_to_bf16(f: float) -> int:
    return int(lib().oracle_f32_to_bf16(float(np.float32(f))))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------ activations ---

def quant_act(x_bf16: np.ndarray, s_act: float) -> np.ndarray:
    """x_q = satRNE_E4M3(fl32(x / s_act)) for bf16 bits x[M, K] (row stride = K)."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    out = np.empty((M, K), np.uint8)
    lib().oracle_quant_act(_ptr(x), K, M, K, float(s_act), _ptr(out))
    return out


def rmsnorm(x_bf16: np.ndarray, gamma_bf16: np.ndarray, eps: float) -> np.ndarray:
    """Unfused RMSNorm to bf16 bits."""
    x = _c(x_bf16, np.uint16)
    g = _c(gamma_bf16, np.uint16)
    M, K = x.shape
    y = np.empty((M, K), np.uint16)
    lib().oracle_rmsnorm(_ptr(x), K, _ptr(g), float(eps), M, K, _ptr(y))
    return y


def quant_rmsnorm(x_bf16: np.ndarray, gamma_bf16: np.ndarray, eps: float, s_act: float) -> np.ndarray:
    """Fused RMSNorm -> static E4M3 quant (one pass per row)."""
    x = _c(x_bf16, np.uint16)
    g = _c(gamma_bf16, np.uint16)
    M, K = x.shape
    out = np.empty((M, K), np.uint8)
    lib().oracle_quant_rmsnorm(_ptr(x), K, _ptr(g), float(eps), float(s_act), M, K, _ptr(out))
    return out


def act_scale(x_bf16: np.ndarray, gamma_bf16: np.ndarray | None = None, eps: float = 1e-6) -> float:
    """Static per-tensor scale fl32(amax / 448) of the tensor that gets quantized."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    g = None if gamma_bf16 is None else _c(gamma_bf16, np.uint16)
    return float(np.float32(lib().oracle_act_scale(_ptr(x), K, _ptr(g), float(eps), M, K)))


def silu_mul(gate_bf16: np.ndarray, up_bf16: np.ndarray) -> np.ndarray:
    """Unfused MLP activation: bf16 bits of fl32(silu(gate) * up), [M, I]."""
    g = _c(gate_bf16, np.uint16)
    u = _c(up_bf16, np.uint16)
    M, I = g.shape
    assert u.shape == (M, I)
    h = np.empty((M, I), np.uint16)
    lib().oracle_silu_mul(_ptr(g), I, _ptr(u), I, M, I, _ptr(h))
    return h


def silu_mul_quant(gate_bf16: np.ndarray, up_bf16: np.ndarray, s_act: float) -> np.ndarray:
    """Fused SiLU*mul -> static E4M3 quant (one pass), uint8 codes [M, I]."""
    g = _c(gate_bf16, np.uint16)
    u = _c(up_bf16, np.uint16)
    M, I = g.shape
    assert u.shape == (M, I)
    out = np.empty((M, I), np.uint8)
    lib().oracle_silu_mul_quant(_ptr(g), I, _ptr(u), I, float(s_act), M, I, _ptr(out))
    return out


# ---------------------------------------------------------------- weights ---

def quant_weight(w_f32: np.ndarray):
    """Per-output-channel E4M3 quant: returns (W_q uint8 [N,K], s_w float32 [N])."""
    w = _c(w_f32, np.float32)
    N, K = w.shape
    wq = np.empty((N, K), np.uint8)
    sw = np.empty(N, np.float32)
    lib().oracle_quant_weight(_ptr(w), N, K, _ptr(wq), _ptr(sw))
    return wq, sw


def quant_weight_per_tensor(w_f32: np.ndarray):
    """Per-tensor E4M3 quant: returns (W_q uint8 [N,K], s float32 scalar)."""
    w = _c(w_f32, np.float32)
    N, K = w.shape
    wq = np.empty((N, K), np.uint8)
    s = np.empty(1, np.float32)
    lib().oracle_quant_weight_per_tensor(_ptr(w), N, K, _ptr(wq), _ptr(s))
    return wq, s[0]


def requant_max_scale(wq: np.ndarray, rows, scales):
    """Requantize the shards (``rows[i]`` weight rows with per-tensor scale
    ``scales[i]``) of a merged [sum rows, K] weight to the largest scale:
    returns (W_q' uint8 [sum rows, K], s_max float32)."""
    w = _c(wq, np.uint8)
    r = np.ascontiguousarray(rows, np.int64)
    sc = np.ascontiguousarray(scales, np.float32)
    assert r.shape == sc.shape and r.size >= 1 and int(r.sum()) == w.shape[0]
    out = np.empty_like(w)
    s = np.empty(1, np.float32)
    lib().oracle_requant_max_scale(_ptr(w), _ptr(r), _ptr(sc), int(r.size), w.shape[1], _ptr(out), _ptr(s))
    return out, s[0]


def merged_max_scale_layer(x_bf16: np.ndarray, wq_shards, w_scales, in_scales, want_v: bool = False):
    """One merged projection built the lossy way from shards that each carry a
    per-tensor weight scale and a static input scale: the input is quantized
    once at the largest input scale, the weight is requantized to the largest
    weight scale, and one GEMM with that scale on every column runs.  Returns
    (x_q, W_q', s_act, s_max, out[, v])."""
    s_act = np.float32(max(np.float32(s) for s in in_scales))
    xq = quant_act(x_bf16, float(s_act))
    wq_cat = np.concatenate([_c(w, np.uint8) for w in wq_shards], axis=0)
    wq2, s_max = requant_max_scale(wq_cat, [w.shape[0] for w in wq_shards], w_scales)
    sw = np.full(wq2.shape[0], s_max, np.float32)
    res = scaled_mm(xq, wq2, float(s_act), sw, want_v=want_v)
    return (xq, wq2, s_act, s_max) + (res if want_v else (res,))


# ------------------------------------------------------------------- GEMM ---

def scaled_mm(xq: np.ndarray, wq: np.ndarray, s_act: float, s_w: np.ndarray, want_v: bool = False):
    """out bf16 bits [M, N] (and the unrounded fp64 v if want_v)."""
    a = _c(xq, np.uint8)
    b = _c(wq, np.uint8)
    sw = _c(s_w, np.float32)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2 and sw.shape == (N,)
    out = np.empty((M, N), np.uint16)
    v = np.empty((M, N), np.float64) if want_v else None
    lib().oracle_scaled_mm(_ptr(a), _ptr(b), float(s_act), _ptr(sw), M, N, K, _ptr(out), N, _ptr(v))
    return (out, v) if want_v else out


# Largest K for which every partial sum of the accumulation is exact in fp64:
# each E4M3 value is a multiple of 2^-9 with magnitude <= 448, so a product is
# a multiple of 2^-18 of magnitude <= 448^2, and a sum of K of them needs fewer
# than 53 bits while K * 448^2 * 2^18 < 2^53.
EXACT_K_MAX = int(2 ** 35 // (448 * 448))


def scaled_mm_blas(xq: np.ndarray, wq: np.ndarray, s_act: float, s_w: np.ndarray, want_v: bool = False):
    """The GEMM of ``scaled_mm`` with its accumulation taken by a library fp64
    matmul (numpy / BLAS) on the decoded operands: the same definition,
    acc[m, n] = sum_k dec(x_q[m, k]) dec(w_q[n, k]), for large shapes.  The
    matmul may block, reorder and fuse as it likes: while K <= EXACT_K_MAX
    every product and every partial sum is exact in fp64, so any order gives
    the one exact sum.  The epilogue is scaled_mm's, (acc * s_act) * s_w[n] in
    fp64 with one rounding to bf16."""
    a = _c(xq, np.uint8)
    b = _c(wq, np.uint8)
    sw = _c(s_w, np.float32)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2 and sw.shape == (N,)
    assert K <= EXACT_K_MAX, "fp64 accumulation is exact only up to EXACT_K_MAX"
    tab = e4m3_table()
    v = np.matmul(tab[a], tab[b].T)              # exact sums, [M, N] fp64
    v *= np.float64(np.float32(s_act))
    v *= sw.astype(np.float64)[None, :]
    out = f64_to_bf16_array(v)
    return (out, v) if want_v else out


def quant_per_token(x_bf16: np.ndarray, gamma_bf16: np.ndarray | None = None, eps: float = 1e-6):
    """Per-token dynamic quant: (codes uint8 [M, K], scales float32 [M]); each
    row quantized with its own amax / 448 (RMSNorm first when gamma is given)."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    g = None if gamma_bf16 is None else _c(gamma_bf16, np.uint16)
    xq = np.empty((M, K), np.uint8)
    s = np.empty(M, np.float32)
    lib().oracle_quant_per_token(_ptr(x), K, _ptr(g), float(eps), M, K, _ptr(xq), _ptr(s))
    return xq, s


def scaled_mm_rows(xq: np.ndarray, wq: np.ndarray, s_rows: np.ndarray, s_w: np.ndarray, want_v: bool = False):
    """Per-row activation scales: out bf16 bits [M, N] (and the fp64 v)."""
    a = _c(xq, np.uint8)
    b = _c(wq, np.uint8)
    sr = _c(s_rows, np.float32)
    sw = _c(s_w, np.float32)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K and sr.shape == (M,) and sw.shape == (N,)
    out = np.empty((M, N), np.uint16)
    v = np.empty((M, N), np.float64) if want_v else None
    lib().oracle_scaled_mm_rows(_ptr(a), _ptr(b), _ptr(sr), _ptr(sw), M, N, K, _ptr(out), N, _ptr(v))
    return (out, v) if want_v else out


def exact_acc(xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    a = _c(xq, np.uint8)
    b = _c(wq, np.uint8)
    M, K = a.shape
    N, _ = b.shape
    acc = np.empty((M, N), np.float64)
    lib().oracle_exact_acc(_ptr(a), _ptr(b), M, N, K, _ptr(acc))
    return acc


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of the oracle's loops (results do not depend on it)."""
    lib().oracle_set_num_threads(int(n))
