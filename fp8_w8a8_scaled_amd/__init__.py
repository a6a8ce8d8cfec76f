"""fp8_w8a8_scaled_amd -- MI355X (gfx950) FP8 E4M3 W8A8 scaled-matmul layer.

Thin ctypes binding over ``libfp8mm.so`` (C ABI in ``include/fp8mm.h``).  This
module only marshals arguments: it checks dtypes, devices and strides, allocates
outputs with ``torch.empty`` and passes raw device pointers plus the current HIP
stream.  Every step of the layer runs in the library's HIP kernels; there is no
fallback.  If the library is missing, importing this package raises.

The layer:  out[m,n] = bf16((sum_k x_q[m,k] w_q[n,k]) * s_act * s_w[n]),
x_q = saturating RNE E4M3(x / s_act) -- bmm_fp8 with a per-tensor activation
scale and per-channel weight scales, bf16 output (vllm.cpp #252 "CORRECTION";
vllm.cpp #417 Finding 1).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8mm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python fp8_w8a8_scaled_amd/build.py` "
                      "(the package has no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, ELAUNCH, ESCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_FLOATS = 65536
SMALL_M_MAX = 64
THRESHOLD_MIN = 16
MAX_SHARDS = 8

_P, _I64, _F32, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t


class Shard(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("out", ctypes.c_void_p), ("ldo", ctypes.c_int64)]


def _decl(name, args, res=ctypes.c_int):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_quant_rmsnorm = _decl("fp8_quant_rmsnorm", [_P, _I64, _P, _F32, _F32, _P, _I64, _I64, _P])
_scaled_mm = _decl("fp8_scaled_mm", [_P, _P, _F32, _P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P])
_scaled_mm_arm = _decl("fp8_scaled_mm_arm", [_P, _P, _F32, _P, _P, _I64, _I64, _I64, _I64, _I32, _P, _SZ, _P])
_scaled_mm_merged = _decl("fp8_scaled_mm_merged", [_P, _P, _F32, _P, ctypes.POINTER(Shard), _I32, _I64, _I64, _P, _SZ, _P])
_quant_scaled_mm_fused = _decl("fp8_quant_scaled_mm_fused", [_I64, _I64, _I64, _I64, _F32, _I32])
_quant_rmsnorm_scaled_mm_merged = _decl("fp8_quant_rmsnorm_scaled_mm_merged",
                                        [_P, _I64, _P, _F32, _F32, _P, _P, _P, ctypes.POINTER(Shard), _I32, _I64,
                                         _I64, _P, _SZ, _P])
_quant_scaled_mm_merged = _decl("fp8_quant_scaled_mm_merged",
                                [_P, _I64, _F32, _P, _P, _P, ctypes.POINTER(Shard), _I32, _I64, _I64, _P, _SZ, _P])
_gate_up_silu_quant = _decl("fp8_gate_up_silu_quant",
                            [_P, _I64, _P, _F32, _F32, _P, _P, _P, _F32, _P, _I64, _I64, _I64, _P])
_gate_up_silu_quant_fused = _decl("fp8_gate_up_silu_quant_fused", [_I64, _I64, _I64, _I64, _F32, _F32, _I32])
_interleave_gate_up = _decl("fp8_interleave_gate_up", [_P, _P, _P, _P, _I64, _I64, _P])
_quant_per_token = _decl("fp8_quant_per_token", [_P, _I64, _P, _F32, _P, _P, _I64, _I64, _P])
_scaled_mm_per_token = _decl("fp8_scaled_mm_per_token", [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P])
_scaled_mm_merged_per_token = _decl("fp8_scaled_mm_merged_per_token",
                                    [_P, _P, _P, _P, ctypes.POINTER(Shard), _I32, _I64, _I64, _P, _SZ, _P])
_scaled_mm_f32 = _decl("fp8_scaled_mm_f32", [_P, _P, _F32, _P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P])
_scaled_mm_merged_f32 = _decl("fp8_scaled_mm_merged_f32",
                              [_P, _P, _F32, _P, ctypes.POINTER(Shard), _I32, _I64, _I64, _P, _SZ, _P])
_workspace_bytes = _decl("fp8_scaled_mm_workspace_bytes", [_I64, _I64, _I64], _SZ)
_select = _decl("fp8_scaled_mm_select", [_I64, _I64, _I64])
_set_threshold = _decl("fp8_set_large_m_threshold", [_I64])
_get_threshold = _decl("fp8_get_large_m_threshold", [], _I64)
_scales_equal = _decl("fp8_scales_bitwise_equal", [_P, _I32])
_strerror = _decl("fp8mm_strerror", [_I32], ctypes.c_char_p)
_quant_weight = _decl("fp8_quant_weight", [_P, _I64, _I64, _P, _P, _P])
_act_scale_ws = _decl("fp8_act_scale_workspace_bytes", [_I64, _I64], _SZ)
_act_scale = _decl("fp8_act_scale", [_P, _I64, _P, _F32, _I64, _I64, _P, _P, _SZ, _P])
_act_scale_noalloc = _decl("fp8_act_scale_noalloc", [_P, _I64, _P, _F32, _I64, _I64, _P, _P])
_silu_mul_quant = _decl("fp8_silu_mul_quant", [_P, _I64, _P, _I64, _F32, _P, _I64, _I64, _P])
_act_scale_silu_mul = _decl("fp8_act_scale_silu_mul", [_P, _I64, _P, _I64, _I64, _I64, _P, _P, _SZ, _P])
_qw_tensor_ws = _decl("fp8_quant_weight_per_tensor_workspace_bytes", [_I64, _I64], _SZ)
_qw_tensor = _decl("fp8_quant_weight_per_tensor", [_P, _I64, _I64, _P, _P, _P, _SZ, _P])
_expand_scales = _decl("fp8_expand_shard_scales", [_P, _P, _I32, _P, _P])
_requant_max = _decl("fp8_requant_max_scale", [_P, _P, _I64, _P, _P, _I32, _P, _P, _P])
_merge_admit = _decl("fp8_merge_admit", [_P, _I32, _I32, _P])
MERGE_EXACT, MERGE_MAX_SCALE = 0, 1


class Fp8mmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {strerror(status)} (status {status})")
        self.status = status


def strerror(status: int) -> str:
    return _strerror(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise Fp8mmError(status, what)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _codes(t: torch.Tensor, name: str) -> torch.Tensor:
    """E4M3 tensors travel as raw bytes: accept uint8 or float8_e4m3fn."""
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be uint8 E4M3 codes or float8_e4m3fn, got {t.dtype}")
    return t


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _row_major(t: torch.Tensor, name: str) -> int:
    _need(t.dim() == 2 and t.stride(1) == 1, f"{name} must be 2-D with unit column stride")
    return t.stride(0)


# ------------------------------------------------------------- activations --

def quant_rmsnorm(x: torch.Tensor, gamma: Optional[torch.Tensor], s_act: float, eps: float = 1e-6,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fused RMSNorm -> static E4M3 quant (gamma given) or plain static quant
    (gamma None) of bf16 x [M, K]; returns uint8 codes [M, K]."""
    _need(x.is_cuda and x.dtype == torch.bfloat16, "x must be a bf16 CUDA tensor")
    ldx = _row_major(x, "x")
    M, K = x.shape
    if gamma is not None:
        _need(gamma.is_cuda and gamma.dtype == torch.bfloat16 and gamma.is_contiguous()
              and gamma.numel() == K, "gamma must be a contiguous bf16 CUDA tensor of K elements")
    if out is None:
        out = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    out = _codes(out, "out")
    _need(out.is_contiguous() and tuple(out.shape) == (M, K), "out must be contiguous uint8 [M, K]")
    _check(_quant_rmsnorm(_ptr(x), ldx, _ptr(gamma), float(eps), float(s_act), _ptr(out), M, K, _stream(x)),
           "fp8_quant_rmsnorm")
    return out


def quant(x: torch.Tensor, s_act: float, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Plain static per-tensor E4M3 quant of bf16 x [M, K]."""
    return quant_rmsnorm(x, None, s_act, 0.0, out)


def act_scale(x: torch.Tensor, gamma: Optional[torch.Tensor] = None, eps: float = 1e-6) -> torch.Tensor:
    """Static scale calibration: device f32 [1] = fl32(amax / 448) of the tensor
    quant_rmsnorm(x, gamma, ., eps) would quantize (1 if amax == 0)."""
    _need(x.is_cuda and x.dtype == torch.bfloat16, "x must be a bf16 CUDA tensor")
    ldx = _row_major(x, "x")
    M, K = x.shape
    if gamma is not None:
        _need(gamma.is_cuda and gamma.dtype == torch.bfloat16 and gamma.is_contiguous() and gamma.numel() == K,
              "gamma must be a contiguous bf16 CUDA tensor of K elements")
    s = torch.empty(1, dtype=torch.float32, device=x.device)
    nbytes = int(_act_scale_ws(M, K))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    _check(_act_scale(_ptr(x), ldx, _ptr(gamma), float(eps), M, K, _ptr(s), _ptr(ws), ws.numel(), _stream(x)),
           "fp8_act_scale")
    return s


def act_scale_noalloc(x: torch.Tensor, gamma: Optional[torch.Tensor] = None, eps: float = 1e-6,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """act_scale without a workspace: the library's static per-GPU scratch holds
    the partial maxima (calls that overlap on one GPU race).  ``out`` (device
    f32 [1]) lets a caller that cannot allocate pass its own result buffer."""
    _need(x.is_cuda and x.dtype == torch.bfloat16, "x must be a bf16 CUDA tensor")
    ldx = _row_major(x, "x")
    M, K = x.shape
    if gamma is not None:
        _need(gamma.is_cuda and gamma.dtype == torch.bfloat16 and gamma.is_contiguous() and gamma.numel() == K,
              "gamma must be a contiguous bf16 CUDA tensor of K elements")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _need(out.is_cuda and out.dtype == torch.float32 and out.numel() >= 1, "out must be a device f32 tensor")
    _check(_act_scale_noalloc(_ptr(x), ldx, _ptr(gamma), float(eps), M, K, _ptr(out), _stream(x)),
           "fp8_act_scale_noalloc")
    return out


def _gate_up(gate: torch.Tensor, up: torch.Tensor):
    _need(gate.is_cuda and gate.dtype == torch.bfloat16 and up.is_cuda and up.dtype == torch.bfloat16,
          "gate and up must be bf16 CUDA tensors")
    _need(tuple(gate.shape) == tuple(up.shape) and gate.dim() == 2, "gate and up must be 2-D of equal shape")
    return _row_major(gate, "gate"), _row_major(up, "up")


def silu_mul_quant(gate: torch.Tensor, up: torch.Tensor, s_act: float,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """E4M3 codes [M, I] of silu(gate) * up (the bf16 MLP activation) quantized
    with the static scale s_act; gate/up may be strided views (the two halves of
    a merged gate_up output)."""
    ldg, ldu = _gate_up(gate, up)
    M, I = gate.shape
    if out is None:
        out = torch.empty((M, I), dtype=torch.uint8, device=gate.device)
    out = _codes(out, "out")
    _need(out.is_contiguous() and tuple(out.shape) == (M, I), "out must be contiguous uint8 [M, I]")
    _check(_silu_mul_quant(_ptr(gate), ldg, _ptr(up), ldu, float(s_act), _ptr(out), M, I, _stream(gate)),
           "fp8_silu_mul_quant")
    return out


def act_scale_silu_mul(gate: torch.Tensor, up: torch.Tensor) -> torch.Tensor:
    """Static scale calibration for silu_mul_quant: device f32 [1] =
    fl32(amax / 448) of the bf16 activation silu(gate) * up (1 if amax == 0)."""
    ldg, ldu = _gate_up(gate, up)
    M, I = gate.shape
    s = torch.empty(1, dtype=torch.float32, device=gate.device)
    nbytes = int(_act_scale_ws(M, I))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=gate.device)
    _check(_act_scale_silu_mul(_ptr(gate), ldg, _ptr(up), ldu, M, I, _ptr(s), _ptr(ws), ws.numel(), _stream(gate)),
           "fp8_act_scale_silu_mul")
    return s


# ------------------------------------------------------------------ weights --

def quant_weight(w: torch.Tensor):
    """Per-output-channel E4M3 quant of f32 w [N, K] -> (w_q uint8 [N, K], s_w f32 [N])."""
    _need(w.is_cuda and w.dtype == torch.float32 and w.dim() == 2 and w.is_contiguous(),
          "w must be a contiguous 2-D f32 CUDA tensor")
    N, K = w.shape
    wq = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    sw = torch.empty(N, dtype=torch.float32, device=w.device)
    _check(_quant_weight(_ptr(w), N, K, _ptr(wq), _ptr(sw), _stream(w)), "fp8_quant_weight")
    return wq, sw


# ------------------------------------- merged shards with per-tensor scales --

def quant_weight_per_tensor(w: torch.Tensor):
    """Per-tensor E4M3 quant of f32 w [N, K] -> (w_q uint8 [N, K], s f32 [1] on the device)."""
    _need(w.is_cuda and w.dtype == torch.float32 and w.dim() == 2 and w.is_contiguous(),
          "w must be a contiguous 2-D f32 CUDA tensor")
    N, K = w.shape
    wq = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty(1, dtype=torch.float32, device=w.device)
    ws = torch.empty(max(int(_qw_tensor_ws(N, K)), 16), dtype=torch.uint8, device=w.device)
    _check(_qw_tensor(_ptr(w), N, K, _ptr(wq), _ptr(s), _ptr(ws), ws.numel(), _stream(w)),
           "fp8_quant_weight_per_tensor")
    return wq, s


def _host_shards(shard_rows: Sequence[int], shard_scales: Sequence[float]):
    import numpy as np
    r = np.ascontiguousarray(np.asarray(shard_rows, dtype=np.int64))
    s = np.ascontiguousarray(np.asarray(shard_scales, dtype=np.float32))
    _need(r.ndim == 1 and r.shape == s.shape and 1 <= r.size <= MAX_SHARDS, f"1..{MAX_SHARDS} shards")
    return r, s


def expand_shard_scales(shard_rows: Sequence[int], shard_scales: Sequence[float], device="cuda") -> torch.Tensor:
    """Per-channel s_w f32 [sum rows] holding each shard's per-tensor scale (exact merge)."""
    r, s = _host_shards(shard_rows, shard_scales)
    sw = torch.empty(int(r.sum()), dtype=torch.float32, device=device)
    _check(_expand_scales(r.ctypes.data, s.ctypes.data, r.size, _ptr(sw), _stream(sw)), "fp8_expand_shard_scales")
    return sw


def requant_max_scale(w_q: torch.Tensor, shard_rows: Sequence[int], shard_scales: Sequence[float],
                      out: Optional[torch.Tensor] = None):
    """Requantize the shards of a merged weight [sum rows, K] to the largest
    shard scale (lossy merge): returns (w_q' uint8, s_w f32 [sum rows] filled
    with s_max, s_max as a Python float).  ``out`` may be ``w_q`` (in place)."""
    w_q = _codes(w_q, "w_q")
    _need(w_q.is_cuda and w_q.dim() == 2 and w_q.is_contiguous(), "w_q must be contiguous [rows, K]")
    r, s = _host_shards(shard_rows, shard_scales)
    _need(int(r.sum()) == w_q.shape[0], "shard rows must sum to the weight rows")
    if out is None:
        out = torch.empty_like(w_q)
    out = _codes(out, "out")
    _need(out.is_contiguous() and out.shape == w_q.shape, "out must be contiguous like w_q")
    sw = torch.empty(w_q.shape[0], dtype=torch.float32, device=w_q.device)
    smax = ctypes.c_float(0.0)
    _check(_requant_max(_ptr(w_q), _ptr(out), w_q.shape[1], r.ctypes.data, s.ctypes.data, r.size, _ptr(sw),
                        ctypes.byref(smax), _stream(w_q)), "fp8_requant_max_scale")
    return out, sw, float(smax.value)


def merge_admit(input_scales: Sequence[float], policy: int = MERGE_EXACT):
    """(merge?, s_act): whether projections with these static input scales run
    as one merged launch under ``policy``, and the one input scale it uses."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(input_scales, dtype=np.float32))
    s = ctypes.c_float(0.0)
    st = _merge_admit(a.ctypes.data, a.size, int(policy), ctypes.byref(s))
    if st < 0:
        raise Fp8mmError(st, "fp8_merge_admit")
    return bool(st), (float(s.value) if st == 1 else None)


# --------------------------------------------------------------------- GEMM --

def _gemm_args(x_q, w_q, s_w):
    x_q = _codes(x_q, "x_q")
    w_q = _codes(w_q, "w_q")
    _need(x_q.is_cuda and x_q.dim() == 2 and x_q.is_contiguous(), "x_q must be contiguous [M, K]")
    _need(w_q.is_cuda and w_q.dim() == 2 and w_q.is_contiguous(), "w_q must be contiguous [N, K]")
    _need(x_q.shape[1] == w_q.shape[1], "x_q and w_q must share K")
    _need(s_w.is_cuda and s_w.dtype == torch.float32 and s_w.is_contiguous() and s_w.numel() == w_q.shape[0],
          "s_w must be a contiguous f32 CUDA tensor of N elements")
    return x_q, w_q


def workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_workspace_bytes(M, N, K))


def _workspace(M, N, K, device, workspace):
    nbytes = workspace_bytes(M, N, K)
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def _out_dtype(out_dtype):
    _need(out_dtype in (torch.bfloat16, torch.float32), "out_dtype must be torch.bfloat16 or torch.float32")
    return out_dtype


def scaled_mm(x_q: torch.Tensor, w_q: torch.Tensor, s_act: float, s_w: torch.Tensor,
              out: Optional[torch.Tensor] = None, arm: Optional[int] = None,
              workspace: Optional[torch.Tensor] = None, out_dtype=None) -> torch.Tensor:
    """[M, N] = (x_q . w_q^T) * s_act * s_w, as bf16 (default) or f32
    (out_dtype=torch.float32, or an f32 ``out``).  arm None = dispatcher,
    0 = force the small-M kernel, 1 = force the large-M kernel (bf16 only)."""
    x_q, w_q = _gemm_args(x_q, w_q, s_w)
    M, K = x_q.shape
    N = w_q.shape[0]
    dt = _out_dtype(out_dtype or (out.dtype if out is not None else torch.bfloat16))
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=x_q.device)
    _need(out.dtype == dt and out.is_cuda and out.shape == (M, N), f"out must be {dt} [M, N]")
    ldo = _row_major(out, "out")
    ws, wsb = _workspace(M, N, K, x_q.device, workspace)
    if dt == torch.float32:
        _need(arm is None, "arm forcing is bf16-only")
        st = _scaled_mm_f32(_ptr(x_q), _ptr(w_q), float(s_act), _ptr(s_w), _ptr(out), ldo, M, N, K,
                            _ptr(ws), wsb, _stream(x_q))
    elif arm is None:
        st = _scaled_mm(_ptr(x_q), _ptr(w_q), float(s_act), _ptr(s_w), _ptr(out), ldo, M, N, K,
                        _ptr(ws), wsb, _stream(x_q))
    else:
        st = _scaled_mm_arm(_ptr(x_q), _ptr(w_q), float(s_act), _ptr(s_w), _ptr(out), ldo, M, N, K, int(arm),
                            _ptr(ws), wsb, _stream(x_q))
    _check(st, "fp8_scaled_mm")
    return out


def scaled_mm_merged(x_q: torch.Tensor, w_q: torch.Tensor, s_act: float, s_w: torch.Tensor,
                     shard_sizes: Sequence[int], outs: Optional[Sequence[torch.Tensor]] = None,
                     workspace: Optional[torch.Tensor] = None, out_dtype=None):
    """One launch over a concatenated weight [sum n_i, K]; returns the list of
    [M, n_i] shard outputs, bf16 (default) or f32 (or fills ``outs``)."""
    x_q, w_q = _gemm_args(x_q, w_q, s_w)
    M, K = x_q.shape
    _need(sum(shard_sizes) == w_q.shape[0], "shard sizes must sum to the weight rows")
    _need(1 <= len(shard_sizes) <= MAX_SHARDS, f"1..{MAX_SHARDS} shards")
    dt = _out_dtype(out_dtype or (outs[0].dtype if outs else torch.bfloat16))
    if outs is None:
        outs = [torch.empty((M, n), dtype=dt, device=x_q.device) for n in shard_sizes]
    arr = (Shard * len(shard_sizes))()
    for i, (n, o) in enumerate(zip(shard_sizes, outs)):
        _need(o.dtype == dt and o.is_cuda and o.shape == (M, n), f"shard outputs must be {dt} [M, n_i]")
        arr[i] = Shard(int(n), o.data_ptr(), _row_major(o, "out"))
    ws, wsb = _workspace(M, w_q.shape[0], K, x_q.device, workspace)
    fn = _scaled_mm_merged_f32 if dt == torch.float32 else _scaled_mm_merged
    _check(fn(_ptr(x_q), _ptr(w_q), float(s_act), _ptr(s_w), arr, len(shard_sizes), M, K,
              _ptr(ws), wsb, _stream(x_q)), "fp8_scaled_mm_merged")
    return list(outs)


def quant_rmsnorm_scaled_mm_merged(x: torch.Tensor, gamma: Optional[torch.Tensor], s_act: float, eps: float,
                                   w_q: torch.Tensor, s_w: torch.Tensor, shard_sizes: Sequence[int],
                                   outs: Optional[Sequence[torch.Tensor]] = None, x_q: Optional[torch.Tensor] = None,
                                   workspace: Optional[torch.Tensor] = None):
    """Fused RMSNorm quant (gamma given) or plain static quant (gamma None) of
    bf16 x [M, K] and the merged GEMM on the codes, one launch where the
    small-M kernel takes the shape: returns (list of bf16 [M, n_i] outputs,
    x_q uint8 [M, K])."""
    _need(x.is_cuda and x.dtype == torch.bfloat16, "x must be a bf16 CUDA tensor")
    ldx = _row_major(x, "x")
    M, K = x.shape
    if gamma is not None:
        _need(gamma.is_cuda and gamma.dtype == torch.bfloat16 and gamma.is_contiguous()
              and gamma.numel() == K, "gamma must be a contiguous bf16 CUDA tensor of K elements")
    w_q = _codes(w_q, "w_q")
    _need(w_q.is_cuda and w_q.dim() == 2 and w_q.shape[1] == K and w_q.is_contiguous(),
          "w_q must be contiguous E4M3 codes [N, K]")
    _need(s_w.is_cuda and s_w.dtype == torch.float32 and s_w.is_contiguous() and s_w.numel() == w_q.shape[0],
          "s_w must be a contiguous f32 CUDA tensor of N elements")
    _need(sum(shard_sizes) == w_q.shape[0], "shard sizes must sum to the weight rows")
    _need(1 <= len(shard_sizes) <= MAX_SHARDS, f"1..{MAX_SHARDS} shards")
    if x_q is None:
        x_q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    x_q = _codes(x_q, "x_q")
    _need(x_q.is_contiguous() and tuple(x_q.shape) == (M, K), "x_q must be contiguous uint8 [M, K]")
    if outs is None:
        outs = [torch.empty((M, n), dtype=torch.bfloat16, device=x.device) for n in shard_sizes]
    arr = (Shard * len(shard_sizes))()
    for i, (n, o) in enumerate(zip(shard_sizes, outs)):
        _need(o.dtype == torch.bfloat16 and o.is_cuda and o.shape == (M, n), "shard outputs must be bf16 [M, n_i]")
        arr[i] = Shard(int(n), o.data_ptr(), _row_major(o, "out"))
    ws, wsb = _workspace(M, w_q.shape[0], K, x.device, workspace)
    if gamma is None:
        _check(_quant_scaled_mm_merged(_ptr(x), ldx, float(s_act), _ptr(x_q), _ptr(w_q), _ptr(s_w), arr,
                                       len(shard_sizes), M, K, _ptr(ws), wsb, _stream(x)), "fp8_quant_scaled_mm_merged")
    else:
        _check(_quant_rmsnorm_scaled_mm_merged(_ptr(x), ldx, _ptr(gamma), float(eps), float(s_act), _ptr(x_q),
                                               _ptr(w_q), _ptr(s_w), arr, len(shard_sizes), M, K, _ptr(ws), wsb,
                                               _stream(x)), "fp8_quant_rmsnorm_scaled_mm_merged")
    return list(outs), x_q


def quant_scaled_mm_merged(x: torch.Tensor, s_act: float, w_q: torch.Tensor, s_w: torch.Tensor,
                           shard_sizes: Sequence[int], outs: Optional[Sequence[torch.Tensor]] = None,
                           x_q: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Static quant of bf16 x [M, K] and the merged GEMM on the codes, one
    launch where the small-M kernel takes the shape (M <= 8): returns (list of
    bf16 [M, n_i] outputs, x_q uint8 [M, K])."""
    return quant_rmsnorm_scaled_mm_merged(x, None, s_act, 0.0, w_q, s_w, shard_sizes, outs, x_q, workspace)


def quant_scaled_mm_fused(M: int, N: int, K: int, ldx: Optional[int] = None, s_act: float = 1.0,
                          rmsnorm: bool = False) -> bool:
    """Whether quant_scaled_mm_merged (or, rmsnorm, quant_rmsnorm_scaled_mm_merged
    with a gamma) runs as one launch for this shape."""
    return bool(_quant_scaled_mm_fused(M, N, K, K if ldx is None else ldx, float(s_act), int(bool(rmsnorm))))


def quant_scaled_mm(x: torch.Tensor, s_act: float, w_q: torch.Tensor, s_w: torch.Tensor,
                    out: Optional[torch.Tensor] = None, x_q: Optional[torch.Tensor] = None):
    """Static quant of bf16 x and one projection: returns (bf16 [M, N], x_q)."""
    outs, xq = quant_scaled_mm_merged(x, s_act, w_q, s_w, [w_q.shape[0]], None if out is None else [out], x_q)
    return outs[0], xq


# ------------------------------------- gate_up with the SiLU*mul epilogue --

def interleave_gate_up(w_q: torch.Tensor, s_w: torch.Tensor):
    """Load-time layout of a merged gate_up weight [W_gate; W_up] (uint8 [2I, K],
    f32 [2I]) for gate_up_silu_quant: 8 gate rows, then the up rows of the same
    8 columns, per 16-row tile.  Returns (w_il, s_il)."""
    w_q = _codes(w_q, "w_q")
    _need(w_q.is_cuda and w_q.dim() == 2 and w_q.is_contiguous() and w_q.shape[0] % 2 == 0,
          "w_q must be contiguous E4M3 codes [2I, K]")
    _need(s_w.is_cuda and s_w.dtype == torch.float32 and s_w.is_contiguous() and s_w.numel() == w_q.shape[0],
          "s_w must be a contiguous f32 CUDA tensor of 2I elements")
    N, K = w_q.shape
    w_il = torch.empty_like(w_q)
    s_il = torch.empty_like(s_w)
    _check(_interleave_gate_up(_ptr(w_q), _ptr(s_w), _ptr(w_il), _ptr(s_il), N // 2, K, _stream(w_q)),
           "fp8_interleave_gate_up")
    return w_il, s_il


def gate_up_silu_quant_fused(M: int, I: int, K: int, s_act: float, s_down: float, quant: int = 0,
                             ldx: Optional[int] = None) -> bool:
    """Whether gate_up_silu_quant takes the shape: quant 0 (x_q given), 1 (plain
    static quant of x in the launch), 2 (fused RMSNorm quant)."""
    return bool(_gate_up_silu_quant_fused(M, I, K, K if ldx is None else ldx, float(s_act), float(s_down),
                                          int(quant)))


def gate_up_silu_quant(w_il: torch.Tensor, s_il: torch.Tensor, s_act: float, s_down: float,
                       x_q: Optional[torch.Tensor] = None, x: Optional[torch.Tensor] = None,
                       gamma: Optional[torch.Tensor] = None, eps: float = 1e-6,
                       out: Optional[torch.Tensor] = None, x_q_out: Optional[torch.Tensor] = None):
    """The merged gate_up projection on the interleaved weight with the SiLU*mul
    -> E4M3 quant (scale s_down) as its epilogue, one launch: returns h_q uint8
    [M, I].  Input: the codes x_q [M, K], or bf16 x [M, K] quantized in the
    launch (with gamma: the fused RMSNorm quant; x_q_out, if given, receives
    the codes).  Raises Fp8mmError (EUNSUPPORTED) where the launch does not
    take the shape (gate_up_silu_quant_fused)."""
    w_il = _codes(w_il, "w_il")
    _need(w_il.is_cuda and w_il.dim() == 2 and w_il.is_contiguous(), "w_il must be contiguous E4M3 codes [2I, K]")
    _need(s_il.is_cuda and s_il.dtype == torch.float32 and s_il.is_contiguous() and s_il.numel() == w_il.shape[0],
          "s_il must be a contiguous f32 CUDA tensor of 2I elements")
    N, K = w_il.shape
    I = N // 2
    if x is not None:
        _need(x_q is None, "give x_q or x, not both")
        _need(x.is_cuda and x.dtype == torch.bfloat16 and x.dim() == 2 and x.shape[1] == K,
              "x must be a bf16 CUDA tensor [M, K]")
        ldx = _row_major(x, "x")
        M = x.shape[0]
        if gamma is not None:
            _need(gamma.is_cuda and gamma.dtype == torch.bfloat16 and gamma.is_contiguous()
                  and gamma.numel() == K, "gamma must be a contiguous bf16 CUDA tensor of K elements")
        xq = None
        if x_q_out is not None:
            xq = _codes(x_q_out, "x_q_out")
            _need(xq.is_contiguous() and tuple(xq.shape) == (M, K), "x_q_out must be contiguous uint8 [M, K]")
        dev = x.device
    else:
        _need(x_q is not None and gamma is None, "x_q (codes) or x (bf16) is needed; gamma only with x")
        xq = _codes(x_q, "x_q")
        _need(xq.is_cuda and xq.is_contiguous() and xq.dim() == 2 and xq.shape[1] == K,
              "x_q must be contiguous E4M3 codes [M, K]")
        M, ldx = xq.shape[0], K
        dev = xq.device
    if out is None:
        out = torch.empty((M, I), dtype=torch.uint8, device=dev)
    out = _codes(out, "out")
    _need(out.is_contiguous() and tuple(out.shape) == (M, I), "out must be contiguous uint8 [M, I]")
    _check(_gate_up_silu_quant(_ptr(x), ldx, _ptr(gamma), float(eps), float(s_act), _ptr(xq), _ptr(w_il),
                               _ptr(s_il), float(s_down), _ptr(out), M, I, K, _stream(w_il)),
           "fp8_gate_up_silu_quant")
    return out


# ------------------------------------------------------ per-token scales --

def quant_per_token(x: torch.Tensor, gamma: Optional[torch.Tensor] = None, eps: float = 1e-6,
                    out: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None):
    """Per-token dynamic E4M3 quant of bf16 x [M, K] (RMSNorm first when gamma
    is given): returns (codes uint8 [M, K], scales f32 [M])."""
    _need(x.is_cuda and x.dtype == torch.bfloat16, "x must be a bf16 CUDA tensor")
    ldx = _row_major(x, "x")
    M, K = x.shape
    if gamma is not None:
        _need(gamma.is_cuda and gamma.dtype == torch.bfloat16 and gamma.is_contiguous() and gamma.numel() == K,
              "gamma must be a contiguous bf16 CUDA tensor of K elements")
    if out is None:
        out = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(M, dtype=torch.float32, device=x.device)
    out = _codes(out, "out")
    _need(out.is_contiguous() and tuple(out.shape) == (M, K), "out must be contiguous uint8 [M, K]")
    _need(scales.dtype == torch.float32 and scales.is_contiguous() and scales.numel() == M, "scales must be f32 [M]")
    _check(_quant_per_token(_ptr(x), ldx, _ptr(gamma), float(eps), _ptr(out), _ptr(scales), M, K, _stream(x)),
           "fp8_quant_per_token")
    return out, scales


def scaled_mm_per_token(x_q: torch.Tensor, w_q: torch.Tensor, s_rows: torch.Tensor, s_w: torch.Tensor,
                        out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [M, N] = bf16((x_q . w_q^T) * s_rows[m] * s_w[n])."""
    x_q, w_q = _gemm_args(x_q, w_q, s_w)
    M, K = x_q.shape
    N = w_q.shape[0]
    _need(s_rows.is_cuda and s_rows.dtype == torch.float32 and s_rows.is_contiguous() and s_rows.numel() == M,
          "s_rows must be a contiguous f32 CUDA tensor of M elements")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x_q.device)
    _need(out.dtype == torch.bfloat16 and out.is_cuda and out.shape == (M, N), "out must be bf16 [M, N]")
    ws, wsb = _workspace(M, N, K, x_q.device, workspace)
    _check(_scaled_mm_per_token(_ptr(x_q), _ptr(w_q), _ptr(s_rows), _ptr(s_w), _ptr(out), _row_major(out, "out"),
                                M, N, K, _ptr(ws), wsb, _stream(x_q)), "fp8_scaled_mm_per_token")
    return out


def scaled_mm_merged_per_token(x_q: torch.Tensor, w_q: torch.Tensor, s_rows: torch.Tensor, s_w: torch.Tensor,
                               shard_sizes: Sequence[int], outs: Optional[Sequence[torch.Tensor]] = None,
                               workspace: Optional[torch.Tensor] = None):
    x_q, w_q = _gemm_args(x_q, w_q, s_w)
    M, K = x_q.shape
    _need(sum(shard_sizes) == w_q.shape[0], "shard sizes must sum to the weight rows")
    _need(1 <= len(shard_sizes) <= MAX_SHARDS, f"1..{MAX_SHARDS} shards")
    _need(s_rows.is_cuda and s_rows.dtype == torch.float32 and s_rows.is_contiguous() and s_rows.numel() == M,
          "s_rows must be a contiguous f32 CUDA tensor of M elements")
    if outs is None:
        outs = [torch.empty((M, n), dtype=torch.bfloat16, device=x_q.device) for n in shard_sizes]
    arr = (Shard * len(shard_sizes))()
    for i, (n, o) in enumerate(zip(shard_sizes, outs)):
        _need(o.dtype == torch.bfloat16 and o.is_cuda and o.shape == (M, n), "shard outputs must be bf16 [M, n_i]")
        arr[i] = Shard(int(n), o.data_ptr(), _row_major(o, "out"))
    ws, wsb = _workspace(M, w_q.shape[0], K, x_q.device, workspace)
    _check(_scaled_mm_merged_per_token(_ptr(x_q), _ptr(w_q), _ptr(s_rows), _ptr(s_w), arr, len(shard_sizes), M, K,
                                       _ptr(ws), wsb, _stream(x_q)), "fp8_scaled_mm_merged_per_token")
    return list(outs)


# --------------------------------------------------------------- dispatcher --

def select(M: int, N: int, K: int) -> int:
    """0 = small-M kernel, 1 = large-M kernel (pure function of M and T)."""
    return int(_select(M, N, K))


def set_large_m_threshold(t: int) -> None:
    _check(_set_threshold(int(t)), "fp8_set_large_m_threshold")


def get_large_m_threshold() -> int:
    return int(_get_threshold())


def scales_bitwise_equal(scales: Sequence[float]) -> bool:
    """Merge predicate: all f32 input scales have the same bit pattern."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(scales, dtype=np.float32))
    st = _scales_equal(a.ctypes.data, a.size)
    if st < 0:
        raise Fp8mmError(st, "fp8_scales_bitwise_equal")
    return bool(st)


def raw_lib() -> ctypes.CDLL:
    """The loaded C library (for direct C-ABI calls)."""
    return _lib
