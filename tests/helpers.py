"""Shared test helpers: host<->device marshalling and the output tolerance.

Tolerance (GPU vs oracle, per element), from the parity bar of the layer:
    |gpu - ref| <= max(2 * ulp_bf16(ref), 1e-3 * ||v[m, :]||_2)
where v is the oracle's unrounded fp64 output row, ulp_bf16(y) = 2^(floor(log2|y|) - 7)
for normal y and 2^-133 below the normal range.  FP8 activation bytes are compared
bit for bit instead.
"""
from __future__ import annotations

import numpy as np


def bf16_dev(a_u16: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16).to(device)


def u8_dev(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def f32_dev(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host_u16(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t) -> np.ndarray:
    import torch
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return t.detach().contiguous().cpu().numpy()


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(y: np.ndarray) -> np.ndarray:
    a = np.abs(y)
    out = np.full(a.shape, 2.0 ** -133)
    nrm = a >= 2.0 ** -126
    out[nrm] = 2.0 ** (np.floor(np.log2(a[nrm])) - 7)
    return out


def assert_within_tolerance(gpu_bits: np.ndarray, ref_bits: np.ndarray, v: np.ndarray, what: str = ""):
    g = bf16_f64(gpu_bits)
    r = bf16_f64(ref_bits)
    assert g.shape == r.shape == v.shape
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    row = np.sqrt(np.sum(v * v, axis=1, keepdims=True))
    tol = np.maximum(2.0 * ulp_bf16(r), 1e-3 * row)
    err = np.abs(g - r)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance, e.g. "
                             + "; ".join(f"[{m},{n}] gpu={g[m, n]!r} ref={r[m, n]!r} tol={tol[m, n]:.3g}"
                                         for m, n in i))
    return float((err / tol).max()) if err.size else 0.0


def ulps_apart(gpu_bits: np.ndarray, ref_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 units at the reference's scale."""
    return np.abs(bf16_f64(gpu_bits) - bf16_f64(ref_bits)) / ulp_bf16(bf16_f64(ref_bits))


def assert_within_tolerance_rows(gpu_bits: np.ndarray, ref_bits: np.ndarray, v: np.ndarray, what: str = "",
                                 block: int = 256):
    """assert_within_tolerance over row blocks (large outputs, bounded memory)."""
    worst = 0.0
    for r0 in range(0, ref_bits.shape[0], block):
        worst = max(worst, assert_within_tolerance(gpu_bits[r0:r0 + block], ref_bits[r0:r0 + block],
                                                   v[r0:r0 + block], f"{what} rows {r0}+"))
    return worst


BF16_NAN = 0x7FC0
