"""Exact-rational second checker for tiny cases (TEST INFRASTRUCTURE ONLY).

Written independently of ``fp8_oracle.c``: every step is exact arithmetic on
``fractions.Fraction`` followed by an explicit rounding rule, so it pins the C
oracle by brute force on small shapes (M=2, N=3, K=4 and the like).

 - E4M3 values come from enumerating sign/exponent/mantissa, and encoding is a
   brute-force nearest search over all 254 finite values (ties to the even code).
 - IEEE fp32 division and bf16 rounding are done by rounding the exact quotient
   or value with round-half-even at the format's quantum.

The layer it checks: out = bf16((sum_k q(x)[m,k] W_q[n,k]) * s_act * s_w[n]),
q(x) = saturating RNE E4M3 of fl32(x / s_act) (vllm.cpp #252 "CORRECTION" for
bmm_fp8's two scales; vllm.cpp #417 Finding 1 for the bf16 output and the
ranked follow-ons for the static per-tensor quant).
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

# ----------------------------------------------------------------- formats --

_E4M3 = {}
for _s in (0, 1):
    for _e in range(16):
        for _m in range(8):
            _code = (_s << 7) | (_e << 3) | _m
            if _e == 15 and _m == 7:
                continue  # NaN
            if _e == 0:
                _mag = Fraction(_m, 512)
            else:
                _mag = Fraction(8 + _m, 8) * (Fraction(2) ** (_e - 7))
            _E4M3[_code] = -_mag if _s else _mag

FINITE_CODES = sorted(_E4M3)          # 254 codes


def e4m3_value(code: int) -> Fraction:
    return _E4M3[code]


def e4m3_encode_exact(t: Fraction, negative: bool) -> int:
    """Saturating RNE of an exact value; ``negative`` carries the sign of zero."""
    if abs(t) >= 448:
        return 0xFE if negative else 0x7E
    best = None
    for c in FINITE_CODES:
        v = _E4M3[c]
        if (c & 0x80) != (0x80 if negative else 0):
            continue
        d = abs(v - t)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    return best[1]


def _round_half_even(q: Fraction) -> int:
    fl = math.floor(q)
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_to_float(v: Fraction, sig_bits: int, emin: int) -> Fraction:
    """Round an exact value to a binary format with ``sig_bits`` significant bits
    and smallest normal exponent ``emin`` (subnormals below), ties to even.
    Overflow is not handled (the callers stay in range)."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix floating log2 rounding
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (sig_bits - 1))
    r = _round_half_even(a / quantum) * quantum
    return r if v > 0 else -r


def fl32(v: Fraction) -> Fraction:
    return round_to_float(v, 24, -126)


def bf16(v: Fraction) -> Fraction:
    return round_to_float(v, 8, -126)


def bf16_bits_value(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    f = struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    return Fraction(f)


def bf16_bits(v: Fraction, negative_zero: bool = False) -> int:
    """Bit pattern of an exactly representable bf16 value."""
    if v == 0:
        return 0x8000 if negative_zero else 0
    f = float(v)
    (u,) = struct.unpack("<I", struct.pack("<f", f))
    assert Fraction(f) == v and (u & 0xFFFF) == 0, "not a bf16 value"
    return u >> 16


# ------------------------------------------------------------------ layer ---

def quant(x_bits, s_act: float):
    """x_q codes for bf16 bit patterns x (list of rows) with fp32 scale s_act."""
    s = Fraction(s_act)
    out = []
    for row in x_bits:
        r = []
        for b in row:
            neg = bool(b & 0x8000)
            if (b & 0x7FFF) >= 0x7F80:                    # inf saturates, NaN stays NaN
                r.append((0x80 if neg else 0) | (0x7E if (b & 0x7FFF) == 0x7F80 else 0x7F))
                continue
            xv = bf16_bits_value(b)
            t = fl32(xv / s)
            r.append(e4m3_encode_exact(t, neg))
        out.append(r)
    return out


def scaled_mm(xq, wq, s_act: float, s_w):
    """Returns (bf16 bit patterns, exact v) with one rounding of the exact v."""
    sa = Fraction(s_act)
    bits, vals = [], []
    for a in xq:
        rb, rv = [], []
        for n, w in enumerate(wq):
            acc = sum((e4m3_value(p) * e4m3_value(q) for p, q in zip(a, w)), Fraction(0))
            v = acc * sa * Fraction(s_w[n])
            r = bf16(v)
            rb.append(bf16_bits(r))
            rv.append(v)
        bits.append(rb)
        vals.append(rv)
    return bits, vals


# ------------------------------------------------------- per-token scales ---

def act_scale(row_bits) -> float:
    """fl32(amax / 448) over the finite values of bf16 patterns (1 when 0)."""
    amax = Fraction(0)
    for b in row_bits:
        if (b & 0x7F80) == 0x7F80:
            continue                                      # inf / NaN
        amax = max(amax, abs(bf16_bits_value(b)))
    if amax == 0:
        return 1.0
    return float(fl32(amax / 448))


def quant_per_token(x_bits):
    """(codes, scales): every row quantized with its own act_scale."""
    codes, scales = [], []
    for row in x_bits:
        s = act_scale(row)
        scales.append(s)
        codes.append(quant([row], s)[0])
    return codes, scales


def scaled_mm_rows(xq, wq, s_rows, s_w):
    """bf16 patterns of (acc[m,n] * s_rows[m]) * s_w[n], one rounding."""
    bits = []
    for a, s in zip(xq, s_rows):
        bits.append(scaled_mm([a], wq, s, s_w)[0][0])
    return bits


# ------------------------------------------------- merged-shard requant ----

def requant_max_scale(codes_by_shard, scales):
    """Exact-rational requant of shards with per-tensor scales to the largest:
    w = fl32(dec(c) * s_i), c' = nearest E4M3 (ties even, saturating) of
    fl32(w / s_max), the sign of zero taken from c.  Returns (shards of codes,
    s_max)."""
    s_max = max(Fraction(s) for s in scales)
    out = []
    for rows, s in zip(codes_by_shard, scales):
        si = Fraction(s)
        o = []
        for row in rows:
            r = []
            for c in row:
                if (c & 0x7F) == 0x7F:
                    r.append(c)                                   # NaN kept
                    continue
                w = fl32(e4m3_value(c) * si)
                t = fl32(w / s_max)
                r.append(e4m3_encode_exact(t, bool(c & 0x80)))
            o.append(r)
        out.append(o)
    return out, float(s_max)
