"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something other than itself: the E4M3FN
and bf16 definitions worked by hand (tests/golden/), brute force over all codes
or all bf16 bit patterns, an exact-rational re-implementation on tiny shapes
(oracle/exact.py), closed forms and invariants of the layer
out = bf16((q(x) W_q^T) s_act s_w[n]).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32(s):
    return np.float32(float.fromhex(s) if s not in ("inf", "-inf", "nan") else float(s))


# ------------------------------------------------------------------ E4M3 ---

def test_e4m3_table_structure():
    t = oracle.e4m3_table()
    finite = [c for c in range(256) if not np.isnan(t[c])]
    assert len(finite) == 254
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9
    mags = t[:0x7F]
    assert np.all(np.diff(mags) > 0), "codes 0x00..0x7E must be strictly increasing"
    assert len(set(mags.tolist())) == 127
    for c in range(0x7F):
        assert t[c | 0x80] == -t[c]
    assert np.signbit(t[0x80]) and t[0x80] == 0.0


def test_e4m3_table_matches_exact_enumeration():
    # exact.py enumerates sign/exponent/mantissa independently with Fractions
    t = oracle.e4m3_table()
    for c in exact.FINITE_CODES:
        assert Fraction(t[c]) == exact.e4m3_value(c), hex(c)


def test_e4m3_roundtrip_all_finite_codes():
    t = oracle.e4m3_table()
    codes = np.array(exact.FINITE_CODES, np.uint8)
    enc = oracle.e4m3_encode(t[codes].astype(np.float32))
    assert np.array_equal(enc, codes)


def test_e4m3_hand_values():
    g = _golden("e4m3_encode_hand.json")
    xs = np.array([_f32(c["x"]) for c in g["cases"]], np.float32)
    want = np.array([int(c["code"], 16) for c in g["cases"]], np.uint8)
    got = oracle.e4m3_encode(xs)
    bad = [(c["x"], c["code"], hex(v)) for c, v, w in zip(g["cases"], got, want) if v != w]
    assert not bad, bad


def _brute_force_encode(t32: np.ndarray) -> np.ndarray:
    """Nearest of the 127 non-negative magnitudes by exhaustive distance, ties to
    the even code, saturation at 448, NaN -> 0x7F, sign bit copied."""
    tab = oracle.e4m3_table()[:0x7F]
    a = np.abs(t32.astype(np.float64))
    out = np.zeros(t32.shape, np.uint8)
    fin = ~np.isnan(a)
    d = np.abs(a[fin, None] - tab[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates choose the even code
    idx = np.arange(0x7F)[None, :]
    even_pref = np.where(cand & (idx % 2 == 0), idx, 10_000).min(axis=1)
    any_pref = np.where(cand, idx, 10_000).min(axis=1)
    code = np.where(even_pref < 10_000, even_pref, any_pref)
    code = np.where(a[fin] >= 448.0, 0x7E, code)
    out[fin] = code.astype(np.uint8)
    out[~fin] = 0x7F
    out |= np.where(np.signbit(t32), 0x80, 0).astype(np.uint8)
    return out


@pytest.mark.parametrize("s_act", [1.0, 0.5, 3.0, 1.0 / 7.0, 0.2])
def test_quant_encoder_exhaustive_bf16(s_act):
    """All 65536 bf16 patterns: x / s_act in IEEE fp32 (numpy), then brute force."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    xf = oracle.bf16_bits_to_f32(bits)
    with np.errstate(all="ignore"):
        t = (xf / np.float32(s_act)).astype(np.float32)
    want = _brute_force_encode(t)
    got = oracle.quant_act(bits.reshape(1, -1), s_act).reshape(-1)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]


def test_encoder_random_fp32_vs_brute_force():
    g = np.random.Generator(np.random.PCG64(1234))
    t = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * np.float32(40),
        (g.random(20000) * 2 - 1).astype(np.float32) * np.float32(2 ** -6),
        (g.random(2000) * 1000).astype(np.float32),
    ])
    assert np.array_equal(oracle.e4m3_encode(t), _brute_force_encode(t))


# ------------------------------------------------------------------ bf16 ---

def test_bf16_rounding_against_exact_and_torch():
    import torch
    g = np.random.Generator(np.random.PCG64(7))
    vals = list(g.standard_normal(3000) * 10.0 ** g.integers(-40, 38, 3000))
    # exact ties between adjacent bf16 values and subnormal-range values
    vals += [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(2.0 + 2 ** -7), 2 ** -130 * 1.5, 2 ** -133 * 0.5,
             2 ** -133 * 1.5, 3.0 * 2 ** -134]
    for v in vals:
        want_val = exact.bf16(Fraction(v))
        got = oracle.f64_to_bf16(v)
        if want_val == 0:
            assert got & 0x7FFF == 0
        else:
            assert got == exact.bf16_bits(want_val), (v, hex(got))
    # fp32 inputs: the library cast (round to nearest even) is a second reference
    f = (g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000)).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(x) for x in f], np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------- the layer ---

def test_tiny_product_hand_worked():
    g = _golden("tiny_product.json")
    xq = np.array([[int(c, 16) for c in g["x_q"]]], np.uint8)
    wq = np.array([[int(c, 16) for c in r] for r in g["W_q"]], np.uint8)
    s_act = float.fromhex(g["s_act"])
    s_w = np.array([float.fromhex(s) for s in g["s_w"]], np.float32)
    acc = oracle.exact_acc(xq, wq)[0]
    assert [Fraction(a) for a in acc] == [Fraction(s) for s in g["acc_exact"]]
    out, v = oracle.scaled_mm(xq, wq, s_act, s_w, want_v=True)
    assert [Fraction(x) for x in v[0]] == [Fraction(s) for s in g["v_exact"]]
    assert [hex(b) for b in out[0]] == g["out_bf16"]


def test_brute_force_2x3x4_against_exact_rationals():
    """Whole pipeline (quant -> exact GEMM -> bf16) in Fractions vs the oracle."""
    g = np.random.Generator(np.random.PCG64(99))
    t = oracle.e4m3_table()
    for it in range(400):
        x = wl.to_bf16_bits(g.standard_normal((2, 4)).astype(np.float32) * np.float32(g.choice([0.01, 1, 30])))
        s_act = float(np.float32(g.choice([1.0, 0.5, 1 / 7, 0.0123, 3.7])))
        codes = wl.FINITE_CODE_VALUES[g.integers(0, 254, (3, 4))]
        if it % 5 == 0:  # restrict to a small code set to hit ties and cancellations
            codes = np.array([0x38, 0xB8, 0x40, 0x01, 0x81, 0x7E, 0xFE], np.uint8)[g.integers(0, 7, (3, 4))]
        s_w = (g.random(3) * 0.01 + 1e-4).astype(np.float32)
        xq = oracle.quant_act(x, s_act)
        xq_exact = np.array(exact.quant(x.tolist(), s_act), np.uint8)
        assert np.array_equal(xq, xq_exact), (x, s_act)
        out = oracle.scaled_mm(xq, codes, s_act, s_w)
        out_exact, _ = exact.scaled_mm(xq_exact.tolist(), codes.tolist(), s_act, s_w.tolist())
        assert np.array_equal(out, np.array(out_exact, np.uint16)), (it, out, out_exact)
        assert not np.isnan(t[xq]).any()


def test_gemm_exact_accumulation_closed_form():
    """Every E4M3 value is a multiple of 2^-9: the integer sum in units of 2^-18
    must equal the fp64 accumulator, and any K permutation gives the same bits."""
    g = np.random.Generator(np.random.PCG64(5))
    M, N, K = 3, 40, 17408
    xq = wl.FINITE_CODE_VALUES[g.integers(0, 254, (M, K))]
    wq = wl.FINITE_CODE_VALUES[g.integers(0, 254, (N, K))]
    t = oracle.e4m3_table()
    xi = np.rint(t[xq] * 512).astype(np.int64)
    wi = np.rint(t[wq] * 512).astype(np.int64)
    acc_int = xi @ wi.T                                  # units of 2^-18, exact in int64
    acc = oracle.exact_acc(xq, wq)
    assert np.array_equal(acc * 2.0 ** 18, acc_int.astype(np.float64))
    assert np.all(np.abs(acc_int) < 2 ** 50)
    perm = g.permutation(K)
    assert np.array_equal(oracle.exact_acc(xq[:, perm], wq[:, perm]), acc)


def test_blas_gemm_is_the_plain_gemm():
    """scaled_mm_blas (library fp64 matmul on decoded codes) against the plain
    loop of scaled_mm, bit for bit in the bf16 output and the fp64 v: on the
    tiny workload, on random codes at K = 17408 with rows of +-448 (the largest
    partial sums the bound allows for), on the hand-worked product, and under a
    consistent K permutation.  An fp32 matmul, a transposed operand or a dropped
    scale fails it."""
    x = wl.activation_bf16(1, 4, 256, outliers=False)
    s_act = oracle.act_scale(x)
    xq = oracle.quant_act(x, s_act)
    wq, sw = oracle.quant_weight(wl.weight_f32(1, 384, 256))
    a, va = oracle.scaled_mm(xq, wq, s_act, sw, want_v=True)
    b, vb = oracle.scaled_mm_blas(xq, wq, s_act, sw, want_v=True)
    assert np.array_equal(a, b) and np.array_equal(va.view(np.uint64), vb.view(np.uint64))
    g = np.random.Generator(np.random.PCG64(77))
    M, N, K = 5, 48, 17408
    xq = wl.FINITE_CODE_VALUES[g.integers(0, 254, (M, K))]
    wq = wl.FINITE_CODE_VALUES[g.integers(0, 254, (N, K))]
    xq[0], wq[0], wq[1] = 0x7E, 0x7E, 0xFE           # sums of +-448^2 K
    xq[1, ::2] = 0x01                                # the smallest subnormal against the largest values
    sw = (g.random(N) * 1e-3 + 1e-5).astype(np.float32)
    s_act = float(np.float32(0.0123))
    a, va = oracle.scaled_mm(xq, wq, s_act, sw, want_v=True)
    b, vb = oracle.scaled_mm_blas(xq, wq, s_act, sw, want_v=True)
    assert np.array_equal(a, b) and np.array_equal(va.view(np.uint64), vb.view(np.uint64))
    assert vb[0, 0] == 448.0 * 448.0 * K * np.float64(np.float32(s_act)) * np.float64(sw[0])
    perm = g.permutation(K)
    assert np.array_equal(oracle.scaled_mm_blas(xq[:, perm], wq[:, perm], s_act, sw), b)
    t = _golden("tiny_product.json")
    xq = np.array([[int(c, 16) for c in t["x_q"]]], np.uint8)
    wq = np.array([[int(c, 16) for c in r] for r in t["W_q"]], np.uint8)
    out = oracle.scaled_mm_blas(xq, wq, float.fromhex(t["s_act"]),
                                np.array([float.fromhex(v) for v in t["s_w"]], np.float32))
    assert [hex(v) for v in out[0]] == t["out_bf16"]
    # the bound behind the exactness: K * 448^2 in units of 2^-18 below 2^53
    assert oracle.EXACT_K_MAX * 448 * 448 * 2 ** 18 < 2 ** 53 <= (oracle.EXACT_K_MAX + 1) * 448 * 448 * 2 ** 18


def test_invariants_scale_zero_identity_sign_merge():
    g = np.random.Generator(np.random.PCG64(11))
    M, N, K = 5, 48, 512
    x = wl.to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    s_act = oracle.act_scale(x)
    xq = oracle.quant_act(x, s_act)
    w = g.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    wq, sw = oracle.quant_weight(w)
    out, v = oracle.scaled_mm(xq, wq, s_act, sw, want_v=True)
    # linearity in s_w: a power of two scales the result bit-exactly
    for j in (-3, 1, 4):
        out2 = oracle.scaled_mm(xq, wq, s_act, (sw * np.float32(2.0 ** j)).astype(np.float32))
        want = wl.to_bf16_bits(oracle.bf16_bits_to_f32(out) * np.float32(2.0 ** j))
        assert np.array_equal(out2, want)
    # general scale: within one bf16 rounding of the scaled exact value
    c = np.float32(1.37)
    out3 = oracle.scaled_mm(xq, wq, s_act, (sw * c).astype(np.float32))
    vc = v * np.float64(c)
    err = np.abs(oracle.bf16_bits_to_f32(out3).astype(np.float64) - vc)
    assert np.all(err <= 2.0 ** -8 * np.abs(vc) + 1e-30)
    # zero row -> +0 row
    xz = xq.copy()
    xz[2] = 0
    oz = oracle.scaled_mm(xz, wq, s_act, sw)
    assert np.all(oz[2] == 0)
    # identity weight with power-of-two s_act: out = bf16(dec(x_q) * s_act) exactly
    Ki = 256
    ident = np.where(np.eye(Ki, dtype=bool), 0x38, 0).astype(np.uint8)
    xi = xq[:, :Ki]
    oi = oracle.scaled_mm(xi, ident, 0.25, np.ones(Ki, np.float32))
    dec = oracle.e4m3_table()[xi] * 0.25
    assert np.array_equal(oracle.bf16_bits_to_f32(oi).astype(np.float64), dec)
    # flipping every W sign bit negates the output exactly
    on = oracle.scaled_mm(xq, wq ^ np.uint8(0x80), s_act, sw)
    nz = (out & 0x7FFF) != 0
    assert np.array_equal(on[nz], out[nz] ^ np.uint16(0x8000))
    # merged == split: concatenated shards equal separate products
    wa, wb = wq[:20], wq[20:]
    oa = oracle.scaled_mm(xq, wa, s_act, sw[:20])
    ob = oracle.scaled_mm(xq, wb, s_act, sw[20:])
    assert np.array_equal(np.concatenate([oa, ob], axis=1), out)


# --------------------------------------------------------------- RMSNorm ---

def test_rmsnorm_closed_forms():
    K = 5120
    eps = 1e-6
    ones = np.ones(K, np.float32)
    gamma1 = wl.to_bf16_bits(ones)
    # rows of +-1: r = fl32(1/sqrt(1 + eps)) rounds y to exactly bf16 1.0
    row = np.where(np.arange(K) % 3 == 0, -1.0, 1.0).astype(np.float32)
    x = wl.to_bf16_bits(row[None, :])
    y = oracle.rmsnorm(x, gamma1, eps)
    assert np.array_equal(oracle.bf16_bits_to_f32(y)[0], row)
    q = oracle.quant_rmsnorm(x, gamma1, eps, np.float32(1.0 / 448.0))
    assert np.array_equal(q[0], np.where(row < 0, 0xFE, 0x7E).astype(np.uint8))
    # constant row c: y = gamma * c / sqrt(c^2 + eps), then rounded
    for c in (0.5, -3.0, 1e-3):
        x = wl.to_bf16_bits(np.full((1, K), c, np.float32))
        cb = float(oracle.bf16_bits_to_f32(x)[0, 0])
        r = np.float32(1.0 / np.sqrt(cb * cb + np.float64(np.float32(eps))))
        want = wl.to_bf16_bits(np.float32(np.float32(cb) * r) * np.float32(1.0))
        assert np.all(oracle.rmsnorm(x, gamma1, eps)[0] == want)
    # a single nonzero entry a at position j: y_j = gamma_j * a / sqrt(a^2/K + eps)
    a, j = np.float32(2.0), 17
    row = np.zeros(K, np.float32)
    row[j] = a
    x = wl.to_bf16_bits(row[None, :])
    g = wl.gamma_bf16(3, K)
    y = oracle.bf16_bits_to_f32(oracle.rmsnorm(x, g, eps))[0]
    r = np.float32(1.0 / np.sqrt(4.0 / K + np.float64(np.float32(eps))))
    want = wl.to_bf16_bits(np.float32(a * r) * oracle.bf16_bits_to_f32(g)[j])
    assert y[j] == oracle.bf16_bits_to_f32(want) and np.all(np.delete(y, j) == 0)


def test_rmsnorm_against_numpy_formula():
    """Independent restatement with numpy (pairwise fp64 sum, fp32 products,
    torch's bf16 cast) on the decode-MLP input distribution."""
    K = 5120
    x = wl.activation_bf16(3, 32, K, outliers=True)
    g = wl.gamma_bf16(3, K)
    xf = oracle.bf16_bits_to_f32(x)
    ss = np.sum(xf.astype(np.float64) ** 2, axis=1)
    r = (1.0 / np.sqrt(ss / K + np.float64(np.float32(1e-6)))).astype(np.float32)
    y = (xf * r[:, None]).astype(np.float32) * oracle.bf16_bits_to_f32(g)[None, :]
    want = wl.to_bf16_bits(y.astype(np.float32))
    assert np.array_equal(oracle.rmsnorm(x, g, 1e-6), want)


@pytest.mark.parametrize("wid,M", [(3, 32), (5, 64)])
def test_fused_quant_is_byte_exact_against_unfused(wid, M):
    """The fused RMSNorm->quant must equal quant(rmsnorm(x)) byte for byte."""
    K = 5120
    x = wl.activation_bf16(wid, M, K, outliers=(wid == 3))
    g = wl.gamma_bf16(wid, K)
    s = oracle.act_scale(x, g, 1e-6)
    fused = oracle.quant_rmsnorm(x, g, 1e-6, s)
    unfused = oracle.quant_act(oracle.rmsnorm(x, g, 1e-6), s)
    assert np.array_equal(fused, unfused)
    # the calibrated scale is amax over the tensor actually quantized
    y = oracle.bf16_bits_to_f32(oracle.rmsnorm(x, g, 1e-6))
    assert s == np.float32(np.abs(y).max() / np.float32(448.0))
    assert np.abs(oracle.e4m3_table()[fused]).max() == 448.0


# ------------------------------------------------------- scales and weights --

def test_act_scale_and_weight_quant_definitions():
    x = wl.activation_bf16(2, 8, 5120, outliers=True)
    xf = oracle.bf16_bits_to_f32(x)
    assert oracle.act_scale(x) == np.float32(np.abs(xf).max()) / np.float32(448.0)
    assert oracle.act_scale(np.zeros((2, 16), np.uint16)) == 1.0
    w = wl.weight_f32(1, 384, 256)
    w[7] = 0.0
    wq, sw = oracle.quant_weight(w)
    amax = np.abs(w).max(axis=1)
    want_sw = np.where(amax == 0, np.float32(1), amax / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(sw, want_sw)
    t = (w / sw[:, None]).astype(np.float32)
    assert np.array_equal(wq, _brute_force_encode(t))
    assert (wq[np.arange(384) != 7] & 0x7F).max(axis=1).min() == 0x7E  # every row reaches +-448


def test_double_rounding_trap():
    """The bf16 output is ONE rounding of the exact value (never through fp32)."""
    g = _golden("tiny_product.json")["double_rounding_trap"]
    xq = np.array([[int(c, 16) for c in g["x_q"]]], np.uint8)
    wq = np.array([[int(c, 16) for c in r] for r in g["W_q"]], np.uint8)
    s_w = np.array([float.fromhex(s) for s in g["s_w"]], np.float32)
    out = oracle.scaled_mm(xq, wq, float.fromhex(g["s_act"]), s_w)
    assert hex(out[0, 0]) == g["out_bf16"]


# ------------------------------------------------------ SiLU*mul -> quant --

def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_bits_to_f32(b)
    return b[np.isfinite(f)]


def test_silu_against_scipy_expit_all_bf16():
    """silu(g) for every finite bf16 g against a different routine: g * expit(g)
    (scipy's logistic function) in fp64, rounded to fp32, then to bf16 (up = 1)."""
    from scipy.special import expit
    g = _all_finite_bf16().reshape(1, -1)
    one = np.full_like(g, 0x3F80)                     # bf16 1.0
    got = oracle.silu_mul(g, one)
    gd = oracle.bf16_bits_to_f32(g).astype(np.float64)
    with np.errstate(over="ignore"):
        want = wl.to_bf16_bits((gd * expit(gd)).astype(np.float32))
    assert np.array_equal(got, want)


def test_silu_closed_forms_and_identities():
    def silu(vals):
        g = wl.to_bf16_bits(np.asarray(vals, np.float32)).reshape(1, -1)
        return oracle.bf16_bits_to_f32(oracle.silu_mul(g, np.full_like(g, 0x3F80)))[0]
    z = silu([0.0, -0.0])
    assert z[0] == 0 and not np.signbit(z[0]) and z[1] == 0 and np.signbit(z[1])
    big = np.array([32.0, 100.0, 3.0e38], np.float32)          # exp(-g) below half an ulp: silu(g) = g
    assert np.array_equal(silu(big), oracle.bf16_bits_to_f32(wl.to_bf16_bits(big)))
    assert np.all(silu([-100.0, -1000.0, -3.0e38]) == 0)       # g / (1 + huge) -> 0 (sign kept)
    assert silu([1.0])[0] == np.float32(oracle.bf16_bits_to_f32(wl.to_bf16_bits(np.float32(1.0 / (1.0 + np.exp(-1.0))))))
    # silu(g) - silu(-g) = g (sigmoid(g) + sigmoid(-g) = 1), checked in fp32 before the bf16 rounding
    gd = np.random.Generator(np.random.PCG64(11)).normal(0, 3, 4096)
    g = oracle.bf16_bits_to_f32(wl.to_bf16_bits(gd.astype(np.float32))).astype(np.float64)
    sp, sm = g / (1 + np.exp(-g)), (-g) / (1 + np.exp(g))
    assert np.allclose(sp - sm, g, rtol=0, atol=4e-16 * np.maximum(1, np.abs(g)))
    # the minimum of silu is -0.27846454... (at g = -1.27846...): over all bf16 g
    # the smallest bf16 output is that value rounded to bf16
    allg = _all_finite_bf16().reshape(1, -1)
    vals = oracle.bf16_bits_to_f32(oracle.silu_mul(allg, np.full_like(allg, 0x3F80)))
    assert np.nanmin(vals) == oracle.bf16_bits_to_f32(wl.to_bf16_bits(np.float32(-0.2784645428)))


def test_silu_mul_product_and_power_of_two_scaling():
    """h = fl32(silu(g) * u): u = 2^j scales h exactly; u = -u flips its sign."""
    g = wl.activation_bf16(3, 4, 512, outliers=True, tensor=wl.T_LAYER0 + 90)
    u = wl.activation_bf16(3, 4, 512, outliers=False, tensor=wl.T_LAYER0 + 91)
    h = oracle.bf16_bits_to_f32(oracle.silu_mul(g, u))
    u4 = wl.to_bf16_bits(oracle.bf16_bits_to_f32(u) * np.float32(4.0))
    assert np.array_equal(oracle.bf16_bits_to_f32(oracle.silu_mul(g, u4)), h * np.float32(4.0))
    assert np.array_equal(oracle.silu_mul(g, u ^ np.uint16(0x8000)), oracle.silu_mul(g, u) ^ np.uint16(0x8000))
    # against a numpy restatement: silu via expit (a different routine), product in fp32
    from scipy.special import expit
    gd = oracle.bf16_bits_to_f32(g).astype(np.float64)
    s32 = (gd * expit(gd)).astype(np.float32)
    assert np.array_equal(oracle.silu_mul(g, u), wl.to_bf16_bits(s32 * oracle.bf16_bits_to_f32(u)))


@pytest.mark.parametrize("M", [1, 32])
def test_silu_mul_quant_is_byte_exact_against_unfused(M):
    """Fused SiLU*mul -> quant equals quant(silu_mul(gate, up)) byte for byte,
    and the calibrated scale puts the largest |h| at +-448."""
    I = 17408
    g = wl.activation_bf16(3, M, I, outliers=True, tensor=wl.T_LAYER0 + 92)
    u = wl.activation_bf16(3, M, I, outliers=True, tensor=wl.T_LAYER0 + 93)
    h = oracle.silu_mul(g, u)
    s = oracle.act_scale(h)
    fused = oracle.silu_mul_quant(g, u, s)
    assert np.array_equal(fused, oracle.quant_act(h, s))
    assert np.abs(oracle.e4m3_table()[fused]).max() == 448.0


# ----------------------------------------------------- per-token scales ----

def test_per_token_brute_force_against_exact_rationals():
    """Per-row dynamic quant (each row: fl32(amax/448), then the static quant)
    and the GEMM with per-row scales, in Fractions vs the oracle; rows of very
    different magnitude, a zero row and non-finite entries included."""
    g = np.random.Generator(np.random.PCG64(314))
    for it in range(150):
        mags = np.array([g.choice([1e-3, 1.0, 50.0]) for _ in range(3)], np.float32)[:, None]
        x = wl.to_bf16_bits(g.standard_normal((3, 8)).astype(np.float32) * mags)
        if it % 7 == 0:
            x[1] = 0x8000 if it % 2 else 0                 # a zero row: scale 1
        if it % 11 == 0:
            x[2, 3] = 0x7F80                               # inf is skipped by the amax, saturates
        xq, s = oracle.quant_per_token(x)
        xq_e, s_e = exact.quant_per_token(x.tolist())
        assert [float(v) for v in s] == s_e, (it, s, s_e)
        assert np.array_equal(xq, np.array(xq_e, np.uint8)), it
        codes = wl.FINITE_CODE_VALUES[g.integers(0, 254, (4, 8))]
        s_w = (g.random(4) * 0.01 + 1e-4).astype(np.float32)
        out = oracle.scaled_mm_rows(xq, codes, s, s_w)
        assert np.array_equal(out, np.array(exact.scaled_mm_rows(xq.tolist(), codes.tolist(), s.tolist(),
                                                                 s_w.tolist()), np.uint16)), it


def test_per_token_rows_are_independent_and_scale_covariant():
    """Multiplying one row by 2^k (exact in bf16) multiplies its scale by 2^k
    and leaves every code of every row unchanged; the other rows' scales do not
    move; a constant row quantizes to +-448 everywhere."""
    x = wl.activation_bf16(2, 6, 5120, outliers=True)
    q0, s0 = oracle.quant_per_token(x)
    for k in (-3, 5):
        y = x.copy()
        f = (y[2].astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** k)
        y[2] = (f.view(np.uint32) >> 16).astype(np.uint16)
        q1, s1 = oracle.quant_per_token(y)
        assert np.array_equal(q0, q1)
        assert s1[2] == np.float32(s0[2] * 2.0 ** k)
        assert np.array_equal(np.delete(s1, 2), np.delete(s0, 2))
    c = np.full((1, 64), 0xC040, np.uint16)               # -3.0
    qc, sc = oracle.quant_per_token(c)
    assert sc[0] == np.float32(3.0) / np.float32(448.0) and np.all(qc == 0xFE)


def test_per_token_rmsnorm_row_is_the_static_quant_of_that_row():
    """With gamma, row m's codes and scale equal the static fused RMSNorm quant
    of that row alone, calibrated on that row alone."""
    x = wl.activation_bf16(3, 5, 5120, outliers=True)
    gm = wl.gamma_bf16(3, 5120)
    q, s = oracle.quant_per_token(x, gm, wl.EPS)
    for m in range(5):
        sm = oracle.act_scale(x[m:m + 1], gm, wl.EPS)
        assert s[m] == np.float32(sm)
        assert np.array_equal(q[m:m + 1], oracle.quant_rmsnorm(x[m:m + 1], gm, wl.EPS, sm))


def test_rows_gemm_with_equal_scales_is_the_per_tensor_gemm():
    g = np.random.Generator(np.random.PCG64(8))
    xq = wl.random_codes(2, 7, 640)
    wq = wl.random_codes(2, 48, 640, tensor=wl.T_W)
    sw = (g.random(48) * 1e-3 + 1e-5).astype(np.float32)
    a, va = oracle.scaled_mm(xq, wq, 0.0123, sw, want_v=True)
    b, vb = oracle.scaled_mm_rows(xq, wq, np.full(7, 0.0123, np.float32), sw, want_v=True)
    assert np.array_equal(a, b) and np.array_equal(va, vb)


# ------------------------------------- merged shards, per-tensor scales ----
# A merged projection whose shards carry one per-tensor weight scale each can
# either keep every shard exact (expand the scales to per-channel form, or
# decline the merge) or requantize every shard to the largest scale (lossy);
# vllm.cpp #417, ranked follow-ons, contrasts the two.

def _shard_rows_scales(g, rows):
    """Per-tensor scales for shards: arbitrary fp32 values, one repeated (an
    exact tie for the max), and a power-of-two ratio."""
    sc = (g.random(len(rows)) * 1e-3 + 1e-5).astype(np.float32)
    if len(rows) >= 3:
        sc[2] = sc[0]
    if len(rows) >= 4:
        sc[3] = np.float32(sc[1] * np.float32(0.25))
    return sc


def test_requant_brute_force_against_exact_rationals():
    g = np.random.Generator(np.random.PCG64(2718))
    for it in range(60):
        rows = [int(r) for r in g.integers(1, 4, size=int(g.integers(1, 5)))]
        K = 6
        codes = [wl.FINITE_CODE_VALUES[g.integers(0, 254, (r, K))] for r in rows]
        if it % 5 == 0:
            codes[0][0, :2] = (0x7F, 0xFF)                       # NaN codes are kept
        sc = _shard_rows_scales(g, rows)
        got, s_max = oracle.requant_max_scale(np.concatenate(codes), rows, sc)
        want, s_max_e = exact.requant_max_scale([c.tolist() for c in codes], sc.tolist())
        assert float(s_max) == s_max_e == float(sc.max())
        assert np.array_equal(got, np.concatenate([np.array(w, np.uint8) for w in want])), it


def test_requant_matches_ieee_steps_and_nearest_search():
    """Large random case: numpy's IEEE fp32 multiply and divide, then the
    exhaustive nearest search, give the oracle's bytes."""
    g = np.random.Generator(np.random.PCG64(99))
    rows = [96, 16, 16, 48]
    K = 256
    wq = wl.random_codes(3, sum(rows), K)
    sc = _shard_rows_scales(g, rows)
    got, s_max = oracle.requant_max_scale(wq, rows, sc)
    per_row = np.repeat(sc, rows).astype(np.float32)
    w = (oracle.e4m3_table()[wq].astype(np.float32) * per_row[:, None]).astype(np.float32)
    t = (w / np.float32(sc.max())).astype(np.float32)
    assert np.array_equal(got, _brute_force_encode(t))


def test_requant_equal_scales_is_the_identity():
    """Every finite code survives dequantize-then-requantize at its own scale
    (the fp32 steps err by 2^-23 relative, far inside half an E4M3 step); the
    shard that holds the largest scale is unchanged inside any merge."""
    codes = wl.FINITE_CODE_VALUES.reshape(2, 127)
    for s in (1.0, 0.02 / 448, 3.7e-5, 0.1234567, 7.5):
        out, s_max = oracle.requant_max_scale(codes, [1, 1], [s, s])
        assert np.array_equal(out, codes) and s_max == np.float32(s)
    g = np.random.Generator(np.random.PCG64(5))
    wq = wl.random_codes(3, 64, 128)
    sc = np.array([3e-4, 9e-4, 1e-4], np.float32)
    out, _ = oracle.requant_max_scale(wq, [16, 32, 16], sc)
    assert np.array_equal(out[16:48], wq[16:48])
    assert not np.array_equal(out[:16], wq[:16])


def test_requant_power_of_two_ratio_closed_form():
    """Scales 2^-7 and 2^(-7-j): the requantized value is dec(c) / 2^j exactly
    before the E4M3 rounding.  Written on the bit fields: a normal result lowers
    the exponent field by j; a subnormal result is round-half-even of
    (value * 2^9) / 2^j on the integer grid m * 2^-9 (grid value 8 = code 0x08)."""
    codes = wl.FINITE_CODE_VALUES
    for j in (1, 2, 3, 5):
        out, s_max = oracle.requant_max_scale(np.stack([codes, codes]), [1, 1], [2.0 ** -7, 2.0 ** (-7 - j)])
        assert s_max == np.float32(2.0 ** -7)
        assert np.array_equal(out[0], codes)
        for c, got in zip(codes.tolist(), out[1].tolist()):
            sgn, e, m = c & 0x80, (c >> 3) & 15, c & 7
            if e > j:
                want = sgn | ((c & 0x7F) - (j << 3))
            else:
                v9 = m if e == 0 else (8 + m) << (e - 1)           # value * 2^9, an integer
                q, r = divmod(v9, 1 << j)
                half = 1 << (j - 1)
                q += 1 if (r > half or (r == half and q % 2 == 1)) else 0
                want = sgn | q
            assert got == want, (j, hex(c), hex(got), hex(want))


def test_requant_sign_symmetry_and_monotone_in_the_ratio():
    wq = wl.random_codes(3, 40, 96)
    rows, sc = [8, 32], np.array([1e-3, 4.3e-4], np.float32)
    a, _ = oracle.requant_max_scale(wq, rows, sc)
    b, _ = oracle.requant_max_scale(wq ^ np.uint8(0x80), rows, sc)
    assert np.array_equal(b, a ^ np.uint8(0x80))
    # A smaller shard scale never gives a larger magnitude.
    c, _ = oracle.requant_max_scale(wq, rows, np.array([1e-3, 2.1e-4], np.float32))
    tab = oracle.e4m3_table()
    assert np.all(np.abs(tab[c[8:]]) <= np.abs(tab[a[8:]]))


def test_weight_per_tensor_definition():
    w = wl.weight_f32(1, 96, 256)
    w[40, 17] = np.float32(0.5)                                  # the tensor max, not in row 0
    wq, s = oracle.quant_weight_per_tensor(w)
    assert s == np.float32(0.5) / np.float32(448.0)
    assert np.array_equal(wq, _brute_force_encode((w / s).astype(np.float32)))
    assert oracle.quant_weight_per_tensor(np.zeros((4, 16), np.float32))[1] == 1.0
    # Rows with equal amax: per-tensor == per-channel.
    v = np.abs(wl.weight_f32(1, 8, 64))
    v[:, 0] = np.float32(0.25)
    q1, s1 = oracle.quant_weight_per_tensor(v)
    q2, s2 = oracle.quant_weight(v)
    assert np.array_equal(q1, q2) and np.all(s2 == s1)


def test_max_scale_layer_with_equal_scales_is_the_exact_merge():
    """Equal input and weight scales: the requantizing merge loses nothing, so
    its output is the exact merged (and split) layer bit for bit."""
    x = wl.activation_bf16(2, 4, 512, outliers=True)
    shards = [wl.random_codes(3, n, 512, m=i) for i, n in enumerate((64, 16, 16))]
    s_in = oracle.act_scale(x)
    xq, wq2, s_act, s_max, out = oracle.merged_max_scale_layer(x, shards, [2e-4] * 3, [s_in] * 3)
    assert s_act == np.float32(s_in) and s_max == np.float32(2e-4)
    want = np.concatenate([oracle.scaled_mm(oracle.quant_act(x, s_in), w, s_in, np.full(w.shape[0], 2e-4,
                                                                                          np.float32))
                           for w in shards], axis=1)
    assert np.array_equal(out, want)
