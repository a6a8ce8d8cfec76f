"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Bar: E4M3 activation and weight bytes and the static scales bit-exact; bf16
outputs within max(2 bf16 ulp, 1e-3 * ||row||_2) per element of the oracle
(tests/helpers.py).  Inputs are the seeded synthetic workloads of workloads/.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import (assert_within_tolerance, assert_within_tolerance_rows, bf16_dev, f32_dev, host_u16,
                     host_u8, u8_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import fp8_w8a8_scaled_amd as m
    return m


def _sync():
    import torch
    torch.cuda.synchronize()


# ------------------------------------------------------------ quantization --

@pytest.mark.parametrize("s_act", [1.0, 0.5, 3.0, 1.0 / 7.0, 0.2])
def test_quant_all_bf16_patterns_bit_exact(fp8, s_act):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(1, -1)
    got = host_u8(fp8.quant(bf16_dev(bits), s_act))
    want = oracle.quant_act(bits, np.float32(s_act))
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]


@pytest.mark.parametrize("s_act", [1.0, 3.0, 1.0 / 7.0, 2.0 ** -99, 2.0 ** 99, 2.0 ** -120])
def test_plain_quant_table_path_all_bf16_patterns(fp8, s_act):
    """Every bf16 pattern in 24 rows (1.5 M elements, past the table path's
    2^20), the rows rotated so each pattern meets several column offsets and
    the workgroups' shares end mid-row; 2^-120 is outside the table's range
    (per-element path)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = np.stack([np.roll(bits, 977 * i) for i in range(24)])
    got = host_u8(fp8.quant(bf16_dev(x), s_act))
    want = oracle.quant_act(x, np.float32(s_act))
    assert np.array_equal(got, want), np.argwhere(got != want)[:10]


@pytest.mark.parametrize("wid,M,K", [(1, 4, 256), (2, 1, 5120), (2, 2, 5120), (2, 4, 5120), (2, 8, 5120),
                                     (3, 1, 17408), (3, 8, 17408), (3, 32, 17408), (5, 6576, 17408)])
def test_plain_quant_and_scale_bit_exact(fp8, wid, M, K):
    x = wl.activation_bf16(wid, M, K, outliers=wid in (2, 3, 4), tensor=wl.T_DOWN_X if K == 17408 else wl.T_X)
    xd = bf16_dev(x)
    s_gpu = fp8.act_scale(xd)
    s_ref = oracle.act_scale(x)
    assert np.float32(s_gpu.item()).view(np.uint32) == np.float32(s_ref).view(np.uint32)
    got = host_u8(fp8.quant(xd, s_ref))
    assert np.array_equal(got, oracle.quant_act(x, s_ref))


@pytest.mark.parametrize("wid,M", [(3, 1), (3, 4), (3, 8), (3, 16), (3, 32), (5, 6576)])
def test_fused_rmsnorm_quant_bit_exact(fp8, wid, M):
    K = 5120
    x = wl.activation_bf16(wid, M, K, outliers=(wid == 3))
    g = wl.gamma_bf16(wid, K)
    xd, gd = bf16_dev(x), bf16_dev(g)
    s_gpu = fp8.act_scale(xd, gd, wl.EPS)
    s_ref = oracle.act_scale(x, g, wl.EPS)
    assert np.float32(s_gpu.item()).view(np.uint32) == np.float32(s_ref).view(np.uint32)
    got = host_u8(fp8.quant_rmsnorm(xd, gd, s_ref, wl.EPS))
    want = oracle.quant_rmsnorm(x, g, wl.EPS, s_ref)
    assert np.array_equal(got, want), f"{int((got != want).sum())} bytes differ"


def _strided(x, ld):
    big = np.zeros((x.shape[0], ld), np.uint16)
    big[:, :x.shape[1]] = x
    xd = bf16_dev(big)[:, :x.shape[1]]
    assert xd.stride(0) == ld
    return xd


def test_quant_strided_input_and_special_rows(fp8):
    M, K, ld = 5, 5120, 5136
    s = np.float32(0.0137)
    x = wl.activation_bf16(3, M, K, outliers=True)
    x[1] = 0                                   # all-zero row: r = 1/sqrt(eps)
    x[2] = 0x8000                              # -0 row
    x[3, :5] = np.array([0x0001, 0x8001, 0x7F7F, 0xFF7F, 0x0080], np.uint16)   # subnormal, +-max, min normal
    g = wl.gamma_bf16(3, K)
    got = host_u8(fp8.quant_rmsnorm(_strided(x, ld), bf16_dev(g), float(s), wl.EPS))
    assert np.array_equal(got, oracle.quant_rmsnorm(x, g, wl.EPS, s))
    # plain quant also takes non-finite inputs: inf saturates, NaN keeps its sign
    x[4, :4] = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1], np.uint16)
    got = host_u8(fp8.quant(_strided(x, ld), float(s)))
    assert np.array_equal(got, oracle.quant_act(x, s))
    assert list(got[4, :4]) == [0x7E, 0xFE, 0x7F, 0xFF]


@pytest.mark.parametrize("M", [37, 130])
@pytest.mark.parametrize("K", [256, 2064, 5120, 8192, 16384])
@pytest.mark.parametrize("s_act", [1.0, 0.37, 2.0 ** -20, 2.0 ** 20, 2.0 ** -99, 2.0 ** 99, 2.0 ** -110])
def test_rmsnorm_quant_wide_gamma_and_special_rows(fp8, M, K, s_act):
    """gamma spans 2^-40 .. 2^41 with random signs, so y_b crosses both edges of
    the band of magnitudes whose code needs the division, under every scale.
    K <= 8192 with 2^-100 <= s_act <= 2^100 takes the row-group kernel (exact
    quotient by multiply and fused multiply-add, hardware conversion), the
    rest the per-element path; all must give the oracle's bytes (130 rows: an
    odd row count for the row groups, rows strided).  Special rows: inf, NaN,
    all zeros with eps = 0 (r = inf), a lone subnormal; then an infinite
    gamma."""
    rng = np.random.default_rng(4200 + K)
    x = wl.to_bf16_bits((rng.standard_normal((M, K)) * np.where(rng.random((M, K)) < 0.01, 20.0, 1.0))
                        .astype(np.float32))
    g = wl.to_bf16_bits((rng.choice([-1.0, 1.0], K) * (1.0 + rng.random(K))
                         * np.exp2(rng.integers(-40, 41, K))).astype(np.float32))
    dev_x = (lambda a: _strided(a, K + 16)) if M > 64 else bf16_dev
    got = host_u8(fp8.quant_rmsnorm(dev_x(x), bf16_dev(g), float(s_act), wl.EPS))
    assert np.array_equal(got, oracle.quant_rmsnorm(x, g, wl.EPS, s_act))

    x[3, 5], x[4, 9], x[6, 0] = 0x7F80, 0x7FC0, 0x0001      # inf, NaN, subnormal in a zero row
    x[5], x[6, 1:] = 0, 0
    got = host_u8(fp8.quant_rmsnorm(dev_x(x), bf16_dev(g), float(s_act), 0.0))
    _assert_codes_equal(got, oracle.quant_rmsnorm(x, g, 0.0, s_act), "special rows")
    g[7] = 0xFF80                                            # gamma = -inf: every row per element
    got = host_u8(fp8.quant_rmsnorm(dev_x(x), bf16_dev(g), float(s_act), wl.EPS))
    _assert_codes_equal(got, oracle.quant_rmsnorm(x, g, wl.EPS, s_act), "infinite gamma")


@pytest.mark.parametrize("N,K", [(384, 256), (10240, 5120), (48, 17408)])
def test_weight_quant_bit_exact(fp8, N, K):
    w = wl.weight_f32(1 if K == 256 else 2, N, K)
    w[3] = 0.0                                  # zero row -> s_w = 1, codes 0
    w[5, 7] = np.float32(3.0e38)                # a huge element sets that row's scale
    wq, sw = fp8.quant_weight(f32_dev(w))
    owq, osw = oracle.quant_weight(w)
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), osw.view(np.uint32))
    assert np.array_equal(host_u8(wq), owq)


# ------------------------------------------------------ SiLU*mul -> E4M3 --

def _assert_codes_equal(got, want, what=""):
    """E4M3 codes bit-exact, except that the sign bit of a NaN code is free: the
    sign of a NaN that the arithmetic creates (g = -inf, 0 * inf) or passes on is
    not fixed by IEEE 754, so only the NaN positions must agree."""
    nan_w = (want & 0x7F) == 0x7F
    assert np.array_equal(nan_w, (got & 0x7F) == 0x7F), f"{what}: NaN positions differ"
    diff = (got != want) & ~nan_w
    assert not diff.any(), f"{what}: {int(diff.sum())} codes differ, first at {np.argwhere(diff)[:5].tolist()}"


def _silu_scale_bit_exact(fp8, gate_d, up_d, gate, up):
    s_gpu = fp8.act_scale_silu_mul(gate_d, up_d)
    s_ref = oracle.act_scale(oracle.silu_mul(gate, up))
    assert np.float32(s_gpu.item()).view(np.uint32) == np.float32(s_ref).view(np.uint32)
    return s_ref


def _silu_table_min_elems():
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fp8mm.h")).read()
    return int(eval(re.search(r"#define FP8MM_SILU_TABLE_MIN_ELEMS \((.*)\)", hdr).group(1).replace("LL", "")))


@pytest.mark.parametrize("s_act", [1.0, 0.37, 1.0 / 448.0])
@pytest.mark.parametrize("rows", [4, 64])
def test_silu_mul_quant_all_bf16_patterns(fp8, s_act, rows):
    """Every bf16 gate pattern (inf, NaN, subnormals, the huge negatives where
    silu underflows to -0) against unit, random and every up pattern, and every
    up pattern against random gates; 4 rows take the per-element fp64 silu, 64
    rows (2^22 elements) the table path."""
    every = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rnd = wl.activation_bf16(1, 2, 65536, outliers=True, tensor=wl.T_GATE_UP)
    gate = np.tile(np.stack([every, every, rnd[0], every]), (rows // 4, 1))
    up = np.tile(np.stack([np.full(65536, 0x3F80, np.uint16), rnd[1], every, every[::-1]]), (rows // 4, 1))
    assert (rows * 65536 >= _silu_table_min_elems()) == (rows == 64)
    got = host_u8(fp8.silu_mul_quant(bf16_dev(gate), bf16_dev(up), s_act))
    _assert_codes_equal(got, oracle.silu_mul_quant(gate, up, np.float32(s_act)), f"all patterns, {rows} rows")
    if rows == 4:
        _silu_scale_bit_exact(fp8, bf16_dev(gate), bf16_dev(up), gate, up)


@pytest.mark.parametrize("wid,M,I", [(1, 3, 48), (1, 7, 208), (3, 1, 17408), (3, 8, 17408), (3, 32, 17408),
                                     (5, 6576, 17408)])
def test_silu_mul_quant_gate_up_halves(fp8, wid, M, I):
    """The two halves of a merged gate_up output [M, 2I] as strided views
    (ldg = ldu = 2I); the static scale calibrated on the GPU bit-exact."""
    gu = wl.activation_bf16(wid, M, 2 * I, outliers=True, tensor=wl.T_GATE_UP)
    gud = bf16_dev(gu)
    gate_d, up_d = gud[:, :I], gud[:, I:]
    assert gate_d.stride(0) == 2 * I
    s = _silu_scale_bit_exact(fp8, gate_d, up_d, gu[:, :I], gu[:, I:])
    got = host_u8(fp8.silu_mul_quant(gate_d, up_d, s))
    _assert_codes_equal(got, oracle.silu_mul_quant(gu[:, :I], gu[:, I:], s), f"M={M} I={I}")


def test_silu_mul_quant_zero_m_and_separate_buffers(fp8):
    import torch
    I = 17408
    g = wl.activation_bf16(2, 4, I, outliers=False, tensor=wl.T_GATE_UP)
    u = wl.activation_bf16(2, 4, I, outliers=False, tensor=wl.T_DOWN_X)
    out = torch.full((4, I), 0xA5, dtype=torch.uint8, device="cuda")
    fp8.silu_mul_quant(bf16_dev(g)[:0], bf16_dev(u)[:0], 0.5, out=out[:0])
    _sync()
    assert int((out != 0xA5).sum().item()) == 0
    fp8.silu_mul_quant(bf16_dev(g), bf16_dev(u), 0.5, out=out)
    _assert_codes_equal(host_u8(out), oracle.silu_mul_quant(g, u, np.float32(0.5)), "separate buffers")


# -------------------------------------------------------------------- GEMM --

def _prepare(wid, M, N, K, outliers, w_tensor=wl.T_W, x_tensor=wl.T_X):
    """Oracle-side inputs: quantized activation, weight, scales."""
    x = wl.activation_bf16(wid, M, K, outliers=outliers, tensor=x_tensor)
    s_act = oracle.act_scale(x)
    xq = oracle.quant_act(x, s_act)
    wq, sw = oracle.quant_weight(wl.weight_f32(wid, N, K, tensor=w_tensor))
    return xq, wq, s_act, sw


def _run_arm(fp8, xq, wq, s_act, sw, arm):
    out = fp8.scaled_mm(u8_dev(xq), u8_dev(wq), s_act, f32_dev(sw), arm=arm)
    return host_u16(out)


@pytest.mark.parametrize("arm", [0, 1])
def test_tiny_all_elements_both_arms(fp8, arm):
    xq, wq, s_act, sw = _prepare(1, 4, 384, 256, outliers=False)
    ref, v = oracle.scaled_mm(xq, wq, s_act, sw, want_v=True)
    assert_within_tolerance(_run_arm(fp8, xq, wq, s_act, sw, arm), ref, v, f"tiny arm {arm}")


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_decode_projection_all_elements(fp8, M):
    xq, wq, s_act, sw = _prepare(2, M, 10240, 5120, outliers=True)
    ref, v = oracle.scaled_mm(xq, wq, s_act, sw, want_v=True)
    got = host_u16(fp8.scaled_mm(u8_dev(xq), u8_dev(wq), s_act, f32_dev(sw)))
    assert fp8.select(M, 10240, 5120) == 0
    assert_within_tolerance(got, ref, v, f"decode proj M={M}")


@pytest.mark.parametrize("M", [1, 4, 8, 16, 32])
def test_decode_mlp_merged_gate_up_and_down(fp8, M):
    """Config of the decode MLP: fused RMSNorm quant -> merged gate_up (two
    17408-column shards, one launch) -> down projection (K = 17408)."""
    K, N = 5120, 34816
    x = wl.activation_bf16(3, M, K, outliers=True)
    g = wl.gamma_bf16(3, K)
    s1 = oracle.act_scale(x, g, wl.EPS)
    xq = oracle.quant_rmsnorm(x, g, wl.EPS, s1)
    xq_gpu = fp8.quant_rmsnorm(bf16_dev(x), bf16_dev(g), s1, wl.EPS)
    assert np.array_equal(host_u8(xq_gpu), xq)
    wq, sw = oracle.quant_weight(wl.weight_f32(3, N, K))
    outs = fp8.scaled_mm_merged(xq_gpu, u8_dev(wq), s1, f32_dev(sw), [17408, 17408])
    ref, v = oracle.scaled_mm(xq, wq, s1, sw, want_v=True)
    got = np.concatenate([host_u16(o) for o in outs], axis=1)
    assert_within_tolerance(got, ref, v, f"gate_up M={M}")
    # SiLU*mul -> E4M3 of the oracle's gate_up output (identical bytes uploaded),
    # then the down projection on those codes
    gate, up = ref[:, :17408], ref[:, 17408:]
    refd = bf16_dev(ref)
    s2 = _silu_scale_bit_exact(fp8, refd[:, :17408], refd[:, 17408:], gate, up)
    xq2 = oracle.silu_mul_quant(gate, up, s2)
    xq2_gpu = fp8.silu_mul_quant(refd[:, :17408], refd[:, 17408:], s2)
    _assert_codes_equal(host_u8(xq2_gpu), xq2, f"silu_mul M={M}")
    wq2, sw2 = oracle.quant_weight(wl.weight_f32(3, 5120, 17408, tensor=wl.T_DOWN_W))
    got2 = host_u16(fp8.scaled_mm(u8_dev(xq2), u8_dev(wq2), s2, f32_dev(sw2)))
    ref2, v2 = oracle.scaled_mm(xq2, wq2, s2, sw2, want_v=True)
    assert_within_tolerance(got2, ref2, v2, f"down M={M}")


def _nan_filled(shape, device="cuda"):
    """A bf16 output buffer full of NaN: an element the kernel never writes stays
    NaN and fails the finiteness check of the tolerance test."""
    import torch
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device=device)


@pytest.mark.timeout(900)
def test_prefill_all_elements(fp8):
    """Prefill chunk, M = 6576 (large-M arm: 26 x 136 tiles of gate_up, about
    14 rounds of the persistent grid, and 35 x 20 of down): every element of the
    merged gate_up [6576, 34816] and of down [6576, 5120] against the oracle,
    into NaN-filled outputs.  The GPU's own quantization of the same inputs
    (fused RMSNorm quant, plain quant, weight quant) is checked bit-exact on the
    side."""
    import torch
    M, K, N = 6576, 5120, 34816
    x = wl.activation_bf16(5, M, K, outliers=False)
    g = wl.gamma_bf16(5, K)
    s1 = oracle.act_scale(x, g, wl.EPS)
    xq = oracle.quant_rmsnorm(x, g, wl.EPS, s1)
    assert np.array_equal(host_u8(fp8.quant_rmsnorm(bf16_dev(x), bf16_dev(g), s1, wl.EPS)), xq)
    w = wl.weight_f32(5, N, K)
    wq, sw = oracle.quant_weight(w)
    wq_gpu, sw_gpu = fp8.quant_weight(f32_dev(w))
    del w
    assert np.array_equal(host_u8(wq_gpu), wq) and np.array_equal(sw_gpu.cpu().numpy().view(np.uint32),
                                                                  sw.view(np.uint32))
    del wq_gpu, sw_gpu
    assert fp8.select(M, N, K) == 1
    outs = [_nan_filled((M, N // 2)), _nan_filled((M, N // 2))]
    fp8.scaled_mm_merged(u8_dev(xq), u8_dev(wq), s1, f32_dev(sw), [N // 2, N // 2], outs=outs)
    _sync()
    got = np.concatenate([host_u16(o) for o in outs], axis=1)
    del outs
    torch.cuda.empty_cache()
    ref, v = oracle.scaled_mm_blas(xq, wq, s1, sw, want_v=True)
    assert_within_tolerance_rows(got, ref, v, "prefill gate_up")
    del got, ref, v, wq
    # down projection K = 17408
    xd = wl.activation_bf16(5, M, 17408, outliers=False, tensor=wl.T_DOWN_X)
    s2 = oracle.act_scale(xd)
    xq2 = oracle.quant_act(xd, s2)
    assert np.array_equal(host_u8(fp8.quant(bf16_dev(xd), s2)), xq2)
    wq2, sw2 = oracle.quant_weight(wl.weight_f32(5, 5120, 17408, tensor=wl.T_DOWN_W))
    out2 = _nan_filled((M, 5120))
    fp8.scaled_mm(u8_dev(xq2), u8_dev(wq2), s2, f32_dev(sw2), out=out2)
    _sync()
    ref2, v2 = oracle.scaled_mm_blas(xq2, wq2, s2, sw2, want_v=True)
    assert_within_tolerance_rows(host_u16(out2), ref2, v2, "prefill down")


# Shapes with more large-M tiles than the 256 CUs, so every workgroup of the
# persistent grid walks more than one tile, with ragged M and N edges:
#   4000 x 8176: 16 x 32 = 512 tiles of 256x256 (the launcher picks them: 2
#                rounds against 3 rounds of 672 tiles of 256x192);
#   2300 x 8176: 12 x 32 = 384 tiles of 256x192 (picked: 2 rounds of
#                three-quarter tiles against 2 full rounds of 288 tiles).
@pytest.mark.parametrize("M,N,K", [(4000, 8176, 1024), (2300, 8176, 1024), (6576, 5120, 2048)])
def test_large_m_multi_round_all_elements(fp8, M, N, K):
    g = np.random.Generator(np.random.PCG64(M + N + K))
    xq = wl.random_codes(9, M, K, m=M)
    wq = wl.random_codes(9, N, K, tensor=wl.T_W, m=N)
    s_act = float(np.float32(0.0071))
    sw = (g.random(N) * 1e-3 + 1e-4).astype(np.float32)
    assert fp8.select(M, N, K) == 1
    out = _nan_filled((M, N))
    fp8.scaled_mm(u8_dev(xq), u8_dev(wq), s_act, f32_dev(sw), out=out)
    _sync()
    ref, v = oracle.scaled_mm_blas(xq, wq, s_act, sw, want_v=True)
    assert_within_tolerance_rows(host_u16(out), ref, v, f"{M}x{N}x{K}")


def test_decode_step_sweep_64_layers(fp8):
    """Decode-step weight sweep at M = 8: 64 layers x {qkvz 12288x5120, out_proj
    5120x6144, merged gate_up 34816x5120, down 5120x17408} (23.15 GB of E4M3,
    far beyond on-chip caches), run as one step of 256 launches; layers 0, 31
    and 63 have their own seeded weights and inputs and are checked in full
    against the oracle, the other layers hold device copies of them."""
    import torch
    M = 8
    checked = (0, 31, 63)
    src = {}
    for l in checked:
        layer = []
        for pi, p in enumerate(wl.DECODE_STEP_LAYER):
            x = wl.activation_bf16(4, M, p.K, outliers=True, tensor=wl.T_LAYER0 + 4 * l + pi)
            s = oracle.act_scale(x)
            xq = oracle.quant_act(x, s)
            wq, sw = oracle.quant_weight(wl.weight_f32(4, p.N, p.K, tensor=wl.T_LAYER0 + 4 * l + pi))
            layer.append((xq, wq, s, sw))
        src[l] = layer
    dev = {l: [(u8_dev(xq), u8_dev(wq), s, f32_dev(sw)) for xq, wq, s, sw in src[l]] for l in checked}
    layers = []
    for l in range(wl.DECODE_STEP_LAYERS):
        if l in dev:
            layers.append(dev[l])
        else:
            base = dev[checked[l % 3]]
            layers.append([(xq, wq.clone(), s, sw) for xq, wq, s, sw in base])
    outs = {}
    for l, layer in enumerate(layers):
        res = []
        for (xq, wq, s, sw), p in zip(layer, wl.DECODE_STEP_LAYER):
            assert fp8.select(M, p.N, p.K) == 0
            if p.shards:
                res.append(torch.cat(fp8.scaled_mm_merged(xq, wq, s, sw, list(p.shards)), dim=1))
            else:
                res.append(fp8.scaled_mm(xq, wq, s, sw))
        if l in checked:
            outs[l] = res
    _sync()
    for l in checked:
        for (xq, wq, s, sw), got, p in zip(src[l], outs[l], wl.DECODE_STEP_LAYER):
            ref, v = oracle.scaled_mm(xq, wq, s, sw, want_v=True)
            assert_within_tolerance(host_u16(got), ref, v, f"layer {l} {p.name}")


@pytest.mark.parametrize("arm", [0, 1])
def test_every_e4m3_code_through_mfma(fp8, arm):
    """One-hot GEMM: x_q = e_k with code 0x38 (1.0), s_act = s_w = 1, so out[0, n]
    = dec(w_q[n, k]) exactly; w_q[:, k] runs over all 254 finite codes.  Pins the
    matrix cores' FP8 decoding (OCP E4M3FN, not FNUZ) and the operand layouts."""
    K, N = 256, 256
    codes = wl.FINITE_CODE_VALUES
    tab = oracle.e4m3_table()
    for k in (0, 77, 255):
        wq = wl.random_codes(1, N, K, m=k)
        wq[:254, k] = codes
        wq[254:, k] = 0
        xq = np.zeros((2, K), np.uint8)
        xq[0, k] = 0x38
        xq[1, k] = 0xB8                        # -1.0 in row 1
        out = _run_arm(fp8, xq, wq, 1.0, np.ones(N, np.float32), arm)
        want = tab[wq[:, k]]
        got0 = (out[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        got1 = (out[1].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.array_equal(got0, want) and np.array_equal(got1, -want)


@pytest.mark.parametrize("M", [1, 8, 16, 32, 64])
def test_both_arms_agree_with_oracle(fp8, M):
    xq, wq, s_act, sw = _prepare(2, M, 2048, 5120, outliers=True)
    ref, v = oracle.scaled_mm(xq, wq, s_act, sw, want_v=True)
    a0 = _run_arm(fp8, xq, wq, s_act, sw, 0)
    a1 = _run_arm(fp8, xq, wq, s_act, sw, 1)
    assert_within_tolerance(a0, ref, v, f"small-M arm M={M}")
    assert_within_tolerance(a1, ref, v, f"large-M arm M={M}")


@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (3, 48, 48), (17, 32, 272), (33, 64, 400), (65, 80, 144),
                                   (129, 144, 1040), (257, 272, 2064), (300, 1040, 17408),
                                   # x_q fragments staged through LDS: 8 rows (M = 5) and 16 rows (M = 11, 13),
                                   # with a balanced last round (4112 = 257 tiles) and 5 waves (K = 3072)
                                   (5, 10240, 5120), (13, 4112, 5120), (11, 6144, 3072),
                                   # K % 1024 == 0 but the ring kernel's LDS plan does not fit: the generic kernel
                                   (1, 33168, 32768), (12, 10240, 32768),
                                   # large-M tiles with one K stage (first and last at once) and with two
                                   (300, 528, 128), (520, 272, 256)])
def test_ragged_shapes_both_arms(fp8, M, N, K):
    g = np.random.Generator(np.random.PCG64(M * 1000 + N + K))
    xq = wl.random_codes(9, M, K, m=M)
    wq = wl.random_codes(9, N, K, tensor=wl.T_W, m=N)
    s_act = float(np.float32(0.0071))
    sw = (g.random(N) * 1e-3 + 1e-4).astype(np.float32)
    ref, v = oracle.scaled_mm(xq, wq, s_act, sw, want_v=True)
    arms = [1] if M > 64 else [0, 1]
    for arm in arms:
        assert_within_tolerance(_run_arm(fp8, xq, wq, s_act, sw, arm), ref, v, f"{M}x{N}x{K} arm {arm}")


@pytest.mark.parametrize("M,N,K,shards", [(32, 5120, 17408, [5120]), (17, 5120, 17408, [4112, 1008]),
                                          (29, 6400, 17408, [6400]), (24, 4112, 12288, [2048, 16, 2048]),
                                          (8, 5120, 17408, [5120]), (1, 5120, 17408, [2560, 2560]),
                                          (8, 6240, 17408, [6240]), (32, 6240, 17408, [3120, 3120])])
def test_two_tile_streamed_fragment_kernel(fp8, M, N, K, shards):
    """Long rows and at most two tiles per workgroup (a whole tile and a
    balanced share of the rest, or two whole tiles: 6400 rows): both tiles'
    chunks multiply the same streamed fragments.  Shares of at most 8 rows
    (5120, 4112 rows on 256 CUs) take 3 KB ring slots, larger ones (6240: up
    to 12 rows) 4 KB slots.  Within the oracle's tolerance on every element,
    and merged == one call per shard bit for bit (the single shards run other
    kernels: the same bits by construction)."""
    xq = wl.random_codes(8, M, K, m=M)
    wq = wl.random_codes(8, N, K, tensor=wl.T_W, m=N)
    sw = (np.random.Generator(np.random.PCG64(N + K)).random(N) * 1e-3 + 1e-5).astype(np.float32)
    s_act = 0.0093
    xd, wd, swd = u8_dev(xq), u8_dev(wq), f32_dev(sw)
    merged = [host_u16(o) for o in fp8.scaled_mm_merged(xd, wd, s_act, swd, shards)]
    ref, v = oracle.scaled_mm(xq, wq, s_act, sw, want_v=True)
    assert_within_tolerance(np.concatenate(merged, axis=1), ref, v, f"two-tile {M}x{N}x{K}")
    start = 0
    for n, mo in zip(shards, merged):
        split = host_u16(fp8.scaled_mm(xd, wd[start:start + n], s_act, swd[start:start + n]))
        assert np.array_equal(split, mo), f"shard at {start} differs"
        start += n


def test_strided_output_and_zero_m(fp8):
    import torch
    xq, wq, s_act, sw = _prepare(1, 4, 384, 256, outliers=False)
    big = torch.full((4, 400), -7.0, dtype=torch.bfloat16, device="cuda")
    view = big[:, 8:392]
    fp8.scaled_mm(u8_dev(xq), u8_dev(wq), s_act, f32_dev(sw), out=view)
    ref, v = oracle.scaled_mm(xq, wq, s_act, sw, want_v=True)
    assert_within_tolerance(host_u16(view), ref, v, "strided out")
    assert torch.all(big[:, :8] == -7) and torch.all(big[:, 392:] == -7)
    empty = fp8.scaled_mm(u8_dev(xq[:0]), u8_dev(wq), s_act, f32_dev(sw))
    assert empty.shape == (0, 384)


# ------------------------------------------------------------ F32 output ----

def _f32_bits_to_bf16_rne(a):
    """bf16 RNE of finite f32 values (bit arithmetic on the host)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("M,N,K", [(1, 10240, 5120), (8, 10240, 5120), (16, 384, 256), (17, 32, 272),
                                   (65, 80, 144), (300, 1040, 5120), (600, 544, 1088), (8, 5120, 17408),
                                   (32, 5120, 17408)])
def test_f32_output_rounds_to_the_bf16_output(fp8, M, N, K):
    """The F32 variant stores the same scaled fp32 value the bf16 variant
    rounds: bf16_RNE(f32 out) equals the bf16 out bit for bit, on both arms
    (M <= 64: small-M, the two-tile kernel at K = 17408; larger M: large-M),
    and the f32 values meet the oracle's tolerance."""
    xq, wq, s_act, sw = _prepare(2, M, N, K, outliers=True)
    xd, wd, swd = u8_dev(xq), u8_dev(wq), f32_dev(sw)
    o16 = host_u16(fp8.scaled_mm(xd, wd, s_act, swd))
    o32 = fp8.scaled_mm(xd, wd, s_act, swd, out_dtype=__import__("torch").float32).cpu().numpy()
    assert np.all(np.isfinite(o32))
    assert np.array_equal(_f32_bits_to_bf16_rne(o32), o16)
    rows = np.unique(np.linspace(0, M - 1, min(M, 24)).astype(int))
    _, v = oracle.scaled_mm(xq[rows], wq, s_act, sw, want_v=True)
    tol = np.maximum(2.0 * np.abs(v) * 2.0 ** -23, 1e-3 * np.sqrt(np.sum(v * v, axis=1, keepdims=True)))
    assert np.all(np.abs(o32[rows].astype(np.float64) - v) <= tol)


@pytest.mark.parametrize("M", [8, 300])
def test_f32_merged_equals_split_and_strided(fp8, M):
    import torch
    K = 5120
    xq = wl.random_codes(4, M, K, m=M)
    wq = wl.random_codes(4, 1040, K, tensor=wl.T_W)
    sw = (np.random.Generator(np.random.PCG64(1)).random(1040) * 1e-3 + 1e-5).astype(np.float32)
    xd, wd, swd = u8_dev(xq), u8_dev(wq), f32_dev(sw)
    shards = [512, 16, 512]
    big = torch.full((M, 1100), -7.0, dtype=torch.float32, device="cuda")
    outs = [big[:, 4:516], big[:, 520:536], big[:, 540:1052]]
    fp8.scaled_mm_merged(xd, wd, 0.013, swd, shards, outs=outs)
    start = 0
    for n, mo in zip(shards, outs):
        split = fp8.scaled_mm(xd, wd[start:start + n], 0.013, swd[start:start + n], out_dtype=torch.float32)
        assert torch.equal(split, mo), f"shard at {start} differs"
        start += n
    assert torch.all(big[:, :4] == -7) and torch.all(big[:, 516:520] == -7) and torch.all(big[:, 1052:] == -7)


# ------------------------------------------------------ per-token scales ----

@pytest.mark.parametrize("wid,M,K,rms", [(2, 8, 5120, False), (3, 1, 5120, True), (3, 32, 5120, True),
                                         (3, 7, 17408, False), (5, 6576, 5120, True)])
def test_per_token_quant_bit_exact(fp8, wid, M, K, rms):
    x = wl.activation_bf16(wid, M, K, outliers=wid != 5)
    if M >= 7:
        x[1] = 0                                   # zero row: scale 1, codes 0
        x[2] = 0xC040                              # constant row: +-448 everywhere
        x[3, :4] = np.array([0x7F80, 0xFF80, 0x7FC0, 0x0001], np.uint16) if not rms else x[3, :4]
    g = wl.gamma_bf16(wid, K) if rms else None
    q, s = fp8.quant_per_token(bf16_dev(x), None if g is None else bf16_dev(g), wl.EPS)
    q_ref, s_ref = oracle.quant_per_token(x, g, wl.EPS)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host_u8(q), q_ref), f"{int((host_u8(q) != q_ref).sum())} codes differ"


@pytest.mark.parametrize("M,N,K", [(1, 10240, 5120), (8, 10240, 5120), (8, 5120, 17408), (32, 5120, 17408),
                                   (33, 64, 400), (300, 1040, 5120)])
def test_per_token_gemm_against_oracle(fp8, M, N, K):
    """Per-row scales in the epilogue, on both arms; with every row scale equal
    the result is the per-tensor GEMM bit for bit."""
    x = wl.activation_bf16(2, M, K, outliers=True)
    q, s = oracle.quant_per_token(x)
    wq, sw = oracle.quant_weight(wl.weight_f32(2, N, K))
    qd, sd, wd, swd = u8_dev(q), f32_dev(s), u8_dev(wq), f32_dev(sw)
    got = host_u16(fp8.scaled_mm_per_token(qd, wd, sd, swd))
    rows = np.unique(np.linspace(0, M - 1, min(M, 24)).astype(int))
    ref, v = oracle.scaled_mm_rows(q[rows], wq, s[rows], sw, want_v=True)
    assert_within_tolerance(got[rows], ref, v, f"per-token M={M} N={N} K={K}")
    same = np.full(M, s[0], np.float32)
    a = host_u16(fp8.scaled_mm_per_token(qd, wd, f32_dev(same), swd))
    b = host_u16(fp8.scaled_mm(qd, wd, float(s[0]), swd))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("M", [8, 300])
def test_per_token_merged_equals_split(fp8, M):
    K = 5120
    xq = wl.random_codes(4, M, K, m=M)
    wq = wl.random_codes(4, 1040, K, tensor=wl.T_W)
    g = np.random.Generator(np.random.PCG64(2))
    sw = (g.random(1040) * 1e-3 + 1e-5).astype(np.float32)
    sr = (g.random(M) * 1e-2 + 1e-4).astype(np.float32)
    xd, wd, swd, srd = u8_dev(xq), u8_dev(wq), f32_dev(sw), f32_dev(sr)
    shards = [512, 16, 512]
    merged = [host_u16(o) for o in fp8.scaled_mm_merged_per_token(xd, wd, srd, swd, shards)]
    start = 0
    for n, mo in zip(shards, merged):
        split = host_u16(fp8.scaled_mm_per_token(xd, wd[start:start + n], srd, swd[start:start + n]))
        assert np.array_equal(split, mo), f"shard at {start} differs"
        start += n


# ------------------------------------------------- merge and determinism ----

@pytest.mark.parametrize("M", [1, 8, 32, 300])
def test_merged_equals_split_bitwise(fp8, M):
    K = 5120
    xq = wl.random_codes(4, M, K, m=M)
    wq = wl.random_codes(4, 1040, K, tensor=wl.T_W)
    sw = (np.random.Generator(np.random.PCG64(1)).random(1040) * 1e-3 + 1e-5).astype(np.float32)
    s_act = 0.013
    shards = [512, 16, 512]
    xd, wd, swd = u8_dev(xq), u8_dev(wq), f32_dev(sw)
    merged = [host_u16(o) for o in fp8.scaled_mm_merged(xd, wd, s_act, swd, shards)]
    start = 0
    for n, mo in zip(shards, merged):
        split = host_u16(fp8.scaled_mm(xd, wd[start:start + n], s_act, swd[start:start + n]))
        assert np.array_equal(split, mo), f"shard at {start} differs"
        start += n


# ------------------------------------- static quant fused into the GEMM ----

def _quant_then_merged(fp8, xd, s_act, wd, swd, shards):
    """The two-call path the fused entry must reproduce bit for bit."""
    xq = fp8.quant(xd, s_act)
    return [host_u16(o) for o in fp8.scaled_mm_merged(xq, wd, s_act, swd, shards)], host_u8(xq)


def _check_fused(fp8, x, xd, s_act, wq, sw, shards, fused, what):
    wd, swd = u8_dev(wq), f32_dev(sw)
    M, K = x.shape
    assert fp8.quant_scaled_mm_fused(M, sum(shards), K, xd.stride(0), s_act) == fused, what
    want, want_q = _quant_then_merged(fp8, xd, s_act, wd, swd, shards)
    assert np.array_equal(want_q, oracle.quant_act(x, np.float32(s_act))), what
    for rep in range(2):                      # twice: the second call finds the first's x_q and outputs
        outs, xq = fp8.quant_scaled_mm_merged(xd, s_act, wd, swd, shards)
        assert np.array_equal(host_u8(xq), want_q), f"{what}: x_q (call {rep})"
        for i, (o, w) in enumerate(zip(outs, want)):
            assert np.array_equal(host_u16(o), w), f"{what}: shard {i} (call {rep})"
    return want, want_q


# M = 4 is the last row count with the activation loads interleaved with the
# weight fill, 5 the first with every load first in a rotated chunk order
@pytest.mark.parametrize("M", [1, 3, 4, 5, 8])
@pytest.mark.parametrize("K,shards", [(5120, [10240]), (5120, [17408, 17408]), (6144, [5120]),
                                      (5120, [4096, 1024, 9216]), (2048, [4112, 1008]), (3072, [2048])])
def test_fused_quant_merged_equals_quant_then_merged(fp8, M, K, shards):
    """One launch (static quant in the small-M GEMM kernel) == quant, then the
    merged GEMM: x_q and every shard's output bit for bit, and the outputs
    within the oracle's tolerance."""
    x = wl.activation_bf16(2, M, K, outliers=True)
    s_act = oracle.act_scale(x)
    wq, sw = oracle.quant_weight(wl.weight_f32(2, sum(shards), K))
    want, xq = _check_fused(fp8, x, bf16_dev(x), float(s_act), wq, sw, shards, True, f"M={M} K={K}")
    ref, v = oracle.scaled_mm(xq, wq, s_act, sw, want_v=True)
    assert_within_tolerance(np.concatenate(want, axis=1), ref, v, f"fused M={M} K={K}")


@pytest.mark.parametrize("s_act", [1.0, 1.0 / 7.0, 2.0 ** -99, 2.0 ** 99])
def test_fused_quant_every_bf16_pattern(fp8, s_act):
    """Every bf16 pattern (NaN, inf, subnormals, -0) as an 8 x 8192 activation,
    rotated per row: the in-kernel encoder gives the plain quant's codes."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(8, 8192)
    x = np.stack([np.roll(bits[i], 301 * i) for i in range(8)])
    wq = wl.random_codes(5, 2048, 8192, tensor=wl.T_W)
    sw = (np.random.Generator(np.random.PCG64(5)).random(2048) * 1e-3 + 1e-5).astype(np.float32)
    for M in (8, 5):
        _check_fused(fp8, x[:M], bf16_dev(x[:M]), s_act, wq, sw, [1024, 1024], True, f"patterns M={M}")


def test_fused_quant_strided_activation(fp8):
    M, K, ld = 3, 5120, 5136
    x = wl.activation_bf16(3, M, K, outliers=True)
    s_act = float(oracle.act_scale(x))
    wq, sw = oracle.quant_weight(wl.weight_f32(3, 10240, K))
    _check_fused(fp8, x, _strided(x, ld), s_act, wq, sw, [10240], True, "strided")


@pytest.mark.parametrize("M,K,N,s_act", [(9, 5120, 10240, 0.01), (16, 5120, 10240, 0.01),
                                         (8, 5120, 10240, 2.0 ** -120), (4, 17408, 5120, 0.01),
                                         (2, 256, 384, 0.01), (40, 5120, 2048, 0.01)])
def test_fused_quant_falls_back_to_two_launches(fp8, M, K, N, s_act):
    """Shapes the fused kernel does not take (M > 8, a scale outside the code
    table's range, rows too long or too short for its plan, the large-M arm)
    run the quant and the GEMM as two launches, with the same results."""
    x = wl.activation_bf16(4, M, K, outliers=True)
    wq, sw = oracle.quant_weight(wl.weight_f32(4, N, K))
    _check_fused(fp8, x, bf16_dev(x), s_act, wq, sw, [N], False, f"fallback M={M} K={K} N={N}")


def _check_fused_rms(fp8, x, xd, g, eps, s_act, wq, sw, shards, fused, what):
    """Fused RMSNorm quant + merged GEMM against fp8_quant_rmsnorm then the
    merged GEMM: x_q and every output bit for bit (twice), x_q against the oracle."""
    wd, swd, gd = u8_dev(wq), f32_dev(sw), bf16_dev(g)
    M, K = x.shape
    assert fp8.quant_scaled_mm_fused(M, sum(shards), K, xd.stride(0), s_act, rmsnorm=True) == fused, what
    xq = fp8.quant_rmsnorm(xd, gd, s_act, eps)
    want_q = host_u8(xq)
    assert np.array_equal(want_q, oracle.quant_rmsnorm(x, g, eps, np.float32(s_act))), what
    want = [host_u16(o) for o in fp8.scaled_mm_merged(xq, wd, s_act, swd, shards)]
    for rep in range(2):
        outs, xq2 = fp8.quant_rmsnorm_scaled_mm_merged(xd, gd, s_act, eps, wd, swd, shards)
        assert np.array_equal(host_u8(xq2), want_q), f"{what}: x_q (call {rep})"
        for i, (o, w) in enumerate(zip(outs, want)):
            assert np.array_equal(host_u16(o), w), f"{what}: shard {i} (call {rep})"
    return want, want_q


@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("K,shards", [(5120, [17408, 17408]), (5120, [12288]), (5120, [12288, 1024, 1024]),
                                      (4608, [5120])])
def test_fused_rmsnorm_quant_merged_equals_two_calls(fp8, M, K, shards):
    """The RMSNorm quant in the GEMM's launch (8 waves, rows of 36..40
    chunks): the standalone kernel's bytes and the two calls' outputs, bit for
    bit, and the outputs within the oracle's tolerance."""
    x = wl.activation_bf16(3, M, K, outliers=True)
    g = wl.gamma_bf16(3, K)
    s_act = float(oracle.act_scale(x, g, wl.EPS))
    wq, sw = oracle.quant_weight(wl.weight_f32(3, sum(shards), K))
    want, xq = _check_fused_rms(fp8, x, bf16_dev(x), g, wl.EPS, s_act, wq, sw, shards, True, f"rms M={M} K={K}")
    ref, v = oracle.scaled_mm(xq, wq, np.float32(s_act), sw, want_v=True)
    assert_within_tolerance(np.concatenate(want, axis=1), ref, v, f"fused rms M={M} K={K}")


@pytest.mark.parametrize("eps", [1e-6, 0.0])
def test_fused_rmsnorm_quant_special_rows(fp8, eps):
    """Zero rows (r = 1 / sqrt(eps), or inf at eps = 0: 0 * inf is NaN), -0,
    subnormal, +-max, inf and NaN values, gamma with zeros, extremes and a NaN,
    a strided activation: the same bytes as the standalone RMSNorm quant."""
    M, K, ld = 8, 5120, 5136
    x = wl.activation_bf16(3, M, K, outliers=True)
    x[1] = 0
    x[2] = 0x8000
    x[3, :5] = np.array([0x0001, 0x8001, 0x7F7F, 0xFF7F, 0x0080], np.uint16)
    x[4, 7] = 0x7F80                                   # +inf: r = 0
    x[5, 100] = 0x7FC0                                 # NaN: r NaN
    x[6] = (x[6].astype(np.uint32) & 0x80FF).astype(np.uint16) | 0x0100   # tiny values
    g = wl.gamma_bf16(3, K)
    g[:3] = np.array([0x0000, 0x7F7F, 0x0001], np.uint16)
    g2 = g.copy()
    g2[11] = 0x7FC0                                    # NaN in gamma: that column NaN in every row
    s_act = 0.0137
    wq, sw = oracle.quant_weight(wl.weight_f32(3, 12288, K))
    for gg, nm in ((g, "gamma"), (g2, "NaN gamma")):
        _check_fused_rms(fp8, x, _strided(x, ld), gg, eps, s_act, wq, sw, [12288], True, f"{nm} eps={eps}")


@pytest.mark.parametrize("M,K,N,s_act", [(9, 5120, 12288, 0.01), (8, 4096, 12288, 0.01), (8, 6144, 5120, 0.01),
                                         (8, 5120, 12288, 2.0 ** -120), (40, 5120, 2048, 0.01)])
def test_fused_rmsnorm_quant_falls_back(fp8, M, K, N, s_act):
    """Shapes the fused RMSNorm path does not take (M > 8, rows whose wave
    count is not 8, a scale outside the exact quotient's range, the large-M
    arm): two launches, the same bytes."""
    x = wl.activation_bf16(4, M, K, outliers=True)
    g = wl.gamma_bf16(4, K)
    wq, sw = oracle.quant_weight(wl.weight_f32(4, N, K))
    _check_fused_rms(fp8, x, bf16_dev(x), g, wl.EPS, s_act, wq, sw, [N], False, f"rms fallback M={M} K={K}")


def test_fused_quant_empty_shapes(fp8):
    import torch
    K = 5120
    wq, sw = oracle.quant_weight(wl.weight_f32(4, 64, K))
    x = torch.zeros((0, K), dtype=torch.bfloat16, device="cuda")
    outs, xq = fp8.quant_scaled_mm_merged(x, 0.1, u8_dev(wq), f32_dev(sw), [64])
    assert xq.shape == (0, K) and outs[0].shape == (0, 64)
    # no output columns: only the quant runs
    xh = wl.activation_bf16(4, 2, K, outliers=True)
    empty_w = torch.zeros((0, K), dtype=torch.uint8, device="cuda")
    empty_s = torch.zeros((0,), dtype=torch.float32, device="cuda")
    outs, xq = fp8.quant_scaled_mm_merged(bf16_dev(xh), 0.1, empty_w, empty_s, [0])
    assert np.array_equal(host_u8(xq), oracle.quant_act(xh, np.float32(0.1)))
    # an empty shard between two others, fused
    wq, sw = oracle.quant_weight(wl.weight_f32(4, 2048, K))
    _check_fused(fp8, xh, bf16_dev(xh), 0.1, wq, sw, [1024, 0, 1024], True, "empty middle shard")


@pytest.mark.parametrize("M", [1, 2, 4])
def test_run_to_run_and_graph_capture_bitwise(fp8, M):
    import torch
    xq, wq, s_act, sw = _prepare(2, M, 10240, 5120, outliers=True)
    x = wl.activation_bf16(2, M, 5120, outliers=True)
    xd, wd, swd = bf16_dev(x), u8_dev(wq), f32_dev(sw)
    s = oracle.act_scale(x)
    xq_d = fp8.quant(xd, s)
    eager = fp8.scaled_mm(xq_d, wd, s, swd)
    first = host_u16(eager)
    for _ in range(3):
        assert np.array_equal(host_u16(fp8.scaled_mm(xq_d, wd, s, swd)), first)
    # capture quant + GEMM into a HIP graph; replay several times with eager work between
    xq_g = torch.empty_like(xq_d)
    out_g = torch.empty_like(eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        fp8.quant(xd, s, out=xq_g)
        fp8.scaled_mm(xq_g, wd, s, swd, out=out_g)
    torch.cuda.current_stream().wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fp8.quant(xd, s, out=xq_g)
        fp8.scaled_mm(xq_g, wd, s, swd, out=out_g)
    for i in range(4):
        out_g.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(out_g), first), f"replay {i}"
        assert np.array_equal(host_u8(xq_g), host_u8(xq_d))
        _ = fp8.scaled_mm(xq_d, wd, s, swd)          # eager work between replays
        torch.cuda.synchronize()


def test_dispatcher_routes_to_the_selected_arm(fp8):
    t0 = fp8.get_large_m_threshold()
    try:
        for t in (16, 32, 64):
            fp8.set_large_m_threshold(t)
            for M in (1, 8, t, t + 1):
                xq, wq, s_act, sw = _prepare(2, M, 512, 1024, outliers=True)
                auto = _run_arm(fp8, xq, wq, s_act, sw, None)
                arm = fp8.select(M, 512, 1024)
                assert arm == (0 if M <= t else 1)
                assert np.array_equal(auto, _run_arm(fp8, xq, wq, s_act, sw, arm))
    finally:
        fp8.set_large_m_threshold(t0)


def test_fail_closed_on_device_tensors(fp8):
    import torch
    xq, wq, s_act, sw = _prepare(1, 4, 384, 256, outliers=False)
    xd, wd, swd = u8_dev(xq), u8_dev(wq), f32_dev(sw)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(fp8.Fp8mmError) as e:
            fp8.scaled_mm(xd, wd, bad, swd)
        assert e.value.status == fp8.EINVAL
    raw = torch.zeros(4 * 256 + 1, dtype=torch.uint8, device="cuda")
    mis = raw[1:].view(4, 256)                      # 1-byte misaligned x_q
    with pytest.raises(fp8.Fp8mmError) as e:
        fp8.scaled_mm(mis, wd, s_act, swd)
    assert e.value.status == fp8.EUNSUPPORTED
    x = torch.zeros((4, 24), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fp8.Fp8mmError) as e:
        fp8.quant(x, 1.0)
    assert e.value.status == fp8.EUNSUPPORTED



# ------------------------------------- merged shards, per-tensor scales ----
# Attention q/k/v of the pages' tower: one merged qkv of 14336 x 5120 rows,
# split 12288 | 1024 | 1024, each shard with a per-tensor weight scale and its
# own static input scale (vllm.cpp #417, ranked follow-ons).
QKV_SHARDS = (12288, 1024, 1024)
QKV_K = 5120
IN_SCALE_FACTORS = (1.0, 1.5, 0.75)      # synthetic per-shard input scales around the calibrated one


def _qkv_shard_f32(i):
    return wl.weight_f32(4, QKV_SHARDS[i], QKV_K, tensor=wl.T_SHARD0 + i) * np.float32((1.0, 0.5, 2.0)[i])


_QKV_REF = {}


def _qkv_weights(fp8):
    """Seeded f32 shards (N(0, 0.02), scaled by 1, 0.5 and 2 so their per-tensor
    scales differ), quantized per tensor on the GPU and checked against the
    oracle byte for byte; returns the oracle's codes and scales."""
    codes, scales, devs = [], [], []
    for i in range(len(QKV_SHARDS)):
        w = _qkv_shard_f32(i)
        wq_d, s_d = fp8.quant_weight_per_tensor(f32_dev(w))
        if i not in _QKV_REF:
            _QKV_REF[i] = oracle.quant_weight_per_tensor(w)
        wq_ref, s_ref = _QKV_REF[i]
        assert np.float32(s_d.item()).view(np.uint32) == np.float32(s_ref).view(np.uint32), i
        assert np.array_equal(host_u8(wq_d), wq_ref), f"shard {i}: per-tensor codes differ"
        codes.append(wq_ref)
        scales.append(np.float32(s_ref))
        devs.append(wq_d)
    return codes, np.array(scales, np.float32), devs


def test_quant_weight_per_tensor_bit_exact(fp8):
    _qkv_weights(fp8)
    # The tensor max in the last row, an all-zero weight and inf/NaN entries.
    w = wl.weight_f32(4, 48, 256)
    w[47, 255] = np.float32(-0.75)
    for ww in (w, np.zeros((16, 64), np.float32)):
        wq_d, s_d = fp8.quant_weight_per_tensor(f32_dev(ww))
        wq_ref, s_ref = oracle.quant_weight_per_tensor(ww)
        assert np.float32(s_d.item()) == s_ref and np.array_equal(host_u8(wq_d), wq_ref)
    w2 = w.copy()
    w2[3, 5] = np.nan                                              # skipped by the amax
    wq_d, s_d = fp8.quant_weight_per_tensor(f32_dev(w2))
    wq_ref, s_ref = oracle.quant_weight_per_tensor(w2)
    assert np.float32(s_d.item()) == s_ref
    ok = ~np.isnan(w2)
    assert np.array_equal(host_u8(wq_d)[ok], wq_ref[ok]) and (host_u8(wq_d)[3, 5] & 0x7F) == 0x7F


def test_requant_max_scale_bit_exact(fp8):
    codes, scales, _ = _qkv_weights(fp8)
    cat = np.concatenate(codes)
    want, s_max = oracle.requant_max_scale(cat, QKV_SHARDS, scales)
    d = u8_dev(cat)
    got, sw, s_max_d = fp8.requant_max_scale(d, QKV_SHARDS, scales)
    assert np.float32(s_max_d) == s_max == scales.max()
    assert np.array_equal(host_u8(got), want), f"{int((host_u8(got) != want).sum())} codes differ"
    assert np.all(sw.cpu().numpy() == s_max)
    assert np.array_equal(host_u8(got)[:QKV_SHARDS[0]], cat[:QKV_SHARDS[0]]) or scales[0] != s_max
    # In place gives the same bytes.
    fp8.requant_max_scale(d, QKV_SHARDS, scales, out=d)
    assert np.array_equal(host_u8(d), want)
    # Every code (NaN codes included) under arbitrary and power-of-two scale ratios.
    allc = np.tile(np.arange(256, dtype=np.uint8), 4).reshape(16, 64)
    for sc in ([1e-3, 3.3e-4, 1e-3, 2.5e-4], [2.0 ** -7, 2.0 ** -9, 2.0 ** -8, 2.0 ** -12]):
        want, _ = oracle.requant_max_scale(allc, [4, 4, 4, 4], sc)
        got, _, _ = fp8.requant_max_scale(u8_dev(allc), [4, 4, 4, 4], sc)
        assert np.array_equal(host_u8(got), want)


@pytest.mark.parametrize("M", [1, 8, 96])
def test_expanded_scales_merged_equals_split(fp8, M):
    """Exact merge: per-tensor shard scales expanded to per-channel form give,
    column for column, the bits of one GEMM per shard (both arms: M = 96 takes
    the large-M kernel), and match the oracle."""
    codes, scales, devs = _qkv_weights(fp8)
    x = wl.activation_bf16(4, M, QKV_K, outliers=True)
    s_in = oracle.act_scale(x)
    xq = fp8.quant(bf16_dev(x), s_in)
    sw = fp8.expand_shard_scales(QKV_SHARDS, scales)
    assert np.array_equal(sw.cpu().numpy(), np.repeat(scales, QKV_SHARDS))
    w_cat = u8_dev(np.concatenate(codes))
    outs = fp8.scaled_mm_merged(xq, w_cat, s_in, sw, QKV_SHARDS)
    xq_ref = oracle.quant_act(x, s_in)
    for i, (n, o) in enumerate(zip(QKV_SHARDS, outs)):
        one = fp8.scaled_mm(xq, devs[i], s_in, f32_dev(np.full(n, scales[i], np.float32)))
        assert np.array_equal(host_u16(o), host_u16(one)), f"shard {i}: merged != split"
        ref, v = oracle.scaled_mm(xq_ref, codes[i], s_in, np.full(n, scales[i], np.float32), want_v=True)
        assert_within_tolerance(host_u16(o), ref, v, f"qkv shard {i} M={M}")


@pytest.mark.parametrize("M", [8, 64])
def test_merge_policies_end_to_end(fp8, M):
    """Mismatched input scales.  Exact policy: the merge is declined and each
    shard runs its own quant + GEMM at its own scale.  Max-scale policy: one
    quant at the largest input scale, weights requantized to the largest weight
    scale, one merged GEMM; quant and requant bytes bit-exact and outputs within
    tolerance of the oracle's max-scale layer."""
    codes, scales, devs = _qkv_weights(fp8)
    x = wl.activation_bf16(4, M, QKV_K, outliers=True)
    s_cal = oracle.act_scale(x)
    s_in = [np.float32(s_cal * f) for f in IN_SCALE_FACTORS]
    xd = bf16_dev(x)
    merge, _ = fp8.merge_admit(s_in, fp8.MERGE_EXACT)
    assert not merge
    for i, n in enumerate(QKV_SHARDS):
        xq = fp8.quant(xd, float(s_in[i]))
        xq_ref = oracle.quant_act(x, s_in[i])
        assert np.array_equal(host_u8(xq), xq_ref)
        out = fp8.scaled_mm(xq, devs[i], float(s_in[i]), f32_dev(np.full(n, scales[i], np.float32)))
        ref, v = oracle.scaled_mm(xq_ref, codes[i], s_in[i], np.full(n, scales[i], np.float32), want_v=True)
        assert_within_tolerance(host_u16(out), ref, v, f"split shard {i} M={M}")
    merge, s_act = fp8.merge_admit(s_in, fp8.MERGE_MAX_SCALE)
    assert merge and np.float32(s_act) == max(s_in)
    xq = fp8.quant(xd, s_act)
    w2, sw, s_max = fp8.requant_max_scale(u8_dev(np.concatenate(codes)), QKV_SHARDS, scales)
    outs = fp8.scaled_mm_merged(xq, w2, s_act, sw, QKV_SHARDS)
    xq_ref, w2_ref, s_act_ref, s_max_ref, ref, v = oracle.merged_max_scale_layer(x, codes, scales, s_in,
                                                                                 want_v=True)
    assert np.float32(s_act) == s_act_ref and np.float32(s_max) == s_max_ref
    assert np.array_equal(host_u8(xq), xq_ref) and np.array_equal(host_u8(w2), w2_ref)
    got = np.concatenate([host_u16(o) for o in outs], axis=1)
    assert_within_tolerance(got, ref, v, f"max-scale merged qkv M={M}")


@pytest.mark.parametrize("M", [1, 8, 16])
@pytest.mark.parametrize("N,shards", [(5120, [4112, 1008]), (5632, [4384, 16, 1232])])
def test_balanced_last_round_merged_equals_split(fp8, M, N, shards):
    """Decode widths whose whole 16-row tiles fall unevenly on the CUs (320 or
    352 tiles on 256) take the row-balanced last round: each workgroup's share
    of the leftover rows starts at a multiple of 4, so a shard boundary can fall
    inside it (4112 and 4384 here).  Merged == one call per shard, bit for bit,
    for bf16 and f32 outputs, and within the oracle's tolerance."""
    import torch
    K = 2048
    xq = wl.random_codes(4, M, K, m=M)
    wq = wl.random_codes(4, N, K, tensor=wl.T_W)
    sw = (np.random.Generator(np.random.PCG64(3)).random(N) * 1e-3 + 1e-5).astype(np.float32)
    s_act = 0.011
    xd, wd, swd = u8_dev(xq), u8_dev(wq), f32_dev(sw)
    for dt in (torch.bfloat16, torch.float32):
        merged = fp8.scaled_mm_merged(xd, wd, s_act, swd, shards, out_dtype=dt)
        start = 0
        for n, mo in zip(shards, merged):
            split = fp8.scaled_mm(xd, wd[start:start + n], s_act, swd[start:start + n], out_dtype=dt)
            assert torch.equal(split, mo), f"{dt} shard at {start} differs"
            start += n
        if dt == torch.bfloat16:
            ref, v = oracle.scaled_mm(xq, wq, s_act, sw, want_v=True)
            assert_within_tolerance(np.concatenate([host_u16(o) for o in merged], axis=1), ref, v,
                                    f"balanced M={M} N={N}")
