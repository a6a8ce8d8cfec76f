"""The order of the RMSNorm sum of squares (CPU only).

The oracle sums x_k^2 in fp64 in ascending k.  The GPU kernels sum them in a
fixed order of their own: thread t of a 256-thread row group adds the squares
of its 16-byte pieces t, t + 256, ... (8 values each, in element order), each
64-lane wave adds its lanes by an xor butterfly (offsets 32, 16, ..., 1), and
the four wave sums are added in wave order.  fp64 addition is not
associative, so the two sums can differ in their last bits.  The bytes agree
because r = fl32(1 / sqrt(ss / K + eps)) rounds to fp32: a difference of a
few fp64 ulps changes r only when the exact r lies within that distance of an
fp32 rounding boundary.  This test computes r both ways for every row the
workloads normalise and requires the fp32 values to be bitwise equal.
"""
import numpy as np

import oracle
import workloads as wl

ROW_THREADS = 256


def _f64(x_bits):
    return oracle.bf16_bits_to_f32(x_bits).astype(np.float64)


def _ss_ascending(xf):
    ss = np.zeros(xf.shape[0])
    for k in range(xf.shape[1]):
        ss += xf[:, k] * xf[:, k]
    return ss


def _ss_row_group_order(xf):
    M, K = xf.shape
    nv = K // 8
    part = np.zeros((M, ROW_THREADS))
    for p in range(-(-nv // ROW_THREADS)):
        v = np.arange(ROW_THREADS) + p * ROW_THREADS
        live = v < nv
        for i in range(8):
            col = np.where(live, v * 8 + i, 0)
            sq = xf[:, col] * xf[:, col]
            part += np.where(live[None, :], sq, 0.0)
    part = part.reshape(M, ROW_THREADS // 64, 64)
    lanes = np.arange(64)
    for off in (32, 16, 8, 4, 2, 1):
        part = part + part[:, :, lanes ^ off]
    tot = np.zeros(M)
    for w in range(ROW_THREADS // 64):
        tot = tot + part[:, w, 0]
    return tot


def _r(ss, K, eps):
    return (1.0 / np.sqrt(ss / K + np.float64(np.float32(eps)))).astype(np.float32)


def _rows():
    K = 5120
    yield "decode MLP", np.concatenate([wl.activation_bf16(3, M, K, outliers=True) for M in wl.DECODE_MLP.Ms])
    yield "prefill", wl.activation_bf16(5, 6576, K, outliers=False)
    # the decode-step sweep's norm-fed inputs (qkvz and gate_up of each layer group)
    xs = []
    for gi in range(4):
        for pi in range(4):
            xs.append(wl.activation_bf16(4, 8, K, outliers=True, tensor=wl.T_LAYER0 + 16 * gi + pi))
    yield "decode step", np.concatenate(xs)


def test_row_group_order_gives_the_oracle_r_on_every_workload_row():
    differ = 0
    total = 0
    for what, x in _rows():
        xf = _f64(x)
        a, b = _ss_ascending(xf), _ss_row_group_order(xf)
        differ += int((a != b).sum())
        total += a.size
        ra, rb = _r(a, xf.shape[1], wl.EPS), _r(b, xf.shape[1], wl.EPS)
        assert np.array_equal(ra.view(np.uint32), rb.view(np.uint32)), what
    assert total > 6576
    print(f"{differ} of {total} rows have fp64 sums that differ in the last bits; r equal on all")


def test_emulated_order_is_the_oracle_r_on_a_row_built_to_differ():
    """The emulation is not the ascending sum in disguise: on a row of one huge
    value and many tiny ones the two fp64 sums differ."""
    K = 5120
    x = np.full((1, K), 0x3A00, np.uint16)         # 2^-11: squares 2^-22, below half an ulp of 2^32
    x[0, 0] = 0x4780                               # 2^16: its square swallows each tiny square alone
    xf = _f64(x)
    assert _ss_ascending(xf)[0] != _ss_row_group_order(xf)[0]
