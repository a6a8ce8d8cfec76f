"""The C-ABI library on the host (CPU only, no GPU calls).

Checks that libfp8mm.so loads, exports every function include/fp8mm.h declares,
and that the pure host logic behaves as documented: the M-threshold dispatcher
(a pure function of M; M <= 8 always takes the small-M kernel; thresholds in
[2,16) rejected -- vLLM PR #53014, Marlin large-M commit message), the
bitwise merge predicate (vllm.cpp #213, "merge predicate FIRES"), status
strings, workspace queries, and the fail-closed argument validation that
returns before any HIP call.
"""
import ctypes
import os
import re
import struct
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8mm.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+(fp8\w*)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def fp8():
    import fp8_w8a8_scaled_amd as m
    return m


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("fp8_quant_rmsnorm", "fp8_scaled_mm", "fp8_scaled_mm_merged", "fp8_scaled_mm_select",
                     "fp8_set_large_m_threshold", "fp8_scales_bitwise_equal", "fp8mm_strerror",
                     "fp8_scaled_mm_workspace_bytes", "fp8_quant_weight", "fp8_act_scale"):
        assert required in names


def test_library_exports_every_declared_symbol(fp8):
    lib = ctypes.CDLL(fp8.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    out = subprocess.run(["nm", "-D", "--defined-only", fp8.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(_declared_functions()) <= exported


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-fsyntax-only", "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                        "-x", "c", HEADER], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_dispatcher_is_pure_in_m_and_guards_decode(fp8):
    t0 = fp8.get_large_m_threshold()
    try:
        for t in (16, 32, 64):
            fp8.set_large_m_threshold(t)
            assert fp8.get_large_m_threshold() == t
            for M in range(0, 300):
                want = 0 if M <= t else 1
                assert fp8.select(M, 10240, 5120) == want
                assert fp8.select(M, 16, 16) == want          # N and K do not matter
            for M in range(0, 9):
                assert fp8.select(M, 5120, 17408) == 0
        for bad in (-1, 0, 1, 2, 8, 15, 65, 512, 4096):
            with pytest.raises(fp8.Fp8mmError) as e:
                fp8.set_large_m_threshold(bad)
            assert e.value.status == fp8.EINVAL
            assert fp8.get_large_m_threshold() == 64            # unchanged
        assert fp8.select(-1, 1, 1) == fp8.EINVAL
    finally:
        fp8.set_large_m_threshold(t0)


def test_threshold_env_read_at_load():
    code = ("import fp8_w8a8_scaled_amd as m; print(m.get_large_m_threshold())")
    env = dict(os.environ, FP8MM_LARGE_M_THRESHOLD="48", PYTHONPATH=ROOT)
    assert subprocess.run(["python", "-c", code], env=env, capture_output=True, text=True).stdout.strip() == "48"
    env["FP8MM_LARGE_M_THRESHOLD"] = "4"     # rejected -> built-in default
    r = subprocess.run(["python", "-c", code], env=env, capture_output=True, text=True).stdout.strip()
    assert 16 <= int(r) <= 64 and r != "4"


def test_scales_bitwise_equal(fp8):
    assert fp8.scales_bitwise_equal([0.0123, 0.0123, 0.0123])
    a = np.float32(0.0123)
    b = np.frombuffer(struct.pack("<I", struct.unpack("<I", struct.pack("<f", a))[0] + 1), np.float32)[0]
    assert not fp8.scales_bitwise_equal([a, b])                 # one ulp apart
    assert not fp8.scales_bitwise_equal([0.0, -0.0])            # equal values, different bits
    assert fp8.scales_bitwise_equal([1.5])
    with pytest.raises(fp8.Fp8mmError):
        fp8.scales_bitwise_equal([])


def test_status_strings_and_workspace(fp8):
    for s in (fp8.OK, fp8.EINVAL, fp8.EUNSUPPORTED, fp8.EWORKSPACE, fp8.ELAUNCH):
        assert fp8.strerror(s) and fp8.strerror(s) != "unknown status"
    assert fp8.strerror(12345) == "unknown status"
    assert fp8.workspace_bytes(8, 10240, 5120) == 0
    lib = fp8.raw_lib()
    assert lib.fp8_act_scale_workspace_bytes(6576, 5120) >= 6576 * 4


# Fake, never-dereferenced device addresses: every call below must be rejected
# (or be an M == 0 no-op) by host validation before any HIP call -- never add a
# case here that passes validation with M > 0: it would launch on fake pointers.
A = 0x10000000
B = 0x20000000
C = 0x30000000
D = 0x40000000


def _mm(lib, xq=A, wq=B, s_act=0.5, sw=C, out=D, ldo=10240, M=8, N=10240, K=5120, ws=None, wsb=0):
    f = lib.fp8_scaled_mm
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    return f(xq, wq, s_act, sw, out, ldo, M, N, K, ws, wsb, None)


def test_gemm_validation_fails_closed(fp8):
    lib = fp8.raw_lib()
    E, U = fp8.EINVAL, fp8.EUNSUPPORTED
    assert _mm(lib, xq=None) == E
    assert _mm(lib, out=None) == E
    assert _mm(lib, M=-1) == E
    assert _mm(lib, N=-16) == E
    assert _mm(lib, ldo=16) == E                                # ldo < N
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert _mm(lib, s_act=bad) == E
    assert _mm(lib, K=5121) == U                                # K % 16
    assert _mm(lib, K=5128) == U
    assert _mm(lib, N=10248, ldo=10248) == U                    # N % 16
    assert _mm(lib, ldo=10244) == U                             # ldo % 8
    assert _mm(lib, xq=A + 8) == U                              # 16-byte alignment
    assert _mm(lib, wq=B + 1) == U
    assert _mm(lib, sw=C + 4) == U
    assert _mm(lib, out=D + 2) == U
    assert _mm(lib, M=0) == fp8.OK                              # no-op, no launch
    f = lib.fp8_scaled_mm_arm
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert f(A, B, 0.5, C, D, 16, 65, 16, 16, 0, None, 0, None) == E   # small-M arm beyond its M
    assert f(A, B, 0.5, C, D, 16, 8, 16, 16, 2, None, 0, None) == E    # no such arm
    assert f(A, B, 0.5, C, D, 16, 0, 16, 16, 1, None, 0, None) == fp8.OK


def test_merged_validation_fails_closed(fp8):
    lib = fp8.raw_lib()
    Shard = fp8.Shard
    f = lib.fp8_scaled_mm_merged
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.POINTER(Shard),
                  ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]

    def call(shards, n=None, M=0):
        arr = (Shard * max(1, len(shards)))(*shards)
        return f(A, B, 0.5, C, arr, len(shards) if n is None else n, M, 5120, None, 0, None)

    good = [Shard(17408, D, 17408), Shard(17408, D + 0x1000000, 17408)]
    assert call(good) == fp8.OK                                  # M == 0 no-op
    assert call(good, n=0) == fp8.EINVAL
    assert call(good * 5, n=9) == fp8.EINVAL                     # > 8 shards
    assert call([Shard(17400, D, 17408)]) == fp8.EUNSUPPORTED    # shard n % 16
    assert call([Shard(17408, D + 8, 17408)]) == fp8.EUNSUPPORTED
    assert call([Shard(17408, None, 17408)], M=1) == fp8.EINVAL   # rejected before any launch
    assert call([Shard(17408, None, 17408)]) == fp8.OK           # empty product: null output allowed
    assert call([Shard(17408, D, 16)]) == fp8.EINVAL             # ldo < n


def test_quant_merged_validation_fails_closed(fp8):
    """The one-launch static quant + merged GEMM checks the quant's and the
    GEMM's arguments before launching anything."""
    lib = fp8.raw_lib()
    Shard = fp8.Shard
    f = lib.fp8_quant_scaled_mm_merged
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.POINTER(Shard), ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    E, U = fp8.EINVAL, fp8.EUNSUPPORTED
    good = (Shard * 2)(Shard(17408, D, 17408), Shard(17408, D + 0x1000000, 17408))

    def call(x=A, ldx=5120, s=0.1, xq=B, M=8, K=5120, shards=good, n=2):
        return f(x, ldx, s, xq, C, C + 0x100000, shards, n, M, K, None, 0, None)

    assert call(M=0) == fp8.OK
    assert call(x=None) == E
    assert call(xq=None) == E
    assert call(ldx=5000) == E                                  # ldx < K
    assert call(s=0.0) == E
    assert call(s=float("inf")) == E
    assert call(ldx=5124) == U                                  # ldx % 8
    assert call(K=5112 + 4, ldx=5120) == U                      # K % 16
    assert call(x=A + 2) == U
    assert call(xq=B + 8) == U
    assert call(xq=A + 16) == E                                 # x_q overlaps x
    assert call(n=0) == E
    assert call(shards=(Shard * 1)(Shard(17400, D, 17408)), n=1) == U
    assert call(shards=(Shard * 1)(Shard(17408, None, 17408)), n=1) == E
    q = lib.fp8_quant_scaled_mm_fused
    q.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_float, ctypes.c_int]
    for rms in (0, 1):
        assert q(9, 10240, 5120, 5120, 0.1, rms) == 0           # beyond the fused kernel's M
        assert q(8, 10240, 5120, 5120, 2.0 ** -120, rms) == 0   # outside the quotient's exact range
        assert q(8, 10240, 5120, 5000, 0.1, rms) == 0           # ldx < K
        assert q(8, 10240, 5120, 5120, 0.0, rms) == 0
        assert q(0, 10240, 5120, 5120, 0.1, rms) == 0
    # the fused RMSNorm quant: its own argument checks, before any launch
    h = lib.fp8_quant_rmsnorm_scaled_mm_merged
    h.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Shard), ctypes.c_int, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]

    def rcall(gamma=D + 0x2000000, eps=1e-6, M=8, xq=B):
        return h(A, 5120, gamma, eps, 0.1, xq, C, C + 0x100000, good, 2, M, 5120, None, 0, None)

    assert rcall(M=0) == fp8.OK
    assert rcall(eps=float("nan")) == E
    assert rcall(eps=-1.0) == E
    assert rcall(gamma=D + 0x2000000 + 2) == U
    assert rcall(xq=A + 16) == E                                 # x_q overlaps x
    assert rcall(gamma=None, eps=float("nan"), M=0) == fp8.OK   # no gamma: eps unused


def test_quant_validation_fails_closed(fp8):
    lib = fp8.raw_lib()
    f = lib.fp8_quant_rmsnorm
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_float,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    E, U = fp8.EINVAL, fp8.EUNSUPPORTED
    assert f(None, 5120, C, 1e-6, 0.1, B, 8, 5120, None) == E
    assert f(A, 5000, C, 1e-6, 0.1, B, 8, 5120, None) == E       # ldx < K
    assert f(A, 5120, C, 1e-6, 0.0, B, 8, 5120, None) == E
    assert f(A, 5120, C, float("nan"), 0.1, B, 8, 5120, None) == E
    assert f(A, 5120, C, 1e-6, 0.1, B, 8, 5112 + 4, None) == U   # K % 16
    assert f(A, 5124, C, 1e-6, 0.1, B, 8, 5120, None) == U       # ldx % 8
    assert f(A + 2, 5120, C, 1e-6, 0.1, B, 8, 5120, None) == U
    assert f(A, 5120, C + 2, 1e-6, 0.1, B, 8, 5120, None) == U
    assert f(A, 5120, C, 1e-6, 0.1, A + 16, 8, 5120, None) == E  # x_q overlaps x
    assert f(A, 5120, C, 1e-6, 0.1, B, 0, 5120, None) == fp8.OK
    g = lib.fp8_quant_weight
    g.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert g(A, 16, 24, B, C, None) == U
    assert g(A, 0, 32, B, C, None) == fp8.OK
    assert g(None, 16, 32, B, C, None) == E


def test_silu_mul_validation_fails_closed(fp8):
    lib = fp8.raw_lib()
    f = lib.fp8_silu_mul_quant
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    E, U = fp8.EINVAL, fp8.EUNSUPPORTED
    I, L = 17408, 2 * 17408                                      # gate/up halves of a gate_up row
    assert f(None, L, A + 2 * I, L, 0.1, B, 8, I, None) == E
    assert f(A, L, None, L, 0.1, B, 8, I, None) == E
    assert f(A, L, A + 2 * I, L, 0.1, None, 8, I, None) == E
    assert f(A, I - 8, A + 2 * I, L, 0.1, B, 8, I, None) == E    # ldg < I
    assert f(A, L, A + 2 * I, I - 8, 0.1, B, 8, I, None) == E    # ldu < I
    assert f(A, L, A + 2 * I, L, 0.1, B, -1, I, None) == E
    for s in (0.0, -1.0, float("inf"), float("nan")):
        assert f(A, L, A + 2 * I, L, s, B, 8, I, None) == E
    assert f(A, L, A + 2 * I, L, 0.1, B, 8, I - 8, None) == U    # I % 16
    assert f(A, L + 4, A + 2 * I, L, 0.1, B, 8, I, None) == U    # ldg % 8
    assert f(A + 2, L, A + 2 * I, L, 0.1, B, 8, I, None) == U
    assert f(A, L, A + 2 * I + 2, L, 0.1, B, 8, I, None) == U
    assert f(A, L, A + 2 * I, L, 0.1, B + 8, 8, I, None) == U
    assert f(A, L, A + 2 * I, L, 0.1, A + 64, 8, I, None) == E   # x_q overlaps gate
    assert f(A, L, A + 2 * I, L, 0.1, A + 7 * L * 2 + 2 * I, 8, I, None) == E  # x_q overlaps up's last row
    assert f(A, L, A + 2 * I, L, 0.1, B, 0, I, None) == fp8.OK
    assert f(A, L, A + 2 * I, L, 0.1, None, 0, I, None) == fp8.OK   # empty: nothing written
    g = lib.fp8_act_scale_silu_mul
    g.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    ws = int(lib.fp8_act_scale_workspace_bytes(ctypes.c_int64(8), ctypes.c_int64(I)))
    assert ws > 0
    assert g(A, L, A + 2 * I, L, 0, I, C, D, ws, None) == E      # nothing to calibrate on
    assert g(A, L, A + 2 * I, L, 8, I, None, D, ws, None) == E
    assert g(A, L, A + 2 * I, L, 8, I, C, None, ws, None) == fp8.EWORKSPACE
    assert g(A, L, A + 2 * I, L, 8, I, C, D, ws - 4, None) == fp8.EWORKSPACE
    assert g(A, L, A + 2 * I, L, 8, I - 8, C, D, ws, None) == U
    assert g(A + 2, L, A + 2 * I, L, 8, I, C, D, ws, None) == U
    assert g(A, L, A + 2 * I, L, 8, I, C, D + 8, ws, None) == U


def test_gate_up_silu_validation_fails_closed(fp8):
    """The gate_up launch with the SiLU*mul epilogue, its plan query and the
    weight interleave check their arguments before launching anything; a shape
    outside the fused plans is FP8MM_EUNSUPPORTED (the caller then runs the
    separate calls)."""
    lib = fp8.raw_lib()
    P, I64, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    f = lib.fp8_gate_up_silu_quant
    f.argtypes = [P, I64, P, F32, F32, P, P, P, F32, P, I64, I64, I64, P]
    E, U = fp8.EINVAL, fp8.EUNSUPPORTED

    def call(x=None, ldx=5120, gamma=None, eps=1e-6, s=0.1, xq=B, w=C, sw=C + 0xC000000, sd=0.05, hq=D, M=8,
             I=17408, K=5120):
        return f(x, ldx, gamma, eps, s, xq, w, sw, sd, hq, M, I, K, None)

    assert call(M=0) == fp8.OK
    assert call(I=0) == fp8.OK
    assert call(M=-1) == E
    assert call(s=0.0) == E
    assert call(sd=float("nan")) == E
    assert call(gamma=A) == E                                    # gamma without x
    assert call(x=A, gamma=A + 0x1000000, eps=-1.0) == E
    assert call(x=A, ldx=5000) == E                              # ldx < K
    assert call(I=17400) == U                                    # I % 16
    assert call(K=5112) == U                                     # K % 16
    assert call(x=A, ldx=5124) == U                              # ldx % 8
    assert call(K=0) == U
    assert call(w=None) == E
    assert call(hq=None) == E
    assert call(xq=None) == E                                    # neither x nor x_q
    assert call(hq=D + 8) == U
    assert call(sw=C + 0xC000000 + 4) == U
    assert call(x=A + 2) == U
    assert call(hq=C + 16) == E                                  # h_q overlaps the weight
    assert call(hq=B + 64) == E                                  # h_q overlaps x_q
    assert call(x=A, xq=A + 16) == E                             # x_q (written) overlaps x
    assert call(M=33) == U                                       # the large-M arm (threshold 32)
    assert call(x=A, M=9) == U                                   # the quant in the launch: M <= 8
    assert call(sd=2.0 ** -120) == U                             # outside the quotient's exact range
    q = lib.fp8_gate_up_silu_quant_fused
    q.argtypes = [I64, I64, I64, I64, F32, F32, ctypes.c_int]
    assert q(33, 17408, 5120, 5120, 0.1, 0.05, 0) == 0
    assert q(9, 17408, 5120, 5120, 0.1, 0.05, 1) == 0
    assert q(9, 17408, 5120, 5120, 0.1, 0.05, 2) == 0
    assert q(8, 17408, 5120, 5120, 0.1, 2.0 ** -120, 0) == 0
    assert q(8, 17408, 5120, 5120, 2.0 ** -120, 0.05, 1) == 0
    assert q(8, 17400, 5120, 5120, 0.1, 0.05, 0) == 0
    assert q(8, 17408, 5120, 5120, 0.1, 0.05, 3) == 0
    assert q(8, 17408, 5120, 5000, 0.1, 0.05, 2) == 0
    assert q(0, 17408, 5120, 5120, 0.1, 0.05, 0) == 0
    g = lib.fp8_interleave_gate_up
    g.argtypes = [P, P, P, P, I64, I64, P]

    def icall(w=A, sw=B, wil=C, sil=D, I=17408, K=5120):
        return g(w, sw, wil, sil, I, K, None)

    assert icall(I=0) == fp8.OK
    assert icall(I=-16) == E
    assert icall(I=17400) == U
    assert icall(K=5112) == U
    assert icall(K=0) == U
    assert icall(w=None) == E
    assert icall(sil=None) == E
    assert icall(wil=C + 8) == U
    assert icall(sw=B + 4) == U
    assert icall(wil=A + 16) == E                                # w_il overlaps w_q
    assert icall(sil=B + 16) == E                                # s_il overlaps s_w
    assert icall(sil=C + 64) == E                                # s_il overlaps w_il


def test_f32_output_validation_fails_closed(fp8):
    lib = fp8.raw_lib()
    f = lib.fp8_scaled_mm_f32
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    E, U = fp8.EINVAL, fp8.EUNSUPPORTED
    assert f(A, B, 0.5, C, D, 10240, 0, 10240, 5120, None, 0, None) == fp8.OK     # M == 0
    assert f(A, B, 0.5, C, D, 10244, 0, 10240, 5120, None, 0, None) == fp8.OK     # f32 rows: ldo % 4 suffices
    assert f(A, B, 0.5, C, D, 10242, 8, 10240, 5120, None, 0, None) == U          # ldo % 4
    assert f(A, B, 0.5, C, D + 8, 10240, 8, 10240, 5120, None, 0, None) == U      # 16-byte rows
    assert f(A, B, 0.5, C, None, 10240, 8, 10240, 5120, None, 0, None) == E
    assert f(A, B, 0.0, C, D, 10240, 8, 10240, 5120, None, 0, None) == E
    assert f(A, B, 0.5, C, D, 10000, 8, 10240, 5120, None, 0, None) == E          # ldo < N
    g = lib.fp8_scaled_mm_merged_f32
    Shard = fp8.Shard
    g.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.POINTER(Shard),
                  ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]

    def call(shards, n=None, M=0):
        arr = (Shard * max(1, len(shards)))(*shards)
        return g(A, B, 0.5, C, arr, len(shards) if n is None else n, M, 5120, None, 0, None)

    assert call([Shard(17408, D, 17412), Shard(17408, D + 0x2000000, 17408)]) == fp8.OK
    assert call([Shard(17408, D, 17410)]) == U                   # ldo % 4
    assert call([Shard(17408, None, 17408)], M=1) == E
    assert call([Shard(16, D, 16)] * 9, n=9) == E
    assert g(A, B, 0.5, C, None, 1, 0, 5120, None, 0, None) == E


def test_per_token_validation_fails_closed(fp8):
    lib = fp8.raw_lib()
    f = lib.fp8_quant_per_token
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    E, U = fp8.EINVAL, fp8.EUNSUPPORTED
    assert f(A, 5120, None, 0.0, B, C, 0, 5120, None) == fp8.OK
    assert f(A, 5120, None, 0.0, B, None, 8, 5120, None) == E          # no scale output
    assert f(None, 5120, None, 0.0, B, C, 8, 5120, None) == E
    assert f(A, 5000, None, 0.0, B, C, 8, 5120, None) == E             # ldx < K
    assert f(A, 5120, C, float("nan"), B, C + 0x100000, 8, 5120, None) == E
    assert f(A, 5120, None, 0.0, B, C + 2, 8, 5120, None) == U         # s_rows alignment
    assert f(A, 5120, None, 0.0, B, C, 8, 5112 + 4, None) == U         # K % 16
    assert f(A, 5120, None, 0.0, B, A + 64, 8, 5120, None) == E        # s_rows overlaps x
    assert f(A, 5120, None, 0.0, B, B + 64, 8, 5120, None) == E        # s_rows overlaps x_q
    g = lib.fp8_scaled_mm_per_token
    g.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert g(A, B, None, C, D, 10240, 0, 10240, 5120, None, 0, None) == fp8.OK
    assert g(A, B, None, C, D, 10240, 8, 10240, 5120, None, 0, None) == E   # no per-row scales
    assert g(A, B, C + 2, C, D, 10240, 8, 10240, 5120, None, 0, None) == U
    assert g(A, B, C, C, D, 10244, 8, 10240, 5120, None, 0, None) == U      # bf16 rows: ldo % 8


def test_merge_admit_policies(fp8):
    """Exact policy: merge only on bitwise-equal input scales (vllm.cpp #213,
    "merge predicate FIRES"); max-scale policy: always merge at the largest
    input scale (vllm.cpp #417, ranked follow-ons)."""
    a = np.float32(0.0123)
    b = np.frombuffer(struct.pack("<I", struct.unpack("<I", struct.pack("<f", a))[0] + 1), np.float32)[0]
    assert fp8.merge_admit([a, a, a]) == (True, float(a))
    assert fp8.merge_admit([a, b, a]) == (False, None)                   # one ulp apart: split
    assert fp8.merge_admit([a, b, a], fp8.MERGE_MAX_SCALE) == (True, float(b))
    assert fp8.merge_admit([0.5, 2.0, 1.0], fp8.MERGE_MAX_SCALE) == (True, 2.0)
    assert fp8.merge_admit([3.0]) == (True, 3.0)
    for bad in ([], [0.0, 1.0], [1.0, -1.0], [float("nan")], [float("inf"), 1.0], [1.0] * 9):
        for pol in (fp8.MERGE_EXACT, fp8.MERGE_MAX_SCALE):
            with pytest.raises(fp8.Fp8mmError):
                fp8.merge_admit(bad, pol)
    with pytest.raises(fp8.Fp8mmError):
        fp8.merge_admit([1.0, 1.0], 7)


def test_shard_scale_calls_fail_closed(fp8):
    lib = fp8.raw_lib()
    E, U = fp8.EINVAL, fp8.EUNSUPPORTED
    P = ctypes.c_void_p

    def arr(vals, t):
        a = np.ascontiguousarray(np.asarray(vals, dtype=t))
        return a, a.ctypes.data

    rows, pr = arr([64, 16, 16], np.int64)
    sc, ps = arr([1e-3, 2e-3, 5e-4], np.float32)
    zr, pz = arr([0, 0, 0], np.int64)
    bad_sc, pbs = arr([1e-3, 0.0, 5e-4], np.float32)
    neg, pn = arr([64, -16, 16], np.int64)
    ex = lib.fp8_expand_shard_scales
    ex.argtypes = [P, P, ctypes.c_int, P, P]
    assert ex(pz, ps, 3, None, None) == fp8.OK                          # no rows: no-op
    assert ex(pr, ps, 3, None, None) == E                                # no output
    assert ex(pr, ps, 0, C, None) == E and ex(pr, ps, 9, C, None) == E   # shard count
    assert ex(pr, pbs, 3, C, None) == E and ex(pn, ps, 3, C, None) == E
    assert ex(None, ps, 3, C, None) == E and ex(pr, None, 3, C, None) == E
    assert ex(pr, ps, 3, C + 2, None) == U                               # 4-byte alignment
    rq = lib.fp8_requant_max_scale
    rq.argtypes = [P, P, ctypes.c_int64, P, P, ctypes.c_int, P, P, P]
    smax = ctypes.c_float(0.0)
    assert rq(A, A, 5120, pz, ps, 3, C, ctypes.byref(smax), None) == fp8.OK   # no rows: only s_max
    assert smax.value == np.float32(2e-3)
    assert rq(A, B, 5120, pr, ps, 3, None, None, None) == E              # no s_w
    assert rq(None, B, 5120, pr, ps, 3, C, None, None) == E
    assert rq(A, B, 5120, pr, pbs, 3, C, None, None) == E
    assert rq(A, B, 5112 + 4, pr, ps, 3, C, None, None) == U             # K % 16
    assert rq(A, B + 8, 5120, pr, ps, 3, C, None, None) == U             # alignment
    assert rq(A, A + 5120, 5120, pr, ps, 3, C, None, None) == E          # partial overlap in/out
    assert rq(A, B, 5120, pr, ps, 3, A + 64, None, None) == E            # s_w overlaps the weight
    assert rq(A, B, -16, pr, ps, 3, C, None, None) == E
    qt = lib.fp8_quant_weight_per_tensor
    qt.argtypes = [P, ctypes.c_int64, ctypes.c_int64, P, P, P, ctypes.c_size_t, P]
    wsb = lib.fp8_quant_weight_per_tensor_workspace_bytes
    wsb.argtypes, wsb.restype = [ctypes.c_int64, ctypes.c_int64], ctypes.c_size_t
    need = wsb(1024, 5120)
    assert need >= 4 and wsb(0, 5120) == 0
    assert qt(A, 0, 5120, B, C, D, need, None) == E                      # nothing to take a scale from
    assert qt(A, 1024, 5112 + 4, B, C, D, need, None) == U
    assert qt(None, 1024, 5120, B, C, D, need, None) == E
    assert qt(A, 1024, 5120, B, C, D, need - 4, None) == fp8.EWORKSPACE
    assert qt(A, 1024, 5120, B, C, None, need, None) == fp8.EWORKSPACE
    assert qt(A, 1024, 5120, B, C + 2, D, need, None) == U
    assert qt(A, 1024, 5120, A + 16, C, D, need, None) == E              # w_q overlaps w
