"""The merged gate_up GEMM with the SiLU*mul -> E4M3 quant as its epilogue
(fp8_gate_up_silu_quant: the decode MLP's first projection and the down
projection's input quant in one launch), on the GPU.

Bar: h_q (and x_q where the quant runs in the launch) bit for bit those of the
separate calls on the merged [gate; up] weight -- the merged GEMM, then
fp8_silu_mul_quant -- whose h_q is checked against the oracle's SiLU*mul quant
of that GEMM's bf16 output; the interleave bit for bit the row permutation it
documents.  Activations are finite (the gate_up output then is too).
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import bf16_dev, f32_dev, host_u16, host_u8, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import fp8_w8a8_scaled_amd as m
    return m


def _interleaved_rows(I):
    """Merged row held by each interleaved row: 8 gate rows, then the up rows of
    the same 8 columns, per 16-row tile."""
    r = np.arange(2 * I)
    t, k = r // 16, r % 16
    return np.where(k < 8, 8 * t + k, I + 8 * t + k - 8)


def _separate(fp8, xq_d, wd, swd, s_act, I):
    """The separate calls: merged gate_up GEMM, calibration of the down
    projection's input scale, SiLU*mul quant; h_q checked against the oracle."""
    gate, up = fp8.scaled_mm_merged(xq_d, wd, s_act, swd, [I, I])
    s_down = float(fp8.act_scale_silu_mul(gate, up).item())
    want = host_u8(fp8.silu_mul_quant(gate, up, s_down))
    assert np.array_equal(want, oracle.silu_mul_quant(host_u16(gate), host_u16(up), np.float32(s_down)))
    return s_down, want


def test_interleave_is_the_row_permutation(fp8):
    I, K = 272, 256
    rng = np.random.default_rng(11)
    wq = rng.integers(0, 256, size=(2 * I, K), dtype=np.uint8)
    sw = rng.random(2 * I, dtype=np.float32)
    w_il, s_il = fp8.interleave_gate_up(u8_dev(wq), f32_dev(sw))
    rows = _interleaved_rows(I)
    assert np.array_equal(host_u8(w_il), wq[rows])
    assert np.array_equal(s_il.cpu().numpy().view(np.uint32), sw[rows].view(np.uint32))


# (17408, 5120): the decode MLP (2176 tiles, 8-9 per workgroup); (528, 5120):
# 66 tiles, one per workgroup; (1040, 4096): 7 waves of 5 chunks.  M = 1..8:
# fragments through LDS, 16: 16 rows through LDS, 24 and 32: two B tiles in
# registers.
@pytest.mark.parametrize("M", [1, 4, 8, 16, 24, 32])
@pytest.mark.parametrize("I,K", [(17408, 5120), (528, 5120), (1040, 4096)])
def test_gate_up_silu_from_codes(fp8, M, I, K):
    x = wl.activation_bf16(4, M, K, outliers=True)
    s_act = float(oracle.act_scale(x))
    xq_d = u8_dev(oracle.quant_act(x, np.float32(s_act)))
    wq, sw = oracle.quant_weight(wl.weight_f32(4, 2 * I, K))
    wd, swd = u8_dev(wq), f32_dev(sw)
    s_down, want = _separate(fp8, xq_d, wd, swd, s_act, I)
    w_il, s_il = fp8.interleave_gate_up(wd, swd)
    assert fp8.gate_up_silu_quant_fused(M, I, K, s_act, s_down, 0)
    for rep in range(2):
        got = host_u8(fp8.gate_up_silu_quant(w_il, s_il, s_act, s_down, x_q=xq_d))
        assert np.array_equal(got, want), f"M={M} I={I} K={K} call {rep}: {int((got != want).sum())} codes differ"


@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("rms", [False, True])
def test_gate_up_silu_with_the_quant_in_the_launch(fp8, M, rms):
    """The activation quant in the same launch (plain static quant, or the
    fused RMSNorm quant), x_q written when asked for, also from a strided x."""
    import torch
    I, K, ld = 17408, 5120, 5136
    x = wl.activation_bf16(3, M, K, outliers=True)
    g = wl.gamma_bf16(3, K) if rms else None
    xs = np.zeros((M, ld), np.uint16)
    xs[:, :K] = x
    xd = bf16_dev(xs)[:, :K]
    gd = bf16_dev(g) if rms else None
    s_act = float(oracle.act_scale(x, g, wl.EPS)) if rms else float(oracle.act_scale(x))
    xq_d = fp8.quant_rmsnorm(xd, gd, s_act, wl.EPS) if rms else fp8.quant(xd, s_act)
    wq, sw = oracle.quant_weight(wl.weight_f32(3, 2 * I, K))
    wd, swd = u8_dev(wq), f32_dev(sw)
    s_down, want = _separate(fp8, xq_d, wd, swd, s_act, I)
    w_il, s_il = fp8.interleave_gate_up(wd, swd)
    assert fp8.gate_up_silu_quant_fused(M, I, K, s_act, s_down, 2 if rms else 1, ldx=ld)
    xq_out = torch.full((M, K), 0xA5, dtype=torch.uint8, device="cuda")
    got = fp8.gate_up_silu_quant(w_il, s_il, s_act, s_down, x=xd, gamma=gd, eps=wl.EPS, x_q_out=xq_out)
    assert np.array_equal(host_u8(got), want), f"rms={rms} M={M}"
    assert np.array_equal(host_u8(xq_out), host_u8(xq_d)), f"rms={rms} M={M}: x_q"
    got2 = fp8.gate_up_silu_quant(w_il, s_il, s_act, s_down, x=xd, gamma=gd, eps=wl.EPS)
    assert np.array_equal(host_u8(got2), want), f"rms={rms} M={M}, x_q not written"


def test_gate_up_silu_outside_the_fused_plans(fp8):
    """A width whose tiles leave the workgroups unbalanced (258 tiles on 256
    CUs: balanced rows, not whole tiles), M past the small-M arm, and M > 8
    with the quant in the launch: the query says no and the call raises
    EUNSUPPORTED without launching; the separate calls still serve them."""
    import torch
    M, I, K = 8, 2064, 5120
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the unbalanced width is sized for 256 CUs")
    x = wl.activation_bf16(4, M, K, outliers=False)
    s_act = float(oracle.act_scale(x))
    xq_d = u8_dev(oracle.quant_act(x, np.float32(s_act)))
    wq, sw = oracle.quant_weight(wl.weight_f32(4, 2 * I, K))
    w_il, s_il = fp8.interleave_gate_up(u8_dev(wq), f32_dev(sw))
    assert not fp8.gate_up_silu_quant_fused(M, I, K, s_act, 0.05, 0)
    out = torch.full((M, I), 0xA5, dtype=torch.uint8, device="cuda")
    with pytest.raises(fp8.Fp8mmError) as e:
        fp8.gate_up_silu_quant(w_il, s_il, s_act, 0.05, x_q=xq_d, out=out)
    assert e.value.status == fp8.EUNSUPPORTED
    torch.cuda.synchronize()
    assert int((out != 0xA5).sum().item()) == 0
    assert not fp8.gate_up_silu_quant_fused(40, 17408, 5120, s_act, 0.05, 0)
    assert not fp8.gate_up_silu_quant_fused(9, 17408, 5120, s_act, 0.05, 1)


def test_decode_mlp_under_graph_capture(fp8):
    """The decode MLP as two launches (gate_up with the RMSNorm quant inside and
    the SiLU*mul quant as its epilogue, then down) captured in a HIP graph and
    replayed several times, with eager work between replays: every replay
    gives the eager bytes."""
    import torch
    M, I, K = 8, 17408, 5120
    x = wl.activation_bf16(3, M, K, outliers=True)
    g = wl.gamma_bf16(3, K)
    xd, gd = bf16_dev(x), bf16_dev(g)
    s_act = float(oracle.act_scale(x, g, wl.EPS))
    wq, sw = oracle.quant_weight(wl.weight_f32(3, 2 * I, K))
    wd, swd = u8_dev(wq), f32_dev(sw)
    w2, sw2 = oracle.quant_weight(wl.weight_f32(3, 5120, I, tensor=wl.T_DOWN_W))
    w2d, sw2d = u8_dev(w2), f32_dev(sw2)
    w_il, s_il = fp8.interleave_gate_up(wd, swd)
    xq = fp8.quant_rmsnorm(xd, gd, s_act, wl.EPS)
    gate, up = fp8.scaled_mm_merged(xq, wd, s_act, swd, [I, I])
    s_down = float(fp8.act_scale_silu_mul(gate, up).item())
    assert fp8.gate_up_silu_quant_fused(M, I, K, s_act, s_down, 2)
    hq_e = fp8.gate_up_silu_quant(w_il, s_il, s_act, s_down, x=xd, gamma=gd, eps=wl.EPS)
    out_e = fp8.scaled_mm(hq_e, w2d, s_down, sw2d)
    want_h, want_o = host_u8(hq_e), host_u16(out_e)
    hq_g, out_g = torch.empty_like(hq_e), torch.empty_like(out_e)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        fp8.gate_up_silu_quant(w_il, s_il, s_act, s_down, x=xd, gamma=gd, eps=wl.EPS, out=hq_g)
        fp8.scaled_mm(hq_g, w2d, s_down, sw2d, out=out_g)
    torch.cuda.current_stream().wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fp8.gate_up_silu_quant(w_il, s_il, s_act, s_down, x=xd, gamma=gd, eps=wl.EPS, out=hq_g)
        fp8.scaled_mm(hq_g, w2d, s_down, sw2d, out=out_g)
    for i in range(4):
        hq_g.fill_(0)
        out_g.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_u8(hq_g), want_h), f"replay {i}: h_q"
        assert np.array_equal(host_u16(out_g), want_o), f"replay {i}: down output"
        _ = fp8.gate_up_silu_quant(w_il, s_il, s_act, s_down, x_q=xq)   # eager work between replays
        torch.cuda.synchronize()
