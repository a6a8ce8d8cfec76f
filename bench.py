"""Benchmark of the FP8 E4M3 W8A8 scaled-matmul layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--M 8] [--no-prefill] [--no-cpu-baseline]

Prints ONE JSON line.  The headline (`value`) is the decode projection: a step
is one pass of the layer's decode path over one batch -- static quant of the
bf16 activation [M, 5120] to E4M3, then the scaled GEMM against a 10240 x 5120
E4M3 weight with per-channel scales, bf16 output, the kernel picked by the
M-threshold dispatcher (the small-M arm at M <= 8).  `value` is algorithmic HBM
bytes per step / step time, in GB/s (inputs resident in HBM; weight copies are
rotated so that no step finds its weight in the 256 MB last-level cache).

`prefill` reports the prefill chunk (M = 6576: fused RMSNorm->quant, merged
gate_up 34816 x 5120, plain quant of the down input, down 5120 x 17408, large-M
arm) in TFLOP/s.  `roofline` objects use each path's dominant kernel timed with
HIP events around every launch in the timed region.  `cpu_baseline` is the CPU
oracle timed on a bounded sample of the same workload.

Inputs are seeded synthetic tensors from workloads/ (no datasets, no weights).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 scaled-MM: HBM GB/s at M≤8 (decode), FP8 TFLOPS at prefill M, % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, published (no sparsity)
LLC_BYTES = 256 * 2 ** 20      # Infinity Cache to defeat


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--M", type=int, default=8)
    p.add_argument("--prefill-steps", type=int, default=20)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    return p.parse_args()


def bf16_dev(a_u16):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16).cuda()


def f32_dev(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


class Timer:
    """HIP events around individual launches on the current stream."""

    def __init__(self, n):
        import torch
        self.s = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        self.e = [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def mean_ms(self, n):
        return sum(self.s[i].elapsed_time(self.e[i]) for i in range(n)) / n


def bench_decode(fp8, M, steps, warmup):
    import numpy as np
    import torch
    import workloads as wl

    K, N = 5120, 10240
    x = wl.activation_bf16(wl.DECODE_PROJ.wid, M, K, outliers=True)
    w = wl.weight_f32(wl.DECODE_PROJ.wid, N, K)
    xd = bf16_dev(x)
    s_act = float(fp8.act_scale(xd).item())
    wq, sw = fp8.quant_weight(f32_dev(w))
    del w
    wbytes = N * K
    copies = max(2, -(-2 * LLC_BYTES // wbytes) + 1)          # > 512 MB of weights in rotation
    ws = [wq] + [wq.clone() for _ in range(copies - 1)]
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gemm_bytes = N * K + 4 * N + M * K + 2 * M * N
    quant_bytes = 2 * M * K + M * K
    assert fp8.select(M, N, K) == 0

    def step(i, timer=None):
        fp8.quant(xd, s_act, out=xq)
        if timer is not None:
            timer.s[i].record()
        fp8.scaled_mm(xq, ws[i % copies], s_act, sw, out=out)
        if timer is not None:
            timer.e[i].record()

    for i in range(warmup):
        step(i)
    timer = Timer(steps)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(i, timer)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    gemm_ms = timer.mean_ms(steps)
    step_bytes = gemm_bytes + quant_bytes
    achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
    return {
        "ms_per_step": ms,
        "value": step_bytes / (ms * 1e-3) / 1e9,
        "config": {"workload": f"decode_proj_M{M}_K{K}_N{N}", "M": M, "K": K, "N": N,
                   "weight_copies_rotated": copies, "step": "static quant [M,K] + scaled GEMM (small-M arm)",
                   "algorithmic_bytes_per_step": step_bytes},
        "roofline": {"bound": "hbm", "kernel": "k_gemm_small_m", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": gemm_bytes, "avg_launch_us": gemm_ms * 1e3},
    }


def bench_prefill(fp8, steps, warmup):
    import torch
    import workloads as wl

    M, K1, N1, K2, N2 = 6576, 5120, 34816, 17408, 5120
    wid = wl.PREFILL.wid
    x = wl.activation_bf16(wid, M, K1, outliers=False)
    g = wl.gamma_bf16(wid, K1)
    xdn = wl.activation_bf16(wid, M, K2, outliers=False, tensor=wl.T_DOWN_X)
    xd, gd, xdd = bf16_dev(x), bf16_dev(g), bf16_dev(xdn)
    s1 = float(fp8.act_scale(xd, gd, wl.EPS).item())
    s2 = float(fp8.act_scale(xdd).item())
    wq1, sw1 = fp8.quant_weight(f32_dev(wl.weight_f32(wid, N1, K1)))
    wq2, sw2 = fp8.quant_weight(f32_dev(wl.weight_f32(wid, N2, K2, tensor=wl.T_DOWN_W)))
    xq1 = torch.empty((M, K1), dtype=torch.uint8, device="cuda")
    xq2 = torch.empty((M, K2), dtype=torch.uint8, device="cuda")
    gate = torch.empty((M, N1 // 2), dtype=torch.bfloat16, device="cuda")
    up = torch.empty((M, N1 // 2), dtype=torch.bfloat16, device="cuda")
    down = torch.empty((M, N2), dtype=torch.bfloat16, device="cuda")
    assert fp8.select(M, N1, K1) == 1
    flops1, flops2 = 2 * M * N1 * K1, 2 * M * N2 * K2

    def step(i, t_gu=None, t_dn=None):
        fp8.quant_rmsnorm(xd, gd, s1, wl.EPS, out=xq1)
        if t_gu is not None:
            t_gu.s[i].record()
        fp8.scaled_mm_merged(xq1, wq1, s1, sw1, [N1 // 2, N1 // 2], outs=[gate, up])
        if t_gu is not None:
            t_gu.e[i].record()
        fp8.quant(xdd, s2, out=xq2)
        if t_dn is not None:
            t_dn.s[i].record()
        fp8.scaled_mm(xq2, wq2, s2, sw2, out=down)
        if t_dn is not None:
            t_dn.e[i].record()

    for i in range(warmup):
        step(i)
    t_gu, t_dn = Timer(steps), Timer(steps)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(i, t_gu, t_dn)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    gu_ms, dn_ms = t_gu.mean_ms(steps), t_dn.mean_ms(steps)
    ach = flops1 / (gu_ms * 1e-3) / 1e12
    return {
        "workload": f"prefill_M{M}_gateup_K{K1}_N{N1}_down_K{K2}_N{N2}",
        "value": (flops1 + flops2) / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "ms_per_step": ms,
        "step": "fused RMSNorm quant + merged gate_up GEMM + static quant + down GEMM (large-M arm)",
        "gemm_tflops": {"gate_up": ach, "down": flops2 / (dn_ms * 1e-3) / 1e12},
        "roofline": {"bound": "mfma", "kernel": "k_gemm_large_m (gate_up)", "achieved": ach,
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / FP8_PEAK_TFLOPS, "traffic": None,
                     "algorithmic_flops_per_launch": flops1, "avg_launch_us": gu_ms * 1e3},
    }


def cpu_baseline(M, seconds):
    """The CPU oracle (as it stands) on a bounded sample of the decode step:
    static quant of [M, 5120] + exact GEMM against the full 10240 x 5120 weight,
    repeated for about `seconds`; reported in the metric's unit (GB/s)."""
    import numpy as np
    import oracle
    import workloads as wl
    K, N = 5120, 10240
    x = wl.activation_bf16(wl.DECODE_PROJ.wid, M, K, outliers=True)
    wq, sw = oracle.quant_weight(wl.weight_f32(wl.DECODE_PROJ.wid, N, K))
    s = oracle.act_scale(x)
    reps, t0 = 0, time.perf_counter()
    while True:
        xq = oracle.quant_act(x, s)
        oracle.scaled_mm(xq, wq, s, sw)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    step_bytes = N * K + 4 * N + M * K + 2 * M * N + 3 * M * K
    return {"value": reps * step_bytes / el / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{reps} full decode steps (quant [{M},{K}] + GEMM vs the whole {N}x{K} weight) in {el:.1f} s"}


def main():
    a = _args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE {world}); "
              "this layer has no multi-GPU path to time", file=sys.stderr)
        sys.exit(2)
    import torch
    import fp8_w8a8_scaled_amd as fp8
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    torch.cuda.set_device(0)
    res = bench_decode(fp8, a.M, a.steps, a.warmup)
    line = {
        "metric": METRIC, "value": res["value"], "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic (seeded, workloads/)",
        "config": res["config"], "roofline": res["roofline"],
    }
    if not a.no_prefill:
        line["prefill"] = bench_prefill(fp8, a.prefill_steps, 3)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(a.M, a.cpu_seconds)
    line["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
