"""Benchmark of the FP8 E4M3 W8A8 scaled-matmul layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--M 8] [--no-prefill] [--no-mlp] [--no-sweep] [--no-cpu-baseline] [--headline-only]

Prints ONE JSON line.  The headline (`value`) is the decode projection (M = 8,
K = 5120, N = 10240): a step is one pass of the layer's decode path over one
batch -- static quant of the bf16 activation [M, 5120] to E4M3 and the scaled
GEMM against a 10240 x 5120 E4M3 weight with per-channel scales and a bf16
output, the kernel picked by the M-threshold dispatcher (the small-M arm), in
one launch (fp8_quant_scaled_mm_merged: the quant runs inside the GEMM kernel
and still writes x_q).
`value` is algorithmic bytes per step / step time in GB/s, with inputs resident
in HBM; weight copies are rotated so that no step finds its weight in the
256 MB Infinity Cache.  Steps are captured into a HIP graph of K steps and the
graph is replayed; every time is the median over 10 timed replays (HIP events
on the replay stream), per step.

`roofline` is for the step's kernel (the small-M GEMM with the quant inside:
the step is one launch): algorithmic bytes per launch over its median launch
duration in the graph of K back-to-back steps on the same stream.  The GEMM
alone (x_q given) is reported beside it.  `traffic` comes from a rocprofv3
FETCH_SIZE / WRITE_SIZE summary committed under profiles/ (null if absent or if
the kernel sources changed since it was taken).  `configs` holds every workload: the tiny
case (1), the decode projection at M = 1, 2, 4, 8 (2) and the decode MLP step
at M = 1, 4, 8, 16, 32 (3), each with GB/s and the fraction of the 8 TB/s
peak.  `prefill` reports the prefill chunk (config 5, M = 6576: fused
RMSNorm->quant, merged gate_up 34816 x 5120, fused SiLU*mul quant, down
5120 x 17408 -- the large-M arm) in TFLOP/s, with its own roofline for the
gate_up GEMM and the MFMA counters of a committed summary.  `decode_step_sweep`
is config 4.  `cpu_baseline` is the CPU oracle on the headline workload, all
threads and one thread.

Inputs are seeded synthetic tensors from workloads/ (no datasets, no weights).

Other modes:
    python bench.py --summarize-trace DIR --name NAME --cmd "..."   # kernel-trace stats -> profiles/NAME.md
    python bench.py --summarize-pmc DIR --name NAME --cmd "..."     # FETCH/WRITE_SIZE -> profiles/NAME.md
    python bench.py --summarize-mfma DIR --name NAME --cmd "..."    # MFMA counters -> profiles/NAME.md
    python bench.py --pmc-driver WHICH --meta-out DIR               # the launches a --pmc pass profiles (GPU)
    python bench.py --cpu-table NAME --cmd "..."                    # the oracle on every workload (CPU only)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 scaled-MM: HBM GB/s at M≤8 (decode), FP8 TFLOPS at prefill M, % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
REPLAYS = 10          # further timed replays of the roofline kernels' graphs (median and min reported)
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, published (no sparsity)
LLC_BYTES = 256 * 2 ** 20      # Infinity Cache to defeat
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "fp8_w8a8_scaled_amd", "csrc")


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=240)
    p.add_argument("--warmup", type=int, default=20, help="untimed eager steps before the timed graph")
    p.add_argument("--M", type=int, default=8)
    p.add_argument("--prefill-steps", type=int, default=10)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-sweep", action="store_true", help="skip the 64-layer decode-step weight sweep")
    p.add_argument("--no-mlp", action="store_true", help="skip the decode-MLP entries")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--headline-only", action="store_true",
                   help="only the headline decode workload at --M (for a kernel trace of just its launches)")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--summarize-trace", metavar="DIR")
    p.add_argument("--summarize-pmc", metavar="DIR")
    p.add_argument("--summarize-mfma", metavar="DIR")
    p.add_argument("--cpu-table", metavar="NAME", help="time the oracle on every workload -> profiles/NAME.md")
    p.add_argument("--sweep-threshold", metavar="NAME", help="time both GEMM arms over M -> profiles/NAME.md (GPU)")
    p.add_argument("--pmc-driver", choices=["decode", "prefill", "prefill_f32", "prefill_mfma"],
                   help="run a known-size copy, then a few launches of one GEMM (for rocprofv3 --pmc)")
    p.add_argument("--meta-out", metavar="DIR")
    p.add_argument("--name")
    p.add_argument("--cmd", default="")
    return p.parse_args()


# The sources each profiled kernel is compiled from (its own file and the
# shared device header); a traffic figure is valid only for these bytes.
# The source file each kernel (matched by name prefix) is compiled from; the
# headers it includes are followed from there.
KERNEL_SOURCES = {"k_gemm_small_m": "gemm_small_m.hip", "k_gemm_large_m": "gemm_large_m.hip",
                  "k_silu_mul_quant": "quant.hip"}


def kernel_files(kernel: str) -> list[str]:
    """The source `kernel` is built from, then every header it includes through
    quoted #include lines, transitively (paths relative to the kernel sources,
    sorted)."""
    key = next(k for k in KERNEL_SOURCES if kernel.startswith(k))
    root = KERNEL_SOURCES[key]
    seen, todo = set(), [root]
    while todo:
        rel = todo.pop()
        if rel in seen:
            continue
        seen.add(rel)
        base = os.path.dirname(rel)
        with open(os.path.join(CSRC, rel)) as fh:
            for line in fh:
                m = re.match(r'\s*#\s*include\s+"([^"]+)"', line)
                if m:
                    todo.append(os.path.normpath(os.path.join(base, m.group(1))))
    return [root] + sorted(seen - {root})


def kernel_sources_hash(kernel: str | None = None) -> str:
    """sha256 (16 hex digits) of every kernel source, or of the files `kernel`
    is built from (kernel_files)."""
    if kernel is None:
        files = sorted(glob.glob(os.path.join(CSRC, "*")))
    else:
        files = [os.path.join(CSRC, f) for f in kernel_files(kernel)]
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + fh.read())
    return h.hexdigest()[:16]


def bf16_dev(a_u16):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16).cuda()


def f32_dev(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def graph_time_ms(fn, n, warmup, replays=0):
    """Run `warmup` untimed eager calls of fn(i), capture n calls into one HIP
    graph, replay it once untimed, then time exactly one replay (n calls) with
    HIP events on the capture stream, bracketed by device synchronizations.
    Returns ms per call; with replays > 0 also the ms per call of that many
    further timed replays, as (first, [each])."""
    import torch
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in range(max(1, warmup)):
            fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    first = e0.elapsed_time(e1) / n
    if not replays:
        return first
    each = []
    for _ in range(replays):
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        each.append(e0.elapsed_time(e1) / n)
    return first, each


def timed(fn, n, warmup):
    """ms per call of fn: the median and minimum over REPLAYS timed replays of a
    graph of n calls (and the first timed replay)."""
    import statistics
    first, each = graph_time_ms(fn, n, warmup, replays=REPLAYS)
    return {"median_ms": statistics.median(each), "min_ms": min(each), "first_ms": first}


def _rate(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def replay_stats(each_ms):
    """Median and min (us per launch) over further graph replays."""
    import statistics
    return {"replays": len(each_ms), "median_us": statistics.median(each_ms) * 1e3, "min_us": min(each_ms) * 1e3}


def load_traffic(name: str, kernel: str):
    """Bytes per launch from a committed FETCH_SIZE/WRITE_SIZE summary, or None
    if it is missing or was taken from other sources of `kernel`."""
    path = os.path.join(PROFILES, f"{name}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_h or not m_b or m_h.group(1) != kernel_sources_hash(kernel):
        return None
    return float(m_b.group(1))


def load_mfma(name: str, kernel: str):
    """MFMA counters per launch from a committed summary (written by
    --summarize-mfma), or None if it is missing or was taken from other sources
    of `kernel`."""
    path = os.path.join(PROFILES, f"{name}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_j = re.search(r"```json\n(.*?)\n```", txt, re.S)
    if not m_h or not m_j or m_h.group(1) != kernel_sources_hash(kernel):
        return None
    return json.loads(m_j.group(1))


def bench_decode(fp8, M, steps, warmup):
    """Decode projection (config 2): a step is the static quant of the bf16
    activation [M, 5120] and the scaled GEMM against a 10240 x 5120 E4M3 weight
    through the dispatcher; the weight rotates through copies totalling more
    than twice the Infinity Cache.  Step and GEMM alone, median over REPLAYS
    graph replays."""
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

    def step(i):
        fp8.quant_scaled_mm(xd, s_act, ws[i % copies], sw, out=out, x_q=xq)

    def two_launches(i):
        fp8.quant(xd, s_act, out=xq)
        fp8.scaled_mm(xq, ws[i % copies], s_act, sw, out=out)

    def gemm(i):
        fp8.scaled_mm(xq, ws[i % copies], s_act, sw, out=out)

    st = timed(step, steps, warmup)
    st2 = timed(two_launches, steps, warmup)
    gt = timed(gemm, steps, warmup)
    one = bool(fp8.quant_scaled_mm_fused(M, N, K, K, s_act))
    # one launch reads x, writes x_q and never reads x_q back; two launches do
    two_bytes = gemm_bytes + quant_bytes
    step_bytes = two_bytes - M * K if one else two_bytes
    del ws
    torch.cuda.empty_cache()
    return {"workload": f"decode_proj_M{M}_K{K}_N{N}", "M": M, "K": K, "N": N, "weight_copies_rotated": copies,
            "step_us": st["median_ms"] * 1e3, "step_min_us": st["min_ms"] * 1e3, "step_one_launch": one,
            "step_GBs": _rate(step_bytes, st["median_ms"]), "step_frac": _rate(step_bytes, st["median_ms"]) / HBM_PEAK_GBS,
            "algorithmic_bytes_per_step": step_bytes,
            "two_launches_us": st2["median_ms"] * 1e3, "two_launches_GBs": _rate(two_bytes, st2["median_ms"]),
            "gemm_us": gt["median_ms"] * 1e3, "gemm_min_us": gt["min_ms"] * 1e3,
            "gemm_GBs": _rate(gemm_bytes, gt["median_ms"]), "gemm_frac": _rate(gemm_bytes, gt["median_ms"]) / HBM_PEAK_GBS,
            "algorithmic_bytes_per_gemm": gemm_bytes}


def bench_tiny(fp8, steps, warmup):
    """Config 1, M = 4, K = 256, N = 384: static quant + GEMM (through the
    one-launch entry, which takes two launches at this K).  About 100 KB of
    operands, resident in L2: the time is launch latency, not bandwidth."""
    import torch
    import workloads as wl
    M, K, N = 4, 256, 384
    xd = bf16_dev(wl.activation_bf16(wl.TINY.wid, M, K, outliers=False))
    s_act = float(fp8.act_scale(xd).item())
    wq, sw = fp8.quant_weight(f32_dev(wl.weight_f32(wl.TINY.wid, N, K)))
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step(i):
        fp8.quant_scaled_mm(xd, s_act, wq, sw, out=out, x_q=xq)

    st = timed(step, steps, warmup)
    gt = timed(lambda i: fp8.scaled_mm(xq, wq, s_act, sw, out=out), steps, warmup)
    step_bytes = N * K + 4 * N + M * K + 2 * M * N + 3 * M * K
    return {"workload": f"tiny_M{M}_K{K}_N{N}", "step_us": st["median_ms"] * 1e3,
            "step_GBs": _rate(step_bytes, st["median_ms"]), "gemm_us": gt["median_ms"] * 1e3,
            "algorithmic_bytes_per_step": step_bytes, "bound": "launch latency (L2-resident)"}


def bench_mlp(fp8, Ms, steps, warmup):
    """Decode MLP (config 3) at each M: fused RMSNorm quant [M, 5120] -> merged
    gate_up (34816 x 5120) -> SiLU*mul quant of the gate_up output -> down
    (5120 x 17408).  The step runs the gate_up launch with the SiLU*mul quant as
    its epilogue (interleaved weight; the RMSNorm quant in the same launch at
    M <= 8, else its own launch), then down; the separate calls (RMSNorm quant
    in the gate_up launch where it fits, two bf16 gate_up shards, SiLU*mul
    quant, down) are timed beside it.  Both weights rotate through 4 copies
    (1.07 GB per form), so no launch finds its weight in the Infinity Cache.
    Steps, gate_up alone and down alone, median over REPLAYS graph replays."""
    import torch
    import workloads as wl
    K1, N1, I, N2 = 5120, 34816, 17408, 5120
    wid = wl.DECODE_MLP.wid
    wq1, sw1 = fp8.quant_weight(f32_dev(wl.weight_f32(wid, N1, K1)))
    wq2, sw2 = fp8.quant_weight(f32_dev(wl.weight_f32(wid, N2, I, tensor=wl.T_DOWN_W)))
    copies = 4
    ws1 = [wq1] + [wq1.clone() for _ in range(copies - 1)]
    ws2 = [wq2] + [wq2.clone() for _ in range(copies - 1)]
    il1 = [fp8.interleave_gate_up(w, sw1) for w in ws1]
    gd = bf16_dev(wl.gamma_bf16(wid, K1))
    res = {}
    for M in Ms:
        xd = bf16_dev(wl.activation_bf16(wid, M, K1, outliers=True))
        s1 = float(fp8.act_scale(xd, gd, wl.EPS).item())
        xq1 = torch.empty((M, K1), dtype=torch.uint8, device="cuda")
        xq2 = torch.empty((M, I), dtype=torch.uint8, device="cuda")
        gate = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
        up = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
        down = torch.empty((M, N2), dtype=torch.bfloat16, device="cuda")
        fp8.quant_rmsnorm(xd, gd, s1, wl.EPS, out=xq1)
        fp8.scaled_mm_merged(xq1, wq1, s1, sw1, [I, I], outs=[gate, up])
        s2 = float(fp8.act_scale_silu_mul(gate, up).item())
        # 2: the RMSNorm quant in the gate_up + SiLU*mul launch; 0: that launch from x_q
        q_in = 2 if fp8.gate_up_silu_quant_fused(M, I, K1, s1, s2, 2) else 0
        fused = fp8.gate_up_silu_quant_fused(M, I, K1, s1, s2, q_in)

        def separate(i):
            # the RMSNorm quant inside the gate_up launch where the kernel takes the shape (M <= 8)
            fp8.quant_rmsnorm_scaled_mm_merged(xd, gd, s1, wl.EPS, ws1[i % copies], sw1, [I, I], outs=[gate, up],
                                               x_q=xq1)
            fp8.silu_mul_quant(gate, up, s2, out=xq2)
            fp8.scaled_mm(xq2, ws2[i % copies], s2, sw2, out=down)

        def step(i):
            w_il, s_il = il1[i % copies]
            if q_in == 2:
                fp8.gate_up_silu_quant(w_il, s_il, s1, s2, x=xd, gamma=gd, eps=wl.EPS, out=xq2)
            else:
                fp8.quant_rmsnorm(xd, gd, s1, wl.EPS, out=xq1)
                fp8.gate_up_silu_quant(w_il, s_il, s1, s2, x_q=xq1, out=xq2)
            fp8.scaled_mm(xq2, ws2[i % copies], s2, sw2, out=down)

        sep = timed(separate, steps, warmup)
        st = timed(step if fused else separate, steps, warmup)
        gu = timed(lambda i: fp8.scaled_mm_merged(xq1, ws1[i % copies], s1, sw1, [I, I], outs=[gate, up]),
                   steps, warmup)
        dn = timed(lambda i: fp8.scaled_mm(xq2, ws2[i % copies], s2, sw2, out=down), steps, warmup)
        gu_bytes = N1 * K1 + 4 * N1 + M * K1 + 2 * M * N1
        dn_bytes = N2 * I + 4 * N2 + M * I + 2 * M * N2
        one = fp8.quant_scaled_mm_fused(M, N1, K1, K1, s1, rmsnorm=True)
        # separate calls: one launch for the RMSNorm quant and gate_up never reads x_q back
        sep_bytes = (3 * M * K1 + 2 * K1) + gu_bytes - (M * K1 if one else 0) + 5 * M * I + dn_bytes
        if fused:
            # what each launch reads and writes once: x (or x_q) and gamma, the gate_up weight and scales, h_q;
            # then down (with x_q written and read back where the RMSNorm quant has its own launch)
            step_bytes = (2 * M * K1 + 2 * K1 + (2 * M * K1 if q_in == 0 else 0) + N1 * K1 + 4 * N1 + M * I +
                          dn_bytes)
            launches = 2 if q_in == 2 else 3
        else:
            step_bytes, launches = sep_bytes, 3 if one else 4
        res[f"M{M}"] = {
            "gate_up_silu_one_launch": bool(fused), "rmsnorm_quant_in_gate_up_launch": bool(q_in == 2 or one),
            "launches": launches,
            "step_us": st["median_ms"] * 1e3, "step_GBs": _rate(step_bytes, st["median_ms"]),
            "step_frac": _rate(step_bytes, st["median_ms"]) / HBM_PEAK_GBS, "algorithmic_bytes_per_step": step_bytes,
            "separate_calls_us": sep["median_ms"] * 1e3, "separate_calls_GBs": _rate(sep_bytes, sep["median_ms"]),
            "gate_up_us": gu["median_ms"] * 1e3, "gate_up_GBs": _rate(gu_bytes, gu["median_ms"]),
            "gate_up_frac": _rate(gu_bytes, gu["median_ms"]) / HBM_PEAK_GBS,
            "down_us": dn["median_ms"] * 1e3, "down_GBs": _rate(dn_bytes, dn["median_ms"]),
            "down_frac": _rate(dn_bytes, dn["median_ms"]) / HBM_PEAK_GBS,
            "arm": "small-M" if fp8.select(M, N1, K1) == 0 else "large-M"}
    del ws1, ws2, il1
    torch.cuda.empty_cache()
    return {"workload": "decode_mlp_gateup_K5120_N34816_down_K17408_N5120", "weight_copies_rotated": copies,
            "step": "gate_up with the SiLU*mul quant as its epilogue (fused RMSNorm quant in the launch at M <= 8) + "
                    "down, graph-replayed; the separate calls beside it", **res}


def bench_prefill(fp8, steps, warmup):
    import torch
    import workloads as wl

    M, K1, N1, K2, N2 = 6576, 5120, 34816, 17408, 5120
    wid = wl.PREFILL.wid
    x = wl.activation_bf16(wid, M, K1, outliers=False)
    g = wl.gamma_bf16(wid, K1)
    xd, gd = bf16_dev(x), bf16_dev(g)
    s1 = float(fp8.act_scale(xd, gd, wl.EPS).item())
    wq1, sw1 = fp8.quant_weight(f32_dev(wl.weight_f32(wid, N1, K1)))
    wq2, sw2 = fp8.quant_weight(f32_dev(wl.weight_f32(wid, N2, K2, tensor=wl.T_DOWN_W)))
    xq1 = torch.empty((M, K1), dtype=torch.uint8, device="cuda")
    xq2 = torch.empty((M, K2), dtype=torch.uint8, device="cuda")
    gate = torch.empty((M, N1 // 2), dtype=torch.bfloat16, device="cuda")
    up = torch.empty((M, N1 // 2), dtype=torch.bfloat16, device="cuda")
    down = torch.empty((M, N2), dtype=torch.bfloat16, device="cuda")
    assert fp8.select(M, N1, K1) == 1
    flops1, flops2 = 2 * M * N1 * K1, 2 * M * N2 * K2
    # the down projection's static scale, calibrated on this input's activation
    fp8.quant_rmsnorm(xd, gd, s1, wl.EPS, out=xq1)
    fp8.scaled_mm_merged(xq1, wq1, s1, sw1, [N1 // 2, N1 // 2], outs=[gate, up])
    s2 = float(fp8.act_scale_silu_mul(gate, up).item())

    def step(i):
        fp8.quant_rmsnorm(xd, gd, s1, wl.EPS, out=xq1)
        fp8.scaled_mm_merged(xq1, wq1, s1, sw1, [N1 // 2, N1 // 2], outs=[gate, up])
        fp8.silu_mul_quant(gate, up, s2, out=xq2)
        fp8.scaled_mm(xq2, wq2, s2, sw2, out=down)

    ms = timed(step, steps, warmup)["median_ms"]
    # The GEMMs alone: weight copies rotated past the Infinity Cache (2 x 178 MB
    # for gate_up, 3 x 89 MB for down), as inside the step, where the other
    # kernels' traffic evicts them; back-to-back launches of one weight would
    # find part of it cached.
    ws1 = [wq1, wq1.clone()]
    ws2 = [wq2, wq2.clone(), wq2.clone()]
    gu_ms, gu_each = graph_time_ms(lambda i: fp8.scaled_mm_merged(xq1, ws1[i % 2], s1, sw1, [N1 // 2, N1 // 2],
                                                                  outs=[gate, up]), steps, warmup, replays=REPLAYS)
    gu_ms = replay_stats(gu_each)["median_us"] * 1e-3
    dn_ms, dn_each = graph_time_ms(lambda i: fp8.scaled_mm(xq2, ws2[i % 3], s2, sw2, out=down), steps, warmup,
                                   replays=REPLAYS)
    dn_ms = replay_stats(dn_each)["median_us"] * 1e-3
    # A/B: the same merged gate_up launch with F32 outputs (twice the output bytes)
    gate32 = torch.empty((M, N1 // 2), dtype=torch.float32, device="cuda")
    up32 = torch.empty((M, N1 // 2), dtype=torch.float32, device="cuda")
    gu32_ms = timed(lambda i: fp8.scaled_mm_merged(xq1, ws1[i % 2], s1, sw1, [N1 // 2, N1 // 2],
                                                   outs=[gate32, up32]), steps, warmup)["median_ms"]
    del gate32, up32
    del ws1, ws2
    torch.cuda.empty_cache()
    sq_ms = timed(lambda i: fp8.silu_mul_quant(gate, up, s2, out=xq2), steps, warmup)["median_ms"]
    sq_bytes = 5 * M * K2
    # the step's fused RMSNorm quant alone, and the plain static quant of a bf16
    # [M, 17408] down-projection input (the gate half stands in for it)
    rq_ms = timed(lambda i: fp8.quant_rmsnorm(xd, gd, s1, wl.EPS, out=xq1), steps, warmup)["median_ms"]
    pq_ms = timed(lambda i: fp8.quant(gate, s2, out=xq2), steps, warmup)["median_ms"]
    ach = flops1 / (gu_ms * 1e-3) / 1e12
    return {
        "workload": f"prefill_M{M}_gateup_K{K1}_N{N1}_down_K{K2}_N{N2}",
        "value": (flops1 + flops2) / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "ms_per_step": ms,
        "step": "fused RMSNorm quant + merged gate_up GEMM + fused SiLU*mul quant + down GEMM (large-M arm), "
                "graph-replayed",
        "gemm_tflops": {"gate_up": ach, "down": flops2 / (dn_ms * 1e-3) / 1e12},
        "gemm_frac": {"gate_up": ach / FP8_PEAK_TFLOPS, "down": flops2 / (dn_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS},
        "gemm_us": {"gate_up": gu_ms * 1e3, "down": dn_ms * 1e3},
        "down_further_replays": replay_stats(dn_each),
        "silu_mul_quant": {"us": sq_ms * 1e3, "GBs": sq_bytes / (sq_ms * 1e-3) / 1e9},
        "quant_rmsnorm": {"us": rq_ms * 1e3, "GBs": (3 * M * K1 + 2 * K1) / (rq_ms * 1e-3) / 1e9},
        "plain_quant_M6576_K17408": {"us": pq_ms * 1e3, "GBs": 3 * M * K2 / (pq_ms * 1e-3) / 1e9},
        "f32_out_ab": {"gate_up_bf16_us": gu_ms * 1e3, "gate_up_f32_us": gu32_ms * 1e3,
                       "out_bytes_bf16": 2 * M * N1, "out_bytes_f32": 4 * M * N1,
                       "f32_over_bf16_time": gu32_ms / gu_ms,
                       "traffic_bf16": load_traffic("prefill_gateup_M6576_K5120_N34816_pmc", "k_gemm_large_m_tiled"),
                       "traffic_f32": load_traffic("prefill_gateup_f32out_M6576_K5120_N34816_pmc",
                                                   "k_gemm_large_m_tiled")},
        "roofline": {"bound": "mfma", "kernel": "k_gemm_large_m_tiled (gate_up)", "achieved": ach,
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / FP8_PEAK_TFLOPS,
                     "traffic": load_traffic("prefill_gateup_M6576_K5120_N34816_pmc", "k_gemm_large_m_tiled"),
                     "mfma_counters": load_mfma("prefill_mfma_M6576", "k_gemm_large_m_tiled"),
                     "algorithmic_flops_per_launch": flops1, "avg_launch_us": gu_ms * 1e3,
                     "further_replays": replay_stats(gu_each)},
    }


def bench_per_token(fp8, M, steps, warmup):
    """Per-token dynamic scales beside the per-tensor numbers: the decode step
    (per-token quant [M,5120] + GEMM 10240x5120 with per-row scales, weights
    rotated as in the main line) and the prefill gate_up (per-token fused
    RMSNorm quant [6576,5120] + merged gate_up with per-row scales)."""
    import torch
    import workloads as wl
    K, N = 5120, 10240
    xd = bf16_dev(wl.activation_bf16(wl.DECODE_PROJ.wid, M, K, outliers=True))
    wq, sw = fp8.quant_weight(f32_dev(wl.weight_f32(wl.DECODE_PROJ.wid, N, K)))
    copies = max(2, -(-2 * LLC_BYTES // (N * K)) + 1)
    ws = [wq] + [wq.clone() for _ in range(copies - 1)]
    xq, sr = fp8.quant_per_token(xd)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step(i):
        fp8.quant_per_token(xd, out=xq, scales=sr)
        fp8.scaled_mm_per_token(xq, ws[i % copies], sr, sw, out=out)

    ms = timed(step, steps, warmup)["median_ms"]
    gms = timed(lambda i: fp8.scaled_mm_per_token(xq, ws[i % copies], sr, sw, out=out), steps, warmup)["median_ms"]
    step_bytes = N * K + 4 * N + M * K + 2 * M * N + 3 * M * K + 4 * M
    del ws
    Mp, N1 = 6576, 34816
    wid = wl.PREFILL.wid
    xp = bf16_dev(wl.activation_bf16(wid, Mp, K, outliers=False))
    gp = bf16_dev(wl.gamma_bf16(wid, K))
    wq1, sw1 = fp8.quant_weight(f32_dev(wl.weight_f32(wid, N1, K)))
    xq1, sr1 = fp8.quant_per_token(xp, gp, wl.EPS)
    outs = [torch.empty((Mp, N1 // 2), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    pq_ms = graph_time_ms(lambda i: fp8.quant_per_token(xp, gp, wl.EPS, out=xq1, scales=sr1), 10, 2)
    pg_ms = graph_time_ms(lambda i: fp8.scaled_mm_merged_per_token(xq1, wq1, sr1, sw1, [N1 // 2, N1 // 2],
                                                                   outs=outs), 10, 2)
    return {"decode_step": {"workload": f"decode_proj_M{M}_K{K}_N{N}", "us": ms * 1e3,
                            "GBs": step_bytes / (ms * 1e-3) / 1e9, "gemm_us": gms * 1e3},
            "prefill": {"quant_rmsnorm_per_token_us": pq_ms * 1e3,
                        "gate_up_us": pg_ms * 1e3, "gate_up_TFLOPs": 2 * Mp * N1 * K / (pg_ms * 1e-3) / 1e12}}


def bench_merge_policies(fp8, M, steps, warmup):
    """Attention q/k/v (12288 | 1024 | 1024 rows, K=5120) whose shards carry
    per-tensor weight scales and mismatched static input scales, at decode M:
    the exact policy (merge declined: quant + GEMM per shard, 6 launches)
    against the max-scale policy (one quant at the largest input scale, weights
    requantized to the largest weight scale, one merged GEMM: 2 launches), with
    the accuracy the max-scale merge gives up, measured against the exact split
    outputs.  Weights rotate as in the main line."""
    import numpy as np
    import torch
    import workloads as wl
    shards, K = (12288, 1024, 1024), 5120
    x = wl.activation_bf16(4, M, K, outliers=True)
    xd = bf16_dev(x)
    s_cal = float(fp8.act_scale(xd).item())
    s_in = [float(np.float32(s_cal * f)) for f in (1.0, 1.5, 0.75)]
    wqs, sws = [], []
    for i, n in enumerate(shards):
        w = wl.weight_f32(4, n, K, tensor=wl.T_SHARD0 + i) * np.float32((1.0, 0.5, 2.0)[i])
        wq, s = fp8.quant_weight_per_tensor(f32_dev(w))
        wqs.append(wq)
        sws.append(float(s.item()))
    merge, _ = fp8.merge_admit(s_in, fp8.MERGE_EXACT)
    assert not merge
    _, s_mx = fp8.merge_admit(s_in, fp8.MERGE_MAX_SCALE)
    w_cat = torch.cat(wqs)
    w_mx, sw_mx, _ = fp8.requant_max_scale(w_cat, shards, sws)
    N = sum(shards)
    copies = max(2, -(-2 * LLC_BYTES // (N * K)) + 1)
    split_w = [[w] + [w.clone() for _ in range(copies - 1)] for w in wqs]
    split_sw = [torch.full((n,), s, dtype=torch.float32, device="cuda") for n, s in zip(shards, sws)]
    merged_w = [w_mx] + [w_mx.clone() for _ in range(copies - 1)]
    xq_s = [torch.empty((M, K), dtype=torch.uint8, device="cuda") for _ in shards]
    xq_m = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    out_s = [torch.empty((M, n), dtype=torch.bfloat16, device="cuda") for n in shards]
    out_m = [torch.empty((M, n), dtype=torch.bfloat16, device="cuda") for n in shards]

    def split(i):
        for j in range(len(shards)):
            fp8.quant(xd, s_in[j], out=xq_s[j])
            fp8.scaled_mm(xq_s[j], split_w[j][i % copies], s_in[j], split_sw[j], out=out_s[j])

    def merged(i):
        fp8.quant(xd, s_mx, out=xq_m)
        fp8.scaled_mm_merged(xq_m, merged_w[i % copies], s_mx, sw_mx, list(shards), outs=out_m)

    split_ms = timed(split, steps, warmup)["median_ms"]
    merged_ms = timed(merged, steps, warmup)["median_ms"]
    split(0)
    merged(0)
    torch.cuda.synchronize()
    ex = torch.cat(out_s, dim=1).float().cpu().numpy().astype(np.float64)
    mx = torch.cat(out_m, dim=1).float().cpu().numpy().astype(np.float64)
    row = np.sqrt((ex * ex).sum(axis=1, keepdims=True))
    rel = np.abs(mx - ex) / row
    wbytes = N * K
    return {"workload": f"attn_qkv_M{M}_K{K}_N{N}_shards_12288_1024_1024",
            "split_exact_us": split_ms * 1e3, "split_launches": 6,
            "merged_max_scale_us": merged_ms * 1e3, "merged_launches": 2,
            "split_over_merged_time": split_ms / merged_ms,
            "weight_GBs": {"split": wbytes / (split_ms * 1e-3) / 1e9, "merged": wbytes / (merged_ms * 1e-3) / 1e9},
            "max_scale_error_vs_exact": {"max_abs_over_row_norm": float(rel.max()),
                                         "mean_abs_over_row_norm": float(rel.mean())},
            "input_scales": s_in, "weight_scales": sws}


def bench_sweep(fp8, layers, M, steps, warmup, wid=4):
    """Decode-step weight sweep: `layers` = ((count, projections), ...).  The
    distinct projections of each layer group get their own seeded weights
    (quantized on the GPU); every other layer holds device copies, so a step
    streams count x bytes from HBM (far past the Infinity Cache).  A step is,
    per layer and projection, the static quant of its bf16 input (fused
    RMSNorm quant for the projections a norm feeds: qkv(z) and gate_up; the
    SiLU*mul quant of the gate_up output for down; the RMSNorm or plain quant
    inside the GEMM's launch where the small-M kernel takes the shape) and its
    GEMM, at M tokens.  A gate_up followed by down runs as one launch with the
    SiLU*mul quant as its epilogue (interleaved weight) where that launch
    takes the shape."""
    import torch
    import workloads as wl
    plan, step_bytes, gemm_bytes, launches = [], 0, 0, 0
    for gi, (count, projs) in enumerate(layers):
        srcs = []
        for pi, p in enumerate(projs):
            t = wl.T_LAYER0 + 16 * gi + pi
            norm = p.name.startswith(("qkv", "in_proj", "gate_up"))
            wq, sw = fp8.quant_weight(f32_dev(wl.weight_f32(wid, p.N, p.K, tensor=t)))
            xq = torch.empty((M, p.K), dtype=torch.uint8, device="cuda")
            outs = [torch.empty((M, n), dtype=torch.bfloat16, device="cuda") for n in (p.shards or (p.N,))]
            if p.name == "down":
                # input: SiLU*mul of the gate_up outputs just produced
                gu = srcs[-1]
                assert gu[0].name == "gate_up"
                fp8.quant_rmsnorm(gu[1], gu[2], gu[3], wl.EPS, out=gu[6])
                fp8.scaled_mm_merged(gu[6], gu[4], gu[3], gu[5], list(gu[0].shards), outs=gu[7])
                x, gam = tuple(gu[7]), None
                s = float(fp8.act_scale_silu_mul(*x).item())
            else:
                x = bf16_dev(wl.activation_bf16(wid, M, p.K, outliers=True, tensor=t))
                gam = bf16_dev(wl.gamma_bf16(wid, p.K)) if norm else None
                s = float((fp8.act_scale(x, gam, wl.EPS) if norm else fp8.act_scale(x)).item())
            srcs.append((p, x, gam, s, wq, sw, xq, outs))
        for li in range(count):
            fed = False                                  # the down input came from the gate_up launch
            for k, (p, x, gam, s, wq, sw, xq, outs) in enumerate(srcs):
                w = wq if li == 0 else wq.clone()
                silu = None
                if p.name == "gate_up" and k + 1 < len(srcs) and srcs[k + 1][0].name == "down":
                    dn = srcs[k + 1]
                    q_in = 2 if gam is not None else 1
                    if fp8.gate_up_silu_quant_fused(M, p.N // 2, p.K, s, dn[3], q_in):
                        w_il, s_il = fp8.interleave_gate_up(w, sw)
                        silu = (w_il, s_il, dn[3], dn[6])
                plan.append((p, x, gam, s, w, sw, xq, outs, silu))
                gemm_bytes += p.N * p.K + 4 * p.N + M * p.K + 2 * M * p.N
                if silu is not None:
                    # x (and gamma), the weight and scales, h_q written: one launch
                    step_bytes += p.N * p.K + 4 * p.N + 2 * M * p.K + (2 * p.K if gam is not None else 0) + \
                        M * (p.N // 2)
                    launches += 1
                    fed = True
                    continue
                if isinstance(x, tuple) and fed:
                    # the GEMM reads h_q
                    step_bytes += p.N * p.K + 4 * p.N + M * p.K + 2 * M * p.N
                    launches += 1
                    fed = False
                    continue
                qb = 5 * M * p.K if isinstance(x, tuple) else 3 * M * p.K + (2 * p.K if gam is not None else 0)
                one = not isinstance(x, tuple) and fp8.quant_scaled_mm_fused(M, p.N, p.K, p.K, s,
                                                                             rmsnorm=gam is not None)
                launches += 1 if one else 2
                # one launch never reads x_q back
                step_bytes += p.N * p.K + 4 * p.N + (0 if one else M * p.K) + 2 * M * p.N + qb
    torch.cuda.synchronize()

    def step(i):
        fed = False
        for (p, x, gam, s, wq, sw, xq, outs, silu) in plan:
            if silu is not None:                         # gate_up + SiLU*mul quant: down's input
                w_il, s_il, s_down, hq = silu
                fp8.gate_up_silu_quant(w_il, s_il, s, s_down, x=x, gamma=gam, eps=wl.EPS, out=hq)
                fed = True
                continue
            if isinstance(x, tuple):
                if not fed:
                    fp8.silu_mul_quant(x[0], x[1], s, out=xq)
                fed = False
            else:                                        # RMSNorm or plain quant: in the GEMM's launch where it fits
                fp8.quant_rmsnorm_scaled_mm_merged(x, gam, s, wl.EPS, wq, sw, list(p.shards or (p.N,)), outs=outs,
                                                   x_q=xq)
                continue
            if p.shards:
                fp8.scaled_mm_merged(xq, wq, s, sw, list(p.shards), outs=outs)
            else:
                fp8.scaled_mm(xq, wq, s, sw, out=outs[0])

    def gemms(i):
        for (p, x, gam, s, wq, sw, xq, outs, silu) in plan:
            if p.shards:
                fp8.scaled_mm_merged(xq, wq, s, sw, list(p.shards), outs=outs)
            else:
                fp8.scaled_mm(xq, wq, s, sw, out=outs[0])

    ms = timed(step, steps, warmup)["median_ms"]
    gms = timed(gemms, steps, warmup)["median_ms"]
    n_launch = len(plan)
    res = {"layers": sum(c for c, _ in layers), "launches_per_step": launches, "gemm_launches": n_launch,
           "gate_up_silu_launches": sum(1 for e in plan if e[8] is not None),
           "weight_bytes": sum(e[0].N * e[0].K for e in plan), "ms_per_step": ms,
           "value": step_bytes / (ms * 1e-3) / 1e9, "unit": "GB/s",
           "gemm_only": {"ms": gms, "GBs": gemm_bytes / (gms * 1e-3) / 1e9}}
    del plan
    torch.cuda.empty_cache()
    return res


def sweep_threshold(fp8, name, cmd, steps=40):
    """Both GEMM arms (forced) at M = 1 .. 128 on the decode-MLP shapes (gate_up
    34816 x 5120, down 5120 x 17408), weights rotated past the Infinity Cache,
    median of 10 graph replays; writes profiles/NAME.md with the crossover."""
    import torch
    import workloads as wl
    shapes = (("gate_up", 34816, 5120), ("down", 5120, 17408))
    Ms = (1, 2, 4, 8, 16, 24, 32, 40, 48, 64, 96, 128)
    rows = []
    for nm, N, K in shapes:
        wq, sw = fp8.quant_weight(f32_dev(wl.weight_f32(3, N, K)))
        copies = max(2, -(-2 * LLC_BYTES // (N * K)) + 1)
        ws = [wq] + [wq.clone() for _ in range(copies - 1)]
        for M in Ms:
            xq = fp8.quant(bf16_dev(wl.activation_bf16(3, M, K, outliers=True)), 0.05)
            out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            t = {}
            for arm in (0, 1):
                if arm == 0 and M > fp8.SMALL_M_MAX:
                    t[arm] = None
                    continue
                t[arm] = timed(lambda i: fp8.scaled_mm(xq, ws[i % copies], 0.05, sw, out=out, arm=arm), steps, 3)[
                    "median_ms"] * 1e3
            rows.append((nm, M, N, K, t[0], t[1]))
            print(f"threshold sweep {nm} M={M}: small {t[0]} large {t[1]}", flush=True)
        del ws
        torch.cuda.empty_cache()
    lines = [f"# {name}", "", "Both arms of the dispatcher, forced (`fp8_scaled_mm_arm`), on the decode-MLP shapes; "
             "weights rotated past the Infinity Cache; median of 10 replays of a graph of "
             f"{steps} launches, microseconds per launch.", "", f"Command: `{cmd}`", "",
             f"kernel_sources_sha256_16: {kernel_sources_hash()}", "",
             "| GEMM | M | small-M arm us | large-M arm us | faster |", "|---|---|---|---|---|"]
    for nm, M, N, K, a, b in rows:
        faster = "small" if a is not None and a <= b else "large"
        lines.append(f"| {nm} {N}x{K} | {M} | {'-' if a is None else f'{a:.2f}'} | {b:.2f} | {faster} |")
    out = os.path.join(PROFILES, f"{name}.md")
    os.makedirs(PROFILES, exist_ok=True)
    open(out, "w").write("\n".join(lines) + "\n")
    print(out, flush=True)


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_env():
    import oracle
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": _cpu_model(), "nproc": aff, "threads_all": oracle.num_threads()}


def _median_time(fn, reps=3):
    import statistics
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts)


def cpu_baseline(M, seconds):
    """The CPU oracle (as it stands) on the decode-step workload of the
    headline: static quant of [M, 5120] + exact GEMM against the whole
    10240 x 5120 weight, reported in the metric's unit (GB/s over the same
    algorithmic bytes).  Median of 3 timed runs, each of enough steps to take
    about seconds/6, with all the oracle's OpenMP threads and with one."""
    import oracle
    import workloads as wl
    K, N = 5120, 10240
    x = wl.activation_bf16(wl.DECODE_PROJ.wid, M, K, outliers=True)
    wq, sw = oracle.quant_weight(wl.weight_f32(wl.DECODE_PROJ.wid, N, K))
    s = oracle.act_scale(x)
    step_bytes = N * K + 4 * N + M * K + 2 * M * N + 3 * M * K
    env = _cpu_env()

    def one():
        xq = oracle.quant_act(x, s)
        oracle.scaled_mm(xq, wq, s, sw)

    res = {}
    for label, threads in (("all", env["threads_all"]), ("single", 1)):
        oracle.set_num_threads(threads)
        t1 = _median_time(one, 1)
        reps = max(1, int(seconds / 6 / max(t1, 1e-6)))
        t = _median_time(lambda: [one() for _ in range(reps)]) / reps
        res[label] = (step_bytes / t / 1e9, reps, threads)
    oracle.set_num_threads(env["threads_all"])
    return {"value": res["all"][0], "unit": "GB/s", "cores": res["all"][2], "kind": "oracle",
            "single_thread_value": res["single"][0],
            "sample": f"decode step (quant [{M},{K}] + exact GEMM vs the whole {N}x{K} weight), median of 3 runs of "
                      f"{res['all'][1]} steps on {res['all'][2]} threads and of {res['single'][1]} on 1 thread",
            **env}


def cpu_table(out_name, cmd):
    """The oracle on every workload, with one thread and with all, median of 3
    (writes profiles/<out_name>.md).  Rows are independent, so config 5 is
    timed on a row sample and scaled to 6576 rows; config 4 on one layer,
    scaled to 64."""
    import oracle
    import workloads as wl
    env = _cpu_env()
    rows = []

    def add(what, unit, work, fn, scale=1.0, note=""):
        for label, threads in (("1", 1), ("all", env["threads_all"])):
            oracle.set_num_threads(threads)
            t = _median_time(fn) * scale
            rows.append((what, label if label == "1" else str(threads), t * 1e3, work / t, unit, note))
            print(f"cpu table: {what} threads={threads} {t * 1e3:.1f} ms", flush=True)

    def gemm_case(wid, M, N, K, tensor_w=wl.T_W, tensor_x=wl.T_X, outl=True):
        x = wl.activation_bf16(wid, M, K, outliers=outl, tensor=tensor_x)
        wq, sw = oracle.quant_weight(wl.weight_f32(wid, N, K, tensor=tensor_w))
        s = oracle.act_scale(x)
        return x, wq, sw, s

    # 1, 2: quant + GEMM
    for wid, M, N, K in [(1, 4, 384, 256)] + [(2, m, 10240, 5120) for m in (1, 2, 4, 8)]:
        x, wq, sw, s = gemm_case(wid, M, N, K, outl=wid != 1)
        b = N * K + 4 * N + M * K + 2 * M * N + 3 * M * K
        add(f"config {wid} M={M} quant + GEMM {M}x{N}x{K}", "GB/s", b / 1e9,
            lambda: oracle.scaled_mm(oracle.quant_act(x, s), wq, s, sw))
    # 3: fused RMSNorm quant + gate_up + SiLU*mul quant + down
    wq1, sw1 = oracle.quant_weight(wl.weight_f32(3, 34816, 5120))
    wq2, sw2 = oracle.quant_weight(wl.weight_f32(3, 5120, 17408, tensor=wl.T_DOWN_W))
    g = wl.gamma_bf16(3, 5120)
    for M in wl.DECODE_MLP.Ms:
        x = wl.activation_bf16(3, M, 5120, outliers=True)
        s1 = oracle.act_scale(x, g, wl.EPS)
        gu = oracle.scaled_mm(oracle.quant_rmsnorm(x, g, wl.EPS, s1), wq1, s1, sw1)
        s2 = oracle.act_scale(oracle.silu_mul(gu[:, :17408], gu[:, 17408:]))

        def mlp(x=x, s1=s1, s2=s2):
            h = oracle.scaled_mm(oracle.quant_rmsnorm(x, g, wl.EPS, s1), wq1, s1, sw1)
            oracle.scaled_mm(oracle.silu_mul_quant(h[:, :17408], h[:, 17408:], s2), wq2, s2, sw2)

        b = (3 * M * 5120 + 2 * 5120) + (34816 * 5120 + 4 * 34816 + M * 5120 + 2 * M * 34816) + 5 * M * 17408 + \
            (5120 * 17408 + 4 * 5120 + M * 17408 + 2 * M * 5120)
        add(f"config 3 M={M} MLP step", "GB/s", b / 1e9, mlp)
    # 4: one layer of the 64-layer sweep at M = 8, scaled to 64 layers
    layer = []
    for pi, pr in enumerate(wl.DECODE_STEP_LAYER):
        layer.append(gemm_case(4, 8, pr.N, pr.K, tensor_w=wl.T_LAYER0 + pi, tensor_x=wl.T_LAYER0 + pi))
    b = sum(pr.N * pr.K + 4 * pr.N + 8 * pr.K + 2 * 8 * pr.N + 3 * 8 * pr.K for pr in wl.DECODE_STEP_LAYER) * 64
    add("config 4A 64 layers at M=8 (1 layer timed, x64)", "GB/s", b / 1e9,
        lambda: [oracle.scaled_mm(oracle.quant_act(x, s), wq, s, sw) for x, wq, sw, s in layer], scale=64.0,
        note="scaled")
    # 5: fused RMSNorm quant + gate_up, plain quant + down, at M = 6576: 16 rows
    # timed, scaled by 6576 / 16
    R = 16
    x5 = wl.activation_bf16(5, R, 5120, outliers=False)
    g5 = wl.gamma_bf16(5, 5120)
    s5 = oracle.act_scale(x5, g5, wl.EPS)
    wq5, sw5 = oracle.quant_weight(wl.weight_f32(5, 34816, 5120))
    xd5 = wl.activation_bf16(5, R, 17408, outliers=False, tensor=wl.T_DOWN_X)
    s6 = oracle.act_scale(xd5)
    wq6, sw6 = oracle.quant_weight(wl.weight_f32(5, 5120, 17408, tensor=wl.T_DOWN_W))
    fl = 2 * 6576 * (34816 * 5120 + 5120 * 17408)

    def prefill_rows():
        oracle.scaled_mm(oracle.quant_rmsnorm(x5, g5, wl.EPS, s5), wq5, s5, sw5)
        oracle.scaled_mm(oracle.quant_act(xd5, s6), wq6, s6, sw6)

    add(f"config 5 gate_up + down at M=6576 ({R} rows timed, x{6576 / R:g})", "GFLOP/s", fl / 1e9, prefill_rows,
        scale=6576 / R, note="extrapolated")
    oracle.set_num_threads(env["threads_all"])
    lines = [f"# {out_name}", "", "The CPU oracle (`oracle/fp8_oracle.c`, plain C with OpenMP over rows, fp64 exact "
             "accumulation) on every workload, median of 3 runs, with 1 thread and with all the threads it was given; "
             "rates over the same algorithmic bytes (GB/s) or flops (GFLOP/s) as the GPU figures.", "",
             f"Command: `{cmd}`", "", f"CPU: {env['cpu_model']}; CPUs available to the process: {env['nproc']}; "
             f"oracle threads: {env['threads_all']}", "",
             "| workload | threads | ms | rate | unit | note |", "|---|---|---|---|---|---|"]
    for w, th, ms, rate, unit, note in rows:
        lines.append(f"| {w} | {th} | {ms:.1f} | {rate:.3f} | {unit} | {note} |")
    out = os.path.join(PROFILES, f"{out_name}.md")
    os.makedirs(PROFILES, exist_ok=True)
    open(out, "w").write("\n".join(lines) + "\n")
    print(out, flush=True)


# ------------------------------------------------------- profile summaries --

def _short(name: str) -> str:
    name = name.replace("fp8mm::(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", name)


def summarize_trace(d, name, cmd):
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    assert files, f"no *kernel_stats.csv under {d}"
    rows = list(csv.DictReader(open(files[0])))
    lines = [f"# {name}", "", "rocprofv3 kernel trace, `--stats` summary (times in microseconds).", "",
             f"Command: `{cmd}`", "", f"kernel_sources_sha256_16: {kernel_sources_hash()}", "",
             "| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    # Runs: maximal sequences of back-to-back dispatches of one kernel (a graph
    # replay of n launches of one kernel is one run of n), so a shape-specific
    # average can be read next to the bench line's live per-launch figure.
    tfiles = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if tfiles:
        disp = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _short(r["Kernel_Name"]))
                       for r in csv.DictReader(open(tfiles[0]))), key=lambda x: x[0])
        runs = []
        for st, en, k in disp:
            if runs and runs[-1][0] == k:
                runs[-1][1].append(en - st)
            else:
                runs.append((k, [en - st]))
        lines += ["", "Runs of at least 8 back-to-back dispatches of one kernel, in launch order (a graph replay of "
                  "n launches of one kernel is one run of n; the bench replays each graph back to back, untimed then timed, "
                  "so such a run holds 2n, or 12n for the graphs of the roofline kernels, which get 10 further timed "
                  "replays):", "",
                  "| run | kernel | dispatches | avg us | min us | max us |", "|---|---|---|---|---|---|"]
        for i, (k, ds) in enumerate(runs):
            if len(ds) >= 8:
                lines.append(f"| {i} | {k} | {len(ds)} | {sum(ds) / len(ds) / 1e3:.2f} | {min(ds) / 1e3:.2f} | "
                             f"{max(ds) / 1e3:.2f} |")
    out = os.path.join(PROFILES, f"{name}.md")
    os.makedirs(PROFILES, exist_ok=True)
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


def summarize_pmc(d, name, cmd):
    """FETCH_SIZE / WRITE_SIZE per dispatch of the target kernel, scaled by the
    same counters on the plain copy that `--pmc-driver` runs first (an
    elementwise read-N-bytes / write-N-bytes kernel of known size)."""
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            per.setdefault((r["Counter_Name"], r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    meta = json.load(open(os.path.join(d, "pmc_meta.json")))
    copy_k = meta["copy_kernel"]
    target = meta["kernel"]
    res = {}
    for cname in ("FETCH_SIZE", "WRITE_SIZE"):
        tv = [v for (cn, kn), vals in per.items() if cn == cname and target in kn for v in vals]
        cv = [v for (cn, kn), vals in per.items() if cn == cname and copy_k in kn for v in vals]
        if not tv or not cv:
            raise SystemExit(f"missing {cname} samples for {target} or {copy_k}: {sorted(set(per))}")
        kib = sum(tv) / len(tv)
        copy_kib = max(cv)
        factor = meta["copy_bytes"] / (copy_kib * 1024.0)
        res[cname] = (kib, copy_kib, factor, kib * 1024.0 * factor, len(tv))
    traffic = res["FETCH_SIZE"][3] + res["WRITE_SIZE"][3]
    lines = [f"# {name}", "", "rocprofv3 `--pmc` (one counter per run): HBM traffic of one launch of "
             f"`{target}`, calibrated on a plain copy of {meta['copy_bytes']} bytes "
             f"(`{copy_k}`, read {meta['copy_bytes']} and written {meta['copy_bytes']}).", "",
             f"Commands: `{cmd}`", "", f"kernel_source_sha256_16: {kernel_sources_hash(target)} "
             f"({', '.join(kernel_files(target))})", "",
             "| counter | KiB per launch | copy KiB | scale = copy bytes / copy KiB·1024 | bytes per launch |",
             "|---|---|---|---|---|"]
    for cname, (kib, ck, fac, b, n) in res.items():
        lines.append(f"| {cname} | {kib:.1f} (mean of {n}) | {ck:.1f} | {fac:.4f} | {b:.0f} |")
    lines += ["", f"algorithmic_bytes_per_launch: {meta['algorithmic_bytes']}",
              f"traffic_bytes_per_launch: {traffic:.0f}",
              f"traffic / algorithmic: {traffic / meta['algorithmic_bytes']:.3f}"]
    out = os.path.join(PROFILES, f"{name}.md")
    os.makedirs(PROFILES, exist_ok=True)
    open(out, "w").write("\n".join(lines) + "\n")
    print(out)


def summarize_mfma(d, name, cmd):
    """MFMA counters of the prefill GEMM launches (one rocprofv3 --pmc pass of
    SQ_INSTS_VALU_MFMA_MOPS_F8, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, with
    the kernel trace): per GEMM, the executed FP8 flops (MOPS x 512) against
    the algorithmic 2 M N K, and rocprofv3's MfmaUtil normalisation, busy
    cycles summed over SIMDs / (GRBM_GUI_ACTIVE x SIMDs)."""
    meta = json.load(open(os.path.join(d, "pmc_meta.json")))
    target = meta["kernel"]
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if target not in r["Kernel_Name"]:
                continue
            vals.setdefault(int(r["Dispatch_Id"]), {}).setdefault(r["Counter_Name"], 0.0)
            vals[int(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
    durs = {}
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if target in r["Kernel_Name"]:
                durs[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    ids = sorted(vals)
    assert len(ids) == len(meta["order"]), (ids, meta["order"])
    # GRBM_GUI_ACTIVE comes back summed over the XCDs (one GRBM per XCD);
    # rocprofv3's MfmaUtil takes the largest instance, here the sum / Num_Xcc.
    xcc = 1
    for f in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Name", "").startswith("gfx"):
                xcc = int(r["Num_Xcc"])
    out = {}
    for gemm in ("gate_up", "down"):
        sel = [i for i, g in zip(ids, meta["order"]) if g == gemm]
        mean = {c: sum(vals[i][c] for i in sel) / len(sel) for c in vals[sel[0]]}
        flops = mean["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512
        gui = mean["GRBM_GUI_ACTIVE"] / xcc
        util = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * meta["simds"])
        rec = {"executed_over_algorithmic_flops": flops / meta["flops"][gemm], "mfma_busy_frac": util,
               "grbm_gui_active_cycles_per_xcd": gui}
        if "MfmaUtil" in mean:
            rec["rocprof_MfmaUtil_pct"] = mean["MfmaUtil"]
        if all(i in durs for i in sel):
            t = sum(durs[i] for i in sel) / len(sel)
            rec["profiled_launch_us"] = t * 1e6
            rec["gui_active_clock_GHz"] = gui / t / 1e9
        out[gemm] = rec
    lines = [f"# {name}", "", f"rocprofv3 `--pmc` counters of the prefill GEMM launches (`{target}`), 3 launches each "
             "of gate_up (M=6576, N=34816, K=5120) and down (M=6576, N=5120, K=17408), means per launch.", "",
             f"Command: `{cmd}`", "",
             f"kernel_source_sha256_16: {kernel_sources_hash(target)} "
             f"({', '.join(kernel_files(target))})", "",
             "Normalisation: executed FP8 flops = SQ_INSTS_VALU_MFMA_MOPS_F8 x 512 (the counter counts F8 add/mul ops "
             "/ 512), against 2 M N K; MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES (summed over the SIMDs) / "
             f"(GRBM_GUI_ACTIVE per XCD x {meta['simds']} SIMDs), rocprofv3's MfmaUtil; GRBM_GUI_ACTIVE is reported "
             f"summed over the {xcc} XCDs and is divided by {xcc}.  The GUI-active clock is GRBM_GUI_ACTIVE per XCD "
             "over the profiled launch duration (counter collection serializes launches, so the profiled launches "
             "run longer than in the bench).  Cross-check: 64 busy cycles per 32x32x64 FP8 MFMA at 2048 flops per "
             "SIMD cycle gives busy cycles = executed flops / 2048.", "",
             "| GEMM | executed / algorithmic flops | MFMA busy fraction | profiled launch us | GUI-active clock GHz |",
             "|---|---|---|---|---|"]
    for g, r in out.items():
        lines.append(f"| {g} | {r['executed_over_algorithmic_flops']:.4f} | {r['mfma_busy_frac']:.4f} | "
                     f"{r.get('profiled_launch_us', float('nan')):.1f} | {r.get('gui_active_clock_GHz', float('nan')):.3f} |")
    lines += ["", "```json", json.dumps(out), "```"]
    path = os.path.join(PROFILES, f"{name}.md")
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)


def pmc_driver(fp8, which, meta_dir):
    """Launches profiled by the FETCH_SIZE / WRITE_SIZE passes: first one
    elementwise kernel that reads 256 MiB and writes 256 MiB (the calibration
    copy: torch.neg on float32), then 3 launches of the decode step (the GEMM
    with the static quant inside, on 3 different weight copies, so each launch
    finds its weight cache-cold) or of the prefill gate_up GEMM, on the bench's
    inputs."""
    import torch
    import workloads as wl
    nbytes = 256 * 2 ** 20
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.neg(src)
    torch.cuda.synchronize()
    del dst
    if which == "decode":
        M, K, N = 8, 5120, 10240
        xd = bf16_dev(wl.activation_bf16(wl.DECODE_PROJ.wid, M, K, outliers=True))
        s_act = float(fp8.act_scale(xd).item())
        wq, sw = fp8.quant_weight(f32_dev(wl.weight_f32(wl.DECODE_PROJ.wid, N, K)))
        copies = [wq] + [wq.clone() for _ in range(11)]
        xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        for i in range(3):                          # the one-launch step: quant inside the GEMM
            fp8.quant_scaled_mm(xd, s_act, copies[4 * i + 1], sw, out=out, x_q=xq)
        kernel = "k_gemm_small_m_rx"
    elif which == "prefill_mfma":
        # the prefill gate_up and down GEMMs, 3 launches each, for the MFMA counters
        M, K, N, K2, N2 = 6576, 5120, 34816, 17408, 5120
        xd = bf16_dev(wl.activation_bf16(wl.PREFILL.wid, M, K, outliers=False))
        gd = bf16_dev(wl.gamma_bf16(wl.PREFILL.wid, K))
        s1 = float(fp8.act_scale(xd, gd, wl.EPS).item())
        wq, sw = fp8.quant_weight(f32_dev(wl.weight_f32(wl.PREFILL.wid, N, K)))
        wq2, sw2 = fp8.quant_weight(f32_dev(wl.weight_f32(wl.PREFILL.wid, N2, K2, tensor=wl.T_DOWN_W)))
        xq = fp8.quant_rmsnorm(xd, gd, s1, wl.EPS)
        outs = [torch.empty((M, N // 2), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        fp8.scaled_mm_merged(xq, wq, s1, sw, [N // 2, N // 2], outs=outs)
        s2 = float(fp8.act_scale_silu_mul(outs[0], outs[1]).item())
        xq2 = fp8.silu_mul_quant(outs[0], outs[1], s2)
        down = torch.empty((M, N2), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        for _ in range(3):
            fp8.scaled_mm_merged(xq, wq, s1, sw, [N // 2, N // 2], outs=outs)
        torch.cuda.synchronize()
        for _ in range(3):
            fp8.scaled_mm(xq2, wq2, s2, sw2, out=down)
        torch.cuda.synchronize()
        os.makedirs(meta_dir, exist_ok=True)
        json.dump({"kernel": "k_gemm_large_m_tiled", "order": ["gate_up"] * 4 + ["down"] * 3,
                   "flops": {"gate_up": 2 * M * N * K, "down": 2 * M * N2 * K2}, "simds": 4 * torch.cuda.get_device_properties(0).multi_processor_count},
                  open(os.path.join(meta_dir, "pmc_meta.json"), "w"))
        print("pmc driver done", which, flush=True)
        return
    else:
        M, K, N = 6576, 5120, 34816
        xd = bf16_dev(wl.activation_bf16(wl.PREFILL.wid, M, K, outliers=False))
        gd = bf16_dev(wl.gamma_bf16(wl.PREFILL.wid, K))
        s1 = float(fp8.act_scale(xd, gd, wl.EPS).item())
        wq, sw = fp8.quant_weight(f32_dev(wl.weight_f32(wl.PREFILL.wid, N, K)))
        xq = fp8.quant_rmsnorm(xd, gd, s1, wl.EPS)
        odt = torch.float32 if which == "prefill_f32" else torch.bfloat16
        outs = [torch.empty((M, N // 2), dtype=odt, device="cuda") for _ in range(2)]
        torch.cuda.synchronize()
        for _ in range(3):
            fp8.scaled_mm_merged(xq, wq, s1, sw, [N // 2, N // 2], outs=outs)
        kernel = "k_gemm_large_m_tiled"
    torch.cuda.synchronize()
    alg = N * K + 4 * N + M * K + (4 if which == "prefill_f32" else 2) * M * N
    if which == "decode":
        alg += 2 * M * K                            # x read as bf16, x_q written (and not read back)
    os.makedirs(meta_dir, exist_ok=True)
    json.dump({"kernel": kernel, "copy_kernel": "elementwise_kernel", "copy_bytes": nbytes, "algorithmic_bytes": alg},
              open(os.path.join(meta_dir, "pmc_meta.json"), "w"))
    print("pmc driver done", which, flush=True)


def main():
    a = _args()
    if a.summarize_trace:
        return summarize_trace(a.summarize_trace, a.name, a.cmd)
    if a.summarize_pmc:
        return summarize_pmc(a.summarize_pmc, a.name, a.cmd)
    if a.summarize_mfma:
        return summarize_mfma(a.summarize_mfma, a.name, a.cmd)
    if a.cpu_table:
        return cpu_table(a.cpu_table, a.cmd)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE {world}); "
              "this layer has no multi-GPU path to time", file=sys.stderr)
        sys.exit(2)
    import torch
    import fp8_w8a8_scaled_amd as fp8
    import workloads as wl
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    torch.cuda.set_device(0)
    if a.pmc_driver:
        return pmc_driver(fp8, a.pmc_driver, a.meta_out)
    if a.sweep_threshold:
        return sweep_threshold(fp8, a.sweep_threshold, a.cmd)
    Ms = [a.M] if a.headline_only else sorted(set(wl.DECODE_PROJ.Ms) | {a.M})
    decode = {M: bench_decode(fp8, M, a.steps, a.warmup) for M in Ms}
    head = decode[a.M]
    assert head["step_one_launch"], "the headline step is one launch at this shape"
    achieved = head["step_GBs"]
    line = {
        "metric": METRIC, "value": head["step_GBs"], "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": head["step_us"] * 1e-3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic (seeded, workloads/)",
        "config": {"workload": head["workload"], "M": a.M, "K": head["K"], "N": head["N"],
                   "weight_copies_rotated": head["weight_copies_rotated"],
                   "step": "static quant [M,K] + scaled GEMM via dispatcher (small-M arm), one launch, graph-replayed",
                   "timing": f"median over {REPLAYS} replays of a graph of {a.steps} steps",
                   "algorithmic_bytes_per_step": head["algorithmic_bytes_per_step"]},
        "roofline": {"bound": "hbm", "kernel": "k_gemm_small_m_rx (static quant inside)", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": load_traffic(f"decode_step_M{a.M}_K5120_N10240_pmc", "k_gemm_small_m_rx"),
                     "algorithmic_bytes_per_launch": head["algorithmic_bytes_per_step"], "avg_launch_us": head["step_us"],
                     "min_launch_us": head["step_min_us"],
                     "timing": f"median over {REPLAYS} replays of a graph of {a.steps} back-to-back launches",
                     "gemm_alone": {"avg_launch_us": head["gemm_us"], "achieved": head["gemm_GBs"],
                                    "frac": head["gemm_frac"],
                                    "algorithmic_bytes_per_launch": head["algorithmic_bytes_per_gemm"]}},
    }
    if a.headline_only:
        line["config"]["headline_only"] = True
        print(json.dumps(line), flush=True)
        return
    line["configs"] = {"1_tiny": bench_tiny(fp8, a.steps, a.warmup),
                       "2_decode_proj": {f"M{M}": r for M, r in decode.items()}}
    if not a.no_mlp:
        line["configs"]["3_decode_mlp"] = bench_mlp(fp8, wl.DECODE_MLP.Ms, a.steps, a.warmup)
    if not a.no_prefill:
        line["prefill"] = bench_prefill(fp8, a.prefill_steps, a.warmup)
        line["per_token_scales"] = bench_per_token(fp8, a.M, a.steps, a.warmup)
        line["merge_policies"] = bench_merge_policies(fp8, a.M, a.steps, a.warmup)
    if not a.no_sweep:
        line["decode_step_sweep"] = {
            "4A_64_layers": bench_sweep(fp8, ((wl.DECODE_STEP_LAYERS, wl.DECODE_STEP_LAYER),), a.M, 3, 1),
            "4B_pages_tower": bench_sweep(fp8, wl.DECODE_STEP_4B, a.M, 3, 1),
        }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(a.M, a.cpu_seconds)
    line["kernel_sources_sha256_16"] = kernel_sources_hash()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
