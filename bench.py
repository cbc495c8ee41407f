#!/usr/bin/env python3
"""Benchmark of the W8A8 post-training-quantized linear path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input,
on the hidden-4096 prefill workload (OPT-6.7B-sized MLP: fc1 W [16384,4096]
with X [4096,4096], fc2 W [4096,16384] with X [4096,16384], bf16, 1% outlier
channels x60).  For each of the two layers:

  1. column absmax over the 8 calibration batches (stored back to back as one
     [8*T, K] matrix; the column max of the stack is the running max over batches)
  2. column absmax of the weight (input channels)
  3. smoothing factors s (alpha)
  4. MinMax + SSZ int8 per-output-channel weight quantization with the fold
  5. per-token int8 quantization of the forward batch with the fold
  6. int8 GEMM with the fused dequantization

Inputs are resident in HBM before the timed region.  Kernels run on torch's
current stream; HIP events on that stream bracket every stage, giving
per-kernel durations.  Prints one JSON line.

--workload ssz_scale measures the weight quantization alone at model scale:
MinMax + SSZ over the 128 matrices of 32 hidden-4096 layers (QKV [12288,4096],
out [4096,4096], fc1 [16384,4096], fc2 [4096,16384], bf16, heavy-tailed rows),
back to back on one stream, once as symmetric int8, once as symmetric int4
and once as asymmetric int8; a step is the three passes over all matrices.

--workload mlp_static measures the hidden-4096 MLP block (fc1 -> ReLU -> fc2,
4096 tokens) with static activation scales from a moving average over the
calibration batches: static int8 quantization of the block input, fc1 GEMM
with ReLU writing fc2's int8 input in its epilogue (fc2's smoothing fold and
static scale), fc2 GEMM.  Beside it, the unfused chain: fc1 GEMM + ReLU to
fp32, per-token quantization of that intermediate, fc2 GEMM; and the
per-tensor weight quantization (weight absmax, scale, codes) beside SSZ.

--workload decode measures the decode configuration instead (16 tokens,
X [16,8192] against W [28672,8192]): the weight is calibrated and quantized
once, untimed; a step is the per-token quantization of the token batch and
the int8 GEMM with dequantization.  The int8 weight is rotated over three
copies so that it is read from HBM, not from the 256 MB last-level cache.

The default line also times the same step at alpha 0.8 (the other point of the smoothing sweep) and reports,
beside the oracle on the host cores, the oracle on one host thread on samples of the tiny, hidden-1024 and
decode configurations.

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--alpha 0.5] [--no-cpu-baseline]
                  [--workload opt67b|gpt345m|decode|ssz_scale|mlp_static]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_I8 = 5.0e15           # int8 dense MFMA ops/s
PEAK_ALU = 256 * 64 * 2.4e9  # VALU lane-ops/s: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz
# lane operations per element and pass of the SSZ search: the quotient w / S (the product with the reciprocal and
# its two-multiply-add correction), the rounding, the clamp, and the two sums (w q in fp64, q^2)
SSZ_OPS_PER_ELEM_PASS = 7
METRIC = "W8A8 GEMM TOPS + quant/SSZ GB/s at hidden 4096; % of INT8/HBM peak"


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--alpha", type=float, default=0.5)
    p.add_argument("--calib-batches", type=int, default=8)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle GEMM time of the CPU baseline")
    p.add_argument("--workload", choices=("opt67b", "gpt345m", "decode", "ssz_scale", "mlp_static"), default="opt67b")
    p.add_argument("--momentum", type=float, default=0.9, help="mlp_static: moving-average momentum")
    p.add_argument("--layers", type=int, default=32, help="ssz_scale workload: number of 4-matrix layers")
    p.add_argument("--alpha2", type=float, default=0.8, help="second smoothing strength timed (opt67b; <0: none)")
    p.add_argument("--oracle-single-thread", action="store_true",
                   help="only time the oracle on samples of the tiny, hidden-1024 and decode configurations and print "
                        "one JSON line (run by the default line in a child process with one OpenMP thread)")
    p.add_argument("--probe-clock", action="store_true",
                   help="only run the matrix-core clock probe (four kinds) and the hidden-4096 GEMMs on random and on "
                        "zero operands, and print one JSON line")
    p.add_argument("--copy-ref", action="store_true",
                   help="only run a plain 1 GiB device copy three times (reference for scaling the "
                        "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


def probe_clock():
    """The int8 matrix cores under the power limit: the probe's four kinds (shader clock and throughput with the
    operands random, zero, or read from LDS as the GEMM does), then the fc1 and fc2 GEMMs of the hidden-4096 step
    on random and on zero operands (same instructions and cycle count; the time ratio is the clock ratio)."""
    import torch

    import post_int8_quantization_amd as pq
    torch.cuda.set_device(0)
    out = {"probe": {}, "gemm": {}}
    for kind in ("mfma16_random", "mfma32_random", "mfma16_lds_random", "mfma16_zero"):
        for _ in range(3):  # the clock settles within a few launches
            pq.probe_mfma(kind, iters=4000)
        r = pq.probe_mfma(kind, iters=4000)
        out["probe"][kind] = {"us": round(r["us"], 1), "clock_GHz": round(r["clock_GHz"], 3),
                              "TOPS": round(r["TOPS"], 1), "frac_i8": round(r["TOPS"] * 1e12 / PEAK_I8, 3)}
    g = torch.Generator(device="cuda:0").manual_seed(7)
    for name, (M, N, K) in (("fc1", (4096, 16384, 4096)), ("fc2", (4096, 4096, 16384))):
        ts = torch.rand(M, device="cuda:0", generator=g) * 0.01
        cs = torch.rand(N, device="cuda:0", generator=g) * 0.001
        y = torch.empty(M, N, device="cuda:0")
        res = {}
        for data in ("random", "zero"):
            if data == "random":
                xq = torch.randint(-127, 128, (M, K), device="cuda:0", dtype=torch.int8, generator=g)
                wq = torch.randint(-127, 128, (N, K), device="cuda:0", dtype=torch.int8, generator=g)
            else:
                xq = torch.zeros(M, K, device="cuda:0", dtype=torch.int8)
                wq = torch.zeros(N, K, device="cuda:0", dtype=torch.int8)
            for _ in range(200):  # about 50 ms of back-to-back launches before timing
                pq.w8a8_gemm_dequant(xq, wq, ts, cs, y=y)
            t = []
            for _ in range(20):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                pq.w8a8_gemm_dequant(xq, wq, ts, cs, y=y)
                b.record()
                b.synchronize()
                t.append(a.elapsed_time(b) * 1e3)
            t.sort()
            med = t[len(t) // 2]
            res[data] = {"median_us": round(med, 1), "TOPS": round(2 * M * N * K / med / 1e6, 1)}
        res["time_ratio_random_over_zero"] = round(res["random"]["median_us"] / res["zero"]["median_us"], 3)
        out["gemm"][name] = res
    print(json.dumps(out), flush=True)


def copy_reference():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes": n, "repeats": 3}), flush=True)


def hbm_probe(torch, pq, nbytes=1 << 31, reps=5):
    """The measured HBM peak beside the datasheet's: the stream probe's plain streaming reads of `nbytes` (eight
    times the 256 MB last-level cache) and its copy of half of them, each the median of `reps` launches after two
    warm-up launches.  Rates in GB/s of bytes moved (a copy counts its reads and its writes)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty(nbytes // 2, dtype=torch.uint8, device="cuda:0")
    out = {}
    for kind, a, b in (("read", src, None), ("copy", src[: nbytes // 2], dst)):
        for _ in range(2):
            pq.probe_stream(kind, a, b)
        rates = sorted(pq.probe_stream(kind, a, b)["GBps"] for _ in range(reps))
        out[kind + "_GBps"] = rates[reps // 2]
    del src, dst
    out["bytes"] = nbytes
    return out


class Timer:
    """HIP events on the current stream around named stages."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []  # (name, start_event, end_event)

    def stage(self, name, fn):
        t = self.torch
        a = t.cuda.Event(enable_timing=True)
        b = t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.marks.append((name, a, b))

    def totals(self):
        out = {}
        for name, a, b in self.marks:
            ms, n = out.get(name, (0.0, 0))
            out[name] = (ms + a.elapsed_time(b), n + 1)
        return out

    def medians(self, steps):
        """Median over the steps of each stage's time per step (ms): a stage's launches within a step are
        summed, then the median is taken over steps."""
        per = {}
        for name, a, b in self.marks:
            per.setdefault(name, []).append(a.elapsed_time(b))
        out = {}
        for name, v in per.items():
            k = len(v) // steps  # launches per step
            sums = sorted(sum(v[i * k:(i + 1) * k]) for i in range(steps))
            out[name] = sums[len(sums) // 2] if len(sums) % 2 else 0.5 * (sums[len(sums) // 2 - 1] + sums[len(sums) // 2])
        return out


KERNEL_SOURCES = {"k_ssz": "ssz.hip", "k_ssz_asym": "ssz.hip", "k_gemm_pipe": "gemm.hip", "k_gemm_dec": "gemm.hip",
                  "k_gemm_dec_w": "gemm.hip",
                  "k_absmax_cols": "calib.hip", "k_tensor_scale": "calib.hip", "k_quant_tok": "quant.hip"}


def _code_only(text):
    """Source text without comments and blank space (the sources hold no // or /* inside string literals)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def valu_probe(pq):
    """The VALU probe's three kinds on two waves per SIMD (2048 one-wave blocks), each after one warm-up launch:
    the SSZ pass loop alone (element-passes per second) and plain fp32 / fp64 multiply-adds (per second), with the
    SIMD cycles per wave instruction group and the shader clock the probe read."""
    res = {}
    for kind, iters in (("ssz_loop", 2000), ("fma_f32", 8000), ("fma_f64", 8000)):
        pq.probe_valu(kind, iters=iters)
        r = pq.probe_valu(kind, iters=iters)
        res[kind] = {"lane_ops_per_s": r["lane_ops_per_s"], "simd_cycles_per_wave_op": r["simd_cycles_per_wave_op"],
                     "clock_GHz": r["clock_GHz"]}
    return res


def kernel_source_sha(kernel_tag):
    """Hash of the code a kernel is built from (its .hip file and the shared device header, comments and
    layout ignored), so a traffic record stays valid across comment edits and no longer once the code changes."""
    src = os.path.join(ROOT, "post_int8_quantization_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel_tag], "ptq_dev.hpp"):
        h.update(_code_only(open(os.path.join(src, f)).read()).encode())
    return h.hexdigest()[:16]


class _NoTimer:
    """Stage runner without events (for graph capture)."""

    @staticmethod
    def stage(name, fn):
        fn()


class _OnlyStage:
    """Stage runner that runs one named stage and skips the others (for per-stage graph capture)."""

    def __init__(self, name):
        self.name = name

    def stage(self, name, fn):
        if name == self.name:
            fn()


def graph_stage_ms(torch, step, names, steps, repeat=8):
    """Per-stage time from a graph that holds only that stage's launches (all layers, `repeat` times over,
    so that a replay is long next to the host's cost of launching it), replayed `steps` times: the kernels'
    own time without the host's launch gaps, which dominate eager timings of short kernels."""
    out = {}
    for nm in names:
        only = _OnlyStage(nm)

        def rep(_tm, only=only):
            for _ in range(repeat):
                step(only)

        ms = graph_step_ms(torch, rep, steps)
        out[nm] = None if ms is None else ms / repeat
    return out


def graph_step_ms(torch, step, steps):
    """The same step captured once in a HIP graph and replayed `steps` times: the step's time without
    per-launch host overhead (stage events are not captured).  None if capture is not possible."""
    try:
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            step(_NoTimer)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            step(_NoTimer)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    except RuntimeError:
        return None


def load_counters(kernel_tag, workload):
    """HBM traffic per launch measured with rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE) on this workload, from the
    committed summaries under profiles/, if they were taken on the kernel's current source (hash match);
    else None."""
    digest = kernel_source_sha(kernel_tag)
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*counters*.md"))):
        for m in re.finditer(r"traffic-record:\s*(\{.*\})", open(f).read()):
            rec = json.loads(m.group(1))
            if rec.get("kernel") == kernel_tag and rec.get("workload") == workload and \
                    rec.get("source_sha") == digest:
                return rec
    return None


def main():
    args = parse()
    if args.copy_ref:
        copy_reference()
        return
    if args.oracle_single_thread:
        oracle_single_thread()
        return
    if args.probe_clock:
        probe_clock()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); the path "
              "shards by token rows or weight rows with no collective on the hot path, and this benchmark measures "
              "the one-GPU share.", file=sys.stderr)
        sys.exit(2)

    if args.workload == "decode":
        decode(args)
        return
    if args.workload == "ssz_scale":
        ssz_scale(args)
        return
    if args.workload == "mlp_static":
        mlp_static(args)
        return

    import numpy as np
    import torch

    import post_int8_quantization_amd as pq
    import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    wl = args.workload  # opt67b (the default line) or gpt345m: the same step over the configuration's layers
    cases = synth.cases(wl)
    B = args.calib_batches

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    layers = []
    for c in cases:
        # the calibration set of a layer: its B batches stored back to back as one [B*T, K] matrix
        calib = torch.empty((B * c.T, c.K), dtype=torch.bfloat16, device=dev)
        for b in range(B):
            calib[b * c.T:(b + 1) * c.T] = up(c.x_batch(b))
        L = dict(case=c, calib=calib, x=up(c.x_batch(B)), w=up(c.w()))
        L["ax"] = torch.empty(c.K, dtype=torch.float32, device=dev)
        L["aw"] = torch.empty(c.K, dtype=torch.float32, device=dev)
        L["s"] = torch.empty(c.K, dtype=torch.float32, device=dev)
        L["S"] = torch.empty(c.N, dtype=torch.float32, device=dev)
        L["wq"] = torch.empty((c.N, c.K), dtype=torch.int8, device=dev)
        L["it"] = torch.empty(c.N, dtype=torch.int32, device=dev)
        L["mse"] = torch.empty(c.N, dtype=torch.float64, device=dev)
        L["xq"] = torch.empty((c.T, c.K), dtype=torch.int8, device=dev)
        L["d"] = torch.empty(c.T, dtype=torch.float32, device=dev)
        L["y"] = torch.empty((c.T, c.N), dtype=torch.float32, device=dev)
        layers.append(L)
    torch.cuda.synchronize()

    # every launch goes to the current stream (None), so the same step also captures into a graph
    alpha = [args.alpha]

    def step(tm):
        for L in layers:
            tm.stage("calib_x", lambda: pq.sq_absmax_calib(L["calib"], L["ax"], stream=None))
            tm.stage("calib_w", lambda: pq.sq_absmax_calib(L["w"], L["aw"], stream=None))
            tm.stage("smooth", lambda: pq.sq_smooth_factors(L["ax"], L["aw"], alpha[0], s=L["s"], stream=None))
            tm.stage("ssz", lambda: pq.ssz_weight_qparams(L["w"], L["s"], bits=8, scale=L["S"], wq=L["wq"],
                                                          iters=L["it"], mse=L["mse"], stream=None))
            tm.stage("quant", lambda: pq.quant_per_token_i8(L["x"], L["s"], xq=L["xq"], tok_scale=L["d"],
                                                            stream=None))
            tm.stage("gemm", lambda: pq.w8a8_gemm_dequant(L["xq"], L["wq"], L["d"], L["S"], y=L["y"],
                                                          stream=None))

    for _ in range(args.warmup):
        step(Timer(torch))
    torch.cuda.synchronize()

    tm = Timer(torch)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(tm)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    tot = tm.totals()
    med = tm.medians(args.steps)
    graph_ms = graph_step_ms(torch, step, args.steps)
    graph_stage = graph_stage_ms(torch, step, ("calib_x", "calib_w", "smooth", "ssz", "quant", "gemm"), args.steps)

    # algorithmic work per step
    it_mean = {}
    elem_passes = 0
    gemm_ops = calib_x_bytes = calib_w_bytes = ssz_bytes = quant_bytes = smooth_bytes = gemm_bytes = 0
    for L in layers:
        c = L["case"]
        its = L["it"].cpu().numpy().astype(np.int64)
        it_mean[c.name] = float(its.mean())
        elem_passes += int(c.K * (its + 1).sum())
        gemm_ops += 2 * c.T * c.N * c.K
        calib_x_bytes += B * c.T * c.K * 2 + c.K * 4
        calib_w_bytes += c.N * c.K * 2 + c.K * 4
        smooth_bytes += 3 * c.K * 4
        ssz_bytes += c.N * c.K * 2 + c.N * c.K + c.N * (4 + 4 + 8) + c.K * 4
        quant_bytes += c.T * c.K * 2 + c.T * c.K + c.T * 4 + c.K * 4
        gemm_bytes += c.T * c.K + c.N * c.K + 4 * c.T + 4 * c.N + 4 * c.T * c.N

    K = args.steps

    def sec(name):
        return tot[name][0] / 1e3 / K  # seconds per step

    gemm_s = sec("gemm")
    gemm_tops = gemm_ops / gemm_s / 1e12
    stages = {
        "calib_x": {"ms": sec("calib_x") * 1e3, "GB/s": calib_x_bytes / sec("calib_x") / 1e9,
                    "frac_hbm": calib_x_bytes / sec("calib_x") / PEAK_HBM, "launches_per_step": len(layers)},
        "calib_w": {"ms": sec("calib_w") * 1e3, "GB/s": calib_w_bytes / sec("calib_w") / 1e9,
                    "frac_hbm": calib_w_bytes / sec("calib_w") / PEAK_HBM},
        "smooth": {"ms": sec("smooth") * 1e3},
        "ssz": {"ms": sec("ssz") * 1e3, "GB/s": ssz_bytes / sec("ssz") / 1e9,
                "frac_hbm": ssz_bytes / sec("ssz") / PEAK_HBM, "mean_iters": it_mean,
                "element_passes": elem_passes,
                "frac_alu": SSZ_OPS_PER_ELEM_PASS * elem_passes / sec("ssz") / PEAK_ALU},
        "quant": {"ms": sec("quant") * 1e3, "GB/s": quant_bytes / sec("quant") / 1e9,
                  "frac_hbm": quant_bytes / sec("quant") / PEAK_HBM},
        "gemm": {"ms": gemm_s * 1e3, "TOPS": gemm_tops, "frac_i8": gemm_ops / gemm_s / PEAK_I8},
    }
    for nm in stages:
        stages[nm]["ms_median"] = med[nm]
    stages["gemm"]["TOPS_median"] = gemm_ops / (med["gemm"] / 1e3) / 1e12
    stages["ssz"]["frac_alu_median"] = SSZ_OPS_PER_ELEM_PASS * elem_passes / (med["ssz"] / 1e3) / PEAK_ALU
    stage_bytes = {"calib_x": calib_x_bytes, "calib_w": calib_w_bytes, "quant": quant_bytes}
    for nm, g in graph_stage.items():
        stages[nm]["graph_ms"] = g
        if g and nm in stage_bytes:
            stages[nm]["graph_GB/s"] = stage_bytes[nm] / (g / 1e3) / 1e9
            stages[nm]["graph_frac_hbm"] = stage_bytes[nm] / (g / 1e3) / PEAK_HBM
    if graph_stage.get("gemm"):
        stages["gemm"]["graph_TOPS"] = gemm_ops / (graph_stage["gemm"] / 1e3) / 1e12
        stages["gemm"]["graph_frac_i8"] = gemm_ops / (graph_stage["gemm"] / 1e3) / PEAK_I8
    if graph_stage.get("ssz"):
        stages["ssz"]["graph_frac_alu"] = SSZ_OPS_PER_ELEM_PASS * elem_passes / (graph_stage["ssz"] / 1e3) / PEAK_ALU
    gpu_ms = sum(v[0] for v in tot.values()) / K

    # dominant kernel: the stage with the largest share of the step
    dom = max(("calib_x", "ssz", "quant", "gemm"), key=lambda n: tot[n][0])
    if dom == "gemm":
        launches = len(layers)
        roof = {"kernel": "k_gemm_pipe", "bound": "mfma", "achieved": gemm_ops / launches / (gemm_s / launches) / 1e12,
                "peak": PEAK_I8 / 1e12, "unit": "TOP/s", "per_launch_ops": gemm_ops / launches}
    elif dom == "ssz":
        roof = {"kernel": "k_ssz", "bound": "alu",
                "achieved": SSZ_OPS_PER_ELEM_PASS * elem_passes / sec("ssz") / 1e12,
                "peak": PEAK_ALU / 1e12, "unit": "Tlane-op/s"}
    elif dom == "calib_x":
        roof = {"kernel": "k_absmax_cols", "bound": "hbm", "achieved": calib_x_bytes / sec("calib_x") / 1e9,
                "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        roof = {"kernel": "k_quant_tok", "bound": "hbm", "achieved": quant_bytes / sec("quant") / 1e9,
                "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    rec = load_counters(roof["kernel"], wl)
    roof["traffic"] = None if rec is None else rec.get("traffic_bytes_per_launch")
    roof["avg_launch_us"] = tot[dom][0] * 1e3 / tot[dom][1]
    if wl == "opt67b":
        desc = ("opt67b-prefill hidden 4096: fc1 X[4096,4096] W[16384,4096], fc2 X[4096,16384] W[4096,16384], bf16, "
                "1 percent outlier channels x60")
    else:
        desc = (f"{wl}: " + ", ".join(f"{c.name.split('/')[-1]} X[{c.T},{c.K}] W[{c.N},{c.K}]" for c in cases) +
                ", bf16, 1 percent outlier channels x40")

    out = {
        "metric": METRIC, "value": gemm_tops, "unit": "TOPS", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"{desc}, {B} calibration batches, alpha {args.alpha:g}, int8 SSZ",
                   "tokens": cases[0].T, "hidden": cases[0].K, "calib_batches": B, "alpha": args.alpha, "bits": 8,
                   "parallelism": "single GPU"},
        "gpu_ms_per_step": gpu_ms, "step_tops": gemm_ops / (ms_per_step / 1e3) / 1e12,
        "graph_ms_per_step": graph_ms,
        "stages": stages, "roofline": roof,
    }
    if wl == "opt67b":
        # the matrix cores' throughput under the power limit, on the GEMM's instruction mix (after the timed region)
        probe = {}
        for kind in ("mfma16_random", "mfma16_lds_random"):
            for _ in range(3):
                pq.probe_mfma(kind, iters=4000)
            r = pq.probe_mfma(kind, iters=4000)
            probe[kind] = {"TOPS": r["TOPS"], "clock_GHz": r["clock_GHz"]}
        stages["gemm"]["mfma_probe"] = probe
        stages["gemm"]["frac_of_probe_lds"] = gemm_tops / probe["mfma16_lds_random"]["TOPS"]
    if wl == "opt67b" or dom == "ssz":
        # the vector ALUs on the SSZ search's own pass loop, without its reductions, decisions and memory traffic
        # (after the timed region): the rate its instruction mix reaches, beside the datasheet-derived peak
        vp = valu_probe(pq)
        loop = vp["ssz_loop"]["lane_ops_per_s"]  # element-passes per second
        stages["ssz"]["valu_probe"] = vp
        stages["ssz"]["loop_probe_frac_alu"] = SSZ_OPS_PER_ELEM_PASS * loop / PEAK_ALU
        stages["ssz"]["frac_of_loop_probe"] = elem_passes / sec("ssz") / loop
        if graph_stage.get("ssz"):
            stages["ssz"]["graph_frac_of_loop_probe"] = elem_passes / (graph_stage["ssz"] / 1e3) / loop
        if dom == "ssz":
            roof["measured_peak"] = SSZ_OPS_PER_ELEM_PASS * loop / 1e12
            roof["frac_of_measured_peak"] = roof["achieved"] / roof["measured_peak"]
    # the measured HBM peak (after the timed region): the memory-bound stages against it as well as the datasheet
    hp = hbm_probe(torch, pq)
    out["hbm_probe"] = hp
    for nm in ("calib_x", "calib_w"):
        stages[nm]["frac_of_read_probe"] = stages[nm]["GB/s"] * 1e9 / (hp["read_GBps"] * 1e9)
        if stages[nm].get("graph_GB/s"):
            stages[nm]["graph_frac_of_read_probe"] = stages[nm]["graph_GB/s"] / hp["read_GBps"]
    # per-token quantization moves 2 bytes in for 1 out: held against the copy (1 in, 1 out)
    stages["quant"]["frac_of_copy_probe"] = stages["quant"]["GB/s"] / hp["copy_GBps"]
    if stages["quant"].get("graph_GB/s"):
        stages["quant"]["graph_frac_of_copy_probe"] = stages["quant"]["graph_GB/s"] / hp["copy_GBps"]
    if wl == "opt67b" and args.alpha2 >= 0:
        out["alpha_%g" % args.alpha2] = second_alpha(torch, np, step, layers, alpha, args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layers, args, synth)
        out["cpu_single_thread"] = single_thread_child()
    print(json.dumps(out), flush=True)


def second_alpha(torch, np, step, layers, alpha, args):
    """The same step at the second smoothing strength of the sweep (fewer steps): stage times (mean and
    median over the steps), SSZ steps and its VALU fraction, GEMM rate."""
    alpha[0] = args.alpha2
    step(Timer(torch))
    torch.cuda.synchronize()
    n = max(3, args.steps // 4)
    tm = Timer(torch)
    for _ in range(n):
        step(tm)
    torch.cuda.synchronize()
    alpha[0] = args.alpha
    tot, med = tm.totals(), tm.medians(n)
    passes = sum(int(L["case"].K * (L["it"].cpu().numpy().astype(np.int64) + 1).sum()) for L in layers)
    ops = sum(2 * L["case"].T * L["case"].N * L["case"].K for L in layers)
    out = {"steps": n, "gpu_ms_per_step": sum(v[0] for v in tot.values()) / n,
           "stages_ms": {k: v[0] / n for k, v in tot.items()}, "stages_ms_median": med,
           "ssz_mean_iters": {L["case"].name: float(L["it"].float().mean()) for L in layers},
           "ssz_frac_alu": SSZ_OPS_PER_ELEM_PASS * passes / (tot["ssz"][0] / n / 1e3) / PEAK_ALU,
           "gemm_TOPS": ops / (tot["gemm"][0] / n / 1e3) / 1e12}
    out["gemm_frac_i8"] = out["gemm_TOPS"] * 1e12 / PEAK_I8
    return out


def single_thread_child():
    """The oracle on one host thread (a child process with OMP_NUM_THREADS=1): see oracle_single_thread."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-single-thread"], env=env,
                       capture_output=True, text=True, timeout=600)
    for line in r.stdout.splitlines():
        if line.startswith("{"):
            return json.loads(line)
    return {"error": (r.stderr or r.stdout)[-400:]}


def oracle_single_thread():
    """The oracle on one host thread on samples of three configurations (seconds per sample; reported, not a
    target): the tiny layer whole (calibration, smoothing, SSZ, per-token quantization, GEMM, dequantization);
    the hidden-1024 QKV layer on 64 tokens and 64 weight rows (calibration over all 8 batches, all weight columns);
    the decode layer on its 16 tokens against 2048 weight rows (SSZ on 64 of them)."""
    import oracle
    import synth
    res = {"threads": oracle.num_threads()}

    def path(c, tok, rows, ssz_rows, batches):
        w = synth.widen(c.w())[:rows]
        xs = [synth.widen(c.x_batch(b, T=tok)) for b in range(batches)]
        xe = synth.widen(c.x_batch(c.eval_index(), T=tok))
        t = {}
        t0 = time.perf_counter()
        ax = None
        for xb in xs:
            ax = oracle.absmax_cols(xb, ax)
        aw = oracle.absmax_cols(w)
        sm = oracle.smooth_factors(ax, aw, 0.5)
        t["calib_smooth_s"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        q = oracle.ssz(w[:ssz_rows], sm, 8)
        t["ssz_s"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        xq, d = oracle.quant_per_token(xe, sm)
        t["quant_s"] = time.perf_counter() - t0
        wq = oracle.quant_per_token(w)[0] if rows > ssz_rows else q["q"]  # codes of the sampled rows for the GEMM
        t0 = time.perf_counter()
        acc = oracle.gemm_i8(xq, wq)
        oracle.dequant(acc, d, np.ones(rows, np.float32))
        t["gemm_dequant_s"] = time.perf_counter() - t0
        t["sample"] = {"tokens": tok, "weight_rows": rows, "ssz_rows": ssz_rows, "K": c.K, "calib_batches": batches}
        return t

    import numpy as np
    c1 = synth.cases("tiny")[0]
    res["tiny"] = path(c1, c1.T, c1.N, c1.N, 1)
    c2 = synth.cases("gpt345m")[0]
    res["gpt345m_qkv"] = path(c2, 64, 64, 64, c2.calib_batches)
    c3 = synth.cases("decode")[0]
    res["decode"] = path(c3, c3.T, 2048, 64, c3.calib_batches)
    print(json.dumps(res), flush=True)


def decode(args):
    import numpy as np
    import torch

    import post_int8_quantization_amd as pq
    import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    (c,) = synth.cases("decode")
    B = args.calib_batches

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    stream = torch.cuda.current_stream()
    w = up(c.w())
    ax = torch.empty(c.K, dtype=torch.float32, device=dev)
    for b in range(B):
        pq.sq_absmax_calib(up(c.x_batch(b)), ax, accumulate=b > 0, stream=stream)
    aw = torch.empty(c.K, dtype=torch.float32, device=dev)
    pq.sq_absmax_calib(w, aw, stream=stream)
    s = pq.sq_smooth_factors(ax, aw, args.alpha, stream=stream)
    S, wq0, _, _ = pq.ssz_weight_qparams(w, s, bits=8, stream=stream)
    del w
    wqs = [wq0] + [wq0.clone() for _ in range(2)]
    x = up(c.x_batch(B))
    xq = torch.empty((c.T, c.K), dtype=torch.int8, device=dev)
    d = torch.empty(c.T, dtype=torch.float32, device=dev)
    y = torch.empty((c.T, c.N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    # launches go to the current stream (None), so that the same steps also capture into a graph
    def step(tm, i):
        tm.stage("quant", lambda: pq.quant_per_token_i8(x, s, xq=xq, tok_scale=d, stream=None))
        tm.stage("gemm", lambda: pq.w8a8_gemm_dequant(xq, wqs[i % len(wqs)], d, S, y=y, stream=None))

    for i in range(args.warmup):
        step(Timer(torch), i)
    torch.cuda.synchronize()
    tm = Timer(torch)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(tm, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tot = tm.totals()
    K = args.steps
    # one replay = one step on each of the three weight copies
    graph_ms = graph_step_ms(torch, lambda t: [step(t, i) for i in range(len(wqs))], max(1, K // len(wqs)))
    graph_ms = None if graph_ms is None else graph_ms / len(wqs)

    def sec(name):
        return tot[name][0] / 1e3 / K

    # the GEMM kernel's own duration: a burst of back-to-back launches (over the three weight copies, so no
    # launch finds its weights in a cache) between two events on the launch stream -- the host stays ahead of
    # the GPU, so no host gap enters, unlike the per-stage events of the eager steps above
    burst = 30
    eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    eb0.record()
    for i in range(burst):
        pq.w8a8_gemm_dequant(xq, wqs[i % len(wqs)], d, S, y=y, stream=None)
    eb1.record()
    torch.cuda.synchronize()
    burst_s = eb0.elapsed_time(eb1) / 1e3 / burst

    gemm_ops = 2 * c.T * c.N * c.K
    gemm_bytes = c.T * c.K + c.N * c.K + 4 * c.T + 4 * c.N + 4 * c.T * c.N
    quant_bytes = c.T * c.K * 2 + c.T * c.K + c.T * 4 + c.K * 4
    gemm_s = sec("gemm")
    stages = {
        "quant": {"ms": sec("quant") * 1e3, "GB/s": quant_bytes / sec("quant") / 1e9,
                  "frac_hbm": quant_bytes / sec("quant") / PEAK_HBM},
        "gemm": {"ms": gemm_s * 1e3, "TOPS": gemm_ops / gemm_s / 1e12, "GB/s": gemm_bytes / gemm_s / 1e9,
                 "frac_hbm": gemm_bytes / gemm_s / PEAK_HBM, "burst_ms": burst_s * 1e3,
                 "burst_GB/s": gemm_bytes / burst_s / 1e9, "burst_frac_hbm": gemm_bytes / burst_s / PEAK_HBM},
    }
    roof = {"kernel": "k_gemm_dec_w", "bound": "hbm", "achieved": gemm_bytes / burst_s / 1e9, "peak": PEAK_HBM / 1e9,
            "unit": "GB/s", "per_launch_bytes": gemm_bytes,
            "timing": f"burst of {burst} back-to-back launches between two events (kernel time, no host gaps)"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    rec = load_counters("k_gemm_dec_w", "decode")
    roof["traffic"] = None if rec is None else rec.get("traffic_bytes_per_launch")
    roof["avg_launch_us"] = burst_s * 1e6
    roof["eager_stage_avg_us"] = tot["gemm"][0] * 1e3 / tot["gemm"][1]
    # the measured HBM peak beside the datasheet's: the weight stream against plain streaming reads
    hp = hbm_probe(torch, pq)
    roof["measured_peak"] = hp["read_GBps"]
    roof["frac_of_measured_peak"] = roof["achieved"] / hp["read_GBps"]
    out = {
        "metric": METRIC, "value": gemm_ops / gemm_s / 1e12, "unit": "TOPS", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / K, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": f"decode: X[{c.T},{c.K}] bf16 (0.5 percent outlier channels x60) against "
                               f"W[{c.N},{c.K}] int8 quantized once untimed; step = per-token quantization + "
                               "int8 GEMM with dequantization; weight rotated over 3 copies",
                   "tokens": c.T, "hidden": c.K, "out": c.N, "alpha": args.alpha, "bits": 8,
                   "parallelism": "single GPU"},
        "gpu_ms_per_step": sum(v[0] for v in tot.values()) / K, "graph_ms_per_step": graph_ms,
        "stages": stages, "roofline": roof, "hbm_probe": hp,
    }
    if not args.no_cpu_baseline:
        import oracle
        wh = synth.widen(c.w())
        p0 = time.perf_counter()
        axh = None
        for b in range(B):
            axh = oracle.absmax_cols(synth.widen(c.x_batch(b)), axh)
        sh = oracle.smooth_factors(axh, oracle.absmax_cols(wh), args.alpha)
        qh = oracle.ssz(wh, sh, 8)
        p1 = time.perf_counter()
        xe = synth.widen(c.x_batch(B))
        t0 = time.perf_counter()
        xqh, dh = oracle.quant_per_token(xe, sh)
        t1 = time.perf_counter()
        acc = oracle.gemm_i8(xqh, qh["q"])
        oracle.dequant(acc, dh, qh["S"])
        t2 = time.perf_counter()
        out["cpu_baseline"] = {"value": gemm_ops / (t2 - t1) / 1e12, "unit": "TOPS", "cores": oracle.num_threads(),
                               "kind": "oracle", "sample": "one whole step (16 tokens x all 28672 weight rows): "
                               "per-token quantization, then GEMM + dequantization (the value times the latter); "
                               "the weight's calibration and SSZ run first, untimed like on the GPU",
                               "quant_seconds": t1 - t0, "gemm_dequant_seconds": t2 - t1,
                               "untimed_prep_seconds": p1 - p0}
    print(json.dumps(out), flush=True)


def ssz_scale(args):
    import numpy as np
    import torch

    import post_int8_quantization_amd as pq
    import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cases = synth.cases("ssz_scale")[: 4 * args.layers]
    stream = torch.cuda.current_stream()
    mats = []
    for c in cases:
        a = c.w()
        mats.append((c, torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)))
        del a
    # outputs per matrix shape (overwritten layer after layer), per-row statistics per matrix
    outs = {}
    for c, _ in mats:
        if (c.N, c.K) not in outs:
            outs[(c.N, c.K)] = dict(
                S=torch.empty(c.N, dtype=torch.float32, device=dev), Z=torch.empty(c.N, dtype=torch.int32, device=dev),
                q8=torch.empty((c.N, c.K), dtype=torch.int8, device=dev),
                q4=torch.empty((c.N, c.K // 2), dtype=torch.uint8, device=dev),
                mse=torch.empty(c.N, dtype=torch.float64, device=dev))
    iters = {m: [torch.empty(c.N, dtype=torch.int32, device=dev) for c, _ in mats] for m in ("int8", "int4", "asym8")}
    torch.cuda.synchronize()

    def step(tm):
        for mode in ("int8", "int4", "asym8"):
            def run(mode=mode):
                for i, (c, w) in enumerate(mats):
                    o = outs[(c.N, c.K)]
                    if mode == "asym8":
                        pq.ssz_weight_qparams_asym(w, None, scale=o["S"], zero_point=o["Z"], wq=o["q8"],
                                                   iters=iters[mode][i], mse=o["mse"], stream=stream)
                    else:
                        bits = 8 if mode == "int8" else 4
                        pq.ssz_weight_qparams(w, None, bits=bits, scale=o["S"], wq=o["q8"] if bits == 8 else o["q4"],
                                              iters=iters[mode][i], mse=o["mse"], stream=stream)
            tm.stage(mode, run)

    for _ in range(args.warmup):
        step(Timer(torch))
    torch.cuda.synchronize()
    tm = Timer(torch)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(tm)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tot = tm.totals()
    K = args.steps
    elems = sum(c.N * c.K for c, _ in mats)
    rows = sum(c.N for c, _ in mats)
    stages = {}
    for mode in ("int8", "int4", "asym8"):
        sec = tot[mode][0] / 1e3 / K
        out_b = elems if mode != "int4" else elems // 2
        nbytes = 2 * elems + out_b + rows * (4 + 4 + 8 + (4 if mode == "asym8" else 0))
        its = np.concatenate([t.cpu().numpy() for t in iters[mode]]).astype(np.int64)
        passes = sum(int(c.K * (iters[mode][i].cpu().numpy().astype(np.int64) + 1).sum()) for i, (c, _) in
                     enumerate(mats))
        ops = (SSZ_OPS_PER_ELEM_PASS + (2 if mode == "asym8" else 0)) * passes
        stages[mode] = {"ms": sec * 1e3, "GB/s": nbytes / sec / 1e9, "frac_hbm": nbytes / sec / PEAK_HBM,
                        "mean_iters": float(its.mean()), "element_passes": passes,
                        "frac_alu": ops / sec / PEAK_ALU, "launches": len(mats)}
    v = stages["int8"]
    roof = {"kernel": "k_ssz", "bound": "alu",
            "achieved": SSZ_OPS_PER_ELEM_PASS * v["element_passes"] / (v["ms"] / 1e3) / 1e12,
            "peak": PEAK_ALU / 1e12, "unit": "Tlane-op/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    rec = load_counters("k_ssz", "ssz_scale")
    roof["traffic"] = None if rec is None else rec.get("traffic_bytes_per_launch")
    roof["avg_launch_us"] = v["ms"] * 1e3 / len(mats)
    vp = valu_probe(pq)
    roof["measured_peak"] = SSZ_OPS_PER_ELEM_PASS * vp["ssz_loop"]["lane_ops_per_s"] / 1e12
    roof["frac_of_measured_peak"] = roof["achieved"] / roof["measured_peak"]
    stages["int8"]["valu_probe"] = vp
    out = {
        "metric": METRIC, "value": v["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32+f64", "data": "synthetic",
        "config": {"workload": f"ssz_scale: MinMax + SSZ over {len(mats)} matrices ({args.layers} hidden-4096 layers "
                               "x QKV/out/fc1/fc2), bf16 N(0,0.02) x logU[0.05,1] with 0.1 percent entries x20, no "
                               "smoothing; value = symmetric int8 pass; int4 and asymmetric int8 in stages",
                   "elements": elems, "rows": rows, "parallelism": "single GPU"},
        "gpu_ms_per_step": sum(x[0] for x in tot.values()) / K, "stages": stages, "roofline": roof,
    }
    # beside the single-stream figure: the same symmetric int8 pass with the matrices dealt round-robin over 4
    # streams (each with its own outputs), whose launches overlap each other's last rows and the deferred-row
    # launches -- the tail the one-stream sequence pays per matrix
    ns = 4
    streams = [torch.cuda.Stream() for _ in range(ns)]
    souts = [{k: dict(S=torch.empty_like(v["S"]), q8=torch.empty_like(v["q8"]), mse=torch.empty_like(v["mse"]))
              for k, v in outs.items()} for _ in range(ns)]
    sit = [torch.empty(c.N, dtype=torch.int32, device=dev) for c, _ in mats]

    def run_streams():
        for st in streams:
            st.wait_stream(stream)
        for i, (c, w) in enumerate(mats):
            o = souts[i % ns][(c.N, c.K)]
            pq.ssz_weight_qparams(w, None, bits=8, scale=o["S"], wq=o["q8"], iters=sit[i], mse=o["mse"],
                                  stream=streams[i % ns])
        for st in streams:
            stream.wait_stream(st)

    run_streams()
    ms = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run_streams()
        e1.record(stream)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    ms = sorted(ms)[1]
    same = all(torch.equal(sit[i], iters["int8"][i]) for i in range(len(mats)))
    out["int8_4streams"] = {"ms": ms, "frac_alu": SSZ_OPS_PER_ELEM_PASS * v["element_passes"] / (ms / 1e3) / PEAK_ALU,
                            "iters_identical": same}
    del souts
    if not args.no_cpu_baseline:
        import oracle
        sample = [c for c, _ in mats[:16]]
        secs = 0.0
        nb = 0
        for c in sample:
            wh = synth.widen(c.w())
            t0 = time.perf_counter()
            oracle.ssz(wh, None, 8)
            secs += time.perf_counter() - t0
            nb += c.N * c.K * 3 + c.N * 16
        out["cpu_baseline"] = {"value": nb / secs / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
                               "kind": "oracle", "sample": f"symmetric int8 SSZ of the first {len(sample)} matrices "
                               "(4 layers), every row", "seconds": secs}
    print(json.dumps(out), flush=True)


def mlp_static(args):
    import numpy as np
    import torch

    import post_int8_quantization_amd as pq
    import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    c1, c2 = synth.cases("opt67b")
    B = args.calib_batches
    T = c1.T

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    # untimed calibration, as a deployment would do once
    w1, w2 = up(c1.w()), up(c2.w())
    xs = [up(c1.x_batch(b)) for b in range(B)]
    ax1 = None
    for b, xb in enumerate(xs):
        ax1 = pq.sq_absmax_calib(xb, ax1, accumulate=b > 0)
    aw1 = pq.sq_absmax_calib(w1)
    s1 = pq.sq_smooth_factors(ax1, aw1, args.alpha)
    st1 = torch.zeros(1, dtype=torch.float32, device=dev)
    for b, xb in enumerate(xs):
        _, d1, _ = pq.sq_act_scale_ema(pq.sq_absmax_calib(xb), s1, args.momentum, first=b == 0, state=st1)
    S1, wq1, _, _ = pq.ssz_weight_qparams(w1, s1, bits=8)
    hs = []
    for xb in xs:
        q, rsc = pq.quant_static_i8(xb[:256], d1, s1, "div")
        hs.append(pq.w8a8_gemm_fused(q, wq1, rsc, S1, act="relu", out="f32"))
    ax2 = None
    for b, h in enumerate(hs):
        ax2 = pq.sq_absmax_calib(h, ax2, accumulate=b > 0)
    aw2 = pq.sq_absmax_calib(w2)
    s2 = pq.sq_smooth_factors(ax2, aw2, args.alpha)
    st2 = torch.zeros(1, dtype=torch.float32, device=dev)
    for b, h in enumerate(hs):
        _, d2, _ = pq.sq_act_scale_ema(pq.sq_absmax_calib(h), s2, args.momentum, first=b == 0, state=st2)
    S2, wq2, _, _ = pq.ssz_weight_qparams(w2, s2, bits=8)
    del xs, hs
    x = up(c1.x_batch(B))
    xq1 = torch.empty((T, c1.K), dtype=torch.int8, device=dev)
    rs1 = torch.empty(T, dtype=torch.float32, device=dev)
    h8 = torch.empty((T, c1.N), dtype=torch.int8, device=dev)
    rs2 = torch.empty(T, dtype=torch.float32, device=dev)
    hf = torch.empty((T, c1.N), dtype=torch.float32, device=dev)
    y = torch.empty((T, c2.N), dtype=torch.float32, device=dev)
    dtok = torch.empty(T, dtype=torch.float32, device=dev)
    # per-tensor weight path buffers
    wpt = [dict(w=w1, q=torch.empty_like(wq1), ch=torch.empty(c1.N, dtype=torch.float32, device=dev), s=s1, c=c1),
           dict(w=w2, q=torch.empty_like(wq2), ch=torch.empty(c2.N, dtype=torch.float32, device=dev), s=s2, c=c2)]
    sc = torch.empty(1, dtype=torch.float32, device=dev)
    colw = torch.empty(max(c1.K, c2.K), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def fused(tm):
        tm.stage("quant_static", lambda: pq.quant_static_i8(x, d1, s1, "div", q=xq1, row_scale=rs1, stream=stream))
        tm.stage("fc1_relu_requant", lambda: pq.w8a8_gemm_fused(xq1, wq1, rs1, S1, act="relu", out="i8", next_s=s2,
                                                                  out_scale=d2, y=h8, stream=stream))
        tm.stage("fc2", lambda: pq.w8a8_gemm_dequant(h8, wq2, rs2, S2, y=y, stream=stream))

    def unfused(tm):
        tm.stage("u_quant_tok", lambda: pq.quant_per_token_i8(x, s1, xq=xq1, tok_scale=dtok, stream=stream))
        tm.stage("u_fc1_relu_f32", lambda: pq.w8a8_gemm_fused(xq1, wq1, dtok, S1, act="relu", out="f32", y=hf,
                                                                stream=stream))
        tm.stage("u_quant_tok_h", lambda: pq.quant_per_token_i8(hf, s2, xq=h8, tok_scale=rs2, stream=stream))
        tm.stage("u_fc2", lambda: pq.w8a8_gemm_dequant(h8, wq2, rs2, S2, y=y, stream=stream))

    def per_tensor(tm):
        for L in wpt:
            c = L["c"]
            def run(L=L, c=c):
                col = colw[: c.K]
                pq.sq_absmax_calib(L["w"], col, stream=stream)
                pq.weight_scale_per_tensor(col, L["s"], n=c.N, scale=sc, ch_scale=L["ch"], stream=stream)
                pq.quant_static_i8(L["w"], sc, L["s"], "mul", q=L["q"], want_row_scale=False, stream=stream)
            tm.stage("w_per_tensor", run)

    rs2.fill_(float(d2.item()))  # the static token scale of fc2's int8 input
    for fn in (fused, unfused, per_tensor):
        for _ in range(args.warmup):
            fn(Timer(torch))
    torch.cuda.synchronize()
    res = {}
    walls = {}
    for fn in (fused, unfused, per_tensor):
        tm = Timer(torch)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn(tm)
        torch.cuda.synchronize()
        walls[fn.__name__] = (time.perf_counter() - t0) * 1e3 / args.steps
        res.update(tm.totals())
    K = args.steps

    def ms(name):
        return res[name][0] / K

    ops = 2 * T * c1.N * c1.K + 2 * T * c2.N * c2.K
    fused_ms = ms("quant_static") + ms("fc1_relu_requant") + ms("fc2")
    unfused_ms = ms("u_quant_tok") + ms("u_fc1_relu_f32") + ms("u_quant_tok_h") + ms("u_fc2")
    wpt_bytes = sum(L["c"].N * L["c"].K * (2 + 2 + 1) + L["c"].N * 4 for L in wpt)
    stages = {k: {"ms": ms(k)} for k in res}
    stages["w_per_tensor"]["GB/s"] = wpt_bytes / (ms("w_per_tensor") / 1e3) / 1e9
    stages["w_per_tensor"]["frac_hbm"] = stages["w_per_tensor"]["GB/s"] * 1e9 / PEAK_HBM
    stages["w_per_tensor"]["note"] = "both weights: column absmax read + code pass read/write (5 B/elem)"
    fc1_ops = 2 * T * c1.N * c1.K
    roof = {"kernel": "k_gemm_pipe", "bound": "mfma", "achieved": fc1_ops / (ms("fc1_relu_requant") / 1e3) / 1e12,
            "peak": PEAK_I8 / 1e12, "unit": "TOP/s", "per_launch_ops": fc1_ops}
    roof["frac"] = roof["achieved"] / roof["peak"]
    rec = load_counters("k_gemm_pipe", "mlp_static")
    roof["traffic"] = None if rec is None else rec.get("traffic_bytes_per_launch")
    roof["avg_launch_us"] = ms("fc1_relu_requant") * 1e3
    out = {
        "metric": METRIC, "value": ops / (fused_ms / 1e3) / 1e12, "unit": "TOPS", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": walls["fused"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "mlp_static: hidden-4096 MLP block fc1 [16384,4096] -> ReLU -> fc2 [4096,16384] on "
                               f"{T} bf16 tokens, static activation scales (moving average, momentum "
                               f"{args.momentum:g}, {B} calibration batches), alpha {args.alpha:g}; value = fused "
                               "block GEMM TOPS (static input codes + fc1 GEMM/ReLU/int8 requant + fc2 GEMM)",
                   "tokens": T, "hidden": c1.K, "parallelism": "single GPU"},
        "fused_block_ms": fused_ms, "unfused_block_ms": unfused_ms, "fusion_saving": 1 - fused_ms / unfused_ms,
        "wall_ms": walls, "stages": stages, "roofline": roof,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(layers, args, synth):
    """The oracle (as it stands) on the host cores, on a bounded sample of the same workload: the whole
    path per layer over every weight row and a slice of the token rows (calibration over that slice of
    each calibration batch, SSZ over all rows, per-token quantization, GEMM and dequantization of the
    slice).  The slice is sized so the oracle GEMM takes about --cpu-seconds in total.  Reported in the
    metric's unit: int8 GEMM TOPS of the oracle."""
    import oracle
    probe_tok = 16
    plans = []
    for L in layers:
        c = L["case"]
        w = synth.widen(c.w())
        xe = synth.widen(c.x_batch(args.calib_batches, T=probe_tok))
        xq, _ = oracle.quant_per_token(xe)
        wq = oracle.quant_per_token(w)[0]  # any int8 codes of the right shape serve to time the GEMM
        g0 = time.perf_counter()
        oracle.gemm_i8(xq, wq)
        rate = 2 * probe_tok * c.N * c.K / (time.perf_counter() - g0)
        plans.append((L, w, rate))
    import numpy as np
    gemm_ops = 0
    gemm_s = path_s = 0.0
    detail = {}
    ssz_rows = 256
    for L, w, rate in plans:
        c = L["case"]
        tok = int(args.cpu_seconds / len(plans) * rate / (2 * c.N * c.K))
        tok = max(16, min(c.T, (tok // 16) * 16))
        xs = [synth.widen(c.x_batch(b, T=tok)) for b in range(args.calib_batches)]
        xe = synth.widen(c.x_batch(args.calib_batches, T=tok))
        t0 = time.perf_counter()
        ax = None
        for xb in xs:
            ax = oracle.absmax_cols(xb, ax)
        aw = oracle.absmax_cols(w)
        s = oracle.smooth_factors(ax, aw, args.alpha)
        t1 = time.perf_counter()
        # SSZ on a row sample (the oracle sums in binary128; all rows would take ~30 s on 16 cores); the
        # GEMM below takes codes of every row (any int8 codes of the right shape time the same)
        qs = oracle.ssz(w[:ssz_rows], s, 8)
        t2 = time.perf_counter()
        q = {"q": oracle.quant_per_token(w)[0], "S": np.ones(c.N, np.float32)}
        xq, d = oracle.quant_per_token(xe, s)
        t3 = time.perf_counter()
        acc = oracle.gemm_i8(xq, q["q"])
        t4 = time.perf_counter()
        oracle.dequant(acc, d, q["S"])
        t5 = time.perf_counter()
        gemm_ops += 2 * tok * c.N * c.K
        gemm_s += t4 - t3
        path_s += t5 - t0
        detail[c.name] = {"tokens": tok, "weight_rows": c.N, "calib_s": t1 - t0, "ssz_rows": ssz_rows,
                          "ssz_s": t2 - t1, "ssz_mean_iters": float(qs["iters"].mean()),
                          "ssz_s_all_rows_estimate": (t2 - t1) * c.N / ssz_rows,
                          "quant_s": t3 - t2, "gemm_s": t4 - t3, "dequant_s": t5 - t4}
    return {"value": gemm_ops / gemm_s / 1e12, "unit": "TOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "per layer: a slice of tokens (see detail) of each of the %d calibration batches and of the "
                      "forward batch against all weight rows (GEMM sized to ~%gs), SSZ on the first %d weight rows; "
                      "whole path timed" % (args.calib_batches, args.cpu_seconds, ssz_rows),
            "path_seconds": path_s, "detail": detail}


if __name__ == "__main__":
    main()
