#!/usr/bin/env python3
"""Benchmark of the W4A16 symmetric-INT4 GPTQ linear on one MI355X.

Headline (``value``): HBM GB/s of the decode up-projection GEMV, M=1,
K=5120, N=17408, g=128 (one step = one w4a16_linear call over one batch).
The same line carries the prefill up-projection GEMM, M=2048, K=5120,
N=17408, g=128, in TFLOP/s under ``prefill``.

Timing: W untimed warm-up steps, then exactly K steps captured in one HIP
graph and replayed between HIP events on the launch stream, with a device
synchronisation on both sides.  Each step uses the next of R rotating
(qweight, scales) copies, R chosen so that the copies span at least twice
the 256 MB Infinity Cache, so every weight byte comes from HBM.

Algorithmic bytes per decode step: K*N/2 (codes) + 2*G*N (scales) + 2*M*K (x)
+ 2*M*N (y).  Algorithmic flops per prefill step: 2*M*N*K.

The CPU baseline times the oracle (plain C, fp64, OpenMP) on the host cores
on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
MALL_BYTES = 256 * 2 ** 20


def algorithmic_bytes(M, K, N, G):
    return K * N // 2 + 2 * G * N + 2 * M * K + 2 * M * N


# The sources each measured kernel is built and launched from: its own file
# (kernels and launch logic) and the shared device header.
KERNEL_SOURCES = {"decode": ("decode_gfx950.hip", "w4a16_device.hpp"),
                  "prefill": ("prefill_gfx950.hip", "w4a16_device.hpp")}


def kernel_sources_sha(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "int4_weight_only_w4a16_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha") != kernel_sources_sha(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


class Timed:
    def __init__(self, torch):
        self.torch = torch

    def graph_steps(self, fn, steps):
        """Capture `steps` calls of fn(i) in one graph; return (graph, stream)."""
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)                       # first call outside capture (arch cache, etc.)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                fn(i)
        torch.cuda.synchronize()
        return g, s

    def run(self, fn, steps, warmup, eager=False):
        """Warm up, then time exactly `steps` steps; returns seconds per step."""
        torch = self.torch
        if eager:
            for i in range(warmup):
                fn(i)
            torch.cuda.synchronize()
            st = torch.cuda.current_stream()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for i in range(steps):
                fn(i)
            e1.record(st)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / 1e3 / steps
        gw, sw = self.graph_steps(fn, max(1, warmup))
        gt, stt = self.graph_steps(fn, steps)
        with torch.cuda.stream(sw):
            gw.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stt):
            e0.record(stt)
            gt.replay()
            e1.record(stt)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / steps


def prepare(torch, w4, case, inp, rotations, bf16=False):
    dev = torch.device("cuda:0")
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    s = torch.from_numpy(inp.scales).to(dev)
    qs = [q] + [q.clone() for _ in range(rotations - 1)]
    ss = [s] + [s.clone() for _ in range(rotations - 1)]
    if bf16:   # bfloat16 bit patterns -> a bfloat16 tensor
        x = torch.from_numpy(inp.x.view("int16")).view(torch.bfloat16).to(dev)
    else:
        x = torch.from_numpy(inp.x).to(dev)
    y = torch.empty((case.M, case.N), dtype=x.dtype, device=dev)
    return x, qs, ss, y


def rotations_for(weight_bytes: int, minimum: int = 2) -> int:
    return max(minimum, -(-2 * MALL_BYTES // weight_bytes))


def bench_case(torch, w4, case, steps, warmup, eager, bf16=False, gate_up=False, lora_rank=0,
               zero_points=False):
    import workloads
    inp = workloads.generate_bf16(case) if bf16 else workloads.generate(case)
    wbytes = case.K * case.N // 2 + 2 * case.G * case.N
    R = rotations_for(wbytes)
    x, qs, ss, y = prepare(torch, w4, case, inp, R, bf16)
    if gate_up:
        y = y[:, : case.N // 2].contiguous()
        call = w4.w4a16_gate_up_silu_bf16 if bf16 else w4.w4a16_gate_up_silu
    else:
        call = w4.w4a16_linear_bf16 if bf16 else w4.w4a16_linear

    def step(i):
        call(x, qs[i % R], ss[i % R], y, case.M, case.K, case.N, case.group_size)

    if lora_rank:
        # the adapter rotates with the weights: each layer of a model has its own
        A, B = workloads.lora_adapter(case.K, case.N, lora_rank, case.seed + 500)
        As = [torch.from_numpy(A).to(x.device) for _ in range(R)]
        Bs = [torch.from_numpy(B).to(x.device) for _ in range(R)]
        wsb = w4.w4a16_lora_workspace_bytes(case.M, case.K, lora_rank)
        ws = torch.empty(wsb, dtype=torch.uint8, device=x.device)

        def step(i):  # noqa: F811
            w4.w4a16_linear_lora(x, qs[i % R], ss[i % R], As[i % R], Bs[i % R],
                                 workloads.LORA_SCALE, y, case.M, case.K, case.N,
                                 case.group_size, lora_rank, ws, wsb)

    if zero_points:
        # zero points rotate with the weights, like the scales they belong to
        qz = torch.from_numpy(w4.pack_zeros(workloads.zero_points(case.G, case.N, case.seed + 700)))
        qzs = [qz.to(x.device) for _ in range(R)]
        wsb = w4.w4a16_zp_workspace_bytes(case.M, case.K, case.N, case.group_size)
        ws = torch.empty(wsb, dtype=torch.uint8, device=x.device)

        def step(i):  # noqa: F811
            w4.w4a16_linear_zp(x, qs[i % R], ss[i % R], qzs[i % R], y, case.M, case.K, case.N,
                               case.group_size, ws, wsb)

    sec = Timed(torch).run(step, steps, warmup, eager)
    return inp, y, sec, R


def cpu_baseline_decode(case, inp, seconds):
    """Oracle on the full decode case, repeated for about `seconds` of host time."""
    import oracle
    import numpy as np
    q_o = oracle.pack(inp.codes)
    reps, t0 = 0, time.perf_counter()
    y_ref = None
    while True:
        y_ref = oracle.linear(inp.x, q_o, inp.scales, case.group_size)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    per = el / reps
    B = algorithmic_bytes(case.M, case.K, case.N, case.G)
    return {"value": B / per / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the whole decode case (M=1, K={case.K}, N={case.N}, g={case.group_size}),"
                      f" {reps} repetitions, {el:.1f} s, {per * 1e3:.1f} ms per call"}, y_ref


def cpu_baseline_prefill(case, inp, seconds):
    """Oracle on whole output rows of the prefill case (the rest is the same work)."""
    import numpy as np
    import oracle
    q_o = oracle.pack(inp.codes)
    rows, done, t0 = 0, 0, time.perf_counter()
    chunk = 8
    while True:
        ms = np.repeat(np.arange(rows, rows + chunk) % case.M, case.N)
        ns = np.tile(np.arange(case.N), chunk)
        oracle.linear_at(inp.x, q_o, inp.scales, case.group_size, ms, ns)
        rows += chunk
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    flops = 2.0 * rows * case.N * case.K
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{rows} whole output rows of the prefill case (of {case.M}), "
                      f"{el:.1f} s"}


def parity_summary(y_gpu, y_ref):
    import numpy as np
    d = np.abs(y_gpu.astype(np.float64) - y_ref)
    return {"max_abs": float(d.max()),
            "bound": float(5e-3 * np.abs(y_ref).max() + 1e-3),
            "mean_rel": float(d.sum() / np.abs(y_ref).sum())}


def read_ceiling(torch, w4, nbytes: int = 1 << 30, reps: int = 20) -> float:
    """Attainable HBM read rate (GB/s): the library's streaming-read probe over
    nbytes of device memory, timed with HIP events on the launch stream."""
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.current_stream()
    for _ in range(3):
        w4.w4a16_read_probe(buf, nbytes, sink, s)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        w4.w4a16_read_probe(buf, nbytes, sink, s)
    e1.record(s)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del buf, sink
    torch.cuda.empty_cache()
    return nbytes / sec / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=None,
                    help="steps for the prefill leg (default: steps // 4, at least 10)")
    ap.add_argument("--eager", action="store_true",
                    help="launch each step from the host instead of a graph (for profilers)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", choices=("all", "decode", "prefill"), default="all")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read ceiling measurement")
    ap.add_argument("--no-gate-up", action="store_true",
                    help="skip the merged gate/up (SiLU * mul) decode and prefill lines")
    ap.add_argument("--no-lora", action="store_true",
                    help="skip the linear + LoRA adapter lines")
    ap.add_argument("--no-zero-points", action="store_true",
                    help="skip the stored-zero-point (asymmetric weight) lines")
    ap.add_argument("--no-bf16", action="store_true",
                    help="skip the bfloat16-activation variant's decode and prefill lines")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (PMC calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import int4_weight_only_w4a16_amd as w4
    import workloads

    w4.load_library()
    dev_name = torch.cuda.get_device_name(0)
    out = {"metric": "W4A16 linear: HBM GB/s at M=1 (5120x17408 g128); TFLOPS at M=2048",
           "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
           "config": {"workload": "decode up-projection GEMV M=1 K=5120 N=17408 g=128",
                      "M": 1, "K": 5120, "N": 17408, "group_size": 128}}

    if args.calib_copy_mib:
        n = args.calib_copy_mib * 2 ** 20 // 4
        a = torch.ones(n, dtype=torch.int32, device="cuda:0")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(f"calibration copy: {args.calib_copy_mib} MiB read + written", file=sys.stderr)

    if args.only in ("all", "decode"):
        case = workloads.decode_up()
        inp, y, sec, R = bench_case(torch, w4, case, args.steps, args.warmup, args.eager)
        B = algorithmic_bytes(case.M, case.K, case.N, case.G)
        gbs = B / sec / 1e9
        out["value"] = round(gbs, 1)
        out["ms_per_step"] = sec * 1e3
        out["config"]["rotating_weight_sets"] = R
        traffic = load_traffic("decode")
        out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                           "traffic": traffic, "algorithmic_bytes": B,
                           "kernel": "w4a16::decode_streamk_kernel"}
        if not args.no_ceiling:
            ceil = read_ceiling(torch, w4)
            out["hbm_read_ceiling"] = {"value": round(ceil, 1), "unit": "GB/s",
                                       "bytes": 1 << 30, "kernel": "w4a16::read_probe_kernel"}
            out["roofline"]["frac_of_measured_ceiling"] = round(gbs / ceil, 4)
        if not args.no_cpu_baseline:
            cb, y_ref = cpu_baseline_decode(case, inp, args.cpu_seconds)
            out["cpu_baseline"] = cb
            out["parity_vs_oracle"] = parity_summary(y.cpu().numpy(), y_ref)
        del inp, y
        torch.cuda.empty_cache()

    if args.only in ("all", "prefill"):
        case = workloads.prefill_up()
        psteps = args.prefill_steps or max(10, args.steps // 4)
        pwarm = max(1, min(args.warmup, psteps))
        inp, y, sec, R = bench_case(torch, w4, case, psteps, pwarm, args.eager)
        F = 2.0 * case.M * case.N * case.K
        tflops = F / sec / 1e12
        traffic = load_traffic("prefill")
        pre = {"workload": "prefill up-projection GEMM M=2048 K=5120 N=17408 g=128",
               "value": round(tflops, 1), "unit": "TFLOP/s", "steps": psteps, "warmup": pwarm,
               "ms_per_step": sec * 1e3, "rotating_weight_sets": R,
               "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                            "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                            "traffic": traffic, "algorithmic_flops": F,
                            "kernel": "w4a16::prefill_m256_kernel"}}
        if not args.no_cpu_baseline:
            pre["cpu_baseline"] = cpu_baseline_prefill(case, inp, args.cpu_seconds)
        if args.only == "prefill":
            out.update({"value": pre["value"], "unit": "TFLOP/s",
                        "ms_per_step": pre["ms_per_step"], "roofline": pre["roofline"],
                        "config": {"workload": pre["workload"], "M": 2048, "K": 5120,
                                   "N": 17408, "group_size": 128}})
            if "cpu_baseline" in pre:
                out["cpu_baseline"] = pre["cpu_baseline"]
        else:
            out["prefill"] = pre

    if args.only == "all" and not args.no_bf16:
        # the bfloat16-activation variant on the same two workloads (same
        # algorithmic bytes and flops; x and y in bfloat16)
        bf = {}
        case = workloads.decode_up()
        _, _, sec, R = bench_case(torch, w4, case, args.steps, args.warmup, args.eager, True)
        gbs = algorithmic_bytes(case.M, case.K, case.N, case.G) / sec / 1e9
        bf["decode"] = {"workload": out["config"]["workload"] + ", bfloat16 x/y",
                        "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": sec * 1e3,
                        "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(gbs / HBM_PEAK_GBS, 4)}}
        torch.cuda.empty_cache()
        case = workloads.prefill_up()
        psteps = args.prefill_steps or max(10, args.steps // 4)
        _, _, sec, R = bench_case(torch, w4, case, psteps, max(1, min(args.warmup, psteps)),
                                  args.eager, True)
        tflops = 2.0 * case.M * case.N * case.K / sec / 1e12
        bf["prefill"] = {"workload": "prefill up-projection GEMM M=2048 K=5120 N=17408 g=128, "
                                     "bfloat16 x/y",
                         "value": round(tflops, 1), "unit": "TFLOP/s", "ms_per_step": sec * 1e3,
                         "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                                      "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)}}
        torch.cuda.empty_cache()
        out["bf16"] = bf

    if args.only == "all" and not args.no_gate_up:
        # the merged gate/up projection with the fused SiLU * mul epilogue at
        # the model's MLP shape (gate and up of 17408 columns each)
        gu = {}
        case = workloads.gate_up_decode()
        _, _, sec, R = bench_case(torch, w4, case, args.steps, args.warmup, args.eager,
                                  gate_up=True)
        B = algorithmic_bytes(case.M, case.K, case.N, case.G) - case.M * case.N   # y is N/2 wide
        gbs = B / sec / 1e9
        gu["decode"] = {"workload": "gate_up + SiLU*mul GEMV M=1 K=5120 N=2x17408 g=128",
                        "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": sec * 1e3,
                        "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                                     "algorithmic_bytes": B}}
        torch.cuda.empty_cache()
        case = workloads.gate_up_prefill()
        psteps = max(5, (args.prefill_steps or max(10, args.steps // 4)) // 2)
        _, _, sec, R = bench_case(torch, w4, case, psteps, max(1, min(args.warmup, psteps)),
                                  args.eager, gate_up=True)
        tflops = 2.0 * case.M * case.N * case.K / sec / 1e12
        gu["prefill"] = {"workload": "gate_up + SiLU*mul GEMM M=2048 K=5120 N=2x17408 g=128",
                         "value": round(tflops, 1), "unit": "TFLOP/s", "ms_per_step": sec * 1e3,
                         "steps": psteps,
                         "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                                      "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4)}}
        torch.cuda.empty_cache()
        out["gate_up_silu"] = gu

    if args.only == "all" and not args.no_lora:
        # the linear with a rank-32 LoRA adapter (the pages' suggested rank):
        # the linear's kernel, then the adapter's shrink and expand kernels
        lo, r = {}, 32
        case = workloads.decode_up()
        _, _, sec, R = bench_case(torch, w4, case, args.steps, args.warmup, args.eager,
                                  lora_rank=r)
        B = algorithmic_bytes(case.M, case.K, case.N, case.G) + 2 * r * (case.K + case.N)
        gbs = B / sec / 1e9
        lo["decode"] = {"workload": "decode up-projection GEMV M=1 K=5120 N=17408 g=128 + LoRA r=32",
                        "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": sec * 1e3,
                        "linear_alone_ms": out.get("ms_per_step"),
                        "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                                     "algorithmic_bytes": B}}
        torch.cuda.empty_cache()
        case = workloads.prefill_up()
        psteps = args.prefill_steps or max(10, args.steps // 4)
        _, _, sec, R = bench_case(torch, w4, case, psteps, max(1, min(args.warmup, psteps)),
                                  args.eager, lora_rank=r)
        flops = 2.0 * case.M * (case.N * case.K + r * (case.K + case.N))
        tflops = flops / sec / 1e12
        lo["prefill"] = {"workload": "prefill up-projection GEMM M=2048 K=5120 N=17408 g=128 + LoRA r=32",
                         "value": round(tflops, 1), "unit": "TFLOP/s", "ms_per_step": sec * 1e3,
                         "linear_alone_ms": out.get("prefill", {}).get("ms_per_step"),
                         "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                                      "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4)}}
        torch.cuda.empty_cache()
        out["lora"] = lo

    if args.only == "all" and not args.no_zero_points:
        # asymmetric weights: the linear with stored zero points (int32 [G, N/8])
        zp = {}
        case = workloads.decode_up()
        _, _, sec, R = bench_case(torch, w4, case, args.steps, args.warmup, args.eager,
                                  zero_points=True)
        B = algorithmic_bytes(case.M, case.K, case.N, case.G) + case.G * case.N // 2
        gbs = B / sec / 1e9
        zp["decode"] = {"workload": "decode up-projection GEMV M=1 K=5120 N=17408 g=128, stored zero points",
                        "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": sec * 1e3,
                        "linear_alone_ms": out.get("ms_per_step"),
                        "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                                     "algorithmic_bytes": B}}
        torch.cuda.empty_cache()
        case = workloads.prefill_up()
        psteps = args.prefill_steps or max(10, args.steps // 4)
        _, _, sec, R = bench_case(torch, w4, case, psteps, max(1, min(args.warmup, psteps)),
                                  args.eager, zero_points=True)
        tflops = 2.0 * case.M * case.N * case.K / sec / 1e12
        zp["prefill"] = {"workload": "prefill up-projection GEMM M=2048 K=5120 N=17408 g=128, stored zero points",
                         "value": round(tflops, 1), "unit": "TFLOP/s", "ms_per_step": sec * 1e3,
                         "linear_alone_ms": out.get("prefill", {}).get("ms_per_step"),
                         "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                                      "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4)}}
        torch.cuda.empty_cache()
        out["zero_points"] = zp

    out["device"] = dev_name
    out["timing"] = "eager launches" if args.eager else "one HIP graph of K steps"
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
