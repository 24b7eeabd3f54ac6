#!/usr/bin/env python3
"""Benchmark of the W4A16 symmetric-INT4 GPTQ linear on one MI355X.

Headline (``value``): HBM GB/s of the decode up-projection GEMV, M=1,
K=5120, N=17408, g=128 (one step = one w4a16_linear call over one batch).
The same line carries the prefill up-projection GEMM, M=2048, K=5120,
N=17408, g=128, in TFLOP/s under ``prefill``, the variants (bfloat16 with
fp16 and with bfloat16 scales, merged gate/up + SiLU*mul, LoRA, stored zero
points) at the same two shapes, and
under ``configs`` the other workloads: the tiny linear, the small-batch down
projection (M = 1, 4, 16) and the 72-case group-size / shape sweep.

Timing: W untimed warm-up steps, then exactly K steps captured in one HIP
graph and replayed between HIP events on the launch stream, with a device
synchronisation on both sides; the K-step replay is repeated at least five
times, and until the timed replays add up to 60 ms (the device settles its
clock over tens of milliseconds of work; at most 41 replays), each replay
walking on through the rotating weight sets, and the median is reported with
the replays' spread beside it.  Each step uses the next of R rotating
(qweight, scales) copies, R chosen so that the copies span at least twice the
256 MB Infinity Cache, so every weight byte comes from HBM.

Algorithmic bytes per step: K*N/2 (codes) + 2*G*N (scales) + 2*M*K (x)
+ 2*M*N (y).  Algorithmic flops per step: 2*M*N*K.  A workload is bound by
HBM when its flops per algorithmic byte are below the ridge 2.5e15 / 8e12
(312.5), else by the matrix cores.

The CPU baseline times the oracle (plain C, fp64, OpenMP) on the host cores
on a bounded sample of the same workload, after every GPU measurement.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
RIDGE = FP16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # flop per byte
MALL_BYTES = 256 * 2 ** 20
REPLAYS = 5
MIN_TIMED_S = 0.06
MAX_REPLAYS = 41


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Timed:
    """K-step HIP graphs replayed between HIP events on their own stream."""

    def __init__(self, torch, replays: int = REPLAYS):
        self.torch = torch
        self.replays = replays

    def _capture(self, fn, first, steps, stream):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(first, first + steps):
                fn(i)
        return g

    def run(self, fn, steps, warmup, eager=False):
        """W warm-up steps, then timed replays of exactly `steps` steps each: at
        least `replays` (five), and more, up to MAX_REPLAYS, until the timed
        replays add up to MIN_TIMED_S (the device settles its clock over tens of
        milliseconds of work; the median is then a settled replay).  fn(i) runs
        step i; the replays cycle over five graphs of consecutive steps, so the
        weight sets keep rotating.  Returns (median seconds per step, [ms per
        step of each replay])."""
        torch = self.torch
        if eager:
            for i in range(warmup):
                fn(i)
            torch.cuda.synchronize()
            st = torch.cuda.current_stream()
            per = []
            for r in range(self.replays):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(st)
                for i in range(steps):
                    fn(warmup + r * steps + i)
                e1.record(st)
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) / steps)
            return statistics.median(per) / 1e3, per
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)                       # first call outside capture (arch cache, workspaces)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        gw = self._capture(fn, 0, max(1, warmup), s)
        timed = [self._capture(fn, warmup + r * steps, steps, s) for r in range(self.replays)]
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            gw.replay()
        torch.cuda.synchronize()
        per = []
        total, n = 0.0, self.replays
        while len(per) < n:
            g = timed[len(per) % len(timed)]
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(s):
                e0.record(s)
                g.replay()
                e1.record(s)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            per.append(ms / steps)
            total += ms / 1e3
            if len(per) == n and total < MIN_TIMED_S and n < MAX_REPLAYS:
                n += 2                                    # odd counts: the median is a replay
        return statistics.median(per) / 1e3, per


def rotations_for(weight_bytes: int, minimum: int = 2) -> int:
    return max(minimum, -(-2 * MALL_BYTES // weight_bytes))


def upload_x(torch, x_np, bf16, dev):
    import numpy as np
    x_np = np.ascontiguousarray(x_np)
    if bf16:   # bfloat16 bit patterns -> a bfloat16 tensor
        return torch.from_numpy(x_np.view("int16")).view(torch.bfloat16).to(dev)
    return torch.from_numpy(x_np).to(dev)


def time_linear(torch, w4, codes, scales, x_np, M, K, N, g, steps, warmup, eager,
                bf16=False, gate_up=False, lora_rank=0, zero_points=None, seed=0,
                scales_bf16=False):
    """Times one workload (the linear or a variant) with R rotating weight sets.
    Returns (y of the last step, seconds per step, per-replay ms, R)."""
    import workloads
    dev = torch.device("cuda:0")
    wbytes = K * N // 2 + 2 * scales.shape[0] * N
    R = rotations_for(wbytes)
    q = torch.from_numpy(w4.pack_gptq_v2(codes)).to(dev)
    s = torch.from_numpy(scales).to(dev)
    if scales_bf16:   # bfloat16 bit patterns -> a bfloat16 tensor
        s = s.view(torch.bfloat16)
    qs = [q] + [q.clone() for _ in range(R - 1)]
    ss = [s] + [s.clone() for _ in range(R - 1)]
    x = upload_x(torch, x_np, bf16, dev)
    ncols = N // 2 if gate_up else N
    y = torch.empty((M, ncols), dtype=x.dtype, device=dev)
    if gate_up:
        call = w4.w4a16_gate_up_silu_bf16 if bf16 else w4.w4a16_gate_up_silu
    else:
        call = w4.w4a16_linear_bf16 if bf16 else w4.w4a16_linear

    def step(i):
        call(x, qs[i % R], ss[i % R], y, M, K, N, g)

    if scales_bf16:
        flags = w4.W4A16_X_BF16 | w4.W4A16_SCALES_BF16

        def step(i):  # noqa: F811
            w4.w4a16_linear_typed(x, qs[i % R], ss[i % R], None, y, M, K, N, g, flags)

    if lora_rank:
        # the adapter rotates with the weights: each layer of a model has its own
        A, B = workloads.lora_adapter(K, N, lora_rank, seed + 500)
        As = [torch.from_numpy(A).to(dev) for _ in range(R)]
        Bs = [torch.from_numpy(B).to(dev) for _ in range(R)]
        wsb = w4.w4a16_lora_workspace_bytes(M, K, lora_rank)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

        def step(i):  # noqa: F811
            w4.w4a16_linear_lora(x, qs[i % R], ss[i % R], As[i % R], Bs[i % R],
                                 workloads.LORA_SCALE, y, M, K, N, g, lora_rank, ws, wsb)

    if zero_points is not None:
        # zero points rotate with the weights, like the scales they belong to
        qz = torch.from_numpy(w4.pack_zeros(zero_points))
        qzs = [qz.to(dev) for _ in range(R)]
        wsb = w4.w4a16_zp_workspace_bytes(M, K, N, g)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

        def step(i):  # noqa: F811
            w4.w4a16_linear_zp(x, qs[i % R], ss[i % R], qzs[i % R], y, M, K, N, g, ws, wsb)

    sec, per = Timed(torch).run(step, steps, warmup, eager)
    return y, sec, per, R


def bench_case(torch, w4, case, steps, warmup, eager, bf16=False, gate_up=False, lora_rank=0,
               zero_points=False, scales_bf16=False):
    import workloads
    if scales_bf16:
        inp = workloads.generate(case, act="bf16", scales_type="bf16")
    else:
        inp = workloads.generate_bf16(case) if bf16 else workloads.generate(case)
    zp = workloads.zero_points(case.G, case.N, case.seed + 700) if zero_points else None
    y, sec, per, R = time_linear(torch, w4, inp.codes, inp.scales, inp.x, case.M, case.K, case.N,
                                 case.group_size, steps, warmup, eager, bf16, gate_up, lora_rank,
                                 zp, case.seed, scales_bf16)
    return y, sec, per, R


def replay_summary(per):
    """Count, first, fastest, median and slowest replay, in ms per step."""
    return {"n": len(per), "first_ms": round(per[0], 5), "min_ms": round(min(per), 5),
            "median_ms": round(statistics.median(per), 5), "max_ms": round(max(per), 5)}


def rate_entry(M, K, N, G, sec, per, extra_bytes=0, extra_flops=0, y_cols=None):
    """Time, rate and roofline fraction of one workload, bound by its intensity."""
    B = algorithmic_bytes(M, K, N, G) + extra_bytes
    if y_cols is not None:
        B -= 2 * M * (N - y_cols)
    F = 2.0 * M * N * K + extra_flops
    gbs = B / sec / 1e9
    tflops = F / sec / 1e12
    if F / B < RIDGE:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4)}
    return {"us_per_step": round(sec * 1e6, 2), "GB/s": round(gbs, 1),
            "TFLOP/s": round(tflops, 2), "replays": replay_summary(per), "roofline": roof}


def cpu_baseline_decode(case, inp, seconds):
    """Oracle on the full decode case, repeated for about `seconds` of host time."""
    import oracle
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
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"the whole decode case (M=1, K={case.K}, N={case.N}, g={case.group_size}),"
                      f" {reps} repetitions, {el:.1f} s, {per * 1e3:.1f} ms per call"}, y_ref


def cpu_baseline_prefill(case, inp, seconds):
    """Oracle on whole output rows of the prefill case (the rest is the same work)."""
    import numpy as np
    import oracle
    q_o = oracle.pack(inp.codes)
    rows, t0 = 0, time.perf_counter()
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
            "kind": "oracle", "cpu_model": cpu_model(),
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


def bench_configs(torch, w4, steps, warmup, eager, with_sweep=True):
    """The workloads besides the two headline shapes: the tiny linear, the
    small-batch down projection and the group-size / shape sweep (summarised
    per group size: worst and median roofline fraction)."""
    import numpy as np
    import workloads
    out = {}
    for case in [workloads.tiny()] + [workloads.down_small_batch(M) for M in (1, 4, 16)]:
        _, sec, per, R = bench_case(torch, w4, case, steps, warmup, eager)
        e = rate_entry(case.M, case.K, case.N, case.G, sec, per)
        e.update({"workload": f"M={case.M} K={case.K} N={case.N} g={case.group_size}",
                  "rotating_weight_sets": R})
        out[case.name] = e
        torch.cuda.empty_cache()
        log(f"{case.name}: {e['us_per_step']} us, frac {e['roofline']['frac']}")
    if not with_sweep:
        return out
    rows, per_g = [], {}
    for g in workloads.SWEEP_GROUPS:
        for K, N in workloads.SWEEP_SHAPES:
            # one draw per weight set: cases differing only in M share weights,
            # and the rows of x are the first rows of the largest M's draw
            big = workloads.Case(f"sweep_g{g}_K{K}_N{N}", max(workloads.SWEEP_MS), K, N, g, 4,
                                 scales="loguniform", zero_cell_frac=0.05)
            inp = workloads.generate(big)
            for M in workloads.SWEEP_MS:
                _, sec, per, _ = time_linear(torch, w4, inp.codes, inp.scales,
                                             np.ascontiguousarray(inp.x[:M]), M, K, N, g,
                                             steps, warmup, eager)
                e = rate_entry(M, K, N, big.G, sec, per)
                rows.append([g, K, N, M, e["us_per_step"], e["roofline"]["bound"],
                             e["roofline"]["frac"]])
                per_g.setdefault(g, []).append((e["roofline"]["frac"], f"K={K} N={N} M={M}"))
                torch.cuda.empty_cache()
            log(f"sweep g={g} K={K} N={N}: " + ", ".join(f"{r[6]:.3f}" for r in rows[-4:]))
    summary = {}
    for g, fr in per_g.items():
        worst = min(fr)
        summary[str(g)] = {"worst_frac": worst[0], "worst_case": worst[1],
                           "median_frac": round(statistics.median(f for f, _ in fr), 4)}
    out["sweep"] = {"cases": len(rows), "per_group_size": summary,
                    "columns": ["g", "K", "N", "M", "us_per_step", "bound", "frac"],
                    "rows": rows}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
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
                    help="skip the bfloat16 variants' decode and prefill lines (bfloat16 x/y "
                         "with fp16 scales, and with bfloat16 scales)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the tiny, down-projection and sweep workloads")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 72-case sweep inside the configs section")
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
    K_steps, W = args.steps, args.warmup
    out = {"metric": "W4A16 linear: HBM GB/s at M=1 (5120x17408 g128); TFLOPS at M=2048",
           "value": None, "unit": "GB/s", "n_gpus": 1, "steps": K_steps,
           "warmup": W, "ms_per_step": None, "higher_is_better": True,
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
        log(f"calibration copy: {args.calib_copy_mib} MiB read + written")

    # the read ceiling first: it is a measurement of its own and leaves the
    # device out of its idle state before the timed workloads
    ceil = None
    if not args.no_ceiling:
        ceil = read_ceiling(torch, w4)
        out["hbm_read_ceiling"] = {"value": round(ceil, 1), "unit": "GB/s",
                                   "bytes": 1 << 30, "kernel": "w4a16::read_probe_kernel"}
        log(f"read ceiling {ceil:.0f} GB/s")

    y_dec = None
    if args.only in ("all", "decode"):
        case = workloads.decode_up()
        y, sec, per, R = bench_case(torch, w4, case, K_steps, W, args.eager)
        y_dec = y.cpu().numpy()
        B = algorithmic_bytes(case.M, case.K, case.N, case.G)
        gbs = B / sec / 1e9
        out["value"] = round(gbs, 1)
        out["ms_per_step"] = sec * 1e3
        out["replays"] = replay_summary(per)
        out["config"]["rotating_weight_sets"] = R
        out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                           "traffic": load_traffic("decode"), "algorithmic_bytes": B,
                           "kernel": "w4a16::decode_streamk_kernel"}
        if ceil:
            out["roofline"]["frac_of_measured_ceiling"] = round(gbs / ceil, 4)
        log(f"decode: {sec * 1e6:.2f} us, {gbs:.0f} GB/s ({len(per)} replays, first "
            f"{per[0] * 1e3:.2f} us)")
        del y
        torch.cuda.empty_cache()

    pre = None
    if args.only in ("all", "prefill"):
        case = workloads.prefill_up()
        _, sec, per, R = bench_case(torch, w4, case, K_steps, W, args.eager)
        F = 2.0 * case.M * case.N * case.K
        tflops = F / sec / 1e12
        pre = {"workload": "prefill up-projection GEMM M=2048 K=5120 N=17408 g=128",
               "value": round(tflops, 1), "unit": "TFLOP/s", "steps": K_steps, "warmup": W,
               "ms_per_step": sec * 1e3, "replays": replay_summary(per),
               "rotating_weight_sets": R,
               "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                            "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                            "traffic": load_traffic("prefill"), "algorithmic_flops": F,
                            "kernel": "w4a16::prefill_m256_kernel"}}
        log(f"prefill: {sec * 1e6:.1f} us, {tflops:.0f} TFLOP/s ({len(per)} replays, first "
            f"{per[0] * 1e3:.1f} us)")
        if args.only == "prefill":
            out.update({"value": pre["value"], "unit": "TFLOP/s",
                        "ms_per_step": pre["ms_per_step"], "roofline": pre["roofline"],
                        "replays": pre["replays"],
                        "config": {"workload": pre["workload"], "M": 2048, "K": 5120,
                                   "N": 17408, "group_size": 128, "rotating_weight_sets": R}})
        else:
            out["prefill"] = pre
        torch.cuda.empty_cache()

    def pair(label, decode_case, prefill_case, **kw):
        """Decode (GB/s) and prefill (TFLOP/s) lines of one variant."""
        res = {}
        for leg, case in (("decode", decode_case), ("prefill", prefill_case)):
            _, sec, per, R = bench_case(torch, w4, case, K_steps, W, args.eager, **kw)
            extra_b = extra_f = 0
            y_cols = None
            if kw.get("gate_up"):
                y_cols = case.N // 2
            if kw.get("lora_rank"):
                r = kw["lora_rank"]
                extra_b = 2 * r * (case.K + case.N)
                extra_f = 2.0 * case.M * r * (case.K + case.N)
            if kw.get("zero_points"):
                extra_b = case.G * case.N // 2
            e = rate_entry(case.M, case.K, case.N, case.G, sec, per, extra_b, extra_f, y_cols)
            e["workload"] = f"{label} M={case.M} K={case.K} N={case.N} g={case.group_size}"
            e["ms_per_step"] = sec * 1e3
            if kw.get("lora_rank") or kw.get("zero_points"):
                base = out.get("ms_per_step") if leg == "decode" else (pre or {}).get("ms_per_step")
                e["linear_alone_ms"] = base
            res[leg] = e
            log(f"{label} {leg}: {sec * 1e6:.1f} us, frac {e['roofline']['frac']}")
            torch.cuda.empty_cache()
        return res

    if args.only == "all" and not args.no_bf16:
        out["bf16"] = pair("bfloat16 x/y", workloads.decode_up(), workloads.prefill_up(),
                           bf16=True)
        out["bf16_scales"] = pair("bfloat16 x/y and scales", workloads.decode_up(),
                                  workloads.prefill_up(), bf16=True, scales_bf16=True)
    if args.only == "all" and not args.no_gate_up:
        out["gate_up_silu"] = pair("gate_up + SiLU*mul (N = 2x17408)", workloads.gate_up_decode(),
                                   workloads.gate_up_prefill(), gate_up=True)
    if args.only == "all" and not args.no_lora:
        out["lora"] = pair("linear + LoRA r=32", workloads.decode_up(), workloads.prefill_up(),
                           lora_rank=32)
    if args.only == "all" and not args.no_zero_points:
        out["zero_points"] = pair("linear with stored zero points", workloads.decode_up(),
                                  workloads.prefill_up(), zero_points=True)
    if args.only == "all" and not args.no_configs:
        out["configs"] = bench_configs(torch, w4, K_steps, W, args.eager,
                                       with_sweep=not args.no_sweep)

    # the CPU baselines last, once every GPU measurement is done
    if not args.no_cpu_baseline:
        if y_dec is not None:
            case = workloads.decode_up()
            cb, y_ref = cpu_baseline_decode(case, workloads.generate(case), args.cpu_seconds)
            out["cpu_baseline"] = cb
            out["parity_vs_oracle"] = parity_summary(y_dec, y_ref)
            log(f"cpu baseline decode: {cb['value']:.3f} GB/s on {cb['cores']} threads")
        if pre is not None:
            case = workloads.prefill_up()
            cbp = cpu_baseline_prefill(case, workloads.generate(case), args.cpu_seconds)
            pre["cpu_baseline"] = cbp
            if args.only == "prefill":
                out["cpu_baseline"] = cbp
            log(f"cpu baseline prefill: {cbp['value']:.4f} TFLOP/s")

    out["device"] = dev_name
    out["timing"] = ("eager launches" if args.eager else
                     f"HIP graphs of K steps, at least {REPLAYS} timed replays and {MIN_TIMED_S * 1e3:.0f} "
                     f"ms of them, median")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
