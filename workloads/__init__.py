"""Seeded synthetic inputs for the W4A16 symmetric-INT4 GPTQ linear.

This module only draws random numbers: 4-bit codes (uint8, values 0..15),
fp16 scales and fp16 activations, in a fixed draw order from a fresh
``numpy.random.default_rng(seed)`` per case.  It holds none of the method's
arithmetic (no packing, no dequantisation, no matmul), so both the CPU oracle
and the HIP path can consume the same inputs without sharing code.

Shapes stand in for the linears of the 27B model named on the
"GPTQ-Pro" README ("Qwen3.8-27B" section: hidden size 5120, FFN size 17408):
up/gate projections are K=5120 -> N=17408 and the down projection is
K=17408 -> N=5120.  Group sizes follow the checkpoints on the pages
(g=32 on the "Qwen3.8-27B-GPTQ-Int4" model card, g=128 as the default of the
GPTQModel "Installation and Quickstart" page, "Defaults and compatibility
decisions" table).

Draw order for every case: codes ``[K, N]``, scales ``[G, N]``, the zero-cell
mask (sweep only), x ``[M, K]``, the outlier channels (prefill only).  Cases
that share (K, N, g) and differ only in M therefore share weights, and row 0
of x is the same for every M.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Iterator, List, Optional

import numpy as np

GROUP_SIZES = (-1, 16, 32, 64, 128, 256, 512, 1024)


def num_groups(K: int, group_size: int) -> int:
    """Rows of the scale grid: one for g = -1, else ceil(K / g)."""
    return 1 if group_size == -1 else -(-K // group_size)


@dataclasses.dataclass(frozen=True)
class Case:
    """One synthetic linear: shapes, group size, input recipe and seed."""

    name: str
    M: int
    K: int
    N: int
    group_size: int
    seed: int
    scales: str = "uniform"          # "uniform" | "halfnormal" | "loguniform" | "pow2" | "wide"
    x_dist: str = "normal"           # "normal" | "normal_half" | "int"
    outlier_frac: float = 0.0        # fraction of K channels of x scaled x20
    zero_cell_frac: float = 0.0      # fraction of (group, column) cells forced to code 8

    @property
    def G(self) -> int:
        return num_groups(self.K, self.group_size)


@dataclasses.dataclass
class Inputs:
    codes: np.ndarray     # uint8 [K, N], values 0..15
    scales: np.ndarray    # float16 [G, N], or bfloat16 bit patterns (uint16)
    x: np.ndarray         # float16 [M, K]
    zero_cells: Optional[np.ndarray] = None   # bool [G, N] (sweep only)
    outlier_channels: Optional[np.ndarray] = None  # int64 [n_out] (prefill only)


def _draw_scales(rng: np.random.Generator, kind: str, G: int, N: int) -> np.ndarray:
    if kind == "uniform":          # U[1e-3, 2e-2]
        s = rng.uniform(1e-3, 2e-2, size=(G, N))
    elif kind == "halfnormal":     # |N(0, 0.01)| + 1e-4
        s = np.abs(rng.normal(0.0, 0.01, size=(G, N))) + 1e-4
    elif kind == "loguniform":     # exp(U(ln 1e-4, ln 5e-2))
        s = np.exp(rng.uniform(math.log(1e-4), math.log(5e-2), size=(G, N)))
    elif kind == "pow2":           # 2^e, e in {-4, -3, -2}: exact-arithmetic inputs
        s = np.exp2(rng.integers(-4, -1, size=(G, N)).astype(np.float64))
    elif kind == "wide":           # exp(U(ln 2^-30, ln 2^-2)): beyond fp16's range (bfloat16 only)
        s = np.exp(rng.uniform(-30 * math.log(2.0), -2 * math.log(2.0), size=(G, N)))
    else:
        raise ValueError(f"unknown scale recipe {kind!r}")
    return s


def _draw_x(rng: np.random.Generator, kind: str, M: int, K: int) -> np.ndarray:
    if kind == "normal":
        return rng.standard_normal((M, K))
    if kind == "normal_half":      # N(0, 0.5): standard deviation 0.5
        return 0.5 * rng.standard_normal((M, K))
    if kind == "int":              # integers in [-4, 4]: exact-arithmetic inputs
        return rng.integers(-4, 5, size=(M, K)).astype(np.float64)
    raise ValueError(f"unknown x recipe {kind!r}")


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """Values -> bfloat16 bit patterns (uint16): through float32, then rounded
    to nearest even on the top 16 bits (finite inputs).  Activations for the
    bfloat16 variant are the same draws as for fp16, given in this type."""
    f = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


def generate_bf16(case: Case) -> Inputs:
    """As generate, with x as bfloat16 bit patterns (uint16 [M, K]) of the
    same draws."""
    return generate(case, act="bf16")


def generate(case: Case, act: str = "f16", scales_type: str = "f16") -> Inputs:
    """Draw one case's inputs in the fixed order stated in the module docstring.
    act / scales_type "bf16": x / the scales as bfloat16 bit patterns of the
    same draws (rounded to nearest even), else fp16."""
    rng = np.random.default_rng(case.seed)
    K, N, M, G, g = case.K, case.N, case.M, case.G, case.group_size
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    s64 = _draw_scales(rng, case.scales, G, N)
    if scales_type == "bf16":
        scales = bf16_bits(s64)
    elif case.scales == "wide":
        raise ValueError("the wide scale recipe is for bfloat16 scales")
    else:
        scales = s64.astype(np.float16)
    zero_cells = None
    if case.zero_cell_frac > 0.0:
        n_cells = int(round(case.zero_cell_frac * G * N))
        flat = rng.choice(G * N, size=n_cells, replace=False)
        zero_cells = np.zeros(G * N, dtype=bool)
        zero_cells[flat] = True
        zero_cells = zero_cells.reshape(G, N)
        rows_per_group = K if g == -1 else g
        row_mask = np.repeat(zero_cells, rows_per_group, axis=0)[:K]
        codes[row_mask] = 8
    x64 = _draw_x(rng, case.x_dist, M, K)
    outliers = None
    if case.outlier_frac > 0.0:
        n_out = int(round(case.outlier_frac * K))
        outliers = np.sort(rng.choice(K, size=n_out, replace=False))
        x64[:, outliers] *= 20.0
    x = bf16_bits(x64) if act == "bf16" else x64.astype(np.float16)
    return Inputs(codes=codes, scales=scales, x=x, zero_cells=zero_cells,
                  outlier_channels=outliers)


# --- the five workloads -------------------------------------------------------

def tiny() -> Case:
    """Tiny linear: M=1, K=256, N=256, g=32, scales U[1e-3,2e-2], x N(0,1), seed 0."""
    return Case("tiny", 1, 256, 256, 32, 0)


def decode_up() -> Case:
    """Decode up-projection GEMV: M=1, K=5120, N=17408, g=128, seed 1."""
    return Case("decode_up", 1, 5120, 17408, 128, 1)


def down_small_batch(M: int) -> Case:
    """Small-batch down projection: M in {1,4,16}, K=17408, N=5120, g=32, seed 2."""
    if M not in (1, 4, 16):
        raise ValueError("down_small_batch takes M in {1, 4, 16}")
    return Case(f"down_small_batch_M{M}", M, 17408, 5120, 32, 2,
                scales="halfnormal", x_dist="normal_half")


def prefill_up() -> Case:
    """Prefill up-projection GEMM: M=2048, K=5120, N=17408, g=128, 1% outlier channels x20, seed 3."""
    return Case("prefill_up", 2048, 5120, 17408, 128, 3, outlier_frac=0.01)


SWEEP_GROUPS = (-1, 16, 64, 256, 512, 1024)
SWEEP_SHAPES = ((5120, 17408), (17408, 5120), (5120, 5120))
SWEEP_MS = (1, 8, 64, 512)


def gate_up_decode() -> Case:
    """Merged gate/up projection (gate and up of 17408 columns each, interleaved:
    N = 34816), M=1, K=5120, g=128, weights drawn as for the up-projection, seed 1."""
    return Case("gate_up_decode", 1, 5120, 34816, 128, 1)


def gate_up_prefill() -> Case:
    """Merged gate/up projection, M=2048, K=5120, N=34816, g=128, seed 3."""
    return Case("gate_up_prefill", 2048, 5120, 34816, 128, 3, x_dist="normal")


LORA_SCALE = 2.0          # alpha / r with alpha = 2r
LORA_RANKS = (8, 16, 32, 64, 128, 256)


def lora_adapter(K: int, N: int, rank: int, seed: int, act: str = "f16"):
    """A seeded LoRA adapter (A [rank, K], B [N, rank]) from its own generator.

    A ~ U(-1/sqrt(K), 1/sqrt(K)), the bound of PEFT's default initialisation
    of lora_A; B ~ N(0, 0.25^2), a stand-in for a trained adapter whose term is
    of the order of the base output (PEFT initialises B to zero, which would
    make the term vanish).  The pages suggest rank 32, then 64, with 128 and
    256 as larger choices ("GPT-QModel" README, "EoRA Accuracy Recovery").
    Draw order: A, then B.  Returned as fp16 arrays, or bfloat16 bit patterns
    (uint16) when act is "bf16"."""
    rng = np.random.default_rng(seed)
    A = rng.uniform(-1.0, 1.0, size=(rank, K)) / math.sqrt(K)
    B = 0.25 * rng.standard_normal((N, rank))
    if act == "bf16":
        return bf16_bits(A), bf16_bits(B)
    return A.astype(np.float16), B.astype(np.float16)


def zero_points(G: int, N: int, seed: int) -> np.ndarray:
    """Seeded zero points for asymmetric weights: uint8 [G, N], uniform over
    0..15 (every code value; 8 is the symmetric one), from their own generator."""
    return np.random.default_rng(seed).integers(0, 16, size=(G, N), dtype=np.uint8)


def sweep() -> List[Case]:
    """Group-size and shape sweep: 6 g x 3 (K,N) x 4 M = 72 cases, 5% zero cells, seed 4."""
    out = []
    for g in SWEEP_GROUPS:
        for K, N in SWEEP_SHAPES:
            for M in SWEEP_MS:
                out.append(Case(f"sweep_g{g}_K{K}_N{N}_M{M}", M, K, N, g, 4,
                                scales="loguniform", zero_cell_frac=0.05))
    return out


def all_cases() -> Iterator[Case]:
    yield tiny()
    yield decode_up()
    for M in (1, 4, 16):
        yield down_small_batch(M)
    yield prefill_up()
    yield from sweep()


def exact_case(name: str, M: int, K: int, N: int, group_size: int, seed: int) -> Case:
    """Exact-arithmetic inputs: integer x in [-4,4], power-of-two scales 2^-4..2^-2.

    Every product x*(q-8)*s is a multiple of 2^-4 and every partial sum stays
    below 2^18 for K <= 17408, so any fp32 summation order gives the same,
    exact value.
    """
    return Case(name, M, K, N, group_size, seed, scales="pow2", x_dist="int")
