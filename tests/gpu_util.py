"""Shared helpers of the GPU parity tests: run a case through the C ABI and
compare with the oracle to the parity bar.

The bar (per case): every element |y - y_ref| <= 5e-3 * max|y_ref| + 1e-3, and
sum|y - y_ref| / sum|y_ref| <= 1e-3, with y_ref the oracle's float64 result.
"""

from __future__ import annotations

import numpy as np

import oracle
import workloads

ABS_TOL = 1e-3
REL_MAX = 5e-3
MEAN_REL = 1e-3


def check_parity(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = "") -> dict:
    y = y_gpu.astype(np.float64)
    d = np.abs(y - y_ref)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    bound = REL_MAX * float(np.abs(y_ref).max()) + ABS_TOL
    denom = float(np.abs(y_ref).sum())
    mean_rel = float(d.sum()) / denom if denom > 0 else float(d.sum())
    worst = int(np.argmax(d)) if d.size else 0
    assert d.size == 0 or float(d.max()) <= bound, \
        f"{what}: max|d| {float(d.max()):.4g} > {bound:.4g} at flat index {worst}"
    assert mean_rel <= MEAN_REL, f"{what}: mean relative error {mean_rel:.4g} > {MEAN_REL}"
    return {"max_abs": float(d.max()) if d.size else 0.0, "bound": bound, "mean_rel": mean_rel}


# bfloat16 activations and output: the bar follows from the arithmetic the C
# ABI states for w4a16_linear_bf16 (u = 2^-8 is half a bfloat16 ulp relative):
# weights rounded once to bfloat16 or summed exactly as 128 + q with the bias
# removed in fp32, fp32 accumulation, y rounded once to bfloat16:
#   |y - y_ref| <= u |y_ref| + 1.02 (u + K 2^-24) sum_k |x||w|
#                  + 1.02 * 35 K 2^-24 * 8 sum_k |x| s          (mag0)
# per element, with sum|x||w| and 8 sum|x| s (the magnitude sum of all-zero
# codes) from the oracle; and, so that a wrong term cannot hide inside that
# worst-case bound, sum|y - y_ref| / sum|y_ref| <= u.
BF16_U = 2.0 ** -8


def check_parity_bf16(y_gpu: np.ndarray, y_ref: np.ndarray, mag: np.ndarray, K: int,
                      what: str = "", mag0=None, extra=None) -> dict:
    y = y_gpu.astype(np.float64)
    d = np.abs(y - y_ref)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    bound = BF16_U * np.abs(y_ref) + 1.02 * (BF16_U + K * 2.0 ** -24) * mag + 1e-30
    if mag0 is not None:
        bound = bound + 1.02 * 35 * K * 2.0 ** -24 * mag0
    if extra is not None:
        bound = bound + extra
    bad = d > bound
    worst = int(np.argmax(d - bound)) if d.size else 0
    assert not np.any(bad), \
        f"{what}: {int(bad.sum())} elements beyond the bound; worst at flat index {worst}: " \
        f"|d| {float(d.flat[worst]):.4g} > {float(bound.flat[worst]):.4g}"
    denom = float(np.abs(y_ref).sum())
    mean_rel = float(d.sum()) / denom if denom > 0 else float(d.sum())
    assert mean_rel <= BF16_U, f"{what}: mean relative error {mean_rel:.4g} > {BF16_U}"
    return {"max_abs": float(d.max()) if d.size else 0.0, "mean_rel": mean_rel}


# Merged gate/up with SiLU * mul: the kernels form the gate and up sums g, u
# as the linear does (error at most eps * sum|x||w| per column), take
# silu(g) * u in fp32 (|silu'| <= 1.1) and round once (half an ulp: r |y| for
# normal outputs, and at most h = half the spacing of the output type's
# subnormals, 2^-25 for fp16 and 2^-134 for bfloat16, below its normal range):
#   |y - y_ref| <= r |y_ref| + h + 1.02 (1.1 |u| eps A_g + |silu(g)| eps A_u
#                                        + 1.1 eps^2 A_g A_u) + 4e-7 |y_ref|
# with A_g, A_u the oracle's magnitude sums of the two columns; plus the mean
# relative error of the linear's bar.
def _silu(z):
    return z / (1.0 + np.exp(-z))


def check_gate_up(y, ref, lin, mag, mag0, K, bf16, what):
    """y [M, N/2] from the GPU; lin, mag (and mag0 for bf16) [M, N] from the oracle."""
    g, u = lin[:, 0::2], lin[:, 1::2]
    a_g, a_u = mag[:, 0::2], mag[:, 1::2]
    if bf16:
        r = 2.0 ** -8
        eps_g = r + K * 2.0 ** -24 + 35 * K * 2.0 ** -24 * mag0[:, 0::2] / np.maximum(a_g, 1e-300)
        eps_u = r + K * 2.0 ** -24 + 35 * K * 2.0 ** -24 * mag0[:, 1::2] / np.maximum(a_u, 1e-300)
        mean_bar = 2.0 ** -8
        h = 2.0 ** -134
    else:
        r = 2.0 ** -11
        eps_g = eps_u = 2.0 ** -11 + K * 2.0 ** -24
        mean_bar = 1e-3
        h = 2.0 ** -25
    dg, du = eps_g * a_g, eps_u * a_u
    bound = (r * np.abs(ref) + h + 1.02 * (1.1 * np.abs(u) * dg + np.abs(_silu(g)) * du + 1.1 * dg * du)
             + 4e-7 * np.abs(ref) + 1e-30)
    d = np.abs(y - ref)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    worst = int(np.argmax(d - bound))
    assert np.all(d <= bound), \
        f"{what}: |d| {float(d.flat[worst]):.4g} > {float(bound.flat[worst]):.4g} at {worst}"
    denom = float(np.abs(ref).sum())
    mean_rel = float(d.sum()) / denom if denom > 0 else float(d.sum())
    assert mean_rel <= mean_bar, f"{what}: mean relative error {mean_rel:.4g}"



# LoRA adapter term (w4a16_linear_lora): beyond the linear's own bound, the
# C ABI states, per element (u half an ulp of the activation type, relative):
#   u |y_lin| + u |y| + u P1 + K 2^-24 P2 + r 2^-24 P1
# with P1 = |s| sum_j |t_j| |B[n,j]| (t exact) and P2 = |s| sum_j
# (sum_k |x| |A[j,k]|) |B[n,j]|: y_lin rounded once, t summed in fp32 and
# rounded to the activation type, the rank-r product in fp32, y rounded once.
def lora_extra_bound(lin, ref, p1, p2, K, r, u):
    return 1.02 * (u * np.abs(lin) + u * np.abs(ref) + u * p1 + K * 2.0 ** -24 * p2
                   + r * 2.0 ** -24 * p1)


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16 or int16) -> float64 (the top half of a float32)."""
    b = np.asarray(bits).view(np.uint16).astype(np.uint32)
    return (b << 16).view(np.float32).astype(np.float64)


class Runner:
    """Uploads a case's inputs and runs the HIP path through the C ABI."""

    def __init__(self, torch_mod, w4_mod):
        self.torch = torch_mod
        self.w4 = w4_mod
        self.dev = torch_mod.device("cuda:0")

    def upload(self, inp, qweight):
        t = self.torch
        return (t.from_numpy(np.ascontiguousarray(inp.x)).to(self.dev),
                t.from_numpy(np.ascontiguousarray(qweight)).to(self.dev),
                t.from_numpy(np.ascontiguousarray(inp.scales)).to(self.dev))

    def run(self, x, q, s, group_size, kernel=0):
        y = self.w4.linear(x, q, s, group_size, kernel=kernel)
        self.torch.cuda.synchronize()
        return y.cpu().numpy()


def sample_indices(M: int, N: int, count: int, seed: int):
    rng = np.random.default_rng(seed)
    ms = rng.integers(0, M, size=count)
    ns = rng.integers(0, N, size=count)
    # always include the corners and the last row/column
    ms = np.concatenate([ms, [0, 0, M - 1, M - 1]])
    ns = np.concatenate([ns, [0, N - 1, 0, N - 1]])
    return ms.astype(np.int64), ns.astype(np.int64)


def oracle_sampled(inp, qweight_o, group_size, ms, ns):
    return oracle.linear_at(inp.x, qweight_o, inp.scales, group_size, ms, ns)


# ---------------------------------------------------------------------------
# Which prefill kernel a shape takes and which tiles a split last round holds,
# mirrored from the library's host-side planning (for a 256-CU device) so the
# tests can pick shapes that reach each path; the results are checked against
# the oracle whichever kernel runs.

def _ceil(a: int, b: int) -> int:
    return -(-a // b)


def _wide_plan(M: int, K: int, N: int, cus: int):
    tiles = _ceil(M, 256) * _ceil(N, 256)
    nst = _ceil(K, 64)
    tail = tiles % cus
    if tail == 0 or 2 * tail > cus:
        return tiles, 0, 1
    chunks = min(cus // tail, nst // 8, cus // tail)
    return (tiles, 0, 1) if chunks < 2 else (tiles, tail, chunks)


def _m128_chunks(M: int, K: int, N: int, cus: int) -> int:
    mt_rows = 32 if M <= 32 else 64 if M <= 64 else 128
    tiles = _ceil(N, 256) * _ceil(M, mt_rows)
    chunks = min(cus // tiles, _ceil(K, 64) // 8, cus * 256 * 256 // (M * N))
    return 1 if chunks < 2 else chunks


def prefill_rows(M: int, K: int, N: int, cus: int = 256) -> int:
    """Rows per tile of the prefill kernel the library picks: 128 or 256."""
    if M <= 128:
        return 128
    if M > 1024:
        return 256
    nst = _ceil(K, 64)
    tiles, tail, chunks = _wide_plan(M, K, N, cus)
    if chunks < 2:
        t256 = _ceil(tiles, cus) * nst * 1.15
    else:
        t256 = ((tiles - tail) // cus) * nst * 1.15 + _ceil(nst, chunks) * 1.15 \
            + tail * chunks * 256 * 256 * 4 * 2.0 / 4e6 + 3.0
    tiles128 = _ceil(N, 256) * _ceil(M, 128)
    c = _m128_chunks(M, K, N, cus)
    if c < 2:
        t128 = _ceil(tiles128, cus) * nst * 0.95
    else:
        t128 = _ceil(nst, c) * 0.95 + c * M * N * 4 * 2.0 / 4e6 + 3.0
    return 256 if t256 <= t128 else 128


def wide_tail_tiles(M: int, K: int, N: int, cus: int = 256):
    """(row, column) origins of the 256 x 256 tiles of a split last round,
    in the library's banded tile order (bands of 4 row blocks, each walked
    strip by strip with its row blocks fastest)."""
    tiles, tail, _ = _wide_plan(M, K, N, cus)
    tm, tn = _ceil(M, 256), _ceil(N, 256)
    out = []
    for t in range(tiles - tail, tiles):
        band = t // (4 * tn)
        first = band * 4
        rows = min(tm - first, 4)
        r = t - band * 4 * tn
        out.append(((first + r % rows) * 256, (r // rows) * 256))
    return out
