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
