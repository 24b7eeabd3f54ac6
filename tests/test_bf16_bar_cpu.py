"""The bfloat16 parity bar (gpu_util.check_parity_bf16) on the CPU: outputs that
carry only the variant's own roundings pass it, and plausible mistakes, made
in the oracle's inputs (never in the HIP path), do not."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import bf16_to_float, check_parity_bf16


@pytest.fixture(scope="module")
def case():
    c = workloads.Case("bf16_bar", 4, 1024, 256, 64, 70, scales="loguniform")
    inp = workloads.generate_bf16(c)
    q = oracle.pack(inp.codes)
    y_ref = oracle.linear(inp.x, q, inp.scales, c.group_size, act="bf16")
    mag = oracle.linear(inp.x, q, inp.scales, c.group_size, act="bf16", absval=True)
    return c, inp, q, y_ref, mag


def _as_bf16(y):
    return bf16_to_float(workloads.bf16_bits(y))


def test_rounded_exact_result_passes(case):
    c, inp, q, y_ref, mag = case
    check_parity_bf16(_as_bf16(y_ref), y_ref, mag, c.K, "exact, rounded to bfloat16")


def test_rounded_weights_pass(case):
    """Weights rounded once to bfloat16 (as the variant does), then y rounded."""
    c, inp, q, y_ref, mag = case
    x = bf16_to_float(inp.x)
    W = oracle.dequant(q, inp.scales, c.group_size).astype(np.float64)
    Wb = bf16_to_float(workloads.bf16_bits(W))
    check_parity_bf16(_as_bf16(x @ Wb), y_ref, mag, c.K, "bfloat16 weights")


@pytest.mark.parametrize("mistake", ["dropped_last_step", "scale_1pct", "zero_point_7",
                                     "columns_swapped"])
def test_plausible_mistakes_fail(case, mistake):
    c, inp, q, y_ref, mag = case
    if mistake == "dropped_last_step":
        x = inp.x.copy()
        x[:, -32:] = 0
        y = oracle.linear(x, q, inp.scales, c.group_size, act="bf16")
    elif mistake == "scale_1pct":
        s = (inp.scales.astype(np.float32) * 1.01).astype(np.float16)
        y = oracle.linear(inp.x, q, s, c.group_size, act="bf16")
    elif mistake == "zero_point_7":
        # (q - 7) s = (q - 8) s + s: add x . s per group to the exact result
        x = bf16_to_float(inp.x)
        gidx = np.arange(c.K) // c.group_size
        y = y_ref + x @ inp.scales.astype(np.float64)[gidx]
    else:
        y = y_ref[:, np.r_[1, 0, 2:c.N]]
    with pytest.raises(AssertionError):
        check_parity_bf16(_as_bf16(y), y_ref, mag, c.K, mistake)
