"""The gate/up SiLU * mul parity bar on the CPU: exact results rounded to fp16
pass it, plausible mistakes (computed from the oracle's outputs, never from
the HIP path) do not."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import check_gate_up


@pytest.fixture(scope="module")
def case():
    c = workloads.Case("gu_bar", 4, 1024, 512, 64, 92, scales="loguniform")
    inp = workloads.generate(c)
    q = oracle.pack(inp.codes)
    ref = oracle.gate_up_silu(inp.x, q, inp.scales, c.group_size)
    lin = oracle.linear(inp.x, q, inp.scales, c.group_size)
    mag = oracle.linear(inp.x, q, inp.scales, c.group_size, absval=True)
    return c, inp, q, ref, lin, mag


def _f16(v):
    return v.astype(np.float16).astype(np.float64)


def test_rounded_exact_passes(case):
    c, inp, q, ref, lin, mag = case
    check_gate_up(_f16(ref), ref, lin, mag, None, c.K, False, "exact")


@pytest.mark.parametrize("mistake", ["swapped", "silu_sign", "no_silu", "dropped_step"])
def test_mistakes_fail(case, mistake):
    c, inp, q, ref, lin, mag = case
    g, u = lin[:, 0::2], lin[:, 1::2]
    if mistake == "swapped":
        y = u / (1.0 + np.exp(-u)) * g
    elif mistake == "silu_sign":
        y = g / (1.0 + np.exp(g)) * u
    elif mistake == "no_silu":
        y = g * u
    else:
        x = inp.x.copy()
        x[:, -32:] = 0
        y = oracle.gate_up_silu(x, q, inp.scales, c.group_size)
    with pytest.raises(AssertionError):
        check_gate_up(_f16(y), ref, lin, mag, None, c.K, False, mistake)
