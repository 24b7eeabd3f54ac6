"""The parity bars of the LoRA and zero-point paths, on the CPU: outputs that carry
only the roundings the C ABI states for them pass, and plausible mistakes fail.

The "GPU-like" outputs are built in numpy from the oracle's exact parts with the
stated roundings (the linear rounded once, t or the group sums and C rounded to
the activation type, fp32 products, y rounded once); the mistakes are planted in
those numpy outputs, never in the oracle or the kernels.
"""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import bf16_to_float, check_parity, check_parity_bf16, lora_extra_bound

S = workloads.LORA_SCALE


def _round(v, act):
    if act == "f16":
        return v.astype(np.float16).astype(np.float64)
    return bf16_to_float(workloads.bf16_bits(v))


def _lora_parts(act, M=3, K=512, N=136, g=32, r=16, seed=11):
    case = workloads.Case("bar_lora", M, K, N, g, seed)
    inp = workloads.generate(case, act=act)
    A, B = workloads.lora_adapter(K, N, r, seed + 500, act=act)
    q = oracle.pack(inp.codes)
    lin = oracle.linear(inp.x, q, inp.scales, g, act=act)
    t = oracle.lora_shrink(inp.x, A, act=act)
    Bv = B.astype(np.float64) if act == "f16" else bf16_to_float(B)
    ref = oracle.linear_lora(inp.x, q, inp.scales, g, A, B, S, act=act)
    return inp, q, A, B, Bv, lin, t, ref


def _lora_gpu_like(lin, t, Bv, act, sign=1.0, scale=S, perm=None):
    d = _round(t, act) @ (Bv if perm is None else Bv[perm]).T
    return _round(_round(lin, act) + sign * scale * d, act)


def _lora_check(act, y, inp, q, A, B, lin, t, ref, K=512, r=16, g=32):
    if act == "f16":
        return check_parity(y, ref, "lora bar")
    mag = oracle.linear(inp.x, q, inp.scales, g, act="bf16", absval=True)
    mag0 = oracle.linear(inp.x, np.zeros_like(q), inp.scales, g, act="bf16", absval=True)
    p1 = oracle.lora_expand(t, B, S, act="bf16", absval=True)
    p2 = oracle.lora_expand(oracle.lora_shrink(inp.x, A, act="bf16", absval=True), B, S,
                            act="bf16", absval=True)
    extra = lora_extra_bound(lin, ref, p1, p2, K, r, 2.0 ** -8)
    return check_parity_bf16(y, ref, mag, K, "lora bar", mag0=mag0, extra=extra)


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_lora_bar_passes_the_stated_roundings_and_rejects_mistakes(act):
    inp, q, A, B, Bv, lin, t, ref = _lora_parts(act)
    _lora_check(act, _lora_gpu_like(lin, t, Bv, act), inp, q, A, B, lin, t, ref)
    r = Bv.shape[1]
    mistakes = {
        "term subtracted": _lora_gpu_like(lin, t, Bv, act, sign=-1.0),
        "scale dropped": _lora_gpu_like(lin, t, Bv, act, scale=1.0),
        "term dropped": _round(lin, act),
        "B rows of the neighbouring column": _lora_gpu_like(lin, t, Bv, act,
                                                            perm=np.arange(Bv.shape[0]) ^ 1),
        "last rank dropped": _round(_round(lin, act) + S * (_round(t[:, : r - 1], act)
                                                            @ Bv[:, : r - 1].T), act),
    }
    for name, y in mistakes.items():
        with pytest.raises(AssertionError):
            _lora_check(act, y, inp, q, A, B, lin, t, ref)
            raise RuntimeError(f"the bar let '{name}' through")


def _zp_parts(act, M=4, K=512, N=136, g=64, seed=12):
    case = workloads.Case("bar_zp", M, K, N, g, seed)
    inp = workloads.generate(case, act=act)
    z = workloads.zero_points(case.G, N, seed + 700)
    q = oracle.pack(inp.codes)
    qz = np.ascontiguousarray(oracle.pack(np.ascontiguousarray(z.T)).T)
    sym = oracle.linear(inp.x, q, inp.scales, g, act=act)
    xv = inp.x.astype(np.float64) if act == "f16" else bf16_to_float(inp.x)
    X = xv.reshape(M, K // g, g).sum(axis=2)                       # group sums
    C = (8.0 - z.astype(np.float64)) * inp.scales.astype(np.float64)
    ref = oracle.linear_zp(inp.x, q, inp.scales, qz, g, act=act)
    return case, inp, z, q, sym, X, C, ref


def _zp_check(act, y, case, inp, z, q, sym, ref):
    K, g = case.K, case.group_size
    if act == "f16":
        return check_parity(y, ref, "zp bar")
    u = 2.0 ** -8
    mag = oracle.linear(inp.x, q, inp.scales, g, act="bf16", absval=True)
    mag0 = oracle.linear(inp.x, np.zeros_like(q), inp.scales, g, act="bf16", absval=True)
    P = oracle.linear(inp.x, oracle.pack(np.repeat(z, g, axis=0)), inp.scales, g, act="bf16",
                      absval=True)
    extra = 1.02 * (u * np.abs(sym) + u * np.abs(ref) + (2 * u + K * 2.0 ** -24) * P)
    return check_parity_bf16(y, ref, mag, K, "zp bar", mag0=mag0, extra=extra)


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_zp_bar_passes_the_stated_roundings_and_rejects_mistakes(act):
    case, inp, z, q, sym, X, C, ref = _zp_parts(act)
    good = _round(_round(sym, act) + _round(X, act) @ _round(C, act), act)
    _zp_check(act, good, case, inp, z, q, sym, ref)
    zr = z.reshape(z.shape[0], -1, 8)[:, :, ::-1].reshape(z.shape)    # nibbles reversed
    mistakes = {
        "correction subtracted": _round(_round(sym, act) - _round(X, act) @ _round(C, act), act),
        "correction dropped": _round(sym, act),
        "zero point added": _round(_round(sym, act) + _round(X, act) @ _round(
            (z.astype(np.float64) - 8.0) * inp.scales.astype(np.float64), act), act),
        "zero-point nibbles reversed": _round(_round(sym, act) + _round(X, act) @ _round(
            (8.0 - zr.astype(np.float64)) * inp.scales.astype(np.float64), act), act),
    }
    for name, y in mistakes.items():
        with pytest.raises(AssertionError):
            _zp_check(act, y, case, inp, z, q, sym, ref)
            raise RuntimeError(f"the bar let '{name}' through")
