"""Parity of the merged gate/up projection with the fused SiLU * mul epilogue
(w4a16_gate_up_silu, columns alternating gate and up) with the CPU oracle,
through the C ABI, for fp16 and bfloat16 activations.

The bar follows from the arithmetic: the kernels form the gate and up sums g
and u as the linear does (error at most eps * sum|x||w| per column, eps the
linear's weight rounding plus K 2^-24 of fp32 accumulation), take silu(g) * u
in fp32 (|silu'| <= 1.1) and round once to the output type (half an ulp):
  |y - y_ref| <= r |y_ref| + 1.02 (1.1 |u| eps A_g + |silu(g)| eps A_u
                                   + 1.1 eps^2 A_g A_u) + 4e-7 |y_ref|
with A_g, A_u the oracle's magnitude sums of the two columns; plus the mean
relative error of the linear's bar.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import bf16_to_float, check_gate_up, prefill_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import int4_weight_only_w4a16_amd as w4  # noqa: E402

DEC, PRE, AUTO = w4.W4A16_KERNEL_DECODE, w4.W4A16_KERNEL_PREFILL, w4.W4A16_KERNEL_AUTO


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    w4.load_library()
    return torch.device("cuda:0")


def _case(M, K, N, g, seed, bf16):
    c = workloads.Case(f"gu_{M}_{K}_{N}_{g}", M, K, N, g, seed, scales="loguniform")
    return c, (workloads.generate_bf16(c) if bf16 else workloads.generate(c))


def _run(inp, q, s, g, kernel, bf16, dev):
    if bf16:
        x = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        x = torch.from_numpy(inp.x).to(dev)
    y = w4.gate_up_silu(x, q, s, g, kernel=kernel)
    torch.cuda.synchronize()
    if bf16:
        return bf16_to_float(y.cpu().view(torch.int16).numpy())
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("bf16", [False, True], ids=["fp16", "bf16"])
@pytest.mark.parametrize("M,K,N,g,kernels", [
    (1, 5120, 2048, 128, (DEC, PRE)),    # stream-K decode: exchange slots
    (4, 2064, 1040, 16, (DEC, PRE)),     # g = 16, ragged K, ragged tiles
    (16, 4096, 1024, 64, (DEC,)),        # three ranges per tile, the two-level exchange
    (16, 1024, 17408, 64, (DEC,)),       # one range per CU: partial slots and the reduce kernel
    (64, 2048, 4096, -1, (PRE,)),        # 128-row prefill, split K
    (300, 1024, 1056, 32, (PRE,)),       # 128-row prefill, three row blocks, split K
    (1100, 1024, 528, 32, (PRE,)),       # 256-row prefill, ragged M: all 15 tiles split along K,
                                         # sums reduced with SiLU applied by the reduce kernel
])
def test_gate_up_silu_parity(dev, bf16, M, K, N, g, kernels):
    if M > 128:
        assert prefill_rows(M, K, N) == (256 if M > 1024 else 128)
    case, inp = _case(M, K, N, g, 80 + M, bf16)
    act = "bf16" if bf16 else "f16"
    q_o = oracle.pack(inp.codes)
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    s = torch.from_numpy(inp.scales).to(dev)
    ref = oracle.gate_up_silu(inp.x, q_o, inp.scales, g, act=act)
    lin = oracle.linear(inp.x, q_o, inp.scales, g, act=act)
    mag = oracle.linear(inp.x, q_o, inp.scales, g, act=act, absval=True)
    mag0 = oracle.linear(inp.x, np.zeros_like(q_o), inp.scales, g, act=act, absval=True)
    for k in kernels:
        runs = [_run(inp, q, s, g, k, bf16, dev) for _ in range(2)]
        check_gate_up(runs[0], ref, lin, mag, mag0, K, bf16, f"{case.name} {act} kernel={k}")
        assert np.array_equal(runs[0], runs[1]), "results differ between runs"


def test_gate_up_silu_model_shape(dev):
    """The pages' 27B MLP: K=5120, gate and up of 17408 each (N = 34816), M=1."""
    case, inp = _case(1, 5120, 34816, 128, 90, False)
    q_o = oracle.pack(inp.codes)
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    s = torch.from_numpy(inp.scales).to(dev)
    ref = oracle.gate_up_silu(inp.x, q_o, inp.scales, 128)
    lin = oracle.linear(inp.x, q_o, inp.scales, 128)
    mag = oracle.linear(inp.x, q_o, inp.scales, 128, absval=True)
    y = _run(inp, q, s, 128, AUTO, False, dev)
    assert y.shape == (1, 17408)
    check_gate_up(y, ref, lin, mag, None, 5120, False, "gate_up model shape")


@pytest.mark.parametrize("bf16", [False, True], ids=["fp16", "bf16"])
def test_gate_up_prefill_model_shape_sampled(dev, bf16):
    """The 27B MLP at M = 2048 (K=5120, N = 2 x 17408): 1024 whole tiles with
    the SiLU epilogue and a last round of 64 tiles split along K, whose sums
    the reduce kernel turns into silu(gate) * up.  Checked on 4096 sampled
    outputs, half of them in the split tiles (outputs 16384 .. 17407), against
    the oracle's linear at both columns of each pair with SiLU applied to the
    gate in float64 (the oracle's gate/up definition)."""
    c = workloads.gate_up_prefill()
    inp = workloads.generate_bf16(c) if bf16 else workloads.generate(c)
    act = "bf16" if bf16 else "f16"
    M, K, N, g = c.M, c.K, c.N, c.group_size
    q_o = oracle.pack(inp.codes)
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    s = torch.from_numpy(inp.scales).to(dev)
    y = _run(inp, q, s, g, AUTO, bf16, dev)
    y2 = _run(inp, q, s, g, AUTO, bf16, dev)
    assert np.array_equal(y, y2), "results differ between runs"
    rng = np.random.default_rng(92)
    ms = rng.integers(0, M, size=4096)
    js = np.concatenate([rng.integers(0, N // 2, size=2048),
                         rng.integers(N // 2 - 1024, N // 2, size=2048)])
    cols = np.stack([2 * js, 2 * js + 1], axis=1).reshape(-1)
    rows = np.repeat(ms, 2)
    lin = oracle.linear_at(inp.x, q_o, inp.scales, g, rows, cols, act=act).reshape(1, -1)
    mag = oracle.linear_at(inp.x, q_o, inp.scales, g, rows, cols, act=act,
                           absval=True).reshape(1, -1)
    mag0 = oracle.linear_at(inp.x, np.zeros_like(q_o), inp.scales, g, rows, cols, act=act,
                            absval=True).reshape(1, -1)
    gg, uu = lin[:, 0::2], lin[:, 1::2]
    with np.errstate(over="ignore"):
        ref = gg / (1.0 + np.exp(-gg)) * uu
    check_gate_up(y[ms, js].reshape(1, -1), ref, lin, mag, mag0, K, bf16,
                  f"gate_up prefill model shape {act}")


def test_gate_up_silu_zero_gate_gives_exact_zero(dev):
    K, N, g = 1024, 512, 64
    rng = np.random.default_rng(91)
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    codes[:, 0::2] = 8                               # gate weights all zero
    q = torch.from_numpy(w4.pack_gptq_v2(codes)).to(dev)
    s = torch.from_numpy(rng.uniform(1e-3, 1.0, size=(K // g, N)).astype(np.float16)).to(dev)
    for M, k in ((1, DEC), (16, DEC), (40, PRE), (257, PRE)):
        x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float16)).to(dev)
        y = w4.gate_up_silu(x, q, s, g, kernel=k)
        torch.cuda.synchronize()
        assert y.shape == (M, N // 2) and torch.count_nonzero(y).item() == 0, (M, k)


@pytest.mark.parametrize("bf16", [False, True], ids=["fp16", "bf16"])
def test_gate_up_decode_tiles_kernel_path(dev, bf16):
    """More than 8 column tiles of 64 per CU (merged width N > 8 * 64 * CUs):
    the SiLU * mul epilogue of the decode tiles kernel, fp16 and bfloat16."""
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = 8 * 64 * n_cus + 16
    act = "bf16" if bf16 else "f16"
    for M, K, g in ((1, 64, 32), (6, 64, 16), (3, 128, 64)):
        case, inp = _case(M, K, N, g, 92 + M, bf16)
        q_o = oracle.pack(inp.codes)
        q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
        s = torch.from_numpy(inp.scales).to(dev)
        ref = oracle.gate_up_silu(inp.x, q_o, inp.scales, g, act=act)
        lin = oracle.linear(inp.x, q_o, inp.scales, g, act=act)
        mag = oracle.linear(inp.x, q_o, inp.scales, g, act=act, absval=True)
        mag0 = oracle.linear(inp.x, np.zeros_like(q_o), inp.scales, g, act=act, absval=True)
        y = _run(inp, q, s, g, DEC, bf16, dev)
        check_gate_up(y, ref, lin, mag, mag0, K, bf16, f"gate_up tiles M={M} g={g} {act}")


@pytest.mark.parametrize("bf16", [False, True], ids=["fp16", "bf16"])
def test_gate_up_graph_capture_on_fresh_stream(dev, bf16):
    """Merged gate/up calls captured on a stream with no workspace yet (decode:
    the tiles kernel; prefill: whole tiles) and replayed several times; every
    replay within the bar and equal to the first."""
    act = "bf16" if bf16 else "f16"
    prepared = []
    for M, K, N, g in ((4, 5120, 2048, 128), (1, 2048, 1040, 32), (80, 1024, 1056, 64),
                       (300, 1024, 1056, 32)):
        case, inp = _case(M, K, N, g, 95 + M, bf16)
        q_o = oracle.pack(inp.codes)
        if bf16:
            x = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            x = torch.from_numpy(inp.x).to(dev)
        prepared.append((case, x, torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev),
                         torch.from_numpy(inp.scales).to(dev),
                         oracle.gate_up_silu(inp.x, q_o, inp.scales, g, act=act),
                         oracle.linear(inp.x, q_o, inp.scales, g, act=act),
                         oracle.linear(inp.x, q_o, inp.scales, g, act=act, absval=True),
                         oracle.linear(inp.x, np.zeros_like(q_o), inp.scales, g, act=act,
                                       absval=True)))
    st = torch.cuda.Stream()
    dt = torch.bfloat16 if bf16 else torch.float16
    outs = [torch.empty((c.M, c.N // 2), dtype=dt, device=dev) for c, *_ in prepared]
    call = w4.w4a16_gate_up_silu_bf16 if bf16 else w4.w4a16_gate_up_silu
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        for (c, x, q, s, *_), y in zip(prepared, outs):
            call(x, q, s, y, c.M, c.K, c.N, c.group_size, st)
    first = None
    for rep in range(3):
        for y in outs:
            y.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = []
        for (c, x, q, s, ref, lin, mag, mag0), y in zip(prepared, outs):
            h = y.cpu()
            v = bf16_to_float(h.view(torch.int16).numpy()) if bf16 else h.numpy().astype(np.float64)
            check_gate_up(v, ref, lin, mag, mag0, c.K, bf16, f"{c.name} {act} replay {rep}")
            got.append(v)
        if first is None:
            first = got
        else:
            assert all(np.array_equal(a, b) for a, b in zip(first, got)), rep
