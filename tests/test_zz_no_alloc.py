"""w4a16_linear_noalloc (the entry point that allocates nothing: its split-K
scratch is the library's file-scope device array) against w4a16_linear and the
oracle, through the C ABI on cuda:0.

Two calls in a row, the second with a smaller input, on the decode kernel
(stream-K with the exchange slots, the two-level exchange, and with partial slots and the reduce
kernel), the small-M prefill kernel (split K) and the wide prefill kernel
(split last round); free device memory unchanged across the calls; and a call
captured on a stream with nothing allocated for it replays to the eager bits.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import check_parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import int4_weight_only_w4a16_amd as w4  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    w4.load_library()
    return torch.device("cuda:0")


def _prepare(M, K, N, g, seed, dev):
    case = workloads.Case(f"noalloc_{M}_{K}_{N}_{g}", M, K, N, g, seed)
    inp = workloads.generate(case)
    q_o = oracle.pack(inp.codes)
    # the dense form for the 2048-row case (the triple loop would take minutes)
    ref = (oracle.linear_dense(inp.x, q_o, inp.scales, g) if M * K * N > 10 ** 10
           else oracle.linear(inp.x, q_o, inp.scales, g))
    return (case, torch.from_numpy(inp.x).to(dev), torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev),
            torch.from_numpy(inp.scales).to(dev), ref)


# pairs of calls: the second smaller than the first
PAIRS = [
    ((1, 5120, 17408, 128), (1, 2048, 4096, 32)),      # decode: exchange slots
    ((16, 5120, 5120, 64), (4, 1024, 2048, 128)),      # decode: three ranges per tile
    ((16, 2048, 17408, 64), (15, 2048, 8192, 128)),    # decode: partial slots + reduce kernel
    ((64, 5120, 5120, 128), (40, 2048, 1024, 32)),     # 128-row prefill: split K
    ((2048, 5120, 17408, 128), (1100, 1024, 1024, 64)),  # 256-row prefill: split last round (20 tiles x 2)
]


def _free_bytes():
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


@pytest.mark.parametrize("first,second", PAIRS, ids=lambda p: "x".join(map(str, p)))
def test_noalloc_matches_linear_two_calls(dev, first, second):
    runs = [_prepare(*first, 31, dev), _prepare(*second, 32, dev)]
    outs = []
    for case, x, q, s, ref in runs:
        y = torch.full((case.M, case.N), 7.0, dtype=torch.float16, device=dev)
        outs.append(y)
    # one call before measuring: the first call on a device looks up the array's address
    w4.w4a16_linear_noalloc(runs[1][1], runs[1][2], runs[1][3], outs[1], runs[1][0].M,
                            runs[1][0].K, runs[1][0].N, runs[1][0].group_size)
    free0 = _free_bytes()
    for (case, x, q, s, ref), y in zip(runs, outs):        # two calls in a row
        w4.w4a16_linear_noalloc(x, q, s, y, case.M, case.K, case.N, case.group_size)
    assert _free_bytes() == free0, "w4a16_linear_noalloc changed free device memory"
    for (case, x, q, s, ref), y in zip(runs, outs):
        got = y.cpu().numpy()
        check_parity(got, ref, f"noalloc {case.name}")
        lin = w4.linear(x, q, s, case.group_size)
        torch.cuda.synchronize()
        check_parity(got.astype(np.float64), lin.cpu().numpy().astype(np.float64),
                     f"noalloc vs w4a16_linear {case.name}")
        if case.M <= w4.W4A16_DECODE_MAX_M:          # same plan: the same bits
            assert torch.equal(y, lin), case.name


def test_noalloc_graph_capture_from_the_first_call_on_a_stream(dev):
    """Captured on a fresh stream (nothing allocated for it), the call runs the
    same kernels as eagerly: every replay equals the eager result bit for bit."""
    runs = [_prepare(4, 5120, 2048, 128, 33, dev), _prepare(96, 1024, 1032, 64, 34, dev),
            _prepare(300, 2048, 2048, 128, 35, dev)]
    eager = []
    for case, x, q, s, ref in runs:
        y = torch.empty((case.M, case.N), dtype=torch.float16, device=dev)
        w4.w4a16_linear_noalloc(x, q, s, y, case.M, case.K, case.N, case.group_size)
        eager.append(y)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    outs = [torch.empty_like(e) for e in eager]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        for (case, x, q, s, ref), y in zip(runs, outs):
            w4.w4a16_linear_noalloc(x, q, s, y, case.M, case.K, case.N, case.group_size, st)
    for rep in range(3):
        for y in outs:
            y.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (case, *_), y, e in zip(runs, outs, eager):
            assert torch.equal(y, e), (case.name, rep)
    for (case, x, q, s, ref), e in zip(runs, eager):
        check_parity(e.cpu().numpy(), ref, f"noalloc eager {case.name}")


def test_noalloc_rejects_invalid_arguments_before_any_launch(dev):
    y = torch.full((1, 8), 5.0, dtype=torch.float16, device=dev)
    x = torch.zeros((1, 24), dtype=torch.float16, device=dev)
    q = torch.zeros((3, 8), dtype=torch.int32, device=dev)
    s = torch.ones((1, 8), dtype=torch.float16, device=dev)
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_linear_noalloc(x, q, s, y, 1, 24, 8, -1)           # K % 16 != 0
    assert e.value.status == w4.W4A16_ERR_SHAPE
    torch.cuda.synchronize()
    assert torch.all(y == 5.0).item()
