"""Parity of the bfloat16-activation variant (w4a16_linear_bf16) with the CPU
oracle, through the C ABI.

Inputs are the seeded draws of ``workloads`` with x given in bfloat16
(``workloads.generate_bf16``); the oracle decodes those bit patterns itself
and returns y and sum_k |x||w| in float64; the bar is ``check_parity_bf16``
(derived from the variant's stated arithmetic).  Small cases are compared
element by element across decode, both prefill kernels, every group size and
ragged K and N; the model shapes on sampled outputs; and runs must be bitwise
repeatable.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import bf16_to_float, check_parity_bf16, sample_indices

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import int4_weight_only_w4a16_amd as w4  # noqa: E402

DEC, PRE, AUTO = w4.W4A16_KERNEL_DECODE, w4.W4A16_KERNEL_PREFILL, w4.W4A16_KERNEL_AUTO


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    w4.load_library()
    return torch.device("cuda:0")


def _upload(case, dev):
    inp = workloads.generate_bf16(case)
    q = w4.pack_gptq_v2(inp.codes)
    assert np.array_equal(q, oracle.pack(inp.codes))
    x = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).to(dev)
    return inp, q, x, torch.from_numpy(q).to(dev), torch.from_numpy(inp.scales).to(dev)


def _run(x, q, s, g, kernel):
    y = w4.linear(x, q, s, g, kernel=kernel)
    assert y.dtype == torch.bfloat16
    torch.cuda.synchronize()
    return y.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("M,K,N,g,kernels", [
    (1, 256, 256, 32, (DEC, PRE)),
    (1, 5120, 1032, 128, (DEC,)),       # stream-K decode, ragged N
    (3, 2064, 520, 16, (DEC, PRE)),     # g = 16 scale rows, ragged K (K % 32 = 16)
    (8, 1024, 2048, 64, (DEC, PRE)),
    (16, 4096, 1024, 256, (DEC, PRE)),
    (15, 5120, 5120, 128, (DEC,)),      # three ranges per tile, the two-level exchange
    (15, 2048, 17408, 128, (DEC,)),     # one range per CU: partial slots and the reduce kernel
    (64, 1040, 776, -1, (PRE,)),        # 128-row prefill kernel, ragged K and N
    (300, 1536, 1032, 512, (PRE,)),     # 256-row prefill kernel, ragged M and N
    (2, 2048, 4096, 1024, (DEC,)),
    (4, 5120, 2048, 32, (DEC,)),        # one step per group (group end every unit)
    (7, 8192, 1032, -1, (DEC,)),        # one group over K: the longest bias sums
])
def test_bf16_parity_full(dev, M, K, N, g, kernels):
    case = workloads.Case(f"bf16_{M}_{K}_{N}_{g}", M, K, N, g, 50 + M, scales="loguniform")
    inp, q_o, x, q, s = _upload(case, dev)
    y_ref = oracle.linear(inp.x, q_o, inp.scales, g, act="bf16")
    mag = oracle.linear(inp.x, q_o, inp.scales, g, act="bf16", absval=True)
    mag0 = oracle.linear(inp.x, np.zeros_like(q_o), inp.scales, g, act="bf16", absval=True)
    for k in kernels:
        y = bf16_to_float(_run(x, q, s, g, k))
        check_parity_bf16(y, y_ref, mag, K, f"{case.name} kernel={k}", mag0)


@pytest.mark.parametrize("M,K,N,g", [
    (1, 5120, 17408, 128),     # the decode up-projection
    (16, 17408, 5120, 32),     # down projection, 16 rows
    (2048, 5120, 17408, 128),  # the prefill up-projection (split last round)
])
def test_bf16_parity_model_shapes_sampled(dev, M, K, N, g):
    case = workloads.Case(f"bf16_model_{M}", M, K, N, g, 60, scales="uniform")
    inp, q_o, x, q, s = _upload(case, dev)
    ms, ns = sample_indices(M, N, 2048, seed=61)
    y_ref = oracle.linear_at(inp.x, q_o, inp.scales, g, ms, ns, act="bf16")
    mag = oracle.linear_at(inp.x, q_o, inp.scales, g, ms, ns, act="bf16", absval=True)
    mag0 = oracle.linear_at(inp.x, np.zeros_like(q_o), inp.scales, g, ms, ns, act="bf16",
                            absval=True)
    runs = [_run(x, q, s, g, AUTO) for _ in range(2)]
    check_parity_bf16(bf16_to_float(runs[0])[ms, ns], y_ref, mag, K, f"{case.name} (sampled)",
                      mag0)
    assert np.array_equal(runs[0], runs[1]), "bfloat16 results differ between runs"


def test_bf16_all_codes_eight_give_exact_zero(dev):
    K, N, g = 1024, 256, 64
    rng = np.random.default_rng(62)
    q = torch.from_numpy(w4.pack_gptq_v2(np.full((K, N), 8, dtype=np.uint8))).to(dev)
    s = torch.from_numpy(rng.uniform(1e-3, 1.0, size=(K // g, N)).astype(np.float16)).to(dev)
    for M, k in ((1, DEC), (16, DEC), (40, PRE), (257, PRE)):
        bits = workloads.bf16_bits(rng.standard_normal((M, K)))
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        y = w4.linear(x, q, s, g, kernel=k)
        torch.cuda.synchronize()
        assert torch.count_nonzero(y).item() == 0, (M, k)


def test_bf16_rejects_mixed_dtypes(dev):
    K, N = 64, 8
    q = torch.zeros((K // 8, N), dtype=torch.int32, device=dev)
    s = torch.ones((1, N), dtype=torch.float16, device=dev)
    x = torch.zeros((1, K), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        w4.linear(x, q, s, -1, out=torch.empty((1, N), dtype=torch.float16, device=dev))


def test_bf16_decode_tiles_kernel_path(dev):
    """More than 8 column tiles of 64 per CU: the bfloat16 decode runs one
    workgroup per tile (the tiles kernel), in all three of its weight forms:
    dequantised before the matrix core (g = 16), offset folded per group with
    one step per group (g = 32) and over several steps (g = 64)."""
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = 8 * 64 * n_cus + 8
    for M, K, g in ((1, 64, 32), (5, 64, 16), (3, 128, 64)):
        case = workloads.Case(f"bf16_tiles_{M}_{g}", M, K, N, g, 64 + M, scales="loguniform")
        inp, q_o, x, q, s = _upload(case, dev)
        y_ref = oracle.linear(inp.x, q_o, inp.scales, g, act="bf16")
        mag = oracle.linear(inp.x, q_o, inp.scales, g, act="bf16", absval=True)
        mag0 = oracle.linear(inp.x, np.zeros_like(q_o), inp.scales, g, act="bf16", absval=True)
        y = bf16_to_float(_run(x, q, s, g, DEC))
        check_parity_bf16(y, y_ref, mag, K, f"bf16 tiles path M={M} g={g}", mag0)


def test_bf16_graph_capture_on_fresh_stream(dev):
    """bfloat16 decode and prefill captured on a stream that has no workspace yet
    (the decode then runs its tiles kernel, the prefill whole tiles), replayed
    several times with eager work in between; every replay within the bar."""
    cases = [workloads.Case("bf16_g_dec", 4, 5120, 2048, 128, 66, scales="loguniform"),
             workloads.Case("bf16_g_dec32", 1, 2048, 1032, 32, 67, scales="loguniform"),
             workloads.Case("bf16_g_pre", 96, 1024, 1032, 64, 68, scales="loguniform")]
    prepared = []
    for c in cases:
        inp, q_o, x, q, s = _upload(c, dev)
        ref = oracle.linear(inp.x, q_o, inp.scales, c.group_size, act="bf16")
        mag = oracle.linear(inp.x, q_o, inp.scales, c.group_size, act="bf16", absval=True)
        mag0 = oracle.linear(inp.x, np.zeros_like(q_o), inp.scales, c.group_size, act="bf16",
                             absval=True)
        prepared.append((c, x, q, s, ref, mag, mag0))
    st = torch.cuda.Stream()
    outs = [torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev) for c, *_ in prepared]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        for (c, x, q, s, *_), y in zip(prepared, outs):
            w4.w4a16_linear_bf16(x, q, s, y, c.M, c.K, c.N, c.group_size, st)
    first = None
    for rep in range(3):
        for y in outs:
            y.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [y.cpu().view(torch.int16).numpy().copy() for y in outs]
        for (c, x, q, s, ref, mag, mag0), bits in zip(prepared, got):
            check_parity_bf16(bf16_to_float(bits), ref, mag, c.K, f"{c.name} replay {rep}", mag0)
        if first is None:
            first = got
        else:
            assert all(np.array_equal(a, b) for a, b in zip(first, got)), rep
