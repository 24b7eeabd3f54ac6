"""Asymmetric weights with stored zero points (w4a16_linear_zp, _bf16) against
the oracle, through the C ABI on cuda:0.

Zero points are drawn uniform over 0..15 (``workloads.zero_points``), so the
correction (8 - z) s is of the order of the weights themselves and a mistake
in it cannot hide inside the linear's tolerance.  fp16: the tolerance of
``gpu_util.check_parity``; bfloat16: the symmetric linear's per-element bound
plus the terms the C ABI states for the correction.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import bf16_to_float, check_parity, check_parity_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import int4_weight_only_w4a16_amd as w4  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    w4.load_library()
    return torch.device("cuda:0")


def _inputs(M, K, N, g, seed, act, zeros=None):
    case = workloads.Case(f"zp_M{M}_K{K}_N{N}_g{g}", M, K, N, g, seed)
    inp = workloads.generate(case, act=act)
    z = workloads.zero_points(case.G, N, seed + 700) if zeros is None else zeros
    return case, inp, z


def _upload_x(x, bf16, dev):
    x = np.ascontiguousarray(x)
    if bf16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(x).to(dev)


def _run(inp, z, g, dev, bf16):
    x = _upload_x(inp.x, bf16, dev)
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    s = torch.from_numpy(inp.scales).to(dev)
    qz = torch.from_numpy(w4.pack_zeros(z)).to(dev)
    y = w4.linear_zp(x, q, s, qz, g)
    torch.cuda.synchronize()
    out = y.cpu()
    return bf16_to_float(out.view(torch.int16).numpy()) if bf16 else out.numpy()


def _zero_codes(case, z):
    """Codes [K, N] holding each row's zero point: |q - 8| s is then |8 - z| s."""
    g = case.K if case.group_size == -1 else case.group_size
    return np.repeat(z, g, axis=0)[: case.K]


def _check(case, inp, z, y, act):
    q_o = oracle.pack(inp.codes)
    qz_o = np.ascontiguousarray(oracle.pack(np.ascontiguousarray(z.T)).T)
    g, K = case.group_size, case.K
    ref = oracle.linear_zp(inp.x, q_o, inp.scales, qz_o, g, act=act)
    what = f"{case.name} {act}"
    if act == "f16":
        return check_parity(y, ref, what)
    u = 2.0 ** -8
    sym = oracle.linear(inp.x, q_o, inp.scales, g, act="bf16")
    mag = oracle.linear(inp.x, q_o, inp.scales, g, act="bf16", absval=True)
    mag0 = oracle.linear(inp.x, np.zeros_like(q_o), inp.scales, g, act="bf16", absval=True)
    P = oracle.linear(inp.x, oracle.pack(_zero_codes(case, z)), inp.scales, g, act="bf16",
                      absval=True)
    extra = 1.02 * (u * np.abs(sym) + u * np.abs(ref) + (2 * u + K * 2.0 ** -24) * P)
    return check_parity_bf16(y, ref, mag, K, what, mag0=mag0, extra=extra)


CASES = [
    # M, K, N, g
    (1, 5120, 17408, 128),          # decode up-projection shape
    (4, 1024, 264, 32),
    (16, 2048, 1032, 16),
    (3, 1040, 136, 16),             # K % 32 == 16, a partial rank block
    (2, 1024, 72, 512),             # two whole groups of 512 (one wave per row and group)
    (17, 1024, 520, -1),            # one group: rank 1 padded to 8
    (100, 1024, 264, 64),
    (129, 512, 264, 128),
    (256, 2048, 1024, 256),
    (33, 4096, 264, 1024),
    (300, 1024, 264, 64),           # 128-row prefill, three row blocks, split K
    (1100, 1024, 264, 128),         # 256-row prefill, split last round
]


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("M,K,N,g", CASES)
def test_zp_parity(dev, M, K, N, g, act):
    case, inp, z = _inputs(M, K, N, g, 80 + M, act)
    y = _run(inp, z, g, dev, act == "bf16")
    _check(case, inp, z, y, act)


# A short last group (K % g != 0: G = ceil(K / g), the last group holds K - (G-1) g
# rows), on both ways the group sums are taken: one thread per row and group
# (g <= 256) and one wave per row and group (g > 256), at decode and prefill
# widths (M <= 16, 17..128, > 128).
PARTIAL_GROUP_CASES = [
    # M, K, N, g              last group
    (3, 272, 136, 256),     # 16 of 256, thread per group
    (20, 400, 264, 64),     # 16 of 64
    (130, 1040, 264, 128),  # 16 of 128
    (2, 1040, 72, 1024),    # 16 of 1024, wave per group
    (40, 1552, 264, 512),   # 16 of 512
    (200, 2064, 264, 1024), # 16 of 1024
    (9, 1104, 136, 512),    # 80 of 512
]


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("M,K,N,g", PARTIAL_GROUP_CASES)
def test_zp_partial_last_group(dev, M, K, N, g, act):
    assert K % g != 0
    case, inp, z = _inputs(M, K, N, g, 180 + M, act)
    assert case.G == -(-K // g)
    y = _run(inp, z, g, dev, act == "bf16")
    _check(case, inp, z, y, act)


def test_zp_prefill_full_shape_sampled(dev):
    """The prefill up-projection shape (M=2048, K=5120, N=17408, g=128) with stored
    zero points: sampled outputs plus whole first and last rows, from the oracle."""
    M, K, N, g = 2048, 5120, 17408, 128
    case, inp, z = _inputs(M, K, N, g, 3, "f16")
    y = _run(inp, z, g, dev, False)
    rng = np.random.default_rng(78)
    ms = np.concatenate([rng.integers(0, M, 4096), np.zeros(N, np.int64), np.full(N, M - 1, np.int64)])
    ns = np.concatenate([rng.integers(0, N, 4096), np.arange(N), np.arange(N)])
    qz_o = np.ascontiguousarray(oracle.pack(np.ascontiguousarray(z.T)).T)
    ref = oracle.linear_zp_at(inp.x, oracle.pack(inp.codes), inp.scales, qz_o, g, ms, ns)
    check_parity(y[ms, ns], ref, "zero points prefill_up (sampled)")


@pytest.mark.parametrize("M", [2, 20])
def test_zp_largest_group_count(dev, M):
    """1536 groups (K = 24576, g = 16), the most the call takes: the expand's t
    tile in LDS is at its largest (49 KiB, plus the delta tile), for the decode
    (M <= 16) and the prefill tile widths."""
    K, N, g = 16 * 1536, 264, 16
    case, inp, z = _inputs(M, K, N, g, 60 + M, "f16")
    assert w4.w4a16_zp_workspace_bytes(M, K, N, g) > 0
    y = _run(inp, z, g, dev, False)
    _check(case, inp, z, y, "f16")


@pytest.mark.parametrize("bf16", [False, True])
def test_zp_all_eight_is_the_symmetric_linear_bitwise(dev, bf16):
    """Every zero point 8 makes the correction exactly zero: y equals the
    symmetric linear bit for bit (decode and prefill)."""
    act = "bf16" if bf16 else "f16"
    for M, K, N, g in ((1, 2048, 1032, 32), (40, 1024, 520, 16), (300, 1024, 264, 128)):
        case = workloads.Case("zp8", M, K, N, g, 9)
        z8 = np.full((case.G, N), 8, dtype=np.uint8)
        _, inp, _ = _inputs(M, K, N, g, 9, act, zeros=z8)
        y = _run(inp, z8, g, dev, bf16)
        x = _upload_x(inp.x, bf16, dev)
        q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
        s = torch.from_numpy(inp.scales).to(dev)
        lin = w4.linear(x, q, s, g).cpu()
        lin = bf16_to_float(lin.view(torch.int16).numpy()) if bf16 else lin.numpy()
        assert np.array_equal(y, lin), (M, K, N, g)


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_zp_deterministic_and_graph_replay(dev, act):
    """Two eager calls agree bit for bit; the call captured in a HIP graph on a
    stream that already holds the linear's workspaces replays to the same bits."""
    st = torch.cuda.Stream()
    runs = []
    for M, K, N, g in ((1, 5120, 2048, 128), (64, 1024, 1032, 32), (300, 2048, 1024, 64)):
        case, inp, z = _inputs(M, K, N, g, 97, act)
        x = _upload_x(inp.x, act == "bf16", dev)
        q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
        s = torch.from_numpy(inp.scales).to(dev)
        qz = torch.from_numpy(w4.pack_zeros(z)).to(dev)
        ws = torch.empty(w4.w4a16_zp_workspace_bytes(M, K, N, g), dtype=torch.uint8, device=dev)
        e1 = w4.linear_zp(x, q, s, qz, g, workspace=ws, stream=st)
        e2 = w4.linear_zp(x, q, s, qz, g, workspace=ws, stream=st)
        torch.cuda.synchronize()
        assert torch.equal(e1, e2), (M, K, N, g)
        runs.append((x, q, s, qz, g, ws, e1, torch.empty_like(e1)))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        for x, q, s, qz, g, ws, _, out in runs:
            w4.linear_zp(x, q, s, qz, g, out=out, workspace=ws, stream=st)
    for rep in range(3):
        for *_, out in runs:
            out.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (*_, eager, out) in enumerate(runs):
            assert torch.equal(out, eager), (i, rep)
