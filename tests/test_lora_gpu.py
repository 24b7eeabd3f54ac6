"""LoRA adapter on the quantised linear (w4a16_linear_lora, _bf16) against the
oracle, through the C ABI on cuda:0.

y = x . dequant(qweight, scales) + s * (x . A^T) . B^T with A [r, K] and
B [N, r] drawn by ``workloads.lora_adapter`` (the term is of the order of the
base output, so a mistake in it cannot hide inside the linear's tolerance).
fp16: the tolerance of ``gpu_util.check_parity``; bfloat16: the per-element
bound of the bfloat16 linear plus the LoRA terms the C ABI states
(``gpu_util.lora_extra_bound``).  A case with all-zero scales leaves only the
adapter term, checked against the oracle's term alone.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (bf16_to_float, check_parity, check_parity_bf16, lora_extra_bound,
                      sample_indices)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import int4_weight_only_w4a16_amd as w4  # noqa: E402

S = workloads.LORA_SCALE


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    w4.load_library()
    return torch.device("cuda:0")


def _inputs(M, K, N, g, r, seed, act):
    case = workloads.Case(f"lora_M{M}_K{K}_N{N}_g{g}_r{r}", M, K, N, g, seed)
    inp = workloads.generate(case, act=act)
    A, B = workloads.lora_adapter(K, N, r, seed + 500, act=act)
    return case, inp, A, B


def _run(inp, A, B, g, dev, bf16, scale=S, scales=None):
    dt = torch.bfloat16 if bf16 else torch.float16

    def up(a):
        a = np.ascontiguousarray(a)
        if bf16:                       # bit patterns: through int16, viewed as bfloat16
            return torch.from_numpy(a.view(np.int16)).view(dt).to(dev)
        return torch.from_numpy(a).to(dev)

    x, a, b = up(inp.x), up(A), up(B)
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    s = torch.from_numpy(inp.scales if scales is None else scales).to(dev)
    y = w4.linear_lora(x, q, s, g, a, b, scale)
    torch.cuda.synchronize()
    out = y.cpu()
    return bf16_to_float(out.view(torch.int16).numpy()) if bf16 else out.numpy()


def _check(case, inp, A, B, y, act, scale=S):
    q_o = oracle.pack(inp.codes)
    g, K, r = case.group_size, case.K, A.shape[0]
    ref = oracle.linear_lora(inp.x, q_o, inp.scales, g, A, B, scale, act=act)
    what = f"{case.name} {act}"
    if act == "f16":
        return check_parity(y, ref, what)
    lin = oracle.linear(inp.x, q_o, inp.scales, g, act="bf16")
    mag = oracle.linear(inp.x, q_o, inp.scales, g, act="bf16", absval=True)
    mag0 = oracle.linear(inp.x, np.zeros_like(q_o), inp.scales, g, act="bf16", absval=True)
    t = oracle.lora_shrink(inp.x, A, act="bf16")
    p1 = oracle.lora_expand(t, B, scale, act="bf16", absval=True)
    p2 = oracle.lora_expand(oracle.lora_shrink(inp.x, A, act="bf16", absval=True), B, scale,
                            act="bf16", absval=True)
    extra = lora_extra_bound(lin, ref, p1, p2, K, r, 2.0 ** -8)
    return check_parity_bf16(y, ref, mag, K, what, mag0=mag0, extra=extra)


CASES = [
    # M, K, N, g, r
    (1, 5120, 17408, 128, 32),      # decode up-projection shape, the suggested rank
    (4, 1024, 264, 32, 16),
    (16, 2048, 1032, 64, 8),
    (3, 1040, 136, 16, 40),         # K % 32 == 16, rank not a multiple of 16
    (17, 1024, 520, -1, 64),        # small-M prefill
    (100, 1024, 264, 16, 24),
    (129, 512, 264, 128, 128),      # 128-row prefill, two row blocks
    (256, 2048, 1024, 128, 256),
    (300, 1024, 264, 128, 32),      # 128-row prefill, three row blocks, split K
    (1100, 1024, 520, 64, 32),      # 256-row prefill, split last round: the first chunk adds the term
    (33, 4096, 264, 32, 1024),      # largest rank
    # decode with the term inside the stream-K launch, and the cases it leaves
    # to the separate shrink and expand kernels
    (8, 2048, 1032, 64, 64),        # in the launch: M r = 512 and 8 M r = 4096, both limits
    (1, 8192, 2048, 128, 128),      # in the launch: rank 128, 32 units x M r = 4096
    (4, 12288, 5120, 128, 16),      # in the launch, wide grid: the reduce kernel adds t'
    (1, 17408, 5120, 32, 16),       # in the launch: 68 shrink units (long K)
    (8, 5120, 5120, 128, 64),       # 20 units x M r = 10240 slab words: separate kernels
    (8, 2304, 1032, 64, 64),        # 9 units x M r = 4608, just past the limit: separate kernels
    (2, 1024, 264, 32, 256),        # rank above 128: separate kernels
    (16, 1024, 136, 32, 64),        # M r = 1024 above 512: separate kernels
    (1, 5120, 256, 128, 32),        # 20 shrink units, 8 workgroups: separate kernels
]


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("M,K,N,g,r", CASES)
def test_lora_parity(dev, M, K, N, g, r, act):
    case, inp, A, B = _inputs(M, K, N, g, r, 60 + M, act)
    y = _run(inp, A, B, g, dev, act == "bf16")
    _check(case, inp, A, B, y, act)


@pytest.mark.parametrize("act", ["f16", "bf16"])
@pytest.mark.parametrize("M,r", [(1, 32), (7, 8), (40, 64)])
def test_lora_term_alone(dev, M, r, act):
    """All-zero scales make the linear exactly zero: y is the adapter term alone,
    compared with the oracle's term under a tolerance relative to the term."""
    K, N, g = 2048, 1032, 64
    case, inp, A, B = _inputs(M, K, N, g, r, 70 + M, act)
    zeros = np.zeros_like(inp.scales)
    y = _run(inp, A, B, g, dev, act == "bf16", scales=zeros)
    t = oracle.lora_shrink(inp.x, A, act=act)
    d = oracle.lora_expand(t, B, S, act=act)
    if act == "f16":
        check_parity(y, d, f"{case.name} term alone")
    else:
        p1 = oracle.lora_expand(t, B, S, act="bf16", absval=True)
        p2 = oracle.lora_expand(oracle.lora_shrink(inp.x, A, act="bf16", absval=True), B, S,
                                act="bf16", absval=True)
        bound = lora_extra_bound(0.0, d, p1, p2, K, r, 2.0 ** -8) + 1e-30
        assert np.all(np.abs(y - d) <= bound), float(np.max(np.abs(y - d) - bound))
    assert np.abs(d).max() > 0.5       # the term is not trivially small


def test_lora_prefill_full_shape_sampled(dev):
    """The prefill up-projection shape (M=2048, K=5120, N=17408, g=128), rank 32:
    sampled outputs plus whole first and last rows, each from the oracle."""
    M, K, N, g, r = 2048, 5120, 17408, 128, 32
    case, inp, A, B = _inputs(M, K, N, g, r, 3, "f16")
    y = _run(inp, A, B, g, dev, False)
    ms, ns = sample_indices(M, N, 4096, seed=77)
    ms = np.concatenate([ms, np.zeros(N, np.int64), np.full(N, M - 1, np.int64)])
    ns = np.concatenate([ns, np.arange(N), np.arange(N)])
    q_o = oracle.pack(inp.codes)
    ref = oracle.linear_at(inp.x, q_o, inp.scales, g, ms, ns)
    ref = ref + oracle.lora_expand_at(oracle.lora_shrink(inp.x, A), B, S, ms, ns)
    check_parity(y[ms, ns], ref, "lora prefill_up (sampled)")


@pytest.mark.parametrize("bf16", [False, True])
def test_lora_scale_zero_equals_linear_and_is_deterministic(dev, bf16):
    """s = 0 adds +0 to every output: y equals the plain linear bit for bit.
    Two calls with the same inputs agree bit for bit."""
    act = "bf16" if bf16 else "f16"
    for M in (2, 48, 200):
        _, inp, A, B = _inputs(M, 1024, 520, 32, 32, 90 + M, act)
        y0 = _run(inp, A, B, 32, dev, bf16, scale=0.0)
        dt = torch.bfloat16 if bf16 else torch.float16
        x = np.ascontiguousarray(inp.x)
        x = (torch.from_numpy(x.view(np.int16)).view(dt) if bf16 else torch.from_numpy(x)).to(dev)
        q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
        s = torch.from_numpy(inp.scales).to(dev)
        lin = w4.linear(x, q, s, 32).cpu()
        lin = bf16_to_float(lin.view(torch.int16).numpy()) if bf16 else lin.numpy()
        assert np.array_equal(y0, lin), M
        y1 = _run(inp, A, B, 32, dev, bf16)
        y2 = _run(inp, A, B, 32, dev, bf16)
        assert np.array_equal(y1, y2), M


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_lora_graph_capture_and_replay(dev, act):
    """Linear + adapter captured in a HIP graph on a stream that already holds
    the linear's workspaces, replayed several times with eager work between the
    replays: every replay equals the eager call bit for bit."""
    st = torch.cuda.Stream()
    runs = []
    for M, K, N, g, r in ((1, 5120, 2048, 128, 32), (64, 1024, 1032, 64, 16),
                          (300, 2048, 1024, 128, 64)):
        _, inp, A, B = _inputs(M, K, N, g, r, 95, act)
        dt = torch.bfloat16 if act == "bf16" else torch.float16

        def up(arr):
            arr = np.ascontiguousarray(arr)
            if act == "bf16":
                return torch.from_numpy(arr.view(np.int16)).view(dt).to(dev)
            return torch.from_numpy(arr).to(dev)

        x = up(inp.x)
        q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
        s = torch.from_numpy(inp.scales).to(dev)
        a, b = up(A), up(B)
        ws = torch.empty(w4.w4a16_lora_workspace_bytes(M, K, r), dtype=torch.uint8, device=dev)
        eager = torch.empty((M, N), dtype=dt, device=dev)
        w4.linear_lora(x, q, s, g, a, b, S, out=eager, workspace=ws, stream=st)
        runs.append((x, q, s, a, b, g, ws, eager, torch.empty_like(eager)))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        for x, q, s, a, b, g, ws, _, out in runs:
            w4.linear_lora(x, q, s, g, a, b, S, out=out, workspace=ws, stream=st)
    for rep in range(3):
        for *_, out in runs:
            out.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (*_, eager, out) in enumerate(runs):
            assert torch.equal(out, eager), (i, rep)


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_lora_decode_repeatable_and_captured_on_fresh_stream(dev, act):
    """The term inside the decode launch: three calls in a row give the same
    bits (its counters start from zero every launch), interleaved with plain
    linears; captured on a fresh stream (no workspace yet: the separate
    kernels) and replayed, it meets the bar against the oracle."""
    M, K, N, g, r = 4, 5120, 4096, 128, 32
    case, inp, A, B = _inputs(M, K, N, g, r, 96, act)
    bf16 = act == "bf16"
    dt = torch.bfloat16 if bf16 else torch.float16

    def up(arr):
        arr = np.ascontiguousarray(arr)
        if bf16:
            return torch.from_numpy(arr.view(np.int16)).view(dt).to(dev)
        return torch.from_numpy(arr).to(dev)

    x, a, b = up(inp.x), up(A), up(B)
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    s = torch.from_numpy(inp.scales).to(dev)
    ws = torch.empty(w4.w4a16_lora_workspace_bytes(M, K, r), dtype=torch.uint8, device=dev)
    outs = []
    for _ in range(3):
        outs.append(w4.linear_lora(x, q, s, g, a, b, S, workspace=ws))
        w4.linear(x, q, s, g)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    y0 = outs[0].cpu()
    _check(case, inp, A, B, bf16_to_float(y0.view(torch.int16).numpy()) if bf16
           else y0.numpy().astype(np.float64), act)
    st = torch.cuda.Stream()
    out = torch.empty((M, N), dtype=dt, device=dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        w4.linear_lora(x, q, s, g, a, b, S, out=out, workspace=ws, stream=st)
    for _ in range(2):
        out.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        yc = out.cpu()
        _check(case, inp, A, B, bf16_to_float(yc.view(torch.int16).numpy()) if bf16
               else yc.numpy().astype(np.float64), act)
    w4.w4a16_stream_release(st)


@pytest.mark.parametrize("M", [3, 20])
def test_lora_and_zero_points_leave_memory_past_y_untouched(dev, M):
    """y is a prefix of a larger buffer filled with a canary: after the LoRA and
    the zero-point calls (ragged N = 136) everything past M*N is unchanged."""
    K, N, g, r = 1040, 136, 16, 24
    _, inp, A, B = _inputs(M, K, N, g, r, 99, "f16")
    x = torch.from_numpy(inp.x).to(dev)
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    s = torch.from_numpy(inp.scales).to(dev)
    qz = torch.from_numpy(w4.pack_zeros(workloads.zero_points(inp.scales.shape[0], N, 5))).to(dev)
    for call in ("lora", "zp"):
        buf = torch.full((M * N + 4096,), 1234.0, dtype=torch.float16, device=dev)
        out = buf[: M * N].view(M, N)
        if call == "lora":
            w4.linear_lora(x, q, s, g, torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                           S, out=out)
        else:
            w4.linear_zp(x, q, s, qz, g, out=out)
        torch.cuda.synchronize()
        assert bool((buf[M * N:] == 1234.0).all()), call
        assert bool(torch.isfinite(out).all()), call
