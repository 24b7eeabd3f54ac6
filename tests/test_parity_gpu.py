"""Parity of the gfx950 HIP path with the CPU oracle, through the C ABI.

Every case draws seeded synthetic inputs (``workloads``), packs them with the
product's ``pack_gptq_v2`` (checked bit-exact against the oracle's own
packing), runs ``w4a16_linear`` / ``w4a16_linear_ex`` on cuda:0 and compares
with the oracle's float64 result to the parity bar of ``gpu_util``.  Cases the
oracle can finish in seconds are compared element by element; at the full
model shapes with large M the comparison uses whole rows, whole columns and
random samples that the oracle computes one by one.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (bf16_to_float, check_parity, check_parity_bf16, prefill_rows, sample_indices,
                      wide_tail_tiles)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import int4_weight_only_w4a16_amd as w4  # noqa: E402

DEC, PRE, AUTO = w4.W4A16_KERNEL_DECODE, w4.W4A16_KERNEL_PREFILL, w4.W4A16_KERNEL_AUTO


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    w4.load_library()
    return torch.device("cuda:0")


_WCACHE = {}


def _weights(case: workloads.Case, inp, dev):
    """Packed and uploaded weights, shared by cases that differ only in M."""
    key = (case.K, case.N, case.group_size, case.seed, case.scales, case.zero_cell_frac)
    if key not in _WCACHE:
        _WCACHE.clear()
        q_p = w4.pack_gptq_v2(inp.codes)
        q_o = oracle.pack(inp.codes)
        assert np.array_equal(q_p, q_o), "product packing differs from the oracle's"
        _WCACHE[key] = (q_o, torch.from_numpy(q_p).to(dev),
                        torch.from_numpy(inp.scales).to(dev))
    return _WCACHE[key]


def _run(inp, q_dev, s_dev, g, dev, kernel=AUTO):
    x = torch.from_numpy(inp.x).to(dev)
    y = w4.linear(x, q_dev, s_dev, g, kernel=kernel)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _full_case(case, dev, kernels=(AUTO,)):
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    y_ref = oracle.linear(inp.x, q_o, inp.scales, case.group_size)
    for k in kernels:
        y = _run(inp, q_dev, s_dev, case.group_size, dev, k)
        check_parity(y, y_ref, f"{case.name} kernel={k}")


def _sampled_case(case, dev, count=4096, kernels=(AUTO,)):
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    M, N = case.M, case.N
    ms, ns = sample_indices(M, N, count, seed=case.seed + 1000)
    # whole first and last rows and columns as well
    rows = np.repeat(np.array([0, M - 1]), N)
    rcols = np.tile(np.arange(N), 2)
    cols = np.tile(np.array([0, N - 1]), M)
    crows = np.repeat(np.arange(M), 2)
    ms = np.concatenate([ms, rows, crows]).astype(np.int64)
    ns = np.concatenate([ns, rcols, cols]).astype(np.int64)
    y_ref = oracle.linear_at(inp.x, q_o, inp.scales, case.group_size, ms, ns)
    for k in kernels:
        y = _run(inp, q_dev, s_dev, case.group_size, dev, k)
        check_parity(y[ms, ns], y_ref, f"{case.name} kernel={k} (sampled)")


# --- the five workloads ---------------------------------------------------------

def test_tiny_both_kernels(dev):
    _full_case(workloads.tiny(), dev, kernels=(AUTO, DEC, PRE))


def test_decode_up_full(dev):
    _full_case(workloads.decode_up(), dev, kernels=(AUTO, PRE))


@pytest.mark.parametrize("M", [1, 4, 16])
def test_down_small_batch_full(dev, M):
    _full_case(workloads.down_small_batch(M), dev, kernels=(AUTO, PRE))


def test_prefill_up_full(dev):
    """The prefill up-projection (M=2048, K=5120, N=17408, g=128) element by element
    over all 35.65 M outputs, against the oracle's dense form (its dequantised W
    and decoded x through numpy's float64 matmul; pinned against the triple loop)."""
    case = workloads.prefill_up()
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    y = _run(inp, q_dev, s_dev, case.group_size, dev)
    y_ref = oracle.linear_dense(inp.x, q_o, inp.scales, case.group_size)
    check_parity(y, y_ref, f"{case.name} (every output)")


def test_prefill_up_sampled(dev):
    _sampled_case(workloads.prefill_up(), dev)


@pytest.mark.parametrize("case", workloads.sweep(), ids=lambda c: c.name)
def test_sweep(dev, case):
    if case.M <= 8:
        _full_case(case, dev)
    else:
        _sampled_case(case, dev, count=2048)


# --- exact arithmetic: bit-exact against the oracle rounded once to fp16 -------

EXACT_SHAPES = [
    # M, K, N, g
    (1, 256, 256, 32),
    (4, 512, 264, 16),
    (5, 48, 64, 32),        # K % 32 == 16, partial last group
    (3, 256, 8, 512),       # g > K
    (16, 1024, 136, -1),
    (2, 16, 8, 16),         # smallest legal shape
    (17, 1024, 136, 64),
    (64, 2048, 520, 128),
    (130, 512, 264, 256),
    (33, 4096, 1032, 1024),
    (1, 17408, 64, 32),     # the longest K of the workloads
    (16, 17408, 64, -1),
    (300, 336, 520, 16),    # 256-row tiles: ragged M and N, K % 64 == 16
    (257, 48, 8, -1),       # 256-row tiles: K shorter than one stage
]


@pytest.mark.parametrize("M,K,N,g", EXACT_SHAPES)
def test_exact_arithmetic_bitwise(dev, M, K, N, g):
    case = workloads.exact_case(f"exact_{M}_{K}_{N}_{g}", M, K, N, g, seed=31)
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    y_ref = oracle.linear(inp.x, q_o, inp.scales, g)
    expect = y_ref.astype(np.float16)               # the exact value, rounded once
    kernels = (DEC, PRE) if M <= 16 else (PRE,)
    for k in kernels:
        y = _run(inp, q_dev, s_dev, g, dev, k)
        bad = np.flatnonzero(y != expect)
        assert bad.size == 0, (k, bad[:5], y.ravel()[bad[:5]], expect.ravel()[bad[:5]])


# --- special cases ----------------------------------------------------------------

@pytest.mark.parametrize("g", [-1, 16, 128])
def test_all_codes_eight_give_exact_zero(dev, g):
    K, N = 512, 264
    G = 1 if g == -1 else K // g
    rng = np.random.default_rng(41)
    codes = np.full((K, N), 8, dtype=np.uint8)
    q = torch.from_numpy(w4.pack_gptq_v2(codes)).to(dev)
    s = torch.from_numpy(rng.uniform(1e-3, 1.0, size=(G, N)).astype(np.float16)).to(dev)
    for M, k in ((1, DEC), (16, DEC), (3, PRE), (200, PRE)):
        x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float16)).to(dev)
        y = w4.linear(x, q, s, g, kernel=k)
        torch.cuda.synchronize()
        assert torch.count_nonzero(y).item() == 0, (M, k)


def test_zero_cell_columns_are_exact_zero(dev):
    """g = -1 with 5% zero cells: whole columns of codes are 8 -> y exactly 0 there."""
    case = workloads.Case("zero_cols", 8, 5120, 5120, -1, 4, scales="loguniform",
                          zero_cell_frac=0.05)
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    zero_cols = np.flatnonzero(inp.zero_cells[0])
    assert zero_cols.size == 256
    for k in (DEC, PRE):
        y = _run(inp, q_dev, s_dev, -1, dev, k)
        assert np.all(y[:, zero_cols] == 0), k


@pytest.mark.parametrize("kernel,M", [(DEC, 1), (DEC, 16), (PRE, 64), (PRE, 300)])
def test_deterministic_bitwise(dev, kernel, M):
    case = workloads.Case("det", M, 5120, 1032, 64, 7, scales="loguniform")
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    runs = [_run(inp, q_dev, s_dev, 64, dev, kernel) for _ in range(3)]
    for r in runs[1:]:
        assert np.array_equal(r.view(np.uint16), runs[0].view(np.uint16))


@pytest.mark.parametrize("M,K,N,g", [
    (1, 5120, 17408, 128),    # stream-K, nearly every tile split: exchange slots
    (2, 5120, 17408, 128),
    (4, 17408, 5120, 32),     # counter protocol
    (16, 5120, 17408, 16),
    (2048, 5120, 17408, 128),  # prefill with a split last round and its reduce pass
])
def test_deterministic_bitwise_full_size(dev, M, K, N, g):
    """Repeated launches at full size give bit-identical y: every split tile and
    split round is added in a fixed order, whichever contributor comes first."""
    print(f"determinism: M={M} K={K} N={N} g={g}", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(11)
    G = 1 if g == -1 else K // g
    q = torch.randint(-2**31, 2**31 - 1, (K // 8, N), dtype=torch.int32, generator=gen).to(dev)
    s = (torch.rand((G, N), generator=gen) * 0.02 + 0.001).half().to(dev)
    x = torch.randn((M, K), generator=gen).half().to(dev)
    ys = [w4.linear(x, q, s, g) for _ in range(8)]
    torch.cuda.synchronize()
    base = ys[0].view(torch.int16)
    for i, y in enumerate(ys[1:], 1):
        assert torch.equal(y.view(torch.int16), base), f"launch {i} differs"


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 15, 16, 17, 31, 63, 64, 65, 127, 128, 129, 512])
def test_dispatch_edges(dev, M):
    case = workloads.Case(f"edge_M{M}", M, 1024, 520, 128, 9)
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    y_ref = oracle.linear(inp.x, q_o, inp.scales, 128)
    y_auto = _run(inp, q_dev, s_dev, 128, dev, AUTO)
    check_parity(y_auto, y_ref, f"M={M} auto")
    expected_kernel = DEC if M <= w4.W4A16_DECODE_MAX_M else PRE
    y_explicit = _run(inp, q_dev, s_dev, 128, dev, expected_kernel)
    assert np.array_equal(y_auto.view(np.uint16), y_explicit.view(np.uint16))


@pytest.mark.parametrize("M,K,N,g", [
    (3, 16, 8, -1), (3, 16, 8, 16), (20, 16, 8, 1024),
    (2, 48, 24, 32), (33, 48, 24, 32),
    (4, 272, 5128, 256), (70, 272, 5128, 256),
    (1, 1040, 8, 1024), (19, 1040, 8, 1024),
    (16, 5120, 5128, 16), (96, 5120, 5128, 16),
    (200, 48, 24, 32), (257, 272, 5128, 256), (300, 1040, 8, 1024), (129, 5120, 5128, 16),
    (520, 336, 264, -1), (1100, 272, 5128, 256), (1030, 48, 24, 32),
])
def test_tails(dev, M, K, N, g):
    case = workloads.Case(f"tail_{M}_{K}_{N}_{g}", M, K, N, g, 13, scales="loguniform")
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    y_ref = oracle.linear(inp.x, q_o, inp.scales, g)
    for k in ((DEC, PRE) if M <= 16 else (PRE,)):
        check_parity(_run(inp, q_dev, s_dev, g, dev, k), y_ref, f"tail {M},{K},{N},{g} k={k}")


def test_output_canaries_untouched(dev):
    M, K, N, g = 5, 256, 264, 32
    case = workloads.Case("canary", M, K, N, g, 17)
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    x = torch.from_numpy(inp.x).to(dev)
    y_ref = oracle.linear(inp.x, q_o, inp.scales, g)
    pad = 4096
    for k in (DEC, PRE):
        buf = torch.full((pad + M * N + pad,), 12345.0, dtype=torch.float16, device=dev)
        y = buf[pad:pad + M * N]
        w4.w4a16_linear_ex(x, q_dev, s_dev, y, M, K, N, g, None, k)
        torch.cuda.synchronize()
        b = buf.cpu().numpy()
        assert np.all(b[:pad] == 12345.0) and np.all(b[pad + M * N:] == 12345.0), k
        check_parity(b[pad:pad + M * N].reshape(M, N), y_ref, f"canary k={k}")


def test_empty_batch_leaves_output_untouched(dev):
    q = torch.zeros((32, 8), dtype=torch.int32, device=dev)
    s = torch.ones((1, 8), dtype=torch.float16, device=dev)
    x = torch.zeros((1, 256), dtype=torch.float16, device=dev)
    y = torch.full((1, 8), 7.0, dtype=torch.float16, device=dev)
    w4.w4a16_linear(x, q, s, y, 0, 256, 8, -1)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0).item()


def test_misaligned_pointer_rejected(dev):
    q = torch.zeros((32, 16), dtype=torch.int32, device=dev)
    s = torch.ones((1, 16), dtype=torch.float16, device=dev)
    x = torch.zeros((1, 256 + 8), dtype=torch.float16, device=dev)
    y = torch.full((1, 16), 3.0, dtype=torch.float16, device=dev)
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_linear(x.data_ptr() + 2, q, s, y, 1, 256, 16, -1)
    assert e.value.status == w4.W4A16_ERR_ALIGN
    torch.cuda.synchronize()
    assert torch.all(y == 3.0).item()


def test_two_streams_concurrently(dev):
    cases = [workloads.Case("s1", 16, 5120, 2048, 128, 21), workloads.Case("s2", 256, 2048, 5120, 32, 22)]
    prepared = []
    for c in cases:
        inp = workloads.generate(c)
        q_o = oracle.pack(inp.codes)
        prepared.append((c, inp, q_o, torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev),
                         torch.from_numpy(inp.scales).to(dev), torch.from_numpy(inp.x).to(dev)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for (c, inp, q_o, q, s, x), st in zip(prepared, streams):
        y = torch.empty((c.M, c.N), dtype=torch.float16, device=dev)
        outs.append(y)
        with torch.cuda.stream(st):
            for _ in range(3):
                w4.w4a16_linear(x, q, s, y, c.M, c.K, c.N, c.group_size, st)
    torch.cuda.synchronize()
    for (c, inp, q_o, q, s, x), y in zip(prepared, outs):
        y_ref = oracle.linear(inp.x, q_o, inp.scales, c.group_size)
        check_parity(y.cpu().numpy(), y_ref, c.name)


def _free_bytes():
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def test_workspace_allocation_stated_and_released(dev):
    """The library's only device allocations, on a stream with none yet: the
    first decode call that splits tiles across workgroups creates the stream's
    decode workspace (12 KiB per CU), the first prefill call that splits K its
    prefill workspace (256 KiB per CU); further calls allocate nothing; and
    w4a16_stream_release frees both, leaving free memory where it started."""
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    case = workloads.Case("alloc", 64, 5120, 5120, 128, 23)
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    x = torch.from_numpy(inp.x).to(dev)
    x16 = x[:16].contiguous()
    y = torch.empty((64, 5120), dtype=torch.float16, device=dev)
    st = torch.cuda.Stream()
    w4.w4a16_stream_release(st)        # pooled streams may hold workspaces of earlier tests
    free0 = _free_bytes()
    w4.w4a16_linear_ex(x16, q_dev, s_dev, y, 16, 5120, 5120, 128, st, DEC)
    free1 = _free_bytes()
    assert free0 - free1 >= n_cus * 12 * 1024, (free0, free1)
    w4.w4a16_linear_ex(x, q_dev, s_dev, y, 64, 5120, 5120, 128, st, PRE)   # split K
    free2 = _free_bytes()
    assert free1 - free2 >= n_cus * 256 * 1024, (free1, free2)
    for _ in range(5):
        w4.w4a16_linear_ex(x16, q_dev, s_dev, y, 16, 5120, 5120, 128, st, DEC)
        w4.w4a16_linear_ex(x, q_dev, s_dev, y, 64, 5120, 5120, 128, st, PRE)
        w4.w4a16_linear_ex(x, q_dev, s_dev, y, 64, 5120, 5120, 128, st, AUTO)
    assert _free_bytes() == free2
    w4.w4a16_stream_release(st)
    assert _free_bytes() == free0
    y_ref = oracle.linear(inp.x, q_o, inp.scales, 128)
    w4.w4a16_linear_ex(x, q_dev, s_dev, y, 64, 5120, 5120, 128, st, AUTO)   # recreated
    torch.cuda.synchronize()
    check_parity(y.cpu().numpy(), y_ref, "after release")
    w4.w4a16_stream_release(st)


def test_stream_release_cycles_leave_memory_unchanged(dev):
    """32 cycles of a new stream, decode and prefill calls on it (the 128-row
    kernel and the 256-row kernel with a split last round, both of which take
    the stream's workspace), release and stream destruction leave the device's
    free memory unchanged."""
    case = workloads.Case("cycles", 1100, 2048, 4096, 64, 24)
    assert prefill_rows(1100, 2048, 4096) == 256 and wide_tail_tiles(1100, 2048, 4096)
    inp = workloads.generate(case)
    _, q_dev, s_dev = _weights(case, inp, dev)
    x = torch.from_numpy(inp.x).to(dev)
    x4 = x[:4].contiguous()
    x64 = x[:64].contiguous()
    y = torch.empty((1100, 4096), dtype=torch.float16, device=dev)

    def cycle():
        st = torch.cuda.Stream()
        w4.w4a16_linear(x4, q_dev, s_dev, y, 4, 2048, 4096, 64, st)
        w4.w4a16_linear(x64, q_dev, s_dev, y, 64, 2048, 4096, 64, st)
        w4.w4a16_linear(x, q_dev, s_dev, y, 1100, 2048, 4096, 64, st)
        w4.w4a16_stream_release(st)
        del st

    # torch hands out streams from a pool of 32 per device: one pass over the
    # pool first releases whatever earlier work left on those streams
    for _ in range(40):
        cycle()
    free0 = _free_bytes()
    for _ in range(32):
        cycle()
    assert _free_bytes() == free0


def test_stream_release_refused_under_capture(dev):
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        with pytest.raises(w4.W4A16Error) as e:
            w4.w4a16_stream_release(st)
    assert e.value.status == w4.W4A16_ERR_CAPTURE


def test_decode_tiles_kernel_path(dev):
    """More than 8 column tiles of 64 per CU: the decode runs one workgroup per tile."""
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = 8 * 64 * n_cus + 8
    for M, g in ((1, 32), (5, 16)):
        case = workloads.Case(f"tiles_{M}_{g}", M, 64, N, g, 27, scales="loguniform")
        inp = workloads.generate(case)
        q_o, q_dev, s_dev = _weights(case, inp, dev)
        y_ref = oracle.linear(inp.x, q_o, inp.scales, g)
        check_parity(_run(inp, q_dev, s_dev, g, dev, DEC), y_ref, f"tiles path M={M} g={g}")


def test_graph_capture_and_replay(dev):
    """Decode and prefill captured in a HIP graph, replayed several times with
    eager work in between; every replay matches the oracle.  On a fresh stream
    (no workspace yet) the captured calls run kernels that need none; on a
    stream that already has its workspaces the graph runs the same kernels as
    eager calls there (split-K partials and their reduce included), so every
    replay equals those bit for bit."""
    cases = [workloads.Case("g_dec", 4, 5120, 2048, 128, 29),
             workloads.Case("g_pre", 96, 1024, 1032, 64, 30),
             workloads.Case("g_pre_wide", 300, 2048, 2048, 128, 31)]
    prepared = []
    for c in cases:
        inp = workloads.generate(c)
        y_ref = oracle.linear(inp.x, oracle.pack(inp.codes), inp.scales, c.group_size)
        prepared.append((c, torch.from_numpy(inp.x).to(dev),
                         torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev),
                         torch.from_numpy(inp.scales).to(dev), y_ref))
    for warm in (False, True):
        st = torch.cuda.Stream()
        eager = None
        if warm:                       # the stream gets its workspaces eagerly first
            eager = []
            for c, x, q, s, _ in prepared:
                e = torch.empty((c.M, c.N), dtype=torch.float16, device=dev)
                w4.w4a16_linear(x, q, s, e, c.M, c.K, c.N, c.group_size, st)
                eager.append(e)
            torch.cuda.synchronize()
        outs = [torch.empty((c.M, c.N), dtype=torch.float16, device=dev)
                for c, *_ in prepared]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for (c, x, q, s, _), y in zip(prepared, outs):
                w4.w4a16_linear(x, q, s, y, c.M, c.K, c.N, c.group_size, st)
        for rep in range(4):
            for y in outs:
                y.fill_(-1.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for i, ((c, x, q, s, y_ref), y) in enumerate(zip(prepared, outs)):
                check_parity(y.cpu().numpy(), y_ref, f"{c.name} warm={warm} replay {rep}")
                if warm:
                    assert torch.equal(y, eager[i]), (c.name, rep)


def test_decode_launches_of_different_grids_share_a_stream(dev):
    """Stream-K launches with small and large grids, interleaved on one stream,
    reuse that stream's workspace; each must be exact (a regression test for a
    workspace layout that once depended on the grid size)."""
    shapes = [(1, 256, 256, 32), (4, 512, 264, 16), (1, 17408, 5120, 32), (2, 16, 8, 16),
              (4, 512, 264, 32), (16, 5120, 5128, 64), (3, 512, 256, -1), (1, 512, 264, 16)]
    prepared = []
    for M, K, N, g in shapes:
        case = workloads.exact_case(f"mix_{M}_{K}_{N}_{g}", M, K, N, g, seed=37)
        inp = workloads.generate(case)
        expect = oracle.linear(inp.x, oracle.pack(inp.codes), inp.scales, g).astype(np.float16)
        prepared.append((case, torch.from_numpy(inp.x).to(dev),
                         torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev),
                         torch.from_numpy(inp.scales).to(dev), expect))
    for rep in range(3):
        for case, x, q, s, expect in prepared:
            y = torch.full((case.M, case.N), 777.0, dtype=torch.float16, device=dev)
            w4.w4a16_linear_ex(x, q, s, y, case.M, case.K, case.N, case.group_size, None, DEC)
            torch.cuda.synchronize()
            got = y.cpu().numpy()
            bad = np.flatnonzero(got != expect)
            assert bad.size == 0, (rep, case.name, bad[:8])


def test_decode_after_other_launches(dev):
    """Decode calls whose workgroups hold uneven parts of split tiles (some
    waves get no units of a tile), run after prefill launches that leave LDS
    full of other data and after decode launches of other shapes on the same
    stream.  Every result must match the oracle on every repetition: a kernel
    that reads LDS or workspace state it did not write itself fails here (a
    regression test for per-tile wave sums that were summed unwritten)."""
    cases = [workloads.tiny(), workloads.decode_up(), workloads.down_small_batch(16),
             workloads.Case("hist_g-1", 1, 5120, 17408, -1, 4, scales="loguniform",
                            zero_cell_frac=0.05),
             workloads.Case("hist_n5120", 8, 5120, 5120, 16, 4, scales="loguniform")]
    big = workloads.Case("hist_prefill", 256, 4096, 4096, 128, 41)
    inp_b = workloads.generate(big)
    xb = torch.from_numpy(inp_b.x).to(dev)
    qb = torch.from_numpy(w4.pack_gptq_v2(inp_b.codes)).to(dev)
    sb = torch.from_numpy(inp_b.scales).to(dev)
    prepared = []
    for c in cases:
        inp = workloads.generate(c)
        q_o = oracle.pack(inp.codes)
        y_ref = oracle.linear(inp.x, q_o, inp.scales, c.group_size)
        prepared.append((c, torch.from_numpy(inp.x).to(dev), torch.from_numpy(q_o).to(dev),
                         torch.from_numpy(inp.scales).to(dev), y_ref))
    for rep in range(2):
        for c, x, q, s, y_ref in prepared:
            w4.linear(xb, qb, sb, big.group_size, kernel=PRE)      # dirty every CU's LDS
            y = w4.linear(x, q, s, c.group_size, kernel=DEC)
            torch.cuda.synchronize()
            check_parity(y.cpu().numpy(), y_ref, f"{c.name} after other launches, rep {rep}")


@pytest.mark.parametrize("M", [1, 2, 3, 8, 14, 15, 16])
def test_decode_split_tiles_exchange(dev, M):
    """Bench-like widths.  K=5120, N=17408 (272 tiles, one range per CU): most
    tiles are split between two workgroups, which meet per output column pair
    in an exchange slot (M <= 14), or leave partial tiles that a second kernel
    adds (M = 15, 16).  K=17408, N=5120 (80 tiles): three ranges per tile,
    finished by the two-level exchange, for every M."""
    for K, N, g in ((5120, 17408, 128), (17408, 5120, 32)):
        case = workloads.Case(f"split_{M}_{K}_{N}", M, K, N, g, 41, scales="loguniform")
        inp = workloads.generate(case)
        q_o, q_dev, s_dev = _weights(case, inp, dev)
        y_ref = oracle.linear(inp.x, q_o, inp.scales, g)
        runs = [_run(inp, q_dev, s_dev, g, dev, DEC) for _ in range(3)]
        check_parity(runs[0], y_ref, f"split M={M} K={K} N={N}")
        for r in runs[1:]:
            assert np.array_equal(r.view(np.uint16), runs[0].view(np.uint16))


@pytest.mark.parametrize("M", [3, 5, 16])
def test_decode_wide_partials_ragged(dev, M):
    """Between a third and a half as many tiles as CUs (6136 columns: 96 tiles)
    and long K with M > 2: every CU takes a range, a tile has up to three
    contributors, and a second kernel adds their partials; ragged K (the last
    32-deep step half inside K) and ragged N."""
    case = workloads.Case(f"wide_{M}", M, 16400, 6136, 16, 45, scales="loguniform")
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    y_ref = oracle.linear(inp.x, q_o, inp.scales, 16)
    runs = [_run(inp, q_dev, s_dev, 16, dev, DEC) for _ in range(3)]
    check_parity(runs[0], y_ref, f"wide M={M}")
    for r in runs[1:]:
        assert np.array_equal(r.view(np.uint16), runs[0].view(np.uint16))


@pytest.mark.parametrize("M,K,N,g", [
    (1, 8192, 1032, 64),       # 17 tiles, three ranges each (long K)
    (4, 1040, 264, 16),        # 5 tiles x 3 (M >= 4), ragged K and N
    (7, 2064, 5432, -1),       # 85 tiles x 3 = 255 workgroups, the most that fit
    (16, 4096, 2056, 128),     # 33 tiles x 3 at M = 16
])
def test_decode_three_contributors(dev, M, K, N, g):
    """Tiles split into exactly three ranges: contributors 0 and 1 meet first,
    whichever comes second meets contributor 2, so y = (p0 + p1) + p2 in any
    arrival order; checked against the oracle and bit for bit across runs,
    bf16 as well, and a second shape on the same stream reuses the slots."""
    case = workloads.Case(f"three_{M}_{K}_{N}", M, K, N, g, 47, scales="loguniform")
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    y_ref = oracle.linear(inp.x, q_o, inp.scales, g)
    runs = [_run(inp, q_dev, s_dev, g, dev, DEC) for _ in range(4)]
    check_parity(runs[0], y_ref, f"three M={M} K={K} N={N}")
    for r in runs[1:]:
        assert np.array_equal(r.view(np.uint16), runs[0].view(np.uint16))
    cb = workloads.Case(f"three_bf16_{M}_{K}_{N}", M, K, N, g, 48, scales="loguniform")
    ib = workloads.generate_bf16(cb)
    qb_o, qb_dev, sb_dev = _weights(cb, ib, dev)
    xb = torch.from_numpy(ib.x.view(np.int16)).view(torch.bfloat16).to(dev)
    yb = w4.linear(xb, qb_dev, sb_dev, g, kernel=DEC)
    torch.cuda.synchronize()
    yb = bf16_to_float(yb.cpu().view(torch.int16).numpy())
    check_parity_bf16(yb, oracle.linear(ib.x, qb_o, ib.scales, g, act="bf16"),
                      oracle.linear(ib.x, qb_o, ib.scales, g, act="bf16", absval=True), K,
                      f"three bf16 M={M}",
                      mag0=oracle.linear(ib.x, np.zeros_like(qb_o), ib.scales, g, act="bf16",
                                         absval=True))


@pytest.mark.parametrize("M,K,N,g,full", [
    (64, 2064, 1032, 16, True),      # 5 tiles x 4 chunks; last stage half inside K
    (17, 5120, 17408, 128, False),   # 68 tiles x 3 chunks
    (128, 17408, 5120, 32, False),   # 20 tiles x 12 chunks
    (100, 1024, 264, -1, True),      # 2 tiles x 2 chunks (16 stages), ragged M and N
    (32, 2048, 1032, 128, True),     # 32-row tiles, exactly full
    (33, 2048, 1032, 32, True),      # 64-row tiles, one row into the second 32
])
def test_prefill_m128_split_k(dev, M, K, N, g, full):
    """M <= 128 with fewer tiles than CUs: each tile's K is split into chunks
    whose fp32 partials a second kernel adds in chunk order."""
    case = workloads.Case(f"m128split_{M}_{K}_{N}", M, K, N, g, 46, scales="loguniform")
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    runs = [_run(inp, q_dev, s_dev, g, dev, PRE) for _ in range(3)]
    if full:
        check_parity(runs[0], oracle.linear(inp.x, q_o, inp.scales, g), f"{case.name}")
    else:
        ms, ns = sample_indices(M, N, 4096, seed=47)
        y_ref = oracle.linear_at(inp.x, q_o, inp.scales, g, ms, ns)
        check_parity(runs[0][ms, ns], y_ref, f"{case.name} (sampled)")
    for r in runs[1:]:
        assert np.array_equal(r.view(np.uint16), runs[0].view(np.uint16))


@pytest.mark.parametrize("M,K,N,g,rows,full", [
    (384, 5120, 17408, 128, 128, False),   # 204 tiles of 128 rows, one round
    (512, 5120, 5120, 128, 128, False),    # 80 tiles of 128 rows x 3 K chunks
    (640, 1024, 2056, 32, 128, True),      # 5 row blocks, ragged N, 2 K chunks
    (1000, 1024, 2056, 32, 128, True),     # 8 row blocks, the last ragged
    (512, 5120, 17408, 128, 256, False),   # 136 tiles of 256 rows, one round
    (256, 5120, 17408, 128, 256, False),   # 68 tiles of 256 rows x 3 K chunks
    (1024, 5120, 5120, 128, 256, False),   # 80 tiles of 256 rows x 3 K chunks
])
def test_prefill_mid_m_kernels(dev, M, K, N, g, rows, full):
    """128 < M <= 1024: the dispatcher prices both prefill kernels and takes
    the cheaper; cases on either side (the 128-row kernel with several row
    blocks, split K or not; the 256-row kernel), bitwise equal runs."""
    assert prefill_rows(M, K, N) == rows
    case = workloads.Case(f"midm_{M}_{K}_{N}", M, K, N, g, 48, scales="loguniform")
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    runs = [_run(inp, q_dev, s_dev, g, dev, AUTO) for _ in range(2)]
    if full:
        check_parity(runs[0], oracle.linear(inp.x, q_o, inp.scales, g), case.name)
    else:
        ms, ns = sample_indices(M, N, 4096, seed=49)
        y_ref = oracle.linear_at(inp.x, q_o, inp.scales, g, ms, ns)
        check_parity(runs[0][ms, ns], y_ref, f"{case.name} (sampled)")
    assert np.array_equal(runs[0].view(np.uint16), runs[1].view(np.uint16))


def test_prefill_split_tail_ragged(dev):
    """A last partial round of 256 x 256 tiles split along K (on a 256-CU
    device: 272 tiles, the last 16 of the banded tile order split in two, the
    second chunk ending in a K tail), ragged M and N: every output of the tail
    tiles, a sample of the rest, and bitwise equal runs."""
    M, K, N, g = 2000, 1040, 8456, 16
    case = workloads.Case("split_tail", M, K, N, g, 43, scales="loguniform")
    inp = workloads.generate(case)
    q_o, q_dev, s_dev = _weights(case, inp, dev)
    tail = wide_tail_tiles(M, K, N)
    assert len(tail) == 16 and any(n0 + 256 > N for _, n0 in tail) and any(m0 + 256 > M for m0, _ in tail)
    ms, ns = [], []
    for m0, n0 in tail:
        rows = np.arange(m0, min(m0 + 256, M))
        cols = np.arange(n0, min(n0 + 256, N))
        ms.append(np.repeat(rows, cols.size))
        ns.append(np.tile(cols, rows.size))
    ms, ns = np.concatenate(ms), np.concatenate(ns)
    sm, sn = sample_indices(M, N, 4096, seed=44)
    ms = np.concatenate([ms, sm]).astype(np.int64)
    ns = np.concatenate([ns, sn]).astype(np.int64)
    y_ref = oracle.linear_at(inp.x, q_o, inp.scales, g, ms, ns)
    runs = [_run(inp, q_dev, s_dev, g, dev, PRE) for _ in range(2)]
    check_parity(runs[0][ms, ns], y_ref, "split tail (sampled)")
    assert np.array_equal(runs[0].view(np.uint16), runs[1].view(np.uint16))
