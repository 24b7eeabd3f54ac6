"""bfloat16 scales and v1-form zero points (w4a16_linear_typed) against the
CPU oracle, through the C ABI on cuda:0.

bfloat16 scales enter each kernel where an fp16 scale does on the bfloat16
path (both convert to fp32 exactly), so the bars are the bfloat16 linear's,
gate/up's and zero-point correction's, with the oracle's y and magnitude
sums taken over the bfloat16 scale values.  The scales are the seeded draws
of ``workloads`` rounded to bfloat16, including a recipe reaching down to
2^-30, far below fp16's range.  v1 zero points (nibble = z - 1) are drawn
uniform over 0..15 (z up to 16).  Also: the flags select exactly the
existing entry points (bit for bit), bfloat16 scales that fp16 holds give
bit-identical results to those fp16 scales, the all-7 v1 checkpoint is the
symmetric linear bit for bit, and invalid flag sets launch nothing.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import bf16_to_float, check_gate_up, check_parity, check_parity_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import int4_weight_only_w4a16_amd as w4  # noqa: E402

DEC, PRE, AUTO = w4.W4A16_KERNEL_DECODE, w4.W4A16_KERNEL_PREFILL, w4.W4A16_KERNEL_AUTO
XB, SB, V1, GU = w4.W4A16_X_BF16, w4.W4A16_SCALES_BF16, w4.W4A16_ZEROS_V1, w4.W4A16_GATE_UP_SILU


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    w4.load_library()
    return torch.device("cuda:0")


def _dev16(a, bf16, dev):
    """A host array (fp16 values, or bfloat16 bit patterns when bf16) on the device."""
    a = np.ascontiguousarray(a)
    if bf16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def _host(y, bf16):
    out = y.cpu()
    if bf16:
        return bf16_to_float(out.view(torch.int16).numpy())
    return out.numpy().astype(np.float64)


def _typed(x, q, s, qz, N, g, flags, kernel=AUTO, ws=None, cols=None):
    M, K = x.shape
    y = torch.empty((M, cols if cols is not None else N), dtype=x.dtype, device=x.device)
    nbytes = 0 if ws is None else ws.numel()
    w4.w4a16_linear_typed(x, q, s, qz, y, M, K, N, g, flags, kernel, ws, nbytes)
    torch.cuda.synchronize()
    return y


def _zp_workspace(M, K, N, g, dev):
    need = w4.w4a16_zp_workspace_bytes(M, K, N, g)
    return torch.empty(max(need, 16), dtype=torch.uint8, device=dev)


# --- bfloat16 scales: the linear -------------------------------------------------

@pytest.mark.parametrize("M,K,N,g,recipe,kernels", [
    (1, 256, 256, 32, "wide", (DEC, PRE)),           # one step per group
    (3, 2064, 520, 16, "wide", (DEC, PRE)),          # g = 16 (scale per 8-deep block), ragged K
    (8, 1024, 2048, 64, "loguniform", (DEC, PRE)),   # scale per group
    (15, 5120, 5120, 128, "loguniform", (DEC,)),     # three ranges per tile, the two-level exchange
    (16, 2048, 17408, 128, "loguniform", (DEC,)),    # one range per CU: partial slots, reduce kernel
    (7, 8192, 1032, -1, "wide", (DEC,)),             # one group over K
    (64, 1040, 776, -1, "wide", (PRE,)),             # 128-row prefill, ragged K and N
    (300, 1536, 1032, 512, "loguniform", (PRE,)),    # 256-row prefill, ragged M and N
    (600, 1024, 1536, 128, "wide", (PRE,)),          # 256-row prefill with a split last round
])
def test_bf16_scales_linear_parity(dev, M, K, N, g, recipe, kernels):
    case = workloads.Case(f"sbf_{M}_{K}_{N}_{g}", M, K, N, g, 300 + M, scales=recipe)
    inp = workloads.generate(case, act="bf16", scales_type="bf16")
    q_o = oracle.pack(inp.codes)
    ref = oracle.linear(inp.x, q_o, inp.scales, g, act="bf16", scales_type="bf16")
    mag = oracle.linear(inp.x, q_o, inp.scales, g, act="bf16", absval=True, scales_type="bf16")
    mag0 = oracle.linear(inp.x, np.zeros_like(q_o), inp.scales, g, act="bf16", absval=True,
                         scales_type="bf16")
    x, s = _dev16(inp.x, True, dev), _dev16(inp.scales, True, dev)
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    for k in kernels:
        runs = [_host(_typed(x, q, s, None, N, g, XB | SB, k), True) for _ in range(2)]
        check_parity_bf16(runs[0], ref, mag, K, f"{case.name} kernel={k}", mag0)
        assert np.array_equal(runs[0], runs[1]), "results differ between runs"
        # the torch-level helper routes bfloat16 scales the same way
        y2 = w4.linear(x, q, s, g, kernel=k)
        torch.cuda.synchronize()
        assert np.array_equal(_host(y2, True), runs[0])


@pytest.mark.parametrize("M,K,N,g", [
    (1, 5120, 17408, 128),      # the decode up-projection
    (2048, 5120, 17408, 128),   # the prefill up-projection
])
def test_bf16_scales_model_shapes_sampled(dev, M, K, N, g):
    case = workloads.Case(f"sbf_model_{M}", M, K, N, g, 320, scales="loguniform")
    inp = workloads.generate(case, act="bf16", scales_type="bf16")
    q_o = oracle.pack(inp.codes)
    rng = np.random.default_rng(321)
    ms = np.concatenate([rng.integers(0, M, 2048), [0, M - 1]])
    ns = np.concatenate([rng.integers(0, N, 2048), [N - 1, 0]])
    ref = oracle.linear_at(inp.x, q_o, inp.scales, g, ms, ns, act="bf16", scales_type="bf16")
    mag = oracle.linear_at(inp.x, q_o, inp.scales, g, ms, ns, act="bf16", absval=True,
                           scales_type="bf16")
    mag0 = oracle.linear_at(inp.x, np.zeros_like(q_o), inp.scales, g, ms, ns, act="bf16",
                            absval=True, scales_type="bf16")
    x, s = _dev16(inp.x, True, dev), _dev16(inp.scales, True, dev)
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    y = _host(_typed(x, q, s, None, N, g, XB | SB), True)
    check_parity_bf16(y[ms, ns], ref, mag, K, f"{case.name} (sampled)", mag0)


def test_bf16_scales_decode_tiles_kernel_path(dev):
    """More than 8 column tiles of 64 per CU: one workgroup per tile, in the
    three weight forms (g = 16, one step per group, scale per group)."""
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = 8 * 64 * n_cus + 8
    for M, K, g in ((1, 64, 32), (5, 64, 16), (3, 128, 64)):
        case = workloads.Case(f"sbf_tiles_{M}_{K}_{g}", M, K, N, g, 330 + M, scales="wide")
        inp = workloads.generate(case, act="bf16", scales_type="bf16")
        q_o = oracle.pack(inp.codes)
        ref = oracle.linear(inp.x, q_o, inp.scales, g, act="bf16", scales_type="bf16")
        mag = oracle.linear(inp.x, q_o, inp.scales, g, act="bf16", absval=True,
                            scales_type="bf16")
        mag0 = oracle.linear(inp.x, np.zeros_like(q_o), inp.scales, g, act="bf16", absval=True,
                             scales_type="bf16")
        x, s = _dev16(inp.x, True, dev), _dev16(inp.scales, True, dev)
        q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
        y = _host(_typed(x, q, s, None, N, g, XB | SB, DEC), True)
        check_parity_bf16(y, ref, mag, K, case.name, mag0)


def _fp16_exact_as_bf16(rng, shape):
    """Scales with at most 8 significant bits inside fp16's normal range: the
    same values as fp16 and as bfloat16 bit patterns."""
    mant = rng.integers(128, 256, size=shape)
    v = np.ldexp(mant.astype(np.float64), rng.integers(-20, -8, size=shape))
    h = v.astype(np.float16)
    b = workloads.bf16_bits(v)
    assert np.array_equal(h.astype(np.float64), v)
    assert np.array_equal(bf16_to_float(b), v)
    return h, b


@pytest.mark.parametrize("M,K,N,g,kernel", [
    (1, 2048, 1024, 32, DEC), (4, 1040, 528, 16, DEC), (16, 4096, 1040, 128, DEC),
    (4, 1040, 528, 16, PRE), (100, 2048, 1040, 64, PRE), (300, 1024, 1552, -1, PRE),
])
def test_bf16_scales_same_values_as_fp16_bitwise(dev, M, K, N, g, kernel):
    """Scales that both types hold exactly give bit-identical y, gate/up and
    zero-point results: the scale type changes only the conversion."""
    rng = np.random.default_rng(340 + M)
    G = workloads.num_groups(K, g)
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    sh, sb = _fp16_exact_as_bf16(rng, (G, N))
    x = _dev16(workloads.bf16_bits(rng.standard_normal((M, K))), True, dev)
    q = torch.from_numpy(w4.pack_gptq_v2(codes)).to(dev)
    s_h, s_b = _dev16(sh, False, dev), _dev16(sb, True, dev)
    qz = torch.from_numpy(w4.pack_zeros(workloads.zero_points(G, N, 341 + M))).to(dev)
    ws = _zp_workspace(M, K, N, g, dev)
    for flags, cols, zeros in ((XB, N, None), (XB | GU, N // 2, None), (XB, N, qz),
                               (XB | V1, N, qz)):
        a = _typed(x, q, s_h, zeros, N, g, flags, kernel, ws, cols)
        b = _typed(x, q, s_b, zeros, N, g, flags | SB, kernel, ws, cols)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (flags, kernel)


# --- bfloat16 scales: the merged gate/up -------------------------------------------

@pytest.mark.parametrize("M,K,N,g,kernels", [
    (1, 5120, 2048, 128, (DEC, PRE)),
    (4, 2064, 1040, 16, (DEC, PRE)),
    (64, 2048, 4096, -1, (PRE,)),
    (300, 1024, 1056, 32, (PRE,)),
])
def test_bf16_scales_gate_up_parity(dev, M, K, N, g, kernels):
    case = workloads.Case(f"sbf_gu_{M}_{K}_{N}_{g}", M, K, N, g, 350 + M, scales="loguniform")
    inp = workloads.generate(case, act="bf16", scales_type="bf16")
    q_o = oracle.pack(inp.codes)
    kw = dict(act="bf16", scales_type="bf16")
    ref = oracle.gate_up_silu(inp.x, q_o, inp.scales, g, **kw)
    lin = oracle.linear(inp.x, q_o, inp.scales, g, **kw)
    mag = oracle.linear(inp.x, q_o, inp.scales, g, absval=True, **kw)
    mag0 = oracle.linear(inp.x, np.zeros_like(q_o), inp.scales, g, absval=True, **kw)
    x, s = _dev16(inp.x, True, dev), _dev16(inp.scales, True, dev)
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    for k in kernels:
        y = w4.gate_up_silu(x, q, s, g, kernel=k)
        torch.cuda.synchronize()
        check_gate_up(_host(y, True), ref, lin, mag, mag0, K, True, f"{case.name} kernel={k}")


# --- zero points: v1 form, bfloat16 scales ------------------------------------------

ZP_CASES = [
    # M, K, N, g
    (1, 5120, 4096, 128),
    (5, 1040, 136, 16),       # g = 16, K % 32 == 16
    (16, 2048, 1032, 32),
    (3, 272, 136, 256),       # short last group (16 of 256)
    (2, 1040, 72, 1024),      # short last group (16 of 1024)
    (40, 1024, 264, 64),
    (200, 2064, 264, 1024),   # short last group at prefill width
]
TYPES = [("f16", "f16", "v1"), ("bf16", "bf16", "v2"), ("bf16", "bf16", "v1"),
         ("bf16", "f16", "v1")]


def _zp_check(inp, z, M, K, N, g, act, st, zeros, y, what):
    q_o = oracle.pack(inp.codes)
    qz_o = np.ascontiguousarray(oracle.pack(np.ascontiguousarray(z.T)).T)
    kw = dict(act=act, scales_type=st)
    ref = oracle.linear_zp(inp.x, q_o, inp.scales, qz_o, g, zeros=zeros, **kw)
    if act == "f16":
        return check_parity(y, ref, what)
    u = 2.0 ** -8
    sym = oracle.linear(inp.x, q_o, inp.scales, g, **kw)
    mag = oracle.linear(inp.x, q_o, inp.scales, g, absval=True, **kw)
    mag0 = oracle.linear(inp.x, np.zeros_like(q_o), inp.scales, g, absval=True, **kw)
    # P = sum_k |x| |8 - z| s: codes all 8 under the same zero points, as magnitudes
    P = oracle.linear_zp(inp.x, oracle.pack(np.full((K, N), 8, dtype=np.uint8)), inp.scales,
                         qz_o, g, absval=True, zeros=zeros, **kw)
    extra = 1.02 * (u * np.abs(sym) + u * np.abs(ref) + (2 * u + K * 2.0 ** -24) * P)
    return check_parity_bf16(y, ref, mag, K, what, mag0=mag0, extra=extra)


@pytest.mark.parametrize("act,st,zeros", TYPES, ids=["-".join(t) for t in TYPES])
@pytest.mark.parametrize("M,K,N,g", ZP_CASES)
def test_zp_typed_parity(dev, M, K, N, g, act, st, zeros):
    case = workloads.Case(f"zpt_{M}_{K}_{N}_{g}", M, K, N, g, 360 + M, scales="loguniform")
    inp = workloads.generate(case, act=act, scales_type=st)
    z = workloads.zero_points(case.G, N, 361 + M)
    bf16 = act == "bf16"
    x, s = _dev16(inp.x, bf16, dev), _dev16(inp.scales, st == "bf16", dev)
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    qz = torch.from_numpy(w4.pack_zeros(z)).to(dev)
    flags = (XB if bf16 else 0) | (SB if st == "bf16" else 0) | (V1 if zeros == "v1" else 0)
    ws = _zp_workspace(M, K, N, g, dev)
    kernels = (AUTO, PRE) if M <= w4.W4A16_DECODE_MAX_M else (AUTO,)
    for k in kernels:
        y = _host(_typed(x, q, s, qz, N, g, flags, k, ws), bf16)
        _zp_check(inp, z, M, K, N, g, act, st, zeros, y, f"{case.name} {act}/{st}/{zeros} k={k}")
    # the one-launch decode path takes no workspace
    if M <= w4.W4A16_DECODE_MAX_M:
        y0 = _host(_typed(x, q, s, qz, N, g, flags, DEC, None), bf16)
        y1 = _host(_typed(x, q, s, qz, N, g, flags, AUTO, ws), bf16)
        assert np.array_equal(y0, y1)
    # the torch-level helper
    y2 = w4.linear_zp(x, q, s, qz, g, zeros_format=zeros)
    torch.cuda.synchronize()
    assert np.array_equal(_host(y2, bf16), _host(_typed(x, q, s, qz, N, g, flags, AUTO, ws), bf16))


@pytest.mark.parametrize("M,K,N,g", [(1, 1024, 264, 32), (16, 2064, 520, 16), (40, 1024, 264, 128),
                                     (300, 1536, 1032, -1)])
def test_zp_v1_all_sevens_is_symmetric_bitwise(dev, M, K, N, g):
    """A symmetric checkpoint in v1 form (every nibble 7, z = 8): bit for bit the
    symmetric linear, fp16 and bfloat16, fp16 and bfloat16 scales (up to the sign
    of a zero)."""
    rng = np.random.default_rng(370 + M)
    G = workloads.num_groups(K, g)
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    q = torch.from_numpy(w4.pack_gptq_v2(codes)).to(dev)
    qz = torch.from_numpy(w4.pack_zeros(np.full((G, N), 7, dtype=np.uint8))).to(dev)
    ws = _zp_workspace(M, K, N, g, dev)
    sv = rng.uniform(1e-3, 2e-2, size=(G, N))
    for flags in (0, XB, XB | SB):
        bf16 = bool(flags & XB)
        xv = rng.standard_normal((M, K))
        x = _dev16(workloads.bf16_bits(xv) if bf16 else xv.astype(np.float16), bf16, dev)
        s = _dev16(workloads.bf16_bits(sv) if flags & SB else sv.astype(np.float16),
                   bool(flags & SB), dev)
        sym = _host(_typed(x, q, s, None, N, g, flags), bf16)
        v1 = _host(_typed(x, q, s, qz, N, g, flags | V1, AUTO, ws), bf16)
        assert np.array_equal(sym, v1), flags


@pytest.mark.parametrize("M", [1, 16, 40, 300])
def test_typed_selects_the_existing_entry_points(dev, M):
    """Each flag set gives bit for bit what the named entry point gives."""
    K, N, g = 1024, 1040, 64
    case = workloads.Case(f"typed_eq_{M}", M, K, N, g, 380 + M)
    inp = workloads.generate(case)
    q = torch.from_numpy(w4.pack_gptq_v2(inp.codes)).to(dev)
    s = _dev16(inp.scales, False, dev)
    qz = torch.from_numpy(w4.pack_zeros(workloads.zero_points(case.G, N, 381))).to(dev)
    ws = _zp_workspace(M, K, N, g, dev)
    for bf16 in (False, True):
        xv = inp.x.astype(np.float64)
        x = _dev16(workloads.bf16_bits(xv) if bf16 else inp.x, bf16, dev)
        flags = XB if bf16 else 0
        ref = torch.empty((M, N), dtype=x.dtype, device=dev)
        (w4.w4a16_linear_bf16 if bf16 else w4.w4a16_linear)(x, q, s, ref, M, K, N, g)
        got = _typed(x, q, s, None, N, g, flags)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), ("linear", bf16)
        ref = torch.empty((M, N // 2), dtype=x.dtype, device=dev)
        (w4.w4a16_gate_up_silu_bf16 if bf16 else w4.w4a16_gate_up_silu)(x, q, s, ref, M, K, N, g)
        got = _typed(x, q, s, None, N, g, flags | GU, cols=N // 2)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), ("gate_up", bf16)
        ref = torch.empty((M, N), dtype=x.dtype, device=dev)
        w4.w4a16_linear_zp(x, q, s, qz, ref, M, K, N, g, ws, ws.numel(), bf16=bf16)
        got = _typed(x, q, s, qz, N, g, flags, AUTO, ws)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), ("zp", bf16)


def test_typed_rejects_invalid_flags_before_any_launch(dev):
    M, K, N, g = 4, 256, 64, 32
    x16 = torch.zeros((M, K), dtype=torch.float16, device=dev)
    xb = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((K // 8, N), dtype=torch.int32, device=dev)
    s = torch.ones((K // g, N), dtype=torch.float16, device=dev)
    qz = torch.zeros((K // g, N // 8), dtype=torch.int32, device=dev)
    ws = _zp_workspace(M, K, N, g, dev)
    bad = [(x16, SB, None), (xb, 0x10, None), (x16, V1, None), (xb, XB | V1, None),
           (x16, GU, qz), (xb, XB | GU | SB, qz), (x16, 0xFFFFFFFF, None)]
    for x, flags, zeros in bad:
        y = torch.full((M, N), 7.0, dtype=x.dtype, device=dev)
        with pytest.raises(w4.W4A16Error) as e:
            w4.w4a16_linear_typed(x, q, s, zeros, y, M, K, N, g, flags, AUTO, ws, ws.numel())
        assert e.value.status == w4.W4A16_ERR_FLAGS, flags
        torch.cuda.synchronize()
        assert torch.all(y == 7.0).item(), flags
    # the torch-level helpers reject fp16 x with bfloat16 scales
    with pytest.raises(ValueError):
        w4.linear(x16, q, s.to(torch.bfloat16), g)
    # the correction path needs its workspace; the one-launch decode path does not
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_linear_typed(x16, q, s, qz, y, M, K, N, g, 0, PRE, None, 0)
    assert e.value.status == w4.W4A16_ERR_NULL
    x17 = torch.zeros((17, K), dtype=torch.float16, device=dev)
    y17 = torch.empty((17, N), dtype=torch.float16, device=dev)
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_linear_typed(x17, q, s, qz, y17, 17, K, N, g, 0, DEC, None, 0)
    assert e.value.status == w4.W4A16_ERR_KERNEL
