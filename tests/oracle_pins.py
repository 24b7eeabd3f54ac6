"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes a loaded oracle build and raises AssertionError
when it disagrees with:
  - hand-derived worked words and a hand-derived worked example
    (``tests/golden/``), which follow from the layout and the definition;
  - closed forms (q=0 -> -8s, q=8 -> 0, q=15 -> 7s; all-8 codes -> y == 0);
  - numpy's own fp16 decoding, over every fp16 bit pattern;
  - a textbook int64 GEMM (g = -1 with integer activations is an exact
    integer matrix product followed by a per-column scale);
  - brute force on tiny inputs with W built from the codes, never from the
    packed words;
  - exact rational arithmetic on an adversarial cancellation case;
  - metamorphic relations (scale doubling, column permutation, linearity);
  - for bfloat16 activations, numpy's own decoding (a float32's top half) over
    every bfloat16 bit pattern, and exact agreement with the fp16 path on
    values both formats hold;
  - for the magnitude sum sum_k |x||w|, a dense product of magnitudes and the
    bounds |y| <= sum|x||w| (equality when every term is non-negative).
  - for the merged gate/up with SiLU * mul, numpy's own exp on the brute-force
    product, and closed forms (zero gate or up weights give exactly 0).
  - for the LoRA adapter, the merged dense weight W + s A^T B^T through
    numpy's matmul, one-hot closed forms (A picking a channel of x, B = I),
    pure-Python loops on tiny inputs, and exact scaling relations.
  - for stored zero points, the symmetric definition exactly when every zero
    point is 8, numpy's matmul on W built from codes and zero points, a
    hand-derived word 0x76543210 (zero point n at column n), and y == 0
    exactly when every code equals its zero point.
  - for bfloat16 scales, numpy's own decoding of the scale patterns (values
    beyond fp16's range both ways) in W built from the codes, and a closed
    form; for v1 zero points (stored z - 1), W built from codes and nibbles,
    the all-7 symmetric checkpoint and the z = 16 closed form.
  - for the dense form (numpy's float64 matmul as the product step), the
    oracle's decoding of every fp16 and bfloat16 pattern against numpy's, and
    agreement with the triple loop within fp64 reordering (bit for bit on
    exact-arithmetic inputs).
``tests/test_oracle_mutants.py`` plants plausible mistakes in copies of the
oracle source and checks that every one of them trips at least one pin.
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
GROUPS = (-1, 16, 32, 64, 128, 256, 512, 1024)


def read_pack_words():
    rows = []
    with open(os.path.join(GOLDEN, "pack_words.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            fields = line.split()
            rows.append((list(map(int, fields[:8])), int(fields[8], 16), int(fields[9])))
    return rows


def read_worked_example():
    rows = []
    with open(os.path.join(GOLDEN, "worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            fields = line.split()
            rows.append((int(fields[0]), fields[1], [float(v) for v in fields[2:]]))
    return rows


def _worked_inputs(g: int, xname: str):
    K, N = 32, 8
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    codes = ((k + n) % 16).astype(np.uint8)
    if g == 16:
        scales = np.stack([np.ones(N), np.arange(1, N + 1)]).astype(np.float16)
    else:
        scales = np.ones((1, N), dtype=np.float16)
    x = np.zeros((1, K))
    if xname == "ones":
        x[:] = 1.0
    elif xname == "mix":
        x[0, 0], x[0, 31] = 0.5, 2.0
    else:
        x[0, int(xname[1:])] = 1.0
    return codes, scales, x.astype(np.float16)


def _brute(codes: np.ndarray, scales: np.ndarray, x: np.ndarray, g: int) -> np.ndarray:
    """Dense fp64 product with W built from the unpacked codes."""
    K = codes.shape[0]
    gidx = np.zeros(K, dtype=np.int64) if g == -1 else np.arange(K) // g
    W = (codes.astype(np.float64) - 8.0) * scales.astype(np.float64)[gidx]
    return x.astype(np.float64) @ W


# --- pins ----------------------------------------------------------------------

def pin_pack_words(o):
    for codes, word, as_i32 in read_pack_words():
        c = np.array(codes, dtype=np.uint8).reshape(8, 1)
        q = o.pack(c)
        assert q.shape == (1, 1)
        assert int(q[0, 0]) == as_i32, (codes, hex(word), int(q[0, 0]))
        back = o.unpack(np.array([[as_i32]], dtype=np.int32))
        assert back[:, 0].tolist() == codes, (hex(word), back[:, 0].tolist())


def pin_pack_roundtrip(o):
    rng = np.random.default_rng(11)
    for K, N in ((8, 8), (64, 24), (48, 40), (16, 1000)):
        codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
        q = o.pack(codes)
        assert q.shape == (K // 8, N)
        assert np.array_equal(o.unpack(q), codes)
    # a column of the words depends only on the same column of the codes
    codes = np.zeros((16, 8), dtype=np.uint8)
    codes[:, 3] = np.arange(16)
    q = o.pack(codes)
    assert np.count_nonzero(q[:, [0, 1, 2, 4, 5, 6, 7]]) == 0
    assert q[0, 3] == 0x76543210 and q[1, 3] == np.int32(-19088744)


def pin_dequant_closed_form(o):
    rng = np.random.default_rng(12)
    svals = np.concatenate([
        np.array([1.0, 0.5, 2.0 ** -14, 2.0 ** -24, 65504.0, 1e-3, 2e-2, 0.0078125]),
        rng.uniform(1e-4, 5e-2, size=56)]).astype(np.float16)
    N = svals.size
    s32 = svals.astype(np.float32)
    scales = svals.reshape(1, N)
    for code, factor in ((0, -8.0), (8, 0.0), (15, 7.0), (9, 1.0), (1, -7.0)):
        codes = np.full((16, N), code, dtype=np.uint8)
        W = o.dequant(o.pack(codes), scales, -1)
        expect = (np.float32(factor) * s32)[None, :].repeat(16, axis=0)
        assert np.array_equal(W, expect), (code, W[0, :4], expect[0, :4])


def pin_half_decode_all_patterns(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    svals = bits.view(np.float16)
    scales = svals.reshape(1, 65536)
    codes = np.full((16, 65536), 9, dtype=np.uint8)      # q - 8 = 1 -> w = s
    W = o.dequant(o.pack(codes), scales, -1)[0]
    ref = svals.astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(W), nan)
    assert np.array_equal(W[~nan], ref[~nan])
    assert np.array_equal(np.signbit(W[~nan]), np.signbit(ref[~nan]))


def pin_worked_example(o):
    for g, xname, expect in read_worked_example():
        codes, scales, x = _worked_inputs(g, xname)
        y = o.linear(x, o.pack(codes), scales, g)
        assert y.shape == (1, 8)
        assert y[0].tolist() == expect, (g, xname, y[0].tolist(), expect)


def pin_all_eights_zero(o):
    rng = np.random.default_rng(13)
    for g in GROUPS:
        K, N, M = 128, 48, 3
        G = 1 if g == -1 else -(-K // g)
        codes = np.full((K, N), 8, dtype=np.uint8)
        scales = rng.uniform(1e-3, 1.0, size=(G, N)).astype(np.float16)
        x = rng.standard_normal((M, K)).astype(np.float16)
        y = o.linear(x, o.pack(codes), scales, g)
        assert np.all(y == 0.0), g


def pin_per_channel_integer_gemm(o):
    """g = -1 with integer x is an int64 GEMM then a per-column scale, exactly."""
    rng = np.random.default_rng(14)
    for M, K, N in ((3, 96, 40), (5, 256, 16), (1, 2048, 8)):
        codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
        scales = rng.normal(0.0, 0.05, size=(1, N)).astype(np.float16)
        xi = rng.integers(-8, 9, size=(M, K)).astype(np.int64)
        x = xi.astype(np.float16)
        exact_int = xi @ (codes.astype(np.int64) - 8)            # textbook integer GEMM
        expect = exact_int.astype(np.float64) * scales.astype(np.float64)
        y = o.linear(x, o.pack(codes), scales, -1)
        assert np.array_equal(y, expect), (M, K, N)


def pin_group_equivalences(o):
    """g=-1, g=K and any g whose group rows carry equal scales give identical y."""
    rng = np.random.default_rng(15)
    K, N, M = 256, 24, 4
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    q = o.pack(codes)
    s1 = rng.uniform(1e-3, 2e-2, size=(1, N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    base = o.linear(x, q, s1, -1)
    assert np.array_equal(o.linear(x, q, s1, 256), base)
    assert np.array_equal(o.linear(x, q, s1, 512), base)      # g > K: one group
    for g in (16, 32, 64, 128):
        assert np.array_equal(o.linear(x, q, np.repeat(s1, K // g, axis=0), g), base), g


def pin_brute_force_tiny(o):
    rng = np.random.default_rng(16)
    shapes = ((1, 16, 8), (2, 32, 16), (4, 48, 24), (3, 64, 8), (4, 256, 64), (2, 80, 40))
    for M, K, N in shapes:
        for g in GROUPS:
            G = 1 if g == -1 else -(-K // g)
            codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
            scales = rng.uniform(1e-3, 2e-2, size=(G, N)).astype(np.float16)
            x = rng.standard_normal((M, K)).astype(np.float16)
            y = o.linear(x, o.pack(codes), scales, g)
            ref = _brute(codes, scales, x, g)
            tol = 1e-12 * max(1.0, float(np.abs(ref).max()))
            assert np.abs(y - ref).max() <= tol, (M, K, N, g)


def pin_exact_rational(o):
    """fp64 accumulation: an adversarial cancellation case vs exact rationals."""
    K, N = 32, 8
    codes = np.full((K, N), 15, dtype=np.uint8)                 # w = 7 s
    codes[1:K - 1, :] = (np.arange(1, K - 1)[:, None] + np.arange(N)[None, :]) % 16
    scales = np.ones((1, N), dtype=np.float16)
    x = np.full((1, K), 0.0010004, dtype=np.float64)
    x[0, 0], x[0, K - 1] = 16384.0, -16384.0                   # big terms cancel last
    x = x.astype(np.float16)
    y = o.linear(x, o.pack(codes), scales, -1)
    for n in range(N):
        exact = sum(Fraction(float(x[0, k])) * Fraction(int(codes[k, n]) - 8)
                    for k in range(K))
        mag = sum(abs(float(x[0, k]) * (int(codes[k, n]) - 8)) for k in range(K))
        assert abs(Fraction(y[0, n]) - exact) <= Fraction(K * mag) * Fraction(2) ** -53, n


def pin_metamorphic(o):
    rng = np.random.default_rng(17)
    M, K, N, g = 3, 128, 32, 32
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    q = o.pack(codes)
    scales = rng.uniform(1e-3, 2e-2, size=(K // g, N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    y = o.linear(x, q, scales, g)
    # doubling every scale doubles y exactly (no fp16 overflow/underflow here)
    assert np.array_equal(o.linear(x, q, (scales.astype(np.float32) * 2).astype(np.float16), g), 2 * y)
    # permuting output columns (with their weight and scale columns) permutes y
    perm = rng.permutation(N)
    assert np.array_equal(o.linear(x, o.pack(codes[:, perm]), scales[:, perm], g), y[:, perm])
    # permuting rows of x permutes rows of y
    assert np.array_equal(o.linear(x[::-1].copy(), q, scales, g), y[::-1])
    # linearity over disjoint supports (the fp16 sum is exact there)
    xa, xb = x.copy(), x.copy()
    xa[:, 1::2] = 0
    xb[:, 0::2] = 0
    ya, yb = o.linear(xa, q, scales, g), o.linear(xb, q, scales, g)
    assert np.abs(ya + yb - y).max() <= 1e-12 * np.abs(y).max()


def pin_sampled_matches_full(o):
    rng = np.random.default_rng(18)
    M, K, N, g = 5, 512, 64, 64
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    q = o.pack(codes)
    scales = rng.uniform(1e-3, 2e-2, size=(K // g, N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    y = o.linear(x, q, scales, g)
    ms = rng.integers(0, M, size=40)
    ns = rng.integers(0, N, size=40)
    assert np.array_equal(o.linear_at(x, q, scales, g, ms, ns), y[ms, ns])


# --- bfloat16 activations and the magnitude sum ---------------------------------

def _bf16_value(bits: np.ndarray) -> np.ndarray:
    """numpy's own decoding of bfloat16 bit patterns: the top half of a float32."""
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_bf16_decode_all_patterns(o):
    """Every bfloat16 pattern, as x[m, 0] against unit weights, comes back as
    numpy's own float32-top-half decoding of it."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    M, K, N = 65536, 16, 8
    x = np.zeros((M, K), dtype=np.uint16)
    x[:, 0] = bits
    q = o.pack(np.full((K, N), 9, dtype=np.uint8))            # q - 8 = 1 -> w = s = 1
    y = o.linear(x, q, np.ones((1, N), dtype=np.float16), -1, act="bf16")[:, 3]
    ref = _bf16_value(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(y), nan)
    assert np.array_equal(y[~nan], ref[~nan])
    nz = ~nan & (ref != 0)
    assert np.array_equal(np.signbit(y[nz]), np.signbit(ref[nz]))


def _shared_values(rng, shape):
    """Values with at most 8 significant bits inside fp16's normal range, so that
    fp16 and bfloat16 both hold them exactly."""
    mant = rng.integers(128, 256, size=shape) * rng.choice([-1, 1], size=shape)
    exp = rng.integers(-21, 8, size=shape)
    return np.ldexp(mant.astype(np.float64), exp)


def pin_bf16_agrees_with_half(o):
    """On values both formats hold exactly, bfloat16 and fp16 activations give
    bit-identical y."""
    rng = np.random.default_rng(19)
    for M, K, N, g in ((3, 64, 16, 16), (2, 256, 40, 128), (4, 96, 8, -1)):
        G = 1 if g == -1 else -(-K // g)
        codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
        scales = rng.uniform(1e-3, 2e-2, size=(G, N)).astype(np.float16)
        v = _shared_values(rng, (M, K))
        xh = v.astype(np.float16)
        assert np.array_equal(xh.astype(np.float64), v)
        xb = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal(_bf16_value(xb), v)
        q = o.pack(codes)
        assert np.array_equal(o.linear(xb, q, scales, g, act="bf16"), o.linear(xh, q, scales, g))


def _brute_abs(codes, scales, xv, g):
    K = codes.shape[0]
    gidx = np.zeros(K, dtype=np.int64) if g == -1 else np.arange(K) // g
    W = (codes.astype(np.float64) - 8.0) * scales.astype(np.float64)[gidx]
    return np.abs(xv) @ np.abs(W)


def pin_abs_brute_force(o):
    """sum_k |x||w| against a dense fp64 product of magnitudes, W built from the
    codes; fp16 and bfloat16 activations."""
    rng = np.random.default_rng(20)
    for M, K, N, g in ((1, 16, 8, 16), (3, 64, 24, 32), (2, 256, 16, -1), (4, 80, 40, 16)):
        G = 1 if g == -1 else -(-K // g)
        codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
        scales = rng.uniform(1e-3, 2e-2, size=(G, N)).astype(np.float16)
        q = o.pack(codes)
        xh = rng.standard_normal((M, K)).astype(np.float16)
        xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        for x, act, xv in ((xh, "f16", xh.astype(np.float64)), (xb, "bf16", _bf16_value(xb))):
            a = o.linear(x, q, scales, g, act=act, absval=True)
            ref = _brute_abs(codes, scales, xv, g)
            assert np.abs(a - ref).max() <= 1e-12 * max(1.0, float(ref.max())), (M, K, N, g, act)


def pin_abs_bounds_signed(o):
    """|y| <= sum|x||w| everywhere, with equality when every term is >= 0."""
    rng = np.random.default_rng(21)
    M, K, N, g = 4, 128, 32, 32
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    scales = rng.uniform(1e-3, 2e-2, size=(K // g, N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    q = o.pack(codes)
    y = o.linear(x, q, scales, g)
    a = o.linear(x, q, scales, g, absval=True)
    assert np.all(np.abs(y) <= a * (1 + 1e-12))
    pos_codes = rng.integers(8, 16, size=(K, N), dtype=np.uint8)
    xp = np.abs(x)
    qp = o.pack(pos_codes)
    assert np.array_equal(o.linear(xp, qp, scales, g, absval=True), o.linear(xp, qp, scales, g))


def pin_sampled_matches_full_bf16_abs(o):
    rng = np.random.default_rng(22)
    M, K, N, g = 4, 256, 48, 32
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    q = o.pack(codes)
    scales = rng.uniform(1e-3, 2e-2, size=(K // g, N)).astype(np.float16)
    xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ms = rng.integers(0, M, size=30)
    ns = rng.integers(0, N, size=30)
    for absval in (False, True):
        y = o.linear(xb, q, scales, g, act="bf16", absval=absval)
        assert np.array_equal(o.linear_at(xb, q, scales, g, ms, ns, act="bf16", absval=absval),
                              y[ms, ns]), absval


# --- merged gate/up with SiLU * mul --------------------------------------------

def pin_gate_up_silu_brute_force(o):
    """silu(gate) * up against numpy: W from the codes, numpy's own exp, both
    activation types."""
    rng = np.random.default_rng(23)
    for M, K, N, g in ((1, 16, 8, 16), (3, 64, 24, 32), (2, 256, 16, -1), (4, 96, 40, 16)):
        G = 1 if g == -1 else -(-K // g)
        codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
        scales = rng.uniform(1e-2, 8e-2, size=(G, N)).astype(np.float16)
        q = o.pack(codes)
        xh = rng.standard_normal((M, K)).astype(np.float16)
        xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        for x, act, xv in ((xh, "f16", xh.astype(np.float64)), (xb, "bf16", _bf16_value(xb))):
            y = _brute(codes, scales, xv, g)
            gate, up = y[:, 0::2], y[:, 1::2]
            ref = gate * up / (1.0 + np.exp(-gate))
            out = o.gate_up_silu(x, q, scales, g, act=act)
            assert out.shape == (M, N // 2)
            assert np.abs(out - ref).max() <= 1e-12 * max(1.0, float(np.abs(ref).max())), \
                (M, K, N, g, act)


def pin_gate_up_silu_closed_forms(o):
    """Zero gate weights give silu(0) = 0, zero up weights give 0 (exactly);
    with gate = ln 3 and up = 1, silu(ln 3) * 1 = 0.75 ln 3."""
    K, N = 32, 8
    rng = np.random.default_rng(24)
    x = rng.standard_normal((2, K)).astype(np.float16)
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    s = np.ones((1, N), dtype=np.float16)
    c_gate0 = codes.copy()
    c_gate0[:, 0::2] = 8
    assert np.all(o.gate_up_silu(x, o.pack(c_gate0), s, -1) == 0.0)
    c_up0 = codes.copy()
    c_up0[:, 1::2] = 8
    assert np.all(o.gate_up_silu(x, o.pack(c_up0), s, -1) == 0.0)
    # one nonzero x = ln 3 (fp16-rounded) on a code 9 (w = 1) column pair
    xv = np.zeros((1, K), dtype=np.float16)
    xv[0, 0] = np.float16(np.log(3.0))
    c = np.full((K, N), 8, dtype=np.uint8)
    c[0, :] = 9
    z = float(xv[0, 0])
    out = o.gate_up_silu(xv, o.pack(c), s, -1)
    assert np.allclose(out, z * z / (1.0 + np.exp(-z)), rtol=1e-15, atol=0)
    assert abs(z / (1.0 + np.exp(-z)) - 0.75 * z) < 1e-3


# --- LoRA adapter: A [r, K], B [N, r] in the activation type ---------------------

def _lora_case(rng, M, K, N, g, r, act):
    """Codes, scales, x, A and B with decoded values, for either activation type."""
    G = 1 if g == -1 else -(-K // g)
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    scales = rng.uniform(1e-2, 8e-2, size=(G, N)).astype(np.float16)
    x = rng.standard_normal((M, K))
    A = rng.uniform(-1.0, 1.0, size=(r, K)) / np.sqrt(K)
    B = 0.25 * rng.standard_normal((N, r))
    if act == "f16":
        vals = [v.astype(np.float16) for v in (x, A, B)]
        return codes, scales, vals, [v.astype(np.float64) for v in vals]
    bits = [(v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) for v in (x, A, B)]
    return codes, scales, bits, [_bf16_value(b) for b in bits]


def pin_lora_merged_weight(o):
    """The adapter equals a dense weight update: x . (W + s A^T B^T) with W built
    from the codes and the products taken by numpy's matmul in fp64."""
    rng = np.random.default_rng(31)
    for M, K, N, g, r, s in ((1, 64, 16, 16, 8, 2.0), (5, 128, 40, 32, 16, 0.5),
                             (3, 256, 24, -1, 32, -1.25), (2, 96, 8, 16, 4, 3.0)):
        for act in ("f16", "bf16"):
            codes, scales, (x, A, B), (xv, Av, Bv) = _lora_case(rng, M, K, N, g, r, act)
            q = o.pack(codes)
            G = scales.shape[0]
            grp = np.zeros(K, dtype=np.int64) if g == -1 else np.arange(K) // g
            W = (codes.astype(np.float64) - 8.0) * scales.astype(np.float64)[grp]
            ref = xv @ (W + s * (Av.T @ Bv.T))
            y = o.linear_lora(x, q, scales, g, A, B, s, act=act)
            assert y.shape == (M, N) and G == scales.shape[0]
            tol = 1e-12 * max(1.0, float(np.abs(ref).max()))
            assert np.abs(y - ref).max() <= tol, (M, K, N, g, r, act)
            t = o.lora_shrink(x, A, act=act)
            assert np.abs(t - xv @ Av.T).max() <= 1e-13 * max(1.0, float(np.abs(t).max()))
            d = o.lora_expand(t, B, s, act=act)
            assert np.abs(d - s * (t @ Bv.T)).max() <= 1e-13 * max(1.0, float(np.abs(d).max()))


def pin_lora_brute_force_tiny(o):
    """Pure-Python loops over decoded values on tiny inputs (no numpy products)."""
    rng = np.random.default_rng(32)
    M, K, N, g, r, s = 2, 16, 8, 16, 3, 1.5
    for act in ("f16", "bf16"):
        codes, scales, (x, A, B), (xv, Av, Bv) = _lora_case(rng, M, K, N, g, r, act)
        y = o.linear_lora(x, o.pack(codes), scales, g, A, B, s, act=act)
        for m in range(M):
            t = [sum(float(xv[m, k]) * float(Av[j, k]) for k in range(K)) for j in range(r)]
            for n in range(N):
                base = sum(float(xv[m, k]) * (int(codes[k, n]) - 8) * float(scales[k // g, n])
                           for k in range(K))
                want = base + s * sum(t[j] * float(Bv[n, j]) for j in range(r))
                assert abs(y[m, n] - want) <= 1e-12 * max(1.0, abs(want)), (act, m, n)


def pin_lora_closed_forms(o):
    """One-hot A rows pick channels of x and B = I copies t: d[m, n] = s x[m, c_n]
    exactly.  A zero adapter or s = 0 leaves the linear unchanged; d is odd and
    linear in s (exact in binary floating point for s -> 2s and s -> -s)."""
    rng = np.random.default_rng(33)
    M, K, N, r, s = 3, 32, 8, 8, 0.75
    x = rng.standard_normal((M, K)).astype(np.float16)
    chans = rng.choice(K, size=r, replace=False)
    A = np.zeros((r, K), dtype=np.float16)
    A[np.arange(r), chans] = 1.0
    B = np.eye(N, r, dtype=np.float16)
    d = o.lora_expand(o.lora_shrink(x, A), B, s)
    assert np.array_equal(d, s * x[:, chans].astype(np.float64))
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    scales = rng.uniform(1e-2, 8e-2, size=(1, N)).astype(np.float16)
    q = o.pack(codes)
    base = o.linear(x, q, scales, -1)
    assert np.array_equal(o.linear_lora(x, q, scales, -1, A, B, 0.0), base)
    assert np.array_equal(o.linear_lora(x, q, scales, -1, np.zeros_like(A), B, s), base)
    assert np.array_equal(o.linear_lora(x, q, scales, -1, A, np.zeros_like(B), s), base)
    assert np.array_equal(o.linear_lora(x, q, scales, -1, A, B, s), base + d)
    Ar = (rng.standard_normal((r, K)) * 0.2).astype(np.float16)
    Br = (rng.standard_normal((N, r)) * 0.2).astype(np.float16)
    t = o.lora_shrink(x, Ar)
    d1 = o.lora_expand(t, Br, s)
    assert np.array_equal(o.lora_expand(t, Br, 2 * s), 2 * d1)
    assert np.array_equal(o.lora_expand(t, Br, -s), -d1)


def pin_lora_magnitudes_and_samples(o):
    """absval returns dense products of magnitudes (|x| |A|^T, |s| |t| |B|^T) that
    bound the signed results, and the sampled expansion equals the full one."""
    rng = np.random.default_rng(34)
    M, K, N, r, s = 4, 64, 24, 16, -0.5
    for act in ("f16", "bf16"):
        _, _, (x, A, B), (xv, Av, Bv) = _lora_case(rng, M, K, N, 16, r, act)
        t = o.lora_shrink(x, A, act=act)
        ta = o.lora_shrink(x, A, act=act, absval=True)
        assert np.abs(ta - np.abs(xv) @ np.abs(Av).T).max() <= 1e-13 * float(ta.max())
        assert np.all(np.abs(t) <= ta * (1 + 1e-12))
        d = o.lora_expand(t, B, s, act=act)
        da = o.lora_expand(t, B, s, act=act, absval=True)
        assert np.abs(da - abs(s) * (np.abs(t) @ np.abs(Bv).T)).max() <= 1e-13 * float(da.max())
        assert np.all(np.abs(d) <= da * (1 + 1e-12))
        ms = rng.integers(0, M, size=40)
        ns = rng.integers(0, N, size=40)
        assert np.array_equal(o.lora_expand_at(t, B, s, ms, ns, act=act), d[ms, ns])
        assert np.array_equal(o.lora_expand_at(t, B, s, ms, ns, act=act, absval=True),
                              da[ms, ns])


# --- stored zero points: qzeros int32 [G, N/8], packed along N ------------------

def _pack_zeros(o, z):
    """uint8 zero points [G, N] -> int32 [G, N/8]: the K packing applied to z^T."""
    return np.ascontiguousarray(o.pack(np.ascontiguousarray(z.T)).T)


def pin_zp_eight_is_symmetric(o):
    """Every zero point 8: bit for bit the symmetric linear, both activation types."""
    rng = np.random.default_rng(41)
    for M, K, N, g in ((2, 64, 16, 16), (3, 256, 24, -1), (1, 96, 40, 32)):
        G = 1 if g == -1 else -(-K // g)
        codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
        scales = rng.uniform(1e-2, 8e-2, size=(G, N)).astype(np.float16)
        q = o.pack(codes)
        qz = _pack_zeros(o, np.full((G, N), 8, dtype=np.uint8))
        x = rng.standard_normal((M, K)).astype(np.float16)
        assert np.array_equal(o.linear_zp(x, q, scales, qz, g), o.linear(x, q, scales, g))
        xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal(o.linear_zp(xb, q, scales, qz, g, act="bf16"),
                              o.linear(xb, q, scales, g, act="bf16"))


def pin_zp_against_numpy(o):
    """W[k,n] = (q - z[k/g, n]) s[k/g, n] built in numpy from the codes and zero
    points (never from packed words), products by numpy's matmul in fp64; the
    magnitude form against |x| |W|."""
    rng = np.random.default_rng(42)
    for M, K, N, g in ((1, 16, 8, 16), (4, 128, 40, 32), (3, 96, 24, 64), (2, 64, 16, -1),
                       (5, 80, 8, 32)):
        G = 1 if g == -1 else -(-K // g)
        grp = np.zeros(K, dtype=np.int64) if g == -1 else np.arange(K) // g
        codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
        z = rng.integers(0, 16, size=(G, N), dtype=np.uint8)
        scales = rng.uniform(1e-2, 8e-2, size=(G, N)).astype(np.float16)
        W = (codes.astype(np.float64) - z.astype(np.float64)[grp]) * scales.astype(np.float64)[grp]
        x = rng.standard_normal((M, K)).astype(np.float16)
        xv = x.astype(np.float64)
        y = o.linear_zp(x, o.pack(codes), scales, _pack_zeros(o, z), g)
        ref = xv @ W
        assert np.abs(y - ref).max() <= 1e-12 * max(1.0, float(np.abs(ref).max())), (M, K, N, g)
        ya = o.linear_zp(x, o.pack(codes), scales, _pack_zeros(o, z), g, absval=True)
        refa = np.abs(xv) @ np.abs(W)
        assert np.abs(ya - refa).max() <= 1e-12 * max(1.0, float(refa.max()))


def pin_zp_worked_word_and_zero_output(o):
    """Zero point n at column n packs to the word 0x76543210; with x = e_0 and
    code 0 in row 0, y[n] = (0 - n) s[n] exactly.  Codes equal to their zero
    points give y == 0 exactly."""
    N, K = 8, 16
    z = np.arange(N, dtype=np.uint8)[None, :]
    qz = _pack_zeros(o, z)
    assert qz.shape == (1, 1) and int(qz.view(np.uint32)[0, 0]) == 0x76543210
    s = np.array([[0.5, 0.25, 1.0, 2.0, 0.125, 0.75, 1.5, 3.0]], dtype=np.float16)
    codes = np.full((K, N), 5, dtype=np.uint8)
    codes[0, :] = 0
    x = np.zeros((1, K), dtype=np.float16)
    x[0, 0] = 1.0
    y = o.linear_zp(x, o.pack(codes), s, qz, -1)
    assert np.array_equal(y[0], -np.arange(N) * s[0].astype(np.float64))
    rng = np.random.default_rng(43)
    K, N, g = 64, 16, 16
    zz = rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    codes = np.repeat(zz, g, axis=0)
    xs = rng.standard_normal((3, K)).astype(np.float16)
    sc = rng.uniform(1e-2, 8e-2, size=(K // g, N)).astype(np.float16)
    assert np.all(o.linear_zp(xs, o.pack(codes), sc, _pack_zeros(o, zz), g) == 0.0)


def pin_zp_sampled_matches_full(o):
    """Sampled zero-point outputs equal the full ones bit for bit (same fp32
    weights, k ascending, fp64 sums), both activation types."""
    rng = np.random.default_rng(44)
    M, K, N, g = 5, 192, 48, 64
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    scales = rng.uniform(1e-2, 8e-2, size=(K // g, N)).astype(np.float16)
    q, qz = o.pack(codes), _pack_zeros(o, z)
    ms = rng.integers(0, M, size=60)
    ns = rng.integers(0, N, size=60)
    xh = rng.standard_normal((M, K)).astype(np.float16)
    xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    for x, act in ((xh, "f16"), (xb, "bf16")):
        full = o.linear_zp(x, q, scales, qz, g, act=act)
        assert np.array_equal(o.linear_zp_at(x, q, scales, qz, g, ms, ns, act=act), full[ms, ns])



# --- the dense form (a library matmul as the product step) ------------------------

def pin_decode_act_all_patterns(o):
    """The oracle's field-by-field decoding of every fp16 and every bfloat16
    pattern against numpy's own (fp16 -> float64; bfloat16 as a float32's top half)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    for act, ref in (("f16", bits.view(np.float16).astype(np.float64)),
                     ("bf16", _bf16_value(bits))):
        x = bits.view(np.float16) if act == "f16" else bits
        got = o.decode_act(x, act)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), act
        assert np.array_equal(got[~nan], ref[~nan]), act
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), act


def pin_dense_matches_triple_loop(o):
    """linear_dense (numpy's float64 matmul over the oracle's W and decoded x)
    agrees with the k-ascending triple loop to within fp64 reordering, K 2^-52
    of the magnitude sum, for every group size, ragged K and both activation
    types; and bit for bit where every partial sum is exact (integer x, power-
    of-two scales)."""
    rng = np.random.default_rng(45)
    for M, K, N in ((3, 272, 40), (17, 1040, 64), (2, 4096, 24)):
        for g in GROUPS:
            G = 1 if g == -1 else -(-K // g)
            codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
            scales = rng.uniform(1e-3, 2e-2, size=(G, N)).astype(np.float16)
            q = o.pack(codes)
            xh = rng.standard_normal((M, K)).astype(np.float16)
            xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            for x, act in ((xh, "f16"), (xb, "bf16")):
                ref = o.linear(x, q, scales, g, act=act)
                mag = o.linear(x, q, scales, g, act=act, absval=True)
                d = np.abs(o.linear_dense(x, q, scales, g, act=act) - ref)
                assert np.all(d <= K * 2.0 ** -52 * mag + 1e-300), (M, K, N, g, act)
    M, K, N = 4, 2048, 32
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    scales = np.exp2(rng.integers(-4, -1, size=(K // 64, N)).astype(np.float64)).astype(np.float16)
    x = rng.integers(-4, 5, size=(M, K)).astype(np.float16)
    q = o.pack(codes)
    assert np.array_equal(o.linear_dense(x, q, scales, 64), o.linear(x, q, scales, 64))



# --- bfloat16 scales and v1 zero points ---------------------------------------------

def _bf16_bits_random(rng, shape, lo_exp, hi_exp):
    """Random positive bfloat16 bit patterns with exponents in [lo_exp, hi_exp]
    (values 2^e (1 + f/128)); the range runs past fp16's in both directions."""
    e = rng.integers(lo_exp, hi_exp + 1, size=shape)
    f = rng.integers(0, 128, size=shape)
    return (((e + 127) << 7) | f).astype(np.uint16)


def pin_bf16_scales_against_numpy(o):
    """bfloat16 scales (bit patterns, values from 2^-30 to 2^20, outside fp16's
    range both ways): W = (q - 8) s built in numpy from the codes and numpy's
    own decoding of the scales, products by numpy's matmul in fp64, against
    linear, linear_at, dequant, gate_up_silu, linear_lora and linear_zp (zero
    points 8) with either activation type; and a closed form: x all ones, every
    code 9, scale 3 * 2^20 (bits 0x4A40) gives y = 3 * 2^20 * K exactly."""
    rng = np.random.default_rng(46)
    for M, K, N, g in ((2, 64, 16, 16), (3, 272, 24, 128), (1, 96, 40, -1), (4, 160, 8, 32)):
        G = 1 if g == -1 else -(-K // g)
        grp = np.zeros(K, dtype=np.int64) if g == -1 else np.arange(K) // g
        codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
        sb = _bf16_bits_random(rng, (G, N), -30, 20)
        sv = _bf16_value(sb)
        W = (codes.astype(np.float64) - 8.0) * sv[grp]
        q = o.pack(codes)
        assert np.array_equal(o.dequant(q, sb, g, scales_type="bf16").astype(np.float64), W)
        xh = rng.standard_normal((M, K)).astype(np.float16)
        xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        for x, act, xv in ((xh, "f16", xh.astype(np.float64)), (xb, "bf16", _bf16_value(xb))):
            ref = xv @ W
            tol = 1e-12 * (np.abs(xv) @ np.abs(W)) + 1e-300
            y = o.linear(x, q, sb, g, act=act, scales_type="bf16")
            assert np.all(np.abs(y - ref) <= tol), (M, K, N, g, act)
            ms = rng.integers(0, M, size=20)
            ns = rng.integers(0, N, size=20)
            assert np.array_equal(o.linear_at(x, q, sb, g, ms, ns, act=act, scales_type="bf16"),
                                  y[ms, ns])
            if N % 2 == 0:
                gu = o.gate_up_silu(x, q, sb, g, act=act, scales_type="bf16")
                gg, uu = y[:, 0::2], y[:, 1::2]
                with np.errstate(over="ignore"):
                    ref_gu = gg / (1.0 + np.exp(-gg)) * uu
                fin = np.isfinite(ref_gu)
                assert np.allclose(gu[fin], ref_gu[fin], rtol=1e-12, atol=0.0)
            qz = _pack_zeros(o, np.full((G, N), 8, dtype=np.uint8))
            assert np.array_equal(o.linear_zp(x, q, sb, qz, g, act=act, scales_type="bf16"), y)
        r = 8
        A = rng.standard_normal((r, K)).astype(np.float16)
        B = rng.standard_normal((N, r)).astype(np.float16)
        yl = o.linear_lora(xh, q, sb, g, A, B, 0.5, scales_type="bf16")
        refl = xh.astype(np.float64) @ (W + 0.5 * A.astype(np.float64).T @ B.astype(np.float64).T)
        magl = np.abs(xh.astype(np.float64)) @ (np.abs(W) + 0.5 * np.abs(A.astype(np.float64)).T
                                                @ np.abs(B.astype(np.float64)).T)
        assert np.all(np.abs(yl - refl) <= 1e-12 * magl + 1e-300)
    K, N = 48, 8
    ones = np.ones((1, K), dtype=np.float16)
    y = o.linear(ones, o.pack(np.full((K, N), 9, dtype=np.uint8)),
                 np.full((1, N), 0x4A40, dtype=np.uint16), -1, scales_type="bf16")
    assert np.all(y == 3.0 * 2.0 ** 20 * K)


def pin_zp_v1_form(o):
    """v1 zero points (stored z - 1): W = (q - (nibble + 1)) s built in numpy from
    the codes and nibbles (15 gives z = 16), products by numpy's matmul, with
    fp16 and bfloat16 scales; a symmetric checkpoint in v1 form (every nibble
    7, word 0x77777777) is bit for bit the symmetric linear; code 0 under
    nibble 15 gives w = -16 s exactly; sampled outputs equal the full ones."""
    rng = np.random.default_rng(47)
    for M, K, N, g in ((2, 64, 16, 16), (3, 272, 24, 128), (1, 96, 40, -1)):
        G = 1 if g == -1 else -(-K // g)
        grp = np.zeros(K, dtype=np.int64) if g == -1 else np.arange(K) // g
        codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
        nib = rng.integers(0, 16, size=(G, N), dtype=np.uint8)
        nib[0, 0] = 15
        q, qz = o.pack(codes), _pack_zeros(o, nib)
        sh = rng.uniform(1e-2, 8e-2, size=(G, N)).astype(np.float16)
        sb = _bf16_bits_random(rng, (G, N), -12, 3)
        x = rng.standard_normal((M, K)).astype(np.float16)
        xv = x.astype(np.float64)
        for sc, st, sv in ((sh, "f16", sh.astype(np.float64)), (sb, "bf16", _bf16_value(sb))):
            W = (codes.astype(np.float64) - (nib.astype(np.float64) + 1.0)[grp]) * sv[grp]
            y = o.linear_zp(x, q, sc, qz, g, scales_type=st, zeros="v1")
            ref = xv @ W
            assert np.all(np.abs(y - ref) <= 1e-12 * (np.abs(xv) @ np.abs(W)) + 1e-300), (g, st)
            ms = rng.integers(0, M, size=16)
            ns = rng.integers(0, N, size=16)
            assert np.array_equal(o.linear_zp_at(x, q, sc, qz, g, ms, ns, scales_type=st,
                                                 zeros="v1"), y[ms, ns])
        q7 = _pack_zeros(o, np.full((G, N), 7, dtype=np.uint8))
        assert np.all(q7.view(np.uint32) == 0x77777777)
        assert np.array_equal(o.linear_zp(x, q, sh, q7, g, zeros="v1"), o.linear(x, q, sh, g))
    K, N = 16, 8
    e0 = np.zeros((1, K), dtype=np.float16)
    e0[0, 0] = 1.0
    s = np.full((1, N), 0.5, dtype=np.float16)
    y = o.linear_zp(e0, o.pack(np.zeros((K, N), dtype=np.uint8)), s,
                    _pack_zeros(o, np.full((1, N), 15, dtype=np.uint8)), -1, zeros="v1")
    assert np.all(y == -8.0)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
