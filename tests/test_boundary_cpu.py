"""The C ABI on the CPU: the library loads, exports what include/w4a16.h declares,
rejects every invalid argument before any HIP call, and its host packing is
bit-exact against the oracle's independent packing."""

import ctypes
import os
import re

import numpy as np
import pytest

import int4_weight_only_w4a16_amd as w4
import oracle
import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4.LIB_PATH):
        from int4_weight_only_w4a16_amd import _build
        _build.build()
    return w4.load_library()


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:int|size_t|const char \*)\s*\*?\s*(\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(w4.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_header_compiles_as_c():
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        with open(src, "w") as f:
            f.write('#include "w4a16.h"\nint main(void){return W4A16_OK;}\n')
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                        src, "-o", os.path.join(d, "t")], check=True)


def _call(lib, x=0x1000, q=0x2000, s=0x3000, y=0x4000, M=1, K=32, N=8, g=32, kernel=0,
          bf16=False):
    f = lib.w4a16_linear_bf16_ex if bf16 else lib.w4a16_linear_ex
    return f(x, q, s, y, M, K, N, g, None, kernel)


@pytest.mark.parametrize("kw,status", [
    (dict(K=24), w4.W4A16_ERR_SHAPE),           # K % 16
    (dict(K=0), w4.W4A16_ERR_SHAPE),
    (dict(K=-16), w4.W4A16_ERR_SHAPE),
    (dict(N=12), w4.W4A16_ERR_SHAPE),           # N % 8
    (dict(N=0), w4.W4A16_ERR_SHAPE),
    (dict(M=-1), w4.W4A16_ERR_SHAPE),
    (dict(M=1 << 20, K=1 << 20), w4.W4A16_ERR_SHAPE),   # x reaches 2^31 bytes
    (dict(K=1 << 16, N=1 << 16), w4.W4A16_ERR_SHAPE),   # qweight reaches 2^31 bytes
    (dict(g=48), w4.W4A16_ERR_GROUP),
    (dict(g=0), w4.W4A16_ERR_GROUP),
    (dict(g=2048), w4.W4A16_ERR_GROUP),
    (dict(g=-2), w4.W4A16_ERR_GROUP),
    (dict(x=0), w4.W4A16_ERR_NULL),
    (dict(q=0), w4.W4A16_ERR_NULL),
    (dict(s=0), w4.W4A16_ERR_NULL),
    (dict(y=0), w4.W4A16_ERR_NULL),
    (dict(x=0x1008), w4.W4A16_ERR_ALIGN),
    (dict(q=0x2004), w4.W4A16_ERR_ALIGN),
    (dict(s=0x3002), w4.W4A16_ERR_ALIGN),
    (dict(y=0x4001), w4.W4A16_ERR_ALIGN),
    (dict(M=17, kernel=1), w4.W4A16_ERR_KERNEL),  # decode kernel takes M <= 16
    (dict(kernel=3), w4.W4A16_ERR_KERNEL),
    (dict(kernel=-1), w4.W4A16_ERR_KERNEL),
])
@pytest.mark.parametrize("bf16", [False, True], ids=["fp16", "bf16"])
def test_invalid_arguments_rejected_before_any_hip_call(lib, kw, status, bf16):
    assert _call(lib, bf16=bf16, **kw) == status


@pytest.mark.parametrize("bf16", [False, True], ids=["fp16", "bf16"])
def test_empty_batch_is_a_noop(lib, bf16):
    # M == 0: OK without touching the (null) pointers or the device
    assert _call(lib, x=0, q=0, s=0, y=0, M=0, bf16=bf16) == w4.W4A16_OK
    auto = lib.w4a16_linear_bf16 if bf16 else lib.w4a16_linear
    assert auto(0, 0, 0, 0, 0, 5120, 17408, 128, None) == w4.W4A16_OK
    # ...but an invalid shape is still an error at M == 0
    assert _call(lib, M=0, K=40, bf16=bf16) == w4.W4A16_ERR_SHAPE


@pytest.mark.parametrize("name", ["w4a16_gate_up_silu_ex", "w4a16_gate_up_silu_bf16_ex"])
def test_gate_up_validation(lib, name):
    f = getattr(lib, name)
    # the output has N/2 columns: N must be a multiple of 16
    assert f(0x1000, 0x2000, 0x3000, 0x4000, 1, 32, 8, 32, None, 0) == w4.W4A16_ERR_SHAPE
    assert f(0x1000, 0x2000, 0x3000, 0x4000, 1, 32, 24, 32, None, 0) == w4.W4A16_ERR_SHAPE
    assert f(0x1000, 0x2000, 0x3000, 0x4000, 1, 32, 16, 48, None, 0) == w4.W4A16_ERR_GROUP
    assert f(0, 0x2000, 0x3000, 0x4000, 1, 32, 16, 32, None, 0) == w4.W4A16_ERR_NULL
    assert f(0x1008, 0x2000, 0x3000, 0x4000, 1, 32, 16, 32, None, 0) == w4.W4A16_ERR_ALIGN
    assert f(0x1000, 0x2000, 0x3000, 0x4000, 17, 32, 16, 32, None, 1) == w4.W4A16_ERR_KERNEL
    assert f(0, 0, 0, 0, 0, 32, 16, 32, None, 0) == w4.W4A16_OK


def _lora(lib, x=0x1000, q=0x2000, s=0x3000, a=0x5000, b=0x6000, y=0x4000, M=1, K=32, N=8,
          g=32, r=8, ws=0x7000, wsb=1 << 20, bf16=False, scale=1.0):
    f = lib.w4a16_linear_lora_bf16 if bf16 else lib.w4a16_linear_lora
    return f(x, q, s, a, b, scale, y, M, K, N, g, r, ws, wsb, None)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(r=0), w4.W4A16_ERR_RANK),
    (dict(r=12), w4.W4A16_ERR_RANK),
    (dict(r=-8), w4.W4A16_ERR_RANK),
    (dict(r=1032), w4.W4A16_ERR_RANK),
    (dict(a=0), w4.W4A16_ERR_NULL),
    (dict(b=0), w4.W4A16_ERR_NULL),
    (dict(ws=0), w4.W4A16_ERR_NULL),
    (dict(a=0x5008), w4.W4A16_ERR_ALIGN),
    (dict(b=0x6004), w4.W4A16_ERR_ALIGN),
    (dict(ws=0x7008), w4.W4A16_ERR_ALIGN),
    (dict(wsb=0), w4.W4A16_ERR_WORKSPACE),
    (dict(wsb=511), w4.W4A16_ERR_WORKSPACE),
    (dict(K=40), w4.W4A16_ERR_SHAPE),
    (dict(N=12), w4.W4A16_ERR_SHAPE),
    (dict(g=48), w4.W4A16_ERR_GROUP),
    (dict(x=0), w4.W4A16_ERR_NULL),
    (dict(K=1 << 20, r=1024), w4.W4A16_ERR_SHAPE),     # A reaches 2^31 bytes
    (dict(N=1 << 20, r=1024), w4.W4A16_ERR_SHAPE),     # B reaches 2^31 bytes
])
def test_lora_invalid_arguments_rejected_before_any_hip_call(lib, kw, status, bf16):
    assert _lora(lib, bf16=bf16, **kw) == status


def test_lora_workspace_size_and_empty_batch(lib):
    # M=1, K=32, r=8: one 16-row block, one K chunk of 8 fp32 columns, then
    # t' (M x r in the activation type)
    assert w4.w4a16_lora_workspace_bytes(1, 32, 8) == 16 * 8 * 4 + 1 * 8 * 2
    assert _lora(lib, wsb=16 * 8 * 4 + 16) != w4.W4A16_ERR_WORKSPACE
    assert _lora(lib, wsb=16 * 8 * 4) == w4.W4A16_ERR_WORKSPACE
    assert w4.w4a16_lora_workspace_bytes(0, 32, 8) == 0
    assert w4.w4a16_lora_workspace_bytes(1, 32, 12) == 0
    assert w4.w4a16_lora_workspace_bytes(1, 40, 8) == 0
    # at most 16 chunks of K, and never more chunks than 4-step pieces of K
    for M, K, r in ((1, 5120, 32), (16, 17408, 64), (2048, 5120, 32), (300, 16, 8)):
        b = w4.w4a16_lora_workspace_bytes(M, K, r) - M * r * 2
        rows = 16 * ((M + 15) // 16)
        chunks = b // (rows * r * 4)
        assert b == chunks * rows * r * 4 and 1 <= chunks <= 16
        assert chunks <= max(1, -(-((K + 31) // 32) // 4))
    # M == 0 is a no-op whatever the pointers (shapes still checked)
    assert _lora(lib, x=0, q=0, s=0, a=0, b=0, y=0, ws=0, wsb=0, M=0) == w4.W4A16_OK
    assert _lora(lib, M=0, r=12) == w4.W4A16_ERR_RANK


def _zp(lib, x=0x1000, q=0x2000, s=0x3000, z=0x5000, y=0x4000, M=1, K=32, N=8, g=16,
        ws=0x7000, wsb=1 << 20, bf16=False):
    f = lib.w4a16_linear_zp_bf16 if bf16 else lib.w4a16_linear_zp
    return f(x, q, s, z, y, M, K, N, g, ws, wsb, None)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(z=0), w4.W4A16_ERR_NULL),
    (dict(ws=0), w4.W4A16_ERR_NULL),
    (dict(z=0x5004), w4.W4A16_ERR_ALIGN),
    (dict(ws=0x7008), w4.W4A16_ERR_ALIGN),
    (dict(wsb=16 * 8 * 4 + 8 * 8 * 2 - 1), w4.W4A16_ERR_WORKSPACE),
    (dict(K=40), w4.W4A16_ERR_SHAPE),
    (dict(g=48), w4.W4A16_ERR_GROUP),
    (dict(K=16 * 1544, g=16), w4.W4A16_ERR_SHAPE),      # more than 1536 groups
    (dict(x=0), w4.W4A16_ERR_NULL),
])
def test_zp_invalid_arguments_rejected_before_any_hip_call(lib, kw, status, bf16):
    assert _zp(lib, bf16=bf16, **kw) == status


def test_zp_workspace_size_and_packing(lib):
    # M=1, K=32, N=8, g=16: 2 groups padded to 8, one 16-row block, C^T [8, 8]
    assert w4.w4a16_zp_workspace_bytes(1, 32, 8, 16) == 16 * 8 * 4 + 8 * 8 * 2
    assert w4.w4a16_zp_workspace_bytes(33, 5120, 264, 128) == 48 * 40 * 4 + 264 * 40 * 2
    assert w4.w4a16_zp_workspace_bytes(1, 5120, 8, -1) == 16 * 8 * 4 + 8 * 8 * 2
    assert w4.w4a16_zp_workspace_bytes(0, 32, 8, 16) == 0
    assert w4.w4a16_zp_workspace_bytes(1, 32, 8, 48) == 0
    assert w4.w4a16_zp_workspace_bytes(1, 32, 12, 16) == 0
    assert w4.w4a16_zp_workspace_bytes(1, 16 * 1544, 8, 16) == 0
    assert _zp(lib, x=0, q=0, s=0, z=0, y=0, ws=0, wsb=0, M=0) == w4.W4A16_OK
    # zero points packed along N: the product's packing against the oracle's
    rng = np.random.default_rng(5)
    z = rng.integers(0, 16, size=(7, 48), dtype=np.uint8)
    want = np.ascontiguousarray(oracle.pack(np.ascontiguousarray(z.T)).T)
    assert np.array_equal(w4.pack_zeros(z), want)
    z8 = np.arange(8, dtype=np.uint8)[None, :]
    assert int(w4.pack_zeros(z8).view(np.uint32)[0, 0]) == 0x76543210


def test_status_strings(lib):
    for st in range(0, 11):
        assert w4.w4a16_status_string(st)
    assert w4.w4a16_status_string(99) == "unknown status"


def test_pack_matches_oracle_bit_exact(lib):
    rng = np.random.default_rng(21)
    for K, N in ((8, 8), (16, 24), (256, 264), (5120, 64)):
        codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
        q = w4.pack_gptq_v2(codes)
        assert np.array_equal(q, oracle.pack(codes))
        assert np.array_equal(w4.unpack_gptq_v2(q), codes)
        assert np.array_equal(w4.unpack_gptq_v2(q), oracle.unpack(q))


def test_pack_worked_words(lib):
    for codes, word, as_i32 in oracle_pins.read_pack_words():
        q = w4.pack_gptq_v2(np.array(codes, dtype=np.uint8).reshape(8, 1))
        assert int(q[0, 0]) == as_i32, hex(word)
        assert w4.unpack_gptq_v2(q)[:, 0].tolist() == codes


def test_pack_rejects_bad_input(lib):
    with pytest.raises(w4.W4A16Error) as e:
        w4.pack_gptq_v2(np.full((8, 8), 16, dtype=np.uint8))
    assert e.value.status == w4.W4A16_ERR_CODE
    codes = np.zeros((12, 8), dtype=np.uint8)
    assert lib.pack_gptq_v2(codes.ctypes.data, np.zeros(16, np.int32).ctypes.data, 12, 8) == \
        w4.W4A16_ERR_SHAPE
    assert lib.pack_gptq_v2(None, None, 8, 8) == w4.W4A16_ERR_NULL
    assert lib.unpack_gptq_v2(None, None, 8, 8) == w4.W4A16_ERR_NULL
    assert lib.unpack_gptq_v2(None, None, 7, 8) == w4.W4A16_ERR_SHAPE


@pytest.mark.parametrize("data, nbytes, sink, status", [
    (0x1000, 0, 0x2000, w4.W4A16_ERR_SHAPE),
    (0x1000, -16, 0x2000, w4.W4A16_ERR_SHAPE),
    (0x1000, 24, 0x2000, w4.W4A16_ERR_SHAPE),       # not a multiple of 16
    (None, 64, 0x2000, w4.W4A16_ERR_NULL),
    (0x1000, 64, None, w4.W4A16_ERR_NULL),
    (0x1008, 64, 0x2000, w4.W4A16_ERR_ALIGN),
    (0x1000, 64, 0x2002, w4.W4A16_ERR_ALIGN),
])
def test_read_probe_rejects_bad_arguments_before_any_hip_call(lib, data, nbytes, sink, status):
    assert lib.w4a16_read_probe(data, nbytes, sink, None) == status
