"""CPU oracle for the W4A16 symmetric-INT4 GPTQ linear (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path never imports this
package, and this package never imports the product.

The arithmetic lives in ``w4a16_oracle.c`` (plain C, fp64 accumulation); this
file only compiles it with gcc and marshals numpy arrays.  See the C file's
header for the definition it follows and the passages of the pages it cites.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(_HERE, "w4a16_oracle.c")
LIB_PATH = os.path.join(_HERE, "libw4a16_oracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra"]


def compile_source(src: str, out: str) -> str:
    """Compile one oracle source file to a shared library with the oracle's flags."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no FP contraction, no fast-math)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    return compile_source(SRC_PATH, LIB_PATH)


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


_ACTS = {"f16": 0, "bf16": 1}
_SCALES = {"f16": 0, "bf16": 1}
_ZEROS = {"v2": 0, "v1": 1}


def _act_bits(x: np.ndarray, act: str) -> np.ndarray:
    """Activations as contiguous uint16 bit patterns: fp16 values for "f16",
    bfloat16 bit patterns (given as uint16) for "bf16"."""
    if act == "f16":
        return np.ascontiguousarray(x, dtype=np.float16).view(np.uint16)
    if act == "bf16":
        if x.dtype != np.uint16:
            raise TypeError("bf16 activations are passed as uint16 bit patterns")
        return np.ascontiguousarray(x)
    raise ValueError(f"unknown activation type {act!r}")


def _scale_bits(scales: np.ndarray, scales_type: str) -> np.ndarray:
    """Scales as contiguous uint16 bit patterns: fp16 values for "f16",
    bfloat16 bit patterns (given as uint16) for "bf16"."""
    if scales_type == "f16":
        return np.ascontiguousarray(scales, dtype=np.float16).view(np.uint16)
    if scales_type == "bf16":
        if scales.dtype != np.uint16:
            raise TypeError("bf16 scales are passed as uint16 bit patterns")
        return np.ascontiguousarray(scales)
    raise ValueError(f"unknown scale type {scales_type!r}")


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


class Oracle:
    """One loaded build of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_unpack.argtypes = [p, i64, i64, p]
        lib.oracle_pack.argtypes = [p, i64, i64, p]
        lib.oracle_dequant.argtypes = [p, p, i64, i64, i64, p]
        lib.oracle_dequant_ex.argtypes = [p, p, ctypes.c_int, i64, i64, i64, p]
        lib.oracle_dequant_ex.restype = ctypes.c_int
        lib.oracle_linear.argtypes = [p, p, p, i64, i64, i64, i64, p]
        lib.oracle_linear_at.argtypes = [p, p, p, i64, i64, i64, i64, p, p, i64, p]
        i32 = ctypes.c_int
        lib.oracle_linear_ex.argtypes = [p, i32, i32, p, p, i32, i64, i64, i64, i64, p]
        lib.oracle_decode_act.argtypes = [p, i32, i64, p]
        lib.oracle_decode_act.restype = ctypes.c_int
        lib.oracle_linear_at_ex.argtypes = [p, i32, i32, p, p, i32, i64, i64, i64, i64, p, p,
                                            i64, p]
        lib.oracle_gate_up_silu.argtypes = [p, i32, p, p, i32, i64, i64, i64, i64, p]
        f64 = ctypes.c_double
        lib.oracle_lora_shrink.argtypes = [p, p, i32, i32, i64, i64, i64, p]
        lib.oracle_lora_expand.argtypes = [p, p, i32, i32, f64, i64, i64, i64, p]
        lib.oracle_lora_expand_at.argtypes = [p, p, i32, i32, f64, i64, i64, i64, p, p, i64, p]
        lib.oracle_linear_lora.argtypes = [p, i32, p, p, i32, p, p, f64, i64, i64, i64, i64, i64,
                                           p]
        lib.oracle_linear_zp.argtypes = [p, i32, i32, p, p, i32, p, i32, i64, i64, i64, i64, p]
        lib.oracle_linear_zp.restype = ctypes.c_int
        lib.oracle_linear_zp_at.argtypes = [p, i32, p, p, i32, p, i32, i64, i64, i64, i64, p, p,
                                            i64, p]
        lib.oracle_linear_zp_at.restype = ctypes.c_int
        for f in (lib.oracle_unpack, lib.oracle_pack, lib.oracle_dequant,
                  lib.oracle_linear, lib.oracle_linear_at, lib.oracle_linear_ex,
                  lib.oracle_linear_at_ex, lib.oracle_gate_up_silu, lib.oracle_lora_shrink,
                  lib.oracle_lora_expand, lib.oracle_lora_expand_at, lib.oracle_linear_lora):
            f.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def pack(self, codes: np.ndarray) -> np.ndarray:
        """uint8 codes [K, N] -> int32 qweight [K/8, N]."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        K, N = codes.shape
        out = np.empty((K // 8, N), dtype=np.int32)
        _check(self.lib.oracle_pack(_ptr(codes), K, N, _ptr(out)), "pack")
        return out

    def unpack(self, qweight: np.ndarray) -> np.ndarray:
        """int32 qweight [K/8, N] -> uint8 codes [K, N]."""
        qweight = np.ascontiguousarray(qweight, dtype=np.int32)
        R, N = qweight.shape
        out = np.empty((8 * R, N), dtype=np.uint8)
        _check(self.lib.oracle_unpack(_ptr(qweight), 8 * R, N, _ptr(out)), "unpack")
        return out

    def dequant(self, qweight: np.ndarray, scales: np.ndarray, group_size: int,
                scales_type: str = "f16") -> np.ndarray:
        """Dense fp32 weight [K, N] = (q - 8) * s (scales fp16, or bfloat16 bit
        patterns as uint16 for scales_type "bf16")."""
        qweight = np.ascontiguousarray(qweight, dtype=np.int32)
        sb = _scale_bits(scales, scales_type)
        K, N = 8 * qweight.shape[0], qweight.shape[1]
        out = np.empty((K, N), dtype=np.float32)
        if scales_type == "f16":
            rc = self.lib.oracle_dequant(_ptr(qweight), _ptr(sb), K, N, group_size, _ptr(out))
        else:
            rc = self.lib.oracle_dequant_ex(_ptr(qweight), _ptr(sb), _SCALES[scales_type], K, N,
                                            group_size, _ptr(out))
        _check(rc, "dequant")
        return out

    def decode_act(self, x: np.ndarray, act: str = "f16") -> np.ndarray:
        """Activations (fp16 values, or bfloat16 bit patterns as uint16) -> float64,
        decoded field by field by the oracle."""
        xb = _act_bits(x, act)
        out = np.empty(xb.shape, dtype=np.float64)
        _check(self.lib.oracle_decode_act(_ptr(xb), _ACTS[act], xb.size, _ptr(out)),
               "decode_act")
        return out

    def linear_dense(self, x: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
                     group_size: int, act: str = "f16", scales_type: str = "f16") -> np.ndarray:
        """y [M, N] float64 = x . W through numpy's float64 matmul, with W the
        oracle's fp32 dequantised weight and x decoded by the oracle: the
        definition with a library matmul as its product step (any summation
        order, in fp64), for shapes too large for the triple loop."""
        xd = self.decode_act(x, act)
        W = self.dequant(qweight, scales, group_size, scales_type).astype(np.float64)
        if xd.shape[1] != W.shape[0]:
            raise ValueError("oracle linear_dense: x and qweight disagree on K")
        return np.matmul(xd, W)

    def linear(self, x: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
               group_size: int, act: str = "f16", absval: bool = False,
               scales_type: str = "f16") -> np.ndarray:
        """y [M, N] float64 = x [M, K] . dequant(qweight, scales).

        act "f16": x is fp16; act "bf16": x holds bfloat16 bit patterns (uint16).
        scales_type likewise for the scales.
        absval: return sum_k |x| * |w| instead (the error-bound magnitude)."""
        xb = _act_bits(x, act)
        qweight = np.ascontiguousarray(qweight, dtype=np.int32)
        sb = _scale_bits(scales, scales_type)
        M, K = xb.shape
        N = qweight.shape[1]
        if qweight.shape[0] * 8 != K:
            raise ValueError("qweight rows must be K/8")
        y = np.empty((M, N), dtype=np.float64)
        if act == "f16" and scales_type == "f16" and not absval:
            rc = self.lib.oracle_linear(_ptr(xb), _ptr(qweight), _ptr(sb), M, K, N, group_size,
                                        _ptr(y))
        else:
            rc = self.lib.oracle_linear_ex(_ptr(xb), _ACTS[act], int(absval), _ptr(qweight),
                                           _ptr(sb), _SCALES[scales_type], M, K, N, group_size,
                                           _ptr(y))
        _check(rc, "linear")
        return y

    def linear_at(self, x: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
                  group_size: int, ms: np.ndarray, ns: np.ndarray, act: str = "f16",
                  absval: bool = False, scales_type: str = "f16") -> np.ndarray:
        """y[ms[i], ns[i]] for sampled outputs, each computed from the definition
        (act, absval and scales_type as in linear)."""
        xb = _act_bits(x, act)
        qweight = np.ascontiguousarray(qweight, dtype=np.int32)
        sb = _scale_bits(scales, scales_type)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        M, K = xb.shape
        N = qweight.shape[1]
        out = np.empty(ms.shape[0], dtype=np.float64)
        if act == "f16" and scales_type == "f16" and not absval:
            rc = self.lib.oracle_linear_at(_ptr(xb), _ptr(qweight), _ptr(sb), M, K, N,
                                           group_size, _ptr(ms), _ptr(ns), ms.shape[0], _ptr(out))
        else:
            rc = self.lib.oracle_linear_at_ex(_ptr(xb), _ACTS[act], int(absval), _ptr(qweight),
                                              _ptr(sb), _SCALES[scales_type], M, K, N,
                                              group_size, _ptr(ms), _ptr(ns), ms.shape[0],
                                              _ptr(out))
        _check(rc, "linear_at")
        return out


    def gate_up_silu(self, x: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
                     group_size: int, act: str = "f16", scales_type: str = "f16") -> np.ndarray:
        """out [M, N/2] float64 = silu(y[:, 0::2]) * y[:, 1::2], y the linear (columns
        alternate gate and up)."""
        xb = _act_bits(x, act)
        qweight = np.ascontiguousarray(qweight, dtype=np.int32)
        sb = _scale_bits(scales, scales_type)
        M, K = xb.shape
        N = qweight.shape[1]
        out = np.empty((M, N // 2), dtype=np.float64)
        _check(self.lib.oracle_gate_up_silu(_ptr(xb), _ACTS[act], _ptr(qweight), _ptr(sb),
                                            _SCALES[scales_type], M, K, N, group_size,
                                            _ptr(out)), "gate_up_silu")
        return out

    # ---- LoRA adapter: A [r, K] and B [N, r] in the activation type ----

    def lora_shrink(self, x: np.ndarray, A: np.ndarray, act: str = "f16",
                    absval: bool = False) -> np.ndarray:
        """t [M, r] float64 = x . A^T (absval: sum_k |x| |A|)."""
        xb, Ab = _act_bits(x, act), _act_bits(A, act)
        M, K = xb.shape
        r = Ab.shape[0]
        if Ab.shape[1] != K:
            raise ValueError("A must be [r, K]")
        t = np.empty((M, r), dtype=np.float64)
        _check(self.lib.oracle_lora_shrink(_ptr(xb), _ptr(Ab), _ACTS[act], int(absval), M, K,
                                           r, _ptr(t)), "lora_shrink")
        return t

    def lora_expand(self, t: np.ndarray, B: np.ndarray, scale: float, act: str = "f16",
                    absval: bool = False) -> np.ndarray:
        """d [M, N] float64 = scale * t . B^T (absval: |scale| sum_j |t| |B|)."""
        t = np.ascontiguousarray(t, dtype=np.float64)
        Bb = _act_bits(B, act)
        M, r = t.shape
        N = Bb.shape[0]
        if Bb.shape[1] != r:
            raise ValueError("B must be [N, r]")
        d = np.empty((M, N), dtype=np.float64)
        _check(self.lib.oracle_lora_expand(_ptr(t), _ptr(Bb), _ACTS[act], int(absval),
                                           float(scale), M, N, r, _ptr(d)), "lora_expand")
        return d

    def lora_expand_at(self, t: np.ndarray, B: np.ndarray, scale: float, ms: np.ndarray,
                       ns: np.ndarray, act: str = "f16", absval: bool = False) -> np.ndarray:
        """d[ms[i], ns[i]] for sampled outputs (arguments as lora_expand)."""
        t = np.ascontiguousarray(t, dtype=np.float64)
        Bb = _act_bits(B, act)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        M, r = t.shape
        N = Bb.shape[0]
        out = np.empty(ms.shape[0], dtype=np.float64)
        _check(self.lib.oracle_lora_expand_at(_ptr(t), _ptr(Bb), _ACTS[act], int(absval),
                                              float(scale), M, N, r, _ptr(ms), _ptr(ns),
                                              ms.shape[0], _ptr(out)), "lora_expand_at")
        return out

    def linear_lora(self, x: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
                    group_size: int, A: np.ndarray, B: np.ndarray, scale: float,
                    act: str = "f16", scales_type: str = "f16") -> np.ndarray:
        """y [M, N] float64 = x . dequant(qweight, scales) + scale * (x . A^T) . B^T."""
        xb, Ab, Bb = _act_bits(x, act), _act_bits(A, act), _act_bits(B, act)
        qweight = np.ascontiguousarray(qweight, dtype=np.int32)
        sb = _scale_bits(scales, scales_type)
        M, K = xb.shape
        N = qweight.shape[1]
        r = Ab.shape[0]
        if Ab.shape != (r, K) or Bb.shape != (N, r):
            raise ValueError("A must be [r, K] and B [N, r]")
        y = np.empty((M, N), dtype=np.float64)
        _check(self.lib.oracle_linear_lora(_ptr(xb), _ACTS[act], _ptr(qweight), _ptr(sb),
                                           _SCALES[scales_type], _ptr(Ab), _ptr(Bb),
                                           float(scale), M, K, N, group_size, r, _ptr(y)),
               "linear_lora")
        return y

    def linear_zp(self, x: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
                  qzeros: np.ndarray, group_size: int, act: str = "f16",
                  absval: bool = False, scales_type: str = "f16",
                  zeros: str = "v2") -> np.ndarray:
        """y [M, N] float64 = x . W with W[k,n] = (q - z[k/g, n]) * s[k/g, n]; qzeros
        int32 [G, N/8], nibble j of word c the zero point of column 8c+j ("v2"),
        or that zero point minus one ("v1")."""
        xb = _act_bits(x, act)
        qweight = np.ascontiguousarray(qweight, dtype=np.int32)
        sb = _scale_bits(scales, scales_type)
        qzeros = np.ascontiguousarray(qzeros, dtype=np.int32)
        M, K = xb.shape
        N = qweight.shape[1]
        if qweight.shape[0] * 8 != K or qzeros.shape != (sb.shape[0], N // 8):
            raise ValueError("qweight must be [K/8, N] and qzeros [G, N/8]")
        y = np.empty((M, N), dtype=np.float64)
        _check(self.lib.oracle_linear_zp(_ptr(xb), _ACTS[act], int(absval), _ptr(qweight),
                                         _ptr(sb), _SCALES[scales_type], _ptr(qzeros),
                                         _ZEROS[zeros], M, K, N, group_size, _ptr(y)),
               "linear_zp")
        return y

    def linear_zp_at(self, x: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
                     qzeros: np.ndarray, group_size: int, ms: np.ndarray, ns: np.ndarray,
                     act: str = "f16", scales_type: str = "f16",
                     zeros: str = "v2") -> np.ndarray:
        """y[ms[i], ns[i]] of linear_zp for sampled outputs, each from the definition."""
        xb = _act_bits(x, act)
        qweight = np.ascontiguousarray(qweight, dtype=np.int32)
        sb = _scale_bits(scales, scales_type)
        qzeros = np.ascontiguousarray(qzeros, dtype=np.int32)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        M, K = xb.shape
        N = qweight.shape[1]
        if qzeros.shape != (sb.shape[0], N // 8):
            raise ValueError("qzeros must be [G, N/8]")
        out = np.empty(ms.shape[0], dtype=np.float64)
        _check(self.lib.oracle_linear_zp_at(_ptr(xb), _ACTS[act], _ptr(qweight), _ptr(sb),
                                            _SCALES[scales_type], _ptr(qzeros), _ZEROS[zeros],
                                            M, K, N, group_size, _ptr(ms), _ptr(ns),
                                            ms.shape[0], _ptr(out)), "linear_zp_at")
        return out


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle built from ``w4a16_oracle.c`` (compiled on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def num_threads() -> int:
    return default().num_threads()


def pack(codes):
    return default().pack(codes)


def unpack(qweight):
    return default().unpack(qweight)


def dequant(qweight, scales, group_size, scales_type="f16"):
    return default().dequant(qweight, scales, group_size, scales_type)


def decode_act(x, act="f16"):
    return default().decode_act(x, act)


def linear_dense(x, qweight, scales, group_size, act="f16", scales_type="f16"):
    return default().linear_dense(x, qweight, scales, group_size, act, scales_type)


def linear(x, qweight, scales, group_size, act="f16", absval=False, scales_type="f16"):
    return default().linear(x, qweight, scales, group_size, act, absval, scales_type)


def linear_at(x, qweight, scales, group_size, ms, ns, act="f16", absval=False,
              scales_type="f16"):
    return default().linear_at(x, qweight, scales, group_size, ms, ns, act, absval, scales_type)


def gate_up_silu(x, qweight, scales, group_size, act="f16", scales_type="f16"):
    return default().gate_up_silu(x, qweight, scales, group_size, act, scales_type)


def lora_shrink(x, A, act="f16", absval=False):
    return default().lora_shrink(x, A, act, absval)


def lora_expand(t, B, scale, act="f16", absval=False):
    return default().lora_expand(t, B, scale, act, absval)


def lora_expand_at(t, B, scale, ms, ns, act="f16", absval=False):
    return default().lora_expand_at(t, B, scale, ms, ns, act, absval)


def linear_lora(x, qweight, scales, group_size, A, B, scale, act="f16", scales_type="f16"):
    return default().linear_lora(x, qweight, scales, group_size, A, B, scale, act, scales_type)


def linear_zp(x, qweight, scales, qzeros, group_size, act="f16", absval=False,
              scales_type="f16", zeros="v2"):
    return default().linear_zp(x, qweight, scales, qzeros, group_size, act, absval, scales_type,
                               zeros)


def linear_zp_at(x, qweight, scales, qzeros, group_size, ms, ns, act="f16", scales_type="f16",
                 zeros="v2"):
    return default().linear_zp_at(x, qweight, scales, qzeros, group_size, ms, ns, act,
                                  scales_type, zeros)
