"""MI355X-native W4A16 symmetric-INT4 GPTQ linear: Python binding of libw4a16.so.

The binding only marshals arguments: every step of the linear runs in the
gfx950 HIP kernels of ``libw4a16.so``; PyTorch supplies device memory and
streams.  There is no fallback: if the library is missing or the device is
not a gfx950, calls raise.

Names match the C ABI in ``include/w4a16.h``:
  w4a16_linear, w4a16_linear_noalloc, w4a16_linear_ex, w4a16_linear_bf16,
  w4a16_linear_bf16_ex,
  w4a16_gate_up_silu(_ex, _bf16, _bf16_ex), w4a16_linear_lora(_bf16),
  w4a16_lora_workspace_bytes, w4a16_linear_zp(_bf16), w4a16_zp_workspace_bytes,
  w4a16_linear_typed, w4a16_stream_release, pack_gptq_v2, unpack_gptq_v2,
  w4a16_status_string, and the measurement aid w4a16_read_probe
plus ``linear``, ``gate_up_silu``, ``linear_lora`` and ``linear_zp`` (allocate
y, and a workspace, with torch, then call the entry point of x's and the
scales' dtypes).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

W4A16_OK = 0
W4A16_ERR_NULL = 1
W4A16_ERR_SHAPE = 2
W4A16_ERR_GROUP = 3
W4A16_ERR_ALIGN = 4
W4A16_ERR_CODE = 5
W4A16_ERR_DEVICE = 6
W4A16_ERR_LAUNCH = 7
W4A16_ERR_KERNEL = 8
W4A16_ERR_RANK = 9
W4A16_ERR_WORKSPACE = 10
W4A16_ERR_CAPTURE = 11
W4A16_ERR_SCRATCH = 12
W4A16_ERR_FLAGS = 13
W4A16_LORA_MAX_RANK = 1024

W4A16_DECODE_MAX_M = 16
W4A16_KERNEL_AUTO = 0
W4A16_KERNEL_DECODE = 1
W4A16_KERNEL_PREFILL = 2

W4A16_X_BF16 = 0x1
W4A16_SCALES_BF16 = 0x2
W4A16_ZEROS_V1 = 0x4
W4A16_GATE_UP_SILU = 0x8

EXPORTS = ("w4a16_linear", "w4a16_linear_noalloc", "w4a16_linear_ex", "w4a16_linear_bf16", "w4a16_linear_bf16_ex",
           "w4a16_gate_up_silu", "w4a16_gate_up_silu_ex", "w4a16_gate_up_silu_bf16",
           "w4a16_gate_up_silu_bf16_ex", "w4a16_linear_lora", "w4a16_linear_lora_bf16",
           "w4a16_lora_workspace_bytes", "w4a16_linear_zp", "w4a16_linear_zp_bf16",
           "w4a16_zp_workspace_bytes", "w4a16_linear_typed", "w4a16_stream_release",
           "pack_gptq_v2", "unpack_gptq_v2",
           "w4a16_read_probe", "w4a16_status_string")

_lib: Optional[ctypes.CDLL] = None


class W4A16Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {w4a16_status_string(status)} (status {status})")


def load_library() -> ctypes.CDLL:
    """Load libw4a16.so (built in-tree).  torch is imported first so that the
    library binds to the HIP runtime torch already loaded."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (HIP runtime shared with torch)
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.w4a16_linear.argtypes = [p, p, p, p, i64, i64, i64, i64, p]
    lib.w4a16_linear.restype = i32
    lib.w4a16_linear_noalloc.argtypes = [p, p, p, p, i64, i64, i64, i64, p]
    lib.w4a16_linear_noalloc.restype = i32
    lib.w4a16_linear_ex.argtypes = [p, p, p, p, i64, i64, i64, i64, p, i32]
    lib.w4a16_linear_ex.restype = i32
    lib.w4a16_linear_bf16.argtypes = [p, p, p, p, i64, i64, i64, i64, p]
    lib.w4a16_linear_bf16.restype = i32
    lib.w4a16_linear_bf16_ex.argtypes = [p, p, p, p, i64, i64, i64, i64, p, i32]
    lib.w4a16_linear_bf16_ex.restype = i32
    for name in ("w4a16_gate_up_silu", "w4a16_gate_up_silu_bf16"):
        getattr(lib, name).argtypes = [p, p, p, p, i64, i64, i64, i64, p]
        getattr(lib, name).restype = i32
    for name in ("w4a16_gate_up_silu_ex", "w4a16_gate_up_silu_bf16_ex"):
        getattr(lib, name).argtypes = [p, p, p, p, i64, i64, i64, i64, p, i32]
        getattr(lib, name).restype = i32
    f32, sz = ctypes.c_float, ctypes.c_size_t
    for name in ("w4a16_linear_lora", "w4a16_linear_lora_bf16"):
        getattr(lib, name).argtypes = [p, p, p, p, p, f32, p, i64, i64, i64, i64, i64, p, sz, p]
        getattr(lib, name).restype = i32
    lib.w4a16_lora_workspace_bytes.argtypes = [i64, i64, i64]
    lib.w4a16_lora_workspace_bytes.restype = sz
    for name in ("w4a16_linear_zp", "w4a16_linear_zp_bf16"):
        getattr(lib, name).argtypes = [p, p, p, p, p, i64, i64, i64, i64, p, sz, p]
        getattr(lib, name).restype = i32
    lib.w4a16_zp_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.w4a16_zp_workspace_bytes.restype = sz
    lib.w4a16_linear_typed.argtypes = [p, p, p, p, p, i64, i64, i64, i64, ctypes.c_uint, i32, p,
                                       sz, p]
    lib.w4a16_linear_typed.restype = i32
    lib.w4a16_stream_release.argtypes = [p]
    lib.w4a16_stream_release.restype = i32
    lib.pack_gptq_v2.argtypes = [p, p, i64, i64]
    lib.pack_gptq_v2.restype = i32
    lib.unpack_gptq_v2.argtypes = [p, p, i64, i64]
    lib.unpack_gptq_v2.restype = i32
    lib.w4a16_read_probe.argtypes = [p, i64, p, p]
    lib.w4a16_read_probe.restype = i32
    lib.w4a16_status_string.argtypes = [i32]
    lib.w4a16_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def w4a16_status_string(status: int) -> str:
    return load_library().w4a16_status_string(int(status)).decode()


def _addr(t) -> Optional[int]:
    """Device address of a torch tensor, or an integer address as given."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def w4a16_linear_noalloc(x, qweight, scales, y, M: int, K: int, N: int, group_size: int,
                         stream=None) -> None:
    """Same as the C ``w4a16_linear_noalloc``: w4a16_linear (fp16) with its split-K
    scratch in the library's static device array (allocates nothing; calls that
    overlap in time on one device race)."""
    st = load_library().w4a16_linear_noalloc(_addr(x), _addr(qweight), _addr(scales), _addr(y),
                                             int(M), int(K), int(N), int(group_size),
                                             _stream_handle(stream))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_linear_noalloc")


def w4a16_stream_release(stream=None) -> None:
    """Free the workspaces the library holds for `stream` (torch stream, raw
    handle, or None for the current stream) on the current device, after the
    stream's queued work; raises W4A16Error on a nonzero status."""
    st = load_library().w4a16_stream_release(_stream_handle(stream))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_stream_release")


def w4a16_linear_ex(x, qweight, scales, y, M: int, K: int, N: int, group_size: int,
                    stream=None, kernel: int = W4A16_KERNEL_AUTO) -> None:
    """Enqueue y = x . dequant(qweight, scales); raises W4A16Error on a nonzero status.

    Tensors (or raw device addresses) are passed through as pointers; the
    C library validates shapes, group size and alignment."""
    st = load_library().w4a16_linear_ex(_addr(x), _addr(qweight), _addr(scales), _addr(y),
                                        int(M), int(K), int(N), int(group_size),
                                        _stream_handle(stream), int(kernel))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_linear")


def w4a16_linear(x, qweight, scales, y, M: int, K: int, N: int, group_size: int,
                 stream=None) -> None:
    """Same as the C ``w4a16_linear`` (kernel chosen by M)."""
    w4a16_linear_ex(x, qweight, scales, y, M, K, N, group_size, stream, W4A16_KERNEL_AUTO)


def w4a16_linear_bf16_ex(x, qweight, scales, y, M: int, K: int, N: int, group_size: int,
                         stream=None, kernel: int = W4A16_KERNEL_AUTO) -> None:
    """As w4a16_linear_ex with bfloat16 x and y (scales stay fp16)."""
    st = load_library().w4a16_linear_bf16_ex(_addr(x), _addr(qweight), _addr(scales), _addr(y),
                                             int(M), int(K), int(N), int(group_size),
                                             _stream_handle(stream), int(kernel))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_linear_bf16")


def w4a16_linear_bf16(x, qweight, scales, y, M: int, K: int, N: int, group_size: int,
                      stream=None) -> None:
    """Same as the C ``w4a16_linear_bf16`` (kernel chosen by M)."""
    w4a16_linear_bf16_ex(x, qweight, scales, y, M, K, N, group_size, stream, W4A16_KERNEL_AUTO)


def w4a16_gate_up_silu_ex(x, qweight, scales, y, M: int, K: int, N: int, group_size: int,
                          stream=None, kernel: int = W4A16_KERNEL_AUTO, bf16: bool = False) -> None:
    """Merged gate/up projection with SiLU * mul: y [M, N/2] = silu(gate) * up, the
    columns of qweight and scales alternating gate and up (the C
    w4a16_gate_up_silu_ex, or its _bf16 form when bf16)."""
    lib = load_library()
    f = lib.w4a16_gate_up_silu_bf16_ex if bf16 else lib.w4a16_gate_up_silu_ex
    st = f(_addr(x), _addr(qweight), _addr(scales), _addr(y), int(M), int(K), int(N),
           int(group_size), _stream_handle(stream), int(kernel))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_gate_up_silu")


def w4a16_gate_up_silu(x, qweight, scales, y, M: int, K: int, N: int, group_size: int,
                       stream=None) -> None:
    """Same as the C ``w4a16_gate_up_silu`` (fp16, kernel chosen by M)."""
    w4a16_gate_up_silu_ex(x, qweight, scales, y, M, K, N, group_size, stream)


def w4a16_gate_up_silu_bf16(x, qweight, scales, y, M: int, K: int, N: int, group_size: int,
                            stream=None) -> None:
    """Same as the C ``w4a16_gate_up_silu_bf16``."""
    w4a16_gate_up_silu_ex(x, qweight, scales, y, M, K, N, group_size, stream, bf16=True)


def gate_up_silu(x, qweight, scales, group_size: int, out=None, stream=None,
                 kernel: int = W4A16_KERNEL_AUTO):
    """Allocate y ([M, N/2], x's dtype) and run the merged gate/up projection with
    SiLU * mul (columns of qweight and scales alternate gate and up); scales
    fp16, or bfloat16 with bfloat16 x."""
    import torch
    flags = _type_flags(x, scales)
    _check_tensors(("x", x, x.dtype), ("qweight", qweight, torch.int32),
                   ("scales", scales, scales.dtype))
    M, K = x.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 8 != K:
        raise ValueError("qweight must be [K/8, N]")
    if out is None:
        out = torch.empty((M, N // 2), dtype=x.dtype, device=x.device)
    elif out.dtype != x.dtype:
        raise ValueError("out must have x's dtype")
    if flags & W4A16_SCALES_BF16:
        w4a16_linear_typed(x, qweight, scales, None, out, M, K, N, group_size,
                           flags | W4A16_GATE_UP_SILU, kernel, stream=stream)
    else:
        w4a16_gate_up_silu_ex(x, qweight, scales, out, M, K, N, group_size, stream, kernel,
                              x.dtype == torch.bfloat16)
    return out


def w4a16_lora_workspace_bytes(M: int, K: int, rank: int) -> int:
    """Workspace bytes w4a16_linear_lora needs (0 for arguments it rejects)."""
    return int(load_library().w4a16_lora_workspace_bytes(int(M), int(K), int(rank)))


def w4a16_linear_lora(x, qweight, scales, lora_a, lora_b, lora_scale: float, y, M: int, K: int,
                      N: int, group_size: int, rank: int, workspace, workspace_bytes: int,
                      stream=None, bf16: bool = False) -> None:
    """y = x . dequant(qweight, scales) + lora_scale * (x . A^T) . B^T with
    A = lora_a [rank, K] and B = lora_b [N, rank] (the C w4a16_linear_lora, or
    its _bf16 form when bf16)."""
    lib = load_library()
    f = lib.w4a16_linear_lora_bf16 if bf16 else lib.w4a16_linear_lora
    st = f(_addr(x), _addr(qweight), _addr(scales), _addr(lora_a), _addr(lora_b),
           float(lora_scale), _addr(y), int(M), int(K), int(N), int(group_size), int(rank),
           _addr(workspace), int(workspace_bytes), _stream_handle(stream))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_linear_lora")


def w4a16_linear_lora_bf16(x, qweight, scales, lora_a, lora_b, lora_scale: float, y, M: int,
                           K: int, N: int, group_size: int, rank: int, workspace,
                           workspace_bytes: int, stream=None) -> None:
    """Same as the C ``w4a16_linear_lora_bf16``."""
    w4a16_linear_lora(x, qweight, scales, lora_a, lora_b, lora_scale, y, M, K, N, group_size,
                      rank, workspace, workspace_bytes, stream, bf16=True)


def linear_lora(x, qweight, scales, group_size: int, lora_a, lora_b, lora_scale: float,
                out=None, workspace=None, stream=None):
    """Allocate y (x's dtype, [M, N]) and, unless given, the workspace (a uint8
    device tensor) with torch, then run the linear with the LoRA term.  lora_a
    [rank, K] and lora_b [N, rank] have x's dtype."""
    import torch
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("x must be float16 or bfloat16")
    for name, t, dt in (("x", x, x.dtype), ("qweight", qweight, torch.int32),
                        ("scales", scales, torch.float16), ("lora_a", lora_a, x.dtype),
                        ("lora_b", lora_b, x.dtype)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} device tensor")
    M, K = x.shape
    N = qweight.shape[1]
    rank = lora_a.shape[0]
    if qweight.shape[0] * 8 != K:
        raise ValueError("qweight must be [K/8, N]")
    if tuple(lora_a.shape) != (rank, K) or tuple(lora_b.shape) != (N, rank):
        raise ValueError("lora_a must be [rank, K] and lora_b [N, rank]")
    need = w4a16_lora_workspace_bytes(M, K, rank)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    elif out.dtype != x.dtype:
        raise ValueError("out must have x's dtype")
    w4a16_linear_lora(x, qweight, scales, lora_a, lora_b, lora_scale, out, M, K, N, group_size,
                      rank, workspace, workspace.numel() * workspace.element_size(), stream,
                      x.dtype == torch.bfloat16)
    return out


def w4a16_zp_workspace_bytes(M: int, K: int, N: int, group_size: int) -> int:
    """Workspace bytes w4a16_linear_zp needs (0 for arguments it rejects)."""
    return int(load_library().w4a16_zp_workspace_bytes(int(M), int(K), int(N), int(group_size)))


def w4a16_linear_zp(x, qweight, scales, qzeros, y, M: int, K: int, N: int, group_size: int,
                    workspace, workspace_bytes: int, stream=None, bf16: bool = False) -> None:
    """y = x . W with W[k,n] = (q - z[k/g, n]) s[k/g, n], qzeros int32 [G, N/8] (the C
    w4a16_linear_zp, or its _bf16 form when bf16)."""
    lib = load_library()
    f = lib.w4a16_linear_zp_bf16 if bf16 else lib.w4a16_linear_zp
    st = f(_addr(x), _addr(qweight), _addr(scales), _addr(qzeros), _addr(y), int(M), int(K),
           int(N), int(group_size), _addr(workspace), int(workspace_bytes), _stream_handle(stream))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_linear_zp")


def w4a16_linear_zp_bf16(x, qweight, scales, qzeros, y, M: int, K: int, N: int,
                         group_size: int, workspace, workspace_bytes: int, stream=None) -> None:
    """Same as the C ``w4a16_linear_zp_bf16``."""
    w4a16_linear_zp(x, qweight, scales, qzeros, y, M, K, N, group_size, workspace,
                    workspace_bytes, stream, bf16=True)


def pack_zeros(zeros: np.ndarray) -> np.ndarray:
    """uint8 zero points [G, N] (values 0..15) -> int32 qzeros [G, N/8] packed along N
    (pack_gptq_v2 of the transpose, transposed back)."""
    z = np.ascontiguousarray(np.asarray(zeros, dtype=np.uint8).T)
    return np.ascontiguousarray(pack_gptq_v2(z).T)


def linear_zp(x, qweight, scales, qzeros, group_size: int, out=None, workspace=None,
              stream=None, zeros_format: str = "v2", kernel: int = W4A16_KERNEL_AUTO):
    """Allocate y (x's dtype, [M, N]) and, unless given, the workspace with torch, then
    run the linear with stored zero points (qzeros int32 [G, N/8]; zeros_format "v2":
    each nibble is the zero point, "v1": the zero point minus one).  Scales fp16,
    or bfloat16 with bfloat16 x."""
    import torch
    flags = _type_flags(x, scales)
    if zeros_format not in ("v1", "v2"):
        raise ValueError("zeros_format must be 'v1' or 'v2'")
    _check_tensors(("x", x, x.dtype), ("qweight", qweight, torch.int32),
                   ("scales", scales, scales.dtype), ("qzeros", qzeros, torch.int32))
    M, K = x.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 8 != K or tuple(qzeros.shape) != (scales.shape[0], N // 8):
        raise ValueError("qweight must be [K/8, N] and qzeros [G, N/8]")
    need = w4a16_zp_workspace_bytes(M, K, N, group_size)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    elif out.dtype != x.dtype:
        raise ValueError("out must have x's dtype")
    if zeros_format == "v1":
        flags |= W4A16_ZEROS_V1
    nbytes = workspace.numel() * workspace.element_size()
    if flags & (W4A16_SCALES_BF16 | W4A16_ZEROS_V1) or kernel != W4A16_KERNEL_AUTO:
        w4a16_linear_typed(x, qweight, scales, qzeros, out, M, K, N, group_size, flags, kernel,
                           workspace, nbytes, stream)
    else:
        w4a16_linear_zp(x, qweight, scales, qzeros, out, M, K, N, group_size, workspace, nbytes,
                        stream, x.dtype == torch.bfloat16)
    return out


def w4a16_linear_typed(x, qweight, scales, qzeros, y, M: int, K: int, N: int, group_size: int,
                       flags: int, kernel: int = W4A16_KERNEL_AUTO, workspace=None,
                       workspace_bytes: int = 0, stream=None) -> None:
    """Same as the C ``w4a16_linear_typed``: the variant chosen by flags
    (W4A16_X_BF16, W4A16_SCALES_BF16, W4A16_ZEROS_V1, W4A16_GATE_UP_SILU) and by
    whether qzeros is None; raises W4A16Error on a nonzero status."""
    st = load_library().w4a16_linear_typed(_addr(x), _addr(qweight), _addr(scales),
                                           _addr(qzeros), _addr(y), int(M), int(K), int(N),
                                           int(group_size), int(flags), int(kernel),
                                           _addr(workspace), int(workspace_bytes),
                                           _stream_handle(stream))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_linear_typed")


def _type_flags(x, scales) -> int:
    """Flags for x's and the scales' dtypes (fp16 x takes fp16 scales only)."""
    import torch
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("x must be float16 or bfloat16")
    if scales.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("scales must be float16 or bfloat16")
    if scales.dtype == torch.bfloat16 and x.dtype != torch.bfloat16:
        raise ValueError("bfloat16 scales need bfloat16 x")
    return ((W4A16_X_BF16 if x.dtype == torch.bfloat16 else 0)
            | (W4A16_SCALES_BF16 if scales.dtype == torch.bfloat16 else 0))


def _check_tensors(*specs) -> None:
    for name, t, dt in specs:
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} device tensor")


def w4a16_read_probe(data, nbytes: int, sink, stream=None) -> None:
    """Enqueue the streaming-read probe over nbytes at data (a measurement
    aid: the attainable HBM read rate); raises W4A16Error on a nonzero status."""
    st = load_library().w4a16_read_probe(_addr(data), int(nbytes), _addr(sink),
                                         _stream_handle(stream))
    if st != W4A16_OK:
        raise W4A16Error(st, "w4a16_read_probe")


def pack_gptq_v2(codes: np.ndarray) -> np.ndarray:
    """Host uint8 codes [K, N] (0..15) -> int32 qweight [K/8, N]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    K, N = codes.shape
    out = np.empty((K // 8, N), dtype=np.int32)
    st = load_library().pack_gptq_v2(codes.ctypes.data, out.ctypes.data, K, N)
    if st != W4A16_OK:
        raise W4A16Error(st, "pack_gptq_v2")
    return out


def unpack_gptq_v2(qweight: np.ndarray) -> np.ndarray:
    """Host int32 qweight [K/8, N] -> uint8 codes [K, N]."""
    qweight = np.ascontiguousarray(qweight, dtype=np.int32)
    R, N = qweight.shape
    out = np.empty((8 * R, N), dtype=np.uint8)
    st = load_library().unpack_gptq_v2(qweight.ctypes.data, out.ctypes.data, 8 * R, N)
    if st != W4A16_OK:
        raise W4A16Error(st, "unpack_gptq_v2")
    return out


def linear(x, qweight, scales, group_size: int, out=None, stream=None,
           kernel: int = W4A16_KERNEL_AUTO):
    """Allocate y (x's dtype, [M, N]) with torch on x's device and run the linear.

    x: fp16 or bfloat16 [M, K] (y has the same dtype); qweight: int32 [K/8, N];
    scales: fp16 [G, N], or bfloat16 with bfloat16 x; all CUDA (HIP) tensors,
    contiguous."""
    import torch
    flags = _type_flags(x, scales)
    _check_tensors(("x", x, x.dtype), ("qweight", qweight, torch.int32),
                   ("scales", scales, scales.dtype))
    M, K = x.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 8 != K:
        raise ValueError("qweight must be [K/8, N]")
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    elif out.dtype != x.dtype:
        raise ValueError("out must have x's dtype")
    if flags & W4A16_SCALES_BF16:
        w4a16_linear_typed(x, qweight, scales, None, out, M, K, N, group_size, flags, kernel,
                           stream=stream)
    else:
        call = w4a16_linear_bf16_ex if x.dtype == torch.bfloat16 else w4a16_linear_ex
        call(x, qweight, scales, out, M, K, N, group_size, stream, kernel)
    return out
