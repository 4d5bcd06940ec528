"""Thin ctypes binding of libmxq.so (argument marshalling only).

Every step of the computation runs in libmxq's HIP kernels; this module only
checks tensor metadata, passes raw device pointers and the current HIP stream,
and turns a non-OK status into an exception.  PyTorch is used for device
memory and streams only.  There is no fallback: if the library is missing or
fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxq.so")

MXQ_OK, MXQ_ERR_INVALID_ARG, MXQ_ERR_UNSUPPORTED, MXQ_ERR_MISALIGNED, MXQ_ERR_HIP = range(5)
MXQ_F16, MXQ_BF16, MXQ_F32 = 0, 1, 2
ABI_VERSION = 4

_lock = threading.Lock()
_lib = None


class MxqError(RuntimeError):
    """A libmxq call returned a status other than MXQ_OK."""

    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name
        self.detail = detail


class QmvProblem(ctypes.Structure):
    """ctypes mirror of ``mxq_qmv_problem`` (include/mxq.h)."""

    _fields_ = [("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64)]


def _declare(lib):
    c_i64, c_int, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    fused = [vp, vp, vp, vp, vp, c_i64, c_i64, c_i64, c_int, c_int, c_int, vp]
    for name in ("mxq_qmv", "mxq_qmm", "mxq_qmm_noalloc"):
        f = getattr(lib, name)
        f.argtypes, f.restype = fused, c_int
    lib.mxq_linear.argtypes = [vp, vp, vp, vp, vp, vp, c_i64, c_i64, c_i64, c_int, c_int, c_int, vp]
    lib.mxq_linear.restype = c_int
    lib.mxq_linear_act.argtypes = [vp, vp, vp, vp, vp, vp, c_i64, c_i64, c_i64, c_int, c_int, c_int, c_int, vp]
    lib.mxq_linear_act.restype = c_int
    lib.mxq_linear_a8.argtypes = [vp, vp, vp, vp, vp, vp, c_i64, c_i64, c_i64, c_int, c_int, c_int, vp]
    lib.mxq_linear_a8.restype = c_int
    lib.mxq_qmv_grouped.argtypes = [ctypes.POINTER(QmvProblem), c_int, c_i64, c_int, c_int, c_int, vp]
    lib.mxq_qmv_grouped.restype = c_int
    lib.mxq_dequant.argtypes = [vp, vp, vp, vp, c_i64, c_i64, c_int, c_int, c_int, c_int, vp]
    lib.mxq_dequant.restype = c_int
    lib.mxq_pack.argtypes = [vp, vp, c_i64, c_i64, c_int]
    lib.mxq_pack.restype = c_int
    lib.mxq_describe.argtypes = [ctypes.c_char_p, c_i64, c_i64, c_i64, c_int, c_int, c_int]
    lib.mxq_describe.restype = ctypes.c_char_p
    lib.mxq_describe_grouped.argtypes = [ctypes.POINTER(QmvProblem), c_int, c_i64, c_int, c_int, c_int]
    lib.mxq_describe_grouped.restype = ctypes.c_char_p
    lib.mxq_release_workspaces.argtypes, lib.mxq_release_workspaces.restype = [], c_int
    lib.mxq_read_probe.argtypes, lib.mxq_read_probe.restype = [vp, c_i64, vp, vp], c_int
    lib.mxq_workspace_bytes.argtypes, lib.mxq_workspace_bytes.restype = [], c_i64
    lib.mxq_status_str.argtypes, lib.mxq_status_str.restype = [c_int], ctypes.c_char_p
    lib.mxq_last_error.argtypes, lib.mxq_last_error.restype = [], ctypes.c_char_p
    lib.mxq_abi_version.argtypes, lib.mxq_abi_version.restype = [], c_int
    return lib


def load(build_if_missing: bool = True):
    """Load libmxq.so (building it first only if no built library exists)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            if not build_if_missing:
                raise OSError(f"{LIB_PATH} is not built")
            from . import build as _build
            _build.build()
        lib = _declare(ctypes.CDLL(LIB_PATH))
        if lib.mxq_abi_version() != ABI_VERSION:
            raise OSError(f"libmxq ABI {lib.mxq_abi_version()} != binding ABI {ABI_VERSION}")
        _lib = lib
        return lib


def _check(lib, status: int):
    if status != MXQ_OK:
        raise MxqError(status, lib.mxq_status_str(status).decode(), lib.mxq_last_error().decode())


# --------------------------------------------------------------------------
# torch-facing wrappers
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _sb_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return MXQ_F16
    if t.dtype == torch.bfloat16:
        return MXQ_BF16
    raise TypeError(f"scales/biases must be float16 or bfloat16, got {t.dtype}")


def _stream_handle(dev, stream):
    torch = _torch()
    s = torch.cuda.current_stream(dev) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_packed(x, w, scales, biases, bits, group_size, who, act_dtypes=None):
    torch = _torch()
    if bits not in (4, 8):
        raise ValueError(f"{who}: bits must be 4 or 8")
    act_dtypes = (torch.float16,) if act_dtypes is None else act_dtypes
    if x.dtype not in act_dtypes or x.dim() != 2:
        names = " or ".join(str(d).replace("torch.", "") for d in act_dtypes)
        raise TypeError(f"{who}: x must be a 2-D {names} tensor")
    if w.dtype not in (torch.int32, torch.uint32) or w.dim() != 2:
        raise TypeError(f"{who}: w must be a 2-D int32/uint32 tensor of packed words")
    if scales.dtype != biases.dtype or scales.shape != biases.shape or scales.dim() != 2:
        raise TypeError(f"{who}: scales and biases must share dtype and a 2-D shape")
    for name, t in (("x", x), ("w", w), ("scales", scales), ("biases", biases)):
        if not t.is_cuda:
            raise ValueError(f"{who}: {name} must be a device tensor")
        if t.device != x.device:
            raise ValueError(f"{who}: all tensors must be on one device")
        if not t.is_contiguous():
            raise ValueError(f"{who}: {name} must be contiguous")
    M, K = x.shape
    N, kw = w.shape
    if kw * (32 // bits) != K:
        raise ValueError(f"{who}: w has {kw} words per row, x has K={K} ({bits}-bit codes)")
    if K % group_size or tuple(scales.shape) != (N, K // group_size):
        raise ValueError(f"{who}: scales/biases must be [N, K/group_size] = {(N, K // max(group_size, 1))}")
    return M, N, K


def _fused(name, x, w, scales, biases, y, bits, group_size, stream):
    torch = _torch()
    lib = load()
    M, N, K = _check_packed(x, w, scales, biases, bits, group_size, name)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    elif y.dtype != torch.float16 or tuple(y.shape) != (M, N) or not y.is_contiguous() \
            or y.device != x.device:
        raise ValueError(f"{name}: y must be a contiguous float16 [M, N] tensor on x's device")
    with torch.cuda.device(x.device):
        st = getattr(lib, name)(x.data_ptr(), w.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                                y.data_ptr(), M, N, K, bits, group_size, _sb_code(scales),
                                _stream_handle(x.device, stream))
    _check(lib, st)
    return y


def mxq_qmv(x, w, scales, biases, y=None, *, bits: int = 4, group_size: int = 64, stream=None):
    """y = x @ dequant(w).T via the decode kernel (any M; tuned for M <= 8)."""
    return _fused("mxq_qmv", x, w, scales, biases, y, bits, group_size, stream)


def mxq_qmv_grouped(problems, *, bits: int = 4, group_size: int = 64, stream=None):
    """Several independent qmv problems in one launch.

    ``problems`` is a sequence of ``(x, w, scales, biases)`` or
    ``(x, w, scales, biases, y)`` tuples of device tensors sharing M, bits,
    group size and scale dtype; returns the list of y tensors."""
    torch = _torch()
    lib = load()
    if not problems:
        return []
    arr = (QmvProblem * len(problems))()
    ys, M0, sb0, dev0 = [], None, None, None
    for i, prob in enumerate(problems):
        x, w, s, b = prob[:4]
        y = prob[4] if len(prob) > 4 else None
        M, N, K = _check_packed(x, w, s, b, bits, group_size, f"mxq_qmv_grouped[{i}]")
        if M0 is None:
            M0, sb0, dev0 = M, _sb_code(s), x.device
        elif M != M0 or _sb_code(s) != sb0 or x.device != dev0:
            raise ValueError("mxq_qmv_grouped: problems must share M, scale dtype and device")
        if y is None:
            y = torch.empty((M, N), dtype=torch.float16, device=x.device)
        elif y.dtype != torch.float16 or tuple(y.shape) != (M, N) or not y.is_contiguous() \
                or y.device != x.device:
            raise ValueError(f"mxq_qmv_grouped[{i}]: y must be a contiguous float16 [M, N] tensor")
        arr[i] = QmvProblem(x.data_ptr(), w.data_ptr(), s.data_ptr(), b.data_ptr(), y.data_ptr(), N, K)
        ys.append(y)
    with torch.cuda.device(dev0):
        st = lib.mxq_qmv_grouped(arr, len(problems), M0, bits, group_size, sb0, _stream_handle(dev0, stream))
    _check(lib, st)
    return ys


def mxq_qmm(x, w, scales, biases, y=None, *, bits: int = 4, group_size: int = 64, stream=None):
    """y = x @ dequant(w).T via the MFMA prefill kernel (any M; MFMA for M > 8)."""
    return _fused("mxq_qmm", x, w, scales, biases, y, bits, group_size, stream)


def mxq_qmm_noalloc(x, w, scales, biases, y=None, *, bits: int = 4, group_size: int = 64, stream=None):
    """mxq_qmm that allocates no device memory: split-K partial results go to
    the library's fixed 32 MiB scratch per GPU (calls needing more are
    rejected; calls that overlap on one GPU race)."""
    return _fused("mxq_qmm_noalloc", x, w, scales, biases, y, bits, group_size, stream)


def mxq_linear(x, w, scales, biases, bias=None, y=None, *, bits: int = 4, group_size: int = 64,
               stream=None):
    """y = x @ dequant(w).T + bias: a quantized linear layer with an optional
    float16 output bias [N] (None: same result as mxq_qmm)."""
    torch = _torch()
    lib = load()
    M, N, K = _check_packed(x, w, scales, biases, bits, group_size, "mxq_linear")
    if bias is not None and (bias.dtype != torch.float16 or tuple(bias.shape) != (N,) or not bias.is_cuda
                             or not bias.is_contiguous() or bias.device != x.device):
        raise ValueError("mxq_linear: bias must be a contiguous float16 [N] tensor on x's device")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    elif y.dtype != torch.float16 or tuple(y.shape) != (M, N) or not y.is_contiguous() or y.device != x.device:
        raise ValueError("mxq_linear: y must be a contiguous float16 [M, N] tensor on x's device")
    with torch.cuda.device(x.device):
        st = lib.mxq_linear(x.data_ptr(), w.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                            None if bias is None else bias.data_ptr(), y.data_ptr(), M, N, K, bits,
                            group_size, _sb_code(scales), _stream_handle(x.device, stream))
    _check(lib, st)
    return y


def mxq_linear_act(x, w, scales, biases, bias=None, y=None, *, bits: int = 4, group_size: int = 64,
                   stream=None):
    """mxq_linear for float16 or bfloat16 activations: x, the optional output
    bias [N] and y share x's dtype (float16 gives exactly mxq_linear's result)."""
    torch = _torch()
    lib = load()
    M, N, K = _check_packed(x, w, scales, biases, bits, group_size, "mxq_linear_act",
                            (torch.float16, torch.bfloat16))
    act = MXQ_BF16 if x.dtype == torch.bfloat16 else MXQ_F16
    if bias is not None and (bias.dtype != x.dtype or tuple(bias.shape) != (N,) or not bias.is_cuda
                             or not bias.is_contiguous() or bias.device != x.device):
        raise ValueError("mxq_linear_act: bias must be a contiguous [N] tensor of x's dtype on x's device")
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    elif y.dtype != x.dtype or tuple(y.shape) != (M, N) or not y.is_contiguous() or y.device != x.device:
        raise ValueError("mxq_linear_act: y must be a contiguous [M, N] tensor of x's dtype on x's device")
    with torch.cuda.device(x.device):
        st = lib.mxq_linear_act(x.data_ptr(), w.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                                None if bias is None else bias.data_ptr(), y.data_ptr(), M, N, K, bits,
                                group_size, _sb_code(scales), act, _stream_handle(x.device, stream))
    _check(lib, st)
    return y


def mxq_linear_a8(x, w, scales, biases, bias=None, y=None, *, bits: int = 4, group_size: int = 64,
                  stream=None):
    """mxq_linear on the native int8 path: float16 x quantized per row to int8
    inside the kernel (the scheme is stated in include/mxq.h), v_dot4 products;
    optional float16 output bias [N]; float16 y."""
    torch = _torch()
    lib = load()
    M, N, K = _check_packed(x, w, scales, biases, bits, group_size, "mxq_linear_a8")
    if bias is not None and (bias.dtype != torch.float16 or tuple(bias.shape) != (N,) or not bias.is_cuda
                             or not bias.is_contiguous() or bias.device != x.device):
        raise ValueError("mxq_linear_a8: bias must be a contiguous float16 [N] tensor on x's device")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    elif y.dtype != torch.float16 or tuple(y.shape) != (M, N) or not y.is_contiguous() or y.device != x.device:
        raise ValueError("mxq_linear_a8: y must be a contiguous float16 [M, N] tensor on x's device")
    with torch.cuda.device(x.device):
        st = lib.mxq_linear_a8(x.data_ptr(), w.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                               None if bias is None else bias.data_ptr(), y.data_ptr(), M, N, K, bits,
                               group_size, _sb_code(scales), _stream_handle(x.device, stream))
    _check(lib, st)
    return y


def mxq_dequant(w, scales, biases, out=None, *, bits: int = 4, group_size: int = 64,
                out_dtype=None, stream=None):
    """out[n, k] = q*s + b as float32 (default), float16 or bfloat16, bit-exact."""
    torch = _torch()
    lib = load()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    codes = {torch.float16: MXQ_F16, torch.bfloat16: MXQ_BF16, torch.float32: MXQ_F32}
    if out_dtype not in codes:
        raise TypeError("out_dtype must be float32, float16 or bfloat16")
    if w.dim() != 2 or not w.is_cuda or not w.is_contiguous():
        raise ValueError("mxq_dequant: w must be a contiguous 2-D device tensor")
    N, kw = w.shape
    K = kw * (32 // bits)
    for name, t in (("scales", scales), ("biases", biases)):
        if not t.is_cuda or not t.is_contiguous() or t.device != w.device:
            raise ValueError(f"mxq_dequant: {name} must be contiguous on w's device")
    if out is None:
        out = torch.empty((N, K), dtype=out_dtype, device=w.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (N, K) or not out.is_contiguous():
        raise ValueError("mxq_dequant: out must be a contiguous [N, K] tensor of out_dtype")
    with torch.cuda.device(w.device):
        st = lib.mxq_dequant(w.data_ptr(), scales.data_ptr(), biases.data_ptr(), out.data_ptr(),
                             N, K, bits, group_size, _sb_code(scales), codes[out_dtype],
                             _stream_handle(w.device, stream))
    _check(lib, st)
    return out


def mxq_describe(op: str, M: int, N: int, K: int, bits: int = 4, group_size: int = 64,
                 sb_dtype: str = "f16") -> str:
    """Kernel instantiation and launch shape mxq_qmv ("qmv") / mxq_qmm ("qmm") would use."""
    lib = load()
    sb = {"f16": MXQ_F16, "bf16": MXQ_BF16}[sb_dtype]
    return lib.mxq_describe(op.encode(), M, N, K, bits, group_size, sb).decode()


def mxq_describe_grouped(shapes, M: int, bits: int = 4, group_size: int = 64, sb_dtype: str = "f16") -> str:
    """Launches mxq_qmv_grouped would make for problems of these (N, K) shapes."""
    lib = load()
    sb = {"f16": MXQ_F16, "bf16": MXQ_BF16}[sb_dtype]
    arr = (QmvProblem * len(shapes))(*[QmvProblem(None, None, None, None, None, N, K) for N, K in shapes])
    return lib.mxq_describe_grouped(arr, len(shapes), M, bits, group_size, sb).decode()


def mxq_release_workspaces() -> None:
    """Free the cached split workspaces (waits for enqueued work first)."""
    lib = load()
    _check(lib, lib.mxq_release_workspaces())


def mxq_workspace_bytes() -> int:
    """Bytes of split workspace cached for the current device."""
    return int(load().mxq_workspace_bytes())


def mxq_pack(codes, bits: int = 4) -> np.ndarray:
    """Host packer: uint8 codes [N, K] -> uint32 words [N, K*bits/32]."""
    lib = load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    if c.ndim != 2:
        raise ValueError("mxq_pack: codes must be 2-D")
    N, K = c.shape
    per = 32 // bits if bits in (4, 8) else 1
    out = np.zeros((N, K // per if per else 0), dtype=np.uint32)
    _check(lib, lib.mxq_pack(c.ctypes.data, out.ctypes.data, N, K, bits))
    return out
