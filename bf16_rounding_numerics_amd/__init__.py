"""Python binding of libaddrmsnorm.so: fused residual-add + RMSNorm forward
for MI355X (gfx950) with round-to-nearest-even bf16 stores.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C entry points declared in include/add_rmsnorm.h; the
functions here carry the same names, take torch tensors (used only as device
memory) and pass their pointers, shapes and the current HIP stream through.
There is no fallback: without the built library, or without a GPU tensor,
the calls raise.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libaddrmsnorm.so")

ABI_VERSION = 10
MAX_HIDDEN = 32768

OK = 0
EINVAL = -1
EALIGN = -2
EALIAS = -3
ERANGE = -4
EHIP = -5

PATH_AUTO = 0
PATH_WAVE_ROW = 1
PATH_WG_ROW = 2
PATH_LDS_TWO_PASS = 3
PATH_GENERAL = 4
PATH_PACKED = 5
FLAG_LATE_WEIGHT = 1  # flags on PATH_WG_ROW: the weight read after each row's barrier


class AddRmsnormError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("add_rmsnorm status %d: %s" % (status, message))
        self.status = status


LOG1P_FLAG_ACCURATE_ONLY = 1


class Log1pCfg(ctypes.Structure):
    """struct log1p_launch_cfg."""
    _fields_ = [("block_threads", ctypes.c_int32), ("elems_per_thread", ctypes.c_int32),
                ("grid_blocks", ctypes.c_int32), ("flags", ctypes.c_int32)]


class LaunchCfg(ctypes.Structure):
    """struct add_rmsnorm_launch_cfg."""
    _fields_ = [("path", ctypes.c_int32), ("block_threads", ctypes.c_int32),
                ("grid_blocks", ctypes.c_int32), ("flags", ctypes.c_int32)]


_lib = None

EXPORTS = ("add_rmsnorm_fwd", "add_rmsnorm_fwd_cfg", "add_rmsnorm_fwd_strided",
           "rmsnorm_fwd_strided", "add_rmsnorm_quant_fwd", "add_rmsnorm_quant_fwd_cfg",
           "rmsnorm_fwd", "rmsnorm_fwd_cfg", "rmsnorm_quant_fwd", "rmsnorm_quant_fwd_cfg",
           "add_rmsnorm_quant_fp8_fwd", "add_rmsnorm_quant_fp8_fwd_cfg", "rmsnorm_quant_fp8_fwd",
           "rmsnorm_quant_fp8_fwd_cfg", "add_rmsnorm_quant_fwd_strided",
           "add_rmsnorm_quant_fp8_fwd_strided", "rmsnorm_quant_fwd_strided",
           "rmsnorm_quant_fp8_fwd_strided", "qk_rmsnorm_fwd", "qk_rmsnorm_fwd_cfg",
           "log1p_f32", "log1p_f32_cfg",
           "add_rmsnorm_test_cvt_range", "add_rmsnorm_test_cvt_e4m3_range",
           "add_rmsnorm_test_copy2", "add_rmsnorm_test_copy_rows",
           "add_rmsnorm_test_stream", "add_rmsnorm_strerror", "add_rmsnorm_last_hip_error",
           "add_rmsnorm_abi_version", "add_rmsnorm_build_info")


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise ImportError(
            "%s is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')"
            % LIBRARY)
    L = ctypes.CDLL(LIBRARY)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    L.add_rmsnorm_fwd.restype = i32
    L.add_rmsnorm_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, vp]
    L.add_rmsnorm_fwd_cfg.restype = i32
    L.add_rmsnorm_fwd_cfg.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32,
                                      ctypes.POINTER(LaunchCfg), vp]
    L.add_rmsnorm_quant_fwd.restype = i32
    L.add_rmsnorm_quant_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, vp]
    L.add_rmsnorm_quant_fwd_cfg.restype = i32
    L.add_rmsnorm_quant_fwd_cfg.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32,
                                            ctypes.POINTER(LaunchCfg), vp]
    L.add_rmsnorm_fwd_strided.restype = i32
    L.add_rmsnorm_fwd_strided.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, i64, f32,
                                          ctypes.POINTER(LaunchCfg), vp]
    L.rmsnorm_fwd_strided.restype = i32
    L.rmsnorm_fwd_strided.argtypes = [vp, i64, vp, i64, vp, i64, i64, f32,
                                      ctypes.POINTER(LaunchCfg), vp]
    L.rmsnorm_fwd.restype = i32
    L.rmsnorm_fwd.argtypes = [vp, vp, vp, i64, i64, f32, vp]
    L.rmsnorm_fwd_cfg.restype = i32
    L.rmsnorm_fwd_cfg.argtypes = [vp, vp, vp, i64, i64, f32, ctypes.POINTER(LaunchCfg), vp]
    L.rmsnorm_quant_fwd.restype = i32
    L.rmsnorm_quant_fwd.argtypes = [vp, vp, vp, vp, i64, i64, f32, vp]
    L.rmsnorm_quant_fwd_cfg.restype = i32
    L.rmsnorm_quant_fwd_cfg.argtypes = [vp, vp, vp, vp, i64, i64, f32,
                                        ctypes.POINTER(LaunchCfg), vp]
    L.log1p_f32.restype = i32
    for name in ("add_rmsnorm_quant_fp8_fwd", "add_rmsnorm_quant_fp8_fwd_cfg"):
        getattr(L, name).restype = i32
    L.add_rmsnorm_quant_fp8_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, vp]
    L.add_rmsnorm_quant_fp8_fwd_cfg.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32,
                                                ctypes.POINTER(LaunchCfg), vp]
    L.rmsnorm_quant_fp8_fwd.restype = i32
    L.rmsnorm_quant_fp8_fwd.argtypes = [vp, vp, vp, vp, i64, i64, f32, vp]
    L.rmsnorm_quant_fp8_fwd_cfg.restype = i32
    L.rmsnorm_quant_fp8_fwd_cfg.argtypes = [vp, vp, vp, vp, i64, i64, f32,
                                            ctypes.POINTER(LaunchCfg), vp]
    L.add_rmsnorm_test_cvt_e4m3_range.restype = i32
    L.add_rmsnorm_test_cvt_e4m3_range.argtypes = [vp, ctypes.c_uint32, i64, vp]
    for name in ("add_rmsnorm_quant_fwd_strided", "add_rmsnorm_quant_fp8_fwd_strided"):
        getattr(L, name).restype = i32
        getattr(L, name).argtypes = [vp, vp, vp, i64, vp, i64, vp, i64, vp, i64, i64, f32,
                                     ctypes.POINTER(LaunchCfg), vp]
    for name in ("rmsnorm_quant_fwd_strided", "rmsnorm_quant_fp8_fwd_strided"):
        getattr(L, name).restype = i32
        getattr(L, name).argtypes = [vp, vp, vp, i64, vp, i64, i64, f32,
                                     ctypes.POINTER(LaunchCfg), vp]
    L.qk_rmsnorm_fwd.restype = i32
    L.qk_rmsnorm_fwd.argtypes = [vp] * 6 + [i64] * 8 + [f32, vp]
    L.qk_rmsnorm_fwd_cfg.restype = i32
    L.qk_rmsnorm_fwd_cfg.argtypes = [vp] * 6 + [i64] * 8 + [f32, ctypes.POINTER(LaunchCfg), vp]
    L.log1p_f32.argtypes = [vp, vp, i64, vp]
    L.log1p_f32_cfg.restype = i32
    L.log1p_f32_cfg.argtypes = [vp, vp, i64, ctypes.POINTER(Log1pCfg), vp]
    L.add_rmsnorm_test_cvt_range.restype = i32
    L.add_rmsnorm_test_cvt_range.argtypes = [vp, ctypes.c_uint32, i64, vp]
    L.add_rmsnorm_test_copy2.restype = i32
    L.add_rmsnorm_test_copy2.argtypes = [vp, vp, vp, vp, i64, vp]
    L.add_rmsnorm_test_copy_rows.restype = i32
    L.add_rmsnorm_test_copy_rows.argtypes = [vp, vp, vp, vp, i64, i64, i32, vp]
    L.add_rmsnorm_test_stream.restype = i32
    L.add_rmsnorm_test_stream.argtypes = [vp, vp, i64, i32, vp]
    L.add_rmsnorm_strerror.restype = ctypes.c_char_p
    L.add_rmsnorm_strerror.argtypes = [i32]
    L.add_rmsnorm_last_hip_error.restype = ctypes.c_char_p
    L.add_rmsnorm_last_hip_error.argtypes = []
    L.add_rmsnorm_abi_version.restype = i32
    L.add_rmsnorm_abi_version.argtypes = []
    L.add_rmsnorm_build_info.restype = ctypes.c_char_p
    L.add_rmsnorm_build_info.argtypes = []
    got = L.add_rmsnorm_abi_version()
    if got != ABI_VERSION:
        raise ImportError("libaddrmsnorm ABI %d, binding expects %d: rebuild" % (got, ABI_VERSION))
    _lib = L
    return L


def add_rmsnorm_strerror(status: int) -> str:
    return lib().add_rmsnorm_strerror(status).decode()


def add_rmsnorm_last_hip_error() -> str:
    return lib().add_rmsnorm_last_hip_error().decode()


def add_rmsnorm_abi_version() -> int:
    return int(lib().add_rmsnorm_abi_version())


def add_rmsnorm_build_info() -> str:
    return lib().add_rmsnorm_build_info().decode()


def _check(status: int) -> None:
    if status != OK:
        msg = add_rmsnorm_strerror(status)
        if status == EHIP:
            msg += " (" + add_rmsnorm_last_hip_error() + ")"
        raise AddRmsnormError(status, msg)


_DTYPES = None


def _dtypes():
    global _DTYPES
    if _DTYPES is None:
        import torch

        _DTYPES = (torch.bfloat16, torch.int16, torch.uint16)
    return _DTYPES


def _marshal(out, residual_out, x, residual, weight):
    """Check the tensors and return (n_rows, hidden, device index)."""
    import torch

    dts = _dtypes()
    if not isinstance(x, torch.Tensor) or not isinstance(weight, torch.Tensor):
        raise TypeError("expected torch tensors")
    dev = x.get_device()  # -1 for a CPU tensor
    if dev < 0:
        raise ValueError("tensors must live on the GPU")
    shape = x.shape
    for t in (x, out, residual_out, residual):
        if not isinstance(t, torch.Tensor):
            raise TypeError("expected torch tensors")
        if t.shape != shape:
            raise ValueError("out, residual_out and residual must have x's shape %s"
                             % (tuple(shape),))
        if t.get_device() != dev:
            raise ValueError("all tensors must be on one GPU")
        if t.dtype not in dts:
            raise TypeError("tensors must hold bf16 (bfloat16, or raw 16-bit patterns)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if weight.get_device() != dev or weight.dtype not in dts or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous bf16 tensor on x's GPU")
    if weight.dim() != 1 or len(shape) < 1 or shape[-1] != weight.shape[0]:
        raise ValueError("x must be [..., hidden] and weight [hidden]")
    hidden = weight.shape[0]
    return (x.numel() // hidden if hidden else 0), hidden, dev


_RAW_STREAM = None


def _stream_handle(dev, stream):
    """The HIP stream to enqueue on: the given torch stream, else torch's
    current stream for the device."""
    global _RAW_STREAM
    if stream is not None:
        return stream.cuda_stream
    if _RAW_STREAM is None:
        import torch

        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None) or (
            lambda d: torch.cuda.current_stream(d).cuda_stream)
    return _RAW_STREAM(dev)


_CURRENT_DEVICE = None


def _current_device():
    """HIP's current device index.  The caller's tensors already live on a GPU,
    so torch's lazy initialisation has run and its raw query is enough."""
    global _CURRENT_DEVICE
    if _CURRENT_DEVICE is None:
        import torch

        _CURRENT_DEVICE = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device
    return _CURRENT_DEVICE()


def _on_device(dev, fn):
    """Call fn with HIP's current device set to dev (switching only if needed)."""
    if _current_device() == dev:
        return fn()
    import torch

    with torch.cuda.device(dev):
        return fn()


def add_rmsnorm_fwd(out, residual_out, x, residual, weight, eps: float = 1e-6,
                    stream=None) -> None:
    """out, residual_out <- fused add + RMSNorm of x, residual with weight.

    All tensors bf16 on one GPU, contiguous, x/residual/out/residual_out of
    shape [..., hidden] and weight [hidden].  Enqueued on ``stream`` (default:
    torch's current stream for that device); does not synchronise.
    """
    n_rows, hidden, dev = _marshal(out, residual_out, x, residual, weight)
    L = lib()
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.add_rmsnorm_fwd(
        out.data_ptr(), residual_out.data_ptr(), x.data_ptr(), residual.data_ptr(),
        weight.data_ptr(), n_rows, hidden, eps, h)))


def add_rmsnorm_fwd_cfg(out, residual_out, x, residual, weight, eps: float = 1e-6,
                        path: int = PATH_AUTO, block_threads: int = 0, grid_blocks: int = 0,
                        stream=None, rows_per_lane: int = 0, late_weight: bool = False) -> None:
    """add_rmsnorm_fwd with an explicit launch configuration (same results).
    rows_per_lane (the packed path) or late_weight (the register path) go to
    the configuration's flags."""
    n_rows, hidden, dev = _marshal(out, residual_out, x, residual, weight)
    L = lib()
    cfg = LaunchCfg(path, block_threads, grid_blocks,
                    FLAG_LATE_WEIGHT if late_weight else rows_per_lane)
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.add_rmsnorm_fwd_cfg(
        out.data_ptr(), residual_out.data_ptr(), x.data_ptr(), residual.data_ptr(),
        weight.data_ptr(), n_rows, hidden, eps, ctypes.byref(cfg), h)))


def _code_dtypes(fp8: bool):
    import torch

    if not fp8:
        return (torch.int8,)
    return tuple(t for t in (torch.uint8, getattr(torch, "float8_e4m3fn", None)) if t is not None)


def _marshal_quant(out_q, out_scale, residual_out, x, residual, weight, fp8=False):
    import torch

    n_rows, hidden, dev = _marshal(residual_out, residual_out, x, residual, weight)
    if not isinstance(out_q, torch.Tensor) or out_q.dtype not in _code_dtypes(fp8) or \
            out_q.shape != x.shape or not out_q.is_contiguous() or out_q.get_device() != dev:
        raise ValueError("out_q must be a contiguous %s tensor of x's shape on x's GPU"
                         % ("uint8 or float8_e4m3fn" if fp8 else "int8"))
    if not isinstance(out_scale, torch.Tensor) or out_scale.dtype != torch.float32 or \
            out_scale.numel() != n_rows or not out_scale.is_contiguous() or \
            out_scale.get_device() != dev:
        raise ValueError("out_scale must be a contiguous float32 tensor with one value per row")
    return n_rows, hidden, dev


def add_rmsnorm_quant_fwd(out_q, out_scale, residual_out, x, residual, weight,
                          eps: float = 1e-6, stream=None) -> None:
    """out_q (int8 codes), out_scale (fp32 per row), residual_out <- the
    quantised fused add + RMSNorm.  out_q has x's shape, out_scale one value
    per row (x.shape[:-1]); everything else as add_rmsnorm_fwd."""
    n_rows, hidden, dev = _marshal_quant(out_q, out_scale, residual_out, x, residual, weight)
    L = lib()
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.add_rmsnorm_quant_fwd(
        out_q.data_ptr(), out_scale.data_ptr(), residual_out.data_ptr(), x.data_ptr(),
        residual.data_ptr(), weight.data_ptr(), n_rows, hidden, eps, h)))


def add_rmsnorm_quant_fwd_cfg(out_q, out_scale, residual_out, x, residual, weight,
                              eps: float = 1e-6, path: int = PATH_AUTO, block_threads: int = 0,
                              grid_blocks: int = 0, stream=None,
                              rows_per_lane: int = 0) -> None:
    """add_rmsnorm_quant_fwd with an explicit launch configuration."""
    n_rows, hidden, dev = _marshal_quant(out_q, out_scale, residual_out, x, residual, weight)
    L = lib()
    cfg = LaunchCfg(path, block_threads, grid_blocks, rows_per_lane)
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.add_rmsnorm_quant_fwd_cfg(
        out_q.data_ptr(), out_scale.data_ptr(), residual_out.data_ptr(), x.data_ptr(),
        residual.data_ptr(), weight.data_ptr(), n_rows, hidden, eps, ctypes.byref(cfg), h)))


def add_rmsnorm_quant_fp8_fwd(out_q, out_scale, residual_out, x, residual, weight,
                              eps: float = 1e-6, stream=None) -> None:
    """add_rmsnorm_quant_fwd with OCP FP8 E4M3 codes (scale = amax / 448).
    out_q: uint8 or torch.float8_e4m3fn of x's shape."""
    n_rows, hidden, dev = _marshal_quant(out_q, out_scale, residual_out, x, residual, weight, True)
    L = lib()
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.add_rmsnorm_quant_fp8_fwd(
        out_q.data_ptr(), out_scale.data_ptr(), residual_out.data_ptr(), x.data_ptr(),
        residual.data_ptr(), weight.data_ptr(), n_rows, hidden, eps, h)))


def add_rmsnorm_quant_fp8_fwd_cfg(out_q, out_scale, residual_out, x, residual, weight,
                                  eps: float = 1e-6, path: int = PATH_AUTO,
                                  block_threads: int = 0, grid_blocks: int = 0,
                                  stream=None,
                                  rows_per_lane: int = 0) -> None:
    """add_rmsnorm_quant_fp8_fwd with an explicit launch configuration."""
    n_rows, hidden, dev = _marshal_quant(out_q, out_scale, residual_out, x, residual, weight, True)
    L = lib()
    cfg = LaunchCfg(path, block_threads, grid_blocks, rows_per_lane)
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.add_rmsnorm_quant_fp8_fwd_cfg(
        out_q.data_ptr(), out_scale.data_ptr(), residual_out.data_ptr(), x.data_ptr(),
        residual.data_ptr(), weight.data_ptr(), n_rows, hidden, eps, ctypes.byref(cfg), h)))


def _row_view(t, hidden, dev, name):
    """(pointer, row stride in elements) of a 2-D row-strided bf16 view."""
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.get_device() != dev:
        raise ValueError("%s must be a GPU tensor on the weight's device" % name)
    if t.dtype not in _dtypes():
        raise TypeError("%s must hold bf16 (bfloat16, or raw 16-bit patterns)" % name)
    if t.dim() != 2 or t.shape[1] != hidden or (t.shape[0] > 1 and t.stride(1) != 1):
        raise ValueError("%s must be [n_rows, hidden] with unit column stride" % name)
    return t.data_ptr(), (t.stride(0) if t.shape[0] > 1 else hidden)


def add_rmsnorm_fwd_strided(out, residual_out, x, residual, weight, eps: float = 1e-6,
                            path: int = PATH_AUTO, block_threads: int = 0, grid_blocks: int = 0,
                            stream=None, rows_per_lane: int = 0) -> None:
    """The fused forward on 2-D views whose rows may be strided (e.g. column
    slices of wider matrices): each tensor [n_rows, hidden] with unit column
    stride; weight [hidden] contiguous."""
    if weight.dim() != 1 or not weight.is_cuda or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous 1-D GPU tensor")
    hidden, dev = weight.shape[0], weight.get_device()
    po, so = _row_view(out, hidden, dev, "out")
    pro, sro = _row_view(residual_out, hidden, dev, "residual_out")
    px, sx = _row_view(x, hidden, dev, "x")
    pr, sr = _row_view(residual, hidden, dev, "residual")
    n_rows = x.shape[0]
    if not (out.shape[0] == residual_out.shape[0] == residual.shape[0] == n_rows):
        raise ValueError("all views need the same number of rows")
    L = lib()
    cfg = LaunchCfg(path, block_threads, grid_blocks, rows_per_lane)
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.add_rmsnorm_fwd_strided(
        po, so, pro, sro, px, sx, pr, sr, weight.data_ptr(), n_rows, hidden, eps,
        ctypes.byref(cfg), h)))


def rmsnorm_fwd_strided(out, x, weight, eps: float = 1e-6, path: int = PATH_AUTO,
                        block_threads: int = 0, grid_blocks: int = 0, stream=None,
                        rows_per_lane: int = 0) -> None:
    """Plain RMSNorm on 2-D views whose rows may be strided."""
    if weight.dim() != 1 or not weight.is_cuda or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous 1-D GPU tensor")
    hidden, dev = weight.shape[0], weight.get_device()
    po, so = _row_view(out, hidden, dev, "out")
    px, sx = _row_view(x, hidden, dev, "x")
    if out.shape[0] != x.shape[0]:
        raise ValueError("out and x need the same number of rows")
    L = lib()
    cfg = LaunchCfg(path, block_threads, grid_blocks, rows_per_lane)
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.rmsnorm_fwd_strided(
        po, so, px, sx, weight.data_ptr(), x.shape[0], hidden, eps, ctypes.byref(cfg), h)))


def rmsnorm_fwd(out, x, weight, eps: float = 1e-6, stream=None) -> None:
    """out <- RMSNorm of x with weight (no residual add); out may be x.
    Tensors and stream as add_rmsnorm_fwd."""
    n_rows, hidden, dev = _marshal(out, out, x, x, weight)
    L = lib()
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.rmsnorm_fwd(
        out.data_ptr(), x.data_ptr(), weight.data_ptr(), n_rows, hidden, eps, h)))


def rmsnorm_fwd_cfg(out, x, weight, eps: float = 1e-6, path: int = PATH_AUTO,
                    block_threads: int = 0, grid_blocks: int = 0, stream=None,
                    rows_per_lane: int = 0, late_weight: bool = False) -> None:
    """rmsnorm_fwd with an explicit launch configuration (same results)."""
    n_rows, hidden, dev = _marshal(out, out, x, x, weight)
    L = lib()
    cfg = LaunchCfg(path, block_threads, grid_blocks,
                    FLAG_LATE_WEIGHT if late_weight else rows_per_lane)
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.rmsnorm_fwd_cfg(
        out.data_ptr(), x.data_ptr(), weight.data_ptr(), n_rows, hidden, eps,
        ctypes.byref(cfg), h)))


def rmsnorm_quant_fwd(out_q, out_scale, x, weight, eps: float = 1e-6, stream=None) -> None:
    """out_q (int8 codes), out_scale (fp32 per row) <- quantised RMSNorm of x
    (no residual add).  Shapes as add_rmsnorm_quant_fwd."""
    n_rows, hidden, dev = _marshal_quant(out_q, out_scale, x, x, x, weight)
    L = lib()
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.rmsnorm_quant_fwd(
        out_q.data_ptr(), out_scale.data_ptr(), x.data_ptr(), weight.data_ptr(), n_rows, hidden,
        eps, h)))


def rmsnorm_quant_fwd_cfg(out_q, out_scale, x, weight, eps: float = 1e-6, path: int = PATH_AUTO,
                          block_threads: int = 0, grid_blocks: int = 0, stream=None,
                          rows_per_lane: int = 0) -> None:
    """rmsnorm_quant_fwd with an explicit launch configuration."""
    n_rows, hidden, dev = _marshal_quant(out_q, out_scale, x, x, x, weight)
    L = lib()
    cfg = LaunchCfg(path, block_threads, grid_blocks, rows_per_lane)
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.rmsnorm_quant_fwd_cfg(
        out_q.data_ptr(), out_scale.data_ptr(), x.data_ptr(), weight.data_ptr(), n_rows, hidden,
        eps, ctypes.byref(cfg), h)))


def rmsnorm_quant_fp8_fwd(out_q, out_scale, x, weight, eps: float = 1e-6, stream=None) -> None:
    """rmsnorm_quant_fwd with OCP FP8 E4M3 codes (out_q uint8 or float8_e4m3fn)."""
    n_rows, hidden, dev = _marshal_quant(out_q, out_scale, x, x, x, weight, True)
    L = lib()
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.rmsnorm_quant_fp8_fwd(
        out_q.data_ptr(), out_scale.data_ptr(), x.data_ptr(), weight.data_ptr(), n_rows, hidden,
        eps, h)))


def rmsnorm_quant_fp8_fwd_cfg(out_q, out_scale, x, weight, eps: float = 1e-6,
                              path: int = PATH_AUTO, block_threads: int = 0,
                              grid_blocks: int = 0, stream=None,
                              rows_per_lane: int = 0) -> None:
    """rmsnorm_quant_fp8_fwd with an explicit launch configuration."""
    n_rows, hidden, dev = _marshal_quant(out_q, out_scale, x, x, x, weight, True)
    L = lib()
    cfg = LaunchCfg(path, block_threads, grid_blocks, rows_per_lane)
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.rmsnorm_quant_fp8_fwd_cfg(
        out_q.data_ptr(), out_scale.data_ptr(), x.data_ptr(), weight.data_ptr(), n_rows, hidden,
        eps, ctypes.byref(cfg), h)))


def _code_view(q, sc, n_rows, hidden, dev, fp8):
    """Check contiguous codes [n_rows, hidden] and scales [n_rows]."""
    import torch

    cd = torch.uint8 if fp8 else torch.int8
    if not isinstance(q, torch.Tensor) or q.dtype != cd or tuple(q.shape) != (n_rows, hidden) \
            or not q.is_contiguous() or q.get_device() != dev:
        raise ValueError("out_q must be a contiguous [n_rows, hidden] %s GPU tensor" % cd)
    if not isinstance(sc, torch.Tensor) or sc.dtype != torch.float32 or \
            tuple(sc.shape) != (n_rows,) or not sc.is_contiguous() or sc.get_device() != dev:
        raise ValueError("out_scale must be a contiguous [n_rows] float32 GPU tensor")


def add_rmsnorm_quant_fwd_strided(out_q, out_scale, residual_out, x, residual, weight,
                                  eps: float = 1e-6, fp8: bool = False, path: int = PATH_AUTO,
                                  block_threads: int = 0, grid_blocks: int = 0,
                                  rows_per_lane: int = 0, stream=None) -> None:
    """Quantised fused forward (int8, or E4M3 with fp8=True) on 2-D views of
    x, residual and residual_out whose rows may be strided; codes [n_rows,
    hidden] and scales [n_rows] contiguous."""
    if weight.dim() != 1 or not weight.is_cuda or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous 1-D GPU tensor")
    hidden, dev = weight.shape[0], weight.get_device()
    pro, sro = _row_view(residual_out, hidden, dev, "residual_out")
    px, sx = _row_view(x, hidden, dev, "x")
    pr, sr = _row_view(residual, hidden, dev, "residual")
    n_rows = x.shape[0]
    if not (residual_out.shape[0] == residual.shape[0] == n_rows):
        raise ValueError("all views need the same number of rows")
    _code_view(out_q, out_scale, n_rows, hidden, dev, fp8)
    L = lib()
    fn = L.add_rmsnorm_quant_fp8_fwd_strided if fp8 else L.add_rmsnorm_quant_fwd_strided
    cfg = LaunchCfg(path, block_threads, grid_blocks, rows_per_lane)
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: fn(out_q.data_ptr(), out_scale.data_ptr(), pro, sro, px, sx,
                                      pr, sr, weight.data_ptr(), n_rows, hidden, eps,
                                      ctypes.byref(cfg), h)))


def rmsnorm_quant_fwd_strided(out_q, out_scale, x, weight, eps: float = 1e-6, fp8: bool = False,
                              path: int = PATH_AUTO, block_threads: int = 0,
                              grid_blocks: int = 0, rows_per_lane: int = 0,
                              stream=None) -> None:
    """Quantised plain RMSNorm on a 2-D view of x whose rows may be strided."""
    if weight.dim() != 1 or not weight.is_cuda or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous 1-D GPU tensor")
    hidden, dev = weight.shape[0], weight.get_device()
    px, sx = _row_view(x, hidden, dev, "x")
    n_rows = x.shape[0]
    _code_view(out_q, out_scale, n_rows, hidden, dev, fp8)
    L = lib()
    fn = L.rmsnorm_quant_fp8_fwd_strided if fp8 else L.rmsnorm_quant_fwd_strided
    cfg = LaunchCfg(path, block_threads, grid_blocks, rows_per_lane)
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: fn(out_q.data_ptr(), out_scale.data_ptr(), px, sx,
                                      weight.data_ptr(), n_rows, hidden, eps, ctypes.byref(cfg),
                                      h)))


def _head_view(t, dev, name, head_dim, tensor_type, dts):
    """(pointer, tokens, heads, token stride in elements) of a [tokens, heads,
    head_dim] bf16 view with heads contiguous within a token, or
    (0, 0, 0, 0) for None."""
    if t is None:
        return 0, 0, 0, 0
    if not isinstance(t, tensor_type) or t.get_device() != dev:
        raise ValueError("%s must be a GPU tensor on the weights' device" % name)
    if t.dtype not in dts:
        raise TypeError("%s must hold bf16 (bfloat16, or raw 16-bit patterns)" % name)
    sh = t.shape
    if len(sh) != 3 or sh[2] != head_dim:
        raise ValueError("%s must be [tokens, heads, head_dim]" % name)
    tokens, heads = sh[0], sh[1]
    st = t.stride()
    if heads > 0 and (st[2] != 1 or (heads > 1 and st[1] != head_dim)):
        raise ValueError("%s: heads must be contiguous within a token" % name)
    stride = st[0] if tokens > 1 else heads * head_dim
    return t.data_ptr(), tokens, heads, stride


def _qk_call(q_out, k_out, q, k, q_weight, k_weight, eps, cfg, stream):
    import torch

    T, dts = torch.Tensor, _dtypes()
    for w, name in ((q_weight, "q_weight"), (k_weight, "k_weight")):
        if not isinstance(w, T) or w.get_device() < 0 or len(w.shape) != 1 or \
                not w.is_contiguous() or w.dtype not in dts:
            raise ValueError("%s must be a contiguous 1-D bf16 GPU tensor" % name)
    d, dev = q_weight.shape[0], q_weight.get_device()
    if k_weight.shape[0] != d or k_weight.get_device() != dev:
        raise ValueError("q_weight and k_weight must have one length and device")
    pq, tq, hq, sq = _head_view(q, dev, "q", d, T, dts)
    pk, tk, hk, sk = _head_view(k, dev, "k", d, T, dts)
    pqo, tqo, hqo, sqo = _head_view(q_out, dev, "q_out", d, T, dts)
    pko, tko, hko, sko = _head_view(k_out, dev, "k_out", d, T, dts)
    if hqo != hq or hko != hk:
        raise ValueError("q_out and k_out must have the heads of q and k")
    tokens = set()
    if hq > 0:
        tokens.update((tq, tqo))
    if hk > 0:
        tokens.update((tk, tko))
    if len(tokens) > 1:
        raise ValueError("q, k and the outputs need the same number of tokens")
    n_tokens = tokens.pop() if tokens else 0
    L = lib()
    h = _stream_handle(dev, stream)
    args = (pqo or None, pko or None, pq or None, pk or None, q_weight.data_ptr(),
            k_weight.data_ptr(), n_tokens, hq, hk, d, sq, sk, sqo, sko, eps)
    if cfg is None:
        _check(_on_device(dev, lambda: L.qk_rmsnorm_fwd(*args, h)))
    else:
        _check(_on_device(dev, lambda: L.qk_rmsnorm_fwd_cfg(*args, ctypes.byref(cfg), h)))


def qk_rmsnorm_fwd(q_out, k_out, q, k, q_weight, k_weight, eps: float = 1e-6,
                   stream=None) -> None:
    """Per-head RMSNorm of q [tokens, q_heads, head_dim] with q_weight
    [head_dim] and of k [tokens, k_heads, head_dim] with k_weight, into q_out
    and k_out (same shapes; may be q and k themselves).  Views may have any
    token stride (e.g. column slices of a fused qkv tensor, reshaped); heads
    are contiguous within a token.  k and k_out may be None (q only)."""
    _qk_call(q_out, k_out, q, k, q_weight, k_weight, eps, None, stream)


def qk_rmsnorm_fwd_cfg(q_out, k_out, q, k, q_weight, k_weight, eps: float = 1e-6,
                       path: int = PATH_AUTO, block_threads: int = 0, grid_blocks: int = 0,
                       rows_per_lane: int = 0, stream=None) -> None:
    """qk_rmsnorm_fwd with an explicit launch configuration (same results)."""
    cfg = LaunchCfg(path, block_threads, grid_blocks, rows_per_lane)
    _qk_call(q_out, k_out, q, k, q_weight, k_weight, eps, cfg, stream)


def _marshal_log1p(out, x):
    import torch

    for t in (out, x):
        if not isinstance(t, torch.Tensor):
            raise TypeError("expected torch tensors")
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("out and x must be contiguous float32 GPU tensors")
    if out.shape != x.shape or out.get_device() != x.get_device():
        raise ValueError("out must have x's shape and GPU")
    return x.numel(), x.get_device()


def log1p_f32(out, x, stream=None) -> None:
    """out <- log1p(x), correctly rounded binary32 (out may be x)."""
    n, dev = _marshal_log1p(out, x)
    L = lib()
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.log1p_f32(out.data_ptr(), x.data_ptr(), n, h)))


def log1p_f32_cfg(out, x, block_threads: int = 0, elems_per_thread: int = 0,
                  grid_blocks: int = 0, flags: int = 0, stream=None) -> None:
    """log1p_f32 with an explicit launch configuration (same results)."""
    n, dev = _marshal_log1p(out, x)
    L = lib()
    cfg = Log1pCfg(block_threads, elems_per_thread, grid_blocks, flags)
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.log1p_f32_cfg(out.data_ptr(), x.data_ptr(), n,
                                                   ctypes.byref(cfg), h)))


def add_rmsnorm_test_cvt_range(out, start: int, stream=None) -> None:
    """out[i] <- bf16 (nearest-even, by the kernels' store routine) of the fp32
    bit pattern (start + i) mod 2^32.  out: contiguous 16-bit GPU tensor."""
    if not out.is_cuda or out.element_size() != 2 or not out.is_contiguous():
        raise ValueError("out must be a contiguous 16-bit GPU tensor")
    dev = out.get_device()
    L = lib()
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.add_rmsnorm_test_cvt_range(
        out.data_ptr(), start & 0xFFFFFFFF, out.numel(), h)))


def add_rmsnorm_test_cvt_e4m3_range(out, start: int, stream=None) -> None:
    """out[i] <- E4M3 code (by the fp8 variant's code routine, inv = 1) of the
    fp32 bit pattern (start + i) mod 2^32.  out: contiguous 8-bit GPU tensor."""
    if not out.is_cuda or out.element_size() != 1 or not out.is_contiguous():
        raise ValueError("out must be a contiguous 8-bit GPU tensor")
    dev = out.get_device()
    L = lib()
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.add_rmsnorm_test_cvt_e4m3_range(
        out.data_ptr(), start & 0xFFFFFFFF, out.numel(), h)))


def add_rmsnorm_test_copy2(dst0, dst1, src0, src1, stream=None) -> None:
    """dst0 <- src0, dst1 <- src1 with the fused kernels' streaming access
    pattern and no arithmetic (a reference rate).  Contiguous 16-bit GPU
    tensors of equal size."""
    ts = (dst0, dst1, src0, src1)
    n = src0.numel()
    for t in ts:
        if not t.is_cuda or t.element_size() != 2 or not t.is_contiguous() or t.numel() != n:
            raise ValueError("copy2 takes four contiguous 16-bit GPU tensors of equal size")
    dev = src0.get_device()
    L = lib()
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.add_rmsnorm_test_copy2(
        dst0.data_ptr(), dst1.data_ptr(), src0.data_ptr(), src1.data_ptr(), n, h)))


def add_rmsnorm_test_copy_rows(dst0, dst1, src0, src1, rows_per_burst: int = 1,
                               stream=None) -> None:
    """dst0 <- src0, dst1 <- src1 with the register kernel's row structure,
    rows_per_burst rows loaded per workgroup before any store (a reference
    rate).  Contiguous 16-bit GPU tensors of one shape [..., hidden]."""
    ts = (dst0, dst1, src0, src1)
    for t in ts:
        if not t.is_cuda or t.element_size() != 2 or not t.is_contiguous() or \
                t.shape != src0.shape or t.dim() < 1:
            raise ValueError("copy_rows takes four contiguous 16-bit GPU tensors of one shape")
    hidden = src0.shape[-1]
    n_rows = src0.numel() // hidden if hidden else 0
    dev = src0.get_device()
    L = lib()
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.add_rmsnorm_test_copy_rows(
        dst0.data_ptr(), dst1.data_ptr(), src0.data_ptr(), src1.data_ptr(), n_rows, hidden,
        rows_per_burst, h)))


def add_rmsnorm_test_stream(dst, src, mode: int, stream=None) -> None:
    """Measurement hook: mode 0 reads src (dst, of src's size, receives almost
    nothing), mode 1 writes dst.  Contiguous 16-bit GPU tensors."""
    for t in (dst,) + ((src,) if mode == 0 else ()):
        if not t.is_cuda or t.element_size() != 2 or not t.is_contiguous():
            raise ValueError("tensors must be contiguous 16-bit GPU tensors")
    dev = dst.get_device()
    L = lib()
    h = _stream_handle(dev, stream)
    _check(_on_device(dev, lambda: L.add_rmsnorm_test_stream(
        dst.data_ptr(), src.data_ptr() if mode == 0 else None, dst.numel(), mode, h)))
