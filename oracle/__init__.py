"""CPU oracle for the fused residual-add + RMSNorm forward (bf16 storage).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
imports, links or calls it, and it imports nothing from the GPU library.

The arithmetic lives in ``add_rmsnorm_oracle.c`` (plain C, single thread,
binary64 after the fp32 add, bit-level round-to-nearest-even); this module
builds and loads it with ctypes and adds the measurement helpers of the same
page (ROCm/aiter issue "rmsnorm2d_fwd_with_add truncates fp32->bf16 on gfx942,
biasing residual_out and compounding across layers", "Steps to Reproduce"):
the magnitude-bias metric, the residual-stream RMS and the cosine similarity
it prints, plus the binary64 chain that never rounds.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "add_rmsnorm_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")
LOG1P_SOURCE = os.path.join(HERE, "log1p_oracle.c")
LOG1P_LIBRARY = os.path.join(HERE, "liblog1p_oracle.so")

RNE = 0
TRUNC = 1

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fno-tree-vectorize"]


def build(force: bool = True) -> str:
    """Compile the C oracles with gcc into shared libraries next to their sources."""
    if force or not os.path.exists(LIBRARY) or (
            os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
        compile_library(SOURCE, LIBRARY)
    if force or not os.path.exists(LOG1P_LIBRARY) or (
            os.path.getmtime(LOG1P_LIBRARY) < os.path.getmtime(LOG1P_SOURCE)):
        compile_log1p_library(LOG1P_SOURCE, LOG1P_LIBRARY)
    return LIBRARY


def compile_library(source: str, target: str) -> str:
    """Compile an oracle source file into a shared library at ``target``."""
    tmp = target + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, source, "-lm"], check=True)
    os.replace(tmp, target)
    return target


def compile_log1p_library(source: str, target: str) -> str:
    """Compile the log1p oracle (binary128 through libquadmath)."""
    tmp = target + ".tmp%d" % os.getpid()
    flags = [f if f != "-std=c11" else "-std=gnu11" for f in CFLAGS]
    subprocess.run(["gcc", *flags, "-o", tmp, source, "-lquadmath", "-lm"], check=True)
    os.replace(tmp, target)
    return target


class Oracle:
    """ctypes front end of one build of the C oracle."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        L.orc_rne16.restype = ctypes.c_uint16
        L.orc_rne16.argtypes = [ctypes.c_uint32]
        L.orc_trunc16.restype = ctypes.c_uint16
        L.orc_trunc16.argtypes = [ctypes.c_uint32]
        L.orc_rne16_from_f64.restype = ctypes.c_uint16
        L.orc_rne16_from_f64.argtypes = [ctypes.c_double]
        L.orc_rne16_array.restype = None
        L.orc_rne16_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        L.orc_rne16_range.restype = None
        L.orc_rne16_range.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p]
        L.orc_rne16_from_f64_array.restype = None
        L.orc_rne16_from_f64_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_int64]
        L.orc_add_rmsnorm.restype = ctypes.c_int
        L.orc_add_rmsnorm.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                      ctypes.c_int]
        L.orc_add_rmsnorm_quant.restype = ctypes.c_int
        L.orc_add_rmsnorm_quant.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_float]
        L.orc_e4m3_rne.restype = ctypes.c_int
        L.orc_e4m3_rne.argtypes = [ctypes.c_float]
        L.orc_add_rmsnorm_quant_fp8.restype = ctypes.c_int
        L.orc_add_rmsnorm_quant_fp8.argtypes = [ctypes.c_void_p] * 7 + [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_float]
        L.orc_qk_rmsnorm.restype = ctypes.c_int
        L.orc_qk_rmsnorm.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 6 + [
            ctypes.c_float]
        self.path = path
        self.lib = L

    # ------------------------------------------------------------ converters

    def rne16(self, u32: int) -> int:
        """fp32 bit pattern -> bf16 bit pattern, nearest-even (NaN -> quiet NaN)."""
        return int(self.lib.orc_rne16(int(u32) & 0xFFFFFFFF))

    def trunc16(self, u32: int) -> int:
        """fp32 bit pattern -> bf16 bit pattern by truncation (negative control)."""
        return int(self.lib.orc_trunc16(int(u32) & 0xFFFFFFFF))

    def rne16_from_f64(self, y: float) -> int:
        """binary64 -> bf16 bit pattern, correctly rounded, nearest-even."""
        return int(self.lib.orc_rne16_from_f64(float(y)))

    def rne16_array(self, u32: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(u32, dtype=np.uint32)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.orc_rne16_array(_ptr(a), _ptr(out), a.size)
        return out

    def rne16_range(self, start: int, count: int) -> np.ndarray:
        """bf16 results for the fp32 bit patterns start .. start+count-1."""
        out = np.empty(count, dtype=np.uint16)
        self.lib.orc_rne16_range(start, count, _ptr(out))
        return out

    def rne16_from_f64_array(self, y: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(y, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.orc_rne16_from_f64_array(_ptr(a), _ptr(out), a.size)
        return out

    # ------------------------------------------------------------ the fused op

    def add_rmsnorm(self, x: np.ndarray, residual: np.ndarray, weight: np.ndarray,
                    eps: float = 1e-6, rounding: int = RNE, want_exact: bool = False):
        """Oracle forward.  x, residual: uint16 [n, hidden] bf16 bits; weight [hidden].

        Returns (out, residual_out) as uint16 arrays, plus the unrounded
        binary64 out values when ``want_exact`` is set.
        """
        x = np.ascontiguousarray(x, dtype=np.uint16)
        residual = np.ascontiguousarray(residual, dtype=np.uint16)
        weight = np.ascontiguousarray(weight, dtype=np.uint16)
        if x.ndim != 2 or residual.shape != x.shape or weight.shape != (x.shape[1],):
            raise ValueError("shape mismatch: x %s residual %s weight %s"
                             % (x.shape, residual.shape, weight.shape))
        n, h = x.shape
        out = np.empty_like(x)
        res_out = np.empty_like(x)
        y = np.empty(x.shape, dtype=np.float64) if want_exact else None
        rc = self.lib.orc_add_rmsnorm(_ptr(out), _ptr(res_out),
                                      _ptr(y) if y is not None else None,
                                      _ptr(x), _ptr(residual), _ptr(weight), n, h,
                                      ctypes.c_float(eps), rounding)
        if rc != 0:
            raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
        if want_exact:
            return out, res_out, y
        return out, res_out


    def add_rmsnorm_quant(self, x: np.ndarray, residual: np.ndarray, weight: np.ndarray,
                          eps: float = 1e-6, want_exact: bool = False):
        """Quantised variant: (codes int8 [n, hidden], scale fp32 [n],
        residual_out uint16 [n, hidden]) plus the binary64 y when asked."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        residual = np.ascontiguousarray(residual, dtype=np.uint16)
        weight = np.ascontiguousarray(weight, dtype=np.uint16)
        if x.ndim != 2 or residual.shape != x.shape or weight.shape != (x.shape[1],):
            raise ValueError("shape mismatch")
        n, h = x.shape
        q = np.empty(x.shape, dtype=np.int8)
        sc = np.empty(n, dtype=np.float32)
        res_out = np.empty_like(x)
        y = np.empty(x.shape, dtype=np.float64) if want_exact else None
        rc = self.lib.orc_add_rmsnorm_quant(_ptr(q), _ptr(sc), _ptr(res_out),
                                            _ptr(y) if y is not None else None, _ptr(x),
                                            _ptr(residual), _ptr(weight), n, h,
                                            ctypes.c_float(eps))
        if rc != 0:
            raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
        if want_exact:
            return q, sc, res_out, y
        return q, sc, res_out


    # ------------------------------------------------------------ plain RMSNorm

    def rmsnorm(self, x: np.ndarray, weight: np.ndarray, eps: float = 1e-6,
                rounding: int = RNE, want_exact: bool = False):
        """Plain RMSNorm (no residual): acc = fp32(x), the rest as add_rmsnorm.

        Returns out (uint16 [n, hidden]), plus the binary64 out values when
        ``want_exact`` is set.
        """
        x = np.ascontiguousarray(x, dtype=np.uint16)
        weight = np.ascontiguousarray(weight, dtype=np.uint16)
        if x.ndim != 2 or weight.shape != (x.shape[1],):
            raise ValueError("shape mismatch: x %s weight %s" % (x.shape, weight.shape))
        n, h = x.shape
        out = np.empty_like(x)
        y = np.empty(x.shape, dtype=np.float64) if want_exact else None
        rc = self.lib.orc_add_rmsnorm(_ptr(out), None, _ptr(y) if y is not None else None,
                                      _ptr(x), None, _ptr(weight), n, h, ctypes.c_float(eps),
                                      rounding)
        if rc != 0:
            raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
        return (out, y) if want_exact else out

    def rmsnorm_quant(self, x: np.ndarray, weight: np.ndarray, eps: float = 1e-6,
                      want_exact: bool = False):
        """Plain RMSNorm with int8 out: (codes, scale), plus the binary64 y
        when asked."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        weight = np.ascontiguousarray(weight, dtype=np.uint16)
        if x.ndim != 2 or weight.shape != (x.shape[1],):
            raise ValueError("shape mismatch")
        n, h = x.shape
        q = np.empty(x.shape, dtype=np.int8)
        sc = np.empty(n, dtype=np.float32)
        y = np.empty(x.shape, dtype=np.float64) if want_exact else None
        rc = self.lib.orc_add_rmsnorm_quant(_ptr(q), _ptr(sc), None,
                                            _ptr(y) if y is not None else None, _ptr(x), None,
                                            _ptr(weight), n, h, ctypes.c_float(eps))
        if rc != 0:
            raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
        return (q, sc, y) if want_exact else (q, sc)


    # ------------------------------------------------------------ per-head q/k norm

    @staticmethod
    def _head_view(t, name):
        """(array, token stride in elements) of a [tokens, heads, head_dim] uint16
        view whose heads are contiguous within a token."""
        t = np.asarray(t)
        if t.dtype != np.uint16 or t.ndim != 3:
            raise ValueError("%s must be a [tokens, heads, head_dim] uint16 array" % name)
        d = t.shape[2]
        if t.shape[0] > 1 and t.strides[0] % 2:
            raise ValueError("%s: odd token stride" % name)
        if t.strides[2] != 2 or (t.shape[1] > 1 and t.strides[1] != 2 * d):
            raise ValueError("%s: heads must be contiguous within a token" % name)
        stride = t.strides[0] // 2 if t.shape[0] > 1 else t.shape[1] * d
        return t, stride

    def qk_rmsnorm(self, q, k, q_weight, k_weight, eps: float = 1e-6):
        """Per-head RMSNorm of q [T, Hq, D] with q_weight [D] and of k
        [T, Hk, D] with k_weight [D] (views with any token stride and heads
        contiguous within a token).  Returns (q_out, k_out), contiguous."""
        q, qs = self._head_view(q, "q")
        k, ks = self._head_view(k, "k")
        t_n, hq, d = q.shape
        if k.shape[0] != t_n or k.shape[2] != d:
            raise ValueError("q and k need the same tokens and head_dim")
        hk = k.shape[1]
        qw = np.ascontiguousarray(q_weight, dtype=np.uint16)
        kw = np.ascontiguousarray(k_weight, dtype=np.uint16)
        if qw.shape != (d,) or kw.shape != (d,):
            raise ValueError("q_weight and k_weight must be [head_dim]")
        q_out = np.empty((t_n, hq, d), np.uint16)
        k_out = np.empty((t_n, hk, d), np.uint16)
        rc = self.lib.orc_qk_rmsnorm(
            _ptr(q_out) if q_out.size else None, _ptr(k_out) if k_out.size else None,
            q.ctypes.data if q.size else None, k.ctypes.data if k.size else None,
            _ptr(qw), _ptr(kw), t_n, hq, hk, d, qs, ks, ctypes.c_float(eps))
        if rc != 0:
            raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
        return q_out, k_out

    # ------------------------------------------------------------ fp8 e4m3 out

    def e4m3_rne(self, v: float) -> int:
        """e4m3fn code (0..255) of a finite binary32 value, nearest-even,
        saturating at +-448."""
        return int(self.lib.orc_e4m3_rne(float(np.float32(v))))

    def add_rmsnorm_quant_fp8(self, x, residual, weight, eps: float = 1e-6,
                              want_exact: bool = False):
        """FP8 E4M3 variant: (codes uint8 [n, hidden], scale fp32 [n],
        residual_out uint16 [n, hidden] or None) plus the binary64 y when
        asked.  residual None is plain RMSNorm."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        weight = np.ascontiguousarray(weight, dtype=np.uint16)
        if residual is not None:
            residual = np.ascontiguousarray(residual, dtype=np.uint16)
            if residual.shape != x.shape:
                raise ValueError("shape mismatch")
        if x.ndim != 2 or weight.shape != (x.shape[1],):
            raise ValueError("shape mismatch")
        n, h = x.shape
        q = np.empty(x.shape, dtype=np.uint8)
        sc = np.empty(n, dtype=np.float32)
        res_out = np.empty_like(x) if residual is not None else None
        y = np.empty(x.shape, dtype=np.float64) if want_exact else None
        rc = self.lib.orc_add_rmsnorm_quant_fp8(
            _ptr(q), _ptr(sc), _ptr(res_out) if res_out is not None else None,
            _ptr(y) if y is not None else None, _ptr(x),
            _ptr(residual) if residual is not None else None, _ptr(weight), n, h,
            ctypes.c_float(eps))
        if rc != 0:
            raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
        return (q, sc, res_out, y) if want_exact else (q, sc, res_out)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


_default = None


def default() -> Oracle:
    """The oracle built from this package's source (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or (
                os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
            build(force=True)
        _default = Oracle(LIBRARY)
    return _default


def rne16(u32: int) -> int:
    return default().rne16(u32)


def trunc16(u32: int) -> int:
    return default().trunc16(u32)


def rne16_from_f64(y: float) -> int:
    return default().rne16_from_f64(y)


def rne16_array(u32: np.ndarray) -> np.ndarray:
    return default().rne16_array(u32)


def rne16_range(start: int, count: int) -> np.ndarray:
    return default().rne16_range(start, count)


def rne16_from_f64_array(y: np.ndarray) -> np.ndarray:
    return default().rne16_from_f64_array(y)


def add_rmsnorm(x, residual, weight, eps: float = 1e-6, rounding: int = RNE,
                want_exact: bool = False):
    return default().add_rmsnorm(x, residual, weight, eps, rounding, want_exact)


def add_rmsnorm_quant(x, residual, weight, eps: float = 1e-6, want_exact: bool = False):
    return default().add_rmsnorm_quant(x, residual, weight, eps, want_exact)


def add_rmsnorm_quant_fp8(x, residual, weight, eps: float = 1e-6, want_exact: bool = False):
    return default().add_rmsnorm_quant_fp8(x, residual, weight, eps, want_exact)


def e4m3_rne(v: float) -> int:
    return default().e4m3_rne(v)


def e4m3_to_f64(codes) -> np.ndarray:
    """Exact values of e4m3fn codes (NaN for the NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def rmsnorm(x, weight, eps: float = 1e-6, rounding: int = RNE, want_exact: bool = False):
    return default().rmsnorm(x, weight, eps, rounding, want_exact)


def rmsnorm_quant(x, weight, eps: float = 1e-6, want_exact: bool = False):
    return default().rmsnorm_quant(x, weight, eps, want_exact)


def qk_rmsnorm(q, k, q_weight, k_weight, eps: float = 1e-6):
    return default().qk_rmsnorm(q, k, q_weight, k_weight, eps)


# ---------------------------------------------------------------- measurements

def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to binary64."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def magnitude_bias(got: np.ndarray, exp: np.ndarray) -> float:
    """Signed relative error of magnitudes, averaged per element.

    The aiter issue ("Steps to Reproduce") measures the bias of a rounding
    mode as a mean signed magnitude error relative to the exact values.
    Written from that definition: over the elements whose exact value e is
    not zero (a relative error is undefined at zero), the arithmetic mean of
    (|g| - |e|) / |e|.  Negative means the results shrank toward zero.
    Both arguments are real-valued arrays of one size (widen bf16 first);
    at least one exact value must be nonzero.
    """
    g = np.abs(np.asarray(got, dtype=np.float64).ravel())
    e = np.abs(np.asarray(exp, dtype=np.float64).ravel())
    if g.shape != e.shape:
        raise ValueError("got and exp differ in size")
    keep = e > 0
    if not keep.any():
        raise ValueError("no nonzero exact value: the relative error is undefined")
    return float(np.sum((g[keep] - e[keep]) / e[keep]) / np.count_nonzero(keep))


def ratio_bias(got: np.ndarray, exp: np.ndarray) -> float:
    """Ratio-of-sums form of the signed magnitude error: sum(|g|-|e|) / sum(|e|).

    Used for long chains, where the per-element relative error is dominated by
    elements that drift close to zero.
    """
    g = np.abs(np.asarray(got, dtype=np.float64).ravel())
    e = np.abs(np.asarray(exp, dtype=np.float64).ravel())
    return float((g - e).sum() / e.sum())


def rms(a: np.ndarray) -> float:
    """Root mean square over all elements (the page's residual-stream size)."""
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a)))


def cosine_similarity(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b / (np.sqrt(a @ a) * np.sqrt(b @ b)))


def chain_fp64_step(residual64: np.ndarray, x_bf16: np.ndarray) -> np.ndarray:
    """One step of the never-rounded residual stream: R + x in binary64."""
    return residual64 + bf16_to_f64(x_bf16)


# ---------------------------------------------------------------- log1p

class Log1pOracle:
    """ctypes front end of one build of the log1p oracle (log1p_oracle.c):
    ln(1 + x) of binary32 inputs, correctly rounded to binary32."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.orc_log1p_f32.restype = ctypes.c_int
        L.orc_log1p_f32.argtypes = [vp, vp, i64]
        L.orc_log1p_f64.restype = ctypes.c_int
        L.orc_log1p_f64.argtypes = [vp, vp, i64]
        L.orc_log1p_f32_fast.restype = ctypes.c_int
        L.orc_log1p_f32_fast.argtypes = [vp, vp, i64, vp]
        self.path = path
        self.lib = L

    @staticmethod
    def _in(x):
        return np.ascontiguousarray(x, dtype=np.float32)

    def log1p_f32(self, x) -> np.ndarray:
        """Correctly rounded binary32 log1p (binary128 evaluation)."""
        x = self._in(x)
        out = np.empty_like(x)
        if self.lib.orc_log1p_f32(_ptr(out), _ptr(x), x.size) != 0:
            raise ValueError("log1p oracle rejected its arguments")
        return out

    def log1p_f64(self, x) -> np.ndarray:
        """binary64 rounding of the binary128 log1p of binary32 inputs."""
        x = self._in(x)
        out = np.empty(x.shape, dtype=np.float64)
        if self.lib.orc_log1p_f64(_ptr(out), _ptr(x), x.size) != 0:
            raise ValueError("log1p oracle rejected its arguments")
        return out

    def log1p_f32_fast(self, x, threads: int = 1):
        """Same results as log1p_f32 (binary64 decides where it can, binary128
        otherwise); returns (out, number of inputs decided in binary128).
        ``threads`` > 1 splits the array over that many host threads."""
        x = self._in(x)
        out = np.empty_like(x)
        flat_x, flat_o = x.reshape(-1), out.reshape(-1)
        n = flat_x.size
        parts = max(1, min(threads, n // 65536 or 1))
        bounds = [n * k // parts for k in range(parts + 1)]
        counts = [0] * parts

        def run(k):
            lo, hi = bounds[k], bounds[k + 1]
            esc = ctypes.c_int64(0)
            rc = self.lib.orc_log1p_f32_fast(flat_o[lo:].ctypes.data, flat_x[lo:].ctypes.data,
                                             hi - lo, ctypes.byref(esc))
            if rc != 0:
                raise ValueError("log1p oracle rejected its arguments")
            counts[k] = esc.value

        if parts == 1:
            run(0)
        else:
            from concurrent.futures import ThreadPoolExecutor

            with ThreadPoolExecutor(parts) as pool:
                list(pool.map(run, range(parts)))
        return out, sum(counts)


_default_log1p = None


def default_log1p() -> Log1pOracle:
    global _default_log1p
    if _default_log1p is None:
        if not os.path.exists(LOG1P_LIBRARY) or (
                os.path.getmtime(LOG1P_LIBRARY) < os.path.getmtime(LOG1P_SOURCE)):
            compile_log1p_library(LOG1P_SOURCE, LOG1P_LIBRARY)
        _default_log1p = Log1pOracle(LOG1P_LIBRARY)
    return _default_log1p


def log1p_f32(x) -> np.ndarray:
    return default_log1p().log1p_f32(x)


def log1p_f64(x) -> np.ndarray:
    return default_log1p().log1p_f64(x)


def log1p_f32_fast(x, threads: int = 1):
    return default_log1p().log1p_f32_fast(x, threads)


def ulp_error_f32(got, ref64) -> np.ndarray:
    """|got - ref| in units of binary32 epsilon times |ref|, the measure of
    the TE issue's reproducer (finfo(float32).eps * |ref|)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref64, dtype=np.float64)
    return np.abs(g - r) / (np.finfo(np.float32).eps * np.abs(r))
