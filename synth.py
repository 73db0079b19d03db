"""Seeded synthetic inputs: counter-based SplitMix64 + Box-Muller normals -> bf16,
and uniform binary32 values for the log1p workload.

This module is shared by the tests, the smoke check and the benchmark, and by
both sides of every parity comparison.  It holds none of the arithmetic of the
fused op; it only manufactures bf16 input bit patterns.

Generator, per (seed, stream):
  * SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): state_i = s0 + (i + 1) * 0x9E3779B97F4A7C15
    (mod 2^64), output_i = mix(state_i), where mix is SplitMix64's finaliser.
    It is counter-based, so any slice of the stream can be computed directly.
  * s0 = mix(mix(seed) + stream): distinct streams per seed.
  * Box-Muller on consecutive outputs (2k, 2k+1):
      u1 = ((z_2k >> 11) + 1) * 2^-53 in (0, 1],  u2 = (z_2k+1 >> 11) * 2^-53,
      n_2k = sqrt(-2 ln u1) cos(2 pi u2),  n_2k+1 = sqrt(-2 ln u1) sin(2 pi u2).
  * value = mean + std * n, rounded to fp32 (numpy) and then to bf16 by torch's
    CPU conversion, as the pages build their inputs: randn * scale, then
    .to(torch.bfloat16).

Streams used by the workloads: x = 0, residual = 1, weight = 2, and the fresh
x of chain step k = 1000 + k (the pages reseed each chain step with 1000+step).
"""
from __future__ import annotations

import hashlib
import os

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK = (1 << 64) - 1

STREAM_X = 0
STREAM_RESIDUAL = 1
STREAM_WEIGHT = 2
STREAM_CHAIN_BASE = 1000


def _mix_int(z: int) -> int:
    z &= _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> int:
    return _mix_int(_mix_int(seed) + stream)


def splitmix64(s0: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of SplitMix64 started from state s0."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(np.uint64(s0 & _MASK) + i * GAMMA)


def _normal_pairs(key: int, p0: int, p1: int) -> np.ndarray:
    """Box-Muller deviates 2*p0 .. 2*p1-1 of the stream with state key."""
    z = splitmix64(key, 2 * p0, 2 * (p1 - p0))
    scale = 2.0 ** -53
    u1 = ((z[0::2] >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * scale
    u2 = (z[1::2] >> np.uint64(11)).astype(np.float64) * scale
    rad = np.sqrt(-2.0 * np.log(u1))
    th = (2.0 * np.pi) * u2
    pair = np.empty((p1 - p0, 2), dtype=np.float64)
    pair[:, 0] = rad * np.cos(th)
    pair[:, 1] = rad * np.sin(th)
    return pair.reshape(-1)


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor

        _POOL = ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1)))
    return _POOL


def normal(seed: int, stream: int, n: int, mean: float = 0.0, std: float = 1.0,
           chunk: int = 1 << 20) -> np.ndarray:
    """n binary64 normal deviates mean + std * N(0, 1) (Box-Muller).

    Chunks are computed on a thread pool (numpy releases the GIL); the values
    depend only on (seed, stream, index), not on the chunking.
    """
    key = stream_key(seed, stream)
    out = np.empty(n, dtype=np.float64)
    pairs = (n + 1) // 2

    def work(p0):
        p1 = min(pairs, p0 + chunk)
        vals = _normal_pairs(key, p0, p1)
        lo, hi = 2 * p0, min(n, 2 * p1)
        out[lo:hi] = vals[: hi - lo]

    list(_pool().map(work, range(0, pairs, chunk)))
    return mean + std * out


def to_bf16_bits(values: np.ndarray) -> np.ndarray:
    """Round real values to bf16 bit patterns (fp32 first, then torch's CPU cast)."""
    import torch

    f32 = np.ascontiguousarray(values, dtype=np.float32)
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_normal(seed: int, stream: int, shape, mean: float = 0.0,
                std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of shape ``shape`` drawn from N(mean, std^2)."""
    n = int(np.prod(shape))
    return to_bf16_bits(normal(seed, stream, n, mean, std)).reshape(shape)


def workload(seed: int, n_rows: int, hidden: int, x_std: float = 1.0,
             residual_std: float = 1.0, w_std: float = 0.1):
    """(x, residual, weight) bf16 bit arrays: x, residual ~ N(0, std^2),
    weight ~ 1 + w_std * N(0, 1)."""
    x = bf16_normal(seed, STREAM_X, (n_rows, hidden), 0.0, x_std)
    r = bf16_normal(seed, STREAM_RESIDUAL, (n_rows, hidden), 0.0, residual_std)
    w = bf16_normal(seed, STREAM_WEIGHT, (hidden,), 1.0, w_std)
    return x, r, w


def chain_delta(seed: int, step: int, n_rows: int, hidden: int, std: float) -> np.ndarray:
    """Fresh x for chain step ``step`` (stream 1000 + step)."""
    return bf16_normal(seed, STREAM_CHAIN_BASE + step, (n_rows, hidden), 0.0, std)


def uniform_f32(seed: int, stream: int, n: int) -> np.ndarray:
    """n binary32 values uniform on [0, 1): the top 24 bits of each SplitMix64
    output times 2^-24 (exact in binary32), like torch.rand's binary32 draws."""
    z = splitmix64(stream_key(seed, stream), 0, n)
    return ((z >> np.uint64(40)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# The log1p workload of the TE issue's reproducer: N binary32 inputs uniform on
# [0, 1) (its torch.rand(N)); the benchmark uses a larger N of the same kind.
LOG1P_N = 225280
LOG1P_BENCH_N = 1 << 26
LOG1P_SEED = 7

# The five workloads, named rows x hidden.  Distributions as in workload().
CONFIGS = {
    "64x1024": dict(seed=1, n_rows=64, hidden=1024),
    "2048x4096": dict(seed=2, n_rows=2048, hidden=4096),
    "4096x8192": dict(seed=3, n_rows=4096, hidden=8192),
    "8192x2048": dict(seed=4, n_rows=8192, hidden=2048),
    "2048x16384": dict(seed=5, n_rows=2048, hidden=16384),
}
