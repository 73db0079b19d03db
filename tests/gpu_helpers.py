"""Shared helpers of the GPU tests: moving bf16 bit arrays to and from the
device, calling the HIP library through its C ABI, and comparing with the
oracle to the parity bar (residual_out bit-exact, out within one bf16 ULP,
|mean signed relative error| <= 1e-4)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle

POISON = 0x7FC1  # a NaN pattern no kernel writes: unwritten outputs stay visible

BIAS_GATE = 1e-4


def torch_mod():
    import torch

    return torch


def require_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_dev(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to("cuda:0")


def from_dev(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def poisoned_like(t):
    torch = torch_mod()
    return torch.full_like(t, np.int16(np.uint16(POISON).view(np.int16)))


def announce(msg: str) -> None:
    """Name the case on stdout before a GPU step (kept if the step fails)."""
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_fwd(x, r, w, eps=1e-6, path=0, block=0, grid=0, xd=None, rd=None, wd=None,
            stream=None, late=False):
    """Run the HIP forward; returns (out, residual_out) as uint16 arrays."""
    import bf16_rounding_numerics_amd as arn

    torch = torch_mod()
    xd = to_dev(x) if xd is None else xd
    rd = to_dev(r) if rd is None else rd
    wd = to_dev(w) if wd is None else wd
    out = poisoned_like(xd)
    res = poisoned_like(xd)
    if path or block or grid or late:
        arn.add_rmsnorm_fwd_cfg(out, res, xd, rd, wd, eps, path=path, block_threads=block,
                                grid_blocks=grid, stream=stream, late_weight=late)
    else:
        arn.add_rmsnorm_fwd(out, res, xd, rd, wd, eps, stream=stream)
    torch.cuda.synchronize()
    return from_dev(out), from_dev(res)


def is_nan16(b: np.ndarray) -> np.ndarray:
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 ULPs on the ordered line (+0 and -0 coincide);
    NaN vs NaN is 0, NaN vs a number is a huge value."""
    def ordered(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)

    d = np.abs(ordered(a) - ordered(b))
    na, nb = is_nan16(a), is_nan16(b)
    d = np.where(na & nb, 0, d)
    d = np.where(na ^ nb, 1 << 20, d)
    return d


def check_parity(x, r, w, eps, got_out, got_res, bias=None, label=""):
    """Assert the parity bar against the oracle; returns stats."""
    exp_out, exp_res, y = oracle.add_rmsnorm(x, r, w, eps, want_exact=True)
    nan_res = is_nan16(exp_res)
    # residual_out: bit-exact (NaN payloads are not compared, NaN-ness is).
    bad_res = (got_res != exp_res) & ~(nan_res & is_nan16(got_res))
    assert not bad_res.any(), "%s residual_out differs in %d elements, first at %s" % (
        label, int(bad_res.sum()), np.argwhere(bad_res)[:3].tolist())
    d = ulp_distance(got_out, exp_out)
    assert d.max() <= 1, "%s out off by %d ULP at %s" % (label, int(d.max()),
                                                          np.argwhere(d > 1)[:3].tolist())
    stats = dict(n=int(d.size), off_by_one=int((d == 1).sum()))
    if bias is not None:
        finite = np.isfinite(y)
        b = oracle.magnitude_bias(oracle.bf16_to_f64(got_out)[finite], y[finite])
        stats["bias_out"] = b
        assert abs(b) <= bias, "%s out bias %.3e" % (label, b)
        acc = oracle.bf16_to_f64(x) + oracle.bf16_to_f64(r)
        fin = np.isfinite(acc)
        b2 = oracle.magnitude_bias(oracle.bf16_to_f64(got_res)[fin], acc[fin])
        stats["bias_residual_out"] = b2
        assert abs(b2) <= bias, "%s residual_out bias %.3e" % (label, b2)
    return stats
