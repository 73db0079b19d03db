"""Plain RMSNorm (no residual add) on the GPU, bf16 and int8 out.

Bars, as for the fused op:
  * out bit-exact against the fp32 model of the kernels' arithmetic, and
    within one bf16 ULP of the binary64 oracle, with |mean signed relative
    error| <= 1e-4 on random workloads;
  * bit for bit the fused kernel's out over an all -0 residual (x + -0 = x);
  * signed zeros kept (no addition happens);
  * bitwise invariance over kernel paths, workgroup sizes and grids;
  * int8: codes and scales bit-exact against the fp32 model, and within the
    oracle's near-tie allowance.
"""
import math

import numpy as np
import pytest

import bf16_rounding_numerics_amd as arn
import fp32_model
import oracle
import synth
from gpu_helpers import (BIAS_GATE, announce, from_dev, gpu_fwd, is_nan16, poisoned_like,
                         require_gpu, to_dev, ulp_distance)
from test_gpu_invariance import configurations
from test_gpu_parity import RAGGED, _special_rows

pytestmark = pytest.mark.gpu

NEG_ZERO = 0x8000


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def gpu_plain(x, w, eps=1e-6, path=0, block=0, grid=0, xd=None, wd=None, late=False):
    import torch

    xd = to_dev(x) if xd is None else xd
    wd = to_dev(w) if wd is None else wd
    out = poisoned_like(xd)
    if path or block or grid or late:
        arn.rmsnorm_fwd_cfg(out, xd, wd, eps, path=path, block_threads=block, grid_blocks=grid,
                            late_weight=late)
    else:
        arn.rmsnorm_fwd(out, xd, wd, eps)
    torch.cuda.synchronize()
    return from_dev(out)


def gpu_plain_quant(x, w, eps=1e-6, path=0, block=0, grid=0, xd=None, wd=None):
    import torch

    xd = to_dev(x) if xd is None else xd
    wd = to_dev(w) if wd is None else wd
    n = x.shape[0]
    q = torch.full(x.shape, 99, dtype=torch.int8, device=xd.device)       # not a valid code
    sc = torch.full((n,), float("nan"), dtype=torch.float32, device=xd.device)
    if path or block or grid:
        arn.rmsnorm_quant_fwd_cfg(q, sc, xd, wd, eps, path=path, block_threads=block,
                                  grid_blocks=grid)
    else:
        arn.rmsnorm_quant_fwd(q, sc, xd, wd, eps)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sc.cpu().numpy()


def check_plain(x, w, eps, out, label, bias=False):
    m_out, _ = fp32_model.add_rmsnorm(x, None, w, eps)
    bad = (out != m_out) & ~(is_nan16(out) & is_nan16(m_out))
    assert not bad.any(), "%s differs from the fp32 model in %d elements, first %s" % (
        label, int(bad.sum()), np.argwhere(bad)[:3].tolist())
    o_out, y = oracle.rmsnorm(x, w, eps, want_exact=True)
    d = ulp_distance(out, o_out)
    assert d.max() <= 1, "%s out off by %d ULP" % (label, int(d.max()))
    if bias:
        assert (d == 1).mean() <= 1e-3
        fin = np.isfinite(y)
        b = oracle.magnitude_bias(oracle.bf16_to_f64(out)[fin], y[fin])
        assert abs(b) <= BIAS_GATE, "%s bias %.3e" % (label, b)


def same_scale_bits(a, b):
    both_nan = np.isnan(a) & np.isnan(b)
    return np.array_equal(a.view(np.uint32)[~both_nan], b.view(np.uint32)[~both_nan])


def check_plain_quant(x, w, eps, q, sc, label):
    mq, ms, _ = fp32_model.add_rmsnorm_quant(x, None, w, eps)
    assert same_scale_bits(sc, ms), "%s scales differ from the model" % label
    d = q != mq
    assert not d.any(), "%s codes differ from the model in %d" % (label, int(d.sum()))
    oq, os_, y = oracle.rmsnorm_quant(x, w, eps, want_exact=True)
    assert np.array_equal(np.isnan(sc), np.isnan(os_))
    with np.errstate(all="ignore"):
        amax32 = np.abs(y.astype(np.float32)).max(axis=1)
    fin = np.isfinite(amax32) & (amax32 >= np.float32(2.0 ** -120))
    assert np.allclose(sc[fin], os_[fin], rtol=2e-6, atol=0), label
    assert (q[~fin] == 0).all() and (oq[~fin] == 0).all()
    rows = np.where(fin)[0]
    if rows.size:
        y32 = y[rows].astype(np.float32)
        inv = (np.float32(127) / amax32[rows]).astype(np.float32)
        quo = (y32 * inv[:, None]).astype(np.float64)
        near_tie = np.abs(np.abs(quo - np.floor(quo)) - 0.5) < 1e-3
        dq = np.abs(q[rows].astype(np.int32) - oq[rows].astype(np.int32))
        assert (dq[~near_tie] == 0).all() and (dq <= 1).all(), label
        step = sc[rows, None].astype(np.float64)
        assert (np.abs(q[rows] * step - y[rows]) <= step * (0.5 + 1e-3)).all(), label


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_plain_workloads(name):
    c = synth.CONFIGS[name]
    announce("plain %s" % name)
    x, r, w = synth.workload(c["seed"], c["n_rows"], c["hidden"])
    # x + residual as the normalised input: the fused op's acc distribution
    acc = synth.to_bf16_bits(oracle.bf16_to_f64(x) + oracle.bf16_to_f64(r))
    out = gpu_plain(acc, w)
    check_plain(acc, w, 1e-6, out, name, bias=True)


def test_plain_qk_norm_shape():
    """Per-head q/k norm: rows of head_dim 128, 4096 tokens x 32 heads."""
    announce("plain q/k norm 131072x128")
    x = synth.bf16_normal(5100, 0, (131072, 128), 0.0, 1.0)
    w = synth.bf16_normal(5100, 2, (128,), 1.0, 0.1)
    out = gpu_plain(x, w)
    check_plain(x, w, 1e-6, out, "qk", bias=True)
    q, sc = gpu_plain_quant(x, w)
    check_plain_quant(x, w, 1e-6, q, sc, "qk quant")


@pytest.mark.parametrize("n,h", RAGGED)
def test_plain_ragged(n, h):
    announce("plain ragged %dx%d" % (n, h))
    x, _, w = synth.workload(1300 + h, n, h)
    out = gpu_plain(x, w)
    check_plain(x, w, 1e-6, out, "%dx%d" % (n, h))
    q, sc = gpu_plain_quant(x, w)
    check_plain_quant(x, w, 1e-6, q, sc, "quant %dx%d" % (n, h))


@pytest.mark.parametrize("h", [64, 1024, 4096, 8192, 16384])
def test_plain_special_values_and_signed_zeros(h):
    announce("plain special hidden %d" % h)
    x, _ = _special_rows(h)
    rng = np.random.default_rng(h)
    extra = synth.to_bf16_bits(rng.standard_normal((3, h)))
    extra[0, ::4] = NEG_ZERO
    extra[1, :] = NEG_ZERO
    extra[2, ::2] = 0
    x = np.concatenate([x, extra])
    w = synth.bf16_normal(81, 2, (h,), 1.0, 0.5)
    out = gpu_plain(x, w)
    check_plain(x, w, 1e-6, out, "special h=%d" % h)
    # a -0 input gives a zero whose sign is that of -0 * w
    zero_neg = x == NEG_ZERO
    expect = np.where((w[None, :] & 0x8000) != 0, 0, NEG_ZERO)
    fin_rows = ~is_nan16(out).any(axis=1)
    sel = zero_neg & fin_rows[:, None]
    assert np.array_equal(out[sel], np.broadcast_to(expect, x.shape)[sel])
    q, sc = gpu_plain_quant(x, w)
    check_plain_quant(x, w, 1e-6, q, sc, "quant special h=%d" % h)


@pytest.mark.parametrize("h", [64, 1024, 8192, 16384])
def test_plain_is_fused_over_negative_zero_residual(h):
    announce("plain vs fused(-0) hidden %d" % h)
    x, _, w = synth.workload(1400 + h, 21, h)
    x[0, ::3] = NEG_ZERO
    out = gpu_plain(x, w)
    f_out, f_res = gpu_fwd(x, np.full_like(x, NEG_ZERO), w, 1e-6)
    assert np.array_equal(out, f_out)
    assert np.array_equal(f_res, x)


@pytest.mark.parametrize("h", [64, 1000, 2048, 4096, 8192, 12288, 16384, 32768])
def test_plain_every_launch_configuration(h):
    n = 23
    x, _, w = synth.workload(3300 + h, n, h)
    announce("plain invariance hidden %d" % h)
    ref = gpu_plain(x, w)
    check_plain(x, w, 1e-6, ref, "auto h=%d" % h)
    qref = gpu_plain_quant(x, w)
    xd, wd = to_dev(x), to_dev(w)
    for path, b, grid, late in configurations(h, late=True):
        got = gpu_plain(x, w, path=path, block=b, grid=grid, xd=xd, wd=wd, late=late)
        assert np.array_equal(got, ref), (path, b, grid, late)
        if late:
            continue  # the late weight read is built for bf16 out only
        gq = gpu_plain_quant(x, w, path=path, block=b, grid=grid, xd=xd, wd=wd)
        assert np.array_equal(gq[0], qref[0]) and same_scale_bits(gq[1], qref[1]), (path, b, grid)


@pytest.mark.parametrize("h", [1024, 8192, 16384])
def test_plain_in_place(h):
    x, _, w = synth.workload(3400 + h, 40, h)
    announce("plain in place hidden %d" % h)
    ref = gpu_plain(x, w)
    xd = to_dev(x)
    arn.rmsnorm_fwd(xd, xd, to_dev(w), 1e-6)
    import torch

    torch.cuda.synchronize()
    assert np.array_equal(from_dev(xd), ref)
