"""The quantised variant on the GPU: per-row int8 codes and fp32 scales.

Bars:
  * bit-exact codes, scales and residual_out against the fp32 model of the
    kernels' arithmetic (tests/pins/fp32_model.c);
  * against the binary64 oracle (which decides codes in binary32 from its
    own y): residual_out bit-exact, scales within 2e-6 relative, codes equal
    except where the oracle's product y * (127 / amax) lies within 1e-3 of a
    half-integer, where the two fp32 pipelines may round either way (+-1);
  * dequantisation within half a step of the oracle's y, and no bias;
  * bitwise invariance over kernel paths, workgroup sizes and grids.
"""
import math

import numpy as np
import pytest

import bf16_rounding_numerics_amd as arn
import fp32_model
import oracle
import synth
from gpu_helpers import announce, from_dev, is_nan16, poisoned_like, require_gpu, to_dev
from test_gpu_invariance import configurations
from test_gpu_parity import RAGGED, _special_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def gpu_quant(x, r, w, eps=1e-6, path=0, block=0, grid=0, xd=None, rd=None, wd=None):
    import torch

    xd = to_dev(x) if xd is None else xd
    rd = to_dev(r) if rd is None else rd
    wd = to_dev(w) if wd is None else wd
    n = x.shape[0]
    q = torch.full(x.shape, 99, dtype=torch.int8, device=xd.device)        # not a valid code
    sc = torch.full((n,), float("nan"), dtype=torch.float32, device=xd.device)
    res = poisoned_like(xd)
    if path or block or grid:
        arn.add_rmsnorm_quant_fwd_cfg(q, sc, res, xd, rd, wd, eps, path=path, block_threads=block,
                                      grid_blocks=grid)
    else:
        arn.add_rmsnorm_quant_fwd(q, sc, res, xd, rd, wd, eps)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sc.cpu().numpy(), from_dev(res)


def same_scale_bits(a, b):
    both_nan = np.isnan(a) & np.isnan(b)
    return np.array_equal(a.view(np.uint32)[~both_nan], b.view(np.uint32)[~both_nan])


def check_model(x, r, w, eps, q, sc, res, label):
    mq, ms, mr = fp32_model.add_rmsnorm_quant(x, r, w, eps)
    bad = (res != mr) & ~(is_nan16(res) & is_nan16(mr))
    assert not bad.any(), "%s residual_out differs in %d" % (label, int(bad.sum()))
    assert same_scale_bits(sc, ms), "%s scales differ" % label
    d = q != mq
    assert not d.any(), "%s codes differ in %d elements, first %s" % (
        label, int(d.sum()), np.argwhere(d)[:3].tolist())


def check_oracle(x, r, w, eps, q, sc, res, label, stats=False):
    oq, os_, orr, y = oracle.add_rmsnorm_quant(x, r, w, eps, want_exact=True)
    assert np.array_equal(res, orr) or not (
        (res != orr) & ~(is_nan16(res) & is_nan16(orr))).any(), label
    # Rows with a finite inverse scale (2^-120 <= amax <= FLT_MAX) are
    # quantised; the others have zero codes.
    with np.errstate(all="ignore"):
        amax32 = np.abs(y.astype(np.float32)).max(axis=1)
    fin = np.isfinite(amax32) & (amax32 >= np.float32(2.0 ** -120))
    assert np.allclose(sc[np.isfinite(os_)], os_[np.isfinite(os_)], rtol=2e-6, atol=0) or \
        (np.abs(sc[np.isfinite(os_)] - os_[np.isfinite(os_)]) <= 2e-6 * np.abs(os_[np.isfinite(os_)])
         + 2.0 ** -140).all(), label
    assert np.array_equal(np.isnan(sc), np.isnan(os_))
    assert np.allclose(sc[fin], os_[fin], rtol=2e-6, atol=0), label
    assert (q[~fin] == 0).all() and (oq[~fin] == 0).all()
    rows = np.where(fin)[0]
    if rows.size == 0:
        return
    # The oracle's binary32 product y * (127 / amax), and how close it is to a
    # rounding boundary.
    y32 = y[rows].astype(np.float32)
    amax = amax32[rows]
    inv = (np.float32(127) / amax).astype(np.float32)
    quo = (y32 * inv[:, None]).astype(np.float64)
    near_tie = np.abs(np.abs(quo - np.floor(quo)) - 0.5) < 1e-3
    dq = np.abs(q[rows].astype(np.int32) - oq[rows].astype(np.int32))
    assert (dq[~near_tie] == 0).all(), "%s codes differ away from ties: %d" % (
        label, int((dq[~near_tie] != 0).sum()))
    assert (dq <= 1).all()
    step = sc[rows, None].astype(np.float64)
    err = q[rows] * step - y[rows]
    assert (np.abs(err) <= step * (0.5 + 1e-3)).all(), label
    if stats:
        steps = (q[rows] - y[rows] / step)
        assert abs(steps.mean()) < 5 * 0.29 / math.sqrt(steps.size) + 1e-6, steps.mean()


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_quant_workloads(name):
    c = synth.CONFIGS[name]
    announce("quant %s" % name)
    x, r, w = synth.workload(c["seed"], c["n_rows"], c["hidden"])
    q, sc, res = gpu_quant(x, r, w)
    check_model(x, r, w, 1e-6, q, sc, res, name)
    check_oracle(x, r, w, 1e-6, q, sc, res, name, stats=True)


@pytest.mark.parametrize("n,h", RAGGED)
def test_quant_ragged(n, h):
    announce("quant ragged %dx%d" % (n, h))
    x, r, w = synth.workload(1100 + h, n, h)
    q, sc, res = gpu_quant(x, r, w)
    check_model(x, r, w, 1e-6, q, sc, res, "%dx%d" % (n, h))
    check_oracle(x, r, w, 1e-6, q, sc, res, "%dx%d" % (n, h))


@pytest.mark.parametrize("h", [64, 1024, 4096, 8192, 16384])
def test_quant_special_values(h):
    announce("quant special hidden %d" % h)
    x, r = _special_rows(h)
    w = synth.bf16_normal(79, 2, (h,), 1.0, 0.1)
    q, sc, res = gpu_quant(x, r, w)
    check_model(x, r, w, 1e-6, q, sc, res, "special h=%d" % h)
    check_oracle(x, r, w, 1e-6, q, sc, res, "special h=%d" % h)


@pytest.mark.parametrize("h", [64, 1000, 2048, 4096, 8192, 12288, 16384, 32768])
def test_quant_every_launch_configuration(h):
    n = 29
    x, r, w = synth.workload(3100 + h, n, h)
    announce("quant invariance hidden %d" % h)
    ref = gpu_quant(x, r, w)
    check_model(x, r, w, 1e-6, *ref, "auto h=%d" % h)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    for path, b, grid in configurations(h):
        got = gpu_quant(x, r, w, path=path, block=b, grid=grid, xd=xd, rd=rd, wd=wd)
        assert np.array_equal(got[0], ref[0]), (path, b, grid)
        assert same_scale_bits(got[1], ref[1]), (path, b, grid)
        assert np.array_equal(got[2], ref[2]), (path, b, grid)


def test_quant_in_place_residual():
    import torch

    x, r, w = synth.workload(3200, 40, 4096)
    announce("quant in place")
    ref = gpu_quant(x, r, w)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    q = torch.empty(x.shape, dtype=torch.int8, device=xd.device)
    sc = torch.empty(x.shape[0], dtype=torch.float32, device=xd.device)
    arn.add_rmsnorm_quant_fwd(q, sc, rd, xd, rd, wd, 1e-6)   # residual_out == residual
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), ref[0])
    assert same_scale_bits(sc.cpu().numpy(), ref[1])
    assert np.array_equal(from_dev(rd), ref[2])
