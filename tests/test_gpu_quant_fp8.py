"""The FP8 E4M3 quantised variants on the GPU: per-row OCP E4M3 codes and
fp32 scales, fused (add_rmsnorm_quant_fp8_fwd) and plain
(rmsnorm_quant_fp8_fwd).

Bars:
  * the code routine itself (gfx950's packed fp32 -> fp8 conversion) equal to
    the fp32 model's nearest-even E4M3 rounding, itself pinned to torch's CPU
    float8_e4m3fn cast, on every binary32 input below 464 in magnitude;
  * bit-exact codes, scales and residual_out against the fp32 model of the
    kernels' arithmetic;
  * against the binary64 oracle (which decides codes in binary32 from its own
    y): residual_out bit-exact, scales within 2e-6 relative, codes equal
    except where the oracle's product y * (448 / amax) lies within 2^-12 of a
    rounding boundary (relative, or 2^-19 absolute), where the two fp32
    pipelines may round either way (one code apart);
  * dequantisation within half an E4M3 step of the oracle's y, and no bias;
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

NAN_CODE = 0x7F  # E4M3's NaN: never a valid output of these entry points


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def gpu_fp8(x, r, w, eps=1e-6, path=0, block=0, grid=0, xd=None, rd=None, wd=None):
    """Fused (r given) or plain (r None) fp8 quantised forward."""
    import torch

    xd = to_dev(x) if xd is None else xd
    wd = to_dev(w) if wd is None else wd
    n = x.shape[0]
    q = torch.full(x.shape, NAN_CODE, dtype=torch.uint8, device=xd.device)
    sc = torch.full((n,), float("nan"), dtype=torch.float32, device=xd.device)
    cfg = dict(path=path, block_threads=block, grid_blocks=grid)
    if r is None:
        if path or block or grid:
            arn.rmsnorm_quant_fp8_fwd_cfg(q, sc, xd, wd, eps, **cfg)
        else:
            arn.rmsnorm_quant_fp8_fwd(q, sc, xd, wd, eps)
        res = None
    else:
        rd = to_dev(r) if rd is None else rd
        res = poisoned_like(xd)
        if path or block or grid:
            arn.add_rmsnorm_quant_fp8_fwd_cfg(q, sc, res, xd, rd, wd, eps, **cfg)
        else:
            arn.add_rmsnorm_quant_fp8_fwd(q, sc, res, xd, rd, wd, eps)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sc.cpu().numpy(), (from_dev(res) if res is not None else None)


def same_scale_bits(a, b):
    both_nan = np.isnan(a) & np.isnan(b)
    return np.array_equal(a.view(np.uint32)[~both_nan], b.view(np.uint32)[~both_nan])


def code_line(c):
    """Signed E4M3 codes on a monotone integer line (adjacent values differ by 1)."""
    c = np.asarray(c).astype(np.int32)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def check_model(x, r, w, eps, q, sc, res, label):
    mq, ms, mr = fp32_model.add_rmsnorm_quant_fp8(x, r, w, eps)
    if r is not None:
        bad = (res != mr) & ~(is_nan16(res) & is_nan16(mr))
        assert not bad.any(), "%s residual_out differs in %d" % (label, int(bad.sum()))
    assert same_scale_bits(sc, ms), "%s scales differ" % label
    d = q != mq
    assert not d.any(), "%s codes differ in %d elements, first %s" % (
        label, int(d.sum()), np.argwhere(d)[:3].tolist())


def check_oracle(x, r, w, eps, q, sc, res, label, stats=False):
    oq, os_, orr, y = oracle.add_rmsnorm_quant_fp8(x, r, w, eps, want_exact=True)
    if r is not None:
        assert not ((res != orr) & ~(is_nan16(res) & is_nan16(orr))).any(), label
    with np.errstate(all="ignore"):
        amax32 = np.abs(y.astype(np.float32)).max(axis=1)
    fin = np.isfinite(amax32) & (amax32 >= np.float32(2.0 ** -118))
    assert np.array_equal(np.isnan(sc), np.isnan(os_)), label
    both = np.isfinite(os_)
    assert (np.abs(sc[both] - os_[both]) <= 2e-6 * np.abs(os_[both]) + 2.0 ** -140).all(), label
    assert (q[~fin] == 0).all() and (oq[~fin] == 0).all(), label
    assert ((q & 0x7F) != NAN_CODE).all(), label
    rows = np.where(fin)[0]
    if rows.size == 0:
        return
    # The oracle's binary32 product y * (448 / amax) and whether a small
    # nudge either way changes its E4M3 code (a near tie).
    y32 = y[rows].astype(np.float32)
    inv = (np.float32(448) / amax32[rows]).astype(np.float32)
    quo = (y32 * inv[:, None]).astype(np.float32)
    nudge = np.abs(quo).astype(np.float64) * 2.0 ** -12 + 2.0 ** -19
    lo = fp32_model.e4m3_codes((np.abs(quo) - nudge).clip(0).astype(np.float32))
    hi = fp32_model.e4m3_codes((np.abs(quo) + nudge).astype(np.float32))
    near_tie = lo != hi
    dq = np.abs(code_line(q[rows]) - code_line(oq[rows]))
    assert (dq[~near_tie] == 0).all(), "%s codes differ away from ties: %d" % (
        label, int((dq[~near_tie] != 0).sum()))
    assert (dq <= 1).all(), label
    s = sc[rows, None].astype(np.float64)
    deq = oracle.e4m3_to_f64(q[rows]) * s
    t = np.abs(y[rows]) / s
    half = np.where(t < 2.0 ** -6, 2.0 ** -10,
                    np.exp2(np.floor(np.log2(np.maximum(t, 2.0 ** -6))) - 4))
    assert (np.abs(deq - y[rows]) <= s * half * (1 + 1e-3) + s * 448 * 2.0 ** -22).all(), label
    if stats:
        big = t > 2.0 ** -6
        rel = (deq - y[rows])[big] / np.abs(y[rows])[big]
        assert abs(rel.mean()) < 5 * 0.02 / math.sqrt(rel.size), rel.mean()


def test_code_routine_on_every_input_below_464():
    """All binary32 patterns with |v| < 464 (2 x 1139277824), in chunks of
    2^26, through the kernels' code routine, against the fp32 model."""
    import torch

    limit = 0x43E80000  # 464.0
    chunk = 1 << 26
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda:0")
    done = 0
    for sign in (0, 0x80000000):
        for lo in range(0, limit, chunk):
            n = min(chunk, limit - lo)
            n8 = (n + 7) // 8 * 8
            arn.add_rmsnorm_test_cvt_e4m3_range(out[:n8], sign | lo)
            torch.cuda.synchronize()
            got = out[:n].cpu().numpy()
            v = (np.arange(lo, lo + n, dtype=np.uint32) | np.uint32(sign)).view(np.float32)
            exp = fp32_model.e4m3_codes(v)
            bad = got != exp
            assert not bad.any(), "pattern 0x%08x: got 0x%02x, expected 0x%02x" % (
                int(v.view(np.uint32)[bad][0]), int(got[bad][0]), int(exp[bad][0]))
            done += 1
            if done % 8 == 0:
                announce("  e4m3 code routine: %d chunks agree" % done)
    assert out is not None


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_fp8_workloads(name):
    c = synth.CONFIGS[name]
    announce("fp8 %s" % name)
    x, r, w = synth.workload(c["seed"], c["n_rows"], c["hidden"])
    q, sc, res = gpu_fp8(x, r, w)
    check_model(x, r, w, 1e-6, q, sc, res, name)
    check_oracle(x, r, w, 1e-6, q, sc, res, name, stats=True)


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_plain_fp8_workloads(name):
    c = synth.CONFIGS[name]
    announce("plain fp8 %s" % name)
    x, _, w = synth.workload(c["seed"], c["n_rows"], c["hidden"])
    q, sc, _ = gpu_fp8(x, None, w)
    check_model(x, None, w, 1e-6, q, sc, None, "plain " + name)
    check_oracle(x, None, w, 1e-6, q, sc, None, "plain " + name, stats=True)


@pytest.mark.parametrize("n,h", RAGGED)
def test_fp8_ragged(n, h):
    announce("fp8 ragged %dx%d" % (n, h))
    x, r, w = synth.workload(1300 + h, n, h)
    for rr in (r, None):
        q, sc, res = gpu_fp8(x, rr, w)
        label = "%s %dx%d" % ("fused" if rr is not None else "plain", n, h)
        check_model(x, rr, w, 1e-6, q, sc, res, label)
        check_oracle(x, rr, w, 1e-6, q, sc, res, label)


@pytest.mark.parametrize("h", [64, 1024, 4096, 8192, 16384])
def test_fp8_special_values(h):
    announce("fp8 special hidden %d" % h)
    x, r = _special_rows(h)
    w = synth.bf16_normal(79, 2, (h,), 1.0, 0.1)
    q, sc, res = gpu_fp8(x, r, w)
    check_model(x, r, w, 1e-6, q, sc, res, "special h=%d" % h)
    check_oracle(x, r, w, 1e-6, q, sc, res, "special h=%d" % h)
    q, sc, _ = gpu_fp8(x, None, w)
    check_model(x, None, w, 1e-6, q, sc, None, "plain special h=%d" % h)


def test_fp8_tiny_rows_threshold():
    """Rows whose amax straddles 2^-118: below it the codes are zero."""
    h = 64
    w = synth.to_bf16_bits(np.linspace(0.5, 2.0, h))
    x = np.zeros((6, h), np.uint16)
    x[0], x[1], x[2], x[3], x[4] = 0x0001, 0x0010, 0x0040, 0x0100, 0x0400
    q, sc, res = gpu_fp8(x, x, w)
    check_model(x, x, w, 1e-6, q, sc, res, "tiny rows")
    check_oracle(x, x, w, 1e-6, q, sc, res, "tiny rows")
    assert (q[0] == 0).all() and ((q[4] & 0x7F).max() == 0x7E)


@pytest.mark.parametrize("h", [64, 1000, 2048, 4096, 8192, 12288, 16384, 32768])
def test_fp8_every_launch_configuration(h):
    n = 29
    x, r, w = synth.workload(3300 + h, n, h)
    announce("fp8 invariance hidden %d" % h)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    for rr, rdd in ((r, rd), (None, None)):
        ref = gpu_fp8(x, rr, w, xd=xd, rd=rdd, wd=wd)
        check_model(x, rr, w, 1e-6, *ref, "auto h=%d" % h)
        for path, b, grid in configurations(h):
            got = gpu_fp8(x, rr, w, path=path, block=b, grid=grid, xd=xd, rd=rdd, wd=wd)
            assert np.array_equal(got[0], ref[0]), (rr is None, path, b, grid)
            assert same_scale_bits(got[1], ref[1]), (rr is None, path, b, grid)
            if rr is not None:
                assert np.array_equal(got[2], ref[2]), (path, b, grid)


def test_fp8_in_place_residual_and_float8_dtype():
    import torch

    x, r, w = synth.workload(3400, 40, 4096)
    announce("fp8 in place")
    ref = gpu_fp8(x, r, w)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    q = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=xd.device)
    sc = torch.empty(x.shape[0], dtype=torch.float32, device=xd.device)
    arn.add_rmsnorm_quant_fp8_fwd(q, sc, rd, xd, rd, wd, 1e-6)   # residual_out == residual
    torch.cuda.synchronize()
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), ref[0])
    assert same_scale_bits(sc.cpu().numpy(), ref[1])
    assert np.array_equal(from_dev(rd), ref[2])
    # torch's own decoding of the codes times the scale: the dequantised row
    deq = q.float().cpu().numpy() * sc.cpu().numpy()[:, None]
    _, _, _, y = oracle.add_rmsnorm_quant_fp8(x, r, w, 1e-6, want_exact=True)
    assert np.abs(deq - y).max() <= np.abs(y).max() * 2.0 ** -4


def test_fp8_rejects_bad_arguments():
    import torch

    x, r, w = synth.workload(3500, 4, 64)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    sc = torch.empty(4, dtype=torch.float32, device="cuda:0")
    with pytest.raises(ValueError):
        arn.add_rmsnorm_quant_fp8_fwd(torch.empty(x.shape, dtype=torch.int8, device="cuda:0"), sc,
                                      poisoned_like(xd), xd, rd, wd)
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda:0")
    L = arn.lib()
    assert L.add_rmsnorm_quant_fp8_fwd(q.data_ptr(), sc.data_ptr(), None, xd.data_ptr(), None,
                                       wd.data_ptr(), 4, 64, 1e-6, None) == arn.EINVAL
    assert L.rmsnorm_quant_fp8_fwd(q.data_ptr(), sc.data_ptr(), xd.data_ptr(), wd.data_ptr(), 4,
                                   60, 1e-6, None) == arn.EALIGN
    assert L.rmsnorm_quant_fp8_fwd(q.data_ptr(), sc.data_ptr(), xd.data_ptr(), wd.data_ptr(), 0,
                                   64, 1e-6, None) == arn.OK
