"""The quantised entry points on row-strided views (GPU): x, residual and
residual_out as column blocks of wider matrices, codes and scales
contiguous.  Codes, scales and residual_out must equal the contiguous entry
points' on the same rows bit for bit, on every kernel path the hidden size
selects (packed, wavefront, workgroup and LDS two-pass), with the gaps
between the views untouched; residual_out may run in place on residual."""
import numpy as np
import pytest

import bf16_rounding_numerics_amd as arn
import synth
from gpu_helpers import POISON, announce, from_dev, require_gpu, to_dev
from test_gpu_quant import same_scale_bits

pytestmark = pytest.mark.gpu


def _codes(torch, n, h, fp8, dev):
    q = torch.full((n, h), 99, dtype=torch.uint8 if fp8 else torch.int8, device=dev)
    sc = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    return q, sc


@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
@pytest.mark.parametrize("h", [128, 2048, 8192, 16384, 24576])
def test_strided_quant_matches_contiguous(h, fp8):
    require_gpu()
    import torch

    n = 37
    x, r, w = synth.workload(4700 + h, n, h)
    dev = torch.device("cuda:0")
    wd = to_dev(w)
    # contiguous reference
    xd, rd = to_dev(x), to_dev(r)
    q0, s0 = _codes(torch, n, h, fp8, dev)
    ro0 = torch.empty_like(xd)
    call = arn.add_rmsnorm_quant_fp8_fwd if fp8 else arn.add_rmsnorm_quant_fwd
    call(q0, s0, ro0, xd, rd, wd, 1e-6)
    pq0, ps0 = _codes(torch, n, h, fp8, dev)
    (arn.rmsnorm_quant_fp8_fwd if fp8 else arn.rmsnorm_quant_fwd)(pq0, ps0, xd, wd, 1e-6)
    torch.cuda.synchronize()
    ref = (q0.cpu().numpy(), s0.cpu().numpy(), from_dev(ro0))
    pref = (pq0.cpu().numpy(), ps0.cpu().numpy())

    # x, residual, residual_out as column blocks of one [n, 3h + 8] matrix
    ld = 3 * h + 8
    big = np.full((n, ld), POISON, np.uint16)
    big[:, :h] = x
    big[:, h:2 * h] = r
    bd = to_dev(big)
    xs, rs, ros = bd[:, :h], bd[:, h:2 * h], bd[:, 2 * h:3 * h]
    announce("strided quant h=%d fp8=%s" % (h, fp8))
    q1, s1 = _codes(torch, n, h, fp8, dev)
    arn.add_rmsnorm_quant_fwd_strided(q1, s1, ros, xs, rs, wd, 1e-6, fp8=fp8)
    torch.cuda.synchronize()
    got = from_dev(bd)
    assert np.array_equal(q1.cpu().numpy(), ref[0]), (h, fp8)
    assert same_scale_bits(s1.cpu().numpy(), ref[1]), (h, fp8)
    assert np.array_equal(got[:, 2 * h:3 * h], ref[2]), (h, fp8)
    assert np.array_equal(got[:, :2 * h], big[:, :2 * h]) and (got[:, 3 * h:] == POISON).all()

    # plain on the strided x, then in place: residual_out on residual's view
    q2, s2 = _codes(torch, n, h, fp8, dev)
    arn.rmsnorm_quant_fwd_strided(q2, s2, xs, wd, 1e-6, fp8=fp8)
    q3, s3 = _codes(torch, n, h, fp8, dev)
    arn.add_rmsnorm_quant_fwd_strided(q3, s3, rs, xs, rs, wd, 1e-6, fp8=fp8)
    torch.cuda.synchronize()
    assert np.array_equal(q2.cpu().numpy(), pref[0]) and same_scale_bits(s2.cpu().numpy(),
                                                                         pref[1])
    assert np.array_equal(q3.cpu().numpy(), ref[0]) and same_scale_bits(s3.cpu().numpy(), ref[1])
    assert np.array_equal(from_dev(bd)[:, h:2 * h], ref[2])
