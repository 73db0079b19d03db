"""Bit-exact agreement of the GPU with the fp32 model of the kernels'
documented arithmetic (GPU).

The parity tests hold out to one bf16 ULP of the binary64 oracle.  Here the
GPU's out and residual_out must equal, bit for bit (NaN-ness for NaN), the
CPU model that follows the same fp32 operations in the same order: the fixed
sum-of-squares tree, correctly rounded division and square root, the two
multiplies.  A different reduction order, a contracted multiply-add or an
approximate reciprocal square root anywhere on any path would show here."""
import numpy as np
import pytest

import bf16_rounding_numerics_amd as arn
import fp32_model
import synth
from gpu_helpers import announce, gpu_fwd, is_nan16, require_gpu, to_dev
from test_gpu_invariance import configurations
from test_gpu_parity import RAGGED, _special_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def assert_same_bits(got, exp, label):
    both_nan = is_nan16(got) & is_nan16(exp)
    bad = (got != exp) & ~both_nan
    assert not bad.any(), "%s: %d elements differ, first at %s (got %s, model %s)" % (
        label, int(bad.sum()), np.argwhere(bad)[:3].tolist(),
        [hex(int(v)) for v in got[bad][:3]], [hex(int(v)) for v in exp[bad][:3]])


def check_model(x, r, w, eps, out, res, label):
    m_out, m_res = fp32_model.add_rmsnorm(x, r, w, eps)
    assert_same_bits(res, m_res, label + " residual_out")
    assert_same_bits(out, m_out, label + " out")


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_workloads_bit_exact(name):
    c = synth.CONFIGS[name]
    announce("model %s" % name)
    x, r, w = synth.workload(c["seed"], c["n_rows"], c["hidden"])
    out, res = gpu_fwd(x, r, w, 1e-6)
    check_model(x, r, w, 1e-6, out, res, name)


@pytest.mark.parametrize("n,h", RAGGED)
def test_ragged_bit_exact(n, h):
    announce("model ragged %dx%d" % (n, h))
    x, r, w = synth.workload(1000 + h, n, h)
    for eps in (1e-6, 0.0):
        out, res = gpu_fwd(x, r, w, eps)
        check_model(x, r, w, eps, out, res, "%dx%d eps %g" % (n, h, eps))


@pytest.mark.parametrize("h", [64, 1024, 4096, 8192, 16384])
def test_special_values_bit_exact(h):
    announce("model special hidden %d" % h)
    x, r = _special_rows(h)
    w = synth.bf16_normal(77, 2, (h,), 1.0, 0.1)
    out, res = gpu_fwd(x, r, w, 1e-6)
    check_model(x, r, w, 1e-6, out, res, "special h=%d" % h)


def _tree_rows(h):
    """Rows whose sum of squares depends strongly on the association order:
    one large segment absorbing many unit segments, placed first, last and in
    the middle; and the (2^24, 1, 1, 0) pattern."""
    segs = h // 8
    rows = []
    for big_at in (0, segs // 2, segs - 1):
        a = np.zeros(h, np.float32)
        a[0::8] = 1.0
        a[8 * big_at] = np.float32(4096.0)  # square 2^24
        rows.append(a)
    a = np.zeros(h, np.float32)
    a[[0, 8, 16]] = [4096.0, 1.0, 1.0]
    rows.append(a)
    a = np.asarray(rows, np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("h", [64, 1024, 2048, 4096, 8192, 16384, 32768])
def test_association_order_rows_on_every_path(h):
    x = _tree_rows(h)
    r = np.zeros_like(x)
    w = synth.bf16_normal(78, 2, (h,), 1.0, 0.1)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    for eps in (0.0, 1e-6):
        m_out, m_res = fp32_model.add_rmsnorm(x, r, w, eps)
        for path, b, grid, late in [(0, 0, 0, False)] + configurations(h, late=True):
            announce("model tree rows hidden %d eps %g path %d block %d grid %d late %d"
                     % (h, eps, path, b, grid, late))
            out, res = gpu_fwd(x, r, w, eps, path=path, block=b, grid=grid, xd=xd, rd=rd, wd=wd,
                               late=late)
            assert_same_bits(res, m_res, "tree h=%d residual_out" % h)
            assert_same_bits(out, m_out, "tree h=%d path %d block %d grid %d late %d"
                             % (h, path, b, grid, late))
