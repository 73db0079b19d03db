"""A seeded sweep of random shapes and layouts on the GPU (every draw is
reproducible from its case number).  Each case picks an entry point (fused,
plain, int8 or E4M3 quantised, fused or plain, per-head q/k), a hidden size
between 1 and 32768 (most of them small, where the kernel choice changes
often), a row count, and for the bf16 entry points a row stride and a start
offset that may leave 16-byte alignment.  Every result must equal the fp32
model of the kernels' arithmetic bit for bit and be within one bf16 ULP of the
oracle (quantised: codes and scales equal to the model's); every element
outside the written views must be left as it was."""
import numpy as np
import pytest

import bf16_rounding_numerics_amd as arn
import fp32_model
import oracle
import synth
from gpu_helpers import POISON, announce, from_dev, is_nan16, require_gpu, to_dev, ulp_distance

pytestmark = pytest.mark.gpu

CASES = 140


def _hidden(rng, aligned):
    h = int(rng.choice([rng.integers(1, 65), rng.integers(65, 513), rng.integers(513, 4097),
                        rng.integers(4097, 32769)], p=[0.3, 0.3, 0.25, 0.15]))
    return max(8, h - h % 8) if aligned else h


def _model_check(got, model, label):
    bad = (got != model) & ~(is_nan16(got) & is_nan16(model))
    assert not bad.any(), "%s: %d elements differ from the fp32 model, first %s" % (
        label, int(bad.sum()), np.argwhere(bad)[:3].tolist())


@pytest.mark.parametrize("case", range(CASES))
def test_random_case(case):
    require_gpu()
    import torch

    rng = np.random.default_rng(90000 + case)
    kind = ["fused", "plain", "quant", "quant_fp8", "plain_quant", "plain_quant_fp8",
            "qk"][case % 7]
    if kind == "qk":
        t = int(rng.integers(1, 300))
        hq, hk = int(rng.integers(1, 41)), int(rng.integers(0, 9))
        d = int(rng.choice([8, 16, 24, 40, 64, 96, 128, 192, 256, 512]))
        extra = 8 * int(rng.integers(0, 3))
        width = (hq + 2 * hk) * d + extra
        buf = synth.to_bf16_bits(rng.standard_normal((t, width)) * rng.choice([1e-3, 1, 30]))
        qw = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(d))
        kw = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(d))
        announce("random case %d: qk t=%d hq=%d hk=%d d=%d width=%d" % (case, t, hq, hk, d,
                                                                        width))
        dev = to_dev(buf)
        q = dev[:, :hq * d].view(t, hq, d)
        k = dev[:, hq * d:(hq + hk) * d].view(t, hk, d)
        arn.qk_rmsnorm_fwd(q, k, q, k, to_dev(qw), to_dev(kw), 1e-6)
        torch.cuda.synchronize()
        got = from_dev(dev)
        assert np.array_equal(got[:, (hq + hk) * d:], buf[:, (hq + hk) * d:]), case
        for x, w, g, lab in ((buf[:, :hq * d], qw, got[:, :hq * d], "q"),
                             (buf[:, hq * d:(hq + hk) * d], kw, got[:, hq * d:(hq + hk) * d],
                              "k")):
            if x.size == 0:
                continue
            rows = np.ascontiguousarray(x).reshape(-1, d)
            m_out, _ = fp32_model.add_rmsnorm(rows, None, w, 1e-6)
            _model_check(g.reshape(-1, d), m_out, "case %d %s" % (case, lab))
            o_out = oracle.rmsnorm(rows, w, 1e-6)
            assert ulp_distance(g.reshape(-1, d), o_out).max() <= 1, (case, lab)
        return

    quant = "quant" in kind
    fused = not kind.startswith("plain")
    n = int(rng.integers(1, 400))
    h = _hidden(rng, aligned=quant or rng.random() < 0.5)
    # bf16 entry points: views inside a wider buffer, at a random row stride
    # and start offset (which may leave 16-byte alignment)
    stride = h + (8 * int(rng.integers(0, 3)) if quant else int(rng.integers(0, 24)))
    off = 8 * int(rng.integers(0, 3)) if quant else int(rng.integers(0, 16))
    eps = float(np.float32(rng.choice([1e-6, 1e-5, 0.0]) if h > 1 else 1e-6))
    scale = rng.choice([1e-3, 1.0, 40.0])
    x = synth.to_bf16_bits(rng.standard_normal((n, h)) * scale)
    r = synth.to_bf16_bits(rng.standard_normal((n, h)) * scale)
    w = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(h))
    announce("random case %d: %s n=%d h=%d stride=%d off=%d eps=%g" % (case, kind, n, h, stride,
                                                                       off, eps))

    def place(a):
        big = np.full(off + n * stride, POISON, np.uint16)
        big[off:off + n * stride].reshape(n, stride)[:, :h] = a
        return big

    def view(dev_big):
        return dev_big[off:off + n * stride].view(n, stride)[:, :h]

    bx, br = to_dev(place(x)), to_dev(place(r))
    bo, bro = to_dev(place(np.full((n, h), POISON, np.uint16))), to_dev(
        place(np.full((n, h), POISON, np.uint16)))
    wd = to_dev(w)
    xv, rv, ov, rov = view(bx), view(br), view(bo), view(bro)
    if not quant:
        if fused:
            arn.add_rmsnorm_fwd_strided(ov, rov, xv, rv, wd, eps)
        else:
            arn.rmsnorm_fwd_strided(ov, xv, wd, eps)
        torch.cuda.synchronize()
        got_big = from_dev(bo)
        got = got_big[off:off + n * stride].reshape(n, stride)[:, :h]
        mask = np.ones(got_big.shape, bool)
        mask[off:off + n * stride].reshape(n, stride)[:, :h] = False
        assert (got_big[mask] == POISON).all(), "case %d wrote outside out's view" % case
        m_out, m_res = fp32_model.add_rmsnorm(x, r if fused else None, w, eps)
        _model_check(got, m_out, "case %d out" % case)
        if fused:
            res = from_dev(bro)[off:off + n * stride].reshape(n, stride)[:, :h]
            assert np.array_equal(res, m_res), case
            o_out, o_res = oracle.add_rmsnorm(x, r, w, eps)
            assert np.array_equal(res, o_res), case
        else:
            o_out = oracle.rmsnorm(x, w, eps)
        assert ulp_distance(got, o_out).max() <= 1, case
        assert np.array_equal(from_dev(bx), place(x)), case
        return

    fp8 = kind.endswith("fp8")
    q = torch.full((n, h), 99, dtype=torch.uint8 if fp8 else torch.int8, device=bx.device)
    sc = torch.full((n,), float("nan"), dtype=torch.float32, device=bx.device)
    if fused:
        arn.add_rmsnorm_quant_fwd_strided(q, sc, rov, xv, rv, wd, eps, fp8=fp8)
    else:
        arn.rmsnorm_quant_fwd_strided(q, sc, xv, wd, eps, fp8=fp8)
    torch.cuda.synchronize()
    model = fp32_model.add_rmsnorm_quant_fp8 if fp8 else fp32_model.add_rmsnorm_quant
    mq, ms, mr = model(x, r if fused else None, w, eps)
    gq, gs = q.cpu().numpy(), sc.cpu().numpy()
    assert np.array_equal(gq, mq), "case %d codes differ in %d" % (case, int((gq != mq).sum()))
    both_nan = np.isnan(gs) & np.isnan(ms)
    assert np.array_equal(gs.view(np.uint32)[~both_nan], ms.view(np.uint32)[~both_nan]), case
    if fused:
        res = from_dev(bro)[off:off + n * stride].reshape(n, stride)[:, :h]
        assert np.array_equal(res, mr), case
