"""Pins for the fp32 model of the kernels' arithmetic contract (CPU only).

The model (tests/pins/fp32_model.c) is what the GPU results are compared
with bit for bit; these tests tie it to the binary64 oracle and to hand
cases that fix its reduction order."""
import numpy as np
import pytest

import fp32_model
import oracle
import synth
from gpu_helpers import ulp_distance


@pytest.mark.parametrize("n,h", [(64, 1024), (16, 4096), (8, 8200), (4, 16384), (33, 24)])
def test_model_agrees_with_the_oracle(n, h):
    x, r, w = synth.workload(600 + h, n, h)
    m_out, m_res = fp32_model.add_rmsnorm(x, r, w, 1e-6)
    o_out, o_res = oracle.add_rmsnorm(x, r, w, 1e-6)
    assert np.array_equal(m_res, o_res)
    d = ulp_distance(m_out, o_out)
    assert d.max() <= 1
    assert (d > 0).mean() < 1e-3


def test_sum_of_squares_is_exact_for_small_integers():
    rng = np.random.default_rng(3)
    h = 4096
    vals = rng.integers(-3, 4, size=(6, h)).astype(np.float32)
    x = (vals.view(np.uint32) >> 16).astype(np.uint16)
    r = np.zeros_like(x)
    w = np.full(h, 0x3F80, np.uint16)
    _, _, ss = fp32_model.add_rmsnorm(x, r, w, 1e-6, want_sumsq=True)
    assert np.array_equal(ss.astype(np.float64), (vals.astype(np.float64) ** 2).sum(axis=1))


def _row(segment_values, h):
    """A row whose segments have the given sums of squares: the first element
    of segment s is sqrt(value), the rest zero."""
    a = np.zeros(h, np.float32)
    for s, v in enumerate(segment_values):
        a[8 * s] = np.float32(np.sqrt(v))
    assert ((a.view(np.uint32) & 0xFFFF) == 0).all()
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def test_reduction_is_pairwise_in_index_order():
    # Segment sums (2^24, 1, 1, 0): pairs first give (2^24 + 1) + (1 + 0),
    # where 2^24 + 1 rounds to 2^24 (tie to even) and the total stays 2^24.
    # Sequential or other groupings reach 2^24 + 2.
    h = 32
    x = _row([2.0 ** 24, 1.0, 1.0, 0.0], h)[None]
    _, _, ss = fp32_model.add_rmsnorm(x, np.zeros_like(x), np.full(h, 0x3F80, np.uint16),
                                      1e-6, want_sumsq=True)
    assert ss[0] == np.float32(2.0 ** 24)
    # Segment sums (1, 1, 2^24, 0): (1 + 1) + (2^24 + 0) = 2^24 + 2, exact.
    x = _row([1.0, 1.0, 2.0 ** 24, 0.0], h)[None]
    _, _, ss = fp32_model.add_rmsnorm(x, np.zeros_like(x), np.full(h, 0x3F80, np.uint16),
                                      1e-6, want_sumsq=True)
    assert ss[0] == np.float32(2.0 ** 24 + 2)


def test_segment_sum_uses_fused_multiply_add():
    # acc = 1 + 2^-23 has 24 significant bits, so acc^2 is not an fp32 value
    # and fma(acc, acc, t) differs from t + fl(acc * acc).  A
    # segment of eight such values must give the fma chain t = acc*acc,
    # t = fma(acc, acc, t) x 7, computed here exactly (each exact sum fits in
    # binary64, so one rounding to fp32 is the fma's).
    from fractions import Fraction

    h = 8
    x = np.full((1, h), 0x3F80, np.uint16)                       # 1
    r = np.full((1, h), np.uint16(np.float32(2.0 ** -23).view(np.uint32) >> 16))
    acc = np.float32(np.float32(1.0) + np.float32(2.0 ** -23))
    a2 = Fraction(float(acc)) ** 2
    t_fma = np.float32(acc * acc)
    t_sep = t_fma
    for _ in range(7):
        t_fma = np.float32(float(a2 + Fraction(float(t_fma))))
        t_sep = np.float32(t_sep + np.float32(acc * acc))
    assert t_fma != t_sep  # the case tells the two apart
    _, _, ss = fp32_model.add_rmsnorm(x, r, np.full(h, 0x3F80, np.uint16), 1e-6,
                                      want_sumsq=True)
    assert ss[0] == t_fma


def test_special_rows_match_the_oracle():
    h = 64
    rng = np.random.default_rng(9)
    base = synth.to_bf16_bits(rng.standard_normal((4, h)))
    x = base.copy()
    x[1, 3] = 0x7FC1
    x[2, 5] = 0x7F80
    x[3] = 0x62C0
    r = np.zeros_like(x)
    w = synth.to_bf16_bits(np.linspace(0.5, 2, h))
    m_out, m_res = fp32_model.add_rmsnorm(x, r, w, 1e-6)
    o_out, o_res = oracle.add_rmsnorm(x, r, w, 1e-6)
    assert ulp_distance(m_res, o_res).max() == 0
    assert ulp_distance(m_out, o_out).max() <= 1


@pytest.mark.parametrize("n,h", [(64, 1024), (16, 4096), (4, 16384)])
def test_quant_model_agrees_with_the_oracle(n, h):
    x, r, w = synth.workload(700 + h, n, h)
    mq, ms, mr = fp32_model.add_rmsnorm_quant(x, r, w, 1e-6)
    oq, os_, orr = oracle.add_rmsnorm_quant(x, r, w, 1e-6)
    assert np.array_equal(mr, orr)
    assert np.allclose(ms, os_, rtol=2e-6, atol=0)
    d = np.abs(mq.astype(np.int32) - oq.astype(np.int32))
    assert d.max() <= 1 and (d > 0).mean() < 1e-3


def test_quant_model_special_rows():
    h = 64
    w = synth.to_bf16_bits(np.linspace(0.5, 2.0, h))
    x = np.zeros((3, h), np.uint16)
    x[1] = 0x3F80
    x[1, 3] = 0x7FC1
    x[2] = 0x62C0
    q, sc, _ = fp32_model.add_rmsnorm_quant(x, np.zeros_like(x), w, 1e-6)
    assert sc[0] == 0 and np.isnan(sc[1]) and sc[2] == 0 and (q == 0).all()


@pytest.mark.parametrize("n,h", [(64, 1024), (8, 8200), (4, 16384)])
def test_plain_model_agrees_with_the_oracle(n, h):
    x, _, w = synth.workload(800 + h, n, h)
    x[0, ::5] = 0x8000                      # -0 must stay -0 (no addition)
    m_out, m_res = fp32_model.add_rmsnorm(x, None, w, 1e-6)
    assert m_res is None
    o_out = oracle.rmsnorm(x, w, 1e-6)
    d = ulp_distance(m_out, o_out)
    assert d.max() <= 1 and (d > 0).mean() < 1e-3
    assert np.array_equal(m_out[0, ::5], o_out[0, ::5])
    # and it is the fused model over an all -0 residual, bit for bit
    f_out, _ = fp32_model.add_rmsnorm(x, np.full_like(x, 0x8000), w, 1e-6)
    assert np.array_equal(m_out, f_out)
    mq, ms, _ = fp32_model.add_rmsnorm_quant(x, None, w, 1e-6)
    fq, fs, _ = fp32_model.add_rmsnorm_quant(x, np.full_like(x, 0x8000), w, 1e-6)
    assert np.array_equal(mq, fq) and np.array_equal(ms.view(np.uint32), fs.view(np.uint32))
    oq, os_ = oracle.rmsnorm_quant(x, w, 1e-6)
    assert np.allclose(ms, os_, rtol=2e-6, atol=0)
    dq = np.abs(mq.astype(np.int32) - oq.astype(np.int32))
    assert dq.max() <= 1 and (dq > 0).mean() < 1e-3


@pytest.mark.parametrize("h", [1, 3, 7, 9, 15, 100, 1001, 4095, 8193])
def test_model_with_a_partial_last_segment_agrees_with_the_oracle(h):
    x, r, w = synth.workload(900 + h, 6, h)
    m_out, m_res = fp32_model.add_rmsnorm(x, r, w, 1e-6)
    o_out, o_res = oracle.add_rmsnorm(x, r, w, 1e-6)
    assert np.array_equal(m_res, o_res)
    assert ulp_distance(m_out, o_out).max() <= 1
    p_out, _ = fp32_model.add_rmsnorm(x, None, w, 1e-6)
    assert ulp_distance(p_out, oracle.rmsnorm(x, w, 1e-6)).max() <= 1


def test_partial_segment_is_zero_padding():
    # hidden 13 equals hidden 16 with three zero columns (weights irrelevant there)
    x, r, w = synth.workload(950, 5, 16)
    x[:, 13:] = 0
    r[:, 13:] = 0
    full, _, s16 = fp32_model.add_rmsnorm(x, r, w, 1e-6, want_sumsq=True)
    part, _, s13 = fp32_model.add_rmsnorm(x[:, :13], r[:, :13], w[:13], 1e-6, want_sumsq=True)
    assert np.array_equal(s16.view(np.uint32), s13.view(np.uint32))


def test_e4m3_model_codes_match_torch_and_the_oracle():
    """The model's bit-arithmetic E4M3 rounding against torch's CPU
    float8_e4m3fn cast (every 61st binary32 pattern below 464 in magnitude,
    and every pattern within 64 units of each E4M3 value and midpoint), and
    against the oracle's search on a sample."""
    import torch

    u = np.arange(0, 0x43E80000, 61, dtype=np.uint32)
    vals = oracle.e4m3_to_f64(np.arange(127))
    pts = np.concatenate([vals, (vals[:-1] + vals[1:]) / 2]).astype(np.float32).view(np.uint32)
    near = (pts[:, None].astype(np.int64) + np.arange(-64, 65)[None, :]).ravel()
    near = near[(near >= 0) & (near < 0x43E80000)].astype(np.uint32)
    u = np.concatenate([u, near])
    v = np.concatenate([u, u | np.uint32(0x80000000)]).view(np.float32)
    got = fp32_model.e4m3_codes(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    rng = np.random.default_rng(91)
    sample = v[rng.integers(0, v.size, 3000)]
    assert all(int(c) == oracle.e4m3_rne(float(x)) for c, x in zip(fp32_model.e4m3_codes(sample), sample))


def _code_steps(a, b):
    """Distance in E4M3 codes between two code arrays (signed codes mapped to
    a monotone integer line)."""
    def line(c):
        c = c.astype(np.int32)
        return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)
    return np.abs(line(a) - line(b))


@pytest.mark.parametrize("n,h", [(64, 1024), (16, 4096), (4, 16384)])
def test_fp8_model_agrees_with_the_oracle(n, h):
    x, r, w = synth.workload(710 + h, n, h)
    mq, ms, mr = fp32_model.add_rmsnorm_quant_fp8(x, r, w, 1e-6)
    oq, os_, orr = oracle.add_rmsnorm_quant_fp8(x, r, w, 1e-6)
    assert np.array_equal(mr, orr)
    assert np.allclose(ms, os_, rtol=2e-6, atol=0)
    d = _code_steps(mq, oq)
    assert d.max() <= 1 and (d > 0).mean() < 1e-3
    pq, ps, _ = fp32_model.add_rmsnorm_quant_fp8(x, None, w, 1e-6)
    oq, os_, _ = oracle.add_rmsnorm_quant_fp8(x, None, w, 1e-6)
    assert np.allclose(ps, os_, rtol=2e-6, atol=0)
    d = _code_steps(pq, oq)
    assert d.max() <= 1 and (d > 0).mean() < 1e-3


def test_fp8_model_special_rows():
    h = 64
    w = synth.to_bf16_bits(np.linspace(0.5, 2.0, h))
    x = np.zeros((4, h), np.uint16)
    x[1] = 0x3F80
    x[1, 3] = 0x7FC1
    x[2] = 0x62C0
    x[3] = 0x0001
    q, sc, _ = fp32_model.add_rmsnorm_quant_fp8(x, x, w, 1e-6)
    assert sc[0] == 0 and np.isnan(sc[1]) and sc[2] == 0 and 0 < sc[3] < 2.0 ** -118 / 448
    assert (q == 0).all()
