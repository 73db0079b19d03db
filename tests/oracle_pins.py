"""Checks that pin the fused oracle to facts other than itself.

Each ``pin_*`` function takes an oracle object (oracle.Oracle) and raises
AssertionError when the oracle disagrees with a closed form, an invariant,
exact rational arithmetic or a value printed on the aiter issue
"rmsnorm2d_fwd_with_add truncates fp32->bf16 on gfx942, biasing residual_out
and compounding across layers".  The tests call them on the real oracle and on
copies with planted mistakes, which must fail at least one of them.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ helpers

def f32_to_bits16_exact(v) -> np.ndarray:
    """Bit patterns of values that bf16 represents exactly (checked)."""
    a = np.asarray(v, dtype=np.float32)
    u = a.view(np.uint32)
    assert not (u & 0xFFFF).any(), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def bits16_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def is_nan16(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)


def random_bf16_weights(rng, h, lo=0.5, hi=2.0, negative=True):
    w = rng.uniform(lo, hi, size=h)
    if negative:
        w *= np.where(rng.random(h) < 0.3, -1.0, 1.0)
    return synth.to_bf16_bits(w)


# ------------------------------------------------------------------ closed forms

def pin_constant_rows(orc):
    """acc = c in every position: out = sign(c) * w exactly for |c| >= 1/16."""
    rng = np.random.default_rng(11)
    for h in (8, 1000, 4096):
        w = random_bf16_weights(rng, h)
        for c in (1.0 / 16, -1.0 / 16, 1.0, -3.5, 1024.0, -(2.0 ** 40), 2.0 ** 56):
            x = np.full((1, h), f32_to_bits16_exact([c / 2])[0], dtype=np.uint16)
            r = x.copy()
            out, ro = orc.add_rmsnorm(x, r, w, 1e-6)
            assert (ro == f32_to_bits16_exact([c])[0]).all(), ("residual_out", h, c)
            expect = w if c > 0 else w ^ np.uint16(0x8000)
            assert np.array_equal(out[0], expect), ("out", h, c)


def pin_eps_inside_sqrt_after_mean(orc):
    """acc = c = 2^-10 everywhere and eps = 3 c^2: rinv = 1/(2c), out = w/2."""
    rng = np.random.default_rng(12)
    h = 512
    w = random_bf16_weights(rng, h)
    c = 2.0 ** -10
    for sign in (1.0, -1.0):
        x = np.full((1, h), f32_to_bits16_exact([sign * c])[0], dtype=np.uint16)
        r = np.zeros((1, h), dtype=np.uint16)
        out, _ = orc.add_rmsnorm(x, r, w, 3.0 * 2.0 ** -20)
        expect = f32_to_bits16_exact(sign * bits16_to_f32(w) / 2)
        assert np.array_equal(out[0], expect), sign
        out0, _ = orc.add_rmsnorm(x, r, w, 0.0)
        expect0 = w if sign > 0 else w ^ np.uint16(0x8000)
        assert np.array_equal(out0[0], expect0)


def pin_one_hot_rows(orc):
    """A single nonzero a = +-16 at k: out_k = sign(a) sqrt(H) w_k (population
    mean, so a divisor of H - 1 would miss); elsewhere +-0 with w's sign."""
    rng = np.random.default_rng(13)
    for h in (1024, 4096, 16384):
        w = random_bf16_weights(rng, h)
        root = math.isqrt(h)
        ks = rng.choice(h, size=4, replace=False)
        for k in ks:
            for a in (16.0, -16.0):
                x = np.zeros((1, h), dtype=np.uint16)
                x[0, k] = f32_to_bits16_exact([a])[0]
                r = np.zeros((1, h), dtype=np.uint16)
                out, ro = orc.add_rmsnorm(x, r, w, 1e-6)
                wk = bits16_to_f32(w[k])
                assert out[0, k] == f32_to_bits16_exact([math.copysign(1, a) * root * wk])[0], \
                    (h, k, a)
                others = np.delete(np.arange(h), k)
                expect = np.where(bits16_to_f32(w[others]) < 0, 0x8000, 0).astype(np.uint16)
                assert np.array_equal(out[0, others], expect)
                assert np.array_equal(ro, x)


def pin_zero_rows(orc):
    """Zero rows: residual_out keeps IEEE's zero sign, out is +-0."""
    rng = np.random.default_rng(14)
    h = 256
    w = random_bf16_weights(rng, h)
    wneg = bits16_to_f32(w) < 0
    for xs, rs, ro_expect in ((0x0000, 0x0000, 0x0000), (0x8000, 0x0000, 0x0000),
                              (0x8000, 0x8000, 0x8000)):
        x = np.full((1, h), xs, dtype=np.uint16)
        r = np.full((1, h), rs, dtype=np.uint16)
        out, ro = orc.add_rmsnorm(x, r, w, 1e-6)
        assert (ro == ro_expect).all()
        acc_neg = ro_expect == 0x8000
        expect = np.where(wneg != acc_neg, 0x8000, 0).astype(np.uint16)
        assert np.array_equal(out[0], expect)


def pin_zero_row_eps_zero(orc):
    """eps = 0 and a zero row: the mean of squares is 0, rinv = 1/sqrt(0) = +Inf
    and every (acc * rinv) * w is 0 * Inf, a NaN (IEEE, as in the page's fp32
    reference); residual_out is the zero itself.  A nonzero row beside it is
    unaffected: rows are independent."""
    rng = np.random.default_rng(15)
    h = 192
    w = random_bf16_weights(rng, h)
    x = np.zeros((2, h), dtype=np.uint16)
    r = np.zeros((2, h), dtype=np.uint16)
    x[1, 7] = 0x3F80  # 1.0 at k = 7: out_7 = sqrt(h) w_7 / 1, the rest +-0
    out, ro = orc.add_rmsnorm(x, r, w, 0.0)
    assert is_nan16(out[0]).all()
    assert (ro[0] == 0).all()
    assert not is_nan16(out[1]).any()
    wf = bits16_to_f32(w).astype(np.float64)
    y7 = np.sqrt(float(h)) * wf[7]
    got7 = float(bits16_to_f32(out[1:2, 7:8])[0, 0])
    assert abs(got7 - y7) <= abs(y7) * 2.0 ** -8  # within one bf16 rounding
    others = np.delete(out[1], 7)
    assert ((others & 0x7FFF) == 0).all()


def pin_power_of_two_scaling(orc):
    """eps = 0: scaling x and residual by 2^k leaves out unchanged, bit for bit,
    and scales residual_out exactly (correct rounding commutes with it)."""
    x, r, w = synth.workload(seed=21, n_rows=8, hidden=1024)
    out0, ro0 = orc.add_rmsnorm(x, r, w, 0.0)
    for k in (-30, -7, 3, 20):
        xs = f32_to_bits16_exact(bits16_to_f32(x) * np.float32(2.0 ** k))
        rs = f32_to_bits16_exact(bits16_to_f32(r) * np.float32(2.0 ** k))
        out, ro = orc.add_rmsnorm(xs, rs, w, 0.0)
        assert np.array_equal(out, out0), k
        assert np.array_equal(ro, f32_to_bits16_exact(bits16_to_f32(ro0) * np.float32(2.0 ** k)))


# ------------------------------------------------------------------ exact arithmetic

def _exact_round_quotient(t: Fraction, v: Fraction) -> int:
    """bf16 (nearest-even) of y = t / sqrt(v), decided exactly: |y| > m iff
    t^2 > m^2 v for a candidate midpoint m."""
    sign = 0x8000 if t < 0 else 0
    if t == 0:
        return sign
    approx = abs(float(t)) / math.sqrt(float(v))
    # bf16 magnitudes around the approximation, as exact rationals.
    e = math.frexp(approx)[1] - 1
    q = Fraction(2) ** (max(e, -126) - 7)
    k0 = int(Fraction(approx) // q)
    t2 = t * t

    def above(m: Fraction) -> int:  # sign of |y| - m
        lhs, rhs = t2, m * m * v
        return (lhs > rhs) - (lhs < rhs)

    # Candidates k*q for k in k0-2 .. k0+3 bracket |y| (the approximation is
    # far closer than one spacing); pick the nearest by exact midpoint tests.
    cands = [k * q for k in range(max(k0 - 2, 0), k0 + 4)]
    for lo, hi in zip(cands, cands[1:]):
        if above(lo) >= 0 and above(hi) <= 0:
            mid = (lo + hi) / 2
            s = above(mid)
            kk = lo / q
            if s < 0 or (s == 0 and kk.numerator % 2 == 0):
                r = lo
            else:
                r = hi
            f = np.float32(float(r))
            assert Fraction(float(f)) == r
            return sign | int(np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16)
    raise AssertionError("bracketing failed")


def _near_tie_rows():
    """Rows whose out lands a hair below a bf16 midpoint: acc = (3, 4, 0, ...)
    with H = 25, so S/H = 1 and rinv = 1/sqrt(1 + eps) with eps = 2^-30; a
    weight w with 3w exactly a midpoint above an odd bf16 value puts y_0 just
    below it.  Correct rounding goes down; rounding through fp32 first lands
    on the midpoint and then goes up to the even neighbour."""
    ws = []
    for b in range(0x3F80, 0x4000):
        w = float(bits16_to_f32(b))
        m = 3 * w  # exact in binary64
        u = int(np.array([m], dtype=np.float32).view(np.uint32)[0])
        if np.float32(m) == m and (u & 0xFFFF) == 0x8000 and (u >> 16) & 1:
            ws.append(b)
    assert ws, "no midpoint weights found"
    rows = []
    for b in ws[:6]:
        for sgn in (1.0, -1.0):
            h = 25
            x = np.zeros(h, dtype=np.uint16)
            x[0] = f32_to_bits16_exact([sgn * 3.0])[0]
            x[1] = f32_to_bits16_exact([4.0])[0]
            w = np.full(h, 0x3F80, dtype=np.uint16)
            w[0] = b
            rows.append((x, np.zeros(h, dtype=np.uint16), w, 2.0 ** -30))
    return rows


def _random_small_rows(rng):
    for h in (8, 16, 24, 40, 64):
        for _ in range(12):
            x = synth.to_bf16_bits(rng.standard_normal(h) * rng.choice([1e-3, 1.0, 50.0]))
            r = synth.to_bf16_bits(rng.standard_normal(h) * rng.choice([1e-3, 1.0, 50.0]))
            w = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(h))
            eps = float(np.float32(rng.choice([1e-6, 0.5, 0.0])))
            yield x, r, w, eps


def pin_exact_rationals_small_rows(orc):
    """Small rows computed in exact rational arithmetic: acc from the fp32 add,
    S = sum acc^2 exactly, v = S/H + eps, out = nearest-even bf16 of acc w / sqrt(v)."""
    rng = np.random.default_rng(15)
    cases = list(_random_small_rows(rng)) + _near_tie_rows()
    for row, (x, r, w, eps) in enumerate(cases):
        h = x.shape[0]
        out, ro, y = orc.add_rmsnorm(x[None], r[None], w, eps, want_exact=True)
        acc = bits16_to_f32(x) + bits16_to_f32(r)  # the definition's fp32 add
        accq = [Fraction(float(a)) for a in acc]
        s = sum(a * a for a in accq)
        v = s / h + Fraction(eps)
        for j in range(h):
            t = accq[j] * Fraction(float(bits16_to_f32(w[j])))
            expect = _exact_round_quotient(t, v)
            assert out[0, j] == expect, (h, row, j, hex(out[0, j]), hex(expect))
            exact = float(t) / math.sqrt(float(v))
            assert abs(y[0, j] - exact) <= 1e-12 * abs(exact) + 1e-300


# ------------------------------------------------------------------ special values

def pin_special_values(orc):
    """NaN, Inf and overflow follow IEEE arithmetic through each step."""
    h = 16
    w = synth.to_bf16_bits(np.linspace(0.5, 2.0, h))
    one = f32_to_bits16_exact([1.0])[0]
    # NaN in one element: that residual_out element is NaN, the whole out row NaN.
    x = np.full((1, h), one, dtype=np.uint16)
    r = np.zeros((1, h), dtype=np.uint16)
    x[0, 3] = 0x7FC1
    out, ro = orc.add_rmsnorm(x, r, w, 1e-6)
    assert is_nan16(ro[0, 3]) and (ro[0, np.arange(h) != 3] == one).all()
    assert is_nan16(out).all()
    # +Inf in one element: residual_out Inf there; rinv = 0, so out is NaN
    # there (Inf * 0) and +-0 elsewhere.
    x[0, 3] = 0x7F80
    out, ro = orc.add_rmsnorm(x, r, w, 1e-6)
    assert ro[0, 3] == 0x7F80
    assert is_nan16(out[0, 3]) and (out[0, np.arange(h) != 3] == 0).all()
    # +Inf + -Inf = NaN.
    r2 = r.copy()
    r2[0, 3] = 0xFF80
    out, ro = orc.add_rmsnorm(x, r2, w, 1e-6)
    assert is_nan16(ro[0, 3]) and is_nan16(out).all()
    # Finite overflow of the fp32 add: max bf16 + max bf16 = +Inf.
    xm = np.full((1, h), 0x7F7F, dtype=np.uint16)
    out, ro = orc.add_rmsnorm(xm, xm, w, 1e-6)
    assert (ro == 0x7F80).all() and is_nan16(out).all()
    # Sum of squares beyond fp32 range with finite acc: fp32 accumulation gives
    # Inf, rinv = 0, out = +-0 with sign(acc) * sign(w).
    big = f32_to_bits16_exact([2.0 ** 70])[0]
    xb = np.full((1, h), big, dtype=np.uint16)
    xb[0, ::2] |= 0x8000
    out, ro = orc.add_rmsnorm(xb, np.zeros_like(xb), w, 1e-6)
    assert np.array_equal(ro, xb)
    assert np.array_equal(out[0], (xb[0] & 0x8000))
    # Just inside fp32 range the row normalises as usual: 16 * (2^63)^2 = 2^130
    # overflows, 16 * (2^61)^2 = 2^126 does not -> out = sign * w.
    ok = f32_to_bits16_exact([2.0 ** 61])[0]
    xo = np.full((1, h), ok, dtype=np.uint16)
    out, _ = orc.add_rmsnorm(xo, np.zeros_like(xo), w, 1e-6)
    assert np.array_equal(out[0], w)


# ------------------------------------------------------------------ metric

def pin_magnitude_bias_metric(_orc=None):
    """magnitude_bias on hand examples.

    ((1-2)/2 + (3-4)/4 + 0) / 3 = -0.25, with the exp == 0 element left out.
    Signs do not matter, only magnitudes: got -3 against exp 2 is +1/2.
    A uniform shrink by 2^-8 gives exactly -2^-8; growth gives a positive
    value; a single element is its own relative error.
    """
    got = np.array([1.0, -3.0, 2.0, 5.0])
    exp = np.array([2.0, -4.0, 2.0, 0.0])
    assert oracle.magnitude_bias(got, exp) == -0.25
    assert oracle.ratio_bias(got, exp) == (1 + 3 + 2 + 5 - 2 - 4 - 2) / 8.0
    assert oracle.magnitude_bias(np.array([-3.0]), np.array([2.0])) == 0.5
    e = np.array([1.0, -2.0, 4.0, 0.5, -0.25])
    assert oracle.magnitude_bias(e * (1 - 2.0 ** -8), e) == -(2.0 ** -8)
    assert oracle.magnitude_bias(np.array([3.0, 5.0]), np.array([2.0, 4.0])) == (0.5 + 0.25) / 2
    # the mean is over the nonzero exact values only: zeros neither count nor divide
    assert oracle.magnitude_bias(np.array([9.0, 1.5, 7.0]), np.array([0.0, 1.0, 0.0])) == 0.5
    with pytest.raises(ValueError):
        oracle.magnitude_bias(np.array([1.0]), np.array([0.0]))


# ------------------------------------------------------------------ page experiments

def page_values():
    with open(os.path.join(GOLDEN, "page_printed_values.json")) as f:
        return json.load(f)


def rounding_mode_experiment(orc, rows, x_std, residual_std, seed):
    """Section 1 of the page's script with our generator: bias of a truncating
    residual_out against the nearest-even one, and how many elements differ."""
    h = 4096
    x = synth.bf16_normal(seed, synth.STREAM_X, (rows, h), 0.0, x_std)
    r = synth.bf16_normal(seed, synth.STREAM_RESIDUAL, (rows, h), 0.0, residual_std)
    w = synth.bf16_normal(seed, synth.STREAM_WEIGHT, (h,), 1.0, 0.05)
    _, ro_t = orc.add_rmsnorm(x, r, w, 1e-6, rounding=oracle.TRUNC)
    _, ro_r = orc.add_rmsnorm(x, r, w, 1e-6, rounding=oracle.RNE)
    bias = oracle.magnitude_bias(oracle.bf16_to_f64(ro_t), oracle.bf16_to_f64(ro_r))
    frac = float((ro_t != ro_r).mean())
    return bias, frac


def pin_page_rounding_mode_experiment(orc):
    pv = page_values()["rounding_mode_experiment"]
    for i, case in enumerate(pv["cases"]):
        bias, frac = rounding_mode_experiment(orc, case["rows"], case["x_std"],
                                              case["residual_std"], seed=100 + i)
        assert abs(bias - case["bias"]) <= pv["bias_rel_tol"] * abs(case["bias"]), \
            (case, bias)
        lo, hi = pv["differing_fraction_range"]
        # The page rounds the fraction to whole percent; allow half a point.
        assert lo - 0.005 <= frac <= hi + 0.005, (case, frac)


def chain_experiment(orc, rows, hidden, depth, delta_std, w_std, seed, init="normal",
                     record=(24, 48, 72)):
    """Section 2 of the page's script: feed residual_out back ``depth`` times
    through a truncating and a nearest-even oracle (and a binary64 stream that
    never rounds).  Returns per recorded step: RMS ratio trunc/rne, out cosine
    similarity trunc vs rne, and the RMS drifts of both against binary64."""
    h0 = synth.bf16_normal(seed, synth.STREAM_RESIDUAL, (rows, hidden), 0.0, 1.0)
    w = synth.bf16_normal(seed, synth.STREAM_WEIGHT, (hidden,), 1.0, w_std)
    res_t = h0.copy()
    res_r = h0.copy()
    res64 = oracle.bf16_to_f64(h0)
    rec = {}
    for step in range(depth):
        delta = synth.chain_delta(seed, step, rows, hidden, delta_std)
        out_t, res_t = orc.add_rmsnorm(delta, res_t, w, 1e-6, rounding=oracle.TRUNC)
        out_r, res_r = orc.add_rmsnorm(delta, res_r, w, 1e-6, rounding=oracle.RNE)
        res64 = oracle.chain_fp64_step(res64, delta)
        if step + 1 in record:
            rms_t = oracle.rms(oracle.bf16_to_f64(res_t))
            rms_r = oracle.rms(oracle.bf16_to_f64(res_r))
            rms64 = oracle.rms(res64)
            rec[step + 1] = dict(
                ratio=rms_t / rms_r,
                cos=oracle.cosine_similarity(oracle.bf16_to_f64(out_t),
                                             oracle.bf16_to_f64(out_r)),
                drift_rne=rms_r / rms64 - 1.0,
                drift_trunc=rms_t / rms64 - 1.0,
                bias_rne=oracle.ratio_bias(oracle.bf16_to_f64(res_r), res64),
            )
    return rec


def pin_page_chain_experiment(orc):
    pv = page_values()["chain_experiment"]
    rec = chain_experiment(orc, pv["rows"], pv["hidden"], pv["depth"], pv["delta_std"],
                           pv["w_std"], seed=200)
    for i, k in enumerate(pv["after"]):
        assert abs(rec[k]["ratio"] - pv["ratio"][i]) <= pv["ratio_abs_tol"], (k, rec[k])
        assert abs(rec[k]["cos"] - pv["cos_sim"][i]) <= pv["cos_sim_abs_tol"], (k, rec[k])
    return rec


FAST_PINS = [pin_constant_rows, pin_eps_inside_sqrt_after_mean, pin_one_hot_rows,
             pin_zero_rows, pin_zero_row_eps_zero, pin_power_of_two_scaling,
             pin_exact_rationals_small_rows, pin_special_values]
