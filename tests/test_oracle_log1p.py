"""Pins for the log1p oracle (CPU only).

The oracle's binary32 log1p must be ln(1 + x) rounded once to the nearest
binary32.  It is pinned to things other than itself:
  * the IEEE 754 special cases of log1p;
  * Python's decimal module (an independent arbitrary-precision ln, correctly
    rounded at its context precision) at 60 digits, on inputs spread over
    every binade of the domain, rounded to binary32 in exact rational
    arithmetic;
  * the closed form log1p(2^k - 1) = k ln 2;
  * log1p(x) = x after rounding for |x| <= 2^-25 (the x^2/2 term is below
    half a quantum);
  * the hardest inputs of a scan, those whose binary64 value lies within
    2^-20 quanta of a binary32 midpoint, decided by decimal;
  * monotonicity on a dense sweep.
The fast variant (binary64 with escalation to binary128) must equal the
binary128 one, and must escalate exactly on the near-midpoint inputs.
Copies of the oracle with planted mistakes fail at least one pin.
"""
from decimal import Context, Decimal
from fractions import Fraction

import numpy as np
import pytest

import oracle

F32 = np.float32
ADD_CTX = Context(prec=400)   # exact 1 + x for every binary32 x
LN_CTX = Context(prec=60)


def decimal_log1p(x: float) -> Decimal:
    return LN_CTX.ln(ADD_CTX.add(Decimal(1), Decimal(float(x))))


def round_to_f32(d: Decimal) -> np.float32:
    """Nearest binary32 (ties to even) of the decimal value d, decided in
    exact rational arithmetic."""
    exact = Fraction(d)
    c = F32(float(d))
    cands = [np.nextafter(c, F32(-np.inf)), c, np.nextafter(c, F32(np.inf))]
    best = None
    for v in cands:
        if not np.isfinite(v):
            continue
        dist = abs(Fraction(float(v)) - exact)
        key = (dist, int(np.array([v]).view(np.uint32)[0]) & 1)   # ties: even significand
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def spread_inputs(rng, n):
    """Positive inputs log-uniform over every binade, negative ones near 0
    and near -1, and small integers."""
    pos = (2.0 ** rng.uniform(-149, 127.9, n)).astype(np.float32)
    neg_small = -(2.0 ** rng.uniform(-149, -1, n // 2)).astype(np.float32)
    near_m1 = (-1.0 + 2.0 ** rng.uniform(-24, -1, n // 2)).astype(np.float32)
    ints = np.arange(1, 200, dtype=np.float32)
    x = np.concatenate([pos, neg_small, near_m1, ints])
    return x[(x > -1) & np.isfinite(x)]


def pin_special_values(o):
    x = np.array([0.0, -0.0, -1.0, -1.5, -np.inf, np.inf, np.nan, -3e38], np.float32)
    r = o.log1p_f32(x)
    assert bits(r[0]) == 0 and bits(r[1]) == 0x80000000
    assert r[2] == -np.inf
    assert np.isnan(r[3]) and np.isnan(r[4]) and np.isnan(r[7])
    assert r[5] == np.inf and np.isnan(r[6])
    f, _ = o.log1p_f32_fast(x)
    assert np.array_equal(bits(f)[~np.isnan(f)], bits(r)[~np.isnan(r)])
    assert np.array_equal(np.isnan(f), np.isnan(r))


def pin_decimal_brute_force(o):
    rng = np.random.default_rng(61)
    x = spread_inputs(rng, 1500)
    r = o.log1p_f32(x)
    for xi, ri in zip(x, r):
        expect = round_to_f32(decimal_log1p(xi))
        assert bits(ri) == bits(expect), (float(xi), float(ri), float(expect))


def pin_powers_of_two_minus_one(o):
    ln2 = LN_CTX.ln(Decimal(2))
    xs, expect = [], []
    for k in range(1, 25):
        xs.append(F32(2.0 ** k - 1))               # exact in binary32 for k <= 24
        expect.append(round_to_f32(LN_CTX.multiply(k, ln2)))
        xs.append(F32(2.0 ** -k - 1))              # 1 + x = 2^-k
        expect.append(round_to_f32(LN_CTX.multiply(-k, ln2)))
    r = o.log1p_f32(np.array(xs, np.float32))
    assert np.array_equal(bits(r), bits(np.array(expect, np.float32)))


def pin_tiny_inputs_round_to_themselves(o):
    rng = np.random.default_rng(62)
    mags = (2.0 ** rng.uniform(-149, -25, 2000)).astype(np.float32)
    x = np.concatenate([mags, -mags, np.array([2.0 ** -149, -(2.0 ** -149), 2.0 ** -126],
                                              np.float32)])
    r = o.log1p_f32(x)
    assert np.array_equal(bits(r), bits(x))


def near_midpoint_inputs(lo_bits, count):
    """Inputs among `count` consecutive binary32 patterns from lo_bits whose
    binary64 log1p lies within 2^-20 quanta of a binary32 midpoint."""
    x = (np.arange(count, dtype=np.uint64) + lo_bits).astype(np.uint32).view(np.float32)
    y = np.log1p(x.astype(np.float64))
    r = y.astype(np.float32)
    q = np.spacing(np.abs(r)).astype(np.float64)
    d = np.abs(np.abs(y - r.astype(np.float64)) - q / 2) / q
    return x[d < 2.0 ** -20]


HARD_SCANS = [(0x3F800000, 1 << 21), (0x3E000000, 1 << 21), (0xBF000000, 1 << 21),
              (0x4B000000, 1 << 20)]


def pin_hardest_cases_of_a_scan(o):
    hard = np.concatenate([near_midpoint_inputs(lo, n) for lo, n in HARD_SCANS])
    assert hard.size >= 4, hard.size
    r = o.log1p_f32(hard)
    for xi, ri in zip(hard, r):
        d = decimal_log1p(xi)
        expect = round_to_f32(d)
        assert bits(ri) == bits(expect), (float(xi), float(ri), float(expect))
    f, esc = o.log1p_f32_fast(hard)
    assert esc == hard.size                       # every one decided in binary128
    assert np.array_equal(bits(f), bits(r))


def pin_fast_equals_quad(o):
    rng = np.random.default_rng(63)
    x = np.concatenate([spread_inputs(rng, 20000),
                        rng.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(
                            np.uint32).view(np.float32)])
    q = o.log1p_f32(x)
    f, _ = o.log1p_f32_fast(x, threads=4)
    nan = np.isnan(q)
    assert np.array_equal(nan, np.isnan(f))
    assert np.array_equal(bits(f)[~nan], bits(q)[~nan])


def pin_monotone_dense_sweep(o):
    for lo in (0x3F7FF000, 0x00000000, 0xBF7FF000 - 4096, 0x7F7FF000):
        u = np.arange(lo, lo + 8192, dtype=np.uint64).astype(np.uint32)
        x = u.view(np.float32)
        x = np.sort(x[np.isfinite(x) & (x > -1)])
        r, _ = o.log1p_f32_fast(x)
        assert (np.diff(r.astype(np.float64)) >= 0).all()


PINS = [pin_special_values, pin_decimal_brute_force, pin_powers_of_two_minus_one,
        pin_tiny_inputs_round_to_themselves, pin_hardest_cases_of_a_scan, pin_fast_equals_quad,
        pin_monotone_dense_sweep]


@pytest.fixture(scope="module")
def lo():
    return oracle.default_log1p()


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_log1p_pin(lo, pin):
    with np.errstate(all="ignore"):
        pin(lo)


def test_f64_reference_is_within_half_a_binary64_ulp_of_decimal(lo):
    rng = np.random.default_rng(64)
    x = spread_inputs(rng, 300)
    y = lo.log1p_f64(x)
    for xi, yi in zip(x, y):
        d = Fraction(decimal_log1p(xi))
        assert abs(Fraction(float(yi)) - d) <= Fraction(np.spacing(abs(yi))) / 2 * (1 + 1e-9)


def test_ulp_error_metric_hand_example():
    # ref 1.0: eps = 2^-23, so got = 1 + 2^-23 is one unit; 1 + 2^-24 half a unit
    got = np.array([1.0 + 2.0 ** -23, 1.0 + 2.0 ** -24, 1.0])
    assert np.allclose(oracle.ulp_error_f32(got, np.ones(3)), [1.0, 0.5, 0.0])


def test_rejects_bad_arguments(lo):
    assert lo.lib.orc_log1p_f32(None, None, -1) == -1
    assert lo.lib.orc_log1p_f32(None, None, 0) == 0


LOG1P_MUTATIONS = {
    "log_of_one_plus_x": ("log1pq((__float128)x)", "logq(1 + (__float128)x)"),
    "zero_loses_sign": ("*r = x; /* keeps the sign of zero */", "*r = 0.0f;"),
    "minus_one_is_nan": ("*r = -INFINITY;", "*r = NAN;"),
    "fast_never_escalates": ("ldexp(fabs(y), -36)", "ldexp(fabs(y), -80)"),
    "fast_checks_one_side": ("return fabs(y - m_lo) <= tol || fabs(y - m_hi) <= tol;",
                             "return fabs(y - m_hi) <= tol;"),
    "fast_rounds_toward_zero": ("r = (float)y;\n      if (isinf(r)",
                                "r = nextafterf((float)y, 0.0f);\n      if (isinf(r)"),
}


@pytest.mark.parametrize("name", sorted(LOG1P_MUTATIONS))
def test_log1p_pins_catch_planted_mistake(tmp_path, name):
    old, new = LOG1P_MUTATIONS[name]
    src = open(oracle.LOG1P_SOURCE).read()
    assert old in src, name
    path = tmp_path / (name + ".c")
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / ("lib" + name + ".so"))
    oracle.compile_log1p_library(str(path), lib)
    mut = oracle.Log1pOracle(lib)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mut)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught %s" % name
