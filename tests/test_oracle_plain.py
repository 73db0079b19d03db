"""Pins for the oracle's plain RMSNorm (no residual add), CPU only.

Plain RMSNorm is the fused computation with acc = fp32(x) and no
residual_out.  It is pinned to:
  * exact rational arithmetic on small rows (acc = x, S = sum x^2 exactly,
    out = nearest-even bf16 of x w / sqrt(S / H + eps));
  * IEEE's x + (-0) = x for every x, signed zeros included: plain RMSNorm must
    equal the already pinned fused op with a residual of all -0, bit for bit,
    in both the bf16 and the int8 variant;
  * signed zeros passing through: a -0 input gives a zero out whose sign is
    that of -0 * w;
  * closed forms on constant and one-hot rows.
Copies of the oracle with planted mistakes in the plain branch must fail at
least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle_pins import (_exact_round_quotient, _near_tie_rows, _random_small_rows,
                         bits16_to_f32, f32_to_bits16_exact, is_nan16, random_bf16_weights)

NEG_ZERO = 0x8000


def pin_plain_exact_rationals_small_rows(orc):
    rng = np.random.default_rng(41)
    cases = [(x, w, eps) for x, _r, w, eps in _random_small_rows(rng)]
    cases += [(x, w, eps) for x, _r, w, eps in _near_tie_rows()]
    for row, (x, w, eps) in enumerate(cases):
        h = x.shape[0]
        out, y = orc.rmsnorm(x[None], w, eps, want_exact=True)
        accq = [Fraction(float(a)) for a in bits16_to_f32(x)]
        v = sum(a * a for a in accq) / h + Fraction(eps)
        for j in range(h):
            t = accq[j] * Fraction(float(bits16_to_f32(w[j])))
            expect = _exact_round_quotient(t, v)
            assert out[0, j] == expect, (h, row, j, hex(out[0, j]), hex(expect))
            exact = float(t) / float(v) ** 0.5
            assert abs(y[0, j] - exact) <= 1e-12 * abs(exact) + 1e-300


def _rows_with_specials(rng, n, h):
    x = synth.to_bf16_bits(rng.standard_normal((n, h)))
    x[0, :] = 0                                  # an all +0 row
    x[1, :] = NEG_ZERO                           # an all -0 row
    x[2, ::3] = NEG_ZERO                         # scattered -0 and +0
    x[2, 1::3] = 0
    x[3, 5] = 0x7FC1                             # NaN
    x[4, 7] = 0x7F80                             # +Inf
    x[5, :] = 0x0001                             # the smallest subnormal
    x[6, :] = f32_to_bits16_exact([2.0 ** 70])[0]  # sum of squares beyond fp32
    x[6, ::2] |= 0x8000
    x[7, :] = 0x7F7F                             # the largest bf16
    return x


def pin_plain_equals_fused_with_negative_zero_residual(orc):
    rng = np.random.default_rng(42)
    for h in (8, 64, 1000, 4096):
        x = _rows_with_specials(rng, 12, h)
        w = random_bf16_weights(rng, h)
        r = np.full_like(x, NEG_ZERO)
        for eps in (1e-6, 0.0):
            out, y = orc.rmsnorm(x, w, eps, want_exact=True)
            fo, fro, fy = orc.add_rmsnorm(x, r, w, eps, want_exact=True)
            assert np.array_equal(fro[~is_nan16(x)], x[~is_nan16(x)])   # x + (-0) = x
            assert np.array_equal(out, fo), (h, eps)
            assert np.array_equal(np.isnan(y), np.isnan(fy))
            assert np.array_equal(y[~np.isnan(y)].view(np.uint64),
                                  fy[~np.isnan(fy)].view(np.uint64))
            q, sc = orc.rmsnorm_quant(x, w, eps)
            fq, fsc, _ = orc.add_rmsnorm_quant(x, r, w, eps)
            assert np.array_equal(q, fq), (h, eps)
            assert np.array_equal(np.isnan(sc), np.isnan(fsc))
            assert np.array_equal(sc[~np.isnan(sc)].view(np.uint32),
                                  fsc[~np.isnan(fsc)].view(np.uint32))


def pin_plain_signed_zeros(orc):
    h = 24
    w = synth.to_bf16_bits(np.linspace(-2.0, 2.0, h))
    w[w == 0] = f32_to_bits16_exact([0.5])[0]
    x = np.full((2, h), f32_to_bits16_exact([1.0])[0], np.uint16)
    zeros = np.arange(0, h, 2)
    x[0, zeros] = NEG_ZERO
    x[1, zeros] = 0
    out = orc.rmsnorm(x, w, 1e-6)
    wneg = (w & 0x8000) != 0
    # -0 * rinv * w is -0 for w > 0 and +0 for w < 0; +0 the other way round.
    expect_neg = np.where(wneg[zeros], 0, NEG_ZERO)
    expect_pos = np.where(wneg[zeros], NEG_ZERO, 0)
    assert np.array_equal(out[0, zeros], expect_neg)
    assert np.array_equal(out[1, zeros], expect_pos)


def pin_plain_constant_and_one_hot(orc):
    rng = np.random.default_rng(43)
    for h in (64, 1024, 16384):
        w = random_bf16_weights(rng, h)
        # constant c: acc / rms = sign(c) (up to eps), out = sign(c) * w
        for c in (1.5, -3.0, 2.0 ** -20):
            x = np.full((1, h), f32_to_bits16_exact([c])[0], np.uint16)
            out = orc.rmsnorm(x, w, 0.0 if c < 1e-3 else 1e-6)
            expect = w ^ (0x8000 if c < 0 else 0)
            assert np.array_equal(out[0], expect), (h, c)
        # one-hot a at k: y_k = sign(a) sqrt(h) w_k (h is a power of 4, so
        # that is exact up to eps); +0 elsewhere times w: zeros with w's sign.
        k = h // 3
        x = np.zeros((1, h), np.uint16)
        x[0, k] = f32_to_bits16_exact([16.0])[0]
        out = orc.rmsnorm(x, w, 1e-9)
        root = int(round(h ** 0.5))
        wk = float(bits16_to_f32(w[k]))
        assert out[0, k] == f32_to_bits16_exact([root * wk])[0], (h, k)
        rest = np.delete(np.arange(h), k)
        assert np.array_equal(out[0, rest], w[rest] & 0x8000)
    # quantised: a constant row maps to +-127 everywhere with constant weight
    w = np.full(256, f32_to_bits16_exact([0.75])[0], np.uint16)
    x = np.full((1, 256), f32_to_bits16_exact([-2.0])[0], np.uint16)
    q, sc = orc.rmsnorm_quant(x, w, 1e-6)
    assert (q == -127).all() and abs(sc[0] - 0.75 / 127) <= 1e-6 * 0.75 / 127


PLAIN_PINS = [pin_plain_exact_rationals_small_rows,
              pin_plain_equals_fused_with_negative_zero_residual, pin_plain_signed_zeros,
              pin_plain_constant_and_one_hot]


@pytest.mark.parametrize("pin", PLAIN_PINS, ids=lambda f: f.__name__)
def test_plain_pin(orc, pin):
    with np.errstate(all="ignore"):
        pin(orc)


def test_plain_rejects_half_given_residual(orc):
    # residual and residual_out are both given or both absent
    lib = orc.lib
    x = np.zeros((1, 8), np.uint16)
    out = np.empty_like(x)
    rc = lib.orc_add_rmsnorm(out.ctypes.data, None, None, x.ctypes.data, x.ctypes.data,
                             x[0].ctypes.data, 1, 8, 1e-6, 0)
    assert rc == -1


PLAIN_MUTATIONS = {
    "plain_adds_zero": ("if (!rr) return bf16_to_f32(xr[j]);",
                        "if (!rr) return bf16_to_f32(xr[j]) + 0.0f;"),
    "plain_neighbour_element": ("if (!rr) return bf16_to_f32(xr[j]);",
                                "if (!rr) return bf16_to_f32(xr[j ? j - 1 : 0]);"),
    "plain_doubles_x": ("if (!rr) return bf16_to_f32(xr[j]);",
                        "if (!rr) return bf16_to_f32(xr[j]) + bf16_to_f32(xr[j]);"),
}


@pytest.mark.parametrize("name", sorted(PLAIN_MUTATIONS))
def test_plain_pins_catch_planted_mistake(tmp_path, name):
    old, new = PLAIN_MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert old in src, name
    path = tmp_path / (name + ".c")
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / ("lib" + name + ".so"))
    oracle.compile_library(str(path), lib)
    mut = oracle.Oracle(lib)
    failed = []
    for pin in PLAIN_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mut)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught %s" % name
