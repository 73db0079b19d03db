"""Pins for the oracle's quantised variant (CPU only).

Per-row symmetric int8: scale = amax / 127, q = nearest-even(y * (127/amax))
in [-127, 127], decided in binary32 from the binary64 y.  The pins are closed
forms (constant and one-hot rows), the documented special-value rules, and
invariants any correct quantiser satisfies (range, the row maximum at +-127,
dequantisation error within half a step, no bias).  Copies of the oracle
with planted mistakes must fail at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle_pins import bits16_to_f32, f32_to_bits16_exact, random_bf16_weights


def pin_constant_rows_constant_weight(orc):
    for h in (64, 4096):
        for c in (1.0, -3.5, 2.0 ** 20):
            for W in (1.0, 0.375, -2.0):
                x = np.full((2, h), f32_to_bits16_exact([c])[0], np.uint16)
                r = np.zeros_like(x)
                w = np.full(h, f32_to_bits16_exact([W])[0], np.uint16)
                q, sc, ro = orc.add_rmsnorm_quant(x, r, w, 1e-6)
                sign = 1 if c * W > 0 else -1
                assert (q == 127 * sign).all(), (h, c, W)
                assert abs(sc[0] - abs(W) / 127) <= 1e-4 * abs(W) / 127
                assert np.array_equal(ro, x)


def pin_constant_rows_varied_weight(orc):
    rng = np.random.default_rng(21)
    h = 512
    w = random_bf16_weights(rng, h, 0.25, 2.0)
    wf = bits16_to_f32(w).astype(np.float64)
    wmax = np.abs(wf).max()
    x = np.full((1, h), f32_to_bits16_exact([1.5])[0], np.uint16)
    q, sc, _ = orc.add_rmsnorm_quant(x, np.zeros_like(x), w, 1e-6)
    checked = 0
    for j in range(h):
        t = Fraction(127) * Fraction(float(wf[j])) / Fraction(float(wmax))
        frac = t - math.floor(t)
        if abs(frac - Fraction(1, 2)) < Fraction(1, 100):
            continue  # too close to a tie for the binary32 decision to be fixed
        assert q[0, j] == round(t), (j, float(t), q[0, j])
        checked += 1
    assert checked > 0.9 * h


def pin_one_hot_rows(orc):
    rng = np.random.default_rng(22)
    for h in (1024, 16384):
        w = random_bf16_weights(rng, h)
        for k in (0, h // 3, h - 1):
            for a in (16.0, -16.0):
                x = np.zeros((1, h), np.uint16)
                x[0, k] = f32_to_bits16_exact([a])[0]
                q, sc, _ = orc.add_rmsnorm_quant(x, np.zeros_like(x), w, 1e-6)
                wk = float(bits16_to_f32(w[k]))
                assert q[0, k] == (127 if a * wk > 0 else -127)
                assert (np.delete(q[0], k) == 0).all()
                expect = math.sqrt(h) * abs(wk) / 127
                assert abs(sc[0] - expect) <= 1e-4 * expect


def pin_special_rows(orc):
    h = 64
    w = synth.to_bf16_bits(np.linspace(0.5, 2.0, h))
    one = f32_to_bits16_exact([1.0])[0]
    z = np.zeros((1, h), np.uint16)
    # zero row: scale 0, codes 0
    q, sc, _ = orc.add_rmsnorm_quant(z, z, w, 1e-6)
    assert sc[0] == 0 and (q == 0).all()
    # NaN in the row: scale NaN, codes 0
    x = np.full((1, h), one, np.uint16)
    x[0, 3] = 0x7FC1
    q, sc, _ = orc.add_rmsnorm_quant(x, z, w, 1e-6)
    assert math.isnan(sc[0]) and (q == 0).all()
    # +Inf in the row: rinv = 0, y = NaN there -> scale NaN, codes 0
    x[0, 3] = 0x7F80
    q, sc, _ = orc.add_rmsnorm_quant(x, z, w, 1e-6)
    assert math.isnan(sc[0]) and (q == 0).all()
    # sum of squares beyond fp32 with finite acc: y = +-0 -> scale 0, codes 0
    x = np.full((1, h), f32_to_bits16_exact([2.0 ** 70])[0], np.uint16)
    q, sc, _ = orc.add_rmsnorm_quant(x, z, w, 1e-6)
    assert sc[0] == 0 and (q == 0).all()
    # A row whose amax is below 2^-120 (subnormal inputs, eps dominating) has
    # no finite inverse scale: codes 0, scale amax / 127 (tiny, nonzero).  Just
    # above the threshold the row is quantised as usual.
    x = np.full((1, h), 0x0001, np.uint16)           # 2^-133: acc = 2^-132, y ~ 2^-122
    q, sc, _ = orc.add_rmsnorm_quant(x, x, w, 1e-6)
    assert 0 < sc[0] < 2.0 ** -120 / 127 and (q == 0).all()
    x = np.full((1, h), 0x0100, np.uint16)           # 2^-125: y ~ 2^-115
    q, sc, _ = orc.add_rmsnorm_quant(x, z, w, 1e-6)
    assert sc[0] > 2.0 ** -120 / 127 and np.abs(q).max() == 127


def pin_random_rows_invariants(orc):
    x, r, w = synth.workload(23, 256, 4096)
    q, sc, ro, y = orc.add_rmsnorm_quant(x, r, w, 1e-6, want_exact=True)
    out, ro2 = orc.add_rmsnorm(x, r, w, 1e-6)
    assert np.array_equal(ro, ro2)
    assert (np.abs(q.astype(np.int32)) <= 127).all()
    assert (np.abs(q).max(axis=1) == 127).all()           # the row maximum maps to +-127
    s = sc.astype(np.float64)[:, None]
    err = q * s - y
    assert (np.abs(err) <= s * (0.5 + 1e-5)).all()        # within half a step
    steps = q - y / s                                      # signed error in steps
    n = steps.size
    assert abs(steps.mean()) < 5 * 0.29 / math.sqrt(n)    # unbiased (uniform error, sd ~0.29)
    big = np.abs(y) > s
    assert (np.sign(q[big]) == np.sign(y[big])).all()
    # scale = amax / 127 to fp32 accuracy
    amax = np.abs(y).max(axis=1)
    assert np.allclose(sc, amax / 127, rtol=2e-7, atol=0)


PINS = [pin_constant_rows_constant_weight, pin_constant_rows_varied_weight, pin_one_hot_rows,
        pin_special_rows, pin_random_rows_invariants]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_quant_pin(orc, pin):
    pin(orc)


QUANT_MUTATIONS = {
    "truncating_codes": ("float t = nearbyintf(y32 * inv);", "float t = truncf(y32 * inv);"),
    "no_tiny_row_rule": ("isfinite(amax) && amax >= ldexpf(1.0f, -120)",
                         "isfinite(amax) && amax > 0.0f"),
    "scale_128": ("const float sc = amax / 127.0f;", "const float sc = amax / 128.0f;"),
    "inverse_128": ("const float inv = 127.0f / amax;", "const float inv = 128.0f / amax;"),
    "max_without_abs": ("amax = max_nan(amax, fabsf((float)y));",
                        "amax = max_nan(amax, (float)y);"),
    "scale_from_rms": ("const float inv = 127.0f / amax;",
                       "const float inv = 127.0f * (float)rinv;"),
    "codes_from_acc": ("float y32 = (float)((a * rinv) * (double)bf16_to_f32(weight[j]));",
                       "float y32 = (float)(a * rinv);"),
}


@pytest.mark.parametrize("name", sorted(QUANT_MUTATIONS))
def test_quant_pins_catch_planted_mistake(tmp_path, name):
    old, new = QUANT_MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert old in src, name
    path = tmp_path / (name + ".c")
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / ("lib" + name + ".so"))
    oracle.compile_library(str(path), lib)
    mut = oracle.Oracle(lib)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mut)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught %s" % name
