"""Pins for the oracle's FP8 E4M3 quantised variant (CPU only).

The aiter issue's quantised configurations cast out to int8, fp8 or fp4 with a
per-row scale ("Cost of fixing").  The fp8 reading: OCP E4M3 ("e4m3fn", largest
finite 448, no infinities), scale = amax / 448 and code = nearest-even E4M3 of
y * (448/amax), saturating at +-448, decided in binary32 from the binary64 y.

The converter is pinned to torch's own CPU float8_e4m3fn cast (an independent
implementation of the same format, below its NaN boundary at 464), to the
format's printed landmarks and to exact midpoints.  The quantised rows are
pinned to closed forms (constant and one-hot rows), the special-value rules
and invariants of any correct quantiser.  Copies of the oracle with planted
mistakes must fail at least one pin.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle_pins import bits16_to_f32, f32_to_bits16_exact, random_bf16_weights

# Values fixed by the OCP 8-bit floating point format for E4M3.
LANDMARKS = {
    0.0: 0x00, 2.0 ** -9: 0x01, 7 * 2.0 ** -9: 0x07, 2.0 ** -6: 0x08, 0.5: 0x30,
    1.0: 0x38, 1.125: 0x39, 2.0: 0x40, 240.0: 0x77, 256.0: 0x78, 448.0: 0x7E,
}


def exact_values():
    """The 127 non-negative finite E4M3 values by code, from the format's
    definition (subnormals m * 2^-9, normals (8 + m) * 2^(E - 10))."""
    vals = []
    for code in range(127):
        e, m = code >> 3, code & 7
        vals.append(Fraction(m, 512) if e == 0 else Fraction(8 + m) * Fraction(2) ** (e - 10))
    return vals


def torch_e4m3(v):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(v, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def codes_of(orc, v):
    return np.array([orc.e4m3_rne(float(x)) for x in np.asarray(v, np.float32)], np.int64)


# ------------------------------------------------------------------ converter

def pin_landmarks(orc):
    for v, c in LANDMARKS.items():
        assert orc.e4m3_rne(v) == c, (v, c)
        assert orc.e4m3_rne(-v) == c | 0x80, (-v, c)


def pin_every_value_maps_to_itself_and_midpoints_to_even(orc):
    vals = exact_values()
    for c, v in enumerate(vals):
        assert orc.e4m3_rne(float(v)) == c, c
    for c in range(126):
        mid = (vals[c] + vals[c + 1]) / 2
        fm = np.float32(float(mid))
        assert Fraction(float(fm)) == mid            # midpoints are binary32 numbers
        even = c if c % 2 == 0 else c + 1
        assert orc.e4m3_rne(float(fm)) == even, ("midpoint", c)
        assert orc.e4m3_rne(float(np.nextafter(fm, np.float32(0)))) == c, ("below", c)
        assert orc.e4m3_rne(float(np.nextafter(fm, np.float32(1e9)))) == c + 1, ("above", c)


def pin_agrees_with_torch_cast(orc):
    rng = np.random.default_rng(81)
    mag = np.exp2(rng.uniform(-14, math.log2(463.9), 20000)).astype(np.float32)
    v = np.concatenate([mag, -mag, np.float32(rng.uniform(-2.0 ** -8, 2.0 ** -8, 2000)),
                        np.float32([448.0, 463.99997, -463.99997, 2.0 ** -10, 2.0 ** -149])])
    assert np.array_equal(codes_of(orc, v), torch_e4m3(v).astype(np.int64))


def pin_saturation(orc):
    for v in (464.0, 480.0, 1e6, 3.4e38):
        assert orc.e4m3_rne(v) == 0x7E and orc.e4m3_rne(-v) == 0xFE, v


# ------------------------------------------------------------------ quantised rows

def pin_constant_rows(orc):
    for h in (64, 4096):
        for c in (1.0, -3.5, 2.0 ** 20):
            for W in (1.0, 0.375, -2.0):
                x = np.full((2, h), f32_to_bits16_exact([c])[0], np.uint16)
                w = np.full(h, f32_to_bits16_exact([W])[0], np.uint16)
                q, sc, ro = orc.add_rmsnorm_quant_fp8(x, np.zeros_like(x), w, 1e-6)
                assert (q == (0x7E if c * W > 0 else 0xFE)).all(), (h, c, W)
                assert abs(sc[0] - abs(W) / 448) <= 1e-4 * abs(W) / 448
                assert np.array_equal(ro, x)


def pin_constant_row_varied_weight(orc):
    """acc constant: y_j / amax = w_j / max|w|, so code_j is the nearest E4M3
    value of 448 w_j / max|w|, computed here in exact arithmetic."""
    rng = np.random.default_rng(82)
    h = 512
    w = random_bf16_weights(rng, h, 0.01, 2.0)
    wf = bits16_to_f32(w).astype(np.float64)
    wmax = np.abs(wf).max()
    x = np.full((1, h), f32_to_bits16_exact([1.5])[0], np.uint16)
    q, sc, _ = orc.add_rmsnorm_quant_fp8(x, np.zeros_like(x), w, 1e-6)
    vals = exact_values()
    checked = 0
    for j in range(h):
        t = abs(Fraction(448) * Fraction(float(wf[j])) / Fraction(float(wmax)))
        k = max(i for i, v in enumerate(vals) if v <= t)
        if k == 126:
            nearest = 126
        else:
            lo, hi = t - vals[k], vals[k + 1] - t
            if abs(lo - hi) < (vals[k + 1] - vals[k]) / 100:
                continue  # too close to a tie for the binary32 decision to be fixed
            nearest = k if lo < hi else k + 1
        assert q[0, j] == (nearest | (0x80 if wf[j] < 0 else 0)), (j, float(t), q[0, j])
        checked += 1
    assert checked > 0.9 * h


def pin_one_hot_rows(orc):
    rng = np.random.default_rng(83)
    for h in (1024, 16384):
        w = random_bf16_weights(rng, h)
        for k in (0, h // 3, h - 1):
            for a in (16.0, -16.0):
                x = np.zeros((1, h), np.uint16)
                x[0, k] = f32_to_bits16_exact([a])[0]
                q, sc, _ = orc.add_rmsnorm_quant_fp8(x, np.zeros_like(x), w, 1e-6)
                wk = float(bits16_to_f32(w[k]))
                assert q[0, k] == (0x7E if a * wk > 0 else 0xFE)
                rest = np.delete(q[0], k)
                assert ((rest == 0) | (rest == 0x80)).all()    # signed zeros elsewhere
                expect = math.sqrt(h) * abs(wk) / 448
                assert abs(sc[0] - expect) <= 1e-4 * expect


def pin_special_rows(orc):
    h = 64
    w = synth.to_bf16_bits(np.linspace(0.5, 2.0, h))
    one = f32_to_bits16_exact([1.0])[0]
    z = np.zeros((1, h), np.uint16)
    q, sc, _ = orc.add_rmsnorm_quant_fp8(z, z, w, 1e-6)
    assert sc[0] == 0 and (q == 0).all()
    x = np.full((1, h), one, np.uint16)
    x[0, 3] = 0x7FC1
    q, sc, _ = orc.add_rmsnorm_quant_fp8(x, z, w, 1e-6)
    assert math.isnan(sc[0]) and (q == 0).all()
    x[0, 3] = 0x7F80
    q, sc, _ = orc.add_rmsnorm_quant_fp8(x, z, w, 1e-6)
    assert math.isnan(sc[0]) and (q == 0).all()
    # amax below 2^-118: 448/amax is not finite, codes 0, scale amax/448.
    x = np.full((1, h), 0x0001, np.uint16)              # y ~ 2^-122 .. 2^-121
    q, sc, _ = orc.add_rmsnorm_quant_fp8(x, x, w, 1e-6)
    assert 0 < sc[0] < 2.0 ** -118 / 448 and (q == 0).all()
    x = np.full((1, h), 0x0100, np.uint16)              # y ~ 2^-115
    q, sc, _ = orc.add_rmsnorm_quant_fp8(x, z, w, 1e-6)
    assert sc[0] > 2.0 ** -118 / 448 and (q & 0x7F).max() == 0x7E


def pin_random_rows_invariants(orc):
    x, r, w = synth.workload(84, 256, 4096)
    q, sc, ro, y = orc.add_rmsnorm_quant_fp8(x, r, w, 1e-6, want_exact=True)
    _, ro2 = orc.add_rmsnorm(x, r, w, 1e-6)
    assert np.array_equal(ro, ro2)
    assert ((q & 0x7F) <= 0x7E).all()                    # no NaN codes
    assert ((q & 0x7F).max(axis=1) == 0x7E).all()        # the row maximum maps to +-448
    s = sc.astype(np.float64)[:, None]
    deq = oracle.e4m3_to_f64(q) * s
    t = np.abs(y) / s                                     # y in units of the scale
    # half a step of E4M3 at t: 2^-10 below 2^-6, else 2^(floor(log2 t) - 4)
    half = np.where(t < 2.0 ** -6, 2.0 ** -10, np.exp2(np.floor(np.log2(np.maximum(t, 2.0 ** -6))) - 4))
    assert (np.abs(deq - y) <= s * half * (1 + 1e-5) + s * 448 * 2.0 ** -23).all()
    nz = np.abs(y) > s * 2.0 ** -9
    assert (np.sign(deq[nz]) == np.sign(y[nz])).all()
    rel = (deq - y)[t > 2.0 ** -6] / np.abs(y)[t > 2.0 ** -6]
    assert abs(rel.mean()) < 5 * 0.02 / math.sqrt(rel.size)  # unbiased (sd of rel error < 0.02)
    amax = np.abs(y).max(axis=1)
    assert np.allclose(sc, amax / 448, rtol=2e-7, atol=0)


def pin_plain_matches_zero_residual(orc):
    """Plain RMSNorm (no residual) equals the fused form over an all -0 residual."""
    x, _, w = synth.workload(85, 16, 1024)
    qp, sp, rop = orc.add_rmsnorm_quant_fp8(x, None, w, 1e-6)
    qf, sf, _ = orc.add_rmsnorm_quant_fp8(x, np.full_like(x, 0x8000), w, 1e-6)
    assert rop is None and np.array_equal(qp, qf) and np.array_equal(sp, sf)


PINS = [pin_landmarks, pin_every_value_maps_to_itself_and_midpoints_to_even,
        pin_agrees_with_torch_cast, pin_saturation, pin_constant_rows,
        pin_constant_row_varied_weight, pin_one_hot_rows, pin_special_rows,
        pin_random_rows_invariants, pin_plain_matches_zero_residual]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_fp8_pin(orc, pin):
    pin(orc)


FP8_MUTATIONS = {
    "ties_away": ("(dhi == dlo && (lo & 1))", "(dhi == dlo)"),
    "ties_down": ("(dhi == dlo && (lo & 1))", "(dhi == dlo && 0)"),
    "truncating": ("if (dhi < dlo || (dhi == dlo && (lo & 1))) code = lo + 1;", ""),
    "subnormal_step": ("if (e == 0) return ldexp((double)m, -9);",
                       "if (e == 0) return ldexp((double)m, -10);"),
    "bias_8": ("return ldexp(1.0 + m / 8.0, e - 7);", "return ldexp(1.0 + m / 8.0, e - 8);"),
    "saturate_at_240": ("if (a >= 448.0) return sign | 0x7E;", "if (a >= 240.0) return sign | 0x77;"),
    "sign_dropped": ("const int sign = signbit(v) ? 0x80 : 0;", "const int sign = 0;"),
    "scale_240": ("const float sc = amax / 448.0f;", "const float sc = amax / 240.0f;"),
    "inverse_240": ("const float inv = 448.0f / amax;", "const float inv = 240.0f / amax;"),
    "no_tiny_row_rule": ("isfinite(amax) && amax >= ldexpf(1.0f, -118)",
                         "isfinite(amax) && amax > 0.0f"),
    "codes_without_weight": (
        "float y32 = (float)((a * rinv) * (double)bf16_to_f32(weight[j]));\n"
        "        code = (uint8_t)orc_e4m3_rne(y32 * inv);",
        "float y32 = (float)(a * rinv);\n        code = (uint8_t)orc_e4m3_rne(y32 * inv);"),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTATIONS))
def test_fp8_pins_catch_planted_mistake(tmp_path, name):
    old, new = FP8_MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, name
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


def test_decoder_matches_the_format_definition():
    """oracle.e4m3_to_f64, used by the invariants above, against the values
    listed from the definition, for all 256 codes."""
    vals = exact_values()
    dec = oracle.e4m3_to_f64(np.arange(256))
    for c in range(256):
        mag = c & 0x7F
        if mag == 0x7F:
            assert math.isnan(dec[c])
            continue
        v = float(vals[mag])
        assert dec[c] == (-v if c & 0x80 else v) and math.copysign(1, dec[c]) == (-1 if c & 0x80 else 1), c
