"""Pins for the fused oracle (CPU only), and proof that they bite.

The pins themselves live in tests/oracle_pins.py.  Here they run against the
oracle, and against copies of its C source with one plausible mistake planted
in each: every planted mistake must fail at least one pin.
"""
import pytest

import oracle
import oracle_pins as P


@pytest.mark.parametrize("pin", P.FAST_PINS, ids=lambda f: f.__name__)
def test_fast_pin(orc, pin):
    pin(orc)


def test_magnitude_bias_metric():
    P.pin_magnitude_bias_metric()


def test_page_rounding_mode_experiment(orc):
    P.pin_page_rounding_mode_experiment(orc)


def test_page_chain_experiment(orc):
    rec = P.pin_page_chain_experiment(orc)
    # Nearest-even keeps the residual stream within 0.1% of the binary64 stream
    # after 72 calls; truncation drifts far past that (the page: -8.98%
    # relative to nearest-even).
    assert abs(rec[72]["drift_rne"]) <= 1e-3, rec[72]
    assert rec[72]["drift_trunc"] < -0.05, rec[72]


def test_chain_gate_separates_rounding_modes(orc):
    # The long-chain workload's distributions (fresh x ~ N(0, 0.1^2) per call,
    # weight 1 + 0.1 N(0,1)) at 256 rows: the 0.1% RMS-drift gate passes
    # nearest-even and fails truncation.
    rec = P.chain_experiment(orc, rows=256, hidden=4096, depth=72, delta_std=0.1,
                             w_std=0.1, seed=300)
    assert abs(rec[72]["drift_rne"]) <= 1e-3, rec[72]
    assert abs(rec[72]["drift_trunc"]) > 1e-3, rec[72]


def test_zero_rows_and_bad_arguments(orc):
    import numpy as np

    x = np.zeros((0, 64), dtype=np.uint16)
    out, ro = orc.add_rmsnorm(x, x, np.zeros(64, dtype=np.uint16))
    assert out.shape == (0, 64) and ro.shape == (0, 64)
    with pytest.raises(ValueError):
        orc.add_rmsnorm(np.zeros((2, 8), np.uint16), np.zeros((2, 8), np.uint16),
                        np.zeros(8, np.uint16), rounding=7)


# ------------------------------------------------------------------ planted mistakes

FUSED_MUTATIONS = {
    "divisor_h_minus_1": ("s / (double)hidden", "s / (double)(hidden - 1)"),
    "eps_outside_sqrt": ("1.0 / sqrt(s / (double)hidden + (double)eps)",
                         "1.0 / sqrt(s / (double)hidden) + (double)eps"),
    "eps_dropped": ("+ (double)eps)", ")"),
    "abs_not_square": ("s += a * a;", "s += fabs(a);"),
    "sqrt_not_rsqrt": ("1.0 / sqrt(", "sqrt("),
    "weight_shifted": ("weight[j]", "weight[(j + 1) % hidden]"),
    "acc_from_x_only": ("double a = (double)row_acc(xr, rr, j);",
                        "double a = (double)row_acc(xr, NULL, j);"),
    "out_truncated": ("orc_rne16_from_f64(y)", "orc_trunc16(f32_bits((float)y))"),
    "residual_out_truncated": ("ro[j] = rounding == ORC_RNE ? orc_rne16(ab)",
                               "ro[j] = rounding == ORC_RNE ? orc_trunc16(ab)"),
    "no_overflow_emulation": ("if (s >= f32_overflow) s = INFINITY;", ""),
    "rne16_ties_away": ("(u + 0x7FFFu + ((u >> 16) & 1u)) >> 16", "(u + 0x8000u) >> 16"),
    "f64_round_via_float": ("return (uint16_t)(sign | (f32_bits((float)r) >> 16));",
                            "return orc_rne16(f32_bits((float)y));"),
}


def _mutant_oracle(tmp_path, name):
    old, new = FUSED_MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert old in src, "mutation anchor missing for %s" % name
    path = tmp_path / (name + ".c")
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / ("lib" + name + ".so"))
    oracle.compile_library(str(path), lib)
    return oracle.Oracle(lib)


@pytest.mark.parametrize("name", sorted(FUSED_MUTATIONS))
def test_pins_catch_planted_mistake(tmp_path, name):
    mut = _mutant_oracle(tmp_path, name)
    failed = []
    for pin in P.FAST_PINS + [P.pin_page_rounding_mode_experiment]:
        try:
            pin(mut)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake %s" % name
