"""Pins for the oracle's bf16 converters (CPU only).

The converters are checked against things other than themselves: the hand
cases in tests/golden/rne_hand_cases.txt, two independent formulations over
every fp32 bit pattern (exhaustive C checker), torch's CPU .to(torch.bfloat16)
(the round-to-nearest-even reference that the aiter issue "rmsnorm2d_fwd_with_add
truncates fp32->bf16 on gfx942, ..." compares against), and exact rational
rounding for the binary64 converter.  Planted mistakes must make them fail.
"""
import os
import random
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _is_nan16(b):
    return (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0


def _hand_cases():
    cases = []
    with open(os.path.join(GOLDEN, "rne_hand_cases.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            cases.append((int(parts[0], 16), parts[1]))
    return cases


@pytest.mark.parametrize("u,expected", _hand_cases())
def test_rne_hand_cases(orc, u, expected):
    got = orc.rne16(u)
    if expected == "nan":
        assert _is_nan16(got) and (got >> 15) == (u >> 31), hex(got)
    else:
        assert got == int(expected, 16), "%08x -> %04x, expected %s" % (u, got, expected)
    # The binary64 converter must agree on every value that fp32 can hold.
    f = np.array([u], dtype=np.uint32).view(np.float32)[0]
    g64 = orc.rne16_from_f64(float(f))
    if expected == "nan":
        assert _is_nan16(g64)
    else:
        assert g64 == int(expected, 16)


def test_rne_value_readback(orc):
    # bf16 1.0 must read back as 1.0 (not as the integer 16256 = 0x3F80).
    b = orc.rne16(0x3F800000)
    val = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
    assert val == 1.0


def test_truncation_control_is_truncation(orc):
    for u in (0x3F80FFFF, 0xBF80FFFF, 0x3F818000, 0x7F7FFFFF):
        assert orc.trunc16(u) == u >> 16


@pytest.mark.slow
def test_rne_exhaustive_against_independent_forms(pins_exe):
    r = subprocess.run([pins_exe, oracle.LIBRARY, "rne"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "4294967296 patterns, 0 mismatches" in r.stdout


@pytest.mark.slow
def test_bf16_pair_sum_theorem_exhaustive(pins_exe):
    # residual_out = bf16(fl32(x + r)) equals the bf16 nearest to the exact
    # x + r for every pair of bf16 values: the fp32 add loses nothing.
    r = subprocess.run([pins_exe, oracle.LIBRARY, "sum"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "4294967296 pairs, 0 mismatches" in r.stdout


def _torch_rne(u32):
    t = torch.from_numpy(np.ascontiguousarray(u32).view(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_rne_matches_torch_on_full_high_halves(orc):
    # Every low half for 4096 high halves: the special ones (zeros, subnormals,
    # the smallest normal, 1.0, the largest finite, infinities, NaN space) and
    # a seeded random selection of the rest.
    special = [0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F81, 0x7F7E, 0x7F7F, 0x7F80,
               0x7FC0, 0x8000, 0x8001, 0x807F, 0x8080, 0xBF80, 0xFF7F, 0xFF80, 0xFFC0]
    rng = random.Random(20261202)
    highs = sorted(set(special) | set(rng.sample(range(65536), 4096 - len(special))))
    low = np.arange(65536, dtype=np.uint32)
    u = (np.array(highs, dtype=np.uint32)[:, None] << 16 | low[None, :]).ravel()
    got = orc.rne16_array(u)
    ref = _torch_rne(u)
    nan_in = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x7FFFFF) != 0)
    assert np.array_equal(got[~nan_in], ref[~nan_in])
    got_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    assert got_nan[nan_in].all()


def _exact_bf16_round(y: float) -> int:
    """Nearest-even bf16 of a finite binary64 value, by rational arithmetic."""
    sign = 0x8000 if np.signbit(y) else 0
    a = Fraction(abs(y))
    if a == 0:
        return sign
    # Walk the bf16 grid: find e with 2^e <= a < 2^(e+1).
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 7)
    k = a // q
    lo, hi = k * q, (k + 1) * q
    if a - lo < hi - a or (a - lo == hi - a and k % 2 == 0):
        r = lo
    else:
        r = hi
    if r > Fraction(255) * Fraction(2) ** 120:
        return sign | 0x7F80
    f = np.float32(float(r))
    assert Fraction(float(f)) == r
    return sign | int(np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16)


def test_rne_from_f64_against_exact_rationals(orc):
    rng = random.Random(7)
    vals = []
    for _ in range(3000):
        vals.append(rng.uniform(-4, 4) * 2.0 ** rng.randint(-140, 127))
    # Near-ties: a bf16 midpoint nudged by a few binary64 ULPs either way.
    for _ in range(2000):
        m = rng.randint(0x0001, 0x7F7E)
        base = float(np.array([(m << 16) | 0x8000], dtype=np.uint32).view(np.float32)[0])
        for k in (-2, -1, 0, 1, 2):
            v = base
            for _ in range(abs(k)):
                v = np.nextafter(v, np.inf if k > 0 else -np.inf)
            vals.append(float(v) * (-1 if rng.random() < 0.5 else 1))
    # Overflow boundary and subnormal range.
    top = float(np.float32(3.3961775e38))  # 0x7F7F8000, the overflow midpoint
    vals += [top, np.nextafter(top, 0), np.nextafter(top, np.inf), 2.0 ** 128, 1e300,
             2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -135, 1e-300, -1e-300]
    got = orc.rne16_from_f64_array(np.array(vals))
    for v, g in zip(vals, got):
        assert g == _exact_bf16_round(v), (v, hex(g))


def _mutant(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert old in src, "mutation anchor missing: %r" % old
    path = tmp_path / (name + ".c")
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / ("lib" + name + ".so"))
    oracle.compile_library(str(path), lib)
    return lib


MUTATIONS = {
    # rounding ties away from zero instead of to even
    "ties_away": ("(u + 0x7FFFu + ((u >> 16) & 1u)) >> 16", "(u + 0x8000u) >> 16"),
    # plain truncation (the bug in the issue)
    "truncate": ("(u + 0x7FFFu + ((u >> 16) & 1u)) >> 16", "u >> 16"),
    # NaN check dropped: a NaN with a small payload would carry into Inf
    "no_nan_guard": ("(u & 0x007FFFFFu) != 0)", "(u & 0x007FFFFFu) != 0 && 0)"),
    # binary64 converter truncating its quotient
    "f64_floor": ("nearbyint(a / q)", "floor(a / q)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_exhaustive_pins_catch_planted_mistakes(tmp_path, pins_exe, name):
    old, new = MUTATIONS[name]
    lib = _mutant(tmp_path, name, old, new)
    r = subprocess.run([pins_exe, lib, "rne", "17"], capture_output=True, text=True)
    assert r.returncode == 1, r.stdout + r.stderr
