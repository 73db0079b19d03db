"""Pins for the oracle's per-head q/k RMSNorm, CPU only.

Each head vector of q and k is one plain RMSNorm row over head_dim, q heads
with q_weight and k heads with k_weight.  The oracle is pinned to:
  * exact rational arithmetic per head, read from a fused qkv layout whose
    gaps hold other values (S = sum of the head's squares exactly, out = the
    nearest-even bf16 of x w / sqrt(S / head_dim + eps)), with head scales
    that differ by orders of magnitude, so a norm over the whole token, a
    shifted head or the other tensor's weight cannot pass;
  * closed forms: a one-hot head gives sign(a) sqrt(head_dim) w_k exactly
    (head_dim a power of four) and signed zeros elsewhere;
  * per-head scale invariance: with eps = 0, scaling one head by a power of
    two leaves every output bit unchanged.
Copies of the oracle with planted mistakes in the q/k routine must fail at
least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle_pins import _exact_round_quotient, bits16_to_f32, f32_to_bits16_exact


def _qkv(rng, t, hq, hk, d, scales=(1e-3, 1.0, 50.0)):
    """A fused [t, (hq + 2 hk) d] buffer (q heads, k heads, v heads) with a
    random scale per head; returns the buffer and the q and k views."""
    width = (hq + 2 * hk) * d
    buf = np.empty((t, width), np.uint16)
    for tt in range(t):
        for h in range(hq + 2 * hk):
            buf[tt, h * d:(h + 1) * d] = synth.to_bf16_bits(
                rng.standard_normal(d) * rng.choice(scales))
    q = buf[:, :hq * d].reshape(t, hq, d)
    k = buf[:, hq * d:(hq + hk) * d].reshape(t, hk, d)
    return buf, q, k


def _expect_head(x, w, eps):
    d = x.shape[0]
    xq = [Fraction(float(a)) for a in bits16_to_f32(x)]
    v = sum(a * a for a in xq) / d + Fraction(eps)
    return np.array([_exact_round_quotient(xq[j] * Fraction(float(bits16_to_f32(w[j]))), v)
                     for j in range(d)], np.uint16)


def pin_qk_exact_rationals(orc):
    rng = np.random.default_rng(71)
    for d, hq, hk, eps in ((8, 4, 2, 1e-6), (16, 3, 1, 0.5), (24, 2, 2, 0.0), (8, 1, 3, 1e-6)):
        eps = float(np.float32(eps))
        _buf, q, k = _qkv(rng, 3, hq, hk, d)
        qw = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(d))
        kw = synth.to_bf16_bits(-1 + 0.3 * rng.standard_normal(d))
        q_out, k_out = orc.qk_rmsnorm(q, k, qw, kw, eps)
        for t in range(3):
            for h in range(hq):
                assert np.array_equal(q_out[t, h], _expect_head(q[t, h], qw, eps)), (d, t, h)
            for h in range(hk):
                assert np.array_equal(k_out[t, h], _expect_head(k[t, h], kw, eps)), (d, t, h)


def pin_qk_one_hot_heads(orc):
    rng = np.random.default_rng(72)
    for d in (64, 256):
        t_n, hq, hk = 2, 4, 2
        qw = synth.to_bf16_bits(rng.uniform(0.5, 2.0, d))
        kw = synth.to_bf16_bits(-rng.uniform(0.5, 2.0, d))
        buf = np.zeros((t_n, (hq + 2 * hk) * d), np.uint16)
        pos = {}
        for t in range(t_n):
            for h in range(hq + hk):
                kk = (7 * t + 13 * h + 1) % d
                a = 16.0 if (t + h) % 2 else -16.0
                buf[t, h * d + kk] = f32_to_bits16_exact([a])[0]
                pos[(t, h)] = (kk, a)
        q = buf[:, :hq * d].reshape(t_n, hq, d)
        k = buf[:, hq * d:(hq + hk) * d].reshape(t_n, hk, d)
        q_out, k_out = orc.qk_rmsnorm(q, k, qw, kw, 1e-9)
        root = int(round(d ** 0.5))
        for t in range(t_n):
            for h in range(hq + hk):
                out, w = (q_out[t, h], qw) if h < hq else (k_out[t, h - hq], kw)
                kk, a = pos[(t, h)]
                wk = float(bits16_to_f32(w[kk]))
                assert out[kk] == f32_to_bits16_exact([np.sign(a) * root * wk])[0], (d, t, h)
                rest = np.delete(np.arange(d), kk)
                assert np.array_equal(out[rest], w[rest] & 0x8000), (d, t, h)


def pin_qk_head_scale_invariance(orc):
    rng = np.random.default_rng(73)
    d, hq, hk = 128, 4, 2
    buf, q, k = _qkv(rng, 3, hq, hk, d, scales=(1.0,))
    qw = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(d))
    kw = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(d))
    base_q, base_k = orc.qk_rmsnorm(q, k, qw, kw, 0.0)
    for head, power in ((0, 8), (hq - 1, -6), (hq, 5), (hq + hk - 1, -9)):
        scaled = buf.copy()
        for t in range(3):
            seg = scaled[t, head * d:(head + 1) * d]
            f = bits16_to_f32(seg) * np.float32(2.0 ** power)
            scaled[t, head * d:(head + 1) * d] = f32_to_bits16_exact(f)
        q2 = scaled[:, :hq * d].reshape(3, hq, d)
        k2 = scaled[:, hq * d:(hq + hk) * d].reshape(3, hk, d)
        got_q, got_k = orc.qk_rmsnorm(q2, k2, qw, kw, 0.0)
        assert np.array_equal(got_q, base_q) and np.array_equal(got_k, base_k), (head, power)


QK_PINS = [pin_qk_exact_rationals, pin_qk_one_hot_heads, pin_qk_head_scale_invariance]


@pytest.mark.parametrize("pin", QK_PINS, ids=lambda f: f.__name__)
def test_qk_pin(orc, pin):
    with np.errstate(all="ignore"):
        pin(orc)


def test_qk_no_heads_and_bad_arguments(orc):
    rng = np.random.default_rng(74)
    _buf, q, k = _qkv(rng, 2, 2, 1, 16)
    w = synth.to_bf16_bits(np.ones(16))
    # no k heads: q alone
    q_out, k_out = orc.qk_rmsnorm(q, k[:, :0], w, w)
    assert k_out.shape == (2, 0, 16)
    assert np.array_equal(q_out, orc.qk_rmsnorm(q, k, w, w)[0])
    # a weight of the wrong length, a stride below the heads' width
    with pytest.raises(ValueError):
        orc.qk_rmsnorm(q, k, w[:8], w)
    lib = orc.lib
    out = np.empty(32, np.uint16)
    x = np.zeros(32, np.uint16)
    assert lib.orc_qk_rmsnorm(out.ctypes.data, None, x.ctypes.data, None, w.ctypes.data, None,
                              1, 2, 0, 16, 16, 0, 1e-6) == -1


QK_MUTATIONS = {
    "qk_head_offset_dropped": ("const uint16_t* row = q + t * q_stride + h * head_dim;",
                               "const uint16_t* row = q + t * q_stride;"),
    "qk_token_stride_ignored": ("const uint16_t* row = k + t * k_stride + h * head_dim;",
                                "const uint16_t* row = k + t * n_k_heads * head_dim"
                                " + h * head_dim;"),
    "qk_k_takes_q_weight": ("row, NULL, k_weight, 1", "row, NULL, q_weight, 1"),
    "qk_heads_reversed": ("uint16_t* dst = k_out + (t * n_k_heads + h) * head_dim;",
                          "uint16_t* dst = k_out + (t * n_k_heads + (n_k_heads - 1 - h))"
                          " * head_dim;"),
    "qk_first_head_eps_doubled": (
        "if (orc_add_rmsnorm(dst, NULL, NULL, row, NULL, q_weight, 1, head_dim, eps, ORC_RNE))",
        "if (orc_add_rmsnorm(dst, NULL, NULL, row, NULL, q_weight, 1, head_dim, "
        "h ? eps : 2 * eps, ORC_RNE))"),
}


@pytest.mark.parametrize("name", sorted(QK_MUTATIONS))
def test_qk_pins_catch_planted_mistake(tmp_path, name):
    old, new = QK_MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert old in src, name
    path = tmp_path / (name + ".c")
    path.write_text(src.replace(old, new))
    lib = str(tmp_path / ("lib" + name + ".so"))
    oracle.compile_library(str(path), lib)
    mut = oracle.Oracle(lib)
    failed = []
    for pin in QK_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mut)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake %s" % name
