"""Parity of the HIP path with the oracle (GPU).

Bar: residual_out bit-exact; out within one bf16 ULP; on random workloads
|mean signed relative error| <= 1e-4 against the oracle's unrounded values,
for both stores.  Outputs are poisoned with a NaN pattern before each launch,
so an element the kernel fails to write cannot pass.
"""
import numpy as np
import pytest

import bf16_rounding_numerics_amd as arn
import oracle
import synth
from gpu_helpers import (BIAS_GATE, POISON, announce, check_parity, from_dev, gpu_fwd,
                         is_nan16, poisoned_like, require_gpu, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_workloads_full_size(name):
    """The five workloads at full size, default launch (as the benchmark runs
    them), every element compared."""
    c = synth.CONFIGS[name]
    announce("parity %s seed %d" % (name, c["seed"]))
    x, r, w = synth.workload(c["seed"], c["n_rows"], c["hidden"])
    out, res = gpu_fwd(x, r, w, 1e-6)
    stats = check_parity(x, r, w, 1e-6, out, res, bias=BIAS_GATE, label=name)
    # Off-by-one elements are near-ties of the fp32 pipeline: rare.
    assert stats["off_by_one"] <= 1e-3 * stats["n"], stats
    announce("  %s" % stats)


RAGGED = [(1, 8), (3, 16), (5, 24), (7, 504), (9, 520), (13, 1000), (17, 1024), (11, 2040),
          (2, 2048), (19, 2056), (6, 3000), (33, 4096), (3, 5000), (12, 8192), (5, 8200),
          (4, 12288), (3, 16384), (2, 16392), (3, 24576), (2, 32768), (130, 64), (257, 1024)]


@pytest.mark.parametrize("n,h", RAGGED)
def test_ragged_shapes(n, h):
    """Row counts that do not fill a workgroup and hidden sizes that leave
    partial 64-segment blocks, across all three kernels."""
    announce("ragged %dx%d" % (n, h))
    x, r, w = synth.workload(1000 + h, n, h)
    out, res = gpu_fwd(x, r, w, 1e-6)
    check_parity(x, r, w, 1e-6, out, res, label="%dx%d" % (n, h))


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5, 3.0])
def test_eps_values(eps):
    announce("eps %g" % eps)
    x, r, w = synth.workload(31, 16, 4096)
    out, res = gpu_fwd(x, r, w, eps)
    check_parity(x, r, w, eps, out, res, label="eps=%g" % eps)


def _special_rows(h):
    rng = np.random.default_rng(5)
    rows_x, rows_r = [], []

    def add(xv, rv):
        rows_x.append(np.asarray(xv, dtype=np.uint16))
        rows_r.append(np.asarray(rv, dtype=np.uint16))

    base_x = synth.to_bf16_bits(rng.standard_normal(h))
    base_r = synth.to_bf16_bits(rng.standard_normal(h))
    z = np.zeros(h, np.uint16)
    add(base_x, base_r)
    nanx = base_x.copy(); nanx[h // 3] = 0x7FC1; add(nanx, base_r)            # NaN in one element
    infx = base_x.copy(); infx[5] = 0x7F80; add(infx, base_r)                 # +Inf
    ninf = base_x.copy(); ninf[7] = 0xFF80; add(ninf, base_r)                 # -Inf
    cancel = base_x.copy(); cancel[2] = 0x7F80; rr = base_r.copy(); rr[2] = 0xFF80
    add(cancel, rr)                                                           # Inf - Inf
    add(np.full(h, 0x7F7F), np.full(h, 0x7F7F))                               # fp32 add overflow
    big = np.full(h, 0x62C0)  # 2^70 * 1.5: squares overflow fp32 -> rinv = 0
    big[::3] |= 0x8000
    add(big, z)
    add(np.full(h, 0x5E80), z)                                                # 2^62: S near 2^124*h
    add(z, z)                                                                 # zeros
    add(np.full(h, 0x8000), np.full(h, 0x8000))                               # -0 + -0
    add(np.full(h, 0x0001), np.full(h, 0x0001))                               # subnormals
    sub = synth.to_bf16_bits(rng.standard_normal(h) * 1e-39)                  # subnormal mix
    add(sub, synth.to_bf16_bits(rng.standard_normal(h) * 1e-39))
    tiny = synth.to_bf16_bits(rng.standard_normal(h) * 1e-30)
    add(tiny, z)                                                              # eps dominates
    onehot = z.copy(); onehot[h - 1] = 0x4180; add(onehot, z)                 # 16 at the end
    alt = np.where(np.arange(h) % 2 == 0, 0x3F80, 0xBF80); add(alt, z)        # +-1
    gap = synth.to_bf16_bits(rng.standard_normal(h) * 2.0 ** 40)              # exponent gaps
    add(gap, synth.to_bf16_bits(rng.standard_normal(h) * 2.0 ** -30))
    return np.stack(rows_x), np.stack(rows_r)


@pytest.mark.parametrize("h", [64, 1024, 4096, 8192, 16384])
def test_special_values(h):
    announce("special values hidden %d" % h)
    x, r = _special_rows(h)
    w = synth.bf16_normal(77, 2, (h,), 1.0, 0.1)
    w[1] ^= 0x8000  # a negative weight
    out, res = gpu_fwd(x, r, w, 1e-6)
    exp_out, exp_res = oracle.add_rmsnorm(x, r, w, 1e-6)
    # Row with fp32 sums of squares near 2^124 * h stays finite on both sides:
    # check it is not within 2^-20 of the fp32 overflow point (it is not).
    check_parity(x, r, w, 1e-6, out, res, label="special h=%d" % h)
    # NaN in an input row makes the whole out row NaN.
    assert is_nan16(out[1]).all() and is_nan16(exp_out[1]).all()


@pytest.mark.parametrize("h", [256, 1024, 4096, 8192, 16384])
def test_zero_row_with_eps_zero_is_nan(h):
    """eps = 0: a zero row's out is NaN throughout on both sides (0 * Inf), its
    residual_out zero; the other rows are untouched by it."""
    announce("zero row, eps 0, hidden %d" % h)
    x, r, w = synth.workload(41, 6, h)
    x[2] = 0
    r[2] = 0
    out, res = gpu_fwd(x, r, w, 0.0)
    check_parity(x, r, w, 0.0, out, res, label="zero row eps 0 h=%d" % h)
    assert is_nan16(out[2]).all() and (res[2] == 0).all()
    assert not is_nan16(np.delete(out, 2, axis=0)).any()


@pytest.mark.parametrize("k", [-40, -9, 5, 30])
def test_power_of_two_scaling_bitwise(k):
    """With eps = 0, scaling x and residual by 2^k must leave out unchanged
    bit for bit: every fp32 step is correctly rounded, which commutes with
    exact power-of-two scaling."""
    announce("scaling 2^%d" % k)
    x, r, w = synth.workload(41, 24, 4096)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    g = lambda v: (v.view(np.uint32) >> 16).astype(np.uint16)
    xs = g(f(x) * np.float32(2.0 ** k))
    rs = g(f(r) * np.float32(2.0 ** k))
    assert np.array_equal(f(g(f(x) * np.float32(2.0 ** k))), f(x) * np.float32(2.0 ** k))
    out0, _ = gpu_fwd(x, r, w, 0.0)
    out1, _ = gpu_fwd(xs, rs, w, 0.0)
    assert np.array_equal(out0, out1)


def test_zero_rows_writes_nothing():
    """n_rows = 0 through the C ABI, with the outputs pointing into poisoned
    buffers of real rows: every path returns OK and leaves them untouched."""
    import ctypes

    import torch

    import bf16_rounding_numerics_amd as arn

    announce("zero rows")
    h = 1024
    x, r, w = synth.workload(5, 4, h)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    out, res = poisoned_like(xd), poisoned_like(xd)
    L = arn.lib()
    torch.cuda.synchronize()
    for path in (arn.PATH_AUTO, arn.PATH_WAVE_ROW, arn.PATH_WG_ROW, arn.PATH_LDS_TWO_PASS,
                 arn.PATH_GENERAL, arn.PATH_PACKED):
        cfg = arn.LaunchCfg(path, 0, 0, 0)
        assert L.add_rmsnorm_fwd_cfg(out.data_ptr(), res.data_ptr(), xd.data_ptr(),
                                     rd.data_ptr(), wd.data_ptr(), 0, h, 1e-6,
                                     ctypes.byref(cfg), None) == arn.OK
    assert L.add_rmsnorm_fwd(out.data_ptr(), res.data_ptr(), xd.data_ptr(), rd.data_ptr(),
                             wd.data_ptr(), 0, h, 1e-6, None) == arn.OK
    assert L.rmsnorm_fwd(out.data_ptr(), xd.data_ptr(), wd.data_ptr(), 0, h, 1e-6,
                         None) == arn.OK
    torch.cuda.synchronize()
    assert (from_dev(out) == POISON).all()
    assert (from_dev(res) == POISON).all()
    # the same buffers are then written by a call with rows (the check can fail)
    arn.add_rmsnorm_fwd(out, res, xd, rd, wd, 1e-6)
    torch.cuda.synchronize()
    assert not (from_dev(out) == POISON).any()


def test_side_stream_and_leading_dims():
    """Launch on a non-default stream, tensors of shape [batch, seq, hidden]."""
    import torch

    import bf16_rounding_numerics_amd as arn

    announce("side stream")
    x, r, w = synth.workload(51, 6 * 10, 2048)
    xd = to_dev(x).view(6, 10, 2048)
    rd = to_dev(r).view(6, 10, 2048)
    wd = to_dev(w)
    out = poisoned_like(xd)
    res = poisoned_like(xd)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        arn.add_rmsnorm_fwd(out, res, xd, rd, wd, 1e-6, stream=s)
    s.synchronize()
    check_parity(x, r, w, 1e-6, from_dev(out).reshape(60, 2048), from_dev(res).reshape(60, 2048))


def test_binding_rejects_partial_aliasing_on_gpu():
    import bf16_rounding_numerics_amd as arn

    announce("partial aliasing rejected")
    x, r, w = synth.workload(61, 5, 1024)
    buf = to_dev(np.concatenate([x, r]))          # rows 0-4 x, rows 5-9 residual
    xd, wd = buf[:5], to_dev(w)
    shifted = buf[1:6]                            # overlaps x by four rows
    out = poisoned_like(xd)
    with pytest.raises(arn.AddRmsnormError) as e:
        arn.add_rmsnorm_fwd(out, shifted, xd, buf[5:10], wd)
    assert e.value.status == arn.EALIAS
    assert (from_dev(out) == 0x7FC1).all()
    assert np.array_equal(from_dev(buf), np.concatenate([x, r]))


def test_copy_reference_copies_bit_exactly():
    """The measurement hook (the streaming copy the benchmark uses as its
    reference rate) must really move every byte."""
    import torch

    announce("copy2 reference")
    x, r, _ = synth.workload(91, 333, 1024)
    xd, rd = to_dev(x), to_dev(r)
    d0, d1 = poisoned_like(xd), poisoned_like(xd)
    arn.add_rmsnorm_test_copy2(d0, d1, xd, rd)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(d0), x) and np.array_equal(from_dev(d1), r)


@pytest.mark.parametrize("burst", [1, 2, 4])
@pytest.mark.parametrize("n,h", [(333, 1024), (37, 12288), (5, 16384), (1, 8)])
def test_row_copy_reference_copies_bit_exactly(burst, n, h):
    """The row-structured measurement copy moves every byte of every row,
    for row counts that leave a partial burst and hidden that leaves a
    partial set of 512-thread segments."""
    import torch

    announce("copy_rows reference %dx%d burst %d" % (n, h, burst))
    x, r, _ = synth.workload(92, n, h)
    xd, rd = to_dev(x), to_dev(r)
    d0, d1 = poisoned_like(xd), poisoned_like(xd)
    arn.add_rmsnorm_test_copy_rows(d0, d1, xd, rd, burst)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(d0), x) and np.array_equal(from_dev(d1), r)


def test_stream_hooks():
    """The read-only and write-only measurement streams: writing fills every
    element with bf16 1.0; reading leaves the sink untouched (its fold of
    these inputs is not the trigger pattern)."""
    import torch

    announce("stream hooks")
    n = (1 << 20) + 8
    src = to_dev(synth.bf16_normal(91, 0, (n,), 0.0, 1.0))
    sink = poisoned_like(src)
    arn.add_rmsnorm_test_stream(sink, src, 0)
    dst = poisoned_like(src)
    arn.add_rmsnorm_test_stream(dst, dst, 1)
    torch.cuda.synchronize()
    assert (from_dev(sink) == POISON).all()
    assert (from_dev(dst) == 0x3F80).all()


def test_empty_inputs_through_every_entry_point():
    """Zero rows (and zero log1p elements): every entry point returns at once
    and touches nothing."""
    import torch

    announce("empty inputs")
    dev = "cuda:0"
    e = torch.empty(0, 1024, dtype=torch.int16, device=dev)
    w = torch.ones(1024, dtype=torch.int16, device=dev)
    arn.add_rmsnorm_fwd(e, e.clone(), e, e.clone(), w, 1e-6)
    arn.rmsnorm_fwd(e, e.clone(), w, 1e-6)
    arn.add_rmsnorm_quant_fwd(torch.empty(0, 1024, dtype=torch.int8, device=dev),
                              torch.empty(0, dtype=torch.float32, device=dev), e, e.clone(),
                              e.clone(), w, 1e-6)
    arn.rmsnorm_quant_fwd(torch.empty(0, 1024, dtype=torch.int8, device=dev),
                          torch.empty(0, dtype=torch.float32, device=dev), e, w, 1e-6)
    arn.add_rmsnorm_quant_fp8_fwd(torch.empty(0, 1024, dtype=torch.uint8, device=dev),
                                  torch.empty(0, dtype=torch.float32, device=dev), e, e.clone(),
                                  e.clone(), w, 1e-6)
    arn.rmsnorm_quant_fp8_fwd(torch.empty(0, 1024, dtype=torch.uint8, device=dev),
                              torch.empty(0, dtype=torch.float32, device=dev), e, w, 1e-6)
    arn.add_rmsnorm_fwd_strided(e, e.clone(), e.clone(), e.clone(), w, 1e-6)
    hw = torch.ones(128, dtype=torch.int16, device=dev)
    qe = torch.empty(0, 32, 128, dtype=torch.int16, device=dev)
    ke = torch.empty(0, 8, 128, dtype=torch.int16, device=dev)
    arn.qk_rmsnorm_fwd(qe, ke, qe.clone(), ke.clone(), hw, hw, 1e-6)
    f = torch.empty(0, dtype=torch.float32, device=dev)
    arn.log1p_f32(f, f.clone())
    torch.cuda.synchronize()
