"""Per-head q/k RMSNorm and the packed short-row kernel on the GPU.

Bars:
  * qk_rmsnorm_fwd: every head bit-exact against the fp32 model of the
    kernels' arithmetic on that head row, within one bf16 ULP of the binary64
    oracle's per-head RMSNorm, |mean signed relative error| <= 1e-4; read from
    and written into a fused qkv tensor (in place and out of place), with the
    v columns and every gap left untouched;
  * bitwise invariance over workgroup sizes, rows per lane and grids;
  * the packed path of the fused and plain entry points bit for bit the
    default kernels' result, on contiguous and strided views;
  * edge cases: head dims whose segments are not a power of two (idle lanes),
    token counts that leave the last wavefront part-filled, q alone, no tokens.
"""
import numpy as np
import pytest

import bf16_rounding_numerics_amd as arn
import fp32_model
import oracle
import synth
from gpu_helpers import (BIAS_GATE, POISON, announce, from_dev, gpu_fwd, is_nan16,
                         poisoned_like, require_gpu, to_dev, ulp_distance)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _qkv(seed, t, hq, hk, d):
    rng = np.random.default_rng(seed)
    buf = synth.to_bf16_bits(rng.standard_normal((t, (hq + 2 * hk) * d)))
    qw = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(d))
    kw = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(d))
    return buf, qw, kw


def _views(dev_buf, hq, hk, d):
    t = dev_buf.shape[0]
    q = dev_buf[:, :hq * d].view(t, hq, d)
    k = dev_buf[:, hq * d:(hq + hk) * d].view(t, hk, d)
    return q, k


def _check_heads(buf, hq, hk, d, qw, kw, eps, q_got, k_got, label):
    """q_got [t, hq, d], k_got [t, hk, d] against the fp32 model and the oracle."""
    t = buf.shape[0]
    q_in = buf[:, :hq * d].reshape(t, hq, d)
    k_in = buf[:, hq * d:(hq + hk) * d].reshape(t, hk, d)
    o_q, o_k = oracle.qk_rmsnorm(q_in, k_in, qw, kw, eps)
    for name, x, w, got, exp in (("q", q_in, qw, q_got, o_q), ("k", k_in, kw, k_got, o_k)):
        if x.shape[1] == 0:
            continue
        rows = x.reshape(-1, d)
        m_out, _ = fp32_model.add_rmsnorm(rows, None, w, eps)
        g = got.reshape(-1, d)
        bad = (g != m_out) & ~(is_nan16(g) & is_nan16(m_out))
        assert not bad.any(), "%s %s: %d elements differ from the fp32 model, first %s" % (
            label, name, int(bad.sum()), np.argwhere(bad)[:3].tolist())
        dist = ulp_distance(g, exp.reshape(-1, d))
        assert dist.max() <= 1, "%s %s: off by %d ULP" % (label, name, int(dist.max()))
        _, y = oracle.rmsnorm(rows, w, eps, want_exact=True)
        fin = np.isfinite(y)
        b = oracle.magnitude_bias(oracle.bf16_to_f64(g)[fin], y[fin])
        assert abs(b) <= BIAS_GATE, "%s %s: bias %.3e" % (label, name, b)


# Qwen3-8B's attention (32 q heads, 8 kv heads, head_dim 128) and other shapes:
# segments not a power of two (24, 40, 200), tiny and the largest head_dim.
QK_SHAPES = [(257, 32, 8, 128), (33, 16, 4, 64), (19, 8, 2, 256), (7, 4, 2, 512),
             (65, 5, 3, 24), (41, 6, 1, 40), (3, 2, 1, 200), (130, 3, 2, 8), (9, 40, 8, 16)]


@pytest.mark.parametrize("t,hq,hk,d", QK_SHAPES)
def test_qk_out_of_place_on_fused_qkv(t, hq, hk, d):
    import torch

    announce("qk out of place t=%d hq=%d hk=%d d=%d" % (t, hq, hk, d))
    buf, qw, kw = _qkv(1000 + d + hq, t, hq, hk, d)
    dev = to_dev(buf)
    q, k = _views(dev, hq, hk, d)
    q_out = poisoned_like(q.contiguous())
    k_out = poisoned_like(k.contiguous())
    arn.qk_rmsnorm_fwd(q_out, k_out, q, k, to_dev(qw), to_dev(kw), 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dev), buf), "the input was modified"
    _check_heads(buf, hq, hk, d, qw, kw, 1e-6, from_dev(q_out), from_dev(k_out),
                 "qk %dx(%d+%d)x%d" % (t, hq, hk, d))


@pytest.mark.parametrize("t,hq,hk,d", [(257, 32, 8, 128), (65, 5, 3, 24), (7, 4, 2, 512)])
def test_qk_in_place_leaves_v_and_gaps(t, hq, hk, d):
    import torch

    announce("qk in place t=%d hq=%d hk=%d d=%d" % (t, hq, hk, d))
    buf, qw, kw = _qkv(2000 + d, t, hq, hk, d)
    # a wider row than q, k and v need: the last 8 columns are a gap
    wide = np.concatenate([buf, np.full((t, 8), POISON, np.uint16)], axis=1)
    dev = to_dev(wide)
    q = dev[:, :hq * d].view(t, hq, d)
    k = dev[:, hq * d:(hq + hk) * d].view(t, hk, d)
    arn.qk_rmsnorm_fwd(q, k, q, k, to_dev(qw), to_dev(kw), 1e-6)
    torch.cuda.synchronize()
    got = from_dev(dev)
    assert np.array_equal(got[:, (hq + hk) * d:], wide[:, (hq + hk) * d:]), "v or gap written"
    _check_heads(buf, hq, hk, d, qw, kw, 1e-6,
                 got[:, :hq * d].reshape(t, hq, d),
                 got[:, hq * d:(hq + hk) * d].reshape(t, hk, d), "qk in place")


def test_qk_launch_invariance():
    import torch

    t, hq, hk, d = 131, 32, 8, 128
    buf, qw, kw = _qkv(3000, t, hq, hk, d)
    dev = to_dev(buf)
    q, k = _views(dev, hq, hk, d)
    qwd, kwd = to_dev(qw), to_dev(kw)
    ref = None
    for block in (0, 64, 256, 1024):
        for rpl in (0, 1, 2, 4):
            for grid in (0, 1, 7, -1):
                announce("qk launch block=%d rows_per_lane=%d grid=%d" % (block, rpl, grid))
                q_out = poisoned_like(q.contiguous())
                k_out = poisoned_like(k.contiguous())
                arn.qk_rmsnorm_fwd_cfg(q_out, k_out, q, k, qwd, kwd, 1e-6,
                                       path=arn.PATH_PACKED, block_threads=block,
                                       grid_blocks=grid, rows_per_lane=rpl)
                torch.cuda.synchronize()
                got = (from_dev(q_out), from_dev(k_out))
                if ref is None:
                    ref = got
                    _check_heads(buf, hq, hk, d, qw, kw, 1e-6, got[0], got[1], "qk launch")
                assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), (
                    block, rpl, grid)


def test_qk_q_only_and_no_tokens():
    import torch

    t, hq, d = 45, 12, 64
    buf, qw, kw = _qkv(4000, t, hq, 0, d)
    dev = to_dev(buf)
    q = dev.view(t, hq, d)
    q_out = poisoned_like(q)
    announce("qk q only")
    arn.qk_rmsnorm_fwd(q_out, None, q, None, to_dev(qw), to_dev(kw), 1e-6)
    torch.cuda.synchronize()
    _check_heads(buf, hq, 0, d, qw, kw, 1e-6, from_dev(q_out), None, "q only")
    empty = dev[:0].view(0, hq, d)
    announce("qk no tokens")
    arn.qk_rmsnorm_fwd(empty, None, empty, None, to_dev(qw), to_dev(kw), 1e-6)
    torch.cuda.synchronize()


def test_qk_special_values_per_head():
    """NaN, Inf, zero and huge heads stay confined to their own head."""
    import torch

    t, hq, hk, d = 4, 4, 2, 128
    buf, qw, kw = _qkv(5000, t, hq, hk, d)
    buf[0, 5] = 0x7FC1                               # NaN in q head 0 of token 0
    buf[1, d + 3] = 0x7F80                           # +Inf in q head 1 of token 1
    buf[2, 2 * d:3 * d] = 0                          # an all-zero head
    buf[3, hq * d:(hq + 1) * d] = 0x7F7F             # the largest bf16: S overflows fp32
    dev = to_dev(buf)
    q, k = _views(dev, hq, hk, d)
    q_out = poisoned_like(q.contiguous())
    k_out = poisoned_like(k.contiguous())
    announce("qk special values")
    arn.qk_rmsnorm_fwd(q_out, k_out, q, k, to_dev(qw), to_dev(kw), 1e-6)
    torch.cuda.synchronize()
    qo, ko = from_dev(q_out), from_dev(k_out)
    assert is_nan16(qo[0, 0]).all() and not is_nan16(qo[0, 1:]).any()
    assert not is_nan16(qo[1, 0]).any() and not is_nan16(qo[1, 2:]).any()
    q_in = buf[:, :hq * d].reshape(t, hq, d)
    k_in = buf[:, hq * d:(hq + hk) * d].reshape(t, hk, d)
    for got, x, w in ((qo, q_in, qw), (ko, k_in, kw)):
        m_out, _ = fp32_model.add_rmsnorm(x.reshape(-1, d), None, w, 1e-6)
        g = got.reshape(-1, d)
        bad = (g != m_out) & ~(is_nan16(g) & is_nan16(m_out))
        assert not bad.any(), np.argwhere(bad)[:3].tolist()


# ------------------------------------------------------------------ the packed path

PACKED_HIDDEN = [8, 16, 24, 64, 120, 128, 200, 256, 504, 512]


@pytest.mark.parametrize("h", PACKED_HIDDEN)
def test_packed_path_matches_default_kernels(h):
    n = 1000 + h % 61
    x, r, w = synth.workload(seed=60 + h, n_rows=n, hidden=h)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    announce("packed fused h=%d default" % h)
    ref_out, ref_res = gpu_fwd(x, r, w, xd=xd, rd=rd, wd=wd)
    for block, rpl, grid in ((0, 0, 0), (64, 1, 3), (1024, 4, -1), (256, 2, 1)):
        import torch

        announce("packed fused h=%d block=%d rpl=%d grid=%d" % (h, block, rpl, grid))
        out, res = poisoned_like(xd), poisoned_like(xd)
        arn.add_rmsnorm_fwd_cfg(out, res, xd, rd, wd, 1e-6, path=arn.PATH_PACKED,
                                block_threads=block, grid_blocks=grid, rows_per_lane=rpl)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(out), ref_out), (h, block, rpl, grid)
        assert np.array_equal(from_dev(res), ref_res), (h, block, rpl, grid)
        outp = poisoned_like(xd)
        arn.rmsnorm_fwd_cfg(outp, xd, wd, 1e-6, path=arn.PATH_PACKED, block_threads=block,
                            grid_blocks=grid, rows_per_lane=rpl)
        refp = poisoned_like(xd)
        arn.rmsnorm_fwd(refp, xd, wd, 1e-6)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(outp), from_dev(refp)), (h, block, rpl, grid)
    exp_out, exp_res = oracle.add_rmsnorm(x, r, w, 1e-6)
    assert np.array_equal(ref_res, exp_res)
    assert ulp_distance(ref_out, exp_out).max() <= 1


def test_packed_path_strided_views():
    import torch

    n, h, ld = 777, 128, 3 * 128 + 8
    rng = np.random.default_rng(77)
    big = synth.to_bf16_bits(rng.standard_normal((n, ld)))
    w = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(h))
    dev = to_dev(big)
    x, r = dev[:, :h], dev[:, h:2 * h]
    out_wide = poisoned_like(dev)
    out, res = out_wide[:, :h], out_wide[:, 2 * h:3 * h]
    wd = to_dev(w)
    announce("packed strided")
    arn.add_rmsnorm_fwd_strided(out, res, x, r, wd, 1e-6, path=arn.PATH_PACKED)
    torch.cuda.synchronize()
    got = from_dev(out_wide)
    xs, rs = big[:, :h].copy(), big[:, h:2 * h].copy()
    exp_out, exp_res = oracle.add_rmsnorm(xs, rs, w, 1e-6)
    m_out, m_res = fp32_model.add_rmsnorm(xs, rs, w, 1e-6)
    assert np.array_equal(got[:, 2 * h:3 * h], exp_res)
    assert np.array_equal(got[:, :h], m_out)
    assert (got[:, h:2 * h] == POISON).all() and (got[:, 3 * h:] == POISON).all()


def test_qk_graph_replays_match_eager():
    """qk_rmsnorm_fwd captured once in a HIP graph, in place on a qkv buffer,
    replayed on fresh inputs with eager work in between; every replay equals
    an eager call on the same inputs."""
    import torch

    t, hq, hk, d = 64, 8, 2, 128
    dev = "cuda:0"
    buf = torch.empty(t, (hq + 2 * hk) * d, dtype=torch.int16, device=dev)
    q, k = _views(buf, hq, hk, d)
    _, qw, kw = _qkv(6000, t, hq, hk, d)
    qwd, kwd = to_dev(qw), to_dev(kw)

    def fresh(rep):
        return to_dev(_qkv(6001 + rep, t, hq, hk, d)[0])

    announce("qk graph capture")
    buf.copy_(fresh(0))
    arn.qk_rmsnorm_fwd(q, k, q, k, qwd, kwd, 1e-6)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        arn.qk_rmsnorm_fwd(q, k, q, k, qwd, kwd, 1e-6)
    torch.cuda.synchronize()
    for rep in range(1, 4):
        announce("qk graph replay %d" % rep)
        x = fresh(rep)
        buf.copy_(x)
        g.replay()
        xq, xk = _views(x, hq, hk, d)
        eq = torch.empty(t, hq, d, dtype=torch.int16, device=dev)
        ek = torch.empty(t, hk, d, dtype=torch.int16, device=dev)
        arn.qk_rmsnorm_fwd(eq, ek, xq, xk, qwd, kwd, 1e-6)
        _ = (x.float() * 2).sum()
        torch.cuda.synchronize()
        assert torch.equal(q, eq) and torch.equal(k, ek), rep
        assert torch.equal(buf[:, (hq + hk) * d:], x[:, (hq + hk) * d:]), rep


def test_qk_tensors_beyond_4gib():
    """A qkv tensor of more than 2^31 elements per view: token offsets past
    2^31 elements exercise the packed kernel's 64-bit addressing.  Tokens are
    copies of a seeded block of 256 (token i is block token (5 i + 1) mod 256);
    sampled tokens, on both sides of the boundary, are checked against the
    oracle and the fp32 model."""
    import torch

    t, hq, hk, d = 2 ** 19 + 3, 32, 8, 128
    width = (hq + 2 * hk) * d
    assert t * width > 2 ** 31 and t * hq * d * 2 > 2 ** 32
    block, qw, kw = _qkv(7000, 256, hq, hk, d)
    idx = (5 * np.arange(t) + 1) % 256
    dev = torch.device("cuda:0")
    announce("qk large: %d tokens, %.1f GiB qkv" % (t, t * width * 2 / 2 ** 30))
    buf = to_dev(block)[torch.from_numpy(idx).to(dev)]
    q, k = _views(buf, hq, hk, d)
    q_out = torch.empty(t, hq, d, dtype=torch.int16, device=dev)
    k_out = torch.empty(t, hk, d, dtype=torch.int16, device=dev)
    arn.qk_rmsnorm_fwd(q_out, k_out, q, k, to_dev(qw), to_dev(kw), 1e-6)
    torch.cuda.synchronize()
    edge = 2 ** 31 // width
    toks = sorted({0, 1, 255, 256, t // 2, edge - 1, edge, edge + 1, 2 ** 31 // (hq * d),
                   2 ** 31 // (hq * d) + 1, t - 2, t - 1})
    sel = torch.tensor(toks, device=dev)
    got_q = q_out[sel].cpu().numpy().view(np.uint16)
    got_k = k_out[sel].cpu().numpy().view(np.uint16)
    _check_heads(block[idx[toks]], hq, hk, d, qw, kw, 1e-6, got_q, got_k,
                 "qk large tokens %s" % toks)
    del buf, q_out, k_out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("h", [8, 24, 64, 128, 200, 256, 512])
def test_packed_quantised_matches_wave_row(h):
    """int8 and E4M3 codes, scales and residual_out on the packed kernel equal
    one wavefront per row's, fused and plain, over several launches."""
    from test_gpu_plain import gpu_plain_quant
    from test_gpu_quant import check_model, gpu_quant, same_scale_bits
    from test_gpu_quant_fp8 import gpu_fp8

    n = 700 + h % 37
    x, r, w = synth.workload(90 + h, n, h)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    runs = {
        "int8": lambda **c: gpu_quant(x, r, w, xd=xd, rd=rd, wd=wd, **c),
        "fp8": lambda **c: gpu_fp8(x, r, w, xd=xd, rd=rd, wd=wd, **c),
        "plain int8": lambda **c: gpu_plain_quant(x, w, xd=xd, wd=wd, **c) + (None,),
        "plain fp8": lambda **c: gpu_fp8(x, None, w, xd=xd, wd=wd, **c),
    }
    for name, run in runs.items():
        announce("packed quantised %s h=%d" % (name, h))
        ref = run(path=arn.PATH_WAVE_ROW)
        if name == "int8":
            check_model(x, r, w, 1e-6, *ref, "wave_row int8 h=%d" % h)
        for path, block, grid in ((0, 0, 0), (arn.PATH_PACKED, 64, 5), (arn.PATH_PACKED, 1024, -1),
                                  (arn.PATH_PACKED, 256, 0)):
            got = run(path=path, block=block, grid=grid)
            assert np.array_equal(got[0], ref[0]), (name, h, path, block, grid)
            assert same_scale_bits(got[1], ref[1]), (name, h, path, block, grid)
            if ref[2] is not None:
                assert np.array_equal(got[2], ref[2]), (name, h, path, block, grid)


@pytest.mark.parametrize("h", [16, 128, 512])
def test_packed_quantised_rows_per_lane(h):
    """Every rows-per-lane setting of the packed kernel gives one wavefront
    per row's codes and scales, int8 and E4M3, fused and plain."""
    import torch

    from test_gpu_quant import same_scale_bits

    n = 300 + h % 29
    x, r, w = synth.workload(95 + h, n, h)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    calls = {
        "int8": (torch.int8, lambda q, sc, res, **c: arn.add_rmsnorm_quant_fwd_cfg(
            q, sc, res, xd, rd, wd, 1e-6, **c)),
        "fp8": (torch.uint8, lambda q, sc, res, **c: arn.add_rmsnorm_quant_fp8_fwd_cfg(
            q, sc, res, xd, rd, wd, 1e-6, **c)),
        "plain int8": (torch.int8, lambda q, sc, res, **c: arn.rmsnorm_quant_fwd_cfg(
            q, sc, xd, wd, 1e-6, **c)),
        "plain fp8": (torch.uint8, lambda q, sc, res, **c: arn.rmsnorm_quant_fp8_fwd_cfg(
            q, sc, xd, wd, 1e-6, **c)),
    }
    for name, (dtype, call) in calls.items():
        def run(**c):
            q = torch.full((n, h), 99, dtype=dtype, device=xd.device)
            sc = torch.full((n,), float("nan"), dtype=torch.float32, device=xd.device)
            res = poisoned_like(xd)
            call(q, sc, res, **c)
            torch.cuda.synchronize()
            return q.cpu().numpy(), sc.cpu().numpy(), from_dev(res)

        announce("packed quantised rows per lane %s h=%d" % (name, h))
        ref = run(path=arn.PATH_WAVE_ROW)
        for rpl in (1, 2, 4):
            for block, grid in ((64, 0), (512, 3)):
                got = run(path=arn.PATH_PACKED, block_threads=block, grid_blocks=grid,
                          rows_per_lane=rpl)
                assert np.array_equal(got[0], ref[0]), (name, h, rpl, block, grid)
                assert same_scale_bits(got[1], ref[1]), (name, h, rpl, block, grid)
                if not name.startswith("plain"):
                    assert np.array_equal(got[2], ref[2]), (name, h, rpl, block, grid)


def test_qk_benchmark_workload_sampled():
    """The benchmark's q/k workload at full size (4096 tokens x (32 + 8) heads
    x 128 from a [4096, 6144] qkv tensor) in its default launch; sampled
    tokens against the oracle and the fp32 model, and q_out and k_out fully
    written (no poison left)."""
    import torch

    t, hq, hk, d = 4096, 32, 8, 128
    buf, qw, kw = _qkv(8000, t, hq, hk, d)
    dev = to_dev(buf)
    q, k = _views(dev, hq, hk, d)
    q_out = poisoned_like(q.contiguous())
    k_out = poisoned_like(k.contiguous())
    announce("qk benchmark workload 4096 x (32 + 8) x 128")
    arn.qk_rmsnorm_fwd(q_out, k_out, q, k, to_dev(qw), to_dev(kw), 1e-6)
    torch.cuda.synchronize()
    qo, ko = from_dev(q_out), from_dev(k_out)
    # finite inputs give finite outputs, so any poison NaN left is an unwritten element
    assert not (qo == POISON).any() and not (ko == POISON).any()
    toks = sorted({0, 1, 2, 3, 63, 64, 1000, 2047, 2048, 4093, 4094, 4095})
    _check_heads(buf[toks], hq, hk, d, qw, kw, 1e-6, qo[toks], ko[toks], "qk benchmark workload")
