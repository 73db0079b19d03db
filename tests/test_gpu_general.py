"""General shapes on the GPU: any hidden, unaligned pointers, row-strided views.

Bars, as for the contiguous fast kernels:
  * bit-exact against the fp32 model (which pads a partial last segment with
    zeros, the canonical tree's own padding), within one bf16 ULP of the
    oracle with residual_out bit-exact;
  * the general kernel gives the fast kernels' bits where both apply, for
    every workgroup size and grid;
  * strided views give the contiguous results on the same rows and write
    nothing outside their rows.
"""
import numpy as np
import pytest

import bf16_rounding_numerics_amd as arn
import fp32_model
import synth
from gpu_helpers import (POISON, announce, check_parity, from_dev, gpu_fwd, is_nan16,
                         poisoned_like, require_gpu, to_dev, ulp_distance)
from test_gpu_parity import _special_rows

pytestmark = pytest.mark.gpu

BLOCKS = (64, 128, 256, 512, 1024)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def same16(a, b):
    return np.array_equal(a, b) or not ((a != b) & ~(is_nan16(a) & is_nan16(b))).any()


def check_model(x, r, w, eps, out, res, label):
    m_out, m_res = fp32_model.add_rmsnorm(x, r, w, eps)
    assert same16(out, m_out), "%s: out differs from the fp32 model in %d" % (
        label, int(((out != m_out) & ~(is_nan16(out) & is_nan16(m_out))).sum()))
    if r is not None:
        assert same16(res, m_res), "%s: residual_out differs from the fp32 model" % label


def gpu_plain(x, w, eps=1e-6, path=0, block=0, grid=0):
    import torch

    xd, wd = to_dev(x), to_dev(w)
    out = poisoned_like(xd)
    arn.rmsnorm_fwd_cfg(out, xd, wd, eps, path=path, block_threads=block, grid_blocks=grid)
    torch.cuda.synchronize()
    return from_dev(out)


HIDDEN = [1, 3, 7, 9, 15, 100, 513, 575, 577, 1001, 1601, 2049, 4095, 4097, 8191, 12289, 16385,
          24577, 32767]


@pytest.mark.parametrize("h", HIDDEN)
def test_any_hidden(h):
    n = 37 if h < 8192 else 9
    announce("general hidden %d, %d rows" % (h, n))
    x, r, w = synth.workload(5200 + h, n, h)
    out, res = gpu_fwd(x, r, w, 1e-6)
    check_model(x, r, w, 1e-6, out, res, "h=%d" % h)
    check_parity(x, r, w, 1e-6, out, res, label="h=%d" % h)
    p = gpu_plain(x, w)
    check_model(x, None, w, 1e-6, p, None, "plain h=%d" % h)


@pytest.mark.parametrize("h", [9, 1001, 16385])
def test_any_hidden_special_values(h):
    announce("general special values hidden %d" % h)
    x, r = _special_rows(h)
    w = synth.bf16_normal(5300 + h, 2, (h,), 1.0, 0.5)
    out, res = gpu_fwd(x, r, w, 1e-6)
    check_model(x, r, w, 1e-6, out, res, "special h=%d" % h)
    p = gpu_plain(x, w)
    check_model(x, None, w, 1e-6, p, None, "plain special h=%d" % h)


@pytest.mark.parametrize("h", [64, 1000, 2048, 4096, 8192, 16384, 32768])
def test_general_path_gives_the_fast_kernels_bits(h):
    import torch

    n = 19
    x, r, w = synth.workload(5400 + h, n, h)
    announce("general vs fast, hidden %d" % h)
    ref_out, ref_res = gpu_fwd(x, r, w, 1e-6)
    ref_plain = gpu_plain(x, w)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    for b in BLOCKS:
        for grid in (0, 7, -1):
            out, res = gpu_fwd(x, r, w, 1e-6, path=arn.PATH_GENERAL, block=b, grid=grid,
                               xd=xd, rd=rd, wd=wd)
            assert np.array_equal(out, ref_out) and np.array_equal(res, ref_res), (b, grid)
            o = poisoned_like(xd)
            arn.rmsnorm_fwd_cfg(o, xd, wd, 1e-6, path=arn.PATH_GENERAL, block_threads=b,
                                grid_blocks=grid)
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(o), ref_plain), (b, grid)


@pytest.mark.parametrize("h", [1100, 1601, 1663, 2600, 4095, 6143, 9001, 12289, 17000, 28001])
def test_general_blocks_and_grids_agree_on_odd_rows(h):
    """Every workgroup size and grid of the general path gives the fp32
    model's bits on rows that start anywhere in a 128-byte line: one to four
    segments per thread, blocks past the row's end (1100 at 64 threads,
    2600 at 128, 9001 and 12289 at 1024), rows that fill every block, the
    line-aligned accesses (last block above 128 elements) beside the
    row-relative ones (1100, 1663), and rows above 16384 (the long-row
    kernel at 1024 threads, the LDS kernel below).  With 22 rows, the grid
    of 7 gives each workgroup three or more rows, so the line-aligned rows
    with one segment per thread take the form that writes shared lines
    whole there."""
    import torch

    n = 22
    x, r, w = synth.workload(5450 + h, n, h)
    announce("general blocks x grids, hidden %d" % h)
    m_out, m_res = fp32_model.add_rmsnorm(x, r, w, 1e-6)
    m_plain, _ = fp32_model.add_rmsnorm(x, None, w, 1e-6)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    for b in BLOCKS:
        for grid in (0, 7, -1):
            out, res = gpu_fwd(x, r, w, 1e-6, path=arn.PATH_GENERAL, block=b, grid=grid,
                               xd=xd, rd=rd, wd=wd)
            assert same16(out, m_out) and same16(res, m_res), (b, grid)
            o = poisoned_like(xd)
            arn.rmsnorm_fwd_cfg(o, xd, wd, 1e-6, path=arn.PATH_GENERAL, block_threads=b,
                                grid_blocks=grid)
            torch.cuda.synchronize()
            assert same16(from_dev(o), m_plain), (b, grid)


@pytest.mark.parametrize("h", [4096, 24000])
def test_unaligned_pointers_take_the_general_kernel(h):
    import torch

    n = 24
    x, r, w = synth.workload(5500, n, h)
    announce("general: pointers offset by one element")
    ref_out, ref_res = gpu_fwd(x, r, w, 1e-6)
    # each tensor one element past a 16-byte boundary
    def shifted(a):
        buf = torch.empty(a.size + 8, dtype=torch.int16, device="cuda:0")
        view = buf[1:1 + a.size]
        view.copy_(to_dev(a.reshape(-1)))
        return view.view(a.shape) if a.ndim > 1 else view

    xd, rd, wd = shifted(x), shifted(r), shifted(w)
    ob = torch.full((n * h + 8,), np.int16(np.uint16(POISON).view(np.int16)), dtype=torch.int16,
                    device="cuda:0")
    rb = ob.clone()
    out, res = ob[1:1 + n * h].view(n, h), rb[1:1 + n * h].view(n, h)
    arn.add_rmsnorm_fwd(out, res, xd, rd, wd, 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out), ref_out) and np.array_equal(from_dev(res), ref_res)
    assert from_dev(ob)[0] == POISON and (from_dev(ob)[1 + n * h:] == POISON).all()


@pytest.mark.parametrize("h", [1100, 4095, 8191, 9001, 16383, 20000])
def test_tensors_at_different_line_offsets(h):
    """x, residual, out and residual_out each start at a different element
    offset (0, 1, 3 and 63 elements past a 256-byte boundary), so every row
    of each tensor sits at its own place in its 128-byte lines: the
    line-aligned accesses (4095, 8191, 16383) and the row-relative ones
    (1100, 9001) give the contiguous bits and write nothing outside."""
    import torch

    n = 23
    x, r, w = synth.workload(5600 + h, n, h)
    announce("general: tensors at different line offsets, hidden %d" % h)
    ref_out, ref_res = gpu_fwd(x, r, w, 1e-6)

    def placed(a, off, fill=None):
        buf = torch.full((a.size + 128,), np.int16(np.uint16(POISON).view(np.int16)),
                         dtype=torch.int16, device="cuda:0")
        view = buf[off:off + a.size]
        if fill is not None:
            view.copy_(to_dev(fill.reshape(-1)))
        return buf, view.view(a.shape)

    _, xd = placed(x, 0, x)
    _, rd = placed(r, 1, r)
    ob, out = placed(x, 3)
    rb, res = placed(x, 63)
    arn.add_rmsnorm_fwd(out, res, xd, rd, to_dev(w), 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out), ref_out) and np.array_equal(from_dev(res), ref_res)
    for buf, off in ((ob, 3), (rb, 63)):
        b = from_dev(buf)
        assert (b[:off] == POISON).all() and (b[off + n * h:] == POISON).all()
    pb, po = placed(x, 7)
    arn.rmsnorm_fwd(po, rd, to_dev(w), 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(po), gpu_plain(r, w))
    b = from_dev(pb)
    assert (b[:7] == POISON).all() and (b[7 + n * h:] == POISON).all()


@pytest.mark.parametrize("h", [16385, 17000, 24001, 32705, 32767, 32768])
def test_long_rows_sharing_a_line_offset_write_only_their_rows(h):
    """Rows above 16384 whose four tensors all start 5 elements past a
    256-byte boundary take the line-aligned long-row kernel (18 to 34
    elements per thread).  At 16385 and 17000 each thread's last access lies
    wholly past every row; from 32705 up the rows need the 34-element form.
    The fused op and plain RMSNorm give the fp32 model's bits at every grid
    tried and write nothing before or after the tensors, including the 4 KiB
    that the accesses past the last row would reach."""
    import torch

    n, off, tail = 7, 5, 4096
    x, r, w = synth.workload(5700 + h, n, h)
    announce("general: long rows sharing a line offset, hidden %d" % h)
    m_out, m_res = fp32_model.add_rmsnorm(x, r, w, 1e-6)
    m_plain, _ = fp32_model.add_rmsnorm(x, None, w, 1e-6)
    wd = to_dev(w)

    def placed(fill=None):
        buf = torch.full((off + n * h + tail,), np.int16(np.uint16(POISON).view(np.int16)),
                         dtype=torch.int16, device="cuda:0")
        view = buf[off:off + n * h]
        if fill is not None:
            view.copy_(to_dev(fill.reshape(-1)))
        return buf, view.view(n, h)

    def untouched(buf):
        b = from_dev(buf)
        return (b[:off] == POISON).all() and (b[off + n * h:] == POISON).all()

    _, xd = placed(x)
    _, rd = placed(r)
    for grid in (0, 3, n):
        ob, out = placed()
        rb, res = placed()
        arn.add_rmsnorm_fwd_cfg(out, res, xd, rd, wd, 1e-6, path=arn.PATH_GENERAL,
                                grid_blocks=grid)
        torch.cuda.synchronize()
        assert same16(from_dev(out), m_out) and same16(from_dev(res), m_res), grid
        assert untouched(ob) and untouched(rb), grid
        pb, po = placed()
        arn.rmsnorm_fwd_cfg(po, xd, wd, 1e-6, path=arn.PATH_GENERAL, grid_blocks=grid)
        torch.cuda.synchronize()
        assert same16(from_dev(po), m_plain) and untouched(pb), grid


IN_PLACE_MODES = ["out=x,residual_out=residual", "out=x", "residual_out=residual",
                  "out=residual,residual_out=x"]


@pytest.mark.parametrize("grid", [0, 2])
@pytest.mark.parametrize("mode", IN_PLACE_MODES)
@pytest.mark.parametrize("h", [1001, 1663, 4095, 9001, 16383, 17000, 32767])
def test_general_kernels_in_place(h, mode, grid):
    """An output that is an input's own buffer, on each general kernel: one
    wavefront per row (1001), the register kernel row-relative (1663) and
    line-aligned (4095, 9001, 16383; with two workgroups, 4095 takes the
    form that writes each line two blocks share whole, after the row's
    barrier), the long-row kernel line-aligned (17000, 32767).  Every
    element's inputs are read before its outputs are written, so the results
    are the fp32 model's bits, as out of place."""
    import torch

    n = 13
    x, r, w = synth.workload(5800 + h, n, h)
    announce("general in place: hidden %d, %s" % (h, mode))
    m_out, m_res = fp32_model.add_rmsnorm(x, r, w, 1e-6)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    out = {"out=x,residual_out=residual": xd, "out=x": xd, "residual_out=residual": None,
           "out=residual,residual_out=x": rd}[mode]
    res = {"out=x,residual_out=residual": rd, "out=x": None, "residual_out=residual": rd,
           "out=residual,residual_out=x": xd}[mode]
    out = poisoned_like(xd) if out is None else out
    res = poisoned_like(xd) if res is None else res
    arn.add_rmsnorm_fwd_cfg(out, res, xd, rd, wd, 1e-6, path=arn.PATH_GENERAL, grid_blocks=grid)
    torch.cuda.synchronize()
    assert same16(from_dev(out), m_out) and same16(from_dev(res), m_res)


@pytest.mark.parametrize("h", [767, 1001, 1025, 1663, 2047, 2600, 4095, 6143, 8191, 8192, 9001,
                               10300, 12287, 12289, 16001, 16383])
def test_whole_line_form_writes_only_its_rows(h):
    """All four tensors 5 elements past a 256-byte boundary, and few enough
    workgroups that each takes three or more rows: the register kernel
    writes every line two blocks share whole, from the first block's
    wavefront (with two segments per thread, 9001 to 16383 at 1024 threads,
    reading that line's x and residual again after the barrier; 9001 and
    12287 with blocks past the row's end; 1025, 1663, 2600, 10300 and 12289
    with a short last block; 767 and 1001, rows one wavefront would take
    otherwise).
    The fp32 model's bits, fused and plain, at every workgroup size with one
    or two segments per thread, and nothing written before or after the
    tensors (the last block's whole-line stores past the row's end are
    dropped)."""
    import torch

    n, off, tail = 12, 5, 1024
    x, r, w = synth.workload(6000 + h, n, h)
    announce("general whole-line form: hidden %d" % h)
    m_out, m_res = fp32_model.add_rmsnorm(x, r, w, 1e-6)
    m_plain, _ = fp32_model.add_rmsnorm(x, None, w, 1e-6)
    wd = to_dev(w)

    def placed(fill=None):
        buf = torch.full((off + n * h + tail,), np.int16(np.uint16(POISON).view(np.int16)),
                         dtype=torch.int16, device="cuda:0")
        view = buf[off:off + n * h]
        if fill is not None:
            view.copy_(to_dev(fill.reshape(-1)))
        return buf, view.view(n, h)

    def untouched(buf):
        b = from_dev(buf)
        return (b[:off] == POISON).all() and (b[off + n * h:] == POISON).all()

    _, xd = placed(x)
    _, rd = placed(r)
    for b in BLOCKS:
        if b * 16 < h:
            continue  # one or two segments per thread only
        for grid in (1, 2, 4):
            ob, out = placed()
            rb, res = placed()
            arn.add_rmsnorm_fwd_cfg(out, res, xd, rd, wd, 1e-6, path=arn.PATH_GENERAL,
                                    block_threads=b, grid_blocks=grid)
            torch.cuda.synchronize()
            assert same16(from_dev(out), m_out) and same16(from_dev(res), m_res), (b, grid)
            assert untouched(ob) and untouched(rb), (b, grid)
            pb, po = placed()
            arn.rmsnorm_fwd_cfg(po, xd, wd, 1e-6, path=arn.PATH_GENERAL, block_threads=b,
                                grid_blocks=grid)
            torch.cuda.synchronize()
            assert same16(from_dev(po), m_plain) and untouched(pb), (b, grid)


@pytest.mark.parametrize("h", [4095, 9001, 20000])
def test_general_in_place_tensors_at_different_offsets(h):
    """out = x and residual_out = residual with x one element past a 256-byte
    boundary and residual on it, so the two streams sit at different places
    in their lines: the register kernel's line-aligned form with a line
    offset per tensor (4095, 9001) and the long-row kernel's row-relative
    form (20000), in place."""
    import torch

    n = 9
    x, r, w = synth.workload(5900 + h, n, h)
    announce("general in place, tensors at different offsets: hidden %d" % h)
    m_out, m_res = fp32_model.add_rmsnorm(x, r, w, 1e-6)
    buf = torch.empty(n * h + 128, dtype=torch.int16, device="cuda:0")
    xv = buf[1:1 + n * h].view(n, h)
    xv.copy_(to_dev(x))
    rd = to_dev(r)
    arn.add_rmsnorm_fwd(xv, rd, xv, rd, to_dev(w), 1e-6)
    torch.cuda.synchronize()
    assert same16(from_dev(xv), m_out) and same16(from_dev(rd), m_res)


def _matrix(rows, cols, fill=POISON):
    import torch

    return torch.full((rows, cols), np.int16(np.uint16(fill).view(np.int16)), dtype=torch.int16,
                      device="cuda:0")


@pytest.mark.parametrize("h,ld,offs", [
    (4096, 3 * 4096, (0, 4096, 8192)),        # column blocks, fast-kernel aligned
    (1024, 1024 + 8, (0, 0, 0)),              # padded rows, aligned
    (2048, 5001, (8, 16, 24)),                # a stride not a multiple of 8: general
    (1000, 3001, (1, 1001, 2001)),            # odd strides and offsets: general
    (16384, 16384 * 2, (0, 16384, 0)),        # two-pass kernel on strided rows
])
def test_strided_views(h, ld, offs):
    import torch

    n = 17
    announce("strided views: hidden %d, row stride %d, column offsets %s" % (h, ld, offs))
    x, r, w = synth.workload(5600 + h, n, h)
    ref_out, ref_res = gpu_fwd(x, r, w, 1e-6)
    ox, orr, oo = offs
    X = _matrix(n, ld)                       # x lives in X, residual in R
    R = _matrix(n, ld)
    X[:, ox:ox + h] = to_dev(x)
    R[:, orr:orr + h] = to_dev(r)
    O = _matrix(n, ld)                       # out and residual_out, poisoned around
    RO = _matrix(n, ld + 16)
    wd = to_dev(w)
    out, res = O[:, oo:oo + h], RO[:, 16:16 + h]
    arn.add_rmsnorm_fwd_strided(out, res, X[:, ox:ox + h], R[:, orr:orr + h], wd, 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out), ref_out)
    assert np.array_equal(from_dev(res), ref_res)
    Oh, ROh = from_dev(O), from_dev(RO)
    mask = np.ones_like(Oh, bool)
    mask[:, oo:oo + h] = False
    assert (Oh[mask] == POISON).all(), "out wrote outside its rows"
    mask = np.ones_like(ROh, bool)
    mask[:, 16:16 + h] = False
    assert (ROh[mask] == POISON).all(), "residual_out wrote outside its rows"
    # plain RMSNorm on the same strided x
    ref_plain = gpu_plain(x, w)
    P = _matrix(n, ld)
    arn.rmsnorm_fwd_strided(P[:, oo:oo + h], X[:, ox:ox + h], wd, 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(P[:, oo:oo + h]), ref_plain)


@pytest.mark.parametrize("h,ld", [(4096, 8192), (1001, 2003)])
def test_strided_in_place(h, ld):
    """out = x and residual_out = residual on strided views (residual stream
    update inside wider buffers)."""
    import torch

    n = 11
    announce("strided in place: hidden %d, row stride %d" % (h, ld))
    x, r, w = synth.workload(5700 + h, n, h)
    ref_out, ref_res = gpu_fwd(x, r, w, 1e-6)
    B = _matrix(n, ld)
    B[:, :h] = to_dev(x)
    B[:, ld - h:] = to_dev(r)
    xv, rv = B[:, :h], B[:, ld - h:]
    arn.add_rmsnorm_fwd_strided(xv, rv, xv, rv, to_dev(w), 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(xv), ref_out) and np.array_equal(from_dev(rv), ref_res)
    if ld - h > h:
        assert (from_dev(B)[:, h:ld - h] == POISON).all()
