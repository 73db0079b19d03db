"""Tensors larger than 4 GiB (GPU): row offsets past 2^31 elements exercise
the 64-bit address arithmetic of every kernel path.

The rows are built on the GPU from a seeded block of 256 rows (x row i is
block row i mod 256, residual row i is block row (7 i + 3) mod 256), so the
oracle can compute any sampled row from the block alone.  Sampled rows,
including those on both sides of the 2^31-element boundary, are compared
with the oracle to the parity bar."""
import numpy as np
import pytest

import bf16_rounding_numerics_amd as arn
import synth
from gpu_helpers import announce, check_parity, require_gpu, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # (rows, hidden, forced configurations besides the default)
    (2 ** 20 + 5, 2048, [(arn.PATH_WG_ROW, 256, 0)]),
    (2 ** 18 + 3, 8192, [(arn.PATH_LDS_TWO_PASS, 1024, -1)]),
    (2 ** 17 + 3, 16384, [(arn.PATH_WG_ROW, 512, 0)]),
    (2 ** 24 + 5, 128, [(arn.PATH_PACKED, 1024, 3), (arn.PATH_WAVE_ROW, 256, 0)]),
]


@pytest.mark.parametrize("n,h,cfgs", CASES, ids=lambda v: str(v) if not isinstance(v, list) else "cfg")
def test_tensors_beyond_4gib(n, h, cfgs):
    require_gpu()
    import torch

    assert n * h > 2 ** 31
    bx, br, w = synth.workload(5000 + h, 256, h)
    ix = np.arange(n) % 256
    ir = (7 * np.arange(n) + 3) % 256
    dev = torch.device("cuda:0")
    announce("large %dx%d: building %.1f GiB per tensor" % (n, h, n * h * 2 / 2 ** 30))
    xd = to_dev(bx)[torch.from_numpy(ix).to(dev)]
    rd = to_dev(br)[torch.from_numpy(ir).to(dev)]
    wd = to_dev(w)
    edge = 2 ** 31 // h
    rows = sorted({0, 1, 255, 256, n // 2, edge - 1, edge, edge + 1, n - 2, n - 1})
    sel = torch.tensor(rows, device=dev)
    for path, block, grid in [(0, 0, 0)] + cfgs:
        announce("  path %d block %d grid %d" % (path, block, grid))
        out = torch.empty_like(xd)
        res = torch.empty_like(xd)
        if path:
            arn.add_rmsnorm_fwd_cfg(out, res, xd, rd, wd, 1e-6, path=path, block_threads=block,
                                    grid_blocks=grid)
        else:
            arn.add_rmsnorm_fwd(out, res, xd, rd, wd, 1e-6)
        torch.cuda.synchronize()
        got_out = out[sel].cpu().numpy().view(np.uint16)
        got_res = res[sel].cpu().numpy().view(np.uint16)
        check_parity(bx[ix[rows]], br[ir[rows]], w, 1e-6, got_out, got_res,
                     label="large %dx%d rows %s" % (n, h, rows))
        del out, res
    del xd, rd
    torch.cuda.empty_cache()


def _build(n, h, seed):
    import torch

    bx, br, w = synth.workload(seed, 256, h)
    ix = np.arange(n) % 256
    ir = (7 * np.arange(n) + 3) % 256
    dev = torch.device("cuda:0")
    xd = to_dev(bx)[torch.from_numpy(ix).to(dev)]
    rd = to_dev(br)[torch.from_numpy(ir).to(dev)]
    return bx, br, w, ix, ir, xd, rd, to_dev(w)


def _rows(n, h):
    edge = 2 ** 31 // h
    return sorted({0, 1, 255, 256, n // 2, edge - 1, edge, edge + 1, n - 2, n - 1})


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("n,h", [(2 ** 18 + 3, 8192), (2 ** 20 + 5, 2048)])
def test_quantised_beyond_4gib(n, h, fmt):
    """Codes and scales of the fused and plain quantised entry points on
    tensors past 2^31 elements, sampled rows bit-exact against the fp32
    model."""
    require_gpu()
    import torch

    import fp32_model

    assert n * h > 2 ** 31
    announce("large quantised %s %dx%d" % (fmt, n, h))
    bx, br, w, ix, ir, xd, rd, wd = _build(n, h, 5100 + h)
    rows = _rows(n, h)
    sel = torch.tensor(rows, device=xd.device)
    code = torch.int8 if fmt == "int8" else torch.uint8
    model = fp32_model.add_rmsnorm_quant if fmt == "int8" else fp32_model.add_rmsnorm_quant_fp8
    for plain in (False, True):
        announce("  %s" % ("plain" if plain else "fused"))
        q = torch.empty(n, h, dtype=code, device=xd.device)
        sc = torch.empty(n, dtype=torch.float32, device=xd.device)
        res = None
        if fmt == "int8" and plain:
            arn.rmsnorm_quant_fwd(q, sc, xd, wd, 1e-6)
        elif fmt == "int8":
            res = torch.empty_like(xd)
            arn.add_rmsnorm_quant_fwd(q, sc, res, xd, rd, wd, 1e-6)
        elif plain:
            arn.rmsnorm_quant_fp8_fwd(q, sc, xd, wd, 1e-6)
        else:
            res = torch.empty_like(xd)
            arn.add_rmsnorm_quant_fp8_fwd(q, sc, res, xd, rd, wd, 1e-6)
        torch.cuda.synchronize()
        mq, ms, mr = model(bx[ix[rows]], None if plain else br[ir[rows]], w, 1e-6)
        assert np.array_equal(q[sel].cpu().numpy().view(mq.dtype), mq), rows
        assert np.array_equal(sc[sel].cpu().numpy().view(np.uint32), ms.view(np.uint32)), rows
        if res is not None:
            assert np.array_equal(res[sel].cpu().numpy().view(np.uint16), mr), rows
        del q, sc, res
    del xd, rd
    torch.cuda.empty_cache()


def test_general_kernel_beyond_4gib():
    """hidden 8191 (no row 16-byte aligned) past 2^31 elements: the general
    kernel's 64-bit row offsets, sampled rows bit-exact against the fp32
    model."""
    require_gpu()
    import torch

    import fp32_model

    n, h = 2 ** 18 + 64, 8191
    assert n * h > 2 ** 31
    announce("large general %dx%d" % (n, h))
    bx, br, w, ix, ir, xd, rd, wd = _build(n, h, 5200)
    rows = _rows(n, h)
    sel = torch.tensor(rows, device=xd.device)
    out = torch.empty_like(xd)
    res = torch.empty_like(xd)
    arn.add_rmsnorm_fwd(out, res, xd, rd, wd, 1e-6)
    torch.cuda.synchronize()
    m_out, m_res = fp32_model.add_rmsnorm(bx[ix[rows]], br[ir[rows]], w, 1e-6)
    assert np.array_equal(out[sel].cpu().numpy().view(np.uint16), m_out), rows
    assert np.array_equal(res[sel].cpu().numpy().view(np.uint16), m_res), rows
    del out, res, xd, rd
    torch.cuda.empty_cache()
