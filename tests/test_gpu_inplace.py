"""In-place operation (GPU): an output may be the very buffer of an input,
the usual residual-stream update being out <- x and residual_out <- residual.
Results must be bit-identical to the out-of-place call, on every kernel path
and with persistent grids."""
import numpy as np
import pytest

import bf16_rounding_numerics_amd as arn
import synth
from gpu_helpers import announce, check_parity, from_dev, gpu_fwd, poisoned_like, require_gpu, to_dev

pytestmark = pytest.mark.gpu

MODES = ["out=x,residual_out=residual", "out=x", "residual_out=residual",
         "out=residual,residual_out=x"]


@pytest.mark.parametrize("grid", [0, -1])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("h", [24, 128, 256, 1024, 2048, 4096, 8192, 16384])
def test_in_place_matches_out_of_place(h, mode, grid):
    require_gpu()
    import torch

    n = 67
    x, r, w = synth.workload(3000 + h, n, h)
    announce("in place hidden %d %s grid %d" % (h, mode, grid))
    ref_out, ref_res = gpu_fwd(x, r, w, 1e-6)
    check_parity(x, r, w, 1e-6, ref_out, ref_res)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    out = {"out=x,residual_out=residual": xd, "out=x": xd, "residual_out=residual": None,
           "out=residual,residual_out=x": rd}[mode]
    res = {"out=x,residual_out=residual": rd, "out=x": None, "residual_out=residual": rd,
           "out=residual,residual_out=x": xd}[mode]
    out = poisoned_like(xd) if out is None else out
    res = poisoned_like(xd) if res is None else res
    arn.add_rmsnorm_fwd_cfg(out, res, xd, rd, wd, 1e-6, grid_blocks=grid)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out), ref_out)
    assert np.array_equal(from_dev(res), ref_res)


def test_in_place_chain():
    """Twelve calls updating the residual stream in place (residual_out ==
    residual) match the same chain run out of place."""
    require_gpu()
    import torch

    n, h = 256, 4096
    _, r0, w = synth.workload(4000, n, h)
    wd = to_dev(w)
    res_in_place = to_dev(r0)
    res_copy = to_dev(r0)
    announce("in-place chain")
    for step in range(12):
        xk = to_dev(synth.chain_delta(4000, step, n, h, 0.1))
        out_a = torch.empty_like(xk)
        arn.add_rmsnorm_fwd(out_a, res_in_place, xk, res_in_place, wd, 1e-6)
        out_b = torch.empty_like(xk)
        nxt = torch.empty_like(xk)
        arn.add_rmsnorm_fwd(out_b, nxt, xk, res_copy, wd, 1e-6)
        res_copy = nxt
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b) and torch.equal(res_in_place, res_copy)
