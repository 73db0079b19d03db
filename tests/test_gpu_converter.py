"""The store epilogue over every fp32 bit pattern (GPU).

The fused kernels round both stores with gfx950's packed fp32 -> bf16
conversion.  The library's test hook runs that same device routine over
consecutive bit patterns; all 2^32 results must equal the oracle's
round-to-nearest-even (any NaN for a NaN input).  This settles subnormal,
overflow, tie and NaN behaviour of the hardware conversion.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import announce, is_nan16, require_gpu

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28


def test_epilogue_matches_oracle_on_all_fp32_patterns():
    require_gpu()
    import torch

    import bf16_rounding_numerics_amd as arn

    buf = torch.empty(CHUNK, dtype=torch.int16, device="cuda:0")
    mismatches = 0
    nan_sign_kept = True
    for start in range(0, 1 << 32, CHUNK):
        announce("cvt range start 0x%08x" % start)
        arn.add_rmsnorm_test_cvt_range(buf, start)
        torch.cuda.synchronize()
        got = buf.cpu().numpy().view(np.uint16)
        exp = oracle.rne16_range(start, CHUNK)
        diff = got != exp
        if diff.any():
            nan_in = is_nan16(exp)
            ok_nan = nan_in & is_nan16(got)
            nan_sign_kept &= bool((((got[ok_nan] ^ exp[ok_nan]) & 0x8000) == 0).all())
            bad = diff & ~ok_nan
            if bad.any():
                idx = np.argwhere(bad)[:5].ravel()
                announce("  mismatches at %s: got %s expected %s" % (
                    [hex(start + int(i)) for i in idx], [hex(int(got[i])) for i in idx],
                    [hex(int(exp[i])) for i in idx]))
            mismatches += int(bad.sum())
    announce("NaN sign kept by the hardware conversion: %s" % nan_sign_kept)
    assert mismatches == 0
