"""The division behind the packed kernel's two-level row addressing: row i of
a group is token i / heads, taken as the high 64 bits of i * M with
M = ceil(2^64 / heads), assembled from 32-bit halves as the kernel does
((i * M_hi + mulhi32(i, M_lo)) >> 32).  Exact for every i < 2^32 because
M * heads - 2^64 < heads; checked here for every head count up to 4096 at the
values of i where a quotient changes, near 2^31 and near 2^32."""
import numpy as np


def _kernel_div(i, heads):
    m = (2 ** 64 - 1) // heads + 1
    lo, hi = m & 0xFFFFFFFF, m >> 32
    a = (i * hi + ((i * lo) >> 32)) & (2 ** 64 - 1)   # the kernel's 64-bit sum
    return a >> 32


def test_reciprocal_division_is_exact():
    rng = np.random.default_rng(3)
    for heads in range(2, 4097):
        tops = [2 ** 32 - 1, 2 ** 32 - 2, 2 ** 31, 2 ** 31 - 1]
        qs = [(2 ** 32 - 1) // heads, (2 ** 31) // heads, 1, 2, 1000]
        ivals = set(tops)
        for q in qs:
            for d in (-1, 0, 1):
                i = q * heads + d
                if 0 <= i < 2 ** 32:
                    ivals.add(i)
        ivals.update(int(v) for v in rng.integers(0, 2 ** 32, 16, dtype=np.uint64))
        for i in ivals:
            assert _kernel_div(i, heads) == i // heads, (i, heads)


def test_the_sum_never_overflows_64_bits():
    # i * M_hi + mulhi32(i, M_lo) < 2^64 for i < 2^32, so no carry is lost
    for heads in (2, 3, 5, 7, 40, 4095):
        m = (2 ** 64 - 1) // heads + 1
        i = 2 ** 32 - 1
        assert i * (m >> 32) + ((i * (m & 0xFFFFFFFF)) >> 32) < 2 ** 64
