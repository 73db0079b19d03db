"""The seeded input generator: SplitMix64 against its published outputs, and
the properties the workloads rely on."""
import numpy as np

import synth


def test_splitmix64_published_sequence():
    # SplitMix64 started from state 0 (Steele, Lea & Flood; the reference
    # implementation's first three outputs).
    z = synth.splitmix64(0, 0, 3)
    assert [int(v) for v in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_splitmix64_is_counter_based():
    full = synth.splitmix64(12345, 0, 1000)
    part = synth.splitmix64(12345, 400, 100)
    assert np.array_equal(full[400:500], part)


def test_normal_moments_and_determinism():
    a = synth.normal(7, 0, 1 << 20)
    b = synth.normal(7, 0, 1 << 20)
    assert np.array_equal(a, b)
    assert abs(a.mean()) < 5e-3 and abs(a.std() - 1) < 5e-3
    c = synth.normal(7, 1, 1 << 20)
    assert not np.array_equal(a, c)
    # odd lengths and chunking do not change values
    d = synth.normal(7, 0, 1001, chunk=16)
    assert np.array_equal(a[:1001], d)


def test_workload_distributions():
    x, r, w = synth.workload(seed=1, n_rows=64, hidden=1024)
    assert x.dtype == np.uint16 and x.shape == (64, 1024) and w.shape == (1024,)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(f(x).std() - 1) < 0.02 and abs(f(r).std() - 1) < 0.02
    assert abs(f(w).mean() - 1) < 0.01 and abs(f(w).std() - 0.1) < 0.01


def test_bf16_rounding_of_generated_values():
    v = np.array([1.0, 1.00390625, 1.01171875, -2.5], dtype=np.float64)
    assert list(synth.to_bf16_bits(v)) == [0x3F80, 0x3F80, 0x3F82, 0xC020]
