"""The library driven from plain C on the GPU, with no Python or torch in the
process: tests/c_abi/gpu_caller (built by build()) allocates with hipMalloc,
calls add_rmsnorm_fwd on its own stream and qk_rmsnorm_fwd in place on a
fused qkv tensor, and writes the results back.  They must meet the parity bar
against the oracle, like the same calls made through the Python binding."""
import os
import subprocess

import numpy as np
import pytest

import synth
from gpu_helpers import announce, check_parity, require_gpu
from test_gpu_qk import _check_heads, _qkv

pytestmark = pytest.mark.gpu

CALLER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "gpu_caller")


def test_c_program_through_the_abi(tmp_path):
    require_gpu()
    assert os.path.exists(CALLER), "tests/c_abi/gpu_caller is missing: run build() first"
    n, h = 257, 4096
    t, hq, hk, d = 33, 32, 8, 128
    x, r, w = synth.workload(61, n, h)
    qkv, qw, kw = _qkv(62, t, hq, hk, d)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    src.write_bytes(b"".join(a.astype(np.uint16).tobytes() for a in (x, r, w, qkv, qw, kw)))
    announce("C caller: %dx%d fused, %d tokens x (%d+%d) x %d q/k" % (n, h, t, hq, hk, d))
    p = subprocess.run([CALLER, str(src), str(dst), str(n), str(h), str(t), str(hq), str(hk),
                        str(d)], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stdout + p.stderr
    raw = np.frombuffer(dst.read_bytes(), dtype=np.uint16)
    out = raw[:n * h].reshape(n, h)
    res = raw[n * h:2 * n * h].reshape(n, h)
    got_qkv = raw[2 * n * h:].reshape(t, -1)
    check_parity(x, r, w, 1e-6, out, res, bias=1e-4, label="C caller")
    assert np.array_equal(got_qkv[:, (hq + hk) * d:], qkv[:, (hq + hk) * d:]), "v was written"
    _check_heads(qkv, hq, hk, d, qw, kw, 1e-6, got_qkv[:, :hq * d].reshape(t, hq, d),
                 got_qkv[:, hq * d:(hq + hk) * d].reshape(t, hk, d), "C caller q/k")
