"""Calls from several host threads at once (GPU): the library keeps no state
between calls and is documented as safe to call from several threads.  Four
threads, each with its own stream and buffers, issue fused, plain, quantised
and q/k calls concurrently (ctypes releases the interpreter lock during each
call); every result must equal the same call made alone, bit for bit."""
import threading

import numpy as np
import pytest

import bf16_rounding_numerics_amd as arn
import synth
from gpu_helpers import announce, from_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _work(kind, seed):
    """(run(stream) -> outputs as numpy) for one thread's calls."""
    import torch

    dev = torch.device("cuda:0")
    if kind == "qk":
        rng = np.random.default_rng(seed)
        t, hq, hk, d = 97, 16, 4, 128
        qkv = to_dev(synth.to_bf16_bits(rng.standard_normal((t, (hq + 2 * hk) * d))))
        qw = to_dev(synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(d)))
        q, k = qkv[:, :hq * d].view(t, hq, d), qkv[:, hq * d:(hq + hk) * d].view(t, hk, d)
        qo = torch.empty(t, hq, d, dtype=torch.int16, device=dev)
        ko = torch.empty(t, hk, d, dtype=torch.int16, device=dev)

        def run(stream):
            arn.qk_rmsnorm_fwd(qo, ko, q, k, qw, qw, 1e-6, stream=stream)
            return from_dev(qo), from_dev(ko)
        return run
    n, h = 333, {"fused": 4096, "plain": 1000, "quant": 128}[kind]
    x, r, w = synth.workload(seed, n, h)
    xd, rd, wd = to_dev(x), to_dev(r), to_dev(w)
    out, res = torch.empty_like(xd), torch.empty_like(xd)
    q = torch.empty(n, h, dtype=torch.int8, device=dev)
    sc = torch.empty(n, dtype=torch.float32, device=dev)

    def run(stream):
        if kind == "fused":
            arn.add_rmsnorm_fwd(out, res, xd, rd, wd, 1e-6, stream=stream)
            return from_dev(out), from_dev(res)
        if kind == "plain":
            arn.rmsnorm_fwd(out, xd, wd, 1e-6, stream=stream)
            return (from_dev(out),)
        arn.add_rmsnorm_quant_fwd(q, sc, res, xd, rd, wd, 1e-6, stream=stream)
        return q.cpu().numpy(), sc.cpu().numpy(), from_dev(res)
    return run


def test_concurrent_host_threads():
    require_gpu()
    import torch

    kinds = ["fused", "plain", "quant", "qk"]
    runs = [_work(k, 5100 + i) for i, k in enumerate(kinds)]
    announce("threads: reference calls")
    ref = []
    for run in runs:
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            out = run(s)
        torch.cuda.synchronize()
        ref.append([a.copy() for a in out])
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            for rep in range(40):
                # the copies back to the host run on this thread's current
                # stream, which must be s so that they follow the kernels
                with torch.cuda.stream(s):
                    got = runs[i](s)
                for a, b in zip(got, ref[i]):
                    if not np.array_equal(a.view(np.uint8), b.view(np.uint8)):
                        errors.append((kinds[i], rep))
                        return
        except Exception as e:  # reported below, with the thread's kind
            errors.append((kinds[i], repr(e)))

    announce("threads: four at once")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(runs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
