"""Capture in HIP graphs, and concurrent streams (GPU).

The entry points only validate on the host and launch on the given stream
(no allocation, no memset, no synchronisation), so a call can be captured in
a graph and replayed.  Each replay here is checked against the eager result,
with fresh inputs copied in and eager work and synchronisation between the
replays; and two streams running at once must give what they give alone.
"""
import numpy as np
import pytest

import bf16_rounding_numerics_amd as arn
import synth
from gpu_helpers import announce, from_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("quant", [False, True])
@pytest.mark.parametrize("h", [1024, 8192, 16384])
def test_graph_replays_match_eager(h, quant):
    require_gpu()
    import torch

    n = 96
    announce("graph replay hidden %d quant %s" % (h, quant))
    w = to_dev(synth.bf16_normal(4100 + h, 2, (h,), 1.0, 0.1))
    xs = torch.empty(n, h, dtype=torch.int16, device="cuda:0")
    rs = torch.empty_like(xs)
    out = torch.empty_like(xs)
    res = torch.empty_like(xs)
    q = torch.empty(n, h, dtype=torch.int8, device="cuda:0")
    sc = torch.empty(n, dtype=torch.float32, device="cuda:0")

    def call(o, ro, x, r, qq, ss):
        if quant:
            arn.add_rmsnorm_quant_fwd(qq, ss, ro, x, r, w, 1e-6)
        else:
            arn.add_rmsnorm_fwd(o, ro, x, r, w, 1e-6)

    # warm up outside the graph, then capture
    call(out, res, xs.zero_(), rs.zero_(), q, sc)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, res, xs, rs, q, sc)
    torch.cuda.synchronize()

    for rep in range(4):
        x, r, _ = synth.workload(4200 + 10 * rep + h, n, h)
        xs.copy_(to_dev(x))
        rs.copy_(to_dev(r))
        g.replay()
        # eager reference on separate buffers, plus unrelated eager work
        eo, er = torch.empty_like(xs), torch.empty_like(xs)
        eq, es = torch.empty_like(q), torch.empty_like(sc)
        call(eo, er, to_dev(x), to_dev(r), eq, es)
        _ = (xs.float() * 2).sum()
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(res), from_dev(er)), rep
        if quant:
            assert torch.equal(q, eq) and torch.equal(sc.view(torch.int32), es.view(torch.int32))
        else:
            assert np.array_equal(from_dev(out), from_dev(eo)), rep


def test_two_streams_at_once():
    require_gpu()
    import torch

    announce("two streams")
    x1, r1, w = synth.workload(4300, 1024, 8192)
    x2, r2, _ = synth.workload(4301, 1024, 8192)
    wd = to_dev(w)
    a = [to_dev(v) for v in (x1, r1, x2, r2)]
    ref = []
    for x, r in ((a[0], a[1]), (a[2], a[3])):
        o, ro = torch.empty_like(x), torch.empty_like(x)
        arn.add_rmsnorm_fwd(o, ro, x, r, wd, 1e-6)
        ref.append((o, ro))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(5):
        o1, ro1 = torch.empty_like(a[0]), torch.empty_like(a[0])
        o2, ro2 = torch.empty_like(a[0]), torch.empty_like(a[0])
        arn.add_rmsnorm_fwd(o1, ro1, a[0], a[1], wd, 1e-6, stream=s1)
        arn.add_rmsnorm_fwd(o2, ro2, a[2], a[3], wd, 1e-6, stream=s2)
        outs.append((o1, ro1, o2, ro2))
    torch.cuda.synchronize()
    for o1, ro1, o2, ro2 in outs:
        assert torch.equal(o1, ref[0][0]) and torch.equal(ro1, ref[0][1])
        assert torch.equal(o2, ref[1][0]) and torch.equal(ro2, ref[1][1])


@pytest.mark.parametrize("kind", ["plain", "plain_quant", "plain_quant_fp8", "strided_general",
                                  "log1p"])
def test_graph_replays_of_the_other_entry_points(kind):
    """Plain RMSNorm (resident grid by default), a strided view on the
    general kernels, and log1p (capped persistent grid), each captured once
    and replayed on fresh inputs, checked against eager calls."""
    require_gpu()
    import torch

    announce("graph replay: %s" % kind)
    n, h = 64, 4096
    dev = "cuda:0"
    if kind == "log1p":
        xs = torch.empty(1 << 20, dtype=torch.float32, device=dev)
        out = torch.empty_like(xs)

        def call(o, x):
            arn.log1p_f32(o, x)
    elif kind == "strided_general":
        h = 1001
        X = torch.zeros(n, 2 * h + 3, dtype=torch.int16, device=dev)
        O = torch.zeros_like(X)
        RO = torch.zeros_like(X)
        xs, out = X[:, 1:1 + h], O[:, 2:2 + h]
        res = RO[:, 3:3 + h]
        rs = torch.empty(n, h, dtype=torch.int16, device=dev)
        w = to_dev(synth.bf16_normal(4400, 2, (h,), 1.0, 0.1))

        def call(o, x):
            arn.add_rmsnorm_fwd_strided(o, res if o is out else torch.empty_like(rs), x, rs, w,
                                        1e-6)
    else:
        xs = torch.empty(n, h, dtype=torch.int16, device=dev)
        w = to_dev(synth.bf16_normal(4400, 2, (h,), 1.0, 0.1))
        if kind == "plain":
            out = torch.empty_like(xs)

            def call(o, x):
                arn.rmsnorm_fwd(o, x, w, 1e-6)
        elif kind == "plain_quant":
            out = torch.empty(n, h, dtype=torch.int8, device=dev)
            sc = torch.empty(n, dtype=torch.float32, device=dev)

            def call(o, x):
                arn.rmsnorm_quant_fwd(o, sc if o is out else torch.empty_like(sc), x, w, 1e-6)
        else:
            out = torch.empty(n, h, dtype=torch.uint8, device=dev)
            sc = torch.empty(n, dtype=torch.float32, device=dev)

            def call(o, x):
                arn.rmsnorm_quant_fp8_fwd(o, sc if o is out else torch.empty_like(sc), x, w, 1e-6)

    def fresh(rep):
        if kind == "log1p":
            return torch.from_numpy(synth.uniform_f32(4500 + rep, 0, xs.numel())).to(dev)
        x, r, _ = synth.workload(4500 + rep, n, h)
        if kind == "strided_general":
            rs.copy_(to_dev(r))
        return to_dev(x)

    xs.copy_(fresh(0))
    call(out, xs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, xs)
    torch.cuda.synchronize()
    for rep in range(1, 4):
        x = fresh(rep)
        xs.copy_(x)
        g.replay()
        eager_out = torch.empty_like(out)
        call(eager_out, x.contiguous() if kind != "strided_general" else xs.contiguous())
        _ = (xs.float() * 2).sum()
        torch.cuda.synchronize()
        assert torch.equal(out.contiguous(), eager_out.contiguous()), (kind, rep)
