"""Benchmark of the fused residual-add + RMSNorm forward on one MI355X.

(--op selects the int8-quantised variant or plain RMSNorm instead; the
default is the fused bf16 op.)

A step is one add_rmsnorm_fwd call over the 4096 x 8192 bf16 workload
(x, residual ~ N(0,1), weight ~ 1 + 0.1 N(0,1), eps = 1e-6), with the inputs
already resident in HBM.  The timed region is K back-to-back steps on one
stream, bracketed by device synchronisation and measured with HIP events on
that stream.  Successive steps rotate over several buffer sets whose total
footprint exceeds MI355X's 256 MB last-level cache, so each step streams from
HBM rather than from cache.

Output: one JSON line with the throughput in GB/s of algorithmic traffic
(read x and residual, write out and residual_out: 8 bytes per element, plus
the weight once), the HBM roofline fraction against 8 TB/s, and the CPU
oracle timed on the host as a baseline.

  python bench.py [--steps K] [--warmup W] [--workload 4096x8192]
                  [--op bf16|quant|quant_fp8|plain|plain_quant|plain_quant_fp8|general|log1p]
                  [--no-cpu-baseline] [--calibrate-copy] [--ceilings] [--size-sweep]
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
CACHE_DEFEAT_BYTES = 1 << 30  # rotate buffer sets until the footprint is >= 1 GiB


OPS = ("bf16", "quant", "quant_fp8", "plain", "plain_quant", "plain_quant_fp8", "general",
       "log1p", "qk", "chain")
ENTRY = {"bf16": "add_rmsnorm_fwd", "quant": "add_rmsnorm_quant_fwd",
         "quant_fp8": "add_rmsnorm_quant_fp8_fwd", "plain": "rmsnorm_fwd",
         "plain_quant": "rmsnorm_quant_fwd", "plain_quant_fp8": "rmsnorm_quant_fp8_fwd",
         "general": "add_rmsnorm_fwd (general kernel)", "log1p": "log1p_f32",
         "qk": "qk_rmsnorm_fwd", "chain": "add_rmsnorm_fwd (72-call chain)"}
QUANT_OPS = ("quant", "quant_fp8", "plain_quant", "plain_quant_fp8")
PLAIN_OPS = ("plain", "plain_quant", "plain_quant_fp8")


def algorithmic_bytes(n_rows: int, hidden: int, op: str = "bf16") -> int:
    """Bytes the method must move per call: x, residual read and residual_out
    written (2 bytes each per element), out written (2 bytes per element, or
    for the quantised variants 1 byte of code per element and a 4-byte scale
    per row); the weight read once.  Plain RMSNorm has no residual and no
    residual_out."""
    per_elem = {"bf16": 8, "general": 8, "quant": 7, "quant_fp8": 7, "plain": 4,
                "plain_quant": 3, "plain_quant_fp8": 3}[op]
    per_row = 4 if op in QUANT_OPS else 0
    return per_elem * n_rows * hidden + per_row * n_rows + 2 * hidden


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="4096x8192")
    p.add_argument("--op", choices=OPS, default="bf16",
                   help="bf16: the fused op (the benchmark); quant, quant_fp8: its int8- "
                        "and FP8 E4M3-quantised variants; plain, plain_quant, "
                        "plain_quant_fp8: RMSNorm without the residual add; "
                        "general: the fused op on the general kernel (the workload's hidden "
                        "minus one, so rows leave 16-byte alignment); "
                        "log1p: the correctly rounded binary32 log1p; "
                        "qk: per-head RMSNorm of q and k read from a fused qkv tensor "
                        "(--qk-shape); chain: the 72-call residual-stream chain on 2048 x 4096 "
                        "(residual_out fed back in place, fresh x ~ N(0, 0.1^2) per call), "
                        "launched eagerly and as one HIP-graph replay")
    p.add_argument("--hot", action="store_true",
                   help="also time the call on one buffer set with no rotation (cache-assisted; "
                        "off by default so that a kernel trace of the default run holds only "
                        "the benchmarked launches)")
    p.add_argument("--no-compare", action="store_true",
                   help="--op qk: skip the same-rows comparison launches (for profiling)")
    p.add_argument("--qk-shape", default="4096x32x8x128",
                   help="tokens x q heads x k heads x head_dim of --op qk (default: "
                        "Qwen3-8B attention at 4096 tokens)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="time budget of the CPU oracle baseline")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain device copy of known size (counter calibration)")
    p.add_argument("--graph", action="store_true",
                   help="launch the timed steps as one HIP graph (replayed once) instead of "
                        "one call each from Python")
    p.add_argument("--size-sweep", action="store_true",
                   help="time the fused call and same-bytes streams at 1024..8192 rows of the "
                        "workload's hidden and fit steady rate and fixed cost per launch")
    p.add_argument("--ceilings", action="store_true",
                   help="measure the device's read-only, write-only and 50/50 copy streaming "
                        "rates at the workload's bytes, beside the fused kernel")
    return p.parse_args(argv)


def env_info(torch, arn):
    """The run's environment: device, software versions, host CPU and the
    library's build identity (target, flags, source digest)."""
    props = torch.cuda.get_device_properties(0)
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", ""),
            "hip": torch.version.hip, "torch": torch.__version__, "host_cpu": cpu,
            "host_nproc": os.cpu_count(), "library_build": arn.add_rmsnorm_build_info()}


def sha256_of(*arrays):
    """Short SHA-256 digests of input buffers (the seeded generator's output
    depends on the host's libm, so the digests identify the inputs)."""
    import hashlib

    return [hashlib.sha256(a.tobytes()).hexdigest()[:16] for a in arrays]


def traffic_from_profiles(kernel_tag: str, workload: str, digest: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s_%s.txt" % (kernel_tag, workload))
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        m = re.match(r"^(\w+):\s*(\S+)", line)
        if m:
            fields[m.group(1)] = m.group(2)
    if fields.get("sources_sha256") != digest:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def run_copy_calibration(torch, nbytes=1 << 30, reps=20):
    """A plain device-to-device copy of nbytes, for reading what FETCH_SIZE and
    WRITE_SIZE report for a known byte count."""
    src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": nbytes, "reps": reps}))


def copy_ceiling(torch, arn, bufs, steps, n_rows, hidden, plain=False):
    """The same bytes moved by the library's reference copy (x -> one output
    buffer, residual -> the other; 16-byte nontemporal loads and stores, no
    arithmetic), rotated like the kernel's buffers: the streaming rate this
    device gives the kernel's 50/50 read/write mix.  For plain RMSNorm the
    copy moves x alone (its two halves), the bytes that op moves."""
    sets = len(bufs)
    half = n_rows * hidden // 2

    def one(i):
        o, ro, xd, rd = bufs[i % sets]
        if plain:
            ov, xv = o.view(-1), xd.view(-1)
            arn.add_rmsnorm_test_copy2(ov[:half], ov[half:], xv[:half], xv[half:])
        else:
            arn.add_rmsnorm_test_copy2(ro, o, xd, rd)

    for i in range(min(steps, 20)):
        one(i)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        one(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    return (4 if plain else 8) * n_rows * hidden / (ms * 1e-3) / 1e9


def cpu_baseline(x, r, w, eps, n_rows, hidden, budget_s, op="bf16"):
    """The oracle (single-threaded C) over the whole workload, repeated until the
    time budget is spent."""
    import oracle

    oracle.default()
    passes = 0
    t0 = time.perf_counter()
    while True:
        if op == "quant":
            oracle.add_rmsnorm_quant(x, r, w, eps)
        elif op == "plain":
            oracle.rmsnorm(x, w, eps)
        elif op == "plain_quant":
            oracle.rmsnorm_quant(x, w, eps)
        elif op == "quant_fp8":
            oracle.add_rmsnorm_quant_fp8(x, r, w, eps)
        elif op == "plain_quant_fp8":
            oracle.add_rmsnorm_quant_fp8(x, None, w, eps)
        else:
            oracle.add_rmsnorm(x, r, w, eps)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    gbps = algorithmic_bytes(n_rows, hidden, op) * passes / el / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d full passes over the %dx%d workload in %.1f s (single thread)"
                      % (passes, n_rows, hidden, el)}


def time_steps(torch, step, steps, warmup, stream):
    """Average milliseconds of `step` over `steps` back-to-back calls on one
    stream (HIP events), after `warmup` untimed ones; also the wall time."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, time.perf_counter() - t_wall


def bench_log1p(args, torch, arn, hip_build, synth):
    """One step: log1p_f32 over 2^26 binary32 inputs uniform on [0, 1) (the TE
    issue's reproducer distribution at a size that streams from HBM), rotating
    over buffer sets like the norm benchmark.  8 bytes per element: read x,
    write out."""
    n = synth.LOG1P_BENCH_N
    dev = torch.device("cuda:0")
    x = synth.uniform_f32(synth.LOG1P_SEED, 1, n)
    sets = max(1, -(-CACHE_DEFEAT_BYTES // (8 * n)))
    xs = [torch.from_numpy(x).to(dev)]
    xs += [xs[0].clone() for _ in range(sets - 1)]
    outs = [torch.empty_like(xs[0]) for _ in range(sets)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ms, wall_s = time_steps(torch, lambda i: arn.log1p_f32(outs[i % sets], xs[i % sets]),
                            args.steps, args.warmup, stream)
    nbytes = 8 * n
    gbps = nbytes / (ms * 1e-3) / 1e9

    # the same bytes through the reference copy: x's halves into out's halves
    def copy(i):
        xv, ov = xs[i % sets].view(torch.int16), outs[i % sets].view(torch.int16)
        arn.add_rmsnorm_test_copy2(ov[:n], ov[n:], xv[:n], xv[n:])

    cms, _ = time_steps(torch, copy, min(args.steps, 500), 10, stream)
    copy_gbps = nbytes / (cms * 1e-3) / 1e9
    traffic = traffic_from_profiles("log1p", "n%d" % n, hip_build.source_digest())
    line = {
        "metric": "log1p_f32 (correctly rounded binary32 log1p) HBM GB/s and % of peak",
        "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "log1p_f32 n=%d fp32, x uniform on [0, 1)" % n, "n": n,
                   "buffer_sets": sets,
                   "elements_per_s": round(n / (ms * 1e-3), 1),
                   "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
                   "wall_s_timed_region": round(wall_s, 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic},
        "copy_ceiling": {"gbps": round(copy_gbps, 2),
                         "kernel_frac_of_copy": round(gbps / copy_gbps, 4),
                         "frac_of_peak": round(copy_gbps / PEAK_HBM_GBPS, 4),
                         "what": "add_rmsnorm_test_copy2 moving x's two halves into out"},
        "inputs_sha256": {"x": sha256_of(x)[0]},
        "env": env_info(torch, arn),
    }
    if not args.no_cpu_baseline:
        import oracle

        lo = oracle.default_log1p()
        sample = x[: 1 << 20]
        passes, t0 = 0, time.perf_counter()
        while True:
            lo.log1p_f32(sample)
            passes += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        line["cpu_baseline"] = {
            "value": round(8 * sample.size * passes / el / 1e9, 5), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d passes over the first 2^20 inputs of the workload in %.1f s "
                      "(binary128 log1pq, single thread)" % (passes, el)}
    print(json.dumps(line))
    return 0


def bench_qk(args, torch, arn, hip_build, synth):
    """One step: qk_rmsnorm_fwd over a [tokens, (q_heads + 2 k_heads) head_dim]
    bf16 qkv tensor (q and k read as strided views, written to contiguous q_out
    and k_out), rotating over buffer sets.  4 bytes per q or k element (read,
    write) plus the two weights."""
    import numpy as np

    t, hq, hk, d = (int(v) for v in args.qk_shape.split("x"))
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(11)
    qkv = synth.to_bf16_bits(rng.standard_normal((t, (hq + 2 * hk) * d)))
    qw = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(d))
    kw = synth.to_bf16_bits(1 + 0.1 * rng.standard_normal(d))
    elems = t * (hq + hk) * d
    nbytes = 4 * elems + 4 * d
    sets = max(1, -(-CACHE_DEFEAT_BYTES // (2 * qkv.size + 2 * elems)))
    base = torch.from_numpy(qkv.view(np.int16)).to(dev)
    bufs = []
    for i in range(sets):
        b = base if i == 0 else base.clone()
        q = b[:, :hq * d].view(t, hq, d)
        k = b[:, hq * d:(hq + hk) * d].view(t, hk, d)
        bufs.append((torch.empty(t, hq, d, dtype=torch.int16, device=dev),
                     torch.empty(t, hk, d, dtype=torch.int16, device=dev), q, k))
    qwd = torch.from_numpy(qw.view(np.int16)).to(dev)
    kwd = torch.from_numpy(kw.view(np.int16)).to(dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def step(i):
        qo, ko, q, k = bufs[i % sets]
        arn.qk_rmsnorm_fwd(qo, ko, q, k, qwd, kwd, 1e-6)

    ms, wall_s = time_steps(torch, step, args.steps, args.warmup, stream)
    gbps = nbytes / (ms * 1e-3) / 1e9

    # The same head rows, contiguous, through rmsnorm_fwd: one wavefront per
    # row (the path before the packed kernel) and the packed path, two
    # launches per step (q rows, then k rows).
    rows = [(torch.empty(t * hq, d, dtype=torch.int16, device=dev),
             torch.empty(t * hk, d, dtype=torch.int16, device=dev)) for _ in range(sets)]
    outs = [(torch.empty_like(a), torch.empty_like(b)) for a, b in rows]

    def rows_step(path):
        def f(i):
            (qr, kr), (qo, ko) = rows[i % sets], outs[i % sets]
            arn.rmsnorm_fwd_cfg(qo, qr, qwd, 1e-6, path=path)
            arn.rmsnorm_fwd_cfg(ko, kr, kwd, 1e-6, path=path)
        return f

    steps_cmp = min(args.steps, 500)
    if not args.no_compare:
        ms_wave, _ = time_steps(torch, rows_step(arn.PATH_WAVE_ROW), steps_cmp, 10, stream)
        ms_pack, _ = time_steps(torch, rows_step(arn.PATH_PACKED), steps_cmp, 10, stream)
    traffic = traffic_from_profiles("pack_rows_qk", args.qk_shape, hip_build.source_digest())
    line = {
        "metric": "per-head q/k RMSNorm (qk_rmsnorm_fwd) HBM GB/s and % of peak",
        "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qk_rmsnorm_fwd tokens=%d q_heads=%d k_heads=%d head_dim=%d "
                               "bf16 from a fused qkv tensor, eps=1e-6, q,k~N(0,1), "
                               "weights~1+0.1N(0,1)" % (t, hq, hk, d),
                   "tokens": t, "q_heads": hq, "k_heads": hk, "head_dim": d,
                   "kernel": "pack_rows", "buffer_sets": sets,
                   "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
                   "wall_s_timed_region": round(wall_s, 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic},
        "inputs_sha256": dict(zip(("qkv", "q_weight", "k_weight"), sha256_of(qkv, qw, kw))),
        "env": env_info(torch, arn),
    }
    if not args.no_compare:
        line["same_rows_two_rmsnorm_calls"] = {
            "wave_row_ms": round(ms_wave, 6), "packed_ms": round(ms_pack, 6),
            "wave_row_gbps": round(nbytes / (ms_wave * 1e-3) / 1e9, 2),
            "packed_gbps": round(nbytes / (ms_pack * 1e-3) / 1e9, 2),
            "what": "the q and k head rows as contiguous [rows, head_dim] tensors, one "
                    "rmsnorm_fwd_cfg call each, forced onto one wavefront per row or the "
                    "packed path"}
    if not args.no_cpu_baseline:
        import oracle

        oracle.default()
        ts = min(t, 256)
        qs = qkv[:ts, :hq * d].reshape(ts, hq, d)
        ks = qkv[:ts, hq * d:(hq + hk) * d].reshape(ts, hk, d)
        passes, t0 = 0, time.perf_counter()
        while True:
            oracle.qk_rmsnorm(qs, ks, qw, kw, 1e-6)
            passes += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        line["cpu_baseline"] = {
            "value": round(4 * ts * (hq + hk) * d * passes / el / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": "%d passes over the first %d tokens of the workload in %.1f s "
                      "(single thread)" % (passes, ts, el)}
    print(json.dumps(line))
    return 0


def bench_chain(args, torch, arn, synth):
    """One step: the 72-call chain of the aiter issue's reproducer at 2048 x
    4096 (36 layers x 2 norms): call k reads a fresh x_k and the residual
    stream, writes out and the new residual stream in place (residual_out is
    residual).  The 72 x_k stay resident (1.2 GB, beyond the last-level
    cache).  Timed eagerly (72 launches per step) and as one HIP graph of the
    72 calls replayed per step."""
    import numpy as np

    n, h, depth, seed = 2048, 4096, 72, 2
    dev = torch.device("cuda:0")
    _, r0, w = synth.workload(seed, n, h)
    # The 72 fresh x_k: N(0, 0.1^2) from numpy's seeded generator (the same
    # distribution as the chain tests' inputs, generated 20x faster; timing
    # does not depend on the values).
    rng = np.random.default_rng(1000 + seed)
    xs_host = [synth.to_bf16_bits(rng.standard_normal((n, h)) * 0.1) for _ in range(depth)]
    xs = [torch.from_numpy(x.view(np.int16)).to(dev) for x in xs_host]
    wd = torch.from_numpy(w.view(np.int16)).to(dev)
    res = torch.from_numpy(r0.view(np.int16)).to(dev)
    out = torch.empty_like(res)
    stream = torch.cuda.current_stream(dev)

    def chain(_i=0):
        for k in range(depth):
            arn.add_rmsnorm_fwd(out, res, xs[k], res, wd, 1e-6)

    steps = max(1, min(args.steps, 200))
    ms_eager, wall_eager = time_steps(torch, chain, steps, max(1, min(args.warmup, 5)), stream)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        chain()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    ms_graph, wall_graph = time_steps(torch, lambda i: g.replay(), steps,
                                      max(1, min(args.warmup, 5)), stream)
    per_call = algorithmic_bytes(n, h)
    gbps_eager = depth * per_call / (ms_eager * 1e-3) / 1e9
    gbps_graph = depth * per_call / (ms_graph * 1e-3) / 1e9
    line = {
        "metric": "72-call fused add+RMSNorm chain (2048 x 4096 bf16) HBM GB/s and % of peak",
        "value": round(gbps_graph, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": max(1, min(args.warmup, 5)), "ms_per_step": round(ms_graph, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "72 x add_rmsnorm_fwd rows=2048 hidden=4096 bf16, residual_out "
                               "fed back in place, fresh x~N(0,0.1^2) per call, residual_0~N(0,1), "
                               "weight~1+0.1N(0,1), eps=1e-6",
                   "calls_per_step": depth, "launch": "one HIP graph of the 72 calls per step",
                   "cache_note": "the residual stream (16 MB, updated in place) and out stay "
                                 "in the 256 MB last-level cache between calls; the 72 x_k "
                                 "(1.2 GB) stream from HBM",
                   "us_per_call": round(ms_graph * 1e3 / depth, 3),
                   "pct_of_peak": round(100 * gbps_graph / PEAK_HBM_GBPS, 2),
                   "wall_s_timed_region": round(wall_graph, 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbps_graph, 2), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(gbps_graph / PEAK_HBM_GBPS, 4),
                     "traffic": None},
        "eager": {"ms_per_step": round(ms_eager, 6), "gbps": round(gbps_eager, 2),
                  "us_per_call": round(ms_eager * 1e3 / depth, 3),
                  "what": "the same 72 calls launched one by one from Python"},
        "inputs_sha256": {"residual_0": sha256_of(r0)[0], "weight": sha256_of(w)[0],
                          "x_0": sha256_of(xs_host[0])[0]},
        "env": env_info(torch, arn),
    }
    if not args.no_cpu_baseline:
        import oracle

        oracle.default()
        rows = 128
        rc = r0[:rows].copy()
        calls, t0 = 0, time.perf_counter()
        while True:
            _o, rc = oracle.add_rmsnorm(xs_host[calls % depth][:rows], rc, w, 1e-6)
            calls += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        line["cpu_baseline"] = {
            "value": round(algorithmic_bytes(rows, h) * calls / el / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": "%d chain calls on the first %d rows in %.1f s (single thread)"
                      % (calls, rows, el)}
    print(json.dumps(line))
    return 0


def ceilings(args, torch, arn, synth):
    """Streaming rates of the device with the fused kernels' access pattern,
    at the bytes of one fused call on the workload (x and residual read, out
    and residual_out written), each over rotated buffers and one launch per
    step: read-only, write-only, the 2-in/2-out copy, and the fused kernel."""
    import numpy as np

    n_rows, hidden = (int(v) for v in args.workload.split("x"))
    dev = torch.device("cuda:0")
    count = n_rows * hidden              # elements per tensor
    sets = max(1, -(-CACHE_DEFEAT_BYTES // (8 * count)))
    x, r, w = synth.workload(3, n_rows, hidden)
    bufs = []
    for _ in range(sets):
        xd = torch.from_numpy(x.view(np.int16)).to(dev)
        rd = torch.from_numpy(r.view(np.int16)).to(dev)
        bufs.append((torch.empty_like(xd), torch.empty_like(xd), xd, rd))
    wd = torch.from_numpy(w.view(np.int16)).to(dev)
    # one contiguous buffer of four tensors' bytes per set, for the
    # one-directional streams
    big = [torch.empty(4 * count, dtype=torch.int16, device=dev) for _ in range(sets)]
    sink = torch.empty_like(big[0])
    stream = torch.cuda.current_stream(dev)
    steps = min(args.steps, 1000)
    moved = 8 * count                    # bytes per step in every case

    def rate(fn):
        ms, _ = time_steps(torch, fn, steps, 20, stream)
        return round(moved / (ms * 1e-3) / 1e9, 1)

    def read(i):
        arn.add_rmsnorm_test_stream(sink, big[i % sets], 0)

    def write(i):
        b = big[i % sets]
        arn.add_rmsnorm_test_stream(b, b, 1)

    def copy(i):
        o, ro, xd, rd = bufs[i % sets]
        arn.add_rmsnorm_test_copy2(ro, o, xd, rd)

    def fused(i):
        o, ro, xd, rd = bufs[i % sets]
        arn.add_rmsnorm_fwd(o, ro, xd, rd, wd, 1e-6)

    def copy_rows(burst):
        def f(i):
            o, ro, xd, rd = bufs[i % sets]
            arn.add_rmsnorm_test_copy_rows(ro, o, xd, rd, burst)
        return f

    def torch_copy(i):
        o, ro, xd, rd = bufs[i % sets]
        ro.copy_(xd)
        o.copy_(rd)

    res = {"read_only": rate(read), "write_only": rate(write), "copy_2in_2out": rate(copy)}
    if hidden % 8 == 0 and hidden <= 16384:
        for burst in (1, 2, 4):
            res["copy_rows_burst%d" % burst] = rate(copy_rows(burst))
    res["torch_device_copy"] = rate(torch_copy)
    res["add_rmsnorm_fwd"] = rate(fused)
    copies = {k: v for k, v in res.items() if k.startswith("copy") or k == "torch_device_copy"}
    best_copy = max(copies, key=copies.get)
    print(json.dumps({"ceilings_GBps": res, "peak_GBps": PEAK_HBM_GBPS,
                      "frac_of_peak": {k: round(v / PEAK_HBM_GBPS, 4) for k, v in res.items()},
                      "best_copy": best_copy,
                      "fused_frac_of_best_copy": round(res["add_rmsnorm_fwd"] / copies[best_copy], 4),
                      "workload": args.workload, "bytes_per_step": moved, "buffer_sets": sets,
                      "what": "8 * rows * hidden bytes per step: read-only and write-only stream "
                              "one buffer of four tensors' size; the copies read two tensors and "
                              "write two: copy_2in_2out grid-stride, copy_rows_burstR one "
                              "workgroup per R rows with all R rows loaded before any store, "
                              "torch_device_copy two device-to-device tensor copies; the fused "
                              "call reads x and residual and writes out and residual_out"}))
    return 0


def size_sweep(args, torch, arn):
    """The fused call and same-bytes streams at several row counts, hidden
    fixed: per-launch time against bytes moved.  A least-squares line
    t = fixed + bytes / rate gives each one's steady streaming rate (the
    slope) and its fixed cost per launch (start-up and drain, the intercept).
    Rows 1024 .. 8192 of the workload's hidden; inputs N(0,1) (weight
    1 + 0.1 N(0,1)) drawn on the device from a seeded generator, the same
    distributions as the benchmark; buffer sets rotated past the last-level
    cache; each case timed in 3 interleaved rounds, the median kept."""
    hidden = int(args.workload.split("x")[1])
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    rows_list = (1024, 2048, 4096, 8192)
    kinds = ("add_rmsnorm_fwd", "copy_2in_2out", "read_only", "write_only")
    # The fused call at the launch its default takes for 4096 rows at this
    # hidden, at every size (smaller calls would otherwise take another).
    if hidden <= 2048:
        pinned = dict(path=arn.PATH_WAVE_ROW, block_threads=256)
    elif hidden <= 8192:
        pinned = dict(path=arn.PATH_WG_ROW, block_threads=512)
    else:
        pinned = dict(path=arn.PATH_LDS_TWO_PASS, block_threads=1024)
    w = (1.0 + 0.1 * torch.randn(hidden, generator=gen, device=dev)).to(torch.bfloat16)
    w = w.view(torch.int16)
    cases = {}
    for n in rows_list:
        count = n * hidden
        sets = max(1, -(-CACHE_DEFEAT_BYTES // (8 * count)))
        bufs = []
        for _ in range(sets):
            xd = torch.randn(n, hidden, generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
            rd = torch.randn(n, hidden, generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
            bufs.append((torch.empty_like(xd), torch.empty_like(xd), xd, rd))
        big = [torch.empty(4 * count, dtype=torch.int16, device=dev) for _ in range(sets)]
        sink = torch.empty_like(big[0])

        def fused(i, bufs=bufs, sets=sets):
            o, ro, xd, rd = bufs[i % sets]
            arn.add_rmsnorm_fwd_cfg(o, ro, xd, rd, w, 1e-6, **pinned)

        def copy(i, bufs=bufs, sets=sets):
            o, ro, xd, rd = bufs[i % sets]
            arn.add_rmsnorm_test_copy2(ro, o, xd, rd)

        def read(i, big=big, sets=sets, sink=sink):
            arn.add_rmsnorm_test_stream(sink, big[i % sets], 0)

        def write(i, big=big, sets=sets):
            b = big[i % sets]
            arn.add_rmsnorm_test_stream(b, b, 1)

        cases[n] = (8 * count, dict(zip(kinds, (fused, copy, read, write))), bufs, big, sink)
    times = {(n, k): [] for n in rows_list for k in kinds}
    steps = min(args.steps, 400)
    for _ in range(3):
        for n in rows_list:
            for k in kinds:
                ms, _ = time_steps(torch, cases[n][1][k], steps, 10, stream)
                times[(n, k)].append(ms * 1e3)
    out = {"workload": "rows 1024..8192 x hidden %d" % hidden, "steps_per_case": steps,
           "fused_launch": {k: v for k, v in pinned.items()}, "us_per_launch": {}, "fit": {}}
    for k in kinds:
        xs, ys = [], []
        for n in rows_list:
            t = sorted(times[(n, k)])[1]
            out["us_per_launch"].setdefault(k, {})[str(n)] = round(t, 3)
            xs.append(cases[n][0])
            ys.append(t)
        mx, my = sum(xs) / len(xs), sum(ys) / len(ys)
        slope = sum((a - mx) * (b - my) for a, b in zip(xs, ys)) / sum((a - mx) ** 2 for a in xs)
        fixed = my - slope * mx
        rate = 1e-3 / slope  # bytes per us -> GB/s
        out["fit"][k] = {"steady_GBps": round(rate, 1), "steady_frac_of_peak": round(rate / PEAK_HBM_GBPS, 4),
                         "fixed_us_per_launch": round(fixed, 3)}
    print(json.dumps(out))
    return 0


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(rows would shard across GPUs with no communication); run with --gpus 1",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import bf16_rounding_numerics_amd as arn
    from bf16_rounding_numerics_amd import build as hip_build
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    arn.lib()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")

    if args.calibrate_copy:
        run_copy_calibration(torch)
        return 0
    if args.ceilings:
        return ceilings(args, torch, arn, synth)
    if args.size_sweep:
        return size_sweep(args, torch, arn)
    if args.op == "log1p":
        return bench_log1p(args, torch, arn, hip_build, synth)
    if args.op == "qk":
        return bench_qk(args, torch, arn, hip_build, synth)
    if args.op == "chain":
        return bench_chain(args, torch, arn, synth)

    n_rows, hidden = (int(v) for v in args.workload.split("x"))
    cfg = synth.CONFIGS.get(args.workload, dict(seed=3, n_rows=n_rows, hidden=hidden))
    if args.op == "general":
        hidden -= 1   # hidden % 8 != 0: every row off 16-byte alignment
    eps = 1e-6
    x, r, w = synth.workload(cfg["seed"], n_rows, hidden)
    tensor_bytes = n_rows * hidden * 2
    plain = args.op in PLAIN_OPS
    touched = (2 if plain else 4) * tensor_bytes   # bf16 tensors one step reads or writes
    sets = max(1, -(-CACHE_DEFEAT_BYTES // touched))
    xd0 = torch.from_numpy(x.view(np.int16)).to(dev)
    rd0 = torch.from_numpy(r.view(np.int16)).to(dev)
    wd = torch.from_numpy(w.view(np.int16)).to(dev)
    bufs = []
    for i in range(sets):
        xd = xd0 if i == 0 else xd0.clone()
        rd = rd0 if i == 0 else rd0.clone()
        bufs.append((torch.empty_like(xd), torch.empty_like(xd), xd, rd))
    qbufs = []
    if args.op in QUANT_OPS:
        code_dtype = torch.uint8 if args.op.endswith("fp8") else torch.int8
        for i in range(sets):
            qbufs.append((torch.empty(n_rows, hidden, dtype=code_dtype, device=dev),
                          torch.empty(n_rows, dtype=torch.float32, device=dev)))
    torch.cuda.synchronize()

    def step(i):
        o, ro, xd, rd = bufs[i % sets]
        if args.op == "quant":
            q, sc = qbufs[i % sets]
            arn.add_rmsnorm_quant_fwd(q, sc, ro, xd, rd, wd, eps)
        elif args.op == "plain":
            arn.rmsnorm_fwd(o, xd, wd, eps)
        elif args.op == "general":
            arn.add_rmsnorm_fwd_cfg(o, ro, xd, rd, wd, eps, path=arn.PATH_GENERAL)
        elif args.op == "plain_quant":
            q, sc = qbufs[i % sets]
            arn.rmsnorm_quant_fwd(q, sc, xd, wd, eps)
        elif args.op == "quant_fp8":
            q, sc = qbufs[i % sets]
            arn.add_rmsnorm_quant_fp8_fwd(q, sc, ro, xd, rd, wd, eps)
        elif args.op == "plain_quant_fp8":
            q, sc = qbufs[i % sets]
            arn.rmsnorm_quant_fp8_fwd(q, sc, xd, wd, eps)
        else:
            arn.add_rmsnorm_fwd(o, ro, xd, rd, wd, eps)

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    graph = None
    if args.graph:
        # All timed steps captured in one HIP graph and replayed once: the
        # same launches back to back with no host work between them, so a
        # profiler's cost per launch leaves no idle gaps between kernels.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    if graph is not None:
        # the replayed results must be those of an eager call on the same set
        last = (args.steps - 1) % sets
        replayed = [t.clone() for t in bufs[last][:2]] + ([t.clone() for t in qbufs[last]]
                                                         if qbufs else [])
        step(last)
        torch.cuda.synchronize()
        eager = list(bufs[last][:2]) + (list(qbufs[last]) if qbufs else [])
        for k in range(len(eager)):
            if args.op in QUANT_OPS and k == 0:
                continue  # the bf16 out buffer is unused by the quantised ops
            if args.op in PLAIN_OPS and k == 1:
                continue  # no residual_out in plain RMSNorm
            if not torch.equal(replayed[k], eager[k]):
                raise RuntimeError("graph replay differs from an eager call")
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps
    nbytes = algorithmic_bytes(n_rows, hidden, args.op)
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9

    copy_gbps = copy_ceiling(torch, arn, bufs, min(args.steps, 500), n_rows, hidden, plain)
    # --hot: the same call on one buffer set, no rotation: the 256 MB
    # last-level cache then keeps part of the working set between steps
    # (labelled as cache-assisted; never the reported value).
    if args.hot:
        hot_ms, _ = time_steps(torch, lambda i: step(0), min(args.steps, 500), 10, stream)
        hot_gbps = nbytes / (hot_ms * 1e-3) / 1e9

    if args.op == "general":
        path = "general"
    elif (args.op in ("bf16", "plain") and hidden <= 256) or (args.op in QUANT_OPS and
                                                                hidden <= 512):
        path = "pack_rows"
    elif args.op == "bf16":
        path = "wave_row" if hidden <= 2048 else "wg_row" if hidden <= 8192 else "lds_two_pass"
    else:  # the quantised and plain variants keep rows in registers up to 16384
        path = "wave_row" if hidden <= 1024 else "wg_row" if hidden <= 16384 else "lds_two_pass"
    digest = hip_build.source_digest()
    tag = path if args.op in ("bf16", "general") else path + "_" + args.op
    traffic = traffic_from_profiles(tag, args.workload, digest)
    roofline = {"bound": "hbm", "achieved": round(gbps, 2), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                "traffic": traffic}

    line = {
        "metric": {"bf16": "fused add+RMSNorm HBM GB/s and % of peak, n=4096 x hidden=8192 bf16",
                   "quant": "fused add+RMSNorm, int8-quantised out, HBM GB/s and % of peak",
                   "quant_fp8": "fused add+RMSNorm, FP8 E4M3-quantised out, HBM GB/s and % "
                                "of peak",
                   "plain_quant_fp8": "RMSNorm (no residual add), FP8 E4M3-quantised out, HBM "
                                      "GB/s and % of peak",
                   "plain": "RMSNorm (no residual add), HBM GB/s and % of peak",
                   "plain_quant": "RMSNorm (no residual add), int8-quantised out, HBM GB/s "
                                  "and % of peak",
                   "general": "fused add+RMSNorm on the general kernel (hidden % 8 != 0), "
                              "HBM GB/s and % of peak"}[args.op],
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s rows=%d hidden=%d bf16, eps=1e-6, "
                               "x,residual~N(0,1), weight~1+0.1N(0,1)"
                               % (ENTRY[args.op], n_rows, hidden),
                   "n_rows": n_rows, "hidden": hidden, "kernel": path,
                   "launch": "one HIP graph of all steps" if args.graph else "one call per step",
                   "buffer_sets": sets, "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
                   "wall_s_timed_region": round(wall_s, 4)},
        "roofline": roofline,
        "copy_ceiling": {"gbps": round(copy_gbps, 2),
                         "kernel_frac_of_copy": round(gbps / copy_gbps, 4)
                         if args.op in ("bf16", "plain", "general") else None,
                         "frac_of_peak": round(copy_gbps / PEAK_HBM_GBPS, 4),
                         "what": "add_rmsnorm_test_copy2 over the same bytes: two 16-byte "
                                 "nontemporal streaming copies, no arithmetic, same buffer rotation"},
        "inputs_sha256": dict(zip(("x", "residual", "weight"), sha256_of(x, r, w))),
        "env": env_info(torch, arn),
    }
    if args.hot:
        line["hot_cache_assisted"] = {
            "gbps": round(hot_gbps, 2), "ms_per_step": round(hot_ms, 6),
            "what": "the same call repeated on one buffer set (no rotation): part of the working "
                    "set stays in the 256 MB last-level cache between steps"}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, r, w, eps, n_rows, hidden, args.cpu_seconds,
                                            args.op)
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
