"""bench.py's output contract.  On the CPU: more than one GPU is refused with a
message and exit status 2.  On the GPU: a short run prints one JSON line with
the metric, the whole-job value, the roofline of the dominant kernel and the
CPU oracle baseline, for the benchmark and for the q/k and chain workloads, and the
--graph, --ceilings and --size-sweep lines."""
import json
import os
import subprocess
import sys

import pytest

from gpu_helpers import require_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def _line(args):
    p = subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert p.returncode == 0, p.stdout[-2000:] + p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, p.stdout
    return json.loads(lines[0])


@pytest.mark.gpu
@pytest.mark.parametrize("args", [
    ["--steps", "50", "--warmup", "5", "--cpu-seconds", "0.5"],
    ["--op", "qk", "--steps", "50", "--warmup", "5", "--cpu-seconds", "0.5"],
    ["--op", "chain", "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5"],
], ids=["benchmark", "qk", "chain"])
def test_json_line(args):
    require_gpu()
    d = _line(args)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["unit"] == "GB/s" and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0 and "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0 and cb["sample"]
    if args[0] == "--steps":
        assert d["metric"].startswith("fused add+RMSNorm HBM GB/s") and d["dtype"] == "bf16"
        assert d["config"]["n_rows"] == 4096 and d["config"]["hidden"] == 8192
        # HBM bytes from the committed counters, or null once the kernel sources
        # have changed since they were taken
        assert "traffic" in rf
        assert rf["traffic"] is None or 1.0 <= rf["traffic"] / 268451840 < 1.01


@pytest.mark.gpu
def test_graph_launch_line():
    """--graph: the timed steps replayed as one HIP graph (checked against an
    eager step inside bench.py), same contract."""
    require_gpu()
    d = _line(["--graph", "--workload", "2048x4096", "--steps", "50", "--warmup", "5",
               "--no-cpu-baseline"])
    assert "graph" in d["config"]["launch"]
    assert d["value"] > 0 and d["roofline"]["frac"] == pytest.approx(d["value"] / 8000.0, abs=1e-3)


@pytest.mark.gpu
def test_ceilings_line():
    """--ceilings: the one-directional streams, the copies and the fused call
    over the same bytes, and the best copy named."""
    require_gpu()
    d = _line(["--ceilings", "--workload", "2048x4096", "--steps", "50"])
    g = d["ceilings_GBps"]
    for k in ("read_only", "write_only", "copy_2in_2out", "copy_rows_burst1", "copy_rows_burst2",
              "copy_rows_burst4", "torch_device_copy", "add_rmsnorm_fwd"):
        assert g[k] > 0, k
    assert d["best_copy"] in g and d["best_copy"].startswith(("copy", "torch"))
    assert d["fused_frac_of_best_copy"] == pytest.approx(
        g["add_rmsnorm_fwd"] / g[d["best_copy"]], rel=1e-3)


@pytest.mark.gpu
def test_size_sweep_line():
    """--size-sweep: per-launch times at 1024..8192 rows and a line fit with a
    positive steady rate for every stream."""
    require_gpu()
    d = _line(["--size-sweep", "--workload", "4096x1024", "--steps", "20"])
    for k in ("add_rmsnorm_fwd", "copy_2in_2out", "read_only", "write_only"):
        times = d["us_per_launch"][k]
        assert set(times) == {"1024", "2048", "4096", "8192"} and min(times.values()) > 0, k
        assert d["fit"][k]["steady_GBps"] > 0, k
