"""The benchmark's command-line contract, checked without a GPU: more than one GPU
is refused with a message, and the committed bench line carries every field the
JSON line must hold (roofline and CPU baseline included)."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LINE = os.path.join(ROOT, "profiles", "bench_line_ep32-group-fwdbwd-p32-s8192-e256-k8-h4096.json")


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_committed_bench_line_has_every_field():
    with open(LINE) as f:
        d = json.loads(f.read().strip().splitlines()[-1])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["config"]["workload"] == "ep32-group-fwdbwd-p32-s8192-e256-k8-h4096"
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["sample"]
    assert c["single_thread"]["threads"] == 1 and c["single_thread"]["value"] > 0
    # the committed line is the default command's: its workload is bench.py's default one
    sys.path.insert(0, ROOT)
    import bench

    assert d["config"]["workload"] == bench.DEFAULT_WORKLOAD
    # tokens per second of the whole step: T / ms_per_step
    assert abs(d["value"] - d["config"]["T"] / (d["ms_per_step"] * 1e-3)) / d["value"] < 1e-6


def test_committed_kernel_trace_agrees_with_the_bench_line():
    """The committed rocprofv3 kernel trace covers the run the committed bench line came from:
    the trace's average duration of the roofline kernel's launches (the fresh and the cached
    dispatch instantiations at the headline grid) agrees with the line's HIP-event average
    launch time within 2%, and the JSON line the trace file quotes is the committed line."""
    import re

    with open(LINE) as f:
        d = json.loads(f.read().strip().splitlines()[-1])
    w = d["config"]["workload"]
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{w}.md")
    with open(path) as f:
        text = f.read()
    r = d["roofline"]
    assert r["kernel"] == "dispatch_kernel"
    # rows: | `ep::dispatch_kernel<1, false, META, ...>` | grid | wg | vgpr | lds | scratch | launches | avg | median | min |
    avgs = []
    for m in re.finditer(r"^\| `ep::dispatch_kernel<([^>]*)>` \| (\d+) \| \d+ \| \d+ \| \d+ \| \d+ \| (\d+) \| ([\d.]+) \|",
                         text, flags=re.M):
        args = [a.strip() for a in m.group(1).split(",")]
        fixed = args[4] == "true"
        if args[1] == "false" and not fixed and int(m.group(3)) >= d["steps"]:  # bf16, exact windows, every step
            avgs.append(float(m.group(4)))
    # the first two such rows are the headline step's fresh and cached dispatch
    assert len(avgs) >= 2, avgs
    trace_avg = sum(avgs[:2]) / 2
    assert abs(trace_avg - r["avg_launch_us"]) / r["avg_launch_us"] < 0.02, (trace_avg, r["avg_launch_us"])
    # the JSON line the trace file quotes (possibly cut short) is the committed line's
    quoted = [ln for ln in text.splitlines() if ln.startswith('{"metric"')]
    assert quoted, "the trace file quotes no JSON line"
    m = re.search(r'"value": ([0-9.e+]+)', quoted[-1])
    assert m and float(m.group(1)) == d["value"], (m and m.group(1), d["value"])
