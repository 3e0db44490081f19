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
