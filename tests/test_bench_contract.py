"""bench.py's command-line contract: the one-GPU refusal and the one JSON line it prints (the line's fields and
their types, on a short GPU run in a subprocess)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args, timeout=600):
    return subprocess.run([sys.executable, BENCH, *args], cwd=ROOT, capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2", timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


@pytest.mark.gpu
@pytest.mark.parametrize("args", [("--steps", "6", "--warmup", "2"), ("--workload", "1", "--steps", "6", "--warmup", "2")])
def test_json_line(args):
    print(f"case: bench {' '.join(args)}", flush=True)
    r = _run(*args, "--warmup-seconds", "0", "--no-cpu-baseline", "--sample-every", "1")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)):
        assert isinstance(d[key], typ), key
    assert d["n_gpus"] == 1 and d["steps"] == 6 and d["value"] > 0 and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["cpu_baseline"] is None and d["data"] == "synthetic"
    assert isinstance(d["config"]["workload"], str)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    # steps run back to back: a step takes at least the verify call it contains
    assert d["ms_per_step"] * 1000 >= 0.9 * rf["median_us"]


@pytest.mark.gpu
def test_gemm_reference_line():
    """--gemm-reference prints one JSON line with the library GEMM's rate and its share of the bf16 peak."""
    print("case: bench --gemm-reference 1024", flush=True)
    r = _run("--gemm-reference", "1024", "--steps", "3", "--warmup-seconds", "0")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    g = json.loads(lines[0])["gemm_reference"]
    assert g["n"] == 1024 and g["launches"] == 3 and g["flop_per_launch"] == 2.0 * 1024 ** 3
    assert g["TFLOPs_median"] > 0 and 0 < g["frac_of_2500TFLOPs"] < 1

