"""The committed benchmark lines (profiles/bench_*.json) against the JSON
contract that bench.py prints: keys, units, one GPU, the roofline fraction
as achieved / peak with the MI355X datasheet peaks, the useful rate as
flops / time, and a CPU baseline from the oracle.  Also: bench.py refuses
more than one GPU before touching one."""
import glob
import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LINES = sorted(glob.glob(os.path.join(ROOT, "profiles", "bench_*.json")))
MFMA_PEAK = {"f64": 78.6, "f32": 157.3, "f16": 2500.0, "bf16": 2500.0}   # dense TFLOP/s, datasheet
HBM_PEAK = 8000.0                                                          # GB/s
VECTOR_PEAK = {"f64": 78.6, "f32": 157.3}   # vector ALU TFLOP/s: 256 CUs x 2.4 GHz x 128 (fp64) / 256 (fp32) per clock


def _load(path):
    with open(path) as fh:
        text = fh.read().strip()
    assert "\n" not in text, "a bench line is one JSON line"
    return json.loads(text)


def test_there_are_bench_lines():
    names = [os.path.basename(p) for p in LINES]
    assert "bench_tlr_tlr_f64_n16384_b512.json" in names


@pytest.mark.parametrize("path", LINES, ids=[os.path.basename(p) for p in LINES])
def test_bench_line_contract(path):
    d = _load(path)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True
    assert d["data"] == "synthetic"
    assert d["dtype"] in MFMA_PEAK
    assert isinstance(d["config"].get("workload"), str)
    assert d["steps"] > 0 and d["warmup"] >= 0 and d["ms_per_step"] > 0

    # useful TFLOP/s = flops counted from the ranks / time per step
    flops = d["config"]["useful_flops"]
    assert math.isclose(d["value"], flops / (d["ms_per_step"] * 1e-3) / 1e12, rel_tol=2e-3)

    r = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in r, k
    if r["bound"] == "mfma":
        assert r["unit"] == "TFLOP/s" and r["peak"] == MFMA_PEAK[d["dtype"]]
    elif r["bound"] == "alu":
        assert r["unit"] == "TFLOP/s" and r["peak"] == VECTOR_PEAK[d["dtype"]]
    else:
        assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == HBM_PEAK
    assert math.isclose(r["frac"], r["achieved"] / r["peak"], rel_tol=2e-3)
    assert 0.0 < r["frac"] <= 1.0
    assert r["traffic"] is None or r["traffic"] > 0

    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["sample"]
    assert c["unit"] == d["unit"]


def test_metric_line_is_the_default_workload():
    d = _load(os.path.join(ROOT, "profiles", "bench_tlr_tlr_f64_n16384_b512.json"))
    assert d["dtype"] == "f64"
    assert d["config"]["N"] == 16384 and d["config"]["b"] == 512
    assert (d["config"]["opA"], d["config"]["opB"]) == ("T", "N")
    assert d["roofline"]["bound"] == "mfma"


@pytest.mark.parametrize("name", ["tlr_tlr_f64_n16384_b512_TN", "tlr_tlr_f16_n16384_b512_TN"])
def test_traffic_of_a_bench_line_is_its_counter_summary(name):
    """A non-null roofline.traffic is the committed FETCH_SIZE + WRITE_SIZE
    figure of the same workload's final-update launch."""
    tpath = os.path.join(ROOT, "profiles", f"stage3_traffic_{name}.json")
    with open(tpath) as fh:
        t = json.load(fh)
    assert math.isclose(t["bytes_per_launch"], t["read_bytes"] + t["write_bytes"], rel_tol=1e-9)
    assert t["fetch_scale"] > 0 and t["write_scale"] > 0
    dtype = "f16" if "f16" in name else "f64"
    for p in LINES:
        d = _load(p)
        if d["config"]["workload"] == name and d["dtype"] == dtype and d["roofline"]["traffic"] is not None:
            assert math.isclose(d["roofline"]["traffic"], t["bytes_per_launch"], rel_tol=1e-9)


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
