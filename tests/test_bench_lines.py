"""The bench lines kept in profiles/ (each the one JSON line bench.py printed
on an MI355X): the fields of the result contract are present and consistent
with each other (value and ms_per_step, the roofline fraction, the traffic
beside the algorithmic bytes), the CPU baseline is the oracle with its core
count and sample, and each line names its workload. Runs on the CPU."""
import glob
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LINES = sorted(glob.glob(os.path.join(ROOT, "profiles", "bench_*.json")))


def test_there_are_bench_lines():
    names = {os.path.basename(p) for p in LINES}
    for need in ("bench_llama3_128k.json", "bench_fp8_llama3_128k.json", "bench_single_256k.json",
                 "bench_ragged_mha.json", "bench_prefill_128k.json", "bench_prefill_16k.json"):
        assert need in names, need


@pytest.mark.parametrize("path", LINES, ids=[os.path.basename(p) for p in LINES])
def test_bench_line_contract(path):
    d = json.load(open(path))
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["data"] == "synthetic" and d["higher_is_better"] is False
    assert d["value"] > 0 and d["ms_per_step"] > 0
    scale = {"us/step": 1e-3, "ms": 1.0}[d["unit"]]
    assert d["ms_per_step"] == pytest.approx(d["value"] * scale, rel=1e-3)
    assert isinstance(d["config"], dict) and d["config"]["workload"]
    r = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in r, k
    assert r["bound"] in ("hbm", "mfma")
    assert r["peak"] == {"hbm": 8000.0, "mfma": 2500.0}[r["bound"]]
    assert r["unit"] == {"hbm": "GB/s", "mfma": "TFLOP/s"}[r["bound"]]
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-3)
    if r["bound"] == "hbm":
        # achieved = algorithmic bytes per call / the call's median time
        assert r["achieved"] == pytest.approx(r["bytes_per_launch"] / (r["avg_launch_us"] * 1e-6) / 1e9, rel=2e-3)
        if r["traffic"] is not None:
            # counter bytes: at least the algorithmic ones; above them by at most 10% plus
            # the split partials written and read back (~5-7 MB at the 128K shape)
            assert 0.98 * r["bytes_per_launch"] <= r["traffic"] <= 1.1 * r["bytes_per_launch"] + 8e6
    c = d["cpu_baseline"]
    if c is not None:
        assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["sample"]
