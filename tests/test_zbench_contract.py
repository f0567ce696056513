"""The bench.py contract: one JSON line carrying the fields a run is read by
(the metric, the timing, the roofline of the fused kernel and the oracle's
CPU baseline), checked on the tiny workload; and the refusal of more than
one GPU, which happens before anything touches a GPU.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.gpu
def test_bench_json_line(lib, capsys, monkeypatch):
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "tiny", "--steps", "3", "--warmup", "1",
                                      "--cpu-heads", "1", "--cpu-rows", "64"])
    print("bench.py --workload tiny", file=sys.stderr, flush=True)
    bench.main()
    lines = [s for s in capsys.readouterr().out.splitlines() if s.strip()]
    assert len(lines) == 1, lines
    r = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in r, key
    assert r["n_gpus"] == 1 and r["steps"] == 3 and r["warmup"] == 1
    assert r["value"] > 0 and r["ms_per_step"] > 0 and r["higher_is_better"] is True
    assert r["config"]["workload"] == "tiny"
    # TOPS over the step time: 4 d (visible pairs) per step (both fields are rounded)
    assert abs(r["value"] - r["config"]["ops_per_step"] / (r["ms_per_step"] * 1e-3) / 1e12) <= 1e-2 * r["value"]
    rf = r["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 5000.0
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = r["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["unit"] == r["unit"]
    # the float64 reference timed on its own; the whole workload extrapolated from the sample
    assert cb["fp64_reference"]["s"] > 0 and cb["fp64_reference"]["TOPS"] > 0
    assert cb["extrapolated_full_workload_s"] > 0 and cb["cpu_model"]
