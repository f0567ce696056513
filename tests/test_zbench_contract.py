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


def test_mode_ceilings_and_quantize_bytes():
    """Host arithmetic of the bench line: the MFMA ceiling of each P.V mode
    (half the ops on INT8, half on the P.V type) and of the per-head mode at
    a share f8 of FP8 heads, which reduces to the single modes at f8 = 0 and
    1; the quantize pass's bytes likewise."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads
    assert abs(bench.mode_peak(0) - 10000 / 3) < 1e-6 and abs(bench.mode_peak(1) - 5000) < 1e-6
    assert abs(bench.mode_peak(2, 0.0) - bench.mode_peak(0)) < 1e-6
    assert abs(bench.mode_peak(2, 1.0) - bench.mode_peak(1)) < 1e-6
    f8 = 15 / 40   # time per op is the share-weighted sum of the two modes'
    want = 1 / (f8 / 5000 + (1 - f8) * (0.5 / 5000 + 0.5 / 2500))
    assert abs(bench.mode_peak(2, f8) - want) < 1e-6
    assert bench.mode_peak(0) < bench.mode_peak(2, f8) < bench.mode_peak(1)
    w = workloads.get("large")
    for pv in (0, 1):
        assert bench.quantize_bytes(w, 2, float(pv)) == bench.quantize_bytes(w, pv)
    lo, mid, hi = (bench.quantize_bytes(w, 2, f)[0] for f in (0.0, f8, 1.0))
    assert lo < mid < hi
    # the minimum in 16-bit mode: K read twice, Q once, codes written
    n = w.B * w.H * w.Nkv * w.d
    assert lo == 2 * n + 2 * 2 * n + n + n


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
    assert sorted(r["input_digests"]) == ["k", "q", "v"] and all(len(h) == 64 for h in r["input_digests"].values())
    # TOPS over the step time: 4 d (visible pairs) per step (both fields are rounded)
    assert abs(r["value"] - r["config"]["ops_per_step"] / (r["ms_per_step"] * 1e-3) / 1e12) <= 1e-2 * r["value"]
    rf = r["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TOPS" and rf["peak"] == 5000.0
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # the fused kernel's launches: mean, median and minimum
    assert 0 < rf["ms_per_launch_min"] <= rf["ms_per_launch_median"] and rf["ms_per_launch"] >= rf["ms_per_launch_min"]
    # the P.V mode's own ceiling: 1 / (0.5 / 5000 + 0.5 / P) with P = 2500 (16-bit P.V) or 5000 (FP8)
    import workloads
    pv = r["config"]["pv"]
    assert pv == ("fp8" if workloads.get("tiny").pv_mode == 1 else "16")   # the workload's own mode
    want = 5000.0 if pv == "fp8" else 10000 / 3
    assert abs(rf["mode_peak"] - want) < 0.1 and abs(rf["mode_frac"] - rf["achieved"] / rf["mode_peak"]) < 1e-3
    qz = r["quantize"]
    assert qz["algorithmic_bytes"] <= qz["design_bytes"]
    # the other P.V mode, with its accuracy and whether it meets both bars
    assert [m["pv"] for m in r["other_pv_modes"]] == ["16" if pv == "fp8" else "fp8"]
    assert isinstance(r["other_pv_modes"][0]["meets_bar"], bool)
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = r["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["unit"] == r["unit"]
    # the float64 reference timed on its own; the whole workload extrapolated from the sample
    assert cb["fp64_reference"]["s"] > 0 and cb["fp64_reference"]["TOPS"] > 0
    assert cb["extrapolated_full_workload_s"] > 0 and cb["cpu_model"]


@pytest.mark.gpu
def test_bench_graph_replay_of_a_streaming_step(lib, capsys, monkeypatch):
    """A frame-cache streaming step, also timed as a replayed HIP graph."""
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "stream-cache", "--steps", "3", "--warmup", "1",
                                      "--no-cpu", "--single-mode", "--graph"])
    print("bench.py --workload stream-cache --graph", file=sys.stderr, flush=True)
    bench.main()
    lines = [s for s in capsys.readouterr().out.splitlines() if s.strip()]
    assert len(lines) == 1, lines
    r = json.loads(lines[0])
    g = r["graph_replay"]
    assert g["ms_per_step"] > 0
    assert abs(g["value"] - r["config"]["ops_per_step"] / (g["ms_per_step"] * 1e-3) / 1e12) <= 1e-2 * g["value"]
