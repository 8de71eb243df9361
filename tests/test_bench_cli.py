"""The benchmark's command line: it measures one GPU only and says so."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_leg_reports_its_sample():
    # the oracle leg runs on the host: a short budget on the tiny fp32 workload
    sys.path.insert(0, ROOT)
    import bench
    from context_attention_ra_amd import configs, layout
    w = configs.TINY_F32
    segs = [layout.split(w.split, w.S, w.P, t) for t in range(w.P)]
    rec = bench.cpu_baseline(w, 0, segs, 0.5)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s" and rec["value"] > 0
    assert rec["cores"] >= 1 and rec["rows_per_s"] > 0
    full_rows = w.B * w.H * w.L
    assert abs(rec["extrapolated_full_s"] - full_rows / rec["rows_per_s"]) < 1e-9 * rec["extrapolated_full_s"] + 1e-12
    assert "extrapolated" in rec["extrapolation"] and "query rows" in rec["sample"]


def test_cpu_full_configs_time_the_small_workloads_in_full():
    # the oracle in full on the tiny ring, the two-rank causal share and the
    # factored video workload (about 10 s of host work)
    sys.path.insert(0, ROOT)
    import bench
    recs = bench.cpu_full_configs()
    names = [r["workload"] for r in recs]
    assert any("tiny-f32-ring" in n for n in names) and any("causal-bf16-4k-cp2" in n for n in names)
    assert any(n.endswith("spatial") for n in names) and any(n.endswith("temporal") for n in names)
    assert all(r["s"] > 0 and r["TFLOP/s"] > 0 for r in recs)
