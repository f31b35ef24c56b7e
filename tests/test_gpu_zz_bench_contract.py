"""bench.py's output line on the GPU: one JSON object with the metric, the throughput,
the roofline of the dominant kernel and the run's configuration.  A short run (two timed
steps, secondary measurements off) through the same code path as the default run."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_line_contract():
    print("case: bench.py --steps 2 --warmup 1, secondary measurements off", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--no-cpu-baseline", "--no-block", "--no-e4m3", "--no-ar-step"],
                       cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "candidates/s" and d["dtype"] == "bf16" and d["vs_baseline"] is None
    # value is the candidates of one step over the step's time
    cfg = d["config"]
    assert "workload" in cfg
    assert d["value"] == pytest.approx(cfg["B"] * cfg["k"] / (d["ms_per_step"] / 1e3), rel=1e-3)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-4)
    assert 0 < rf["frac"] < 1
    # achieved = algorithmic bytes of one launch / its average duration
    assert rf["achieved"] == pytest.approx(rf["algorithmic_bytes_per_launch"] / (rf["avg_launch_ms"] / 1e3) / 1e9,
                                           rel=2e-3)
    assert rf["traffic"] is None or rf["traffic"] > 0
    assert d["hbm_copy_reference"]["gbs"] > 0
    # the secondary keys of the same run: the probes beside the copy, the long-history
    # workload with both peaks' fractions, and which profile summaries match the sources
    pr = d["probes"]
    assert 0 < pr["mfma_loop"]["frac_of_peak"] < 1 and pr["mfma_loop"]["tflops"] > 0
    assert pr["lds_read_bytes_per_ns_per_cu"]["ds_read_b128"] > 0
    assert pr["lds_read_bytes_per_ns_per_cu"]["ds_read_b64_tr_b16"] > 0
    assert all(v > 0 for k, v in pr["mfma_exp_overlap_ns_per_iter"].items() if k != "what")
    lh = d["long_history"]
    for kern in ("prefill", "rank_decode"):
        k = lh[kern]
        assert k["cold_median_ms"] > 0 and k["warm_mean_ms"] > 0
        assert k["cold_tflops"] == pytest.approx(k["algorithmic_gflop"] / k["cold_median_ms"], rel=2e-3)
        assert 0 < k["cold_mfma_frac"] < 1 and 0 < k["cold_hbm_frac"] < 1
    summaries = sorted(f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.endswith(".txt"))
    assert sorted(d["profiles"]) == summaries
    assert all(isinstance(v["current"], bool) for v in d["profiles"].values())
