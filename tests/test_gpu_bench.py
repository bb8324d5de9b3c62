"""The benchmark's one JSON line, from short runs of the default command (the
one-call step) and of its two-call, three-call and per-row variants: every
field of the output contract is there, and the roofline and CPU-baseline
figures are consistent with each other.  (The bench times the GPU, so these are
GPU tests.)"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
          "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline",
          "cpu_baseline", "breakdown_us")


@pytest.mark.parametrize("extra", [[], ["--two-calls"], ["--separate-calls"],
                                   ["--last-step-per-row"]],
                         ids=["one_call", "two_calls", "separate_calls", "row_last_step"])
def test_bench_json_line(extra):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--cpu-seconds", "0.5", *extra],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in FIELDS:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "table10Mx128_zipf1.05_dormancy"
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    assert rf["traffic"] is None or rf["traffic"] > rf["algorithmic_bytes_per_launch"]
    if rf["traffic"] is not None:   # DRAM bytes / time beside algorithmic bytes / time
        # traffic over the mean launch time (achieved is a mean of per-step rates)
        expect = rf["traffic"] / (rf["mean_us"] * 1e-6) / 1e9
        assert abs(rf["traffic_GBs"] - expect) < 1e-6 * expect
        assert abs(rf["traffic_GBs"] / rf["achieved"]
                   / (rf["traffic"] / rf["algorithmic_bytes_per_launch"]) - 1) < 0.05
        assert rf["cold"]["traffic_GBs"] < rf["traffic_GBs"] * 1.5
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0
    assert cb["canonicalise_s"] > 0 and cb["update_s"] > 0 and cb["host"]["nproc"] >= 1
    if extra == ["--separate-calls"]:
        calls = ["coo_from_lookups", "csr_from_coo", "sparse_adam_step"]
    elif extra == ["--two-calls"]:
        calls = ["csr_from_lookups", "sparse_adam_step"]
    else:
        calls = ["sparse_step_from_lookups"]
    assert d["config"]["calls"] == " + ".join(calls)
    extra_keys = ["before_update_launch"] if len(calls) == 1 else []
    assert list(d["breakdown_us"]) == calls + ["update_launch"] + extra_keys + ["step"]
    # the update launch lies inside the step
    assert d["breakdown_us"]["update_launch"]["p50"] < d["breakdown_us"]["step"]["p50"]
    assert ("k_step_lookups" in rf["kernel"]) == (len(calls) == 1)
