"""bench.py end to end on the GPU, as a child process: one JSON line on
stdout with the fields the measurement contract asks for, their types and
the relations between them (tokens/s from the step time, the roofline
fraction from its own achieved and peak bandwidth)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_contract():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("bench.py --steps 20 --warmup 5 --no-sweep --no-cpu", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "20",
                        "--warmup", "5", "--no-sweep", "--no-cpu"],
                       capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 5
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True
    # dtype is the arithmetic type (fp32 throughout); the storage type is io_dtype
    assert d["dtype"] == "f32" and d["config"]["io_dtype"] == "bf16"
    assert d["data"] == "synthetic" and d["vs_baseline"] is None
    assert "workload" in d["config"] and d["config"]["tokens"] == 2048
    # tokens per second = the cell's tokens over the time of one step
    assert d["value"] == pytest.approx(2048 / (d["ms_per_step"] * 1e-3), rel=1e-3)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=2e-4)
    # achieved = algorithmic bytes over the average launch time, below the peak
    assert rf["achieved"] == pytest.approx(
        rf["algorithmic_bytes_per_launch"] / rf["avg_launch_us"] / 1e3, rel=2e-3)
    assert 0 < rf["frac"] < 1
    assert rf["traffic"] is None or rf["traffic"] > rf["algorithmic_bytes_per_launch"] * 0.9
    assert rf["copy_ceiling_GBps"] > 0 and rf["of_copy"] > 0
    # the null arm: the same 20 steps twice more; `value` is the first run
    reps = d["repeats_us_per_step"]
    assert len(reps) == 3 and reps[0] == pytest.approx(1000 * d["ms_per_step"], abs=2e-3)
    assert d["repeat_spread"] == pytest.approx(max(reps) / min(reps) - 1, abs=2e-3)
    assert "cpu_baseline" not in d                      # --no-cpu
    t1 = d["us_per_call_T1"]
    assert 0 < t1["median"] < 50
    # the smallest launch is about the floor of every call, the T = 1 copy
    # included (the two medians can trade places within noise)
    assert 0 < t1["launch_floor_us"] <= t1["copy_floor_us"] * 1.15
    assert len(d["prefill"]) == 24
    for c in d["prefill"]:
        assert c["T"] >= 256 and 0 < c["frac_peak"] < 1 and c["copy_us"] > 0


@pytest.mark.parametrize("args,key", [
    (["--only", "prologue_prefill", "--steps", "30"], "launches"),
    (["--only", "norm_fp8", "--steps", "30"], "launches"),
    (["--only", "prologue", "--steps", "30"], "launches"),
    (["--only", "act_fp8", "--steps", "30"], "launches"),
    (["--only", "act_prefill", "--steps", "30"], "launches"),
    (["--only", "norm_prefill", "--steps", "30"], "launches"),
    (["--copy-probe", "1048576"], "copy_probe_bytes_moved"),
])
def test_bench_profiling_aids(args, key):
    # the commands the committed profiles name: each prints one JSON line
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("bench.py", *args, flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    assert d[key] > 0
