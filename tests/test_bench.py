"""The benchmark's output contract.  CPU: a request for more than one GPU is
refused with one JSON line and exit status 2, before anything touches a GPU.
GPU: a short headline run prints exactly one JSON line with the keys, units
and relations the contract fixes (value = algorithmic bytes / time per step,
the roofline's achieved figure and fraction, the measured traffic close to
the algorithmic bytes when present)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def json_lines(stdout):
    return [json.loads(line) for line in stdout.splitlines() if line.startswith("{")]


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    lines = json_lines(r.stdout)
    assert len(lines) == 1 and lines[0]["n_gpus"] == 2 and "one GPU" in lines[0]["error"]


def test_counter_collection_refuses_cold_mode():
    """Under rocprofv3 counter collection only the short warm form runs: a
    cold request, a long one, or collection without --counters is refused
    with one JSON line and exit status 2, before anything touches a GPU."""
    for args, env in ((["--counters"], {}),
                      (["--counters", "--modes", "warm,cold"], {}),
                      (["--counters", "--modes", "warm", "--steps", "100"], {}),
                      (["--modes", "warm", "--steps", "10"], {"ROCPROF_COUNTER_COLLECTION": "1"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                           capture_output=True, text=True, timeout=120, cwd=ROOT,
                           env={**os.environ, **env})
        assert r.returncode == 2, (args, r.stderr[-2000:])
        lines = json_lines(r.stdout)
        assert len(lines) == 1 and "error" in lines[0], (args, r.stdout)


def test_spacer_rotation_keeps_every_window_cold():
    """Each timed window follows whole rotations over the buffer sets, so the
    set a timed launch uses was last used a full rotation (every other set)
    earlier, whatever the step count."""
    sys.path.insert(0, ROOT)
    import bench
    for sets in (1, 2, 10, 17, 24, 5042):
        for steps in (1, 5, 20, 25, 1000):
            n = bench.spacer_length(sets, steps)
            assert n % sets == 0 and n >= steps and n >= sets
            seq = [i % sets for i in range(n)] + [i % sets for i in range(steps)]
            for p in range(n, n + steps):
                last = max(q for q in range(p) if seq[q] == seq[p])
                assert p - last >= sets


@pytest.mark.gpu
def test_headline_line_keeps_the_contract():
    print("bench --only-headline --steps 20 --warmup 5", flush=True)
    r = run_bench("--only-headline", "--steps", "20", "--warmup", "5", "--no-cpu-baseline")
    assert r.returncode == 0, r.stderr[-3000:]
    lines = json_lines(r.stdout)
    assert len(lines) == 1, r.stdout[-3000:]
    d = lines[0]
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 5
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["config"]["workload"] == "ptok_fp8_2520x3072"
    lo, hi = d["us_range"]
    assert lo <= d["ms_per_step"] * 1e3 <= hi
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] == d["value"] and abs(rf["frac"] - d["value"] / 8000.0) < 1e-3
    assert 0.0 < rf["frac"] < 1.0
    per_step_s = d["ms_per_step"] * 1e-3
    assert abs(rf["algorithmic_bytes_per_launch"] / per_step_s / 1e9 - d["value"]) <= 1e-3 * d["value"]
    if rf["traffic"] is not None:
        assert abs(rf["traffic"] / rf["algorithmic_bytes_per_launch"] - 1.0) < 0.05
    floor = rf.get("practical_floor")
    if floor is not None:
        assert 0.0 < floor["kernel_frac_of_floor"] <= 1.2
