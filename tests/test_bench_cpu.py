"""Host-side checks of bench.py: the one-GPU contract and the CPU-baseline
leg (the oracle timed in forked processes), each run in a fresh interpreter
because the baseline forks before torch is imported."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, timeout=300):
    return subprocess.run([sys.executable, *args], cwd=ROOT, capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _run(["bench.py", "--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line


def test_cpu_baseline_reports_the_oracle():
    code = ("import json, bench; print(json.dumps(bench.cpu_baseline(budget_s=0.5)))")
    r = _run(["-c", code])
    assert r.returncode == 0, r.stderr
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["kind"] == "oracle" and out["unit"] == "Gelem/s"
    assert 1 <= out["cores"] <= 16
    assert out["value"] > 0 and out["single_core"]["value"] > 0 and out["single_core"]["cores"] == 1
    assert out["GBps"] == out["value"] * out["bytes_per_element"]
    assert str(out["cores"]) in out["sample"]
