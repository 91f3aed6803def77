"""The benchmark's command line without a GPU (CPU only): more than one GPU is
refused with a message before anything is imported or launched, and a saved
JSON line renders as the documentation's tables."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2", "--steps", "1"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "--gpus must be 1" in msg["error"]


def test_report_renders_the_committed_run():
    path = os.path.join(ROOT, "profiles", "bench_full_run.md")
    line = json.loads(open(path).read().strip().splitlines()[-1])
    r = subprocess.run([sys.executable, BENCH, "--report", path], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    out = r.stdout
    assert f"{line['value']:.1f} GB/s" in out
    for row, v in line["rows"].items():
        assert f"| {row} | {v['us']} |" in out
    assert "| 16MiB |" in out and "moe_rows7168_ws" in out
