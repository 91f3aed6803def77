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


def test_no_top_level_name_is_defined_twice():
    """A second definition silently replaces the first (a report helper once
    shadowed the sweeps' percentile function, and only the GPU run with the
    sweeps would have failed)."""
    import ast
    tree = ast.parse(open(BENCH).read())
    names = [n.name for n in tree.body if isinstance(n, (ast.FunctionDef, ast.ClassDef))]
    dup = sorted({n for n in names if names.count(n) > 1})
    assert not dup, dup


def test_sweep_percentiles():
    sys.path.insert(0, ROOT)
    try:
        import bench
    finally:
        sys.path.pop(0)
    ts = [float(v) for v in range(1, 101)]
    assert bench._pct(ts, 0.1) <= bench._pct(ts, 0.5) <= bench._pct(ts, 0.9)
    assert bench._pct(ts, 0.0) == 1.0 and bench._pct(ts, 1.0) == 100.0
