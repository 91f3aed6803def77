"""Build libcoll.so (gfx950) in-tree with hipcc.

    python -m collective_communication_amd.build

Each ``csrc/*.hip`` file is compiled to an object in parallel, then linked
into ``collective_communication_amd/libcoll.so``.  Flags:

* ``--offload-arch=gfx950``: MI355X only, no other targets.
* ``-ffp-contract=off``: no a*b+c fused into FMA, so every float operation is
  the one written (the combine's separately rounded products).
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed-fp32
  instructions are emitted.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcoll.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra=(), bdir: str = BUILD_DIR) -> str:
    obj = os.path.join(bdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, defines=(), out: str | None = None,
          build_dir: str | None = None) -> str:
    """Compile every HIP source and link libcoll.so; returns its path.

    ``defines`` (e.g. ``["COLL_A2A_U=8"]``) and ``out`` build a variant of the
    library with other tuning constants elsewhere (used for tuning sweeps)."""
    bdir = build_dir or BUILD_DIR
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    extra = [f"-D{d}" for d in defines]
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, bdir), srcs))
    target = out or LIB
    tmp = target + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, target)
    if verbose:
        print(f"built {target}")
    return target


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
