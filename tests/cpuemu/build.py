"""Build the library's kernels for the CPU emulator -- TEST INFRASTRUCTURE ONLY.

Every ``collective_communication_amd/csrc/*.hip`` source is compiled as plain
C++ for the host against ``tests/cpuemu/hip/hip_runtime.h`` (the emulated
device API) and linked with ``emu.cpp`` into ``tests/cpuemu/_build/
libcoll_emu.so``, which exports the same C ABI as the GPU library.  The host
clang of the ROCm toolchain is used because the kernels rely on clang vector
extensions (``ext_vector_type``, ``__bf16``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "collective_communication_amd", "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(BUILD, "libcoll_emu.so")

CXX = os.environ.get("EMU_CXX") or next(
    (c for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")) if c and os.path.exists(c)),
    "clang++")
FLAGS = ["-x", "c++", "-std=c++17", "-O1", "-g", "-fPIC", "-ffp-contract=off",
         "-fno-omit-frame-pointer", "-Wno-unused-function", "-Wno-unknown-attributes",
         "-I", HERE, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         # the AllReduce switches to its 2 KiB-per-rank LDS tile from 16 KiB per
         # rank here (48 MiB on the GPU), so both tiles meet the emulator's sizes
         "-DCOLL_AR_LDS_BIG_BYTES=16384u",
         # the plain All-to-All-v leaves its resident grid above 64 KiB of
         # receive capacity here (256 MiB on the GPU), so the emulator's cases
         # run both grids
         "-DCOLL_A2A_RESIDENT_MAX_BYTES=65536ull"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _newest_input() -> float:
    files = sources() + [os.path.join(HERE, "emu.cpp"), os.path.join(HERE, "hip", "hip_runtime.h")]
    files += [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    files.append(os.path.join(ROOT, "include", "coll.h"))
    return max(os.path.getmtime(f) for f in files)


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [CXX, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"emulator build failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(force: bool = False) -> str:
    """Compile (when a source is newer than the library) and return its path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= _newest_input():
        return LIB
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources() + [os.path.join(HERE, "emu.cpp")]
    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([CXX, "-shared", "-fPIC", "-o", tmp, *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"emulator link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_selftest() -> str:
    """The emulator's own self-test library: selftest.cpp + emu.cpp."""
    lib = os.path.join(BUILD, "libemu_selftest.so")
    src = os.path.join(HERE, "selftest.cpp")
    inputs = [src, os.path.join(HERE, "emu.cpp"), os.path.join(HERE, "hip", "hip_runtime.h")]
    if os.path.exists(lib) and os.path.getmtime(lib) >= max(os.path.getmtime(f) for f in inputs):
        return lib
    os.makedirs(BUILD, exist_ok=True)
    tmp = lib + ".tmp%d" % os.getpid()
    r = subprocess.run([CXX, *FLAGS, src, os.path.join(HERE, "emu.cpp"), "-shared", "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"emulator self-test build failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(force=True))
