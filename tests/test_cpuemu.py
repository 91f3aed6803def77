"""Every kernel of the library run on the CPU, before any GPU run, with guard
pages around every buffer (CPU only).

The HIP sources are compiled for the host against an emulation of the device
API (tests/cpuemu): each workgroup's lanes run as fibers grouped in wave64s,
so barriers and wave operations (ballot, shuffles, readfirstlane) behave as
on the GPU, LDS is poisoned before each workgroup, and a wave operation
reached under divergent control flow aborts.  Every entry point is called
through its C ABI on small seeded cases that span several tiles and ragged
tails, and its outputs are compared with the oracle.  Buffers sit flush
against inaccessible pages, once at their end and once at their start, so an
access one byte outside any buffer kills the run; each family runs in a
subprocess, whose last printed line then names the case.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = os.path.join(HERE, "cpuemu", "cases.py")
FAMILIES = ["reduce", "copy", "a2av", "exchange", "merge", "moe"]


@pytest.fixture(scope="module")
def emu_lib():
    sys.path.insert(0, os.path.join(HERE, "cpuemu"))
    try:
        import build as emu_build
        return emu_build.build()
    finally:
        sys.path.pop(0)


@pytest.mark.parametrize("place", ["end", "start"])
@pytest.mark.parametrize("family", FAMILIES)
def test_kernels_on_guarded_buffers(emu_lib, family, place):
    env = dict(os.environ, EMU_CUS="4", COLL_A2A_DESC_MIN_BYTES="0")
    r = subprocess.run([sys.executable, CASES, family, place], capture_output=True, text=True,
                       env=env, timeout=900)
    tail = "\n".join((r.stdout + r.stderr).strip().splitlines()[-8:])
    assert r.returncode == 0, f"{family}/{place} exited with {r.returncode}:\n{tail}"
    assert "all cases passed" in r.stdout, tail
