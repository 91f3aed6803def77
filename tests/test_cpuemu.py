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

The emulator checks two more rules at every site: a value the kernel moves
into a scalar register (readfirstlane, COLL_UNIFORM) must be equal in every
active lane, since on the GPU the other lanes would go on with lane 0's value
(an address, a slot, a descriptor); and LDS is read back poisoned, not zeroed,
if a kernel reads it before writing.  Its self-test plants each mistake in a
small kernel of its own and expects the run to stop.
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


SELFTEST = os.path.join(HERE, "cpuemu", "selftest.py")
# which -> (what the planted mistake is, how the run must end, message it prints)
SELF_CASES = {
    0: ("COLL_UNIFORM of a per-lane value", -6, "COLL_UNIFORM of a value that differs"),
    1: ("readfirstlane of a per-lane value", -6, "readfirstlane of a value that differs"),
    2: ("ballot reached by half of a wave", -6, "divergent control flow"),
    3: ("store one element past a buffer", -11, None),
    4: ("LDS read before it is written", 0, None),
}


def _selftest(which, bad):
    r = subprocess.run([sys.executable, SELFTEST, str(which), str(bad)], capture_output=True,
                       text=True, timeout=120)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.parametrize("which", sorted(SELF_CASES))
def test_emulator_stops_a_planted_mistake(emu_lib, which):
    what, code, msg = SELF_CASES[which]
    rc, text = _selftest(which, 0)
    assert rc == 0 and "rc 0" in text, f"clean form of {what}: {text[-400:]}"
    rc, text = _selftest(which, 1)
    if which == 4:
        vals = [int(v) for v in text.split("out")[-1].split()]
        assert rc == 0 and vals and all(v == -1515870811 for v in vals), text[-400:]  # 0xA5A5A5A5
        return
    assert rc == code, f"{what}: exit {rc}\n{text[-400:]}"
    if msg:
        assert msg in text, text[-400:]
