"""Runs one case of the emulator's self-test (selftest.cpp) on a buffer that
ends at a guard page -- TEST INFRASTRUCTURE ONLY.  Usage: selftest.py WHICH BAD;
prints the output buffer's values on success."""
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import build  # noqa: E402
from guarded import Heap, ptr  # noqa: E402

which, bad = int(sys.argv[1]), int(sys.argv[2])
os.environ.setdefault("EMU_CUS", "2")
lib = ctypes.CDLL(build.build_selftest())
lib.emu_selftest.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
heap = Heap("end")
out = heap.empty(64 if which == 4 else 128, np.int32)
out[...] = -1
print("running", which, bad, flush=True)
rc = lib.emu_selftest(which, ptr(out), bad)
print("rc", rc, "out", " ".join(str(int(v)) for v in out), flush=True)
