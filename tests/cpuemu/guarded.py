"""Host buffers fenced by inaccessible pages -- TEST INFRASTRUCTURE ONLY.

Each buffer gets its own anonymous mapping with 64 KiB of PROT_NONE pages on
both sides.  With ``place="end"`` the buffer ends exactly where the trailing
guard starts (any access past its last byte faults); with ``place="start"``
it begins right after the leading guard (any access before its first byte
faults; starts stay page-aligned, so the vector paths run).  The kernels under
CPU emulation read and write these buffers directly.
"""
from __future__ import annotations

import ctypes
import mmap

import numpy as np

PAGE = mmap.PAGESIZE
GUARD = 16 * PAGE
_libc = ctypes.CDLL(None, use_errno=True)
_libc.mprotect.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]


class Heap:
    def __init__(self, place: str):
        assert place in ("start", "end")
        self.place = place
        self._maps = []

    def empty(self, shape, dtype) -> np.ndarray:
        dtype = np.dtype(dtype)
        shape = (shape,) if isinstance(shape, int) else tuple(shape)
        n = int(np.prod(shape, dtype=np.int64)) * dtype.itemsize
        body = -(-max(n, 1) // PAGE) * PAGE
        mm = mmap.mmap(-1, body + 2 * GUARD)
        base = ctypes.addressof(ctypes.c_char.from_buffer(mm))
        for a in (base, base + GUARD + body):
            if _libc.mprotect(ctypes.c_void_p(a), GUARD, 0) != 0:
                raise OSError(ctypes.get_errno(), "mprotect")
        off = GUARD if self.place == "start" else GUARD + body - n
        self._maps.append(mm)
        return np.frombuffer(mm, dtype=np.uint8, count=n, offset=off).view(dtype).reshape(shape)

    def copy(self, a: np.ndarray) -> np.ndarray:
        out = self.empty(a.shape, a.dtype)
        out[...] = a
        return out

    def poison(self, shape, dtype) -> np.ndarray:
        out = self.empty(shape, dtype)
        out.view(np.uint8)[...] = 0xAB
        return out


def ptr(a) -> int:
    """Address of an array's first element (0 for None: a NULL pointer)."""
    if a is None:
        return 0
    return a.ctypes.data


def table(arrs):
    return (ctypes.c_void_p * len(arrs))(*[ptr(a) for a in arrs])
