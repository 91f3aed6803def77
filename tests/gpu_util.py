"""Helpers for the GPU parity tests: numpy <-> device tensors, poison fills."""
import sys

import numpy as np
import torch

NP2TORCH = {np.dtype(np.uint16): torch.bfloat16, np.dtype(np.float16): torch.float16,
            np.dtype(np.float32): torch.float32, np.dtype(np.int32): torch.int32,
            np.dtype(np.uint32): torch.int32, np.dtype(np.int64): torch.int64}


def dev(a: np.ndarray, bf16: bool = True) -> torch.Tensor:
    """numpy -> device tensor.  uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16 if bf16 else torch.float16)
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32))
    else:
        t = torch.from_numpy(a)
    return t.to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy (bf16/fp16 as uint16 bit patterns)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def poison_like(t: torch.Tensor) -> torch.Tensor:
    """Same shape/dtype filled with a recognisable bit pattern (NaN for floats)."""
    out = torch.empty_like(t)
    if t.element_size() == 2:
        out.view(torch.int16).fill_(0x7FAB)        # bf16 / fp16 NaN
    elif t.element_size() == 4:
        out.view(torch.int32).fill_(0x7FBADBAD)    # fp32 NaN / odd int
    else:
        out.view(torch.int64).fill_(0x7FBADBAD7FBADBAD)
    return out


def say(*args):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[gpu case]", *args, file=sys.stderr, flush=True)


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def float_equal_nan_ok(a: np.ndarray, b: np.ndarray, dtype: str) -> bool:
    """Bit equality except that any NaN matches any NaN (payloads not graded)."""
    if dtype in ("bf16", "fp16"):
        a = a.view(np.uint16)
        b = b.view(np.uint16)
        if dtype == "bf16":
            na = ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)
            nb = ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
        else:
            na = ((a & 0x7C00) == 0x7C00) & ((a & 0x3FF) != 0)
            nb = ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)
        return np.array_equal(na, nb) and np.array_equal(a[~na], b[~nb])
    if dtype == "fp32":
        na, nb = np.isnan(a), np.isnan(b)
        return np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))
    return np.array_equal(a, b)
