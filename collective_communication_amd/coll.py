"""ctypes binding of libcoll.so -- argument marshalling only.

Every function takes lists of CUDA (HIP) tensors, one per virtual rank,
checks shapes and dtypes on the host, passes raw device pointers and the
current stream to the C ABI in ``include/coll.h``, and raises ``CollError`` on
a negative status.  All computation happens in the library's HIP kernels;
there is no fallback: if ``libcoll.so`` has not been built this module raises
on first use.

``prepare(fn, *args)`` runs those checks once and returns a ``Plan`` that only
re-issues the C call (on the current stream), for loops that repeat a
collective on persistent buffers.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcoll.so")

COLL_BF16, COLL_FP16, COLL_FP32, COLL_INT32 = 0, 1, 2, 3
OPS = {"sum": 0, "prod": 1, "max": 2, "min": 3}
MAX_RANKS = 16
ARENA_ALIGN = 2 << 20           # COLL_ARENA_ALIGN of include/coll.h

_REDUCE_DTYPES = {torch.bfloat16: COLL_BF16, torch.float16: COLL_FP16,
                  torch.float32: COLL_FP32, torch.int32: COLL_INT32}

# exported symbol -> (restype, argtypes)
_vp, _sz, _i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
SIGNATURES = {
    "coll_status_string": (ctypes.c_char_p, [_i]),
    "coll_version": (_i, []),
    "coll_arena_layout": (_i, [_i, _vp, _vp, _vp]),
    "coll_allreduce": (_i, [_i, _vp, _vp, _sz, _i, _i, _vp]),
    "coll_reduce_scatter": (_i, [_i, _vp, _vp, _sz, _i, _i, _vp]),
    "coll_reduce": (_i, [_i, _vp, _vp, _i, _sz, _i, _i, _vp]),
    "coll_scatter": (_i, [_i, _vp, _vp, _i, _sz, _i, _vp]),
    "coll_all_gather": (_i, [_i, _vp, _vp, _sz, _i, _vp]),
    "coll_gather": (_i, [_i, _vp, _vp, _i, _sz, _sz, _i, _vp]),
    "coll_broadcast": (_i, [_i, _vp, _vp, _i, _sz, _i, _vp]),
    "coll_all_to_all_v": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _sz, _i, _sz, _vp, _vp, _vp]),
    "coll_all_to_all_v_workspace_bytes": (_sz, [_i, _sz, _sz, _i]),
    "coll_all_to_all_v_ws": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _sz, _i, _sz, _vp, _vp, _vp,
                                  _sz, _vp]),
    "coll_all_to_all_v_reverse": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _sz, _i, _sz, _vp, _vp, _vp,
                                       _sz, _vp]),
    "coll_all_to_all_v_ws_build": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _sz, _i, _sz, _vp, _vp,
                                        _vp, _sz, _vp]),
    "coll_all_to_all_v_reverse_build": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _sz, _i, _sz, _vp,
                                             _vp, _vp, _sz, _vp]),
    "coll_all_to_all_v_ws_copy": (_i, [_i, _sz, _i, _sz, _vp, _sz, _vp]),
    "coll_all_to_all": (_i, [_i, _vp, _vp, _sz, _i, _vp]),
    "coll_seq_heads_reshard": (_i, [_i, _vp, _vp, _sz, _sz, _sz, _i, _i, _vp]),
    "coll_lse_merge": (_i, [_i, _vp, _vp, _vp, _vp, _sz, _sz, _i, _vp]),
    "coll_moe_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "coll_moe_layout": (_i, [_i, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "coll_moe_layout_noalloc": (_i, [_i, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "coll_moe_permute": (_i, [_i, _vp, _vp, _i, _i, _sz, _i, _vp, _vp]),
    "coll_moe_expert_workspace_bytes": (_sz, [_i, _i, _sz]),
    "coll_moe_expert_scale": (_i, [_i, _vp, _vp, _vp, _i, _sz, _i, _sz, _vp, _vp, _sz, _vp]),
    "coll_moe_expert_scale_build": (_i, [_i, _vp, _vp, _vp, _i, _sz, _i, _sz, _vp, _vp, _sz,
                                         _vp]),
    "coll_moe_expert_scale_apply": (_i, [_i, _vp, _i, _sz, _i, _sz, _vp, _sz, _vp]),
    "coll_moe_combine": (_i, [_i, _vp, _vp, _vp, _i, _i, _sz, _i, _vp, _vp]),
    "coll_moe_dispatch": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _i, _i, _sz, _i, _vp, _vp, _vp]),
    "coll_moe_combine_recv": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _sz, _i, _vp,
                                   _vp, _vp]),
}


class CollError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().coll_status_string(status).decode()} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcoll.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m collective_communication_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        raise CollError(status, what)


# The current stream's raw handle for a device index.  torch's own accessor
# returns it without building a Stream object: 0.06 us per call on an MI355X
# host, against 2.7 us for torch.cuda.current_stream(), which was most of a
# decode-sized call's host cost.  Falls back to the public API if absent.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _current_stream(device=None) -> int:
    if _raw_stream is not None:
        return int(_raw_stream(torch.cuda.current_device() if device is None else device))
    return torch.cuda.current_stream(device).cuda_stream


def _stream(stream, device=None) -> int:
    if stream is None:
        return _current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, what: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{what}: tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    return t.data_ptr()


def _table(ts: Sequence[torch.Tensor], what: str, R: int):
    """R device pointers as a C array.  Every per-rank list must hold exactly
    R entries: the library reads R pointers from each table it is given."""
    if len(ts) != R:
        raise ValueError(f"{what}: {len(ts)} buffers for {R} ranks (one per rank)")
    return (ctypes.c_void_p * R)(*[_dev(t, what) for t in ts])


def _rows(ts: Sequence[torch.Tensor], row_elems: int):
    """Rows each rank's buffer holds, as the C array of int64 the exchanges
    bound their blocks by (a block whose rows do not all exist is not moved)."""
    return (ctypes.c_int64 * len(ts))(
        *[t.numel() // row_elems if row_elems > 0 else 0 for t in ts])


def _ranks(ts, what) -> int:
    R = len(ts)
    if not 1 <= R <= MAX_RANKS:
        raise ValueError(f"{what}: {R} ranks (1..{MAX_RANKS} supported)")
    return R


def _copy_dtype(t: torch.Tensor) -> tuple[int, int]:
    """(coll dtype code, elements-per-tensor-element) for pure copies."""
    es = t.element_size()
    if es == 2:
        return COLL_BF16, 1
    if es == 4:
        return COLL_FP32, 1
    if es == 8:
        return COLL_FP32, 2
    raise ValueError(f"element size {es} not supported by the copy primitives")


def _reduce_dtype(t: torch.Tensor) -> int:
    if t.dtype not in _REDUCE_DTYPES:
        raise ValueError(f"reductions support bf16/fp16/fp32/int32, got {t.dtype}")
    return _REDUCE_DTYPES[t.dtype]


def _same(ts, dtype, numel, what):
    for t in ts:
        if t.dtype != dtype or t.numel() != numel:
            raise ValueError(f"{what}: every rank needs {numel} elements of {dtype}")


# ------------------------------------------------------------- rank arena

def arena_layout(sizes: Sequence[int]) -> tuple[list[int], int]:
    """Offsets (from an ARENA_ALIGN-aligned base) and total size that
    ``coll_arena_layout`` gives buffers of ``sizes`` bytes, in order."""
    n = len(sizes)
    b = (ctypes.c_size_t * max(n, 1))(*[int(x) for x in sizes])
    o = (ctypes.c_size_t * max(n, 1))()
    tot = ctypes.c_size_t()
    _check(lib().coll_arena_layout(n, b, o, ctypes.byref(tot)), "arena_layout")
    return [int(o[k]) for k in range(n)], int(tot.value)


def rank_arena(groups, device="cuda"):
    """Allocate groups of rank buffers in one device allocation, placed by
    ``coll_arena_layout`` (each buffer on its own 2 MiB boundary plus a 4 KiB
    colour that differs from its neighbours'), so that the R same-offset
    streams of a collective spread over the HBM channels.

    Each group is either ``(count, shape, dtype)`` (``count`` buffers alike)
    or a list of ``(shape, dtype)`` (one per buffer).  Returns one list of
    uninitialised tensors per group, in order; they are views of one
    allocation, which lives as long as any of them."""
    specs, counts = [], []
    for g in groups:
        items = g if isinstance(g, list) else [(g[1], g[2])] * int(g[0])
        counts.append(len(items))
        for shape, dtype in items:
            shape = (shape,) if isinstance(shape, int) else tuple(int(d) for d in shape)
            numel = 1
            for d in shape:
                numel *= d
            specs.append((shape, dtype, numel * torch.empty(0, dtype=dtype).element_size()))
    offs, total = arena_layout([nb for _, _, nb in specs])
    raw = torch.empty(total + ARENA_ALIGN, dtype=torch.uint8, device=device)
    base = (-raw.data_ptr()) % ARENA_ALIGN
    views = [raw[base + o: base + o + nb].view(dtype).view(shape)
             for (shape, dtype, nb), o in zip(specs, offs)]
    out, k = [], 0
    for c in counts:
        out.append(views[k:k + c])
        k += c
    return out


# ----------------------------------------------------------- prepared calls

_PLANNING = threading.local()


class Plan:
    """A library call validated and marshalled once: calling it re-issues the
    same entry point with the same buffers on a stream (default: the current
    one).  The plan holds references to every argument it was made from
    (tensors included), so its device pointers stay valid for its lifetime;
    the caller must not resize or re-point those tensors."""

    __slots__ = ("_fn", "_args", "_what", "_keep", "_dev")

    def __init__(self, fn, args, what):
        self._fn, self._args, self._what = fn, args, what
        self._keep = None
        # the device whose current stream a call without `stream` uses
        self._dev = torch.cuda.current_device() if torch.cuda.is_available() else None

    def __call__(self, stream=None):
        st = _stream(stream, self._dev)
        rc = self._fn(*self._args, st)
        if rc:
            _check(rc, self._what)


def _issue(name: str, what: str, stream, *args):
    """Call entry point `name` with the marshalled `args` and the stream, or,
    inside prepare(), return them as a Plan (which keeps the ctypes pointer
    tables alive)."""
    fn = getattr(lib(), name)
    if getattr(_PLANNING, "on", False):
        return Plan(fn, args, what)
    _check(fn(*args, _stream(stream)), what)
    return None


def prepare(call, *args, **kwargs) -> Plan:
    """Validate and marshal `call(*args, **kwargs)` (any collective of this
    module) once and return a Plan that only re-issues the C call.  For loops
    that repeat one collective on persistent buffers, where the per-call
    argument checks would otherwise dominate small messages."""
    _PLANNING.on = True
    try:
        plan = call(*args, **kwargs)
    finally:
        _PLANNING.on = False
    if not isinstance(plan, Plan):
        raise TypeError(f"{getattr(call, '__name__', call)} cannot be prepared")
    # the plan owns what its pointers came from: a device tensor made inline
    # for the call (e.g. a count table) must not be freed and reused
    plan._keep = (call, args, kwargs)
    return plan


# --------------------------------------------------------------------- API

def allreduce(sends, recvs, op: str = "sum", stream=None):
    """AllReduce: every recvs[r] gets the reduction of all sends (recvs may be sends)."""
    R = _ranks(sends, "allreduce")
    n = sends[0].numel()
    _same(sends, sends[0].dtype, n, "allreduce send")
    _same(recvs, sends[0].dtype, n, "allreduce recv")
    if len(recvs) != R:
        raise ValueError("allreduce: one recv per rank")
    return _issue("coll_allreduce", "allreduce", stream, R, _table(sends, "send", R),
                  _table(recvs, "recv", R), n, _reduce_dtype(sends[0]), OPS[op])


def reduce_scatter(sends, recvs, op: str = "sum", stream=None):
    """ReduceScatter: recvs[r] = chunk r of the reduction (sends hold R chunks)."""
    R = _ranks(sends, "reduce_scatter")
    n = recvs[0].numel()
    _same(sends, sends[0].dtype, R * n, "reduce_scatter send")
    _same(recvs, sends[0].dtype, n, "reduce_scatter recv")
    return _issue("coll_reduce_scatter", "reduce_scatter", stream, R, _table(sends, "send", R),
                  _table(recvs, "recv", R), n, _reduce_dtype(sends[0]), OPS[op])


def reduce(sends, recv_root, root: int, op: str = "sum", stream=None):
    """Reduce: recv_root = reduction of all sends (recv_root may be sends[root])."""
    R = _ranks(sends, "reduce")
    n = sends[0].numel()
    _same(sends, sends[0].dtype, n, "reduce send")
    _same([recv_root], sends[0].dtype, n, "reduce recv")
    return _issue("coll_reduce", "reduce", stream, R, _table(sends, "send", R),
                  _dev(recv_root, "recv"), root, n, _reduce_dtype(sends[0]), OPS[op])


def scatter(send_root, recvs, root: int, stream=None):
    """Scatter: recvs[r] = chunk r of send_root (R equal chunks)."""
    R = _ranks(recvs, "scatter")
    n = recvs[0].numel()
    _same(recvs, send_root.dtype, n, "scatter recv")
    if send_root.numel() != R * n:
        raise ValueError("scatter: the root buffer must hold R chunks")
    dt, mult = _copy_dtype(send_root)
    return _issue("coll_scatter", "scatter", stream, R, _dev(send_root, "send"),
                  _table(recvs, "recv", R), root, n * mult, dt)


def all_gather(sends, recvs, stream=None):
    """AllGather: recvs[r] = concatenation of sends in rank order."""
    R = _ranks(sends, "all_gather")
    n = sends[0].numel()
    _same(sends, sends[0].dtype, n, "all_gather send")
    _same(recvs, sends[0].dtype, R * n, "all_gather recv")
    dt, mult = _copy_dtype(sends[0])
    return _issue("coll_all_gather", "all_gather", stream, R, _table(sends, "send", R),
                  _table(recvs, "recv", R), n * mult, dt)


def gather(sends, recv_root, root: int = 0, stream=None):
    """Gather: sends[q] of shape [outer, inner] concatenated along the last
    axis into recv_root [outer, R*inner]; only the root's buffer is written."""
    R = _ranks(sends, "gather")
    s0 = sends[0]
    outer = s0.shape[0] if s0.dim() == 2 else 1
    inner = s0.shape[-1] if s0.dim() >= 1 else 1
    _same(sends, s0.dtype, outer * inner, "gather send")
    if recv_root.dtype != s0.dtype or recv_root.numel() != outer * R * inner:
        raise ValueError("gather: root buffer must be [outer, R*inner] of the send dtype")
    dt, mult = _copy_dtype(s0)
    return _issue("coll_gather", "gather", stream, R, _table(sends, "send", R),
                  _dev(recv_root, "recv"), root, outer, inner * mult, dt)


def broadcast(send_root, recvs, root: int, stream=None):
    """Broadcast: every recvs[r] = send_root (recvs[root] may be send_root)."""
    R = _ranks(recvs, "broadcast")
    n = send_root.numel()
    _same(recvs, send_root.dtype, n, "broadcast recv")
    dt, mult = _copy_dtype(send_root)
    return _issue("coll_broadcast", "broadcast", stream, R, _dev(send_root, "send"),
                  _table(recvs, "recv", R), root, n * mult, dt)


def _a2av_shape(sends, recvs, row_elems: int, what: str, capacity=None):
    R = _ranks(sends, what)
    if len(recvs) != R:
        raise ValueError(f"{what}: one recv per rank")
    dt, mult = _copy_dtype(sends[0])
    for t in list(sends) + list(recvs):
        if t.dtype != sends[0].dtype:
            raise ValueError(f"{what}: one dtype for every buffer")
    # receive capacity in rows: an upper bound of the rows moved (sizes the
    # launch only); by default the rows the receive buffers hold
    if capacity is None:
        capacity = sum(t.numel() // row_elems for t in recvs) if row_elems > 0 else 0
    elif int(capacity) < 0:
        raise ValueError(f"{what}: capacity must be >= 0")
    return R, dt, mult, int(capacity)


def all_to_all_v_workspace_bytes(sends, recvs, row_elems: int, capacity=None) -> int:
    """Workspace bytes all_to_all_v(..., workspace=) needs for these buffers
    (0: the descriptor form does not apply and no workspace is needed)."""
    R, dt, mult, capacity = _a2av_shape(sends, recvs, row_elems, "all_to_all_v", capacity)
    return int(lib().coll_all_to_all_v_workspace_bytes(R, capacity, row_elems * mult, dt))


def all_to_all_v(sends, sendcounts, sdispls, recvs, rdispls, row_elems: int,
                 stream=None, workspace=None, capacity=None):
    """All-to-All-v with device int64 [R*R] counts (s-major), sdispls (s-major)
    and rdispls (d-major), in rows of ``row_elems`` elements.  With a device
    ``workspace`` (all_to_all_v_workspace_bytes) large exchanges take the
    descriptor form.  ``capacity`` (receive rows the launch is sized for;
    default: the rows the receive buffers hold) shapes the launch, never the
    result."""
    R, dt, mult, capacity = _a2av_shape(sends, recvs, row_elems, "all_to_all_v", capacity)
    for t, name in ((sendcounts, "sendcounts"), (sdispls, "sdispls"), (rdispls, "rdispls")):
        if t.dtype != torch.int64 or t.numel() != R * R:
            raise ValueError(f"all_to_all_v: {name} must be int64 [R*R] on the device")
    args = (R, _table(sends, "send", R), _dev(sendcounts, "counts"), _dev(sdispls, "sdispls"),
            _table(recvs, "recv", R), _dev(rdispls, "rdispls"), row_elems * mult, dt, capacity,
            _rows(sends, row_elems), _rows(recvs, row_elems))
    if workspace is None:
        return _issue("coll_all_to_all_v", "all_to_all_v", stream, *args)
    ws_bytes = workspace.numel() * workspace.element_size()
    return _issue("coll_all_to_all_v_ws", "all_to_all_v", stream, *args,
                  _dev(workspace, "workspace"), ws_bytes)


def all_to_all_v_reverse(recvs, sendcounts, sdispls, sends, rdispls, row_elems: int,
                         stream=None, workspace=None, capacity=None):
    """The reverse of all_to_all_v(sends, sendcounts, sdispls, recvs, rdispls):
    every block of ``recvs`` goes back to its place in ``sends``, reading the
    forward tables as they are (no transposed count matrix).  ``workspace``:
    as all_to_all_v, sized with all_to_all_v_workspace_bytes(recvs, sends, ...).
    ``capacity``: rows the launch is sized for (default: the rows ``sends``
    holds)."""
    R, dt, mult, capacity = _a2av_shape(recvs, sends, row_elems, "all_to_all_v_reverse",
                                        capacity)
    for t, name in ((sendcounts, "sendcounts"), (sdispls, "sdispls"), (rdispls, "rdispls")):
        if t.dtype != torch.int64 or t.numel() != R * R:
            raise ValueError(f"all_to_all_v_reverse: {name} must be int64 [R*R] on the device")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    return _issue("coll_all_to_all_v_reverse", "all_to_all_v_reverse", stream, R,
                  _table(recvs, "recv", R), _dev(sendcounts, "counts"), _dev(sdispls, "sdispls"),
                  _table(sends, "send", R), _dev(rdispls, "rdispls"), row_elems * mult, dt,
                  capacity, _rows(sends, row_elems), _rows(recvs, row_elems), ws_ptr, ws_bytes)


def _desc_need(R, dt, row_bytes_elems, capacity, what):
    need = int(lib().coll_all_to_all_v_workspace_bytes(R, capacity, row_bytes_elems, dt))
    if need == 0:
        raise ValueError(f"{what}: the descriptor form does not apply to these sizes "
                         "(all_to_all_v_workspace_bytes is 0); call the one-call form")
    return need


def all_to_all_v_build(sends, sendcounts, sdispls, recvs, rdispls, row_elems: int, workspace,
                       stream=None, capacity=None):
    """First half of all_to_all_v(..., workspace=): writes the descriptor
    tables (block table with these buffers' addresses, one block index per
    tile) into ``workspace`` and moves nothing.  It needs only the tables and
    the buffers' addresses, so it may run before the send buffers are written,
    e.g. on a second stream.  all_to_all_v_copy(sends, recvs, ...) then moves
    the rows.  Raises ValueError where the descriptor form does not apply."""
    R, dt, mult, capacity = _a2av_shape(sends, recvs, row_elems, "all_to_all_v_build", capacity)
    _layout_tables(R, (sendcounts, sdispls, rdispls), "all_to_all_v_build")
    _desc_need(R, dt, row_elems * mult, capacity, "all_to_all_v_build")
    ws_bytes = workspace.numel() * workspace.element_size()
    return _issue("coll_all_to_all_v_ws_build", "all_to_all_v_build", stream, R,
                  _table(sends, "send", R), _dev(sendcounts, "counts"), _dev(sdispls, "sdispls"),
                  _table(recvs, "recv", R), _dev(rdispls, "rdispls"), row_elems * mult, dt,
                  capacity, _rows(sends, row_elems), _rows(recvs, row_elems),
                  _dev(workspace, "workspace"), ws_bytes)


def all_to_all_v_reverse_build(recvs, sendcounts, sdispls, sends, rdispls, row_elems: int,
                               workspace, stream=None, capacity=None):
    """First half of all_to_all_v_reverse(..., workspace=), as
    all_to_all_v_build; all_to_all_v_copy(recvs, sends, ...) then moves the
    rows back."""
    R, dt, mult, capacity = _a2av_shape(recvs, sends, row_elems, "all_to_all_v_reverse_build",
                                        capacity)
    _layout_tables(R, (sendcounts, sdispls, rdispls), "all_to_all_v_reverse_build")
    _desc_need(R, dt, row_elems * mult, capacity, "all_to_all_v_reverse_build")
    ws_bytes = workspace.numel() * workspace.element_size()
    return _issue("coll_all_to_all_v_reverse_build", "all_to_all_v_reverse_build", stream, R,
                  _table(recvs, "recv", R), _dev(sendcounts, "counts"), _dev(sdispls, "sdispls"),
                  _table(sends, "send", R), _dev(rdispls, "rdispls"), row_elems * mult, dt,
                  capacity, _rows(sends, row_elems), _rows(recvs, row_elems),
                  _dev(workspace, "workspace"), ws_bytes)


def all_to_all_v_copy(sources, dests, row_elems: int, workspace, stream=None, capacity=None):
    """Second half of the descriptor form: the rows move between the buffers
    that the build on ``workspace`` was given.  ``sources`` / ``dests``: those
    buffers in the build's order (sends, recvs for all_to_all_v_build; recvs,
    sends for all_to_all_v_reverse_build); only their sizes and dtype are used
    here, to find the launch's shape."""
    R, dt, mult, capacity = _a2av_shape(sources, dests, row_elems, "all_to_all_v_copy", capacity)
    _desc_need(R, dt, row_elems * mult, capacity, "all_to_all_v_copy")
    ws_bytes = workspace.numel() * workspace.element_size()
    return _issue("coll_all_to_all_v_ws_copy", "all_to_all_v_copy", stream, R, row_elems * mult,
                  dt, capacity, _dev(workspace, "workspace"), ws_bytes)


def all_to_all(sends, recvs, stream=None):
    """all_to_all_single with equal splits: recvs[d][s*n+i] = sends[s][d*n+i]."""
    R = _ranks(sends, "all_to_all")
    total = sends[0].numel()
    if total % R:
        raise ValueError("all_to_all: the send buffer must split into R equal chunks")
    _same(sends, sends[0].dtype, total, "all_to_all send")
    _same(recvs, sends[0].dtype, total, "all_to_all recv")
    dt, mult = _copy_dtype(sends[0])
    return _issue("coll_all_to_all", "all_to_all", stream, R, _table(sends, "send", R),
                  _table(recvs, "recv", R), total // R * mult, dt)


def seq_heads_reshard(ins, outs, heads: int, head_dim: int, to_heads: bool,
                      stream=None):
    """[SL, H, D] per rank <-> [R*SL, H/R, D] per rank (to_heads selects the
    direction)."""
    R = _ranks(ins, "seq_heads_reshard")
    per = ins[0].numel()
    if heads % R or per % (heads * head_dim):
        raise ValueError("seq_heads_reshard: heads must divide by R and rows must be whole")
    SL = per // (heads * head_dim)          # both layouts hold SL*H*D elements per rank
    _same(ins, ins[0].dtype, per, "seq_heads_reshard in")
    _same(outs, ins[0].dtype, per, "seq_heads_reshard out")
    dt, mult = _copy_dtype(ins[0])
    return _issue("coll_seq_heads_reshard", "seq_heads_reshard", stream, R, _table(ins, "in", R),
                  _table(outs, "out", R), SL, heads, head_dim * mult, dt, 1 if to_heads else 0)


def lse_merge(o_parts, lse_parts, o_out, lse_out=None, stream=None):
    """Context-parallel merge: o_parts[r] [rows, D] (bf16/fp32) with fp32
    lse_parts[r] [rows] -> o_out[r] (and lse_out[r]) on every rank."""
    R = _ranks(o_parts, "lse_merge")
    rows = lse_parts[0].numel()
    D = o_parts[0].numel() // max(rows, 1)
    dt = {torch.bfloat16: COLL_BF16, torch.float32: COLL_FP32}.get(o_parts[0].dtype)
    if dt is None:
        raise ValueError("lse_merge: bf16 or fp32 outputs")
    _same(o_parts, o_parts[0].dtype, rows * D, "lse_merge o")
    _same(o_out, o_parts[0].dtype, rows * D, "lse_merge out")
    _same(lse_parts, torch.float32, rows, "lse_merge lse")
    lo = None
    if lse_out is not None:
        _same(lse_out, torch.float32, rows, "lse_merge lse_out")
        lo = _table(lse_out, "lse_out", R)
    return _issue("coll_lse_merge", "lse_merge", stream, R, _table(o_parts, "o", R),
                  _table(lse_parts, "lse", R), _table(o_out, "out", R), lo, rows, D, dt)


def moe_workspace_bytes(R: int, tokens: int, topk: int, n_experts: int) -> int:
    return int(lib().coll_moe_workspace_bytes(R, tokens, topk, n_experts))


def moe_layout(topk_ids, n_experts: int, sendcounts, sdispls, rdispls, expert_counts, pos,
               workspace, stream=None):
    """MoE layout from int32 [T, K] ids per rank into device count tables and
    int32 [T, K] send-slot positions (-1: an id outside [0, E))."""
    R = _ranks(topk_ids, "moe_layout")
    T, K = topk_ids[0].shape
    for t in topk_ids:
        if t.dtype != torch.int32 or tuple(t.shape) != (T, K):
            raise ValueError("moe_layout: ids must be int32 [T, K] on every rank")
    for t in pos:
        if t.dtype != torch.int32 or t.numel() != T * K:
            raise ValueError("moe_layout: pos must be int32 [T, K] on every rank")
    for t in (sendcounts, sdispls, rdispls):
        if t.dtype != torch.int64 or t.numel() != R * R:
            raise ValueError("moe_layout: count tables are int64 [R*R]")
    if expert_counts.dtype != torch.int32 or expert_counts.numel() != R * n_experts:
        raise ValueError("moe_layout: expert_counts is int32 [R*E]")
    ws_bytes = workspace.numel() * workspace.element_size()
    return _issue("coll_moe_layout", "moe_layout", stream, R, _table(topk_ids, "ids", R), T, K,
                  n_experts, _dev(sendcounts, "sc"), _dev(sdispls, "sd"), _dev(rdispls, "rd"),
                  _dev(expert_counts, "ec"), _table(pos, "pos", R), _dev(workspace, "ws"),
                  ws_bytes)


def moe_layout_noalloc(topk_ids, n_experts: int, sendcounts, sdispls, rdispls, expert_counts,
                       pos, stream=None):
    """moe_layout without a workspace: the scratch is the library's per-GPU
    device array (at most COLL_MOE_NOALLOC_MAX_BYTES of layout workspace);
    nothing is allocated.  Calls that overlap on one GPU must not be issued."""
    R = _ranks(topk_ids, "moe_layout_noalloc")
    T, K = topk_ids[0].shape
    for t in topk_ids:
        if t.dtype != torch.int32 or tuple(t.shape) != (T, K):
            raise ValueError("moe_layout_noalloc: ids must be int32 [T, K] on every rank")
    for t in pos:
        if t.dtype != torch.int32 or t.numel() != T * K:
            raise ValueError("moe_layout_noalloc: pos must be int32 [T, K] on every rank")
    for t in (sendcounts, sdispls, rdispls):
        if t.dtype != torch.int64 or t.numel() != R * R:
            raise ValueError("moe_layout_noalloc: count tables are int64 [R*R]")
    if expert_counts.dtype != torch.int32 or expert_counts.numel() != R * n_experts:
        raise ValueError("moe_layout_noalloc: expert_counts is int32 [R*E]")
    return _issue("coll_moe_layout_noalloc", "moe_layout_noalloc", stream, R,
                  _table(topk_ids, "ids", R), T, K, n_experts, _dev(sendcounts, "sc"),
                  _dev(sdispls, "sd"), _dev(rdispls, "rd"), _dev(expert_counts, "ec"),
                  _table(pos, "pos", R))


def moe_permute(xs, pos, sends, stream=None):
    """sends[s][pos[s][t,k]] = xs[s][t] (x [T, H], pos int32 [T, K], sends [T*K, H];
    pairs with pos = -1 are skipped)."""
    R = _ranks(xs, "moe_permute")
    T, H = xs[0].shape
    K = pos[0].shape[1]
    for x in xs:
        if tuple(x.shape) != (T, H) or x.dtype != xs[0].dtype:
            raise ValueError("moe_permute: x must be [T, H] of one dtype")
    for s in sends:
        if s.numel() != T * K * H or s.dtype != xs[0].dtype:
            raise ValueError("moe_permute: send buffers must be [T*K, H]")
    dt, mult = _copy_dtype(xs[0])
    return _issue("coll_moe_permute", "moe_permute", stream, R, _table(xs, "x", R),
                  _table(pos, "pos", R), T, K, H * mult, dt, _table(sends, "send", R))


def moe_expert_workspace_bytes(R: int, n_experts: int, rows_capacity: int = 0) -> int:
    """Workspace bytes of moe_expert_scale: the entry tables, plus 8 bytes per
    receive row of ``rows_capacity`` for the row-descriptor path (the receive
    buffers' rows together, as moe_expert_scale passes them)."""
    return int(lib().coll_moe_expert_workspace_bytes(R, n_experts, rows_capacity))


def moe_expert_scale(recvs, expert_counts, rdispls, n_experts: int, hidden: int, workspace,
                     stream=None):
    """Test expert y = rne(x * (1 + e/256)) in place on received bf16 rows.
    ``workspace``: a device tensor of at least moe_expert_workspace_bytes(R, E)
    bytes; moe_expert_workspace_bytes(R, E, rows) with rows = the receive
    buffers' rows together selects the faster row-descriptor path."""
    R = _ranks(recvs, "moe_expert_scale")
    for r in recvs:
        if r.dtype != torch.bfloat16:
            raise ValueError("moe_expert_scale: bf16 rows only")
    if expert_counts.dtype != torch.int32 or expert_counts.numel() != R * n_experts:
        raise ValueError("moe_expert_scale: expert_counts must be int32 [R*E] (one row per rank)")
    if rdispls.dtype != torch.int64 or rdispls.numel() != R * R:
        raise ValueError("moe_expert_scale: rdispls must be int64 [R*R]")
    capacity = sum(t.numel() // hidden for t in recvs) if hidden > 0 else 0
    ws_bytes = workspace.numel() * workspace.element_size()
    return _issue("coll_moe_expert_scale", "moe_expert_scale", stream, R, _table(recvs, "recv", R),
                  _dev(expert_counts, "ec"), _dev(rdispls, "rd"), n_experts, hidden, COLL_BF16,
                  capacity, _rows(recvs, hidden), _dev(workspace, "ws"), ws_bytes)


def _expert_split(recvs, n_experts, hidden, workspace, what):
    """Checks shared by the two halves of the row-descriptor path; returns
    (R, capacity, workspace bytes)."""
    R = _ranks(recvs, what)
    for r in recvs:
        if r.dtype != torch.bfloat16:
            raise ValueError(f"{what}: bf16 rows only")
    if n_experts < 1 or n_experts % R:
        raise ValueError(f"{what}: n_experts must be a positive multiple of the rank count")
    capacity = sum(t.numel() // hidden for t in recvs) if hidden > 0 else 0
    ws_bytes = workspace.numel() * workspace.element_size()
    if hidden <= 0 or hidden % 8 or capacity == 0 or R * n_experts > 8192 or \
            ws_bytes < moe_expert_workspace_bytes(R, n_experts, capacity):
        raise ValueError(f"{what}: the row-descriptor path does not apply (16-byte rows, a "
                         "nonzero capacity, R*E <= 8192 and a workspace of "
                         "moe_expert_workspace_bytes(R, E, capacity) bytes); call moe_expert_scale")
    return R, capacity, ws_bytes


def moe_expert_scale_build(recvs, expert_counts, rdispls, n_experts: int, hidden: int, workspace,
                           stream=None):
    """First half of moe_expert_scale's row-descriptor path: writes the row
    table and one descriptor per receive row into ``workspace`` and touches no
    row.  It needs only the layout's tables and the buffers' addresses, so it
    may run while the rows are still being exchanged, e.g. on a second stream.
    moe_expert_scale_apply(recvs, ...) then scales the rows.  Raises
    ValueError where that path does not apply."""
    R, capacity, ws_bytes = _expert_split(recvs, n_experts, hidden, workspace,
                                          "moe_expert_scale_build")
    if expert_counts.dtype != torch.int32 or expert_counts.numel() != R * n_experts:
        raise ValueError("moe_expert_scale_build: expert_counts must be int32 [R*E]")
    if rdispls.dtype != torch.int64 or rdispls.numel() != R * R:
        raise ValueError("moe_expert_scale_build: rdispls must be int64 [R*R]")
    return _issue("coll_moe_expert_scale_build", "moe_expert_scale_build", stream, R,
                  _table(recvs, "recv", R), _dev(expert_counts, "ec"), _dev(rdispls, "rd"),
                  n_experts, hidden, COLL_BF16, capacity, _rows(recvs, hidden),
                  _dev(workspace, "ws"), ws_bytes)


def moe_expert_scale_apply(recvs, n_experts: int, hidden: int, workspace, stream=None):
    """Second half: scales the received rows from the descriptors a
    moe_expert_scale_build on the same buffers wrote into ``workspace``."""
    R, capacity, ws_bytes = _expert_split(recvs, n_experts, hidden, workspace,
                                          "moe_expert_scale_apply")
    return _issue("coll_moe_expert_scale_apply", "moe_expert_scale_apply", stream, R,
                  _table(recvs, "recv", R), n_experts, hidden, COLL_BF16, capacity,
                  _dev(workspace, "ws"), ws_bytes)


def moe_combine(backs, pos, weights, outs, stream=None):
    """outs[s][t] = rne(sum_k w[s][t,k] * backs[s][pos[s][t,k]]), k ascending."""
    R = _ranks(backs, "moe_combine")
    T, K = pos[0].shape
    H = outs[0].shape[-1]
    for b in backs:
        if b.dtype != torch.bfloat16 or b.numel() != T * K * H:
            raise ValueError("moe_combine: back buffers are bf16 [T*K, H]")
    for w in weights:
        if w.dtype != torch.float32 or w.numel() != T * K:
            raise ValueError("moe_combine: weights are fp32 [T, K]")
    for o in outs:
        if o.dtype != torch.bfloat16 or o.numel() != T * H:
            raise ValueError("moe_combine: outputs are bf16 [T, H]")
    return _issue("coll_moe_combine", "moe_combine", stream, R, _table(backs, "back", R),
                  _table(pos, "pos", R), _table(weights, "w", R), T, K, H, COLL_BF16,
                  _table(outs, "out", R))


def _layout_tables(R, tables, what):
    for t, name in zip(tables, ("sendcounts", "sdispls", "rdispls")):
        if t.dtype != torch.int64 or t.numel() != R * R:
            raise ValueError(f"{what}: {name} must be int64 [R*R] on the device")


def moe_dispatch(xs, pos, sendcounts, sdispls, rdispls, recvs, stream=None):
    """Fused permute + All-to-All-v: every (t, k) row of xs[s] goes straight
    to its receive row in recvs[d] (the layout of moe_layout)."""
    R = _ranks(xs, "moe_dispatch")
    T, H = xs[0].shape
    K = pos[0].shape[1]
    _layout_tables(R, (sendcounts, sdispls, rdispls), "moe_dispatch")
    if len(recvs) != R:
        raise ValueError("moe_dispatch: one receive buffer per rank")
    for x in xs:
        if tuple(x.shape) != (T, H) or x.dtype != xs[0].dtype:
            raise ValueError("moe_dispatch: x must be [T, H] of one dtype")
    for r in recvs:
        if r.dtype != xs[0].dtype or r.numel() % max(H, 1) != 0:
            raise ValueError("moe_dispatch: receive buffers are [rows, H] of x's dtype")
    dt, mult = _copy_dtype(xs[0])
    return _issue("coll_moe_dispatch", "moe_dispatch", stream, R, _table(xs, "x", R),
                  _table(pos, "pos", R), _dev(sendcounts, "sc"), _dev(sdispls, "sd"),
                  _dev(rdispls, "rd"), T, K, H * mult, dt, _table(recvs, "recv", R),
                  _rows(recvs, H))


def moe_combine_recv(recvs, pos, sendcounts, sdispls, rdispls, weights, outs, topk_ids=None,
                     stream=None):
    """Fused reverse exchange + combine: outs[s][t] = rne(sum_k w * row_k), row_k
    read from the receive buffers where moe_dispatch put it; with topk_ids the
    test expert rne(x * (1 + e/256)) is applied to each row as it is read."""
    R = _ranks(recvs, "moe_combine_recv")
    T, K = pos[0].shape
    H = outs[0].shape[-1]
    _layout_tables(R, (sendcounts, sdispls, rdispls), "moe_combine_recv")
    for r in recvs:
        if r.dtype != torch.bfloat16 or r.numel() % max(H, 1) != 0:
            raise ValueError("moe_combine_recv: receive buffers are bf16 [rows, H]")
    for w in weights:
        if w.dtype != torch.float32 or w.numel() != T * K:
            raise ValueError("moe_combine_recv: weights are fp32 [T, K]")
    for o in outs:
        if o.dtype != torch.bfloat16 or o.numel() != T * H:
            raise ValueError("moe_combine_recv: outputs are bf16 [T, H]")
    ids = None
    if topk_ids is not None:
        for t in topk_ids:
            if t.dtype != torch.int32 or t.numel() != T * K:
                raise ValueError("moe_combine_recv: topk_ids are int32 [T, K]")
        ids = _table(topk_ids, "ids", R)
    return _issue("coll_moe_combine_recv", "moe_combine_recv", stream, R, _table(recvs, "recv", R),
                  _table(pos, "pos", R), _dev(sendcounts, "sc"), _dev(sdispls, "sd"),
                  _dev(rdispls, "rd"), _table(weights, "w", R), ids, T, K, H, COLL_BF16,
                  _table(outs, "out", R), _rows(recvs, H))
