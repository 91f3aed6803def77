"""CPU oracle for the collectives hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library's product path never does:
it shares no code, header, table or helper with the oracle.

The arithmetic lives in ``coll_oracle.c`` (plain C, built with ``gcc -O2
-ffp-contract=off``); this module only marshals numpy arrays.  Buffers are
numpy arrays whose dtype names the element type:

* ``bf16``  -- ``np.uint16`` bit patterns (bfloat16 has no numpy dtype),
* ``fp16``  -- ``np.float16`` (viewed as ``np.uint16`` at the boundary),
* ``fp32``  -- ``np.float32``,
* ``int32`` -- ``np.int32``.

Every function names the page passage it follows in its docstring; the C file
states the readings taken where the pages are silent.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "coll_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libcoll_oracle.so")

DTYPES = {"bf16": 0, "fp16": 1, "fp32": 2, "int32": 3}
OPS = {"sum": 0, "prod": 1, "max": 2, "min": 3}
_ELEM = {"bf16": 2, "fp16": 2, "fp32": 4, "int32": 4}


def build(force: bool = True) -> str:
    """Compile ``coll_oracle.c`` into ``libcoll_oracle.so`` with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load(path: str) -> ctypes.CDLL:
    L = ctypes.CDLL(path)
    vp, sz, i32, i64p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p
    L.oracle_f32_to_bf16.restype = ctypes.c_uint16
    L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    for name in ("oracle_f32_to_bf16_n", "oracle_bf16_to_f32_n",
                 "oracle_f32_to_f16_n", "oracle_f16_to_f32_n", "oracle_f64_to_bf16_n"):
        getattr(L, name).argtypes = [sz, vp, vp]
        getattr(L, name).restype = None
    L.oracle_allreduce.argtypes = [i32, vp, vp, sz, i32, i32]
    L.oracle_reduce.argtypes = [i32, vp, vp, i32, sz, i32, i32]
    L.oracle_reduce_scatter.argtypes = [i32, vp, vp, sz, i32, i32]
    L.oracle_all_gather.argtypes = [i32, vp, vp, sz, sz]
    L.oracle_gather.argtypes = [i32, vp, vp, i32, sz, sz, sz]
    L.oracle_scatter.argtypes = [i32, vp, vp, i32, sz, sz]
    L.oracle_broadcast.argtypes = [i32, vp, vp, i32, sz, sz]
    L.oracle_all_to_all_v.argtypes = [i32, vp, i64p, i64p, vp, i64p, sz, i64p, i64p]
    L.oracle_moe_layout.argtypes = [i32, vp, i32, i32, i32, i64p, i64p, i64p, vp, vp]
    L.oracle_moe_permute.argtypes = [i32, vp, vp, i32, i32, sz, vp]
    L.oracle_moe_expert_scale.argtypes = [i32, vp, vp, i64p, i32, sz]
    L.oracle_moe_combine.argtypes = [i32, vp, vp, vp, i32, i32, sz, vp]
    L.oracle_all_to_all.argtypes = [i32, vp, vp, sz, sz]
    L.oracle_ulysses.argtypes = [i32, vp, vp, sz, sz, sz, sz, i32]
    L.oracle_lse_merge.argtypes = [i32, vp, vp, vp, vp, sz, sz, i32]
    for name in ("oracle_allreduce", "oracle_reduce", "oracle_reduce_scatter",
                 "oracle_all_gather", "oracle_gather", "oracle_scatter",
                 "oracle_broadcast", "oracle_all_to_all_v", "oracle_moe_layout",
                 "oracle_moe_permute", "oracle_moe_expert_scale",
                 "oracle_moe_combine", "oracle_all_to_all", "oracle_ulysses",
                 "oracle_lse_merge"):
        getattr(L, name).restype = ctypes.c_int
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        _lib = _load(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Run the oracle's functions against another build of ``coll_oracle.c``
    (the pin tests use it to show that planted mistakes are caught)."""
    global _lib
    saved = _lib
    _lib = _load(path)
    try:
        yield
    finally:
        _lib = saved


def compile_variant(source_text: str, out_path: str) -> str:
    """Compile a (modified) copy of the oracle source with the same flags."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                           "-w", "-o", out_path, src, "-lm"])
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what}: oracle status {rc}")


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle buffers must be C-contiguous"
    return a.ctypes.data


def _ptrs(arrs) -> ctypes.Array:
    return (ctypes.c_void_p * len(arrs))(*[_ptr(a) for a in arrs])


def _bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """The array as the element storage the C side expects."""
    want = {"bf16": np.uint16, "fp16": np.float16, "fp32": np.float32,
            "int32": np.int32}[dtype]
    if a.dtype != want:
        raise TypeError(f"{dtype} buffer must be {np.dtype(want).name}, got {a.dtype}")
    return np.ascontiguousarray(a)


# ---------------------------------------------------------------- conversions

def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (bfloat16 definition)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_bf16_n(x.size, _ptr(x), _ptr(out))
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_bf16_to_f32_n(h.size, _ptr(h), _ptr(out))
    return out


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits in one rounding, to nearest even (bfloat16 definition)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f64_to_bf16_n(x.size, _ptr(x), _ptr(out))
    return out


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """fp32 -> binary16 bits, round to nearest even (IEEE-754 definition)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_f16_n(x.size, _ptr(x), _ptr(out))
    return out


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_f16_to_f32_n(h.size, _ptr(h), _ptr(out))
    return out


# ----------------------------------------------------------------- primitives

def allreduce(xs, dtype: str, op: str = "sum"):
    """AllReduce (primitives tutorial, section 6): every rank gets the same
    reduction, ranks folded in ascending order in fp32 (int32: wrapping)."""
    xs = [_bits(x, dtype) for x in xs]
    n = xs[0].size
    assert all(x.size == n for x in xs)
    outs = [np.empty_like(x) for x in xs]
    _check(lib().oracle_allreduce(len(xs), _ptrs(xs), _ptrs(outs), n,
                                  DTYPES[dtype], OPS[op]), "allreduce")
    return outs


def reduce(xs, root: int, dtype: str, op: str = "sum"):
    """Reduce (section 3): the reduction lands on ``root`` only."""
    xs = [_bits(x, dtype) for x in xs]
    out = np.empty_like(xs[0])
    _check(lib().oracle_reduce(len(xs), _ptrs(xs), _ptr(out), root, xs[0].size,
                               DTYPES[dtype], OPS[op]), "reduce")
    return out


def reduce_scatter(xs, dtype: str, op: str = "sum"):
    """ReduceScatter (section 5): rank r keeps chunk r of the reduction."""
    xs = [_bits(x, dtype) for x in xs]
    R = len(xs)
    assert xs[0].size % R == 0
    n = xs[0].size // R
    outs = [np.empty(n, xs[0].dtype) for _ in range(R)]
    _check(lib().oracle_reduce_scatter(R, _ptrs(xs), _ptrs(outs), n,
                                       DTYPES[dtype], OPS[op]), "reduce_scatter")
    return outs


def all_gather(xs):
    """AllGather (section 7): rank-order concatenation on every rank."""
    xs = [np.ascontiguousarray(x) for x in xs]
    R, n = len(xs), xs[0].size
    outs = [np.empty(R * n, xs[0].dtype) for _ in range(R)]
    _check(lib().oracle_all_gather(R, _ptrs(xs), _ptrs(outs), n, xs[0].itemsize),
           "all_gather")
    return outs


def gather(xs, root: int = 0):
    """Gather (section 2, 2.2.1): [outer, inner] blocks concatenated along the
    last axis onto the root, giving [outer, R*inner]."""
    xs = [np.ascontiguousarray(x) for x in xs]
    R = len(xs)
    x0 = xs[0] if xs[0].ndim == 2 else xs[0].reshape(1, -1)
    outer, inner = x0.shape
    out = np.empty((outer, R * inner), xs[0].dtype)
    _check(lib().oracle_gather(R, _ptrs(xs), _ptr(out), root, outer, inner,
                               xs[0].itemsize), "gather")
    return out


def scatter(x_root: np.ndarray, R: int, root: int = 0):
    """Scatter (section 4): root's buffer cut into R equal chunks."""
    x = np.ascontiguousarray(x_root).reshape(-1)
    assert x.size % R == 0
    n = x.size // R
    outs = [np.empty(n, x.dtype) for _ in range(R)]
    _check(lib().oracle_scatter(R, _ptr(x), _ptrs(outs), root, n, x.itemsize),
           "scatter")
    return outs


def broadcast(x_root: np.ndarray, R: int, root: int, outs=None):
    """Broadcast (section 1): every rank gets root's bytes.  ``outs`` may hold
    the root's own array at index ``root``; it is then left untouched."""
    x = np.ascontiguousarray(x_root)
    if outs is None:
        outs = [np.empty_like(x) for _ in range(R)]
    _check(lib().oracle_broadcast(R, _ptr(x), _ptrs(outs), root, x.size,
                                  x.itemsize), "broadcast")
    return outs


def packed_displs(counts: np.ndarray):
    """MPI-style packed displacements: sdispls[s][d] = exclusive prefix over d,
    rdispls[d][s] = exclusive prefix over s of counts[s][d]."""
    counts = np.asarray(counts, np.int64)
    R = counts.shape[0]
    sd = np.zeros((R, R), np.int64)
    rd = np.zeros((R, R), np.int64)
    for s in range(R):
        acc = 0
        for d in range(R):
            sd[s, d] = acc
            acc += counts[s, d]
    for d in range(R):
        acc = 0
        for s in range(R):
            rd[d, s] = acc
            acc += counts[s, d]
    return sd, rd


def all_to_all_v(sends, counts, sdispls, rdispls, recv_rows, row_elems: int,
                 recvs=None):
    """All-to-All-v (section 8.1-8.2): rows sent from s to d land at
    rdispls[d][s] of d's buffer, grouped by ascending source."""
    sends = [np.ascontiguousarray(x).reshape(-1) for x in sends]
    R = len(sends)
    counts = np.ascontiguousarray(counts, np.int64).reshape(R, R)
    sdispls = np.ascontiguousarray(sdispls, np.int64).reshape(R, R)
    rdispls = np.ascontiguousarray(rdispls, np.int64).reshape(R, R)
    es = sends[0].itemsize
    send_rows = np.array([x.size // row_elems for x in sends], np.int64)
    recv_rows = np.ascontiguousarray(recv_rows, np.int64)
    if recvs is None:
        recvs = [np.zeros(int(recv_rows[d]) * row_elems, sends[0].dtype) for d in range(R)]
    _check(lib().oracle_all_to_all_v(R, _ptrs(sends), _ptr(counts), _ptr(sdispls),
                                     _ptrs(recvs), _ptr(rdispls), row_elems * es,
                                     _ptr(send_rows), _ptr(recv_rows)), "all_to_all_v")
    return recvs


def moe_layout(ids, E: int):
    """MoE dispatch layout (section 8.4): per-source expert histogram, counts
    per destination rank, displacements and stable send-slot positions.  Ids
    outside [0, E) are skipped (pos = -1)."""
    ids = [np.ascontiguousarray(x, np.int32) for x in ids]
    R = len(ids)
    T, K = ids[0].shape
    sc = np.zeros((R, R), np.int64)
    sd = np.zeros((R, R), np.int64)
    rd = np.zeros((R, R), np.int64)
    ec = np.zeros((R, E), np.int32)
    pos = [np.zeros((T, K), np.int32) for _ in range(R)]
    _check(lib().oracle_moe_layout(R, _ptrs(ids), T, K, E, _ptr(sc), _ptr(sd),
                                   _ptr(rd), _ptr(ec), _ptrs(pos)), "moe_layout")
    return dict(sendcounts=sc, sdispls=sd, rdispls=rd, expert_counts=ec, pos=pos)


def moe_permute(xs, pos):
    """Dispatch permute: send_s[pos_s[t,k]] = x_s[t] (an indexed write)."""
    xs = [np.ascontiguousarray(x) for x in xs]
    pos = [np.ascontiguousarray(p, np.int32) for p in pos]
    R = len(xs)
    T, H = xs[0].shape
    K = pos[0].shape[1]
    sends = [np.zeros((T * K, H), xs[0].dtype) for _ in range(R)]
    _check(lib().oracle_moe_permute(R, _ptrs(xs), _ptrs(pos), T, K,
                                    H * xs[0].itemsize, _ptrs(sends)), "moe_permute")
    return sends


def moe_expert_scale(recvs, expert_counts, rdispls, E: int, hidden: int):
    """Test expert y = rne(x * (1 + e/256)) on received bf16 rows, in place on
    copies of ``recvs``; returns the new buffers."""
    outs = [np.array(r, np.uint16, copy=True).reshape(-1) for r in recvs]
    ec = np.ascontiguousarray(expert_counts, np.int32)
    rd = np.ascontiguousarray(rdispls, np.int64)
    _check(lib().oracle_moe_expert_scale(len(outs), _ptrs(outs), _ptr(ec), _ptr(rd),
                                         E, hidden), "moe_expert_scale")
    return outs


def moe_combine(backs, pos, w, hidden: int):
    """Combine: out_s[t] = rne(sum_k w[t,k] * back_s[pos[t,k]]), k ascending,
    multiply and add rounded separately (results return to the token's owner)."""
    backs = [np.ascontiguousarray(b, np.uint16).reshape(-1) for b in backs]
    pos = [np.ascontiguousarray(p, np.int32) for p in pos]
    w = [np.ascontiguousarray(x, np.float32) for x in w]
    R = len(backs)
    T, K = pos[0].shape
    outs = [np.zeros((T, hidden), np.uint16) for _ in range(R)]
    _check(lib().oracle_moe_combine(R, _ptrs(backs), _ptrs(pos), _ptrs(w), T, K,
                                    hidden, _ptrs(outs)), "moe_combine")
    return outs


def moe_pipeline(xs, ids, w, E: int):
    """The whole MoE exchange of section 8.4: layout -> permute -> A2A-v ->
    expert -> A2A-v with transposed counts -> combine.  Returns every stage."""
    R = len(xs)
    T, H = xs[0].shape
    lay = moe_layout(ids, E)
    sends = moe_permute(xs, lay["pos"])
    sc, sd, rd = lay["sendcounts"], lay["sdispls"], lay["rdispls"]
    recv_rows = sc.sum(axis=0)
    recvs = all_to_all_v(sends, sc, sd, rd, recv_rows, H)
    ys = moe_expert_scale(recvs, lay["expert_counts"], rd, E, H)
    # reverse exchange: d sends back counts[s][d] rows from rdispls[d][s] to
    # s's slot sdispls[s][d]; as matrices that is counts^T with the two
    # displacement tables swapped.
    send_rows_back = np.array([T * ids[0].shape[1]] * R, np.int64)
    backs = all_to_all_v(ys, sc.T.copy(), rd, sd, send_rows_back, H)
    outs = moe_combine(backs, lay["pos"], w, H)
    return dict(layout=lay, sends=sends, recvs=recvs, ys=ys, backs=backs, outs=outs)


def all_to_all(xs):
    """all_to_all_single with equal splits: out[d][s*n+i] = in[s][d*n+i]."""
    xs = [np.ascontiguousarray(x).reshape(-1) for x in xs]
    R = len(xs)
    assert xs[0].size % R == 0
    n = xs[0].size // R
    outs = [np.empty_like(xs[0]) for _ in range(R)]
    _check(lib().oracle_all_to_all(R, _ptrs(xs), _ptrs(outs), n, xs[0].itemsize), "all_to_all")
    return outs


def ulysses(xs, SL: int, H: int, D: int, to_heads: bool):
    """Sequence <-> heads re-shard: to_heads maps x_s [SL, H, D] to
    y_d [R*SL, H/R, D]; otherwise the inverse."""
    xs = [np.ascontiguousarray(x).reshape(-1) for x in xs]
    R = len(xs)
    outs = [np.empty_like(xs[0]) for _ in range(R)]
    _check(lib().oracle_ulysses(R, _ptrs(xs), _ptrs(outs), SL, H, D, xs[0].itemsize,
                                1 if to_heads else 0), "ulysses")
    return outs


def lse_merge(o_parts, lse_parts, dtype: str):
    """Context-parallel merge (primitives tutorial 5.4.2 / 7.4.3): partial
    attention outputs o_r [rows, D] with their log-sum-exps l_r [rows] (fp32)
    -> the corrected sum o and L = log sum exp l_r, in fp64, rounded once.
    Returns (o, L) (every rank receives the same)."""
    o_parts = [_bits(o, dtype) for o in o_parts]
    lse_parts = [np.ascontiguousarray(l, np.float32) for l in lse_parts]
    R = len(o_parts)
    rows = lse_parts[0].size
    D = o_parts[0].size // rows
    outs = [np.empty_like(o_parts[0]) for _ in range(R)]
    ls = [np.empty(rows, np.float32) for _ in range(R)]
    _check(lib().oracle_lse_merge(R, _ptrs(o_parts), _ptrs(lse_parts), _ptrs(outs), _ptrs(ls),
                                  rows, D, DTYPES[dtype]), "lse_merge")
    return outs[0], ls[0]
