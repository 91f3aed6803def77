"""Every entry point of the library run under CPU emulation on guarded host
buffers and compared with the oracle -- TEST INFRASTRUCTURE ONLY.

    python tests/cpuemu/cases.py <family> <start|end>

runs one family of cases, printing a line per case before it starts, and
exits non-zero on a mismatch.  A kernel that touches memory outside its
buffers hits a guard page and the process dies with SIGSEGV: the last
printed line names the case.  Sizes are small but span several tiles plus
ragged tails; grids use a 4-CU machine (EMU_CUS).
"""
from __future__ import annotations

import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from collective_communication_amd import synth  # noqa: E402
from collective_communication_amd.coll import SIGNATURES  # noqa: E402
from guarded import Heap, ptr, table  # noqa: E402

import build as emu_build  # noqa: E402

BF16, FP16, FP32, INT32 = 0, 1, 2, 3
DT = {"bf16": BF16, "fp16": FP16, "fp32": FP32, "int32": INT32}
OPS = {"sum": 0, "prod": 1, "max": 2, "min": 3}
NP = {"bf16": np.uint16, "fp16": np.float16, "fp32": np.float32, "int32": np.int32}

L = None
H = None


def load():
    global L
    L = ctypes.CDLL(emu_build.build())
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


def rows(ns):
    """Per-rank buffer rows as the C ABI's host int64 array."""
    return (ctypes.c_int64 * len(ns))(*[int(n) for n in ns])


def case(*what):
    print("case", *what, flush=True)


def ok(rc, what):
    if rc != 0:
        raise AssertionError(f"{what}: status {rc}")


def same(a, b, what):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    if a.shape != b.shape or not np.array_equal(a.view(np.uint8), b.view(np.uint8)):
        bad = np.flatnonzero(a.reshape(-1).view(np.uint8) != b.reshape(-1).view(np.uint8))
        raise AssertionError(f"{what}: mismatch ({bad.size} bytes, first at byte {bad[:1]})")


def gen(dtype, n, seed):
    if dtype == "int32":
        return synth.uniform_int32(n, -(1 << 20), 1 << 20, seed)
    return synth.gaussian(n, 1.0, seed, dtype)


# ------------------------------------------------------------------ families

def fam_reduce():
    for dtype in ("bf16", "fp16", "fp32", "int32"):
        for R in (1, 2, 3, 4, 8, 16):
            for n in (1, 9, 4100, 9000 + R):
                case("allreduce", dtype, R, n)
                xs = [gen(dtype, n, 17 * R + n + r) for r in range(R)]
                want = oracle.allreduce(xs, dtype)
                ins = [H.copy(x) for x in xs]
                outs = [H.poison(n, NP[dtype]) for _ in range(R)]
                ok(L.coll_allreduce(R, table(ins), table(outs), n, DT[dtype], 0, None), "allreduce")
                for r in range(R):
                    same(outs[r], want[r], f"allreduce rank {r}")
    for op in ("prod", "max", "min"):
        case("allreduce op", op)
        xs = [gen("fp32", 5000, 300 + r) for r in range(8)]
        want = oracle.allreduce(xs, "fp32", op)
        ins = [H.copy(x) for x in xs]
        outs = [H.poison(5000, np.float32) for _ in range(8)]
        ok(L.coll_allreduce(8, table(ins), table(outs), 5000, FP32, OPS[op], None), op)
        for r in range(8):
            same(outs[r], want[r], op)
    case("allreduce in place, R = 8 (staged through LDS)")
    xs = [gen("bf16", 12345, 40 + r) for r in range(8)]
    want = oracle.allreduce(xs, "bf16")
    bufs = [H.copy(x) for x in xs]
    ok(L.coll_allreduce(8, table(bufs), table(bufs), 12345, BF16, 0, None), "in place")
    for r in range(8):
        same(bufs[r], want[r], "in place")
    for R, n in ((3, 9), (8, 1000), (5, 4099), (16, 64)):
        for dtype in ("bf16", "fp32"):
            case("reduce_scatter", dtype, R, n)
            xs = [gen(dtype, R * n, 90 + r) for r in range(R)]
            want = oracle.reduce_scatter(xs, dtype)
            ins = [H.copy(x) for x in xs]
            outs = [H.poison(n, NP[dtype]) for _ in range(R)]
            ok(L.coll_reduce_scatter(R, table(ins), table(outs), n, DT[dtype], 0, None), "rs")
            for r in range(R):
                same(outs[r], want[r], f"reduce_scatter rank {r}")
            case("reduce", dtype, R, n)
            want = oracle.reduce(xs, R - 1, dtype)
            out = H.poison(R * n, NP[dtype])
            ok(L.coll_reduce(R, table(ins), ptr(out), R - 1, R * n, DT[dtype], 0, None), "reduce")
            same(out, want, "reduce")


def fam_copy():
    for R, n in ((1, 7), (3, 1000), (8, 4100), (8, 8 * 1025 + 3)):
        case("all_gather", R, n)
        xs = [gen("bf16", n, 200 + r) for r in range(R)]
        want = oracle.all_gather(xs)
        ins = [H.copy(x) for x in xs]
        outs = [H.poison(R * n, np.uint16) for _ in range(R)]
        ok(L.coll_all_gather(R, table(ins), table(outs), n, BF16, None), "ag")
        for r in range(R):
            same(outs[r], want[r], "all_gather")
        case("broadcast", R, n)
        root = R - 1
        src = H.copy(xs[0])
        outs = [H.poison(n, np.uint16) for _ in range(R)]
        outs[root] = src
        ok(L.coll_broadcast(R, ptr(src), table(outs), root, n, BF16, None), "bcast")
        for r in range(R):
            same(outs[r], xs[0], "broadcast")
        case("scatter", R, n)
        big = gen("bf16", R * n, 77)
        src = H.copy(big)
        outs = [H.poison(n, np.uint16) for _ in range(R)]
        ok(L.coll_scatter(R, ptr(src), table(outs), 0, n, BF16, None), "scatter")
        for r, w in enumerate(oracle.scatter(big, R, 0)):
            same(outs[r], w, "scatter")
    for R, outer, inner in ((8, 3, 19), (8, 16, 400), (4, 1, 4099), (3, 5, 8)):
        for dtype in ("fp32", "bf16"):
            case("gather", R, outer, inner, dtype)
            xs = [gen(dtype, outer * inner, 400 + r).reshape(outer, inner) for r in range(R)]
            want = oracle.gather(xs, 0)
            ins = [H.copy(x) for x in xs]
            out = H.poison((outer, R * inner), NP[dtype])
            ok(L.coll_gather(R, table(ins), ptr(out), 0, outer, inner, DT[dtype], None), "gather")
            same(out, want, "gather")


def _a2av_case(R, counts, W, dtype, cap=None, ws=False, gap=0):
    counts = np.asarray(counts, np.int64)
    sd, rd = oracle.packed_displs(counts)
    if gap:
        sd = sd + gap * np.arange(R)[None, :]          # a hole between blocks
        rd = rd + gap * np.arange(R)[None, :]
    send_rows = [int((sd[s] + counts[s]).max(initial=0)) for s in range(R)]
    recv_rows = [int((rd[d] + counts[:, d]).max(initial=0)) for d in range(R)]
    sends = [gen(dtype, send_rows[s] * W, 600 + s) for s in range(R)]
    want = oracle.all_to_all_v([s.reshape(-1) for s in sends], counts, sd, rd,
                               np.array(recv_rows), W)
    ins = [H.copy(s) if s.size else None for s in sends]
    outs = [H.poison(recv_rows[d] * W, NP[dtype]) if recv_rows[d] else None for d in range(R)]
    tabs = [H.copy(np.ascontiguousarray(t).reshape(-1)) for t in (counts, sd, rd)]
    capacity = sum(recv_rows) if cap is None else cap
    es = np.dtype(NP[dtype]).itemsize
    dt = BF16 if es == 2 else FP32
    if ws:
        need = L.coll_all_to_all_v_workspace_bytes(R, capacity, W, dt)
        work = H.poison(max(need, 256), np.uint8) if need else None
        ok(L.coll_all_to_all_v_ws(R, table(ins), ptr(tabs[0]), ptr(tabs[1]), table(outs),
                                  ptr(tabs[2]), W, dt, capacity, rows(send_rows),
                                  rows(recv_rows), ptr(work), need, None), "a2av_ws")
    else:
        ok(L.coll_all_to_all_v(R, table(ins), ptr(tabs[0]), ptr(tabs[1]), table(outs),
                               ptr(tabs[2]), W, dt, capacity, rows(send_rows), rows(recv_rows),
                               None), "a2av")
    for d in range(R):
        if recv_rows[d]:
            # rows in the gaps are not written: compare the blocks only
            for s in range(R):
                a, c = int(rd[d, s]) * W, int(counts[s, d]) * W
                same(outs[d][a:a + c], want[d][a:a + c], f"a2av block {s}->{d}")
    # the reverse from the same tables restores every block of the send buffers
    backs = [H.poison(send_rows[s] * W, NP[dtype]) if send_rows[s] else None for s in range(R)]
    bcap = sum(send_rows) if cap is None else cap
    work = None
    need = 0
    if ws:
        need = L.coll_all_to_all_v_workspace_bytes(R, bcap, W, dt)
        work = H.poison(max(need, 256), np.uint8) if need else None
    ok(L.coll_all_to_all_v_reverse(R, table(outs), ptr(tabs[0]), ptr(tabs[1]), table(backs),
                                   ptr(tabs[2]), W, dt, bcap, rows(send_rows), rows(recv_rows),
                                   ptr(work), need, None), "reverse")
    for s in range(R):
        for d in range(R):
            a, c = int(sd[s, d]) * W, int(counts[s, d]) * W
            if c:
                same(backs[s][a:a + c], sends[s].reshape(-1)[a:a + c], f"reverse block {d}->{s}")
    return sends, counts, sd, rd, outs


POISON = 0xAB


def _a2av_split_case(R, W, g):
    """coll_all_to_all_v_ws_build + _copy (and the reverse build + copy) give
    the same bytes as the one-call descriptor form."""
    counts = g.integers(0, 60, size=(R, R)).astype(np.int64)
    sd, rd = oracle.packed_displs(counts)
    send_rows = [int(counts[s].sum()) for s in range(R)]
    recv_rows = [int(counts[:, d].sum()) for d in range(R)]
    sends = [gen("bf16", send_rows[s] * W, 950 + s) for s in range(R)]
    want = oracle.all_to_all_v([x.reshape(-1) for x in sends], counts, sd, rd,
                               np.array(recv_rows), W)
    ins = [H.copy(x) if x.size else None for x in sends]
    outs = [H.poison(recv_rows[d] * W, np.uint16) if recv_rows[d] else None for d in range(R)]
    tabs = [H.copy(np.ascontiguousarray(t).reshape(-1)) for t in (counts, sd, rd)]
    cap = sum(recv_rows)
    need = L.coll_all_to_all_v_workspace_bytes(R, cap, W, BF16)
    assert need > 0
    work = H.poison(need, np.uint8)
    ok(L.coll_all_to_all_v_ws_build(R, table(ins), ptr(tabs[0]), ptr(tabs[1]), table(outs),
                                    ptr(tabs[2]), W, BF16, cap, rows(send_rows), rows(recv_rows),
                                    ptr(work), need, None), "build")
    ok(L.coll_all_to_all_v_ws_copy(R, W, BF16, cap, ptr(work), need, None), "copy")
    for d in range(R):
        if recv_rows[d]:
            same(outs[d], want[d].reshape(-1)[:recv_rows[d] * W], f"split form, rank {d}")
    backs = [H.poison(send_rows[s] * W, np.uint16) if send_rows[s] else None for s in range(R)]
    bcap = sum(send_rows)
    bneed = L.coll_all_to_all_v_workspace_bytes(R, bcap, W, BF16)
    bwork = H.poison(bneed, np.uint8)
    ok(L.coll_all_to_all_v_reverse_build(R, table(outs), ptr(tabs[0]), ptr(tabs[1]), table(backs),
                                         ptr(tabs[2]), W, BF16, bcap, rows(send_rows),
                                         rows(recv_rows), ptr(bwork), bneed, None), "reverse build")
    ok(L.coll_all_to_all_v_ws_copy(R, W, BF16, bcap, ptr(bwork), bneed, None), "reverse copy")
    for s in range(R):
        if send_rows[s]:
            same(backs[s], sends[s].reshape(-1), f"split reverse, rank {s}")


def _a2av_bad_case(R, W, ws):
    """Tables that name rows outside the buffers: each bad block moves nothing
    (its receive rows keep their contents), every other block is exact, and
    the guard pages show that nothing outside the buffers is touched.  The
    reverse call on the same tables skips the same blocks."""
    g = np.random.default_rng(77 + R + W)
    counts = g.integers(1, 30, size=(R, R)).astype(np.int64)
    sd, rd = oracle.packed_displs(counts)
    send_rows = [int(counts[s].sum()) for s in range(R)]
    recv_rows = [int(counts[:, d].sum()) for d in range(R)]
    bad_c, bad_sd, bad_rd = counts.copy(), sd.copy(), rd.copy()
    bad = set()
    # a count that runs past the receive buffer; a negative send displacement;
    # a receive displacement whose block ends one row past the buffer; a count
    # that runs past the send buffer; a negative count (a block of nothing)
    picks = [(0, R - 1), (R - 1, 0), (R // 2, R // 2), (1 % R, (R - 2) % R), (R - 1, R - 1)]
    for i, (s, d) in enumerate(picks):
        if (s, d) in bad:
            continue
        if i == 0:
            bad_c[s, d] = counts[s, d] + recv_rows[d]
        elif i == 1:
            bad_sd[s, d] = -3
        elif i == 2:
            bad_rd[d, s] = recv_rows[d] - counts[s, d] + 1
        elif i == 3:
            bad_c[s, d] = send_rows[s] + 1
        else:
            bad_c[s, d] = -5
        bad.add((s, d))
    sends = [gen("bf16", send_rows[s] * W, 900 + s) for s in range(R)]
    eff = counts.copy()
    for s, d in bad:
        eff[s, d] = 0
    want = oracle.all_to_all_v([x.reshape(-1) for x in sends], eff, sd, rd, np.array(recv_rows), W)
    ins = [H.copy(x) for x in sends]
    outs = [H.poison(recv_rows[d] * W, np.uint16) for d in range(R)]
    tabs = [H.copy(np.ascontiguousarray(t).reshape(-1)) for t in (bad_c, bad_sd, bad_rd)]
    cap = sum(recv_rows)
    work, need = None, 0
    if ws:
        need = L.coll_all_to_all_v_workspace_bytes(R, cap, W, BF16)
        work = H.poison(max(need, 256), np.uint8) if need else None
        ok(L.coll_all_to_all_v_ws(R, table(ins), ptr(tabs[0]), ptr(tabs[1]), table(outs),
                                  ptr(tabs[2]), W, BF16, cap, rows(send_rows), rows(recv_rows),
                                  ptr(work), need, None), "a2av_ws bad tables")
    else:
        ok(L.coll_all_to_all_v(R, table(ins), ptr(tabs[0]), ptr(tabs[1]), table(outs),
                               ptr(tabs[2]), W, BF16, cap, rows(send_rows), rows(recv_rows), None),
           "a2av bad tables")
    for s in range(R):
        for d in range(R):
            a, c = int(rd[d, s]) * W, int(counts[s, d]) * W
            if (s, d) in bad:
                assert np.all(outs[d][a:a + c].view(np.uint8) == POISON), f"bad block {s}->{d} written"
            else:
                same(outs[d][a:a + c], want[d][a:a + c], f"good block {s}->{d}")
    backs = [H.poison(send_rows[s] * W, np.uint16) for s in range(R)]
    ok(L.coll_all_to_all_v_reverse(R, table(outs), ptr(tabs[0]), ptr(tabs[1]), table(backs),
                                   ptr(tabs[2]), W, BF16, sum(send_rows), rows(send_rows),
                                   rows(recv_rows), ptr(work), need, None), "reverse bad tables")
    for s in range(R):
        for d in range(R):
            a, c = int(sd[s, d]) * W, int(counts[s, d]) * W
            if (s, d) in bad:
                assert np.all(backs[s][a:a + c].view(np.uint8) == POISON), f"bad block {d}->{s} back"
            else:
                same(backs[s][a:a + c], sends[s].reshape(-1)[a:a + c], f"good block back {d}->{s}")


def _expert_bad_block(R, E, Hd, recvs, lay, want, rrows):
    """The test expert on tables with one bad (d, s) block -- a negative
    expert count, or a receive displacement that runs past recv[d]: that
    block's rows keep their values, every other row is scaled exactly, on
    the row-descriptor path (in one call and in two) and the table search."""
    per = E // R
    ec_h = np.array(lay["expert_counts"], np.int32).reshape(R, E)
    rd_h = np.array(lay["rdispls"], np.int64)
    blocks = [(s, d) for s in range(R) for d in range(R)
              if ec_h[s, d * per:(d + 1) * per].sum() > 0]
    s0, d0 = blocks[len(blocks) // 2]
    n0 = int(ec_h[s0, d0 * per:(d0 + 1) * per].sum())
    for kind in ("negative count", "displacement past the buffer"):
        ec2, rd2 = ec_h.copy(), rd_h.copy()
        if kind == "negative count":
            ec2[s0, d0 * per] = -1
        else:
            rd2[d0, s0] = int(rrows[d0]) - n0 + 1
        # the row-descriptor path (capacity known), the table search (0), and
        # the row-descriptor path in two calls where it applies
        forms = [(int(rrows.sum()), False), (0, False)]
        if Hd % 8 == 0 and R * E <= 8192:
            forms.append((int(rrows.sum()), True))
        for cap, split in forms:
            case("expert with a bad block", kind, "cap", cap, "two calls" if split else "")
            ys = [H.copy(r) if r is not None else None for r in recvs]
            ec_b = H.copy(np.ascontiguousarray(ec2).reshape(-1))
            rd_b = H.copy(np.ascontiguousarray(rd2).reshape(-1))
            need = L.coll_moe_expert_workspace_bytes(R, E, cap)
            ews = H.poison(need, np.uint8)
            if split:                                   # the two-call form of that path
                ok(L.coll_moe_expert_scale_build(R, table(ys), ptr(ec_b), ptr(rd_b), E, Hd, BF16,
                                                 cap, rows(rrows), ptr(ews), need, None),
                   "expert build, bad block")
                ok(L.coll_moe_expert_scale_apply(R, table(ys), E, Hd, BF16, cap, ptr(ews), need,
                                                 None), "expert apply, bad block")
            else:
                ok(L.coll_moe_expert_scale(R, table(ys), ptr(ec_b), ptr(rd_b), E, Hd, BF16, cap,
                                           rows(rrows), ptr(ews), need, None), "expert, bad block")
            for d in range(R):
                if not rrows[d]:
                    continue
                exp = want["ys"][d].reshape(-1, Hd)[:int(rrows[d])].copy()
                if d == d0:
                    a = int(rd_h[d0, s0])
                    exp[a:a + n0] = recvs[d0][a:a + n0]
                same(ys[d], exp, f"expert with a bad block ({kind}), rank {d}")


def _moe_fused_bad_block(R, T, K, Hd, lay, x_b, pos, w_b, id_b, want, rrows):
    """The fused pair with one block's receive displacement past its buffer:
    that block's rows are neither written by the dispatch nor read by the
    combine (its pairs add no term); everything else is exact."""
    sc_h, sd_h, rd_h = (np.array(lay[k], np.int64) for k in ("sendcounts", "sdispls", "rdispls"))
    cand = [(s, d) for s in range(R) for d in range(R) if sc_h[s, d] > 0]
    s0, d0 = cand[len(cand) // 2]
    bad_rd = rd_h.copy()
    bad_rd[d0, s0] = int(rrows[d0]) - int(sc_h[s0, d0]) + 1
    sc, sd, rd = (H.copy(np.ascontiguousarray(t).reshape(-1)) for t in (sc_h, sd_h, bad_rd))
    recv = [H.poison((int(n), Hd), np.uint16) if n else None for n in rrows]
    ok(L.coll_moe_dispatch(R, table(x_b), table(pos), ptr(sc), ptr(sd), ptr(rd), T, K, Hd, BF16,
                           table(recv), rows(rrows), None), "dispatch, bad block")
    for d in range(R):
        for s in range(R):
            a, c = int(rd_h[d, s]), int(sc_h[s, d])
            if not c:
                continue
            got = recv[d][a:a + c]
            if (s, d) == (s0, d0):
                assert np.all(got.view(np.uint8) == POISON), "bad block written by the dispatch"
            else:
                same(got, want["recvs"][d].reshape(-1, Hd)[a:a + c], f"dispatch block {s}->{d}")
    # the combine: pairs whose slot lies in the bad block are dropped
    lo, hi = int(sd_h[s0, d0]), int(sd_h[s0, d0] + sc_h[s0, d0])
    pos_eff = [np.array(lay["pos"][s]) for s in range(R)]
    m = (pos_eff[s0] >= lo) & (pos_eff[s0] < hi)
    pos_eff[s0] = np.where(m, -1, pos_eff[s0]).astype(np.int32)
    good = [H.copy(np.asarray(r)) if r is not None else None for r in recv]
    for d in range(R):          # fill the bad block's rows with the correct data first: the
        if rrows[d]:            # combine must still skip them
            good[d][...] = want["recvs"][d].reshape(-1, Hd)[:int(rrows[d])]
    outs = [H.poison((T, Hd), np.uint16) for _ in range(R)]
    ok(L.coll_moe_combine_recv(R, table(good), table(pos), ptr(sc), ptr(sd), ptr(rd), table(w_b),
                               table(id_b), T, K, Hd, BF16, table(outs), rows(rrows), None),
       "combine_recv, bad block")
    expect = oracle.moe_combine([np.asarray(b) for b in want["backs"]], pos_eff,
                                [np.asarray(w) for w in w_b], Hd)
    for s in range(R):
        same(outs[s], expect[s], f"fused combine with a bad block, rank {s}")


def fam_a2av():
    g = np.random.default_rng(5)
    for R in (1, 2, 3, 8, 16):
        for W in (1, 3, 8, 24):
            case("a2av random", R, W)
            _a2av_case(R, g.integers(0, 40, size=(R, R)), W, "bf16")
    case("a2av empty blocks and an empty rank")
    c = g.integers(0, 30, size=(4, 4))
    c[:, 2] = 0
    c[1, :] = 0
    _a2av_case(4, c, 8, "bf16")
    case("a2av gapped")
    _a2av_case(3, g.integers(1, 20, size=(3, 3)), 8, "bf16", gap=5)
    case("a2av odd-byte rows (chunk kernel)")
    _a2av_case(4, g.integers(0, 50, size=(4, 4)), 5, "bf16")
    case("a2av capacity 0 (resident grid)")
    _a2av_case(3, g.integers(0, 50, size=(3, 3)), 8, "bf16", cap=0)
    case("a2av capacity below the rows received")
    _a2av_case(3, g.integers(20, 50, size=(3, 3)), 8, "bf16", cap=10)
    # the descriptor form (COLL_A2A_DESC_MIN_BYTES=0 in this process)
    for R, W in ((8, 8), (3, 24), (2, 8), (8, 7168 // 64), (16, 8), (1, 16)):
        case("a2av descriptor form", R, W)
        _a2av_case(R, g.integers(0, 60, size=(R, R)), W, "bf16", ws=True)
    case("a2av descriptor form, capacity below the rows (tail loop)")
    _a2av_case(4, g.integers(30, 60, size=(4, 4)), 8, "bf16", ws=True, cap=50)
    for R, W in ((8, 8), (3, 24), (16, 8), (1, 16)):
        case("a2av descriptor form in two calls (build, then copy)", R, W)
        _a2av_split_case(R, W, g)
    case("a2av descriptor form, gapped")
    _a2av_case(3, g.integers(1, 30, size=(3, 3)), 16, "bf16", ws=True, gap=7)
    # blocks much longer than a wave, so that waves locate their units from
    # the block ends held in registers (at most 64 blocks) and only waves that
    # straddle a boundary search: resident grid (capacity 0) and one-pass grid
    for R, W, lo, hi in ((8, 8, 200, 400), (8, 1, 1600, 3200), (4, 8, 100, 300),
                         (2, 24, 50, 90), (16, 8, 70, 150)):
        for cap in (0, None):
            case("a2av long blocks", R, W, "cap", cap)
            _a2av_case(R, g.integers(lo, hi, size=(R, R)), W, "bf16", cap=cap)
    case("a2av long uniform blocks of one-bf16 rows (the aligned chunk path)")
    _a2av_case(8, np.full((8, 8), 2048), 1, "bf16", cap=0)
    # 257 chunks per block: whole tiles, then one that reaches the total
    case("a2av aligned chunk path with a last partial tile")
    _a2av_case(8, np.full((8, 8), 2056), 1, "bf16", cap=0)
    _a2av_case(3, np.full((3, 3), 1000), 1, "bf16", cap=0)
    # small enough for the resident grid: 63 chunks per block, 7 whole tiles
    # and a partial one
    for cap in (0, None):
        _a2av_case(8, np.full((8, 8), 504), 1, "bf16", cap=cap)
    for R, W in ((8, 8), (4, 5), (3, 24), (16, 8), (8, 64), (16, 64)):
        for ws in (False, True):
            case("a2av tables that name rows outside the buffers", R, W, "ws" if ws else "plain")
            _a2av_bad_case(R, W, ws)


def fam_exchange():
    for R, n in ((1, 5), (3, 100), (8, 1000), (8, 8 * 1024 + 8)):
        case("all_to_all", R, n)
        xs = [gen("bf16", R * n, 800 + r) for r in range(R)]
        want = oracle.all_to_all(xs)
        ins = [H.copy(x) for x in xs]
        outs = [H.poison(R * n, np.uint16) for _ in range(R)]
        ok(L.coll_all_to_all(R, table(ins), table(outs), n, BF16, None), "a2a")
        for r in range(R):
            same(outs[r], want[r], "all_to_all")
    for R, SL, Hh, D in ((2, 3, 4, 8), (4, 5, 8, 16), (8, 7, 16, 128), (3, 4, 6, 5)):
        for to_heads in (True, False):
            case("reshard", R, SL, Hh, D, to_heads)
            xs = [gen("bf16", SL * Hh * D, 900 + r) for r in range(R)]
            want = oracle.ulysses(xs, SL, Hh, D, to_heads)
            ins = [H.copy(x) for x in xs]
            outs = [H.poison(SL * Hh * D, np.uint16) for _ in range(R)]
            ok(L.coll_seq_heads_reshard(R, table(ins), table(outs), SL, Hh, D, BF16,
                                        1 if to_heads else 0, None), "reshard")
            for r in range(R):
                same(outs[r], want[r], "reshard")


def fam_merge():
    g = np.random.default_rng(9)
    # whole rows per wave (at most 64 units) and segments of longer rows,
    # vector and scalar forms, ragged last workgroups
    for R, rows, D, dtype in ((1, 10, 128, "bf16"), (2, 37, 64, "fp32"), (8, 300, 128, "bf16"),
                              (4, 10, 5, "bf16"), (16, 30, 16, "fp32"), (3, 9, 1000, "bf16"),
                              (8, 5, 520, "fp32"), (4, 1000, 8, "bf16"), (8, 77, 256, "bf16"),
                              (5, 63, 64, "fp32"), (16, 200, 512, "bf16"), (6, 3, 8, "fp32")):
        case("lse_merge", R, rows, D, dtype)
        o = [gen(dtype, rows * D, 1000 + r) for r in range(R)]
        lse = [(g.normal(size=rows) * 3).astype(np.float32) for _ in range(R)]
        lse[0][:2] = -np.inf                           # rank 0 empty on two rows
        if rows > 3:
            for l in lse:
                l[3] = -np.inf                         # a row with no keys anywhere
        want_o, want_l = oracle.lse_merge(o, lse, dtype)
        ins = [H.copy(x) for x in o]
        lin = [H.copy(x) for x in lse]
        outs = [H.poison(rows * D, NP[dtype]) for _ in range(R)]
        lout = [H.poison(rows, np.float32) for _ in range(R)]
        lout[R - 1] = None                              # a NULL entry: not written
        ok(L.coll_lse_merge(R, table(ins), table(lin), table(outs), table(lout), rows, D,
                            DT[dtype], None), "lse_merge")
        f = (lambda a: oracle.bf16_to_f32(a).astype(np.float64)) if dtype == "bf16" else \
            (lambda a: a.astype(np.float64))
        ulp = 2.0 ** (-7 if dtype == "bf16" else -23)
        for r in range(R):
            got, exp = f(outs[r]), f(want_o)
            mag = np.max(np.abs(exp)) if exp.size else 0
            if not np.all(np.abs(got - exp) <= 2 * ulp * np.abs(exp) + 1e-5 * (mag + 1)):
                raise AssertionError(f"lse_merge o rank {r}")
            if lout[r] is not None and not np.allclose(lout[r], want_l, rtol=1e-5, atol=1e-5,
                                                       equal_nan=True):
                raise AssertionError(f"lse_merge L rank {r}")
        if rows > 3:
            for r in range(R):
                if np.any(f(outs[r]).reshape(rows, D)[3] != 0):
                    raise AssertionError("all-empty row not zero")
    case("lse_merge in place, R = 8")
    R, rows, D = 8, 130, 128
    o = [gen("bf16", rows * D, 1100 + r) for r in range(R)]
    lse = [(g.normal(size=rows) * 3).astype(np.float32) for _ in range(R)]
    want_o, want_l = oracle.lse_merge(o, lse, "bf16")
    bufs = [H.copy(x) for x in o]
    lin = [H.copy(x) for x in lse]
    lout = [H.poison(rows, np.float32) for _ in range(R)]
    ok(L.coll_lse_merge(R, table(bufs), table(lin), table(bufs), table(lout), rows, D, BF16,
                        None), "lse_merge in place")
    exp = oracle.bf16_to_f32(want_o).astype(np.float64)
    for r in range(R):
        got = oracle.bf16_to_f32(bufs[r]).astype(np.float64)
        if not np.all(np.abs(got - exp) <= 2 * 2.0 ** -7 * np.abs(exp) + 1e-5 * (np.max(np.abs(exp)) + 1)):
            raise AssertionError(f"lse_merge in place rank {r}")
        if not np.allclose(lout[r], want_l, rtol=1e-5, atol=1e-5):
            raise AssertionError(f"lse_merge in place L rank {r}")


def _moe(R, E, T, K, Hd, bad=False, seed=5100):
    ids, ws, xs = [], [], []
    for s in range(R):
        i, w = synth.zipf_routing(T, E, K, seed=seed + s)
        ids.append(i)
        ws.append(w)
        xs.append(synth.gaussian((T, Hd), 1.0, seed + 100 + s, "bf16"))
    if bad:
        gb = np.random.default_rng(seed)
        for i in ids:
            m = gb.random(i.shape) < 0.1
            i[m] = gb.choice(np.array([-1, E, 1 << 30], np.int32), size=int(m.sum()))
            if T > 1:
                i[1, :] = E
    return ids, ws, xs


def _layout(R, E, T, K, ids):
    id_b = [H.copy(i) for i in ids]
    sc, sd, rd = (H.poison(R * R, np.int64) for _ in range(3))
    ec = H.poison(R * E, np.int32)
    pos = [H.poison((T, K), np.int32) for _ in range(R)]
    need = L.coll_moe_workspace_bytes(R, T, K, E)
    work = H.poison(max(need, 256), np.uint8)
    ok(L.coll_moe_layout(R, table(id_b), T, K, E, ptr(sc), ptr(sd), ptr(rd), ptr(ec),
                         table(pos), ptr(work), need, None), "layout")
    return id_b, sc, sd, rd, ec, pos


def fam_moe():
    for R, E, T, K, Hd, bad in ((2, 4, 2, 1, 8, False), (1, 8, 100, 2, 16, False),
                                (4, 16, 333, 3, 24, False), (8, 256, 150, 8, 64, False),
                                (2, 8, 50, 2, 5, False), (16, 1024, 40, 8, 8, False),
                                (2, 16, 40, 10, 16, False), (4, 16, 200, 3, 24, True),
                                (8, 64, 100, 8, 8, True), (2, 16, 40, 10, 5, True),
                                # top-17 (a second chunk of slots in the combines);
                                # rows of 1025 units (a ragged last segment)
                                (2, 32, 30, 17, 16, False), (2, 8, 6, 2, 8200, False)):
        case("moe", R, E, T, K, Hd, "bad ids" if bad else "")
        ids, ws, xs = _moe(R, E, T, K, Hd, bad)
        want = oracle.moe_pipeline(xs, ids, ws, E)
        lay = want["layout"]
        id_b, sc, sd, rd, ec, pos = _layout(R, E, T, K, ids)
        for key, got in (("sendcounts", sc), ("sdispls", sd), ("rdispls", rd),
                         ("expert_counts", ec)):
            same(got.reshape(lay[key].shape), lay[key], key)
        for s in range(R):
            same(pos[s], lay["pos"][s], "pos")
        # the layout without a workspace (the library's static scratch)
        tabs2 = [H.poison(R * R, np.int64) for _ in range(3)] + [H.poison(R * E, np.int32)]
        pos2 = [H.poison((T, K), np.int32) for _ in range(R)]
        ok(L.coll_moe_layout_noalloc(R, table(id_b), T, K, E, *[ptr(t) for t in tabs2],
                                     table(pos2), None), "layout_noalloc")
        for a, b in zip(tabs2, (sc, sd, rd, ec)):
            same(a, b, "layout_noalloc tables")
        for s in range(R):
            same(pos2[s], pos[s], "layout_noalloc pos")
        x_b = [H.copy(x) for x in xs]
        w_b = [H.copy(w) for w in ws]
        sends = [H.poison((T * K, Hd), np.uint16) for _ in range(R)]
        ok(L.coll_moe_permute(R, table(x_b), table(pos), T, K, Hd, BF16, table(sends), None),
           "permute")
        nsend = [int(lay["sendcounts"][s].sum()) for s in range(R)]
        for s in range(R):
            same(sends[s][:nsend[s]], want["sends"][s][:nsend[s]], "permute")
        rrows = lay["sendcounts"].sum(axis=0)
        recvs = [H.poison((int(n), Hd), np.uint16) if n else None for n in rrows]
        ok(L.coll_all_to_all_v(R, table(sends), ptr(sc), ptr(sd), table(recvs), ptr(rd), Hd,
                               BF16, int(rrows.sum()), rows([T * K] * R), rows(rrows), None),
           "a2av")
        for d in range(R):
            if rrows[d]:
                same(recvs[d].reshape(-1), want["recvs"][d].reshape(-1)[:int(rrows[d]) * Hd], "recv")
        for cap in (int(rrows.sum()), 0):
            # the row-descriptor path (capacity known) and the table search (0)
            ys = [H.copy(r) if r is not None else None for r in recvs]
            need = L.coll_moe_expert_workspace_bytes(R, E, cap)
            ews = H.poison(need, np.uint8)
            ok(L.coll_moe_expert_scale(R, table(ys), ptr(ec), ptr(rd), E, Hd, BF16, cap,
                                       rows(rrows), ptr(ews),
                                       need, None), "expert")
            for d in range(R):
                if rrows[d]:
                    same(ys[d].reshape(-1), want["ys"][d].reshape(-1)[:int(rrows[d]) * Hd],
                         f"expert cap {cap}")
        if Hd % 8 == 0 and R * E <= 8192:
            # the row-descriptor path in two calls: build, then apply
            case("expert in two calls (build, then apply)")
            ys2 = [H.copy(r) if r is not None else None for r in recvs]
            cap = int(rrows.sum())
            need = L.coll_moe_expert_workspace_bytes(R, E, cap)
            ews = H.poison(need, np.uint8)
            ok(L.coll_moe_expert_scale_build(R, table(ys2), ptr(ec), ptr(rd), E, Hd, BF16, cap,
                                             rows(rrows), ptr(ews), need, None), "expert build")
            ok(L.coll_moe_expert_scale_apply(R, table(ys2), E, Hd, BF16, cap, ptr(ews), need,
                                             None), "expert apply")
            for d in range(R):
                if rrows[d]:
                    same(ys2[d].reshape(-1), want["ys"][d].reshape(-1)[:int(rrows[d]) * Hd],
                         "expert in two calls")
        _expert_bad_block(R, E, Hd, recvs, lay, want, rrows)
        backs = [H.poison((T * K, Hd), np.uint16) for _ in range(R)]
        sc_t = H.copy(np.ascontiguousarray(lay["sendcounts"].T).reshape(-1))
        ok(L.coll_all_to_all_v(R, table(ys), ptr(sc_t), ptr(rd), table(backs), ptr(sd), Hd,
                               BF16, T * K * R, rows(rrows), rows([T * K] * R), None),
           "a2av back")
        for s in range(R):
            same(backs[s].reshape(-1)[:nsend[s] * Hd],
                 want["backs"][s].reshape(-1)[:nsend[s] * Hd], "back")
        # the same return through the reverse call on the forward tables, plain
        # and with a workspace (the descriptor form in this process)
        for use_ws in (False, True):
            backs2 = [H.poison((T * K, Hd), np.uint16) for _ in range(R)]
            need = L.coll_all_to_all_v_workspace_bytes(R, T * K * R, Hd, BF16) if use_ws else 0
            work = H.poison(max(need, 256), np.uint8) if need else None
            ok(L.coll_all_to_all_v_reverse(R, table(ys), ptr(sc), ptr(sd), table(backs2), ptr(rd),
                                           Hd, BF16, T * K * R, rows([T * K] * R), rows(rrows),
                                           ptr(work), need, None), "reverse")
            for s in range(R):
                same(backs2[s].reshape(-1)[:nsend[s] * Hd],
                     want["backs"][s].reshape(-1)[:nsend[s] * Hd], f"reverse ws={use_ws}")
        outs = [H.poison((T, Hd), np.uint16) for _ in range(R)]
        ok(L.coll_moe_combine(R, table(backs), table(pos), table(w_b), T, K, Hd, BF16,
                              table(outs), None), "combine")
        for s in range(R):
            same(outs[s], want["outs"][s], "combine")
        # the fused pair
        recv2 = [H.poison((int(n), Hd), np.uint16) if n else None for n in rrows]
        ok(L.coll_moe_dispatch(R, table(x_b), table(pos), ptr(sc), ptr(sd), ptr(rd), T, K, Hd,
                               BF16, table(recv2), rows(rrows), None), "dispatch")
        for d in range(R):
            if rrows[d]:
                same(recv2[d], recvs[d], "fused dispatch")
        outs2 = [H.poison((T, Hd), np.uint16) for _ in range(R)]
        ok(L.coll_moe_combine_recv(R, table(recv2), table(pos), ptr(sc), ptr(sd), ptr(rd),
                                   table(w_b), table(id_b), T, K, Hd, BF16, table(outs2),
                                   rows(rrows), None), "combine_recv")
        for s in range(R):
            same(outs2[s], want["outs"][s], "fused combine")
        _moe_fused_bad_block(R, T, K, Hd, lay, x_b, pos, w_b, id_b, want, rrows)


FAMILIES = {"reduce": fam_reduce, "copy": fam_copy, "a2av": fam_a2av, "exchange": fam_exchange,
            "merge": fam_merge, "moe": fam_moe}


def main():
    global H
    family, place = sys.argv[1], sys.argv[2]
    H = Heap(place)
    load()
    FAMILIES[family]()
    print("all cases passed", flush=True)


if __name__ == "__main__":
    main()
