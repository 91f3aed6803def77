#!/usr/bin/env python3
"""Benchmark of the collectives hot path on one MI355X.

One step is one pass of every hot-path row over one batch of synthetic,
HBM-resident input, R = 8 virtual ranks, bf16 unless noted:

  ar_160k      AllReduce, R=4, 160 KiB per rank (the four-segment A-D example)
  ar_decode    AllReduce, [64, 7168] per rank (TP decode)
  ar_64m       AllReduce, 64 MiB per rank
  rs_sp        ReduceScatter [8192, 4096] -> 1024-token shards
  ag_sp        AllGather of those shards back to [8192, 4096]
  gather       Gather fp32 logits [256, 19008] x 8 -> [256, 152064] on rank 0
  bcast        Broadcast int32 [256] from rank 7
  moe_layout   expert histogram / scans / stable slots, 4096 x top-8, 256 experts
  moe_permute  dispatch permute into per-destination send buffers
  a2av_dispatch  All-to-All-v of the dispatched rows (hidden 7168), with a
               workspace (the descriptor form)
  moe_expert   the test expert y = x * (1 + e/256) on received rows
  a2av_combine   the reverse All-to-All-v (rows back to their send slots), read
               from the dispatch's own tables, with a workspace
  moe_combine  gate-weighted top-8 sum back to each token

value = algorithmic bytes of the whole step / step time (GB/s).  Algorithmic
bytes are the minimum each row must read plus write (e.g. AllReduce 2*R*S,
All-to-All-v 2 * rows * row_bytes).  Per-row times come from HIP events on the
stream the kernels run on; the dominant kernel (a2av_dispatch) is reported
against the 8 TB/s HBM roofline.  Separate sweeps: AllReduce at 8 KiB .. 64 MiB
per rank and All-to-All-v (uniform and MoE-shaped, plain and with a
workspace), rotating four buffer sets
from 8 MiB up so the 256 MB Infinity Cache cannot serve the large sizes.

The CPU baseline times the oracle (single-threaded C) on whole passes of the
same step at its bench sizes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "AllReduce/A2A-v algorithmic GB/s at R=8 bf16; % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0
R = 8


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--only", default="", help="comma list of rows to run (profiling)")
    p.add_argument("--report", default="",
                   help="print the markdown tables of a saved JSON line (file) and exit")
    return p.parse_args()


# ------------------------------------------------------------------ inputs

def make_inputs(torch, synth, coll):
    import numpy as np

    def dev_bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    W = {}
    print("[bench] generating inputs", file=sys.stderr, flush=True)
    bf = torch.bfloat16
    # every group of rank buffers lives in a rank arena: the buffers one call
    # touches together start on their own 2 MiB pages at distinct 4 KiB colours
    W["ar160_in"], W["ar160_out"] = coll.rank_arena([(4, 81920, bf), (4, 81920, bf)])
    for r, t in enumerate(W["ar160_in"]):
        t.copy_(dev_bf16(synth.gaussian(81920, 1.0, 1000 + r, "bf16")))
    W["ard_in"], W["ard_out"] = coll.rank_arena([(R, (64, 7168), bf), (R, (64, 7168), bf)])
    for r, t in enumerate(W["ard_in"]):
        t.copy_(dev_bf16(synth.gaussian((64, 7168), 0.02, 2000 + r, "bf16")))
    n64 = (64 << 20) // 2
    g = torch.Generator(device="cuda")
    g.manual_seed(26)
    W["ar64_in"], W["ar64_out"] = coll.rank_arena([(R, n64, bf), (R, n64, bf)])
    for t in W["ar64_in"]:
        t.copy_(torch.randn(n64, generator=g, device="cuda") * 0.02)
    W["sp_in"], W["sp_shard"], W["sp_full"] = coll.rank_arena(
        [(R, (8192, 4096), bf), (R, (1024, 4096), bf), (R, (8192, 4096), bf)])
    for r, t in enumerate(W["sp_in"]):
        t.copy_(dev_bf16(synth.gaussian((8192, 4096), 1.0, 3000 + r, "bf16")))
    W["lg_in"], (W["lg_out"],) = coll.rank_arena(
        [(R, (256, 19008), torch.float32), (1, (256, R * 19008), torch.float32)])
    for r, t in enumerate(W["lg_in"]):
        t.copy_(torch.from_numpy(synth.gaussian((256, 19008), 2.0, 4000 + r, "fp32")))
    (W["bc_out"],) = coll.rank_arena([(R, 256, torch.int32)])
    W["bc_src"] = W["bc_out"][7]                 # the root keeps its own buffer
    W["bc_src"].copy_(torch.from_numpy(synth.uniform_int32(256, 0, 152064, 4107)))

    E, T, K, H = 256, 4096, 8, 7168
    W["moe"] = (E, T, K, H)
    ids, ws = [], []
    for s in range(R):
        i, w = synth.zipf_routing(T, E, K, seed=5100 + s)
        ids.append(torch.from_numpy(i).cuda())
        ws.append(torch.from_numpy(w).cuda())
    W["moe_ids"], W["moe_w"] = ids, ws
    W["sc"] = torch.empty(R * R, dtype=torch.int64, device="cuda")
    W["sd"] = torch.empty_like(W["sc"])
    W["rd"] = torch.empty_like(W["sc"])
    W["ec"] = torch.empty(R * E, dtype=torch.int32, device="cuda")
    W["pos"] = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in range(R)]
    W["ws"] = torch.empty(coll.moe_workspace_bytes(R, T, K, E), dtype=torch.uint8, device="cuda")
    # the routing is fixed, so the receive sizes are known once (outside timing)
    coll.moe_layout(ids, E, W["sc"], W["sd"], W["rd"], W["ec"], W["pos"], W["ws"])
    torch.cuda.synchronize()
    sc = W["sc"].view(R, R).cpu()
    W["moe_x"], W["send"], W["recv"], W["back"], W["out"] = coll.rank_arena(
        [(R, (T, H), bf), (R, (T * K, H), bf),
         [((int(sc[:, d].sum()), H), bf) for d in range(R)],
         (R, (T * K, H), bf), (R, (T, H), bf)])
    for s, t in enumerate(W["moe_x"]):
        t.copy_(dev_bf16(synth.gaussian((T, H), 1.0, 5000 + s, "bf16")))
    # the test expert's workspace: entry tables + one descriptor per receive row
    W["ews"] = torch.empty(coll.moe_expert_workspace_bytes(R, E, sum(t.shape[0] for t in W["recv"])),
                           dtype=torch.uint8, device="cuda")
    # workspaces of the two exchanges' descriptor form (block table + one
    # descriptor per 1 KiB tile of the receive capacity)
    W["a2a_ws_d"] = torch.empty(coll.all_to_all_v_workspace_bytes(W["send"], W["recv"], H),
                                dtype=torch.uint8, device="cuda")
    W["a2a_ws_c"] = torch.empty(coll.all_to_all_v_workspace_bytes(W["recv"], W["back"], H),
                                dtype=torch.uint8, device="cuda")
    # their first kernels (the descriptor builds) depend only on the layout's
    # tables and the buffers' addresses: the step issues them on a second
    # stream beside the permute.  Built once here too, so that a copy never
    # meets an unbuilt workspace (e.g. a profiling run of one row).
    W["build_d"] = coll.prepare(coll.all_to_all_v_build, W["send"], W["sc"], W["sd"], W["recv"],
                                W["rd"], H, W["a2a_ws_d"])
    W["build_c"] = coll.prepare(coll.all_to_all_v_reverse_build, W["recv"], W["sc"], W["sd"],
                                W["back"], W["rd"], H, W["a2a_ws_c"])
    # the test expert's row descriptors likewise depend only on the layout
    W["build_e"] = coll.prepare(coll.moe_expert_scale_build, W["recv"], W["ec"], W["rd"], E, H,
                                W["ews"])
    W["build_d"](), W["build_c"](), W["build_e"]()
    torch.cuda.synchronize()
    W["side"] = torch.cuda.Stream()          # default priority
    W["built"] = [None]
    W["laid_out"] = None
    # events of the fork and join, made once: creating them every step cost
    # host time while the GPU waited
    W["ev_laid_out"], W["ev_built"] = torch.cuda.Event(), torch.cuda.Event()
    # plain-copy reference (1 GiB through the library's copy kernel), only for
    # calibrating the HBM counters; not part of the step
    W["copy_src"] = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").normal_()
    W["copy_dst"] = [torch.empty_like(W["copy_src"])]
    W["moe_rows"] = int(sc.sum())
    W["dest_share"] = [round(float(sc[:, d].sum()) / float(sc.sum()), 4) for d in range(R)]
    torch.cuda.synchronize()
    return W


def row_bytes(W):
    """Algorithmic HBM bytes of every row (minimum read + write)."""
    E, T, K, H = W["moe"]
    rows = W["moe_rows"]
    b = {}
    b["ar_160k"] = 2 * 4 * 81920 * 2
    b["ar_decode"] = 2 * R * 64 * 7168 * 2
    b["ar_64m"] = 2 * R * (64 << 20)
    S = 8192 * 4096 * 2
    b["rs_sp"] = (R + 1) * S
    b["ag_sp"] = S + R * S
    b["gather"] = 2 * R * 256 * 19008 * 4
    b["bcast"] = 256 * 4 * R                          # 1 read + 7 writes (root keeps its own)
    b["moe_layout"] = 2 * R * T * K * 4
    b["moe_permute"] = R * T * H * 2 + rows * H * 2 + R * T * K * 4
    b["a2av_dispatch"] = 2 * rows * H * 2
    b["moe_expert"] = 2 * rows * H * 2
    b["a2av_combine"] = 2 * rows * H * 2
    b["moe_combine"] = rows * H * 2 + R * T * H * 2 + R * T * K * 8
    b["copy_ref"] = 2 << 30
    b["moe_dispatch_fused"] = R * T * H * 2 + rows * H * 2 + R * T * K * 4
    b["moe_combine_fused"] = rows * H * 2 + R * T * H * 2 + R * T * K * 12
    return b


def _composite(fn):
    """Mark a row that is already a sequence of prepared calls (it is not
    passed through coll.prepare)."""
    fn.composite = True
    return fn


def step_rows(W, coll, torch):
    """(name, callable) for every row of one step, in order.  The two
    All-to-All-v rows run the descriptor form's copy kernel and the expert row
    its scaling kernel; their descriptor builds wait only for the layout and
    run on a second stream beside the permute, and the dispatch row waits for
    them."""
    E, T, K, H = W["moe"]
    layout = coll.prepare(coll.moe_layout, W["moe_ids"], E, W["sc"], W["sd"], W["rd"], W["ec"],
                          W["pos"], W["ws"])
    copy_d = coll.prepare(coll.all_to_all_v_copy, W["send"], W["recv"], H, W["a2a_ws_d"])

    permute = coll.prepare(coll.moe_permute, W["moe_x"], W["pos"], W["send"])

    @_composite
    def layout_then_mark():
        layout()
        W["ev_laid_out"].record()            # the layout's tables are ready from here
        W["laid_out"] = W["ev_laid_out"]

    @_composite
    def permute_then_builds():
        # the permute is launched first: the host work of the fork below then
        # overlaps it on the GPU, and the builds wait only for the layout
        permute()
        if W["laid_out"] is None:            # no layout row ran (a profiling run of some rows)
            return
        side = W["side"]
        side.wait_event(W["laid_out"])
        with torch.cuda.stream(side):
            W["build_d"]()
            W["build_c"]()
            W["build_e"]()
        W["ev_built"].record(side)
        W["built"][0] = W["ev_built"]

    @_composite
    def dispatch():
        if W["built"][0] is not None:
            torch.cuda.current_stream().wait_event(W["built"][0])
        copy_d()

    return [
        ("ar_160k", lambda: coll.allreduce(W["ar160_in"], W["ar160_out"])),
        ("ar_decode", lambda: coll.allreduce(W["ard_in"], W["ard_out"])),
        ("ar_64m", lambda: coll.allreduce(W["ar64_in"], W["ar64_out"])),
        ("rs_sp", lambda: coll.reduce_scatter(W["sp_in"], W["sp_shard"])),
        ("ag_sp", lambda: coll.all_gather(W["sp_shard"], W["sp_full"])),
        ("gather", lambda: coll.gather(W["lg_in"], W["lg_out"], 0)),
        ("bcast", lambda: coll.broadcast(W["bc_src"], W["bc_out"], 7)),
        ("moe_layout", layout_then_mark),
        ("moe_permute", permute_then_builds),
        ("a2av_dispatch", dispatch),
        ("moe_expert", lambda: coll.moe_expert_scale_apply(W["recv"], E, H, W["ews"])),
        ("a2av_combine", lambda: coll.all_to_all_v_copy(W["recv"], W["back"], H,
                                                        workspace=W["a2a_ws_c"])),
        ("moe_combine", lambda: coll.moe_combine(W["back"], W["pos"], W["moe_w"], W["out"])),
    ]


# rows run only when named with --only
EXTRA_ROWS = {
    "copy_ref": lambda W, coll: coll.broadcast(W["copy_src"], W["copy_dst"], 0),
    # the fused MoE kernels on the step's layout (into the step's buffers)
    "moe_dispatch_fused": lambda W, coll: coll.moe_dispatch(W["moe_x"], W["pos"], W["sc"],
                                                            W["sd"], W["rd"], W["recv"]),
    "moe_combine_fused": lambda W, coll: coll.moe_combine_recv(
        W["recv"], W["pos"], W["sc"], W["sd"], W["rd"], W["moe_w"], W["out"],
        topk_ids=W["moe_ids"]),
}


def bcast_vs_padded_ag(torch, coll, n_toks=(256, 1024, 4096, 16384), H=7168, owner=3,
                       iters=20):
    """The single-image vision-embedding A/B of the sglang PR 33307 digest on
    one GPU: path A pads every rank to max_len rows (= n_tok here, the best
    case for A), AllGathers and keeps the owner's slice; path B broadcasts the
    owner's rows.  Both results are checked bitwise; times are medians."""
    res = {}
    for n in n_toks:
        emb = torch.empty((n, H), dtype=torch.bfloat16, device="cuda").normal_()
        padded = [torch.zeros_like(emb) for _ in range(R)]
        padded[owner].copy_(emb)
        gathered = [torch.empty((R * n, H), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        outs = [torch.empty_like(emb) for _ in range(R)]
        outs[owner] = emb

        def med(fn):
            fn()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(iters)]
            for a, b in ev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            ts = sorted(a.elapsed_time(b) for a, b in ev)
            return ts[len(ts) // 2]

        ta = med(lambda: coll.all_gather(padded, gathered))
        tb = med(lambda: coll.broadcast(emb, outs, owner))
        same = all(torch.equal(gathered[r].view(R, n, H)[owner].view(torch.int16),
                               outs[r].view(torch.int16)) for r in range(R))
        res[str(n)] = {"allgather_us": round(ta * 1e3, 2), "broadcast_us": round(tb * 1e3, 2),
                       "speedup": round(ta / tb, 2), "bitwise_equal": bool(same)}
        del emb, padded, gathered, outs
        torch.cuda.empty_cache()
    return res


def next_rows(torch, coll, iters=20):
    """Rows beyond the step, with their algorithmic bytes: Reduce to a root and
    Scatter from it (R=8, 64 MiB per rank: (R+1)*S and 2*R*S), the uniform
    all-to-all (2*R*S), the sequence <-> heads re-shard of all-to-all
    sequence parallelism (2 * bytes of all ranks) and the context-parallel
    LSE merge (R partials + R lse read, R outputs + R lse written)."""
    res = {}
    bf = torch.bfloat16
    n = (64 << 20) // 2
    xs, (out,), a2a_out = coll.rank_arena([(R, n, bf), (1, n, bf), (R, n, bf)])
    for t in xs:
        t.normal_()
    (root_buf,), chunks = coll.rank_arena([(1, R * n, bf), (R, n, bf)])
    root_buf.normal_()

    def med(fn):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in ev)
        return ts[len(ts) // 2] * 1e-3

    # all-to-all sequence parallelism: 32768-token sequence over 8 ranks,
    # 32 heads x 128, bf16 (32 MiB per rank each way)
    SL, H, D = 4096, 32, 128
    seq, heads, seq_back = coll.rank_arena([(R, (SL, H, D), bf)] * 3)
    for t in seq:
        t.normal_()
    rb = R * SL * H * D * 2
    # context-parallel attention merge: 8192 tokens x 32 heads, head_dim 128
    rows = 8192 * 32
    op_, lp_, oo_, lo_ = coll.rank_arena([(R, (rows, 128), bf), (R, rows, torch.float32),
                                          (R, (rows, 128), bf), (R, rows, torch.float32)])
    for t in op_:
        t.normal_()
    for t in lp_:
        t.normal_(0, 3)
    mb = 2 * R * rows * 128 * 2 + 2 * R * rows * 4
    for name, fn, nbytes in (
            ("reduce_64m", lambda: coll.reduce(xs, out, 0), (R + 1) * n * 2),
            ("scatter_64m", lambda: coll.scatter(root_buf, chunks, 0), 2 * R * n * 2),
            ("all_to_all_64m", lambda: coll.all_to_all(xs, a2a_out), 2 * R * n * 2),
            ("seq_to_heads_32k", lambda: coll.seq_heads_reshard(seq, heads, H, D, True), 2 * rb),
            ("heads_to_seq_32k", lambda: coll.seq_heads_reshard(heads, seq_back, H, D, False),
             2 * rb),
            ("lse_merge_8k_x32h", lambda: coll.lse_merge(op_, lp_, oo_, lo_), mb)):
        t = med(fn)
        gbs = nbytes / t / 1e9
        res[name] = {"us": round(t * 1e6, 2), "bytes": nbytes, "GBps": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}
    del xs, out, root_buf, chunks, a2a_out, seq, heads, seq_back, op_, lp_, oo_, lo_
    torch.cuda.empty_cache()
    return res


def moe_fused(torch, coll, W, per_row_us, iters=10):
    """The fused MoE path on the step's inputs: layout, dispatch straight into
    the receive buffers (permute + All-to-All-v in one pass), combine reading
    them back with the test expert applied as rows are read (expert + reverse
    All-to-All-v + combine in one pass).  Its outputs must equal the unfused
    step's bit for bit.  Bytes: x read + rows written (+ pos) for the
    dispatch; rows read + outputs written (+ w, pos, ids) for the combine."""
    E, T, K, H = W["moe"]
    bf = torch.bfloat16
    recv2, out2 = coll.rank_arena([[(tuple(t.shape), bf) for t in W["recv"]], (R, (T, H), bf)])
    rows = W["moe_rows"]
    b_disp = R * T * H * 2 + rows * H * 2 + R * T * K * 4
    b_comb = rows * H * 2 + R * T * H * 2 + R * T * K * 12
    # prepared calls, as the step's rows: the event pairs time the launches,
    # not the binding's argument checks
    lay = coll.prepare(coll.moe_layout, W["moe_ids"], E, W["sc"], W["sd"], W["rd"], W["ec"],
                       W["pos"], W["ws"])
    disp = coll.prepare(coll.moe_dispatch, W["moe_x"], W["pos"], W["sc"], W["sd"], W["rd"],
                        recv2)
    comb = coll.prepare(coll.moe_combine_recv, recv2, W["pos"], W["sc"], W["sd"], W["rd"],
                        W["moe_w"], out2, topk_ids=W["moe_ids"])
    lay(), disp(), comb()
    torch.cuda.synchronize()
    same = all(torch.equal(a.view(torch.int16), b.view(torch.int16))
               for a, b in zip(out2, W["out"]))
    t = {}
    for name, fn in (("layout", lay), ("dispatch", disp), ("combine", comb)):
        med, _ = _launch_times(torch, lambda i, f=fn: f(), 1, iters)
        t[name] = med
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        lay(), disp(), comb()
    b.record()
    torch.cuda.synchronize()
    pipe = a.elapsed_time(b) / iters * 1e-3
    unfused = sum(per_row_us[n] for n in ("moe_layout", "moe_permute", "a2av_dispatch",
                                          "moe_expert", "a2av_combine", "moe_combine")) * 1e-6
    del recv2, out2
    torch.cuda.empty_cache()
    gb = lambda n, sec: round(n / sec / 1e9, 1)
    return {"dispatch": {"us": round(t["dispatch"] * 1e6, 2), "bytes": b_disp,
                         "GBps": gb(b_disp, t["dispatch"]),
                         "frac": round(b_disp / t["dispatch"] / 1e9 / HBM_PEAK_GBS, 4)},
            "combine": {"us": round(t["combine"] * 1e6, 2), "bytes": b_comb,
                        "GBps": gb(b_comb, t["combine"]),
                        "frac": round(b_comb / t["combine"] / 1e9 / HBM_PEAK_GBS, 4)},
            "layout_us": round(t["layout"] * 1e6, 2),
            "pipeline_us": round(pipe * 1e6, 2),
            "pipeline_GBps": gb(b_disp + b_comb, pipe),
            "unfused_pipeline_us": round(unfused * 1e6, 2),
            "speedup_vs_unfused": round(unfused / pipe, 2),
            "outputs_bitwise_equal_unfused": bool(same)}


def _pct(ts, q):
    return ts[min(len(ts) - 1, int(q * len(ts)))]


def _launch_times(torch, fn, sets, iters, pcts=None):
    """(median of per-launch event pairs, mean over one event pair around
    `iters` back-to-back launches), seconds; launch i uses buffer set i % sets.
    At least 5 warm-up launches come first, every buffer set at least once.
    If `pcts` is a dict, the p10 / p90 of the per-launch times go into it."""
    for i in range(max(sets, 5)):
        fn(i % sets)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record()
        fn(i % sets)
        ev[i][1].record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    if pcts is not None:
        pcts["p10_us"] = round(_pct(ts, 0.1) * 1e3, 2)
        pcts["p90_us"] = round(_pct(ts, 0.9) * 1e3, 2)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(iters):
        fn(i % sets)
    b.record()
    torch.cuda.synchronize()
    return ts[len(ts) // 2] * 1e-3, a.elapsed_time(b) / iters * 1e-3


def _graph_time(torch, fn, sets, n=24, reps=4):
    """Mean time of one launch when `n` launches (launch i on buffer set
    i % sets) are captured in one HIP graph and replayed: the GPU-side cost
    without the host's per-call marshalling in between."""
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        fn(0)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i % sets)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / (n * reps) * 1e-3
    del g
    return t


def copy_ceiling(torch, coll, W):
    """Practical HBM ceiling of this GPU: a plain 1 GiB -> 1 GiB copy through
    the library's copy kernel (2 GiB moved), graph-timed; beside it the same
    copy by the HIP runtime's own device-to-device copy (torch's copy_ of one
    contiguous tensor into another), for comparison."""
    t = _graph_time(torch, lambda i: coll.broadcast(W["copy_src"], W["copy_dst"], 0), 1,
                    n=8, reps=2)
    gbs = (2 << 30) / t / 1e9
    tr = _graph_time(torch, lambda i: W["copy_dst"][0].copy_(W["copy_src"]), 1, n=8, reps=2)
    gbr = (2 << 30) / tr / 1e9
    return {"us": round(t * 1e6, 2), "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
            "runtime_copy_us": round(tr * 1e6, 2), "runtime_copy_GBps": round(gbr, 1),
            "runtime_copy_frac": round(gbr / HBM_PEAK_GBS, 4)}


def expert_table_search(torch, coll, W):
    """The test expert's other path, the table search (a workspace of the
    row-prefix tables alone: no per-row descriptors), on the step's receive
    buffers in place, graph-timed beside the step's row-descriptor path."""
    E, T, K, H = W["moe"]
    R_ = len(W["recv"])
    ws = torch.empty(coll.moe_expert_workspace_bytes(R_, E), dtype=torch.uint8, device="cuda")
    fn = coll.prepare(coll.moe_expert_scale, W["recv"], W["ec"], W["rd"], E, H, ws)
    t = _graph_time(torch, lambda i: fn(), 1, n=8, reps=3)
    nb = 2 * W["moe_rows"] * H * 2
    del ws, fn
    return {"us": round(t * 1e6, 2), "bytes": nb, "GBps": round(nb / t / 1e9, 1),
            "frac": round(nb / t / 1e9 / HBM_PEAK_GBS, 4)}


def fanout_ceiling(torch, coll):
    """The 1 -> 8 fan-out pattern alone, at the MoE permute's volume: the
    library's Broadcast from one 448 MiB buffer to 8 others (4096 tokens x
    7168 bf16 x 8 sources read once, 3.5 GiB written), graph-timed.  Its
    destinations are contiguous, so it is the permute's pattern without the
    row scatter; the outputs are checked against the source."""
    E, T, K, H = 256, 4096, 8, 7168
    n = T * H * R
    bufs = coll.rank_arena([(R + 1, n, torch.bfloat16)])[0]
    g = torch.Generator(device="cuda")
    g.manual_seed(91)
    bufs[0].copy_(torch.randn(n, generator=g, device="cuda"))
    bc = coll.prepare(coll.broadcast, bufs[0], bufs, 0)
    bc()
    torch.cuda.synchronize()
    ok = all(torch.equal(b.view(torch.int16), bufs[0].view(torch.int16)) for b in bufs[1:])
    t = _graph_time(torch, lambda i: bc(), 1, n=8, reps=3)
    nb = (R + 1) * n * 2
    del bufs, bc
    torch.cuda.empty_cache()
    return {"read_bytes": n * 2, "written_bytes": R * n * 2, "us": round(t * 1e6, 2),
            "GBps": round(nb / t / 1e9, 1), "frac": round(nb / t / 1e9 / HBM_PEAK_GBS, 4),
            "outputs_equal_source": bool(ok)}


def latency_rows_graph(torch, coll, W, per_row_us):
    """The latency-bound rows of the step: HIP-graph replay beside the eager
    costs.  `eager_prepared_us` is one back-to-back prepared call (a decode
    loop issuing the collective: 2000 calls between one event pair, so the
    host's issue cost and the GPU time overlap as they would there);
    `eager_prepared_median_us` is the median of single calls each between its
    own event pair; `eager_plain_*` the same for plain binding calls (argument
    checks and marshalling every call); `in_step_us` the row inside the timed
    step, whose per-row event pairs add their own cost."""
    E, T, K, H = W["moe"]
    rows = {
        "ar_160k": (coll.allreduce, (W["ar160_in"], W["ar160_out"])),
        "ar_decode": (coll.allreduce, (W["ard_in"], W["ard_out"])),
        "bcast": (coll.broadcast, (W["bc_src"], W["bc_out"], 7)),
        "moe_layout": (coll.moe_layout, (W["moe_ids"], E, W["sc"], W["sd"], W["rd"], W["ec"],
                                         W["pos"], W["ws"])),
    }
    res = {}
    for name, (call, args) in rows.items():
        plan = coll.prepare(call, *args)
        t = _graph_time(torch, lambda i: plan(), 1)
        med_p, batch_p = _launch_times(torch, lambda i: plan(), 1, 2000)
        med_plain, batch_plain = _launch_times(torch, lambda i: call(*args), 1, 500)
        res[name] = {"graph_us": round(t * 1e6, 2),
                     "eager_prepared_us": round(batch_p * 1e6, 2),
                     "eager_prepared_median_us": round(med_p * 1e6, 2),
                     "eager_plain_us": round(batch_plain * 1e6, 2),
                     "eager_plain_median_us": round(med_plain * 1e6, 2),
                     "in_step_us": per_row_us[name]}
    return res


def _ar_sets(torch, coll, n, sets, arena):
    out = []
    for _ in range(sets):
        if arena:
            ins, outs = coll.rank_arena([(R, n, torch.bfloat16), (R, n, torch.bfloat16)])
            for t in ins:
                t.normal_(0, 0.02)
        else:
            ins = [torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_(0, 0.02)
                   for _ in range(R)]
            outs = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        out.append((ins, outs))
    return out


def ar_sweep(torch, coll, log2_sizes=range(13, 27)):
    """AllReduce R=8 bf16 1-D, S = 8 KiB .. 64 MiB per rank (powers of two),
    N(0, 0.02^2), rank buffers in rank arenas.  From 8 MiB up, 4 buffer sets
    rotate so the working set (>= 1 GiB at 16 MiB) exceeds the Infinity Cache.
    Reports graph-replay time, the median (p10/p90) of per-launch event
    timings over 50 launches (1000 below 1 MiB) and a back-to-back batch."""
    res = {}
    for lg in log2_sizes:
        S = 1 << lg
        sets = 4 if S >= (8 << 20) else 1
        iters = 1000 if S < (1 << 20) else 50
        bufs = _ar_sets(torch, coll, S // 2, sets, True)
        plans = [coll.prepare(coll.allreduce, *b) for b in bufs]
        pc = {}
        med, batch = _launch_times(torch, lambda i: plans[i](), sets, iters, pc)
        gt = _graph_time(torch, lambda i: plans[i](), sets)
        nbytes = 2 * R * S
        algbw = S / gt / 1e9                     # nccl-tests style: S / t
        key = f"{S >> 20}MiB" if S >= (1 << 20) else f"{S >> 10}KiB"
        res[key] = {"graph_us": round(gt * 1e6, 2),
                            "graph_GBps": round(nbytes / gt / 1e9, 1),
                            "graph_frac": round(nbytes / gt / 1e9 / HBM_PEAK_GBS, 4),
                            "algbw_GBps": round(algbw, 1),
                            "busbw_GBps": round(algbw * 2 * (R - 1) / R, 1),
                            "median_us": round(med * 1e6, 2), **pc,
                            "GBps": round(nbytes / med / 1e9, 1),
                            "frac": round(nbytes / med / 1e9 / HBM_PEAK_GBS, 4),
                            "batch_us": round(batch * 1e6, 2),
                            "batch_GBps": round(nbytes / batch / 1e9, 1),
                            "batch_frac": round(nbytes / batch / 1e9 / HBM_PEAK_GBS, 4)}
        del bufs, plans
        torch.cuda.empty_cache()
    return res


def _a2a_entry(torch, fn, sets, iters, nb, graph_n=24, graph_reps=4):
    pc = {}
    med, batch = _launch_times(torch, fn, sets, iters, pc)
    gt = _graph_time(torch, fn, sets, n=graph_n, reps=graph_reps)
    return {"graph_us": round(gt * 1e6, 2), "graph_GBps": round(nb / gt / 1e9, 1),
            "graph_frac": round(nb / gt / 1e9 / HBM_PEAK_GBS, 4),
            "median_us": round(med * 1e6, 2), **pc, "GBps": round(nb / med / 1e9, 1),
            "frac": round(nb / med / 1e9 / HBM_PEAK_GBS, 4),
            "batch_GBps": round(nb / batch / 1e9, 1)}


def a2a_sweep(torch, coll, synth):
    """All-to-All-v at R=8 (bf16): (i) uniform 1-D, S = 8 KiB .. 64 MiB per
    rank in rows of one element, equal counts; (ii) uniform, S = 16 / 32 /
    64 MiB per rank in rows of 8 elements (16 bytes), plain and with a
    workspace (descriptor form); (iii) MoE-shaped, T tokens per rank x top-8
    of 256 experts (Zipf 1.2 routing), rows of 7168, plain and with a
    workspace.  Buffers in rank arenas; sets rotate so that a size's working
    set exceeds the 256 MB Infinity Cache where it can.  Algorithmic bytes
    2 * (rows moved) * row bytes.  Reports the median per-launch time, a batch
    mean and the graph-replay time."""
    import numpy as np
    bf = torch.bfloat16
    res = {"uniform_row1": {}, "uniform_row8": {}, "uniform_row8_ws": {},
           "moe_rows7168": {}, "moe_rows7168_ws": {}}
    dc = lambda a: torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda()
    for lg in range(13, 27):
        S = 1 << lg
        n = S // 2
        c = np.full((R, R), n // R, np.int64)
        sd = np.tile(np.arange(R, dtype=np.int64) * (n // R), (R, 1))
        tabs = (dc(c), dc(sd), dc(sd))          # packed: rdispls[d][s] = s * n/R
        sets = 4 if S >= (8 << 20) else 1
        bufs = []
        for _ in range(sets):
            snd, rcv = coll.rank_arena([(R, n, bf), (R, n, bf)])
            for t in snd:
                t.normal_()
            bufs.append((snd, rcv))
        plans = [coll.prepare(coll.all_to_all_v, b[0], tabs[0], tabs[1], b[1], tabs[2], 1)
                 for b in bufs]
        res["uniform_row1"][f"{S >> 10}KiB"] = _a2a_entry(
            torch, lambda i: plans[i](), sets, 1000 if S < (1 << 20) else 50, 2 * R * S)
        del bufs, plans
    for lg in (24, 25, 26):
        S = 1 << lg
        rows = S // 16                           # rows of 8 bf16 per rank
        c = np.full((R, R), rows // R, np.int64)
        sd = np.tile(np.arange(R, dtype=np.int64) * (rows // R), (R, 1))
        tabs = (dc(c), dc(sd), dc(sd))
        sets = 4
        bufs = []
        for _ in range(sets):
            snd, rcv = coll.rank_arena([(R, (rows, 8), bf), (R, (rows, 8), bf)])
            for t in snd:
                t.normal_()
            bufs.append((snd, rcv))
        ws = [torch.empty(max(coll.all_to_all_v_workspace_bytes(b[0], b[1], 8), 256),
                          dtype=torch.uint8, device="cuda") for b in bufs]
        for key, kw in (("uniform_row8", lambda i: {}),
                        ("uniform_row8_ws", lambda i: {"workspace": ws[i]})):
            plans = [coll.prepare(coll.all_to_all_v, b[0], tabs[0], tabs[1], b[1], tabs[2], 8,
                                  **kw(i)) for i, b in enumerate(bufs)]
            res[key][f"{S >> 10}KiB"] = _a2a_entry(torch, lambda i: plans[i](), sets, 50,
                                                   2 * R * S)
            del plans
        del bufs, ws
    E, K, H = 256, 8, 7168
    for T in (16, 64, 256, 1024, 4096):
        ids = [torch.from_numpy(synth.zipf_routing(T, E, K, seed=5100 + s)[0]).cuda()
               for s in range(R)]
        sc = torch.empty(R * R, dtype=torch.int64, device="cuda")
        sdd, rdd = torch.empty_like(sc), torch.empty_like(sc)
        ec = torch.empty(R * E, dtype=torch.int32, device="cuda")
        pos = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in range(R)]
        ws = torch.empty(coll.moe_workspace_bytes(R, T, K, E), dtype=torch.uint8, device="cuda")
        coll.moe_layout(ids, E, sc, sdd, rdd, ec, pos, ws)
        torch.cuda.synchronize()
        cnt = sc.view(R, R).cpu()
        rows = int(cnt.sum())
        sets = 1 if T >= 4096 else (2 if T >= 256 else 4)
        bufs = []
        for _ in range(sets):
            snd, rcv = coll.rank_arena([(R, (T * K, H), bf),
                                        [((int(cnt[:, d].sum()), H), bf) for d in range(R)]])
            for t in snd:
                t.normal_()
            bufs.append((snd, rcv))
        a2ws = [torch.empty(max(coll.all_to_all_v_workspace_bytes(b[0], b[1], H), 256),
                            dtype=torch.uint8, device="cuda") for b in bufs]
        nb = 2 * rows * H * 2
        for key, kw in (("moe_rows7168", lambda i: {}),
                        ("moe_rows7168_ws", lambda i: {"workspace": a2ws[i]})):
            plans = [coll.prepare(coll.all_to_all_v, b[0], sc, sdd, b[1], rdd, H, **kw(i))
                     for i, b in enumerate(bufs)]
            res[key][f"T{T}"] = {
                "per_rank_MiB": round(T * K * H * 2 / 2**20, 2), "rows": rows,
                **_a2a_entry(torch, lambda i: plans[i](), sets, 50, nb,
                             graph_n=8 if T >= 4096 else 24, graph_reps=2)}
            del plans
        del bufs, ids, pos, ws, a2ws
    torch.cuda.empty_cache()
    return res


def layout_ab(torch, coll, mib=16, sets=4, iters=24):
    """AllReduce R=8 bf16 at `mib` MiB per rank with the 16 buffers of a call
    allocated one by one by torch (each its own large allocation, so they tend
    to share their offset modulo 64 KiB) vs placed in a rank arena."""
    res = {}
    nbytes = 2 * R * (mib << 20)
    for name, arena in (("torch_alloc", False), ("rank_arena", True)):
        bufs = _ar_sets(torch, coll, (mib << 20) // 2, sets, arena)
        plans = [coll.prepare(coll.allreduce, *b) for b in bufs]
        med, batch = _launch_times(torch, lambda i: plans[i](), sets, iters)
        res[name] = {"median_us": round(med * 1e6, 2), "GBps": round(nbytes / med / 1e9, 1),
                     "batch_GBps": round(nbytes / batch / 1e9, 1)}
        del bufs, plans
        torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------- CPU baseline

def cpu_baseline(min_seconds=10.0, max_passes=3):
    """The oracle as it stands, single-threaded, on whole passes of the step at
    its bench sizes, repeated until at least `min_seconds` of CPU work (at
    most `max_passes` passes; inputs generated once)."""
    import numpy as np

    import oracle
    from collective_communication_amd import synth

    oracle.lib()
    t_total = 0.0
    bytes_total = 0

    def timed(fn, nbytes):
        nonlocal t_total, bytes_total
        t0 = time.perf_counter()
        fn()
        t_total += time.perf_counter() - t0
        bytes_total += nbytes

    ar160 = [synth.gaussian(81920, 1.0, 1000 + r, "bf16") for r in range(4)]
    ard = [synth.gaussian(64 * 7168, 0.02, 2000 + r, "bf16") for r in range(R)]
    n = (64 << 20) // 2
    ar64 = [synth.gaussian(n, 0.02, 7000 + r, "bf16") for r in range(R)]
    sp = [synth.gaussian(8192 * 4096, 1.0, 3000 + r, "bf16") for r in range(R)]
    S = 8192 * 4096 * 2
    lg = [synth.gaussian((256, 19008), 2.0, 4000 + r, "fp32") for r in range(R)]
    ids = synth.uniform_int32(256, 0, 152064, 4107)
    E, T, K, H = 256, 4096, 8, 7168
    tid, tw = [], []
    for s in range(R):
        i, w = synth.zipf_routing(T, E, K, seed=5100 + s)
        tid.append(i)
        tw.append(w)
    tx = [synth.gaussian((T, H), 1.0, 5000 + s, "bf16") for s in range(R)]
    rows = R * T * K
    moe_bytes = (2 * R * T * K * 4 + (R * T * H * 2 + rows * H * 2 + R * T * K * 4)
                 + 3 * 2 * rows * H * 2 + rows * H * 2 + R * T * H * 2 + R * T * K * 8)
    passes = 0
    while passes < max_passes and (passes == 0 or t_total < min_seconds):
        timed(lambda: oracle.allreduce(ar160, "bf16"), 2 * 4 * 81920 * 2)
        timed(lambda: oracle.allreduce(ard, "bf16"), 2 * R * 64 * 7168 * 2)
        timed(lambda: oracle.allreduce(ar64, "bf16"), 2 * R * n * 2)
        holder = {}
        timed(lambda: holder.setdefault("rs", oracle.reduce_scatter(sp, "bf16")), (R + 1) * S)
        timed(lambda: oracle.all_gather(holder["rs"]), S + R * S)
        del holder
        timed(lambda: oracle.gather(lg, 0), 2 * R * 256 * 19008 * 4)
        timed(lambda: oracle.broadcast(ids, R, 7), 256 * 4 * R)
        timed(lambda: oracle.moe_pipeline(tx, tid, tw, E), moe_bytes)
        passes += 1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         "")
    except OSError:
        pass
    return {"value": round(bytes_total / t_total / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "host_cpus_visible": len(os.sched_getaffinity(0)), "host_cpu_model": model,
            "seconds": round(t_total, 2), "passes": passes,
            "sample": f"{passes} pass(es) of every step row at its bench size (MoE leg: all "
                      "4096 tokens per rank); single-threaded C oracle (gcc -O2), algorithmic "
                      "bytes of the sample / its wall time"}


# ------------------------------------------------------------------ roofline

def counter_traffic(kernel_src: str):
    """HBM traffic per launch of the dominant kernel from the committed
    rocprofv3 --pmc summary, or None when missing or when the kernel source has
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "a2av_dispatch_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel source sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic bytes per launch:\s*([0-9]+)", text)
    if not m_sha or not m_b:
        return None
    with open(kernel_src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != m_sha.group(1):
            return None
    return int(m_b.group(1))


def _as_pct(f):
    return "—" if f is None else f"{100 * f:.1f}%"


def report(path):
    """Markdown tables of one saved JSON line of this benchmark (the last line
    of the file): the step, its rows, the sweeps and the side measurements, in
    the form the documentation quotes them, so that every figure there can be
    traced back to one run."""
    d = json.loads(open(path).read().strip().splitlines()[-1])
    o = []
    rf = d["roofline"] or {}
    tr = rf.get("traffic")
    o += ["| Step | value |", "|---|---|",
          f"| whole step (`value`) | {d['value']:.1f} GB/s = {_as_pct(d['value'] / HBM_PEAK_GBS)}, "
          f"{d['ms_per_step']} ms per step |"]
    if d.get("step_graph_replay"):
        g = d["step_graph_replay"]
        o.append(f"| the same step by graph replay | {g['GBps']} GB/s = {_as_pct(g['frac'])}, "
                 f"{g['ms_per_step']} ms |")
    if rf:
        o.append(f"| dominant kernel ({rf['kernel'].split(' ')[0]}) | {rf['achieved']} GB/s = "
                 f"{_as_pct(rf['frac'])}, {rf['avg_launch_us']} µs per launch; counter traffic "
                 + (f"{tr / rf['bytes_per_launch']:.4f}× the algorithmic bytes |" if tr else "n/a |"))
    if d.get("cpu_baseline"):
        c = d["cpu_baseline"]
        o.append(f"| CPU baseline (oracle, {c['cores']} core) | {c['value']} GB/s |")
    o += ["", "| Step row | µs | GB/s | % of peak |", "|---|---|---|---|"]
    for k, v in d["rows"].items():
        o.append(f"| {k} | {v['us']} | {v['GBps']} | {_as_pct(v['frac'])} |")
    sw = d.get("allreduce_sweep")
    if sw:
        o += ["", "| AllReduce R=8 bf16, per rank | graph µs | graph | median µs | median |",
              "|---|---|---|---|---|"]
        for k, v in sw.items():
            if isinstance(v, dict) and "graph_us" in v and v["graph_frac"] >= 0.3:
                o.append(f"| {k} | {v['graph_us']} | {_as_pct(v['graph_frac'])} | {v['median_us']} "
                         f"| {_as_pct(v['frac'])} |")
    a2 = d.get("all_to_all_v_sweep")
    if a2:
        o += ["", "| All-to-All-v R=8 | size | graph µs | graph | median |", "|---|---|---|---|---|"]
        for series, pts in a2.items():
            if not isinstance(pts, dict):
                continue
            for k, v in pts.items():
                if not (isinstance(v, dict) and "graph_us" in v):
                    continue
                big = (series.startswith("moe") and k in ("T256", "T1024", "T4096")) or \
                      (k.endswith("KiB") and int(k[:-3]) >= 16384)
                if big:
                    o.append(f"| {series} | {k} | {v['graph_us']} | {_as_pct(v['graph_frac'])} | "
                             f"{_as_pct(v['frac'])} |")
    if d.get("next_rows"):
        o += ["", "| Further row | µs | GB/s | % of peak |", "|---|---|---|---|"]
        for k, v in d["next_rows"].items():
            o.append(f"| {k} | {v['us']} | {v['GBps']} | {_as_pct(v['frac'])} |")
    f = d.get("moe_fused")
    if f:
        o += ["", "| Fused MoE path | value |", "|---|---|",
              f"| dispatch (permute + All-to-All-v) | {f['dispatch']['us']} µs, {_as_pct(f['dispatch']['frac'])} |",
              f"| combine (expert + reverse All-to-All-v + combine) | {f['combine']['us']} µs, "
              f"{_as_pct(f['combine']['frac'])} |",
              f"| pipeline (layout + dispatch + combine) | {f['pipeline_us']} µs against "
              f"{f['unfused_pipeline_us']} µs unfused ({f['speedup_vs_unfused']}×); outputs bitwise "
              f"equal: {f['outputs_bitwise_equal_unfused']} |"]
    lat = d.get("latency_rows_graph")
    if lat:
        o += ["", "| Latency row | graph µs | eager prepared µs (back to back) | eager plain µs "
                  "(back to back) | in the step (event pair) µs |", "|---|---|---|---|---|"]
        for k, v in lat.items():
            o.append(f"| {k} | {v['graph_us']} | {v['eager_prepared_us']} | {v['eager_plain_us']} | "
                     f"{v['in_step_us']} |")
    ex = []
    if d.get("copy_ceiling_1gib"):
        c = d["copy_ceiling_1gib"]
        ex.append(f"| plain 1 GiB copy (graph) | {c['us']} µs, {c['GBps']} GB/s = {_as_pct(c['frac'])} |")
        if "runtime_copy_us" in c:
            ex.append(f"| the same copy by the HIP runtime's device-to-device copy (graph) | "
                      f"{c['runtime_copy_us']} µs, {c['runtime_copy_GBps']} GB/s = "
                      f"{_as_pct(c['runtime_copy_frac'])} |")
    if d.get("fanout_ceiling_1to8"):
        f = d["fanout_ceiling_1to8"]
        ex.append(f"| 1 → 8 fan-out at the permute's volume (Broadcast, 448 MiB to 8 buffers, graph) | "
                  f"{f['us']} µs, {f['GBps']} GB/s = {_as_pct(f['frac'])} |")
    if d.get("moe_expert_table_search"):
        e = d["moe_expert_table_search"]
        ex.append(f"| test expert by table search (no row descriptors), the MoE shape (graph) | "
                  f"{e['us']} µs, {e['GBps']} GB/s = {_as_pct(e['frac'])} |")
    if d.get("allreduce_16mib_layout_ab"):
        a = d["allreduce_16mib_layout_ab"]
        ex.append(f"| AllReduce 16 MiB × 8, torch allocations vs rank arena | "
                  f"{a['torch_alloc']['GBps']} vs {a['rank_arena']['GBps']} GB/s (median) |")
    if d.get("broadcast_vs_padded_allgather"):
        b = d["broadcast_vs_padded_allgather"]
        ex.append("| broadcast vs pad-to-max AllGather, tokens: speedup | "
                  + ", ".join(f"{k}: {v['speedup']}×" for k, v in b.items())
                  + f"; bitwise equal: {all(v['bitwise_equal'] for v in b.values())} |")
    if ex:
        o += ["", "| Other | value |", "|---|---|"] + ex
    print("\n".join(o))


def main():
    args = parse()
    if args.report:
        report(args.report)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "libcoll runs its R ranks as virtual ranks in one GPU's "
                                   "HBM; --gpus must be 1"}))
        sys.exit(2)

    import torch

    from collective_communication_amd import coll, synth
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    coll.lib()
    W = make_inputs(torch, synth, coll)
    rows = step_rows(W, coll, torch)
    if args.only:
        keep = set(args.only.split(","))
        rows = [r for r in rows if r[0] in keep]
        rows += [(n, (lambda f=f: f(W, coll))) for n, f in EXTRA_ROWS.items() if n in keep]
    # every row is a prepared call: argument checks and marshalling happen
    # once, each launch only re-issues the C entry point
    rows = [(n, fn if getattr(fn, "composite", False) else coll.prepare(fn)) for n, fn in rows]
    nbytes = row_bytes(W)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for _, fn in rows:
            fn()
    torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    names = [n for n, _ in rows]
    # the timed steps carry only the two bracketing events; the per-row
    # breakdown comes from as many steps again, each row between event pairs
    # (which add their own cost between rows)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        for _, fn in rows:
            fn()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    print("[bench] per-row breakdown", file=sys.stderr, flush=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(rows) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        e = evs[k]
        e[0].record()
        for j, (_, fn) in enumerate(rows):
            fn()
            e[j + 1].record()
    torch.cuda.synchronize()
    rows_ms = sum(evs[k][0].elapsed_time(evs[k][-1]) for k in range(args.steps)) / args.steps
    per_row = {n: sum(evs[k][j].elapsed_time(evs[k][j + 1]) for k in range(args.steps)) / args.steps
               for j, n in enumerate(names)}
    step_bytes = sum(nbytes[n] for n in names)
    value = step_bytes / (ms_step * 1e-3) / 1e9

    rows_out = {}
    for n in names:
        ms = per_row[n]
        gbs = nbytes[n] / (ms * 1e-3) / 1e9
        rows_out[n] = {"us": round(ms * 1e3, 2), "bytes": nbytes[n], "GBps": round(gbs, 1),
                       "frac": round(gbs / HBM_PEAK_GBS, 4)}

    dom = "a2av_dispatch"
    roof = None
    if dom in per_row:
        ach = nbytes[dom] / (per_row[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm",
                "kernel": "a2av_desc_kernel<16> (All-to-All-v dispatch, descriptor form; its "
                          "descriptor build runs on a second stream beside the permute)",
                "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": counter_traffic(os.path.join(ROOT, "collective_communication_amd",
                                                        "csrc", "a2av.hip")),
                "bytes_per_launch": nbytes[dom],
                "avg_launch_us": round(per_row[dom] * 1e3, 2)}

    sweep = lab = a2s = None
    if not args.no_sweep and not args.only:
        print("[bench] allreduce sweep", file=sys.stderr, flush=True)
        sweep = ar_sweep(torch, coll)
        print("[bench] allocation layout A/B", file=sys.stderr, flush=True)
        lab = layout_ab(torch, coll)
        print("[bench] all-to-all-v sweep", file=sys.stderr, flush=True)
        a2s = a2a_sweep(torch, coll, synth)

    # the same step captured once in a HIP graph and replayed K times: the
    # GPU-side step time without per-row events or host launch gaps
    step_graph = None
    if not args.only:
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            for _, fn in rows:
                fn()
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _, fn in rows:
                fn()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        gms = a.elapsed_time(b) / args.steps
        step_graph = {"ms_per_step": round(gms, 4),
                      "GBps": round(step_bytes / (gms * 1e-3) / 1e9, 1),
                      "frac": round(step_bytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del g

    fused = lat = ceil_ = fan = ets = None
    if not args.only:
        print("[bench] fused MoE path", file=sys.stderr, flush=True)
        fused = moe_fused(torch, coll, W, {n: rows_out[n]["us"] for n in names})
        if not args.no_sweep:
            print("[bench] latency rows by graph replay", file=sys.stderr, flush=True)
            lat = latency_rows_graph(torch, coll, W, {n: rows_out[n]["us"] for n in names})
            ceil_ = copy_ceiling(torch, coll, W)
            fan = fanout_ceiling(torch, coll)
            ets = expert_table_search(torch, coll, W)

    ab = extra = None
    if not args.no_sweep and not args.only:
        print("[bench] broadcast vs padded allgather", file=sys.stderr, flush=True)
        ab = bcast_vs_padded_ag(torch, coll)
        print("[bench] reduce / scatter", file=sys.stderr, flush=True)
        extra = next_rows(torch, coll)

    cpu = None
    if not args.no_cpu_baseline and not args.only:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline()

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "hot path over R=8 virtual ranks in one GPU: AllReduce "
                               "(160 KiB x4, [64,7168] x8, 64 MiB x8), SP ReduceScatter+"
                               "AllGather [8192,4096] x8, Gather fp32 [256,19008] x8 + "
                               "Broadcast int32[256], MoE dispatch/combine 4096 tok x 7168 "
                               "top-8 of 256 experts via All-to-All-v",
                   "ranks": R, "step_bytes": step_bytes,
                   "buffers": "rank arenas (coll_arena_layout: own 2 MiB page + 4 KiB colour per buffer)",
                   "moe_rows": W["moe_rows"], "moe_dest_share": W["dest_share"]},
        "roofline": roof,
        "step_graph_replay": step_graph,
        "ms_per_step_with_row_events": round(rows_ms, 4),
        "cpu_baseline": cpu,
        "rows": rows_out,
        "allreduce_sweep": sweep,
        "allreduce_16mib_layout_ab": lab,
        "all_to_all_v_sweep": a2s,
        "broadcast_vs_padded_allgather": ab,
        "next_rows": extra,
        "moe_fused": fused,
        "latency_rows_graph": lat,
        "copy_ceiling_1gib": ceil_,
        "fanout_ceiling_1to8": fan,
        "moe_expert_table_search": ets,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
