"""Library calls captured in a HIP graph (torch.cuda.CUDAGraph) replay
correctly: every replay, with new inputs copied in eagerly between replays,
matches the oracle bit for bit.  The library enqueues only kernels (no
memsets, no host synchronisation), so a whole decode-style sequence can be
captured and replayed without Python in the loop."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import coll, synth
from gpu_util import bits_equal, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    coll.lib()
    yield
    torch.cuda.synchronize()


def test_graph_replays_decode_allreduce_broadcast_and_a2av():
    R, H = 8, 7168
    say("graph: allreduce + broadcast + a2av")
    # static buffers the graph reads and writes
    ins, outs = coll.rank_arena([(R, (64, H), torch.bfloat16), (R, (64, H), torch.bfloat16)])
    (bc,) = coll.rank_arena([(R, 256, torch.int32)])
    W = 24
    cnt = np.array([[(s * 3 + d) % 5 for d in range(R)] for s in range(R)], np.int64)
    sd, rd = oracle.packed_displs(cnt)
    srows, rrows = cnt.sum(axis=1), cnt.sum(axis=0)
    sends, recvs = coll.rank_arena([[((int(srows[s]), W), torch.bfloat16) for s in range(R)],
                                    [((int(rrows[d]), W), torch.bfloat16) for d in range(R)]])
    dc = lambda a: torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda()
    c_d, sd_d, rd_d = dc(cnt), dc(sd), dc(rd)

    def feed(it):
        xs = [synth.gaussian((64, H), 0.02, 60000 + 100 * it + r, "bf16") for r in range(R)]
        ids = synth.uniform_int32(256, 0, 152064, 61000 + it)
        ys = [synth.random_bits((int(srows[s]), W), 2, 62000 + 100 * it + s) for s in range(R)]
        for t, x in zip(ins, xs):
            t.copy_(dev(x))
        bc[5].copy_(torch.from_numpy(ids))
        for t, y in zip(sends, ys):
            if t.numel():
                t.copy_(dev(y))
        for t in outs + recvs:
            t.view(torch.int16).fill_(0x7FAB)
        for r in range(R):
            if r != 5:
                bc[r].fill_(-1)
        torch.cuda.synchronize()
        return xs, ids, ys

    def calls():
        coll.allreduce(ins, outs)
        coll.broadcast(bc[5], bc, 5)
        coll.all_to_all_v(sends, c_d, sd_d, recvs, rd_d, W)

    feed(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()                                     # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for it in range(1, 5):
        xs, ids, ys = feed(it)
        g.replay()
        torch.cuda.synchronize()
        want = oracle.allreduce([x.reshape(-1) for x in xs], "bf16")
        for r in range(R):
            assert bits_equal(host(outs[r]).reshape(-1), want[r]), (it, r)
            assert np.array_equal(host(bc[r]), ids), (it, r)
        want_a = oracle.all_to_all_v(ys, cnt, sd, rd, rrows, W)
        for d in range(R):
            assert bits_equal(host(recvs[d]).reshape(-1), want_a[d].reshape(-1)), (it, d)


def test_graph_replays_fused_moe_pipeline():
    """Layout + fused dispatch + fused combine (test expert inline) captured
    once; receive buffers sized for the worst case (every row to one rank)."""
    R, E, T, K, H = 8, 64, 96, 4, 128
    say("graph: fused moe")
    id_d = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in range(R)]
    w_d = [torch.empty((T, K), dtype=torch.float32, device="cuda") for _ in range(R)]
    x_d = [torch.empty((T, H), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    sc = torch.empty(R * R, dtype=torch.int64, device="cuda")
    sdd, rdd = torch.empty_like(sc), torch.empty_like(sc)
    ec = torch.empty(R * E, dtype=torch.int32, device="cuda")
    pos = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in range(R)]
    ws = torch.empty(coll.moe_workspace_bytes(R, T, K, E), dtype=torch.uint8, device="cuda")
    recvs = [torch.empty((R * T * K, H), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device="cuda") for _ in range(R)]

    def feed(it):
        ids, wts, xs = [], [], []
        for s in range(R):
            i, w = synth.zipf_routing(T, E, K, seed=63000 + 100 * it + s)
            ids.append(i)
            wts.append(w)
            xs.append(synth.gaussian((T, H), 1.0, 64000 + 100 * it + s, "bf16"))
            id_d[s].copy_(torch.from_numpy(i))
            w_d[s].copy_(torch.from_numpy(w))
            x_d[s].copy_(dev(xs[s]))
            outs[s].view(torch.int16).fill_(0x7FAB)
        torch.cuda.synchronize()
        return xs, ids, wts

    def calls():
        coll.moe_layout(id_d, E, sc, sdd, rdd, ec, pos, ws)
        coll.moe_dispatch(x_d, pos, sc, sdd, rdd, recvs)
        coll.moe_combine_recv(recvs, pos, sc, sdd, rdd, w_d, outs, topk_ids=id_d)

    feed(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for it in range(1, 5):
        xs, ids, wts = feed(it)
        g.replay()
        torch.cuda.synchronize()
        want = oracle.moe_pipeline(xs, ids, wts, E)
        for r in range(R):
            assert bits_equal(host(outs[r]).reshape(-1), want["outs"][r].reshape(-1)), (it, r)


def test_graph_replays_moe_step_with_descriptor_builds_on_a_second_stream():
    """The unfused MoE sequence as the benchmark step runs it: the layout
    marks an event, the permute runs, a second stream waits for that event
    and builds both exchanges' descriptor tables and the test expert's row
    descriptors, the main stream waits for them and runs the two copies
    around the expert's scaling, then the combine.
    Captured once (fork and join by events), replayed with new routing and
    tokens each time.  Each receive buffer holds the most rows any of the
    routings sends it; both directions' capacities (256 MiB and more) are
    above the descriptor form's threshold."""
    R, E, T, K, H = 8, 64, 1024, 4, 4096
    say("graph: moe step, split descriptor form, two streams")
    bf = torch.bfloat16
    id_d = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in range(R)]
    w_d = [torch.empty((T, K), dtype=torch.float32, device="cuda") for _ in range(R)]
    x_d = [torch.empty((T, H), dtype=bf, device="cuda") for _ in range(R)]
    sc = torch.empty(R * R, dtype=torch.int64, device="cuda")
    sdd, rdd = torch.empty_like(sc), torch.empty_like(sc)
    ec = torch.empty(R * E, dtype=torch.int32, device="cuda")
    pos = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in range(R)]
    ws = torch.empty(coll.moe_workspace_bytes(R, T, K, E), dtype=torch.uint8, device="cuda")
    send = [torch.empty((T * K, H), dtype=bf, device="cuda") for _ in range(R)]
    per = E // R
    routes = [[synth.zipf_routing(T, E, K, seed=66000 + 100 * it + s) for s in range(R)]
              for it in range(5)]
    need = [max(sum(int(np.count_nonzero(i // per == d)) for i, _ in rt) for rt in routes)
            for d in range(R)]
    recv = [torch.empty((need[d], H), dtype=bf, device="cuda") for d in range(R)]
    back = [torch.empty((T * K, H), dtype=bf, device="cuda") for _ in range(R)]
    outs = [torch.empty((T, H), dtype=bf, device="cuda") for _ in range(R)]
    wsd = torch.empty(coll.all_to_all_v_workspace_bytes(send, recv, H), dtype=torch.uint8,
                      device="cuda")
    wsc = torch.empty(coll.all_to_all_v_workspace_bytes(recv, back, H), dtype=torch.uint8,
                      device="cuda")
    assert wsd.numel() > 0 and wsc.numel() > 0
    ews = torch.empty(coll.moe_expert_workspace_bytes(R, E, sum(need)), dtype=torch.uint8,
                      device="cuda")
    side = torch.cuda.Stream()
    laid_out, built = torch.cuda.Event(), torch.cuda.Event()

    def feed(it):
        ids, wts, xs = [], [], []
        for s in range(R):
            i, w = routes[it][s]
            ids.append(i)
            wts.append(w)
            xs.append(synth.gaussian((T, H), 1.0, 67000 + 100 * it + s, "bf16"))
            id_d[s].copy_(torch.from_numpy(i))
            w_d[s].copy_(torch.from_numpy(w))
            x_d[s].copy_(dev(xs[s]))
            outs[s].view(torch.int16).fill_(0x7FAB)
        torch.cuda.synchronize()
        return xs, ids, wts

    def calls():
        coll.moe_layout(id_d, E, sc, sdd, rdd, ec, pos, ws)
        laid_out.record()
        coll.moe_permute(x_d, pos, send)
        side.wait_event(laid_out)
        with torch.cuda.stream(side):
            coll.all_to_all_v_build(send, sc, sdd, recv, rdd, H, wsd)
            coll.all_to_all_v_reverse_build(recv, sc, sdd, back, rdd, H, wsc)
            coll.moe_expert_scale_build(recv, ec, rdd, E, H, ews)
        built.record(side)
        torch.cuda.current_stream().wait_event(built)
        coll.all_to_all_v_copy(send, recv, H, wsd)
        coll.moe_expert_scale_apply(recv, E, H, ews)
        coll.all_to_all_v_copy(recv, back, H, wsc)
        coll.moe_combine(back, pos, w_d, outs)

    feed(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for it in range(1, 5):
        xs, ids, wts = feed(it)
        g.replay()
        torch.cuda.synchronize()
        want = oracle.moe_pipeline(xs, ids, wts, E)
        for r in range(R):
            assert bits_equal(host(outs[r]).reshape(-1), want["outs"][r].reshape(-1)), (it, r)
