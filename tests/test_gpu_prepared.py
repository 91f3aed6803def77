"""Prepared calls (coll.prepare): a collective validated and marshalled once,
then re-issued on persistent buffers, gives the oracle's result every time,
eagerly and inside a captured HIP graph."""
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


def test_prepared_allreduce_and_a2av_reissued_with_new_inputs():
    R, n, W = 8, 64 * 7168, 16
    say("prepared allreduce + a2av")
    ins, outs = coll.rank_arena([(R, n, torch.bfloat16), (R, n, torch.bfloat16)])
    cnt = np.array([[(3 * s + d) % 7 for d in range(R)] for s in range(R)], np.int64)
    sd, rd = oracle.packed_displs(cnt)
    srows, rrows = cnt.sum(axis=1), cnt.sum(axis=0)
    sends = [torch.empty((int(srows[s]), W), dtype=torch.bfloat16, device="cuda")
             for s in range(R)]
    recvs = [torch.empty((int(rrows[d]), W), dtype=torch.bfloat16, device="cuda")
             for d in range(R)]
    dc = lambda a: torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda()
    ar = coll.prepare(coll.allreduce, ins, outs)
    a2 = coll.prepare(coll.all_to_all_v, sends, dc(cnt), dc(sd), recvs, dc(rd), W)
    assert isinstance(ar, coll.Plan) and isinstance(a2, coll.Plan)
    for it in range(3):
        xs = [synth.gaussian(n, 0.02, 70000 + 100 * it + r, "bf16") for r in range(R)]
        ys = [synth.random_bits((int(srows[s]), W), 2, 71000 + 100 * it + s) for s in range(R)]
        for t, x in zip(ins, xs):
            t.copy_(dev(x))
        for t, y in zip(sends, ys):
            t.copy_(dev(y))
        ar()
        a2()
        torch.cuda.synchronize()
        want = oracle.allreduce(xs, "bf16")
        for r in range(R):
            assert bits_equal(host(outs[r]), want[r]), (it, r)
        want_a = oracle.all_to_all_v(ys, cnt, sd, rd, rrows, W)
        for d in range(R):
            assert bits_equal(host(recvs[d]).reshape(-1), want_a[d].reshape(-1)), (it, d)


def test_prepared_fused_moe_in_a_graph():
    R, E, T, K, H = 4, 32, 40, 4, 64
    say("prepared fused moe in a graph")
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
    plans = [coll.prepare(coll.moe_layout, id_d, E, sc, sdd, rdd, ec, pos, ws),
             coll.prepare(coll.moe_dispatch, x_d, pos, sc, sdd, rdd, recvs),
             coll.prepare(coll.moe_combine_recv, recvs, pos, sc, sdd, rdd, w_d, outs,
                          topk_ids=id_d)]

    def feed(it):
        ids, wts, xs = [], [], []
        for s in range(R):
            i, w = synth.zipf_routing(T, E, K, seed=72000 + 100 * it + s)
            ids.append(i)
            wts.append(w)
            xs.append(synth.gaussian((T, H), 1.0, 73000 + 100 * it + s, "bf16"))
            id_d[s].copy_(torch.from_numpy(i))
            w_d[s].copy_(torch.from_numpy(w))
            x_d[s].copy_(dev(xs[s]))
            outs[s].view(torch.int16).fill_(0x7FAB)
        torch.cuda.synchronize()
        return xs, ids, wts

    feed(0)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        for p in plans:
            p()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for p in plans:
            p()
    for it in range(1, 4):
        xs, ids, wts = feed(it)
        g.replay()
        torch.cuda.synchronize()
        want = oracle.moe_pipeline(xs, ids, wts, E)
        for r in range(R):
            assert bits_equal(host(outs[r]).reshape(-1), want["outs"][r].reshape(-1)), (it, r)
