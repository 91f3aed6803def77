"""Full-size parity on the MoE dispatch/combine workload -- 8 ranks x 4096
tokens x hidden 7168 bf16, 256 experts, top-8 of a Zipf(1.2) routing -- with
every output element of every stage compared against the oracle.

The oracle runs the whole exchange once (tutorial section 8.4: layout,
permute, All-to-All-v, test expert, the reverse All-to-All-v, combine; about
20 s of CPU on the host that drives the GPU).  Each stage on the GPU is then fed the
oracle's output of the stage before it and its own output, poison-filled
first, is compared in full: the layout tables and slots; the permute's send
buffers; the exchange in both forms (the plain one-pass grid and the
descriptor form with a workspace); the test expert; the reverse exchange read
from the forward tables; the combine; and the fused dispatch and fused
combine.  No sampling: an unwritten or misplaced tile fails.
"""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import coll, synth
from gpu_util import bits_equal, dev, host, poison_like, say

pytestmark = pytest.mark.gpu

R, E, T, K, H = 8, 256, 4096, 8, 7168


@pytest.fixture(scope="module")
def ref():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    coll.lib()
    say("full-size MoE: oracle pipeline (host)")
    ids, ws = [], []
    for s in range(R):
        i, w = synth.zipf_routing(T, E, K, seed=5100 + s)
        ids.append(i)
        ws.append(w)
    xs = [synth.gaussian((T, H), 1.0, 5000 + s, "bf16") for s in range(R)]
    want = oracle.moe_pipeline(xs, ids, ws, E)
    lay = want["layout"]
    tabs = {k: torch.from_numpy(np.ascontiguousarray(lay[k]).reshape(-1)).cuda()
            for k in ("sendcounts", "sdispls", "rdispls", "expert_counts")}
    rows = [int(n) for n in lay["sendcounts"].sum(axis=0)]
    yield dict(ids=ids, ws=ws, xs=xs, want=want, lay=lay, tabs=tabs, rows=rows)
    torch.cuda.synchronize()


def _recv_bufs(rows):
    return [poison_like(torch.empty((n, H), dtype=torch.bfloat16, device="cuda")) for n in rows]


def _upload_rows(arrs, rows):
    return [dev(np.ascontiguousarray(a.reshape(-1)[:n * H]).reshape(n, H)) for a, n in zip(arrs, rows)]


def _check_rows(got, want, rows, what):
    for d, n in enumerate(rows):
        assert bits_equal(host(got[d]).reshape(-1), want[d].reshape(-1)[:n * H]), f"{what} rank {d}"


def test_layout(ref):
    say("full-size layout")
    ids = [torch.from_numpy(i).cuda() for i in ref["ids"]]
    sc = torch.full((R * R,), -7, dtype=torch.int64, device="cuda")
    sd, rd = torch.full_like(sc, -7), torch.full_like(sc, -7)
    ec = torch.full((R * E,), -7, dtype=torch.int32, device="cuda")
    pos = [torch.full((T, K), -7, dtype=torch.int32, device="cuda") for _ in range(R)]
    work = torch.empty(coll.moe_workspace_bytes(R, T, K, E), dtype=torch.uint8, device="cuda")
    coll.moe_layout(ids, E, sc, sd, rd, ec, pos, work)
    torch.cuda.synchronize()
    lay = ref["lay"]
    assert np.array_equal(host(sc).reshape(R, R), lay["sendcounts"])
    assert np.array_equal(host(sd).reshape(R, R), lay["sdispls"])
    assert np.array_equal(host(rd).reshape(R, R), lay["rdispls"])
    assert np.array_equal(host(ec).reshape(R, E), lay["expert_counts"])
    for s in range(R):
        assert np.array_equal(host(pos[s]), lay["pos"][s])


def test_permute(ref):
    say("full-size permute")
    x = [dev(a) for a in ref["xs"]]
    pos = [torch.from_numpy(p).cuda() for p in ref["lay"]["pos"]]
    sends = [poison_like(torch.empty((T * K, H), dtype=torch.bfloat16, device="cuda"))
             for _ in range(R)]
    coll.moe_permute(x, pos, sends)
    torch.cuda.synchronize()
    for s in range(R):
        assert bits_equal(host(sends[s]), ref["want"]["sends"][s]), f"rank {s}"


@pytest.mark.parametrize("form", ["plain one-pass grid", "descriptor form"])
def test_dispatch_exchange(ref, form):
    say("full-size A2A-v", form)
    tb = ref["tabs"]
    sends = [dev(a) for a in ref["want"]["sends"]]
    recvs = _recv_bufs(ref["rows"])
    kw = {}
    if form == "descriptor form":
        nbytes = coll.all_to_all_v_workspace_bytes(sends, recvs, H)
        assert nbytes > 0
        kw["workspace"] = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    coll.all_to_all_v(sends, tb["sendcounts"], tb["sdispls"], recvs, tb["rdispls"], H, **kw)
    torch.cuda.synchronize()
    _check_rows(recvs, ref["want"]["recvs"], ref["rows"], form)


def test_expert(ref):
    say("full-size test expert")
    tb = ref["tabs"]
    recvs = _upload_rows(ref["want"]["recvs"], ref["rows"])
    ews = torch.empty(coll.moe_expert_workspace_bytes(R, E, sum(ref["rows"])), dtype=torch.uint8,
                      device="cuda")
    coll.moe_expert_scale(recvs, tb["expert_counts"], tb["rdispls"], E, H, ews)
    torch.cuda.synchronize()
    _check_rows(recvs, ref["want"]["ys"], ref["rows"], "expert")


@pytest.mark.parametrize("form", ["plain", "descriptor form"])
def test_reverse_exchange(ref, form):
    """The combine's exchange: the reverse of the dispatch, from its tables."""
    say("full-size reverse A2A-v", form)
    tb = ref["tabs"]
    ys = _upload_rows(ref["want"]["ys"], ref["rows"])
    backs = [poison_like(torch.empty((T * K, H), dtype=torch.bfloat16, device="cuda"))
             for _ in range(R)]
    kw = {}
    if form == "descriptor form":
        kw["workspace"] = torch.empty(coll.all_to_all_v_workspace_bytes(ys, backs, H),
                                      dtype=torch.uint8, device="cuda")
    coll.all_to_all_v_reverse(ys, tb["sendcounts"], tb["sdispls"], backs, tb["rdispls"], H, **kw)
    torch.cuda.synchronize()
    for s in range(R):
        assert bits_equal(host(backs[s]).reshape(-1), ref["want"]["backs"][s].reshape(-1)), s


def test_combine(ref):
    say("full-size combine")
    backs = [dev(b.reshape(T * K, H)) for b in ref["want"]["backs"]]
    pos = [torch.from_numpy(p).cuda() for p in ref["lay"]["pos"]]
    w = [torch.from_numpy(a).cuda() for a in ref["ws"]]
    outs = [poison_like(torch.empty((T, H), dtype=torch.bfloat16, device="cuda"))
            for _ in range(R)]
    coll.moe_combine(backs, pos, w, outs)
    torch.cuda.synchronize()
    for s in range(R):
        assert bits_equal(host(outs[s]), ref["want"]["outs"][s]), s


def test_fused_dispatch_and_combine(ref):
    say("full-size fused dispatch / combine")
    tb = ref["tabs"]
    x = [dev(a) for a in ref["xs"]]
    pos = [torch.from_numpy(p).cuda() for p in ref["lay"]["pos"]]
    recvs = _recv_bufs(ref["rows"])
    coll.moe_dispatch(x, pos, tb["sendcounts"], tb["sdispls"], tb["rdispls"], recvs)
    torch.cuda.synchronize()
    _check_rows(recvs, ref["want"]["recvs"], ref["rows"], "fused dispatch")
    w = [torch.from_numpy(a).cuda() for a in ref["ws"]]
    ids = [torch.from_numpy(i).cuda() for i in ref["ids"]]
    outs = [poison_like(torch.empty((T, H), dtype=torch.bfloat16, device="cuda"))
            for _ in range(R)]
    coll.moe_combine_recv(recvs, pos, tb["sendcounts"], tb["sdispls"], tb["rdispls"], w, outs,
                          topk_ids=ids)
    torch.cuda.synchronize()
    for s in range(R):
        assert bits_equal(host(outs[s]), ref["want"]["outs"][s]), f"fused combine rank {s}"
