"""GPU parity of the fused MoE path (coll_moe_dispatch, coll_moe_combine_recv)
against the oracle's unfused pipeline (layout -> permute -> All-to-All-v ->
test expert -> All-to-All-v back -> combine): the fused calls must give the
same receive buffers and the same outputs, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import coll, synth
from gpu_util import bits_equal, dev, host, poison_like, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    coll.lib()
    yield
    torch.cuda.synchronize()


def routing(R, E, T, K):
    ids, ws = [], []
    for s in range(R):
        i, w = synth.zipf_routing(T, E, K, seed=5100 + s)
        ids.append(i)
        ws.append(w)
    return ids, ws


def layout_gpu(id_d, E, T, K):
    R = len(id_d)
    sc = torch.empty((R * R,), dtype=torch.int64, device="cuda")
    sd, rd = torch.empty_like(sc), torch.empty_like(sc)
    ec = torch.empty((R * E,), dtype=torch.int32, device="cuda")
    pos = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in range(R)]
    work = torch.empty(max(coll.moe_workspace_bytes(R, T, K, E), 256), dtype=torch.uint8,
                       device="cuda")
    coll.moe_layout(id_d, E, sc, sd, rd, ec, pos, work)
    torch.cuda.synchronize()
    return sc, sd, rd, ec, pos


def fused_gpu(xs, ids, ws, E, exact_recv=True):
    """Layout, fused dispatch into poisoned receive buffers, fused combine with
    the test expert inline; returns host copies."""
    R = len(xs)
    T, H = xs[0].shape
    K = ids[0].shape[1]
    x_d = [dev(x) for x in xs]
    id_d = [torch.from_numpy(i).cuda() for i in ids]
    w_d = [torch.from_numpy(w).cuda() for w in ws]
    sc, sd, rd, ec, pos = layout_gpu(id_d, E, T, K)
    rows = host(sc).reshape(R, R).sum(axis=0)
    # ranks that receive nothing get an empty tensor (a NULL pointer)
    recvs = [poison_like(torch.empty((int(n), H), dtype=torch.bfloat16, device="cuda"))
             for n in rows]
    coll.moe_dispatch(x_d, pos, sc, sd, rd, recvs)
    torch.cuda.synchronize()
    recv_h = [host(r).copy() for r in recvs]
    outs = [poison_like(x) for x in x_d]
    coll.moe_combine_recv(recvs, pos, sc, sd, rd, w_d, outs, topk_ids=id_d)
    torch.cuda.synchronize()
    return dict(recvs=recv_h, recvs_after=[host(r) for r in recvs],
                outs=[host(o) for o in outs], dev=(recvs, pos, sc, sd, rd, ec, w_d, x_d))


@pytest.mark.parametrize("R,E,T,K,H", [
    (2, 4, 2, 1, 8),
    (1, 8, 100, 2, 16),
    (4, 16, 333, 3, 24),
    (8, 256, 700, 8, 64),
    (8, 256, 64, 8, 7168),
    (2, 8, 50, 2, 5),         # 10-byte rows: scalar element paths
    (3, 12, 1500, 4, 16),
    (16, 1024, 200, 8, 8),
    (2, 16, 40, 10, 16),      # top-10: a second, partial chunk of slots
    (2, 16, 40, 10, 5),
])
def test_fused_moe_matches_unfused_oracle(R, E, T, K, H):
    say("moe fused", R, E, T, K, H)
    ids, ws = routing(R, E, T, K)
    xs = [synth.gaussian((T, H), 1.0, 5000 + s, "bf16") for s in range(R)]
    want = oracle.moe_pipeline(xs, ids, ws, E)
    got = fused_gpu(xs, ids, ws, E)
    lay = want["layout"]
    for d in range(R):
        n = int(lay["sendcounts"][:, d].sum()) * H
        assert got["recvs"][d].size == n
        assert bits_equal(got["recvs"][d].reshape(-1), want["recvs"][d].reshape(-1)[:n]), d
        # the fused combine only reads the receive buffers
        assert bits_equal(got["recvs_after"][d], got["recvs"][d]), d
    for s in range(R):
        assert bits_equal(got["outs"][s].reshape(-1), want["outs"][s].reshape(-1)), s
    # without topk_ids the combine uses the rows as they are: run the test
    # expert in place first and the outputs must not change
    recvs, pos, sc, sd, rd, ec, w_d, x_d = got["dev"]
    ews = torch.empty(coll.moe_expert_workspace_bytes(R, E), dtype=torch.uint8, device="cuda")
    coll.moe_expert_scale(recvs, ec, rd, E, H, ews)
    outs = [poison_like(x) for x in x_d]
    coll.moe_combine_recv(recvs, pos, sc, sd, rd, w_d, outs)
    torch.cuda.synchronize()
    for s in range(R):
        assert bits_equal(host(outs[s]).reshape(-1), want["outs"][s].reshape(-1)), s


@pytest.mark.parametrize("R,E,T,K,H", [
    (4, 16, 333, 3, 24),
    (8, 256, 64, 8, 7168),
    (2, 16, 40, 10, 5),
])
def test_fused_moe_with_bad_expert_ids(R, E, T, K, H):
    """Pairs whose id names no expert are skipped by the fused dispatch (no
    row) and the fused combine (no term): receive rows and every output match
    the oracle on the same ids."""
    from test_gpu_parity import plant_bad_ids
    say("moe fused bad ids", R, E, T, K, H)
    ids, ws = routing(R, E, T, K)
    ids = plant_bad_ids(ids, E, 91)
    xs = [synth.gaussian((T, H), 1.0, 5600 + s, "bf16") for s in range(R)]
    want = oracle.moe_pipeline(xs, ids, ws, E)
    got = fused_gpu(xs, ids, ws, E)
    lay = want["layout"]
    for d in range(R):
        n = int(lay["sendcounts"][:, d].sum()) * H
        assert got["recvs"][d].size == n
        assert bits_equal(got["recvs"][d].reshape(-1), want["recvs"][d].reshape(-1)[:n]), d
    for s in range(R):
        assert bits_equal(got["outs"][s].reshape(-1), want["outs"][s].reshape(-1)), s


def test_fused_moe_ranks_that_receive_nothing():
    """Every token routes to experts of ranks 0 and 1 only: ranks 2 and 3 get
    empty (NULL) receive buffers and no write."""
    R, E, T, K, H = 4, 8, 300, 2, 24
    say("moe fused empty ranks")
    g = np.random.default_rng(3)
    ids = []
    for s in range(R):
        a = np.stack([g.permutation(4)[:K] for _ in range(T)]).astype(np.int32)
        ids.append(a)
    ws = [np.full((T, K), 0.5, np.float32) for _ in range(R)]
    xs = [synth.gaussian((T, H), 1.0, 700 + s, "bf16") for s in range(R)]
    want = oracle.moe_pipeline(xs, ids, ws, E)
    got = fused_gpu(xs, ids, ws, E)
    assert got["recvs"][2].size == 0 and got["recvs"][3].size == 0
    for s in range(R):
        assert bits_equal(got["outs"][s].reshape(-1), want["outs"][s].reshape(-1)), s


def test_fused_moe_full_size_sampled():
    """8 ranks x 4096 tokens x hidden 7168, 256 experts, top-8 Zipf(1.2): the
    fused dispatch's receive buffers equal permute + All-to-All-v's bit for
    bit (whole buffers), and the fused outputs of 64 sampled tokens per rank
    equal the oracle pipeline run on those tokens."""
    R, E, T, K, H = 8, 256, 4096, 8, 7168
    say("moe fused full size")
    ids, ws = routing(R, E, T, K)
    xs = [synth.gaussian((T, H), 1.0, 5000 + s, "bf16") for s in range(R)]
    got = fused_gpu(xs, ids, ws, E)
    recvs, pos, sc, sd, rd, ec, w_d, x_d = got["dev"]
    sends = [torch.empty((T * K, H), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    coll.moe_permute(x_d, pos, sends)
    recvs2 = [poison_like(r) for r in recvs]
    coll.all_to_all_v(sends, sc, sd, recvs2, rd, H)
    torch.cuda.synchronize()
    for d in range(R):
        assert torch.equal(recvs2[d].view(torch.int16), recvs[d].view(torch.int16)), d
    del sends, recvs2
    g = np.random.default_rng(78)
    pick = [np.sort(g.choice(T, 64, replace=False)) for _ in range(R)]
    sub = oracle.moe_pipeline([np.ascontiguousarray(xs[s][pick[s]]) for s in range(R)],
                              [np.ascontiguousarray(ids[s][pick[s]]) for s in range(R)],
                              [np.ascontiguousarray(ws[s][pick[s]]) for s in range(R)], E)
    for s in range(R):
        assert bits_equal(got["outs"][s][pick[s]], sub["outs"][s]), s
