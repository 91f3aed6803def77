"""GPU: exchanges whose tables name rows outside the buffers.

The count and displacement tables of an All-to-All-v live on the device, so
the host cannot check them; the kernels bound every block by the rows each
rank's buffer holds (the binding passes them).  A block that does not lie
wholly inside both of its buffers moves nothing and its receive rows keep
their contents; every other block must still equal the oracle's exchange,
and for the fused MoE pair the pairs whose slots fall in such a block add no
term ("Collective primitives tutorial", sections 8.2 and 8.4).  The same
tables run first under the CPU emulation with guard pages around every
buffer, which shows that no access leaves the buffers.
"""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import coll, synth
from gpu_util import bits_equal, dev, host, poison_like, say

pytestmark = pytest.mark.gpu

POISON = 0x7FAB          # poison_like's bf16 pattern


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    coll.lib()
    yield
    torch.cuda.synchronize()


def dc(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int64).reshape(-1)).cuda()


def bad_tables(counts, sd, rd, send_rows, recv_rows):
    """Five kinds of bad block: a count past the receive buffer, a negative
    send displacement, a receive displacement one row short of fitting, a
    count past the send buffer, a negative count."""
    R = counts.shape[0]
    c, s_, r_ = counts.copy(), sd.copy(), rd.copy()
    bad = set()
    picks = [(0, R - 1), (R - 1, 0), (R // 2, R // 2), (1 % R, (R - 2) % R), (R - 1, R - 1)]
    for i, (s, d) in enumerate(picks):
        if (s, d) in bad:
            continue
        if i == 0:
            c[s, d] = counts[s, d] + recv_rows[d]
        elif i == 1:
            s_[s, d] = -3
        elif i == 2:
            r_[d, s] = recv_rows[d] - counts[s, d] + 1
        elif i == 3:
            c[s, d] = send_rows[s] + 1
        else:
            c[s, d] = -5
        bad.add((s, d))
    return c, s_, r_, bad


@pytest.mark.parametrize("R,W,lo,hi,form", [
    (8, 8, 1, 300, "plain"),
    (4, 5, 1, 200, "plain"),                 # 10-byte rows: the chunk kernel
    (16, 8, 1, 100, "plain"),
    (8, 8192, 200, 330, "plain"),            # ~270 MiB of capacity: the one-pass grid
    (8, 8192, 150, 250, "descriptor form"),  # ~200 MiB of capacity: above the form's threshold
])
def test_blocks_outside_the_buffers_move_nothing(R, W, lo, hi, form):
    say("a2av bounded tables", R, W, form)
    g = np.random.default_rng(4000 + R + W)
    counts = g.integers(lo, hi, size=(R, R)).astype(np.int64)
    sd, rd = oracle.packed_displs(counts)
    send_rows = [int(counts[s].sum()) for s in range(R)]
    recv_rows = [int(counts[:, d].sum()) for d in range(R)]
    c, s_, r_, bad = bad_tables(counts, sd, rd, send_rows, recv_rows)
    xs = [synth.gaussian(send_rows[s] * W, 1.0, 4100 + s, "bf16") for s in range(R)]
    eff = counts.copy()
    for s, d in bad:
        eff[s, d] = 0
    want = oracle.all_to_all_v(xs, eff, sd, rd, np.array(recv_rows), W)
    sends = [dev(x) for x in xs]
    recvs = [poison_like(torch.empty(recv_rows[d] * W, dtype=torch.bfloat16, device="cuda"))
             for d in range(R)]
    kw = {}
    if form == "descriptor form":
        nbytes = coll.all_to_all_v_workspace_bytes(sends, recvs, W)
        assert nbytes > 0
        kw["workspace"] = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    coll.all_to_all_v(sends, dc(c), dc(s_), recvs, dc(r_), W, **kw)
    torch.cuda.synchronize()
    got = [host(r) for r in recvs]
    for s in range(R):
        for d in range(R):
            a, n = int(rd[d, s]) * W, int(counts[s, d]) * W
            if (s, d) in bad:
                assert np.all(got[d][a:a + n] == POISON), f"bad block {s}->{d} was written"
            else:
                assert bits_equal(got[d][a:a + n], want[d][a:a + n]), f"block {s}->{d}"
    # the reverse on the same tables skips the same blocks
    backs = [poison_like(t) for t in sends]
    kw = {}
    if form == "descriptor form":
        kw["workspace"] = torch.empty(coll.all_to_all_v_workspace_bytes(recvs, backs, W),
                                      dtype=torch.uint8, device="cuda")
    coll.all_to_all_v_reverse(recvs, dc(c), dc(s_), backs, dc(r_), W, **kw)
    torch.cuda.synchronize()
    for s in range(R):
        b = host(backs[s])
        for d in range(R):
            a, n = int(sd[s, d]) * W, int(counts[s, d]) * W
            if (s, d) in bad:
                assert np.all(b[a:a + n] == POISON), f"bad block {d}->{s} was returned"
            else:
                assert bits_equal(b[a:a + n], xs[s][a:a + n]), f"returned block {d}->{s}"


def test_fused_moe_skips_a_block_past_its_receive_buffer():
    R, E, T, K, H = 8, 256, 700, 8, 64
    say("fused MoE, a block past its receive buffer")
    ids, ws, xs = [], [], []
    for s in range(R):
        i, w = synth.zipf_routing(T, E, K, seed=5100 + s)
        ids.append(i)
        ws.append(w)
        xs.append(synth.gaussian((T, H), 1.0, 5000 + s, "bf16"))
    want = oracle.moe_pipeline(xs, ids, ws, E)
    lay = want["layout"]
    sc_h, sd_h, rd_h = (np.array(lay[k], np.int64) for k in ("sendcounts", "sdispls", "rdispls"))
    rrows = sc_h.sum(axis=0)
    cand = [(s, d) for s in range(R) for d in range(R) if sc_h[s, d] > 0]
    s0, d0 = cand[len(cand) // 2]
    bad_rd = rd_h.copy()
    bad_rd[d0, s0] = int(rrows[d0]) - int(sc_h[s0, d0]) + 1
    x_d = [dev(x) for x in xs]
    pos = [torch.from_numpy(p).cuda() for p in lay["pos"]]
    id_d = [torch.from_numpy(i).cuda() for i in ids]
    w_d = [torch.from_numpy(w).cuda() for w in ws]
    recvs = [poison_like(torch.empty((int(n), H), dtype=torch.bfloat16, device="cuda"))
             for n in rrows]
    coll.moe_dispatch(x_d, pos, dc(sc_h), dc(sd_h), dc(bad_rd), recvs)
    torch.cuda.synchronize()
    for d in range(R):
        got = host(recvs[d])
        for s in range(R):
            a, n = int(rd_h[d, s]), int(sc_h[s, d])
            if not n:
                continue
            if (s, d) == (s0, d0):
                assert np.all(got[a:a + n] == POISON), "the bad block was written"
            else:
                assert bits_equal(got[a:a + n], want["recvs"][d].reshape(-1, H)[a:a + n]), (s, d)
    # the combine reads the correct rows everywhere, yet must drop the pairs
    # whose slots lie in the bad block
    full = [dev(np.ascontiguousarray(want["recvs"][d].reshape(-1, H)[:int(rrows[d])]))
            for d in range(R)]
    outs = [poison_like(x) for x in x_d]
    coll.moe_combine_recv(full, pos, dc(sc_h), dc(sd_h), dc(bad_rd), w_d, outs, topk_ids=id_d)
    torch.cuda.synchronize()
    lo, hi = int(sd_h[s0, d0]), int(sd_h[s0, d0] + sc_h[s0, d0])
    pos_eff = [np.array(p) for p in lay["pos"]]
    pos_eff[s0] = np.where((pos_eff[s0] >= lo) & (pos_eff[s0] < hi), -1, pos_eff[s0]).astype(np.int32)
    expect = oracle.moe_combine(want["backs"], pos_eff, ws, H)
    for s in range(R):
        assert bits_equal(host(outs[s]), expect[s]), f"rank {s}"


@pytest.mark.parametrize("kind", ["negative count", "displacement past the buffer"])
@pytest.mark.parametrize("path", ["row descriptors", "table search"])
def test_expert_leaves_a_bad_block_as_it_is(kind, path):
    R, E, T, K, H = 8, 256, 700, 8, 64
    say("expert, a bad block", kind, path)
    ids, ws, xs = [], [], []
    for s in range(R):
        i, w = synth.zipf_routing(T, E, K, seed=5200 + s)
        ids.append(i)
        ws.append(w)
        xs.append(synth.gaussian((T, H), 1.0, 5300 + s, "bf16"))
    want = oracle.moe_pipeline(xs, ids, ws, E)
    lay = want["layout"]
    per = E // R
    ec_h = np.array(lay["expert_counts"], np.int32).reshape(R, E)
    rd_h = np.array(lay["rdispls"], np.int64)
    rrows = np.array(lay["sendcounts"], np.int64).sum(axis=0)
    blocks = [(s, d) for s in range(R) for d in range(R) if ec_h[s, d * per:(d + 1) * per].sum()]
    s0, d0 = blocks[len(blocks) // 2]
    n0 = int(ec_h[s0, d0 * per:(d0 + 1) * per].sum())
    ec2, rd2 = ec_h.copy(), rd_h.copy()
    if kind == "negative count":
        ec2[s0, d0 * per] = -1
    else:
        rd2[d0, s0] = int(rrows[d0]) - n0 + 1
    recv_h = [np.ascontiguousarray(want["recvs"][d].reshape(-1, H)[:int(rrows[d])])
              for d in range(R)]
    recvs = [dev(r) for r in recv_h]
    # a workspace for the row descriptors selects that path; one for the
    # table alone, the table search
    cap = int(rrows.sum()) if path == "row descriptors" else 0
    work = torch.empty(coll.moe_expert_workspace_bytes(R, E, cap), dtype=torch.uint8,
                       device="cuda")
    coll.moe_expert_scale(recvs, torch.from_numpy(ec2.reshape(-1)).cuda(), dc(rd2), E, H, work)
    torch.cuda.synchronize()
    for d in range(R):
        exp = want["ys"][d].reshape(-1, H)[:int(rrows[d])].copy()
        if d == d0:
            a = int(rd_h[d0, s0])
            exp[a:a + n0] = recv_h[d0][a:a + n0]
        assert bits_equal(host(recvs[d]), exp), f"rank {d}"
