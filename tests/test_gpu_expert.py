"""GPU parity of the test expert (coll_moe_expert_scale) against the oracle,
through the C ABI, on synthetic expert counts and receive displacements.

The cases cover:
- rows of one 16-byte unit, so a tile spans many entries;
- R = 16 with E = 1024, which needs three search levels over 16384 entries;
- the element-wise path (rows of 5 bf16; a receive buffer 2 bytes off
  16-byte alignment);
- empty experts, all-zero counts and gaps between the source blocks;
- launch capacities that are exact, unknown (0: resident grid), too large
  and too small;
- both paths: the row-descriptor path (a workspace sized for the capacity;
  16-byte rows, R * E <= 8192) and the table-search path (a workspace of the
  tables alone, or rows the descriptor path does not take).
Every output is compared in full and must be bit-identical.
"""
import ctypes

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


def make_case(R, E, H, maxc, zero_frac, gap, seed):
    g = np.random.default_rng(seed)
    per = E // R
    ec = g.integers(0, maxc + 1, size=R * E).astype(np.int32)
    ec[g.random(R * E) < zero_frac] = 0
    rows_sd = ec.reshape(R, R, per).sum(axis=2).astype(np.int64)    # [s, d]
    rd = np.zeros((R, R), np.int64)                                 # [d, s]
    for d in range(R):
        off = 0
        for s in range(R):
            rd[d, s] = off
            off += rows_sd[s, d] + gap
    nrows = [int((rd[d] + rows_sd[:, d]).max()) for d in range(R)]
    recvs = [synth.gaussian((max(n, 1), H), 1.0, 700 + d, "bf16") for d, n in enumerate(nrows)]
    return ec, rd, recvs, int(rows_sd.sum())


CASES = [
    # R, E, H, maxc, zero_frac, gap, capacity, shift
    (2, 4, 8, 5, 0.3, 0, "exact", 0),
    (2, 4, 8, 5, 0.3, 0, "zero", 0),
    (2, 4, 8, 5, 0.3, 0, "big", 0),
    (2, 4, 8, 5, 0.3, 0, "small", 0),
    (4, 16, 24, 5, 0.3, 3, "exact", 0),
    (8, 256, 64, 12, 0.3, 0, "exact", 0),
    (8, 256, 8, 3, 0.3, 0, "small", 0),
    (8, 256, 7168, 12, 0.2, 0, "exact", 0),
    (3, 12, 5, 5, 0.3, 0, "exact", 0),
    (3, 12, 5, 5, 0.3, 0, "zero", 0),
    (4, 16, 16, 5, 0.3, 0, "exact", 1),
    (4, 8, 8, 5, 1.0, 0, "exact", 0),
    (1, 1, 8, 40, 0.0, 0, "exact", 0),
    (16, 1024, 8, 1, 0.7, 0, "exact", 0),
    (16, 1024, 8, 2, 0.5, 0, "zero", 0),
    (16, 1024, 64, 3, 0.2, 5, "big", 0),
    (5, 5, 1000, 3, 0.3, 0, "exact", 0),
    (8, 256, 520, 3, 0.3, 0, "exact", 0),       # 65 units per row: a partial last segment
    (8, 256, 520, 3, 0.3, 2, "small", 0),
    (8, 1024, 16, 2, 0.5, 0, "exact", 0),       # 8192 entries: the largest LDS table
    (16, 512, 16, 2, 0.5, 1, "small", 0),
]


@pytest.mark.parametrize("ws_kind", ["rows", "table"])
@pytest.mark.parametrize("R,E,H,maxc,zero_frac,gap,cap,shift", CASES)
def test_expert_matches_oracle(R, E, H, maxc, zero_frac, gap, cap, shift, ws_kind):
    say("expert", R, E, H, maxc, zero_frac, gap, cap, shift, ws_kind)
    ec, rd, recvs, total = make_case(R, E, H, maxc, zero_frac, gap, seed=R * 1000 + E + H)
    want = oracle.moe_expert_scale([r.copy() for r in recvs], ec, rd.reshape(-1), E, H)
    # a shifted buffer starts 2 bytes past a 16-byte boundary
    bufs = [dev(np.concatenate([np.zeros(shift, np.uint16), r.reshape(-1)])) for r in recvs]
    ptrs = (ctypes.c_void_p * R)(*[b.data_ptr() + 2 * shift for b in bufs])
    ec_d, rd_d = dev(ec), dev(rd.reshape(-1))
    capv = {"exact": total, "zero": 0, "big": 3 * total + 17, "small": max(total // 3, 1)}[cap]
    wsb = coll.moe_expert_workspace_bytes(R, E, capv if ws_kind == "rows" else 0)
    ws = torch.full((wsb,), 0xCD, dtype=torch.uint8, device="cuda")   # contents never read
    rows = (ctypes.c_int64 * R)(*[r.size // H for r in recvs])
    rc = coll.lib().coll_moe_expert_scale(R, ptrs, ec_d.data_ptr(), rd_d.data_ptr(), E, H, 0,
                                          capv, rows, ws.data_ptr(), wsb, None)
    torch.cuda.synchronize()
    assert rc == 0
    for d in range(R):
        got = host(bufs[d])[shift:]
        assert bits_equal(got, want[d].reshape(-1)), d


def test_expert_repeated_calls_share_a_workspace():
    """The table is rebuilt on every call: a second, smaller call with the
    same workspace sees nothing of the first."""
    R, E = 8, 64
    wsb = coll.moe_expert_workspace_bytes(R, E, 1 << 16)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    for seed, maxc, H in ((1, 30, 64), (2, 3, 8)):
        say("expert repeated", seed, maxc, H)
        ec, rd, recvs, _ = make_case(R, E, H, maxc, 0.3, 0, seed)
        want = oracle.moe_expert_scale([r.copy() for r in recvs], ec, rd.reshape(-1), E, H)
        bufs = [dev(r) for r in recvs]
        coll.moe_expert_scale(bufs, dev(ec), dev(rd.reshape(-1)), E, H, ws)
        torch.cuda.synchronize()
        for d in range(R):
            assert bits_equal(host(bufs[d]), want[d].reshape(bufs[d].shape)), d


def test_expert_rejects_a_small_workspace():
    R, E, H = 2, 4, 8
    ec, rd, recvs, _ = make_case(R, E, H, 3, 0.0, 0, 3)
    bufs = [dev(r) for r in recvs]
    small = torch.empty(coll.moe_expert_workspace_bytes(R, E, 0) - 1, dtype=torch.uint8,
                        device="cuda")
    with pytest.raises(coll.CollError):
        coll.moe_expert_scale(bufs, dev(ec), dev(rd.reshape(-1)), E, H, small)


def test_expert_moe_full_size_paths_agree():
    """8 ranks x 4096 tokens x top-8 of 256 experts (Zipf routing), rows of
    7168 bf16 (3.5 GiB in place): the row-descriptor path and the
    table-search path give the same bits, and sampled rows match the oracle's
    formula row by row."""
    R, E, T, K, H = 8, 256, 4096, 8, 7168
    say("expert full size")
    ids = [synth.zipf_routing(T, E, K, seed=5100 + s)[0] for s in range(R)]
    lay = oracle.moe_layout(ids, E)
    ec, rd = lay["expert_counts"], lay["rdispls"]
    rows = lay["sendcounts"].sum(axis=0)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    a = [torch.randn((int(n), H), generator=g, device="cuda").to(torch.bfloat16) for n in rows]
    b = [t.clone() for t in a]
    x0 = [t.clone() for t in a]
    cap = int(rows.sum())
    ws_rows = torch.empty(coll.moe_expert_workspace_bytes(R, E, cap), dtype=torch.uint8,
                          device="cuda")
    ws_tab = torch.empty(coll.moe_expert_workspace_bytes(R, E, 0), dtype=torch.uint8,
                         device="cuda")
    ec_d, rd_d = dev(ec.reshape(-1)), dev(rd.reshape(-1))
    coll.moe_expert_scale(a, ec_d, rd_d, E, H, ws_rows)
    coll.moe_expert_scale(b, ec_d, rd_d, E, H, ws_tab)
    torch.cuda.synchronize()
    for d in range(R):
        assert torch.equal(a[d].view(torch.int16), b[d].view(torch.int16)), d
    # sampled rows against the oracle on just those rows: rank d's rows are,
    # for s ascending from rdispls[d][s], its experts' rows in expert order
    per = E // R
    rng = np.random.default_rng(3)
    for d in rng.choice(R, 3, replace=False):
        e_of = np.concatenate([np.repeat(np.arange(d * per, (d + 1) * per),
                                         ec.reshape(R, E)[s, d * per:(d + 1) * per])
                               for s in range(R)])
        for j in rng.choice(int(rows[d]), 16, replace=False):
            xr = host(x0[d][j]).reshape(1, H)
            one = np.zeros((1, E), np.int32)
            one[0, e_of[j]] = 1
            want = oracle.moe_expert_scale([xr.copy()], one.reshape(-1), np.zeros(1, np.int64),
                                           E, H)[0]
            assert bits_equal(host(a[d][j]).reshape(-1), want.reshape(-1)), (d, j)


# the cases the row-descriptor path takes: 16-byte rows, a nonzero capacity
# (so not the all-empty one), aligned buffers, at most 8192 table entries
SPLIT_CASES = [c for c in CASES if c[2] % 8 == 0 and c[6] != "zero" and c[4] < 1.0
               and c[7] == 0 and c[0] * c[1] <= 8192]


@pytest.mark.parametrize("R,E,H,maxc,zero_frac,gap,cap,shift", SPLIT_CASES)
def test_expert_in_two_calls_matches_oracle(R, E, H, maxc, zero_frac, gap, cap, shift):
    """The row-descriptor path as coll_moe_expert_scale_build on a second
    stream, issued before the rows are written, then
    coll_moe_expert_scale_apply once both are done: the same bits as the
    oracle."""
    say("expert build/apply", R, E, H, maxc, zero_frac, gap, cap)
    ec, rd, recvs, total = make_case(R, E, H, maxc, zero_frac, gap, seed=R * 1000 + E + H)
    want = oracle.moe_expert_scale([r.copy() for r in recvs], ec, rd.reshape(-1), E, H)
    bufs = [torch.empty(r.shape, dtype=torch.bfloat16, device="cuda") for r in recvs]
    ptrs = (ctypes.c_void_p * R)(*[b.data_ptr() for b in bufs])
    ec_d, rd_d = dev(ec), dev(rd.reshape(-1))
    capv = {"exact": total, "big": 3 * total + 17, "small": max(total // 3, 1)}[cap]
    wsb = coll.moe_expert_workspace_bytes(R, E, capv)
    ws = torch.full((wsb,), 0xCD, dtype=torch.uint8, device="cuda")
    rows = (ctypes.c_int64 * R)(*[r.size // H for r in recvs])
    L = coll.lib()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rc = L.coll_moe_expert_scale_build(R, ptrs, ec_d.data_ptr(), rd_d.data_ptr(), E, H, 0,
                                           capv, rows, ws.data_ptr(), wsb, side.cuda_stream)
    built = torch.cuda.Event()
    built.record(side)
    for b, r in zip(bufs, recvs):               # the rows arrive after the build
        b.copy_(dev(r))
    torch.cuda.current_stream().wait_event(built)
    rc2 = L.coll_moe_expert_scale_apply(R, ptrs, E, H, 0, capv, ws.data_ptr(), wsb,
                                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0 and rc2 == 0
    for d in range(R):
        assert bits_equal(host(bufs[d]).reshape(-1), want[d].reshape(-1)), d


def test_expert_split_refuses_the_table_search():
    """Without a workspace for the descriptors the two-call form does not
    apply: the binding refuses, and the C entry points return
    COLL_ERR_UNSUPPORTED without launching."""
    R, E, H = 2, 4, 8
    ec, rd, recvs, total = make_case(R, E, H, 3, 0.0, 0, 3)
    bufs = [dev(r) for r in recvs]
    small = torch.empty(coll.moe_expert_workspace_bytes(R, E, 0), dtype=torch.uint8,
                        device="cuda")
    with pytest.raises(ValueError):
        coll.moe_expert_scale_build(bufs, dev(ec), dev(rd.reshape(-1)), E, H, small)
    with pytest.raises(ValueError):
        coll.moe_expert_scale_apply(bufs, E, H, small)
    ptrs = (ctypes.c_void_p * R)(*[b.data_ptr() for b in bufs])
    assert coll.lib().coll_moe_expert_scale_apply(R, ptrs, E, H, 0, 0, small.data_ptr(),
                                                  small.numel(), None) == -2
