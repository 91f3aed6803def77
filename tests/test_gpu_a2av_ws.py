"""All-to-All-v in its descriptor form (coll_all_to_all_v_ws): the same
exchange as coll_all_to_all_v, checked against the oracle and against the
plain form bit for bit.

The form runs from 192 MiB of receive capacity up (the default threshold);
the capacity only sizes the launch, so small exchanges are sent through it
with a capacity bound at the threshold.  Cases beyond the random-count
parity tests (which run both forms):
- rows received beyond the capacity (262 MB exchanges against a 192 MiB
  bound: the tiles past the descriptors find their blocks in the table);
- gapped receive layouts, all-empty counts;
- the MoE exchange at full size (8 x 4096 x top-8, rows of 7168 bf16),
  compared with the plain form;
- rows that are not whole 16-byte units, buffers off 16-byte alignment,
  and capacities below the threshold: the plain form runs and the workspace
  is untouched;
- HIP-graph capture and replay.
"""
import ctypes

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


def dc(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int64).reshape(-1)).cuda()


def case(R, W, counts, gap=0, seed=0):
    sd, rd = oracle.packed_displs(counts)
    if gap:
        rd = rd + gap * np.arange(R, dtype=np.int64)[None, :]
    send_rows = counts.sum(axis=1)
    recv_rows = (rd + counts.T).max(axis=1)
    xs = [synth.random_bits(max(int(send_rows[s]), 1) * W, 2, 8100 + 31 * seed + s)
          for s in range(R)]
    sends = [dev(x) for x in xs]
    recvs = [poison_like(torch.empty(max(int(recv_rows[d]), 1) * W, dtype=torch.bfloat16,
                                     device="cuda")) for d in range(R)]
    init = [host(r).copy() for r in recvs]
    want = oracle.all_to_all_v([x[:int(send_rows[s]) * W] for s, x in enumerate(xs)], counts,
                               sd, rd, [max(int(v), 1) for v in recv_rows], W,
                               recvs=[a.copy() for a in init])
    return sends, recvs, want, sd, rd


DESC_MIN_BYTES = 192 << 20


def desc_rows(row_bytes):
    """Smallest receive capacity (rows) that takes the descriptor form."""
    return -(-DESC_MIN_BYTES // row_bytes)


def rows_of(bufs, W):
    """Rows of W bf16 each buffer holds, as the C ABI's host int64 array."""
    return (ctypes.c_int64 * len(bufs))(*[t.numel() // W for t in bufs])


def call_ws(R, sends, counts, sd, recvs, rd, W, capacity):
    """coll_all_to_all_v_ws through the C ABI with an explicit capacity."""
    L = coll.lib()
    need = L.coll_all_to_all_v_workspace_bytes(R, capacity, W, 0)
    ws = torch.full((max(need, 256),), 0xCD, dtype=torch.uint8, device="cuda")
    keep = (dc(counts), dc(sd), dc(rd))
    st = torch.cuda.current_stream().cuda_stream
    rc = L.coll_all_to_all_v_ws(R, (ctypes.c_void_p * R)(*[t.data_ptr() for t in sends]),
                                keep[0].data_ptr(), keep[1].data_ptr(),
                                (ctypes.c_void_p * R)(*[t.data_ptr() for t in recvs]),
                                keep[2].data_ptr(), W, 0, capacity, rows_of(sends, W),
                                rows_of(recvs, W), ws.data_ptr(), ws.numel(), st)
    torch.cuda.synchronize()
    return rc


@pytest.mark.parametrize("R,W", [(8, 8), (16, 64)])
def test_rows_beyond_the_capacity(R, W):
    """About 1.3x the rows of a capacity at the threshold (262 MB moved)."""
    say("a2av ws rows beyond capacity", R, W)
    cap = desc_rows(W * 2)
    g = np.random.default_rng(R * 7 + W)
    counts = g.integers(0, 2 * (16 * cap // 10) // (R * R), size=(R, R)).astype(np.int64)
    counts[g.random((R, R)) < 0.2] = 0
    assert int(counts.sum()) > cap + 1024              # tiles past the last descriptor
    sends, recvs, want, sd, rd = case(R, W, counts, seed=R)
    assert call_ws(R, sends, counts, sd, recvs, rd, W, cap) == 0
    for d in range(R):
        assert bits_equal(host(recvs[d]), want[d]), d


@pytest.mark.parametrize("gap,zero", [(3, False), (0, True), (5, False)])
def test_gapped_and_empty(gap, zero):
    R, W = 4, 8
    say("a2av ws gapped/empty", gap, zero)
    counts = (np.zeros((R, R), np.int64) if zero else
              np.array([[3, 0, 2, 1], [1, 1, 1, 1], [0, 0, 0, 7], [2, 5, 0, 0]], np.int64) * 40)
    sends, recvs, want, sd, rd = case(R, W, counts, gap=gap, seed=gap)
    cap = max(sum(t.numel() // W for t in recvs), desc_rows(W * 2))
    assert call_ws(R, sends, counts, sd, recvs, rd, W, cap) == 0
    for d in range(R):
        assert bits_equal(host(recvs[d]), want[d]), d


def test_capacity_below_the_threshold_uses_the_plain_form():
    R, W = 8, 64
    say("a2av ws below threshold")
    g = np.random.default_rng(4)
    counts = g.integers(0, 60, size=(R, R)).astype(np.int64)
    sends, recvs, want, sd, rd = case(R, W, counts, seed=4)
    assert coll.all_to_all_v_workspace_bytes(sends, recvs, W) == 0
    assert coll.all_to_all_v_workspace_bytes(sends, recvs, W, capacity=desc_rows(128)) > 0
    ws = torch.full((256,), 0xCD, dtype=torch.uint8, device="cuda")
    coll.all_to_all_v(sends, dc(counts), dc(sd), recvs, dc(rd), W, workspace=ws)
    torch.cuda.synchronize()
    for d in range(R):
        assert bits_equal(host(recvs[d]), want[d]), d
    assert bool((ws == 0xCD).all())               # untouched


def test_rows_not_whole_units_use_the_plain_form():
    R, W = 4, 3                                   # 6-byte rows
    say("a2av ws fallback")
    g = np.random.default_rng(2)
    counts = g.integers(0, 50, size=(R, R)).astype(np.int64)
    sends, recvs, want, sd, rd = case(R, W, counts, seed=2)
    assert coll.all_to_all_v_workspace_bytes(sends, recvs, W) == 0
    ws = torch.full((256,), 0xCD, dtype=torch.uint8, device="cuda")
    coll.all_to_all_v(sends, dc(counts), dc(sd), recvs, dc(rd), W, workspace=ws)
    torch.cuda.synchronize()
    for d in range(R):
        assert bits_equal(host(recvs[d]), want[d]), d
    assert bool((ws == 0xCD).all())               # untouched


def test_misaligned_buffers_use_the_plain_form():
    """16-byte rows, a capacity above the threshold, but a receive buffer 8
    bytes off 16-byte alignment: the plain form runs (the descriptors address
    whole 16-byte units) and the workspace is not touched."""
    R, W = 4, 8
    say("a2av ws misaligned")
    g = np.random.default_rng(6)
    counts = g.integers(0, 50, size=(R, R)).astype(np.int64)
    sends, recvs, want, sd, rd = case(R, W, counts, seed=6)
    shifted = []
    for r in recvs:                                   # same contents, 8 bytes further on
        big = torch.empty(r.numel() + 4, dtype=torch.bfloat16, device="cuda")
        big[4:].copy_(r)
        shifted.append(big)
    cap = desc_rows(W * 2)
    need = coll.lib().coll_all_to_all_v_workspace_bytes(R, cap, W, 0)
    assert need > 0
    ws = torch.full((need,), 0xCD, dtype=torch.uint8, device="cuda")
    keep = (dc(counts), dc(sd), dc(rd))
    rc = coll.lib().coll_all_to_all_v_ws(
        R, (ctypes.c_void_p * R)(*[t.data_ptr() for t in sends]), keep[0].data_ptr(),
        keep[1].data_ptr(), (ctypes.c_void_p * R)(*[t.data_ptr() + 8 for t in shifted]),
        keep[2].data_ptr(), W, 0, cap, rows_of(sends, W),
        (ctypes.c_int64 * R)(*[(t.numel() - 4) // W for t in shifted]), ws.data_ptr(), need,
        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    for d in range(R):
        assert bits_equal(host(shifted[d][4:]), want[d]), d
    assert bool((ws == 0xCD).all())


def test_moe_exchange_full_size_matches_the_plain_form():
    """8 ranks x 4096 tokens x top-8 of 256 (Zipf routing), rows of 7168 bf16:
    dispatch and the transposed combine exchange, both forms bit for bit."""
    R, E, T, K, H = 8, 256, 4096, 8, 7168
    say("a2av ws moe full size")
    ids = [synth.zipf_routing(T, E, K, seed=5100 + s)[0] for s in range(R)]
    lay = oracle.moe_layout(ids, E)
    sc, sd, rd = lay["sendcounts"], lay["sdispls"], lay["rdispls"]
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    sends = [torch.randn((T * K, H), generator=g, device="cuda").to(torch.bfloat16)
             for _ in range(R)]
    rows = sc.sum(axis=0)
    a = [torch.empty((int(n), H), dtype=torch.bfloat16, device="cuda") for n in rows]
    b = [torch.empty_like(t) for t in a]
    ws = torch.empty(coll.all_to_all_v_workspace_bytes(sends, a, H), dtype=torch.uint8,
                     device="cuda")
    coll.all_to_all_v(sends, dc(sc), dc(sd), a, dc(rd), H)
    coll.all_to_all_v(sends, dc(sc), dc(sd), b, dc(rd), H, workspace=ws)
    torch.cuda.synchronize()
    for d in range(R):
        assert torch.equal(a[d].view(torch.int16), b[d].view(torch.int16)), d
    back_a = [torch.empty_like(s) for s in sends]
    back_b = [torch.empty_like(s) for s in sends]
    ws2 = torch.empty(coll.all_to_all_v_workspace_bytes(b, back_b, H), dtype=torch.uint8,
                      device="cuda")
    coll.all_to_all_v(a, dc(sc.T), dc(rd), back_a, dc(sd), H)
    coll.all_to_all_v(b, dc(sc.T), dc(rd), back_b, dc(sd), H, workspace=ws2)
    torch.cuda.synchronize()
    for s in range(R):
        assert torch.equal(back_a[s].view(torch.int16), back_b[s].view(torch.int16)), s
        assert torch.equal(back_b[s].view(torch.int16), sends[s].view(torch.int16)), s
    # sampled blocks of the dispatch against the oracle, run on just those rows
    rng = np.random.default_rng(5)
    pairs = [(s, d) for s in range(R) for d in range(R) if sc[s, d] > 0]
    for i in rng.choice(len(pairs), 12, replace=False):
        s, d = pairs[i]
        j0 = int(rng.integers(0, sc[s, d]))
        n = min(16, int(sc[s, d]) - j0)
        src = host(sends[s][int(sd[s, d]) + j0:int(sd[s, d]) + j0 + n])
        z = np.zeros((1, 1), np.int64)
        want = oracle.all_to_all_v([src], np.array([[n]], np.int64), z, z, [n], H)[0]
        got = host(b[d][int(rd[d, s]) + j0:int(rd[d, s]) + j0 + n])
        assert bits_equal(got.reshape(-1), want.reshape(-1)), (s, d, j0)


def test_graph_replays_the_descriptor_form():
    R, W = 8, 64
    say("a2av ws graph")
    g = np.random.default_rng(11)
    counts = g.integers(0, 200, size=(R, R)).astype(np.int64)
    sends, recvs, want, sd, rd = case(R, W, counts, seed=11)
    cap = desc_rows(W * 2)
    ws = torch.empty(coll.all_to_all_v_workspace_bytes(sends, recvs, W, capacity=cap),
                     dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    tabs = (dc(counts), dc(sd), dc(rd))
    plan = coll.prepare(coll.all_to_all_v, sends, tabs[0], tabs[1], recvs, tabs[2], W,
                        workspace=ws, capacity=cap)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        plan()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan()
    for rep in range(3):
        for r in recvs:
            r.view(torch.int16).fill_(0x7FAB)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for d in range(R):
            assert bits_equal(host(recvs[d]), want[d]), (rep, d)


@pytest.mark.parametrize("R,W,lo,hi", [(8, 2048, 600, 1000), (4, 8192, 750, 1000),
                                       (16, 1024, 400, 520), (3, 4096, 3000, 4000),
                                       (1, 8192, 13000, 14000)])
def test_build_on_a_second_stream_then_copy(R, W, lo, hi):
    """The descriptor form in two calls, used as intended: the build runs on
    a second stream before the send buffers are written (it reads only the
    tables and the buffers' addresses); the copy runs after both.  Forward and
    reverse, against the oracle."""
    say("a2av build/copy", R, W)
    g = np.random.default_rng(77 + R)
    counts = g.integers(lo, hi, size=(R, R)).astype(np.int64)
    sd, rd = oracle.packed_displs(counts)
    send_rows = counts.sum(axis=1)
    recv_rows = counts.sum(axis=0)
    assert int(recv_rows.sum()) * W * 2 >= DESC_MIN_BYTES
    xs = [synth.gaussian(int(send_rows[s]) * W, 1.0, 8800 + s, "bf16") for s in range(R)]
    want = oracle.all_to_all_v(xs, counts, sd, rd, recv_rows, W)
    sends = [torch.empty(int(n) * W, dtype=torch.bfloat16, device="cuda") for n in send_rows]
    recvs = [poison_like(torch.empty(int(n) * W, dtype=torch.bfloat16, device="cuda"))
             for n in recv_rows]
    tabs = (dc(counts), dc(sd), dc(rd))
    ws = torch.empty(coll.all_to_all_v_workspace_bytes(sends, recvs, W), dtype=torch.uint8,
                     device="cuda")
    bws = torch.empty(coll.all_to_all_v_workspace_bytes(recvs, sends, W), dtype=torch.uint8,
                      device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        coll.all_to_all_v_build(sends, *tabs[:2], recvs, tabs[2], W, ws)
        coll.all_to_all_v_reverse_build(recvs, *tabs[:2], sends, tabs[2], W, bws)
    built = torch.cuda.Event()
    built.record(side)
    for t, x in zip(sends, xs):                 # the send rows arrive after the build
        t.copy_(dev(x))
    torch.cuda.current_stream().wait_event(built)
    coll.all_to_all_v_copy(sends, recvs, W, ws)
    torch.cuda.synchronize()
    for d in range(R):
        assert bits_equal(host(recvs[d]), want[d]), f"rank {d}"
    for t in sends:
        t.view(torch.int16).fill_(0x7FAB)
    coll.all_to_all_v_copy(recvs, sends, W, bws)
    torch.cuda.synchronize()
    for s in range(R):
        assert bits_equal(host(sends[s]), xs[s]), f"returned rank {s}"


def test_copy_refuses_sizes_without_a_descriptor_form():
    sends = [torch.empty(64, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    recvs = [torch.empty(64, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        coll.all_to_all_v_copy(sends, recvs, 8, ws)
