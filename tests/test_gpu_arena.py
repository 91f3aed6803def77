"""GPU parity of collectives whose rank buffers are views of one rank arena
(coll_arena_layout placement): results match the oracle bit for bit, and no
byte of the arena outside the output buffers changes."""
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


def arena_bytes(t):
    """The whole allocation behind an arena view, as bytes."""
    st = t.untyped_storage()
    return torch.empty(0, dtype=torch.uint8, device=t.device).set_(st, 0, (st.nbytes(),), (1,))


def byte_span(t):
    s = t.storage_offset() * t.element_size()
    return s, s + t.numel() * t.element_size()


def outside_unchanged(before, after, written):
    """Every byte outside the `written` views is unchanged."""
    keep = np.ones(before.size, bool)
    for t in written:
        a, b = byte_span(t)
        keep[a:b] = False
    return np.array_equal(before[keep], after[keep])


def fill_arena(full, inputs, arrays):
    full.fill_(0xA5)
    for t, a in zip(inputs, arrays):
        t.copy_(dev(a).view(t.dtype).view(t.shape))
    torch.cuda.synchronize()
    return host(full)


@pytest.mark.parametrize("n", [300001, 1 << 20])
def test_allreduce_on_rank_arena(n):
    R = 8
    say("allreduce arena", n)
    xs = [synth.gaussian(n, 0.02, 91000 + r, "bf16") for r in range(R)]
    ins, outs = coll.rank_arena([(R, n, torch.bfloat16), (R, n, torch.bfloat16)])
    full = arena_bytes(ins[0])
    before = fill_arena(full, ins, xs)
    coll.allreduce(ins, outs)
    torch.cuda.synchronize()
    want = oracle.allreduce(xs, "bf16")
    for r in range(R):
        assert bits_equal(host(outs[r]), want[r]), r
    assert outside_unchanged(before, host(full), outs)


def test_reduce_scatter_then_all_gather_on_rank_arena():
    R, seg = 8, 12352
    say("rs/ag arena", seg)
    xs = [synth.gaussian(R * seg, 1.0, 92000 + r, "bf16") for r in range(R)]
    ins, shards, fulls = coll.rank_arena([(R, R * seg, torch.bfloat16),
                                          (R, seg, torch.bfloat16),
                                          (R, R * seg, torch.bfloat16)])
    full = arena_bytes(ins[0])
    before = fill_arena(full, ins, xs)
    coll.reduce_scatter(ins, shards)
    coll.all_gather(shards, fulls)
    torch.cuda.synchronize()
    want = oracle.allreduce(xs, "bf16")
    for r in range(R):
        assert bits_equal(host(fulls[r]), want[r]), r
    assert outside_unchanged(before, host(full), shards + fulls)


def test_all_to_all_v_on_rank_arena():
    R, W = 8, 136
    say("a2av arena")
    g = np.random.default_rng(7)
    counts = g.integers(0, 40, size=(R, R)).astype(np.int64)
    counts[2, :] = 0                                   # a rank that sends nothing
    sd, rd = oracle.packed_displs(counts)
    send_rows = counts.sum(axis=1)
    recv_rows = counts.sum(axis=0)
    xs = [synth.random_bits((int(send_rows[s]), W), 2, 93000 + s) for s in range(R)]
    sends, recvs = coll.rank_arena([[((int(send_rows[s]), W), torch.bfloat16) for s in range(R)],
                                    [((int(recv_rows[d]), W), torch.bfloat16) for d in range(R)]])
    full = arena_bytes(sends[0])
    nonempty = [(t, x) for t, x in zip(sends, xs) if t.numel()]
    before = fill_arena(full, [t for t, _ in nonempty], [x for _, x in nonempty])
    dc = lambda a: torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda()
    coll.all_to_all_v(sends, dc(counts), dc(sd), recvs, dc(rd), W)
    torch.cuda.synchronize()
    want = oracle.all_to_all_v(xs, counts, sd, rd, recv_rows, W)
    for d in range(R):
        assert bits_equal(host(recvs[d]).reshape(-1), want[d].reshape(-1)), d
    assert outside_unchanged(before, host(full), recvs)
