"""GPU parity past the 32-bit boundaries: buffers of more than 2^31 elements
or 4 GiB, where an index or byte offset computed in 32 bits would wrap.

Inputs are a seeded block of prime length tiled over the large buffer (a
copy made by torch), so every sampled element is known on the host, and an
element 2^31 positions (or 4 GiB) away holds a different value.  The oracle
runs on the sampled elements only; samples cover the region past the
boundary and the very end (the scalar tails)."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import coll, synth
from gpu_util import bits_equal, dev, host, say

pytestmark = pytest.mark.gpu

PERIOD = 1_000_003          # prime: 2^31 and 2^32 are not multiples of it


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    coll.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def tiled(t, block_np):
    """Fill the 1-D tensor t with block_np repeated (a torch copy)."""
    blk = dev(block_np).view(t.dtype)
    n, L = t.numel(), blk.numel()
    k = n // L
    if k:
        t[:k * L].view(k, L).copy_(blk.expand(k, L))
    if n - k * L:
        t[k * L:].copy_(blk[:n - k * L])


def sample_idx(n, seed, boundary=1 << 31):
    g = np.random.default_rng(seed)
    parts = [np.arange(max(0, boundary - 8), min(n, boundary + 8)),
             np.arange(max(0, n - 64), n),
             g.integers(0, n, 2048),
             g.integers(min(boundary, n - 1), n, 2048)]
    return np.unique(np.concatenate(parts)).astype(np.int64)


def gather_host(t, idx):
    return host(t[torch.from_numpy(idx).cuda()])


def test_allreduce_past_2g_elements():
    R, n = 2, (1 << 31) + 27                       # 4 GiB + 54 B per rank; 3-element tail
    say("max-size allreduce", n)
    blocks = [synth.gaussian(PERIOD, 1.0, 97000 + r, "bf16") for r in range(R)]
    ins = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    for t, b in zip(ins, blocks):
        tiled(t, b)
    outs = [torch.empty_like(t) for t in ins]
    coll.allreduce(ins, outs)
    torch.cuda.synchronize()
    idx = sample_idx(n, 1)
    want = oracle.allreduce([np.ascontiguousarray(b[idx % PERIOD]) for b in blocks], "bf16")
    for r in range(R):
        assert bits_equal(gather_host(outs[r], idx), want[r]), r
    del ins, outs


@pytest.mark.parametrize("n", [1 << 23, 1 << 24])
def test_reduce_scatter_store_policy_sides(n):
    """R = 8 ReduceScatter writing 128 MiB in all (sums stored cacheable) and
    256 MiB (stored non-temporally): each output element is the rank-order
    fold of its R inputs, checked on samples against the oracle."""
    R = 8
    say("reduce_scatter store policy", n)
    blocks = [synth.gaussian(PERIOD, 1.0, 98000 + r, "bf16") for r in range(R)]
    ins = [torch.empty(R * n, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    for t, b in zip(ins, blocks):
        tiled(t, b)
    outs = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    coll.reduce_scatter(ins, outs)
    torch.cuda.synchronize()
    idx = sample_idx(n, 5, boundary=n // 2)
    for r in range(R):
        src = (r * n + idx) % PERIOD
        want = oracle.allreduce([np.ascontiguousarray(b[src]) for b in blocks], "bf16")[0]
        assert bits_equal(gather_host(outs[r], idx), want), r
    del ins, outs


def test_all_gather_outputs_past_4gib():
    R, n = 4, (1 << 29) + 40                       # shards of 1 GiB + 80 B; outputs 4 GiB +
    say("max-size all_gather", n)
    blocks = [synth.random_bits(PERIOD, 2, 98000 + q) for q in range(R)]
    ins = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    for t, b in zip(ins, blocks):
        tiled(t, b)
    outs = [torch.empty(R * n, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    coll.all_gather(ins, outs)
    torch.cuda.synchronize()
    idx = sample_idx(R * n, 2)
    q, i = idx // n, idx % n
    want = np.array([blocks[a][b % PERIOD] for a, b in zip(q, i)], np.uint16)
    for r in range(R):
        assert bits_equal(gather_host(outs[r], idx), want), r
    del ins, outs


def test_gather_64bit_index_space():
    """2-byte units (odd inner) and more than 2^31 units in the root's output:
    the 64-bit Gather path."""
    R, outer, inner = 8, 32768, 8193
    total = outer * R * inner
    assert total > (1 << 31)
    say("max-size gather", total)
    blocks = [synth.random_bits(PERIOD, 2, 99000 + q) for q in range(R)]
    ins = [torch.empty((outer, inner), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    for t, b in zip(ins, blocks):
        tiled(t.view(-1), b)
    out = torch.empty((outer, R * inner), dtype=torch.bfloat16, device="cuda")
    coll.gather(ins, out, 0)
    torch.cuda.synchronize()
    idx = sample_idx(total, 3)
    o, rem = idx // (R * inner), idx % (R * inner)
    q, i = rem // inner, rem % inner
    want = np.array([blocks[a][(oo * inner + b) % PERIOD] for oo, a, b in zip(o, q, i)],
                    np.uint16)
    assert bits_equal(gather_host(out.view(-1), idx), want)
    del ins, out


def test_gather_rank_share_past_2g_units():
    """One rank's share alone is more than 2^31 units (2-byte units, odd
    inner): the 64-bit Gather kernel."""
    R, outer, inner = 2, 2, (1 << 30) + 3
    per_rank = outer * inner
    assert per_rank > (1 << 31)
    say("max-size gather, 64-bit share", per_rank)
    blocks = [synth.random_bits(PERIOD, 2, 99100 + q) for q in range(R)]
    ins = [torch.empty((outer, inner), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    for t, b in zip(ins, blocks):
        tiled(t.view(-1), b)
    out = torch.empty((outer, R * inner), dtype=torch.bfloat16, device="cuda")
    coll.gather(ins, out, 0)
    torch.cuda.synchronize()
    total = outer * R * inner
    idx = sample_idx(total, 4, boundary=1 << 31)
    o, rem = idx // (R * inner), idx % (R * inner)
    q, i = rem // inner, rem % inner
    want = np.array([blocks[a][(oo * inner + b) % PERIOD] for oo, a, b in zip(o, q, i)],
                    np.uint16)
    assert bits_equal(gather_host(out.view(-1), idx), want)
    del ins, out
    torch.cuda.empty_cache()


def test_broadcast_past_4gib():
    R, n = 3, (1 << 31) + 5                        # bf16: 4 GiB + 10 B per buffer
    say("max-size broadcast", n)
    block = synth.random_bits(PERIOD, 2, 99500)
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    tiled(src, block)
    outs = [torch.empty_like(src) for _ in range(R)]
    outs[1] = src                                  # the root keeps its buffer
    coll.broadcast(src, outs, 1)
    torch.cuda.synchronize()
    idx = sample_idx(n, 4)
    want = block[idx % PERIOD]
    for r in range(R):
        assert bits_equal(gather_host(outs[r], idx), want), r
    del src, outs


def test_all_to_all_v_receive_past_4gib():
    """Rows of 7168 bf16; rank 0 receives 320,000 rows (4.27 GiB) and rank 1
    a few, so receive offsets pass 2^32 bytes."""
    R, W = 2, 7168
    counts = np.array([[160_000, 3], [160_000, 5]], np.int64)
    sd, rd = oracle.packed_displs(counts)
    srows, rrows = counts.sum(axis=1), counts.sum(axis=0)
    say("max-size a2av", int(rrows[0]))
    prow = 101                                     # rows per block of the pattern (prime)
    blocks = [synth.random_bits((prow, W), 2, 99700 + s) for s in range(R)]
    sends = [torch.empty((int(srows[s]), W), dtype=torch.bfloat16, device="cuda")
             for s in range(R)]
    for t, b in zip(sends, blocks):
        tiled(t.view(-1), b.reshape(-1))
    recvs = [torch.empty((int(rrows[d]), W), dtype=torch.bfloat16, device="cuda")
             for d in range(R)]
    dc = lambda a: torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda()
    coll.all_to_all_v(sends, dc(counts), dc(sd), recvs, dc(rd), W)
    torch.cuda.synchronize()
    g = np.random.default_rng(5)
    for d in range(R):
        nr = int(rrows[d])
        rows = np.unique(np.concatenate([g.integers(0, nr, 64), np.arange(max(0, nr - 3), nr)]))
        got = host(recvs[d][torch.from_numpy(rows).cuda()])
        for k, row in enumerate(rows):
            # receive row -> (source, row within its block) -> source row
            s = int(np.searchsorted(rd[d], row, side="right") - 1)
            srow = int(sd[s, d] + (row - rd[d, s]))
            want = blocks[s].reshape(-1)[(srow * W + np.arange(W)) % (prow * W)]
            assert bits_equal(got[k], want), (d, row)
    del sends, recvs
