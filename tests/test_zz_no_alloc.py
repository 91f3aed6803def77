"""coll_moe_layout_noalloc -- the MoE layout whose scratch is the library's
per-GPU device array -- called through the C ABI and compared with
coll_moe_layout (caller workspace) on the same routing, bit for bit: two
calls in a row, the second smaller than the first (the array keeps the first
call's contents), the second with planted ids outside [0, E)."""
import ctypes

import numpy as np
import pytest
import torch

from collective_communication_amd import coll, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    coll.lib()
    yield
    torch.cuda.synchronize()


def _ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _tables(R, E, T, K, fill):
    sc = torch.full((R * R,), fill, dtype=torch.int64, device="cuda")
    sd, rd = torch.full_like(sc, fill), torch.full_like(sc, fill)
    ec = torch.full((R * E,), fill, dtype=torch.int32, device="cuda")
    pos = [torch.full((T, K), fill, dtype=torch.int32, device="cuda") for _ in range(R)]
    return sc, sd, rd, ec, pos


def _host(tabs):
    sc, sd, rd, ec, pos = tabs
    return [t.cpu().numpy() for t in (sc, sd, rd, ec)] + [p.cpu().numpy() for p in pos]


def _routing(R, E, T, K, seed, bad=False):
    ids = []
    g = np.random.default_rng(seed)
    for s in range(R):
        i = synth.zipf_routing(T, E, K, seed=seed + s)[0]
        if bad:
            m = g.random(i.shape) < 0.05
            i[m] = g.choice(np.array([-1, E, 1 << 30], np.int32), size=int(m.sum()))
        ids.append(torch.from_numpy(i).cuda())
    return ids


@pytest.mark.parametrize("first,second", [
    ((8, 256, 4096, 8), (4, 16, 333, 3)),
    ((8, 256, 8000, 8), (8, 256, 100, 8)),
])
def test_noalloc_layout_equals_the_workspace_form_on_two_calls(first, second):
    L = coll.lib()
    stream = torch.cuda.current_stream().cuda_stream
    for n, (R, E, T, K) in enumerate((first, second)):
        ids = _routing(R, E, T, K, 7100 + 10 * n, bad=(n == 1))
        ref = _tables(R, E, T, K, -7)
        work = torch.empty(coll.moe_workspace_bytes(R, T, K, E), dtype=torch.uint8, device="cuda")
        coll.moe_layout(ids, E, *ref, work)
        got = _tables(R, E, T, K, -9)
        sc, sd, rd, ec, pos = got
        rc = L.coll_moe_layout_noalloc(R, _ptrs(ids), T, K, E, sc.data_ptr(), sd.data_ptr(),
                                       rd.data_ptr(), ec.data_ptr(), _ptrs(pos), stream)
        assert rc == 0
        torch.cuda.synchronize()
        for a, b in zip(_host(ref), _host(got)):
            assert np.array_equal(a, b), (n, R, E, T, K)


def test_noalloc_layout_rejects_sizes_beyond_its_array():
    L = coll.lib()
    R, E, T, K = 16, 1024, 10000, 8
    assert coll.moe_workspace_bytes(R, T, K, E) > 4 << 20
    ids = [torch.zeros((1, K), dtype=torch.int32, device="cuda") for _ in range(R)]
    tabs = _tables(R, E, 1, K, 0)
    sc, sd, rd, ec, pos = tabs
    rc = L.coll_moe_layout_noalloc(R, _ptrs(ids), T, K, E, sc.data_ptr(), sd.data_ptr(),
                                   rd.data_ptr(), ec.data_ptr(), _ptrs(pos), None)
    assert rc == -1
