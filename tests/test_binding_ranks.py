"""Every wrapper of the binding refuses a per-rank list whose length is not
the rank count, before anything reaches the C ABI (CPU only).

The library reads R pointers from every table it is given; a shorter list
would make it read past the end of the host array and the kernels store to
garbage addresses.  Here the device-pointer lookup and the C call are
stubbed: CPU tensors stand in for device buffers, and a call that passes the
checks is recorded instead of issued.
"""
import pytest
import torch

from collective_communication_amd import coll

R = 4


@pytest.fixture
def issued(monkeypatch):
    calls = []
    monkeypatch.setattr(coll, "_dev", lambda t, what: 0x1000)
    monkeypatch.setattr(coll, "_issue", lambda name, what, stream, *args: calls.append(name))
    return calls


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def i64(n):
    return torch.zeros(n, dtype=torch.int64)


T, K, H, E = 6, 2, 8, 8

# wrapper name -> (builder of valid arguments, indices of the per-rank lists)
CASES = {
    "allreduce": (lambda: ([bf(16) for _ in range(R)], [bf(16) for _ in range(R)]), (0, 1)),
    "reduce_scatter": (lambda: ([bf(4 * R) for _ in range(R)], [bf(4) for _ in range(R)]), (0, 1)),
    "all_gather": (lambda: ([bf(4) for _ in range(R)], [bf(4 * R) for _ in range(R)]), (0, 1)),
    "all_to_all": (lambda: ([bf(4 * R) for _ in range(R)], [bf(4 * R) for _ in range(R)]), (0, 1)),
    "all_to_all_v": (lambda: ([bf(8) for _ in range(R)], i64(R * R), i64(R * R),
                              [bf(8) for _ in range(R)], i64(R * R), 1), (0, 3)),
    "all_to_all_v_reverse": (lambda: ([bf(8) for _ in range(R)], i64(R * R), i64(R * R),
                                      [bf(8) for _ in range(R)], i64(R * R), 1), (0, 3)),
    "seq_heads_reshard": (lambda: ([bf(2, 4, 8) for _ in range(R)], [bf(2, 4, 8) for _ in range(R)],
                                   4, 8, True), (0, 1)),
    "lse_merge": (lambda: ([bf(3, 8) for _ in range(R)],
                           [torch.zeros(3) for _ in range(R)],
                           [bf(3, 8) for _ in range(R)],
                           [torch.zeros(3) for _ in range(R)]), (0, 1, 2, 3)),
    "moe_layout": (lambda: ([i32(T, K) for _ in range(R)], E, i64(R * R), i64(R * R), i64(R * R),
                            i32(R * E), [i32(T, K) for _ in range(R)], torch.zeros(256, dtype=torch.uint8)),
                   (0, 6)),
    "moe_layout_noalloc": (lambda: ([i32(T, K) for _ in range(R)], E, i64(R * R), i64(R * R),
                                    i64(R * R), i32(R * E), [i32(T, K) for _ in range(R)]), (0, 6)),
    "moe_permute": (lambda: ([bf(T, H) for _ in range(R)], [i32(T, K) for _ in range(R)],
                             [bf(T * K, H) for _ in range(R)]), (0, 1, 2)),
    "moe_expert_scale": (lambda: ([bf(T * K, H) for _ in range(R)], i32(R * E), i64(R * R), E, H,
                                  torch.zeros(1024, dtype=torch.uint8)), (0,)),
    "moe_combine": (lambda: ([bf(T * K, H) for _ in range(R)], [i32(T, K) for _ in range(R)],
                             [torch.zeros(T, K) for _ in range(R)], [bf(T, H) for _ in range(R)]),
                    (0, 1, 2, 3)),
    "moe_dispatch": (lambda: ([bf(T, H) for _ in range(R)], [i32(T, K) for _ in range(R)],
                              i64(R * R), i64(R * R), i64(R * R),
                              [bf(T * K, H) for _ in range(R)]), (0, 1, 5)),
    "moe_combine_recv": (lambda: ([bf(T * K, H) for _ in range(R)], [i32(T, K) for _ in range(R)],
                                  i64(R * R), i64(R * R), i64(R * R),
                                  [torch.zeros(T, K) for _ in range(R)],
                                  [bf(T, H) for _ in range(R)], [i32(T, K) for _ in range(R)]),
                         (0, 1, 5, 6, 7)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_valid_lists_reach_the_entry_point(issued, name):
    build, _ = CASES[name]
    getattr(coll, name)(*build())
    assert issued == ["coll_" + name]


@pytest.mark.parametrize("name,idx", [(n, i) for n, (_, lists) in sorted(CASES.items())
                                      for i in lists])
@pytest.mark.parametrize("delta", [-1, +1])
def test_a_list_of_the_wrong_length_is_refused(issued, name, idx, delta):
    build, _ = CASES[name]
    args = list(build())
    lst = list(args[idx])
    args[idx] = lst[:-1] if delta < 0 else lst + [lst[0]]
    with pytest.raises(ValueError):
        getattr(coll, name)(*args)
    assert issued == []


def test_one_rank_buffers_for_scatter_broadcast_gather_reduce(issued):
    """The root-side single buffer calls size R by their one list."""
    coll.scatter(bf(4 * R), [bf(4) for _ in range(R)], 0)
    coll.broadcast(bf(4), [bf(4) for _ in range(R)], 0)
    coll.gather([bf(2, 3) for _ in range(R)], bf(2, 3 * R), 0)
    coll.reduce([bf(4) for _ in range(R)], bf(4), 0)
    assert issued == ["coll_scatter", "coll_broadcast", "coll_gather", "coll_reduce"]


BIG = 1 << 24          # rows of 8 bf16: 256 MiB of capacity, above the descriptor threshold
SPLIT = {
    # wrapper -> (C entry point, builder of valid arguments, indices of per-rank lists)
    "all_to_all_v_build": ("coll_all_to_all_v_ws_build",
                           lambda: ([bf(8) for _ in range(R)], i64(R * R), i64(R * R),
                                    [bf(8) for _ in range(R)], i64(R * R), 8,
                                    torch.zeros(256, dtype=torch.uint8), None, BIG), (0, 3)),
    "all_to_all_v_reverse_build": ("coll_all_to_all_v_reverse_build",
                                   lambda: ([bf(8) for _ in range(R)], i64(R * R), i64(R * R),
                                            [bf(8) for _ in range(R)], i64(R * R), 8,
                                            torch.zeros(256, dtype=torch.uint8), None, BIG),
                                   (0, 3)),
    "all_to_all_v_copy": ("coll_all_to_all_v_ws_copy",
                          lambda: ([bf(8) for _ in range(R)], [bf(8) for _ in range(R)], 8,
                                   torch.zeros(256, dtype=torch.uint8), None, BIG), (0, 1)),
}


@pytest.mark.parametrize("name", sorted(SPLIT))
def test_split_descriptor_form_wrappers(issued, name):
    entry, build, lists = SPLIT[name]
    getattr(coll, name)(*build())
    assert issued == [entry]
    for idx in lists:
        for delta in (-1, +1):
            args = list(build())
            lst = list(args[idx])
            args[idx] = lst[:-1] if delta < 0 else lst + [lst[0]]
            with pytest.raises(ValueError):
                getattr(coll, name)(*args)
    assert issued == [entry]
    # sizes without a descriptor form are refused before the C call
    args = list(build())
    args[-1] = 16
    with pytest.raises(ValueError):
        getattr(coll, name)(*args)


def _expert_args(split_rows=T * K):
    ws = torch.zeros(coll.moe_expert_workspace_bytes(R, E, R * split_rows), dtype=torch.uint8)
    return [bf(split_rows, H) for _ in range(R)], i32(R * E), i64(R * R), E, H, ws


@pytest.mark.parametrize("name,entry", [("moe_expert_scale_build", "coll_moe_expert_scale_build"),
                                        ("moe_expert_scale_apply", "coll_moe_expert_scale_apply")])
def test_expert_split_wrappers(issued, name, entry):
    def build(rows=T * K, ws=None):
        recvs, ec, rd, e, h, w = _expert_args(rows)
        w = w if ws is None else ws
        return [recvs, ec, rd, e, h, w] if name.endswith("build") else [recvs, e, h, w]

    getattr(coll, name)(*build())
    assert issued == [entry]
    for delta in (-1, +1):
        args = build()
        lst = list(args[0])
        args[0] = lst[:-1] if delta < 0 else lst + [lst[0]]
        with pytest.raises(ValueError):
            getattr(coll, name)(*args)
    # the row-descriptor path does not apply: a workspace of the tables alone,
    # or no receive rows at all
    with pytest.raises(ValueError):
        getattr(coll, name)(*build(ws=torch.zeros(coll.moe_expert_workspace_bytes(R, E, 0),
                                                  dtype=torch.uint8)))
    with pytest.raises(ValueError):
        getattr(coll, name)(*build(rows=0))
    assert issued == [entry]
