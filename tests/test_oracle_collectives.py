"""Pins for the oracle's collectives (CPU only).

Each primitive is held to something other than its own code: invariants the
pages state (AllReduce = AllGather after ReduceScatter; Gather after Scatter is
the identity; Broadcast leaves every rank equal to the root; All-to-All-v with
transposed counts undoes itself), closed forms (power-of-two scaling, integer
sums, exact products), library routines (numpy concatenate / transpose /
maximum, torch's bf16 cast), the fp64 exact sum within the fp32-accumulate
error bound, brute force on tiny inputs, and the worked examples the pages
print (fixtures under tests/golden/).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import synth
from conftest import golden

DT_NP = {"bf16": np.uint16, "fp16": np.float16, "fp32": np.float32, "int32": np.int32}


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening through library routines (not the oracle's)."""
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()
    return a.astype(np.float64)


def from_f32_lib(x32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> dtype storage through library casts."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "fp16":
        return x32.astype(np.float16)
    return x32.astype(np.float32)


def bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


# ------------------------------------------------------------------ AllReduce

@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32", "int32"])
@pytest.mark.parametrize("R", [1, 2, 3, 4, 8])
def test_allreduce_equals_allgather_of_reducescatter(dtype, R):
    """Tutorial 6.1: AllReduce = ReduceScatter + AllGather, bit for bit."""
    n = R * 1000
    if dtype == "int32":
        xs = [synth.uniform_int32(n, -2**31, 2**31 - 1, 100 + r) for r in range(R)]
    else:
        xs = [synth.gaussian(n, 1.0, 100 + r, dtype) for r in range(R)]
    ar = oracle.allreduce(xs, dtype)
    ag = oracle.all_gather(oracle.reduce_scatter(xs, dtype))
    for r in range(R):
        assert np.array_equal(bits(ar[r]), bits(ag[r]))
        assert np.array_equal(bits(ar[r]), bits(ar[0]))   # identical on all ranks


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("R", [1, 2, 4, 8, 16])
def test_allreduce_identical_inputs_scale_exactly(dtype, R):
    """Same x on R = 2^m ranks: every partial sum k*x is exact in fp32 and
    R*x is exact in the narrow type, so the result is x scaled by R."""
    x = synth.gaussian(4097, 1.0, 5, dtype)
    out = oracle.allreduce([x.copy() for _ in range(R)], dtype)[0]
    expect = from_f32_lib((to_f64(x, dtype) * R).astype(np.float32), dtype)
    assert np.array_equal(bits(out), bits(expect))


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32", "int32"])
@pytest.mark.parametrize("R", [2, 3, 5, 8])
def test_allreduce_small_integers_exact(dtype, R):
    """|x| <= 8 integers: every partial sum is an exact small integer."""
    xs = [synth.small_integers(3001, 8, 40 + r, dtype) for r in range(R)]
    total = sum(to_f64(x, dtype) if dtype != "int32" else x.astype(np.int64) for x in xs)
    out = oracle.allreduce(xs, dtype)[0]
    if dtype == "int32":
        assert np.array_equal(out, total.astype(np.int32))
    else:
        assert np.array_equal(bits(out), bits(from_f32_lib(total.astype(np.float32), dtype)))


def test_allreduce_int32_wraps():
    xs = [synth.uniform_int32(5000, -2**31, 2**31 - 1, 60 + r) for r in range(7)]
    total = sum(x.astype(np.int64) for x in xs)
    wrapped = ((total + 2**31) % 2**32 - 2**31).astype(np.int32)
    assert np.array_equal(oracle.allreduce(xs, "int32")[3], wrapped)


@pytest.mark.parametrize("dtype,u_out", [("bf16", 2.0 ** -8), ("fp16", 2.0 ** -11),
                                         ("fp32", 0.0)])
@pytest.mark.parametrize("R", [2, 4, 8, 16])
def test_allreduce_within_error_bound_of_exact_sum(dtype, u_out, R):
    """The fp64 sum of the (exactly widened) inputs is the exact result up to
    fp32 accumulation (at most (R-1) roundings of 2^-24 relative to the
    running magnitude) and one final rounding to the output type."""
    xs = [synth.gaussian(20000, 1.0, 300 + r, dtype) for r in range(R)]
    w = [to_f64(x, dtype) for x in xs]
    exact = sum(w)
    mag = sum(np.abs(v) for v in w)
    e32 = 1.01 * (R - 1) * 2.0 ** -24 * mag
    out = to_f64(oracle.allreduce(xs, dtype)[0], dtype)
    bound = u_out * (np.abs(exact) + e32) + e32 + 2.0 ** -140
    assert np.all(np.abs(out - exact) <= bound)
    # and the bound is tight enough to notice a dropped rank
    assert np.any(np.abs(to_f64(oracle.allreduce(xs[1:], dtype)[0], dtype) - exact) > bound)


@pytest.mark.parametrize("R", [1, 2, 3])
@pytest.mark.parametrize("n", [0, 1, 2, 3, 5, 8, 17])
def test_allreduce_brute_force_tiny(R, n):
    """numpy fp32 sequential fold in rank order + torch's RNE cast."""
    xs = [synth.gaussian(n, 1.0, 7 * R + n + r, "bf16") for r in range(R)]
    acc = to_f64(xs[0], "bf16").astype(np.float32)
    for r in range(1, R):
        acc = (acc + to_f64(xs[r], "bf16").astype(np.float32)).astype(np.float32)
    expect = from_f32_lib(acc, "bf16")
    for out in oracle.allreduce(xs, "bf16"):
        assert np.array_equal(out, expect)


def test_allreduce_rank_order_is_ascending():
    """(2^24 + 1) - 2^24 style cancellations distinguish fold orders."""
    big, one = np.float32(2.0 ** 24), np.float32(1.0)
    xs = [np.array([big], np.float32), np.array([one], np.float32),
          np.array([-big], np.float32)]
    # ((2^24 + 1) -> 2^24 after rounding) - 2^24 = 0 in ascending order
    assert oracle.allreduce(xs, "fp32")[0][0] == 0.0
    # seeding with rank 0's value, not 0.0: -0 + -0 stays -0
    z = [np.array([-0.0], np.float32)] * 2
    assert np.signbit(oracle.allreduce(z, "fp32")[0][0])


@pytest.mark.parametrize("dtype", ["bf16", "fp32", "int32"])
def test_allreduce_max_min_match_numpy(dtype):
    xs = [synth.gaussian(5000, 1.0, 900 + r, "fp32") for r in range(5)]
    if dtype == "int32":
        xs = [(x * 1000).astype(np.int32) for x in xs]
        ref = xs
    else:
        xs = [from_f32_lib(x, dtype) for x in xs]
        ref = [to_f64(x, dtype) for x in xs]
    mx = oracle.allreduce(xs, dtype, "max")[0]
    mn = oracle.allreduce(xs, dtype, "min")[0]
    get = (lambda a: a) if dtype == "int32" else (lambda a: to_f64(a, dtype))
    assert np.array_equal(get(mx), np.maximum.reduce(ref))
    assert np.array_equal(get(mn), np.minimum.reduce(ref))


# IEEE 754-2019 section 9.6: maximum / minimum propagate a NaN operand and
# order -0 below +0 (so the result does not depend on operand order).  The
# pages fix none of this; the oracle follows that standard, and these are its
# special cases written out value by value.
_NAN, _INF = float("nan"), float("inf")
IEEE_2019_CASES = [
    # rank values, maximum, minimum
    ([+0.0, -0.0], +0.0, -0.0),
    ([-0.0, +0.0], +0.0, -0.0),
    ([-0.0, -0.0], -0.0, -0.0),
    ([+0.0, +0.0], +0.0, +0.0),
    ([1.0, _NAN, 2.0], _NAN, _NAN),
    ([_NAN, 1.0], _NAN, _NAN),
    ([3.0, _NAN], _NAN, _NAN),
    ([_INF, _NAN], _NAN, _NAN),
    ([-_INF, 3.0], 3.0, -_INF),
    ([-1.5, -0.0, -2.5], -0.0, -2.5),
    ([-0.0, 0.5, +0.0], 0.5, -0.0),
]


def _same_value(got, want):
    """Equal as IEEE values, with the sign of zero significant and any NaN
    matching any NaN (payloads are not fixed)."""
    if np.isnan(want):
        return bool(np.isnan(got))
    return got == want and np.signbit(got) == np.signbit(want)


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("vals,mx,mn", IEEE_2019_CASES)
def test_allreduce_max_min_special_values_follow_ieee754_2019(dtype, vals, mx, mn):
    xs = [from_f32_lib(np.array([v], np.float32), dtype) for v in vals]
    got_mx = to_f64(oracle.allreduce(xs, dtype, "max")[0], dtype)[0]
    got_mn = to_f64(oracle.allreduce(xs, dtype, "min")[0], dtype)[0]
    assert _same_value(got_mx, mx), (vals, got_mx)
    assert _same_value(got_mn, mn), (vals, got_mn)


def test_allreduce_max_min_propagate_nan_like_numpy():
    """A NaN anywhere among the ranks gives NaN at that element, as
    numpy.maximum / numpy.minimum document for a NaN operand; elsewhere the
    values are numpy's."""
    g = np.random.default_rng(12)
    xs = [g.standard_normal(4000).astype(np.float32) for _ in range(5)]
    for r, x in enumerate(xs):
        x[g.random(4000) < 0.02] = np.nan
    ref_mx, ref_mn = np.maximum.reduce(xs), np.minimum.reduce(xs)
    mx = oracle.allreduce(xs, "fp32", "max")[0]
    mn = oracle.allreduce(xs, "fp32", "min")[0]
    assert np.array_equal(np.isnan(mx), np.isnan(ref_mx))
    assert np.array_equal(np.isnan(mn), np.isnan(ref_mn))
    ok = ~np.isnan(ref_mx)
    assert np.array_equal(mx[ok], ref_mx[ok]) and np.array_equal(mn[ok], ref_mn[ok])


def test_allreduce_prod_powers_of_two_exact():
    g = np.random.default_rng(3)
    xs = [(2.0 ** g.integers(-6, 7, size=999) * g.choice([-1, 1], size=999)).astype(np.float32)
          for _ in range(4)]
    expect = np.prod(np.stack([x.astype(np.float64) for x in xs]), axis=0)
    b = [from_f32_lib(x, "bf16") for x in xs]
    assert np.array_equal(to_f64(oracle.allreduce(b, "bf16", "prod")[0], "bf16"), expect)
    assert np.array_equal(oracle.allreduce(xs, "fp32", "prod")[0].astype(np.float64), expect)


def test_reduce_is_allreduce_on_root():
    xs = [synth.gaussian(777, 1.0, 50 + r, "bf16") for r in range(6)]
    assert np.array_equal(oracle.reduce(xs, 4, "bf16"), oracle.allreduce(xs, "bf16")[4])


def test_four_segment_owner_layout():
    """IPC AllReduce blog: 160 KB per GPU on 4 GPUs, segments A-D; GPU j sums
    segment j, so ReduceScatter's chunk j is exactly AllReduce's segment j."""
    g = golden("ar_four_segment_owner.json")
    R, n = g["ranks"], g["elements_per_rank"]
    assert n * 2 == g["bytes_per_rank"]
    xs = [synth.gaussian(n, 1.0, 1000 + r, "bf16") for r in range(R)]
    ar = oracle.allreduce(xs, "bf16")
    rs = oracle.reduce_scatter(xs, "bf16")
    seg = n // R
    for name, owner in g["segment_owner"].items():
        j = g["segments"].index(name)
        assert owner == j
        for r in range(R):
            assert np.array_equal(ar[r][j * seg:(j + 1) * seg], rs[owner])


def test_sequence_parallel_worked_example():
    """Tutorial 5.3 / 7.3: two GPUs, four tokens.  Token t_i is a row of value
    i+1; partial y_i from GPU0 is 10*(i+1), from GPU1 is (i+1)."""
    g = golden("sp_two_gpu_four_token.json")
    H = 6
    tok = {f"t{i}": np.full(H, i + 1, np.float32) for i in range(4)}
    shards = [np.concatenate([tok[t] for t in g["shards"][str(r)]]) for r in range(2)]
    ag = oracle.all_gather(shards)
    for r in range(2):
        want = np.concatenate([tok[t] for t in g["allgather_result"][str(r)]])
        assert np.array_equal(ag[r], want)
    parts = [np.concatenate([np.full(H, 10 * (i + 1), np.float32) for i in range(4)]),
             np.concatenate([np.full(H, (i + 1), np.float32) for i in range(4)])]
    y = {f"y{i}": np.full(H, 11 * (i + 1), np.float32) for i in range(4)}
    rs = oracle.reduce_scatter(parts, "fp32")
    for r in range(2):
        want = np.concatenate([y[t] for t in g["reducescatter_result"][str(r)]])
        assert np.array_equal(rs[r], want)


# ------------------------------------------------- Gather / Scatter / Broadcast

@pytest.mark.parametrize("R,outer,inner", [(8, 16, 19), (3, 1, 5), (1, 4, 4), (5, 7, 1)])
def test_gather_is_last_axis_concatenate(R, outer, inner):
    xs = [synth.gaussian((outer, inner), 2.0, 4000 + r, "fp32") for r in range(R)]
    out = oracle.gather(xs, root=0)
    assert np.array_equal(out, np.concatenate(xs, axis=-1))


def test_gather_of_scatter_is_identity():
    R = 7
    x = synth.random_bits(R * 333, 4, 9)
    chunks = oracle.scatter(x, R, root=2)
    back = oracle.gather([c.reshape(1, -1) for c in chunks], root=2)
    assert np.array_equal(back.reshape(-1), x)


def test_broadcast_every_rank_equals_root():
    R, root = 8, 7
    ids = synth.uniform_int32(256, 0, 152064, 4107)
    poison = [np.full(256, 0x5EADBEEF, np.int32) for _ in range(R)]
    poison[root] = ids                      # root passes its own buffer
    outs = oracle.broadcast(ids, R, root, outs=poison)
    for r in range(R):
        assert np.array_equal(outs[r], ids)
    assert outs[root] is ids


def test_broadcast_equals_owner_slice_of_padded_allgather():
    """sglang 33307 digest: the single-image broadcast from the owner is
    bitwise equal to the owner's slice of the pad-to-max AllGather."""
    R, owner, n_tok, H, max_len = 4, 2, 37, 8, 50
    emb = synth.gaussian((n_tok, H), 1.0, 77, "bf16")
    padded = [np.zeros((max_len, H), np.uint16) for _ in range(R)]
    padded[owner][:n_tok] = emb
    ag = oracle.all_gather([p.reshape(-1) for p in padded])
    via_ag = ag[0].reshape(R, max_len, H)[owner, :n_tok]
    via_bc = oracle.broadcast(emb, R, owner)
    for r in range(R):
        assert np.array_equal(via_bc[r], via_ag)


# --------------------------------------------------------------- All-to-All-v

def _random_counts(R, rows, seed):
    g = np.random.default_rng(seed)
    return g.integers(0, rows + 1, size=(R, R)).astype(np.int64)


@pytest.mark.parametrize("R", [1, 2, 3, 8])
def test_a2av_transposed_counts_restore_input(R):
    W = 5
    counts = _random_counts(R, 6, R)
    sd, rd = oracle.packed_displs(counts)
    send_rows = counts.sum(axis=1)
    recv_rows = counts.sum(axis=0)
    sends = [synth.random_bits(int(send_rows[s]) * W, 2, 30 + s) for s in range(R)]
    recvs = oracle.all_to_all_v(sends, counts, sd, rd, recv_rows, W)
    back = oracle.all_to_all_v(recvs, counts.T.copy(), rd, sd, send_rows, W)
    for s in range(R):
        assert np.array_equal(back[s], sends[s])


@pytest.mark.parametrize("R", [2, 4, 8])
def test_a2av_uniform_is_block_transpose(R):
    n = 12
    sends = [synth.random_bits(R * n, 4, 70 + s) for s in range(R)]
    counts = np.full((R, R), n, np.int64)
    sd, rd = oracle.packed_displs(counts)
    recvs = oracle.all_to_all_v(sends, counts, sd, rd, counts.sum(axis=0), 1)
    blocks = np.stack(sends).reshape(R, R, n).transpose(1, 0, 2)
    for d in range(R):
        assert np.array_equal(recvs[d], blocks[d].reshape(-1))


def test_a2av_three_rank_figure():
    g = golden("a2a_three_rank_figure.json")
    R = g["ranks"]
    label = {f"{s}->{d}": 100 * s + d for s in range(R) for d in range(R)}
    sends = [np.array([label[b] for b in g["before"][str(s)]], np.int32) for s in range(R)]
    counts = np.ones((R, R), np.int64)
    sd, rd = oracle.packed_displs(counts)
    recvs = oracle.all_to_all_v(sends, counts, sd, rd, counts.sum(axis=0), 1)
    for d in range(R):
        assert list(recvs[d]) == [label[b] for b in g["after"][str(d)]]


def test_a2av_single_rank_is_copy():
    """sglang 27492 digest: world size 1 degenerates to a copy."""
    x = synth.random_bits(40, 2, 1)
    c = np.array([[8]], np.int64)
    out = oracle.all_to_all_v([x], c, [[0]], [[0]], [8], 5)
    assert np.array_equal(out[0], x)


def test_a2av_exhaustive_two_rank_counts():
    """Every 2x2 count matrix with entries in {0,1,2}: brute force with lists."""
    W = 3
    for flat in itertools.product(range(3), repeat=4):
        counts = np.array(flat, np.int64).reshape(2, 2)
        sd, rd = oracle.packed_displs(counts)
        rows = [[(s, j) for j in range(int(counts[s].sum()))] for s in range(2)]
        sends = [np.array([[10 * s + j] * W for (s, j) in rows[s]], np.int32).reshape(-1)
                 for s in range(2)]
        recvs = oracle.all_to_all_v(sends, counts, sd, rd, counts.sum(axis=0), W)
        for d in range(2):
            want = []
            for s in range(2):                     # grouped by ascending source
                start = sum(int(counts[s][dd]) for dd in range(d))
                for j in range(int(counts[s][d])):
                    want += [10 * s + start + j] * W
            assert list(recvs[d]) == want, flat


def test_a2av_rejects_bad_layouts():
    x = [np.zeros(4, np.int32)] * 2
    c = np.array([[2, 2], [2, 2]], np.int64)
    sd, rd = oracle.packed_displs(c)
    with pytest.raises(oracle.OracleError):          # receive capacity too small
        oracle.all_to_all_v(x, c, sd, rd, [3, 4], 1)
    with pytest.raises(oracle.OracleError):          # overlapping receive blocks
        oracle.all_to_all_v(x, c, sd, np.zeros((2, 2), np.int64), [4, 4], 1)


# ---------------------------------------------------------------------- MoE

@pytest.mark.parametrize("R,E,T,K", [(2, 4, 5, 1), (8, 256, 64, 8), (4, 16, 33, 3), (1, 8, 10, 2)])
def test_moe_layout_is_stable_argsort(R, E, T, K):
    ids = [np.random.default_rng(s).integers(0, E, size=(T, K)).astype(np.int32) for s in range(R)]
    lay = oracle.moe_layout(ids, E)
    per = E // R
    for s in range(R):
        f = ids[s].reshape(-1)
        order = np.argsort(f, kind="stable")
        inv = np.empty_like(order)
        inv[order] = np.arange(f.size)
        assert np.array_equal(lay["pos"][s].reshape(-1), inv)
        cnt = np.bincount(f, minlength=E)
        assert np.array_equal(lay["expert_counts"][s], cnt)
        assert np.array_equal(lay["sendcounts"][s], cnt.reshape(R, per).sum(axis=1))
        assert lay["sendcounts"][s].sum() == T * K
        assert np.array_equal(lay["sdispls"][s],
                              np.concatenate([[0], np.cumsum(lay["sendcounts"][s])[:-1]]))
    for d in range(R):
        col = lay["sendcounts"][:, d]
        assert np.array_equal(lay["rdispls"][d], np.concatenate([[0], np.cumsum(col)[:-1]]))


def test_moe_two_rank_four_expert_example():
    """Tutorial 8.4: rank 0 holds tA->E2, tB->E0; rank 1 holds tC->E1, tD->E3.
    After dispatch rank 0 computes [tB, tC] and rank 1 computes [tA, tD]."""
    g = golden("moe_two_rank_four_expert.json")
    R, E, H = g["ranks"], g["experts"], 4
    names = {r: g["tokens"][str(r)] for r in range(R)}
    val = {n: np.full(H, 0x3F80 + i, np.uint16) for i, n in enumerate("tA tB tC tD".split())}
    xs = [np.stack([val[n] for n in names[r]]) for r in range(R)]
    ids = [np.array([[g["route"][n]] for n in names[r]], np.int32) for r in range(R)]
    w = [np.ones((2, 1), np.float32) for _ in range(R)]
    res = oracle.moe_pipeline(xs, ids, w, E)
    for d in range(R):
        want = np.stack([val[n] for n in g["computed_on"][str(d)]])
        assert np.array_equal(res["recvs"][d].reshape(-1, H), want)
        for n in g["computed_on"][str(d)]:
            assert g["expert_owner"][str(g["route"][n])] == d


def test_moe_expert_scale_exact_product():
    """y = rne(x * (1 + e/256)) with the product exact: fp64 product + torch cast."""
    R, E, T, K, H = 2, 8, 16, 2, 32
    ids = [np.random.default_rng(s).integers(0, E, size=(T, K)).astype(np.int32) for s in range(R)]
    xs = [synth.gaussian((T, H), 1.0, 10 + s, "bf16") for s in range(R)]
    w = [np.ones((T, K), np.float32)] * R
    res = oracle.moe_pipeline(xs, ids, w, E)
    lay = res["layout"]
    for d in range(R):
        rows = res["recvs"][d].reshape(-1, H)
        ys = res["ys"][d].reshape(-1, H)
        r = 0
        for s in range(R):
            for e in range(d * (E // R), (d + 1) * (E // R)):
                for _ in range(lay["expert_counts"][s][e]):
                    prod = to_f64(rows[r], "bf16") * (1.0 + e / 256.0)
                    assert np.array_equal(ys[r], from_f32_lib(prod.astype(np.float32), "bf16"))
                    if e == 0:
                        assert np.array_equal(ys[r], rows[r])
                    r += 1


def test_moe_round_trip_one_hot_on_expert_zero():
    """Every token routes slot 0 to expert 0 with weight 1 (others weight 0):
    the full dispatch -> expert -> return -> combine gives x back exactly."""
    R, E, T, K, H = 4, 16, 40, 4, 24
    g = np.random.default_rng(2)
    ids = []
    for s in range(R):
        a = g.integers(1, E, size=(T, K)).astype(np.int32)
        a[:, 0] = 0
        ids.append(a)
    w = [np.tile(np.array([1, 0, 0, 0], np.float32), (T, 1)) for _ in range(R)]
    xs = [synth.gaussian((T, H), 1.0, 20 + s, "bf16") for s in range(R)]
    res = oracle.moe_pipeline(xs, ids, w, E)
    for s in range(R):
        assert np.array_equal(res["outs"][s], xs[s])


def test_moe_one_hot_on_expert_e():
    R, E, T, K, H = 2, 8, 30, 3, 16
    g = np.random.default_rng(5)
    ids = [np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32) for _ in range(R)]
    w = [np.tile(np.array([0, 1, 0], np.float32), (T, 1)) for _ in range(R)]
    xs = [synth.gaussian((T, H), 1.0, 60 + s, "bf16") for s in range(R)]
    res = oracle.moe_pipeline(xs, ids, w, E)
    for s in range(R):
        e = ids[s][:, 1].astype(np.float64)[:, None]
        want = from_f32_lib((to_f64(xs[s], "bf16") * (1 + e / 256)).astype(np.float32), "bf16")
        assert np.array_equal(res["outs"][s], want)


def test_moe_combine_closed_form_bound():
    """With bf16 unit roundoff u = 2^-8 and gate weights >= 0, each expert
    output y_k = rne(x s_k) is within u |x| s_k of x s_k, the fp32 fold adds at
    most K 2^-24 relative, and the final rounding at most u of the sum:
    |out - x S| <= u |x| S + u |x| S (1 + u) + K 2^-23 |x| S,  S = sum w_k s_k."""
    R, E, T, K, H = 8, 256, 32, 8, 64
    ids, ws = [], []
    for s in range(R):
        i, w = synth.zipf_routing(T, E, K, seed=5100 + s)
        ids.append(i)
        ws.append(w)
    xs = [synth.gaussian((T, H), 1.0, 5000 + s, "bf16") for s in range(R)]
    res = oracle.moe_pipeline(xs, ids, ws, E)
    for s in range(R):
        scale = (ws[s].astype(np.float64) * (1 + ids[s] / 256.0)).sum(axis=1)[:, None]
        x = to_f64(xs[s], "bf16")
        exact = x * scale
        out = to_f64(res["outs"][s], "bf16")
        u = 2.0 ** -8
        a = np.abs(exact)
        bound = u * a + u * a * (1 + u) + K * 2.0 ** -23 * a + 2.0 ** -130
        assert np.all(np.abs(out - exact) <= bound)
        # a dropped expert term is far outside the bound for most elements
        drop = (ws[s][:, 1:].astype(np.float64) * (1 + ids[s][:, 1:] / 256.0)).sum(axis=1)[:, None]
        assert np.mean(np.abs(x * drop - exact) > bound) > 0.9


# ---------------------------------------- uniform all-to-all, Ulysses re-shard

@pytest.mark.parametrize("R", [1, 2, 3, 8])
def test_uniform_all_to_all_is_block_transpose(R):
    n = 7
    xs = [synth.random_bits(R * n, 2, 80 + s) for s in range(R)]
    outs = oracle.all_to_all(xs)
    blocks = np.stack(xs).reshape(R, R, n).transpose(1, 0, 2)
    for d in range(R):
        assert np.array_equal(outs[d], blocks[d].reshape(-1))
    # it is All-to-All-v with equal counts
    counts = np.full((R, R), n, np.int64)
    sd, rd = oracle.packed_displs(counts)
    v = oracle.all_to_all_v(xs, counts, sd, rd, counts.sum(axis=0), 1)
    for d in range(R):
        assert np.array_equal(outs[d], v[d])


def test_uniform_all_to_all_single_rank_is_copy():
    x = synth.random_bits(33, 4, 3)
    assert np.array_equal(oracle.all_to_all([x])[0], x)


@pytest.mark.parametrize("R,SL,H,D", [(1, 3, 4, 2), (2, 4, 4, 3), (4, 5, 8, 16), (8, 3, 32, 8)])
def test_ulysses_matches_concat_and_head_slice(R, SL, H, D):
    """to_heads: rank d's result is the full sequence (ranks' chunks in rank
    order) of heads [d*H/R, (d+1)*H/R) -- numpy concatenate + slice."""
    xs = [synth.random_bits((SL, H, D), 2, 200 + s) for s in range(R)]
    ys = oracle.ulysses(xs, SL, H, D, to_heads=True)
    full = np.concatenate(xs, axis=0)                # [R*SL, H, D]
    HR = H // R
    for d in range(R):
        assert np.array_equal(ys[d].reshape(R * SL, HR, D), full[:, d * HR:(d + 1) * HR, :])
    back = oracle.ulysses(ys, SL, H, D, to_heads=False)
    for s in range(R):
        assert np.array_equal(back[s], xs[s].reshape(-1))


def test_ulysses_with_one_sequence_row_is_the_uniform_all_to_all():
    R, H, D = 4, 8, 5
    xs = [synth.random_bits((1, H, D), 4, 300 + s) for s in range(R)]
    assert all(np.array_equal(a, b) for a, b in
               zip(oracle.ulysses(xs, 1, H, D, True), oracle.all_to_all(xs)))


# -------------------------------------------- context-parallel LSE merge

def _partial_attention(q, k, v):
    """fp64 softmax attention of queries q [T, D] over keys k [N, D]: returns
    (o [T, D], lse [T]).  An empty key set gives o = 0, lse = -inf."""
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)
    s = q @ k.T
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    z = p.sum(axis=1, keepdims=True)
    return (p @ v) / z, (m + np.log(z))[:, 0]


@pytest.mark.parametrize("R,N", [(1, 40), (2, 64), (4, 100), (8, 333)])
def test_lse_merge_reproduces_full_attention(R, N):
    """Attention over all keys = the merge of attention over R key chunks
    (independent full-softmax formulation, numpy fp64)."""
    g = np.random.default_rng(R * 31 + N)
    T, D = 24, 16
    q, k, v = g.normal(size=(T, D)), g.normal(size=(N, D)), g.normal(size=(N, D))
    full_o, full_l = _partial_attention(q, k, v)
    cuts = np.linspace(0, N, R + 1).astype(int)
    parts = [_partial_attention(q, k[a:b], v[a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
    o, l = oracle.lse_merge([p[0].astype(np.float32) for p in parts],
                            [p[1].astype(np.float32) for p in parts], "fp32")
    assert np.allclose(o.reshape(T, D), full_o, rtol=1e-5, atol=1e-6)
    assert np.allclose(l, full_l, rtol=1e-6, atol=1e-5)


def test_lse_merge_with_empty_chunks_and_all_empty_rows():
    g = np.random.default_rng(5)
    T, D, N = 6, 8, 10
    q, k, v = g.normal(size=(T, D)), g.normal(size=(N, D)), g.normal(size=(N, D))
    full_o, full_l = _partial_attention(q, k, v)
    parts = [_partial_attention(q, k[:0], v[:0]), _partial_attention(q, k, v),
             _partial_attention(q, k[:0], v[:0])]
    o, l = oracle.lse_merge([p[0].astype(np.float32) for p in parts],
                            [p[1].astype(np.float32) for p in parts], "fp32")
    assert np.allclose(o.reshape(T, D), full_o, rtol=1e-5, atol=1e-6)
    empty = [_partial_attention(q, k[:0], v[:0])] * 2
    o, l = oracle.lse_merge([p[0].astype(np.float32) for p in empty],
                            [p[1].astype(np.float32) for p in empty], "fp32")
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_lse_merge_single_rank_is_identity_and_equal_lse_is_mean():
    x = synth.gaussian((50, 8), 1.0, 9, "bf16")
    l = np.linspace(-3, 3, 50).astype(np.float32)
    o, lo = oracle.lse_merge([x], [l], "bf16")
    assert np.array_equal(o, x) and np.array_equal(lo, l)
    # equal LSEs on 4 ranks with identical parts: weights 1/4 each -> the part
    o, lo = oracle.lse_merge([x] * 4, [l] * 4, "bf16")
    assert np.array_equal(o, x)
    assert np.allclose(lo, l + np.log(4.0), atol=1e-6)


def test_lse_merge_bf16_rounds_the_exact_mean_once():
    """Equal LSEs on 4 ranks weigh every part by exactly 1/4, so the merged
    value is the exact mean of the parts.  Parts 4, 2^-6, 2^-26, 0 (all bf16)
    have mean 1 + 2^-8 + 2^-28: just above the bf16 tie between 1 and 1 + 2^-7,
    and below half an fp32 ulp above it.  Rounded once (bfloat16 definition)
    it is 1 + 2^-7; rounded to fp32 first it would land on the tie and go to
    1.  Without the 2^-26 part the mean is the tie itself -> 1 (even)."""
    bf = lambda *vals: oracle.f32_to_bf16(np.array(vals, np.float32))
    parts = [bf(4.0, -4.0, 4.0), bf(2.0 ** -6, -(2.0 ** -6), 2.0 ** -6),
             bf(2.0 ** -26, -(2.0 ** -26), 0.0), bf(0.0, 0.0, 0.0)]
    lse = [np.zeros(1, np.float32)] * 4
    o, lo = oracle.lse_merge([p.reshape(1, 3) for p in parts], lse, "bf16")
    assert o.reshape(-1).tolist() == [0x3F81, 0xBF81, 0x3F80]
    assert np.allclose(lo, np.log(4.0), atol=1e-6)


# ------------------------------------------- expert ids outside [0, E)

def _moe_inputs(R, E, T, K, H, seed):
    ids, ws, xs = [], [], []
    for s in range(R):
        i, w = synth.zipf_routing(T, E, K, seed=seed + s)
        ids.append(i)
        ws.append(w)
        xs.append(synth.gaussian((T, H), 1.0, seed + 50 + s, "bf16"))
    return ids, ws, xs


@pytest.mark.parametrize("bad", [-1, 16, 1 << 30, -(1 << 31)])
@pytest.mark.parametrize("col", ["last", "first"])
def test_moe_bad_ids_are_pairs_that_do_not_exist(bad, col):
    """A pair whose id names no expert is skipped: the pipeline with a whole
    top-k column of bad ids equals the pipeline run without that column
    (same counts, displacements and slots, same outputs bit for bit), and
    the bad pairs get slot -1."""
    R, E, T, K, H = 4, 16, 37, 3, 8
    ids, ws, xs = _moe_inputs(R, E, T, K, H, 700)
    keep = slice(0, K - 1) if col == "last" else slice(1, K)
    drop = K - 1 if col == "last" else 0
    bad_ids = [i.copy() for i in ids]
    for i in bad_ids:
        i[:, drop] = bad
    full = oracle.moe_pipeline(xs, bad_ids, ws, E)
    sub = oracle.moe_pipeline(xs, [np.ascontiguousarray(i[:, keep]) for i in ids],
                              [np.ascontiguousarray(w[:, keep]) for w in ws], E)
    for key in ("sendcounts", "sdispls", "rdispls", "expert_counts"):
        assert np.array_equal(full["layout"][key], sub["layout"][key]), key
    for s in range(R):
        assert np.all(full["layout"]["pos"][s][:, drop] == -1)
        assert np.array_equal(full["layout"]["pos"][s][:, keep], sub["layout"]["pos"][s])
        assert np.array_equal(full["outs"][s], sub["outs"][s])


def test_moe_token_with_only_bad_ids_gets_zero():
    """Every pair of a token skipped: no term, the output row is +0."""
    R, E, T, K, H = 2, 8, 10, 2, 8
    ids, ws, xs = _moe_inputs(R, E, T, K, H, 900)
    ids[1][3, :] = [E, -5]
    out = oracle.moe_pipeline(xs, ids, ws, E)["outs"]
    assert np.all(out[1][3] == 0)
    assert np.any(out[1][2] != 0) and np.any(out[0][3] != 0)
