"""CPU checks of the C-ABI boundary: the library loads, exports every entry
point include/coll.h declares, and rejects bad arguments on the host before
touching the GPU (so these calls are safe without one)."""
import ctypes
import os
import re

import pytest

from collective_communication_amd import coll

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    with open(os.path.join(ROOT, "include", "coll.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coll_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(coll.LIB_PATH):
        from collective_communication_amd import build
        build.build()
    return coll.lib()


def test_every_declared_symbol_is_exported(L):
    syms = declared_symbols()
    assert len(syms) >= 13
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(coll.SIGNATURES)


def test_status_strings(L):
    for st in (0, -1, -2, -3, 5):
        assert L.coll_status_string(st)


NULL = None


@pytest.mark.parametrize("R", [0, -1, 17, 1000])
def test_rank_count_rejected(L, R):
    assert L.coll_allreduce(R, NULL, NULL, 8, 0, 0, NULL) == -1
    assert L.coll_reduce_scatter(R, NULL, NULL, 8, 0, 0, NULL) == -1
    assert L.coll_all_gather(R, NULL, NULL, 8, 0, NULL) == -1
    assert L.coll_gather(R, NULL, NULL, 0, 1, 8, 0, NULL) == -1
    assert L.coll_broadcast(R, NULL, NULL, 0, 8, 0, NULL) == -1
    assert L.coll_all_to_all_v(R, NULL, NULL, NULL, NULL, NULL, 8, 0, 0, NULL, NULL, NULL) == -1


def test_zero_count_is_a_no_op(L):
    assert L.coll_allreduce(4, NULL, NULL, 0, 0, 0, NULL) == 0
    assert L.coll_reduce_scatter(4, NULL, NULL, 0, 0, 0, NULL) == 0
    assert L.coll_all_gather(4, NULL, NULL, 0, 0, NULL) == 0
    assert L.coll_gather(4, NULL, NULL, 0, 0, 8, 0, NULL) == 0
    assert L.coll_broadcast(4, NULL, NULL, 0, 0, 0, NULL) == 0
    assert L.coll_moe_permute(4, NULL, NULL, 0, 8, 16, 0, NULL, NULL) == 0


def test_null_pointers_rejected(L):
    assert L.coll_allreduce(2, NULL, NULL, 8, 0, 0, NULL) == -1
    two = (ctypes.c_void_p * 2)(0x1000, 0)          # second rank NULL
    ok = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert L.coll_allreduce(2, two, ok, 8, 0, 0, NULL) == -1
    assert L.coll_allreduce(2, ok, two, 8, 0, 0, NULL) == -1
    assert L.coll_broadcast(2, NULL, ok, 0, 8, 0, NULL) == -1
    assert L.coll_gather(2, ok, NULL, 0, 1, 8, 0, NULL) == -1


def test_root_range(L):
    ok = (ctypes.c_void_p * 4)(0x1000, 0x2000, 0x3000, 0x4000)
    for root in (-1, 4, 99):
        assert L.coll_broadcast(4, 0x1000, ok, root, 8, 0, NULL) == -1
        assert L.coll_gather(4, ok, 0x1000, root, 1, 8, 0, NULL) == -1


def test_dtype_and_op_rejected(L):
    assert L.coll_allreduce(2, NULL, NULL, 8, 7, 0, NULL) == -1
    assert L.coll_allreduce(2, NULL, NULL, 8, 0, 9, NULL) == -2
    assert L.coll_reduce_scatter(2, NULL, NULL, 8, 0, -1, NULL) == -2
    assert L.coll_moe_expert_scale(2, NULL, NULL, NULL, 4, 8, 2, 0, NULL, NULL, 0, NULL) == -2   # fp32
    assert L.coll_moe_combine(2, NULL, NULL, NULL, 4, 2, 8, 1, NULL, NULL) == -2


def test_size_overflow_rejected(L):
    ok = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert L.coll_allreduce(2, ok, ok, 1 << 62, 0, 0, NULL) == -1


def test_moe_workspace_and_layout_validation(L):
    assert L.coll_moe_workspace_bytes(8, 4096, 8, 256) > 8 * 256 * 4
    assert L.coll_moe_workspace_bytes(8, 4096, 8, 250) == 0      # E % R != 0
    assert L.coll_moe_workspace_bytes(8, 4096, 8, 2048) == 0     # E > 1024
    assert L.coll_moe_workspace_bytes(8, 1 << 28, 8, 256) == 0   # T*K >= 2^31
    assert L.coll_moe_workspace_bytes(3, 10, 0, 3) == 0
    # workspace too small -> rejected before any launch
    t = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert L.coll_moe_layout(2, t, 10, 2, 4, 0x100, 0x200, 0x300, 0x400, t, 0x1000, 16, NULL) == -1
    # misaligned workspace
    need = L.coll_moe_workspace_bytes(2, 10, 2, 4)
    assert L.coll_moe_layout(2, t, 10, 2, 4, 0x100, 0x200, 0x300, 0x400, t, 0x1008, need, NULL) == -1


def test_moe_layout_noalloc_validation(L):
    """The no-allocation layout refuses, on the host, any size whose workspace
    would exceed its per-GPU array, and the usual bad arguments."""
    assert _header_define("COLL_MOE_NOALLOC_MAX_BYTES").strip() == "(4u << 20)"
    limit = 4 << 20
    t16 = (ctypes.c_void_p * 16)(*range(0x1000, 0x11000, 0x1000))
    assert L.coll_moe_workspace_bytes(16, 10000, 8, 1024) > limit
    assert L.coll_moe_layout_noalloc(16, t16, 10000, 8, 1024, 0x100, 0x200, 0x300, 0x400, t16,
                                     NULL) == -1
    assert L.coll_moe_workspace_bytes(8, 65000, 8, 256) <= limit       # the header's example
    assert L.coll_moe_workspace_bytes(8, 65409, 8, 256) > limit
    t = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert L.coll_moe_layout_noalloc(2, t, 10, 2, 3, 0x100, 0x200, 0x300, 0x400, t, NULL) == -1
    assert L.coll_moe_layout_noalloc(2, t, 10, 2, 4, NULL, 0x200, 0x300, 0x400, t, NULL) == -1
    assert L.coll_moe_layout_noalloc(0, t, 10, 2, 4, 0x100, 0x200, 0x300, 0x400, t, NULL) == -1


def test_moe_expert_workspace_validation(L):
    # two int64 tables of R*E entries, rounded up to 256 bytes ...
    assert L.coll_moe_expert_workspace_bytes(8, 256, 0) == 8 * 256 * 16
    assert L.coll_moe_expert_workspace_bytes(2, 4, 0) == 256
    assert L.coll_moe_expert_workspace_bytes(16, 1024, 0) == 16 * 1024 * 16
    # ... then 8 bytes per row of the capacity, rounded up to 256
    assert L.coll_moe_expert_workspace_bytes(8, 256, 262144) == 8 * 256 * 16 + 262144 * 8
    assert L.coll_moe_expert_workspace_bytes(2, 4, 1) == 256 + 256
    assert L.coll_moe_expert_workspace_bytes(2, 4, 33) == 256 + 512
    assert L.coll_moe_expert_workspace_bytes(8, 250, 0) == 0    # E % R != 0
    assert L.coll_moe_expert_workspace_bytes(8, 2048, 0) == 0   # E > 1024
    assert L.coll_moe_expert_workspace_bytes(17, 17, 0) == 0    # R > 16
    assert L.coll_moe_expert_workspace_bytes(2, 4, 1 << 62) == 0  # absurd capacity
    t = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    need = L.coll_moe_expert_workspace_bytes(2, 4, 0)           # the least any call accepts
    # NULL, misaligned or too small workspace -> rejected before any launch
    assert L.coll_moe_expert_scale(2, t, 0x100, 0x200, 4, 8, 0, 16, NULL, NULL, need, NULL) == -1
    assert L.coll_moe_expert_scale(2, t, 0x100, 0x200, 4, 8, 0, 16, NULL, 0x1008, need, NULL) == -1
    assert L.coll_moe_expert_scale(2, t, 0x100, 0x200, 4, 8, 0, 16, NULL, 0x1000, need - 1, NULL) == -1
    # NULL receive buffer / tables
    z = (ctypes.c_void_p * 2)(0x1000, None)
    assert L.coll_moe_expert_scale(2, z, 0x100, 0x200, 4, 8, 0, 16, NULL, 0x1000, need, NULL) == -1
    assert L.coll_moe_expert_scale(2, t, NULL, 0x200, 4, 8, 0, 16, NULL, 0x1000, need, NULL) == -1
    # hidden 0: nothing to do, nothing launched
    assert L.coll_moe_expert_scale(2, t, 0x100, 0x200, 4, 0, 0, 16, NULL, NULL, 0, NULL) == 0


def test_a2av_workspace_size_and_validation(L):
    def size(R, tiles):          # 32-byte block entries, 2-byte tile indices in
        slots = -(-tiles // 512) * 512                    # groups of 512, rounded to 256
        return -(-(R * R * 32 + slots * 2) // 256) * 256
    # rows of 7168 bf16 (896 sixteen-byte units), 262144 rows of capacity:
    # 64 block entries + 3670016 indices of 64-unit (1 KiB) tiles
    assert L.coll_all_to_all_v_workspace_bytes(8, 262144, 7168, 0) == 64 * 32 + 3670016 * 2
    assert L.coll_all_to_all_v_workspace_bytes(8, 262144, 7, 0) == 0     # 14-byte rows
    assert L.coll_all_to_all_v_workspace_bytes(8, 0, 7168, 0) == 0       # no capacity
    assert L.coll_all_to_all_v_workspace_bytes(17, 10, 8, 0) == 0        # R > 16
    # the descriptor form starts at 192 MiB of receive capacity (the default
    # of COLL_A2A_DESC_MIN_BYTES); below it no workspace is needed
    K = (192 << 20) // 16                                                # rows of 8 bf16
    assert "COLL_A2A_DESC_MIN_BYTES" not in os.environ
    assert L.coll_all_to_all_v_workspace_bytes(2, K - 1, 8, 0) == 0
    assert L.coll_all_to_all_v_workspace_bytes(2, 1, 8, 0) == 0
    need = L.coll_all_to_all_v_workspace_bytes(2, K, 8, 0)
    assert need == size(2, K // 64)
    # one unit more: one tile more, which starts a new group of 512
    assert L.coll_all_to_all_v_workspace_bytes(2, K + 1, 8, 0) == size(2, K // 64 + 1)
    assert size(2, K // 64 + 1) == size(2, K // 64) + 512 * 2
    t = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    # a needed workspace that is NULL, misaligned or too small: rejected
    assert L.coll_all_to_all_v_ws(2, t, 0x100, 0x200, t, 0x300, 8, 0, K, NULL, NULL, NULL, need, NULL) == -1
    assert L.coll_all_to_all_v_ws(2, t, 0x100, 0x200, t, 0x300, 8, 0, K, NULL, NULL, 0x1010, need, NULL) == -1
    assert L.coll_all_to_all_v_ws(2, t, 0x100, 0x200, t, 0x300, 8, 0, K, NULL, NULL, 0x1000, need - 1,
                                  NULL) == -1
    # NULL tables rejected as in coll_all_to_all_v; rows of 0 elements: nothing to do
    assert L.coll_all_to_all_v_ws(2, t, NULL, 0x200, t, 0x300, 8, 0, K, NULL, NULL, 0x1000, need, NULL) == -1
    assert L.coll_all_to_all_v_ws(2, t, 0x100, 0x200, t, 0x300, 0, 0, K, NULL, NULL, NULL, 0, NULL) == 0


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(coll, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(coll, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        coll.lib()


def test_a2av_null_arrays_rejected_but_null_entries_allowed_on_host(L):
    # the pointer arrays themselves are required
    assert L.coll_all_to_all_v(2, NULL, 0x10, 0x20, NULL, 0x30, 8, 0, 0, NULL, NULL, NULL) == -1
    # device count tables are required
    ok = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert L.coll_all_to_all_v(2, ok, NULL, 0x20, ok, 0x30, 8, 0, 0, NULL, NULL, NULL) == -1
    assert L.coll_all_to_all_v(2, ok, 0x10, 0x20, ok, NULL, 8, 0, 0, NULL, NULL, NULL) == -1
    # negative buffer rows are rejected on either side (rows only bound blocks)
    neg = (ctypes.c_int64 * 2)(4, -1)
    assert L.coll_all_to_all_v(2, ok, 0x10, 0x20, ok, 0x30, 8, 0, 0, neg, NULL, NULL) == -1
    assert L.coll_all_to_all_v(2, ok, 0x10, 0x20, ok, 0x30, 8, 0, 0, NULL, neg, NULL) == -1
    assert L.coll_all_to_all_v_reverse(2, ok, 0x10, 0x20, ok, 0x30, 8, 0, 0, neg, NULL, NULL, 0,
                                       NULL) == -1
    # an absurd capacity is rejected (it would overflow the launch size)
    assert L.coll_all_to_all_v(2, ok, 0x10, 0x20, ok, 0x30, 8, 0, 1 << 62, NULL, NULL, NULL) == -1


def test_reduce_and_scatter_validation(L):
    ok = (ctypes.c_void_p * 4)(0x1000, 0x2000, 0x3000, 0x4000)
    assert L.coll_reduce(4, ok, 0x5000, 4, 8, 0, 0, NULL) == -1      # root out of range
    assert L.coll_reduce(4, ok, NULL, 0, 8, 0, 0, NULL) == -1        # no root buffer
    assert L.coll_reduce(4, ok, 0x5000, 0, 8, 0, 7, NULL) == -2      # bad op
    assert L.coll_reduce(4, ok, 0x5000, 0, 0, 0, 0, NULL) == 0       # empty
    assert L.coll_scatter(4, 0x1000, ok, -1, 8, 0, NULL) == -1
    assert L.coll_scatter(4, NULL, ok, 0, 8, 0, NULL) == -1
    holes = (ctypes.c_void_p * 4)(0x1000, 0, 0x3000, 0x4000)
    assert L.coll_scatter(4, 0x9000, holes, 0, 8, 0, NULL) == -1     # NULL only at the root
    assert L.coll_scatter(4, 0x9000, ok, 0, 0, 0, NULL) == 0


def test_all_to_all_and_reshard_validation(L):
    ok = (ctypes.c_void_p * 4)(0x1000, 0x2000, 0x3000, 0x4000)
    assert L.coll_all_to_all(0, ok, ok, 8, 0, NULL) == -1
    assert L.coll_all_to_all(4, ok, ok, 0, 0, NULL) == 0
    assert L.coll_all_to_all(4, NULL, ok, 8, 0, NULL) == -1
    assert L.coll_seq_heads_reshard(4, ok, ok, 16, 6, 128, 0, 1, NULL) == -1   # 6 % 4 != 0
    assert L.coll_seq_heads_reshard(4, ok, ok, 0, 8, 128, 0, 1, NULL) == 0
    assert L.coll_seq_heads_reshard(4, ok, NULL, 16, 8, 128, 0, 1, NULL) == -1


def test_lse_merge_validation(L):
    ok = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert L.coll_lse_merge(2, ok, ok, ok, NULL, 16, 128, 1, NULL) == -2     # fp16 unsupported
    assert L.coll_lse_merge(2, ok, ok, ok, NULL, 0, 128, 0, NULL) == 0
    assert L.coll_lse_merge(2, NULL, ok, ok, NULL, 16, 128, 0, NULL) == -1
    assert L.coll_lse_merge(0, ok, ok, ok, NULL, 16, 128, 0, NULL) == -1


@pytest.mark.parametrize("out_ptrs", [
    (0x10000, 0x20000),          # lse_out[r] == lse_parts[r] (in place)
    (0x90000, 0x10000),          # lse_out[1] == lse_parts[0]
    (0x90000, 0x20000 + 60),     # lse_out[1] starts inside lse_parts[1] (16 rows = 64 B)
    (0x10000 - 60, 0x90000),     # lse_out[0] ends inside lse_parts[0]
])
def test_lse_merge_rejects_lse_outputs_overlapping_inputs(L, out_ptrs):
    """An LSE output that overlaps any LSE input is rejected on the host
    before any launch (a row's inputs could be read after L is stored).
    Disjoint outputs and NULL entries pass these checks; they run in the
    CPU-emulation and GPU tests, since here nothing may launch."""
    o = (ctypes.c_void_p * 2)(0x100000, 0x200000)
    lse_in = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    lse_out = (ctypes.c_void_p * 2)(*out_ptrs)
    assert L.coll_lse_merge(2, o, lse_in, o, lse_out, 16, 128, 0, NULL) == -1


# ------------------------------------------------------------- rank arena

def _header_define(name):
    with open(os.path.join(ROOT, "include", "coll.h")) as f:
        text = f.read()
    return re.search(rf"#define {name} (.+)", text).group(1)


def test_arena_constants_match_header():
    unit = int(_header_define("COLL_ARENA_COLOR_BYTES").rstrip("u"))
    colors = int(_header_define("COLL_ARENA_COLORS").rstrip("u"))
    assert unit == 4096 and colors == 32
    assert _header_define("COLL_ARENA_ALIGN") == "(2u << 20)"
    assert coll.ARENA_ALIGN == 2 << 20


@pytest.mark.parametrize("seed", range(6))
def test_arena_layout_colours_and_no_overlap(L, seed):
    import numpy as np
    g = np.random.default_rng(seed)
    n = int(g.integers(1, 80))
    pick = g.integers(0, 4, size=n)
    sizes = [int(x) for x in np.where(pick == 0, 0, np.where(
        pick == 1, g.integers(1, 5000, size=n),
        np.where(pick == 2, g.integers(1, 64, size=n) << 20, g.integers(1, 1 << 30, size=n))))]
    offs, total = coll.arena_layout(sizes)
    end = 0
    page = coll.ARENA_ALIGN
    for k, (o, b) in enumerate(zip(offs, sizes)):
        assert o % page == (k % 32) * 4096          # its page plus its colour
        assert o - o % page >= end                   # a 2 MiB boundary after the previous end
        assert o - end < page + 32 * 4096            # wastes less than 2 MiB + 128 KiB
        end = o + b
    assert total == end
    # any 32 consecutive buffers start at distinct colours
    for k in range(max(0, n - 31)):
        assert len({(o // 4096) % 32 for o in offs[k:k + 32]}) == min(32, n - k)


def test_arena_layout_edge_cases(L):
    assert coll.arena_layout([]) == ([], 0)
    M = 1 << 20
    assert coll.arena_layout([0, 0, 0]) == ([0, 4096, 2 * M + 8192], 2 * M + 8192)
    assert coll.arena_layout([2 * M, 5, 1]) == ([0, 2 * M + 4096, 4 * M + 8192], 4 * M + 8193)
    offs, total = coll.arena_layout([16 * M] * 3)
    assert offs == [0, 16 * M + 4096, 34 * M + 8192] and total == 50 * M + 8192
    tot = ctypes.c_size_t()
    sz = (ctypes.c_size_t * 2)(8, 8)
    out = (ctypes.c_size_t * 2)()
    assert L.coll_arena_layout(-1, sz, out, ctypes.byref(tot)) == -1
    assert L.coll_arena_layout(2, NULL, out, ctypes.byref(tot)) == -1
    assert L.coll_arena_layout(2, sz, NULL, ctypes.byref(tot)) == -1
    assert L.coll_arena_layout(2, sz, out, NULL) == -1
    huge = (ctypes.c_size_t * 2)(1 << 54, 1 << 54)
    assert L.coll_arena_layout(2, huge, out, ctypes.byref(tot)) == 0
    assert tot.value == (1 << 55) + 4096
    huge = (ctypes.c_size_t * 3)(1 << 55, 1 << 55, 1 << 55)
    out3 = (ctypes.c_size_t * 3)()
    assert L.coll_arena_layout(3, huge, out3, ctypes.byref(tot)) == -1   # past 2^56
    assert L.coll_arena_layout(1, (ctypes.c_size_t * 1)(1 << 56), out, ctypes.byref(tot)) == -1


def test_rank_arena_views_on_host(L):
    import torch
    ins, outs, one = coll.rank_arena([(8, (64, 7168), torch.bfloat16),
                                      (8, 64 * 7168, torch.bfloat16),
                                      (1, (3,), torch.int32)], device="cpu")
    ts = ins + outs + one
    assert [tuple(t.shape) for t in ins] == [(64, 7168)] * 8
    assert [tuple(t.shape) for t in outs] == [(64 * 7168,)] * 8
    assert one[0].dtype == torch.int32 and one[0].numel() == 3
    base = ts[0].data_ptr()
    assert base % coll.ARENA_ALIGN == 0
    spans = sorted((t.data_ptr(), t.data_ptr() + t.numel() * t.element_size()) for t in ts)
    for (a0, a1), (b0, _) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert [(t.data_ptr() // 4096) % 32 for t in ts] == list(range(17))
    for k, t in enumerate(ts):                       # writes land in their own views
        t.view(-1)[:1].fill_(k + 1)
    assert [int(t.view(-1)[0]) for t in ts][:16] == [k + 1 for k in range(16)]


def test_rank_arena_per_buffer_shapes_on_host(L):
    import torch
    (a,), recv = coll.rank_arena([(1, 5, torch.float32),
                                  [((3, 7), torch.bfloat16), ((0, 7), torch.bfloat16),
                                   ((11,), torch.int64)]], device="cpu")
    assert tuple(a.shape) == (5,)
    assert [tuple(t.shape) for t in recv] == [(3, 7), (0, 7), (11,)]
    assert [t.dtype for t in recv] == [torch.bfloat16, torch.bfloat16, torch.int64]
    # (torch reports data_ptr() 0 for the empty view)
    assert [(t.data_ptr() // 4096) % 32 for t in [a] + recv if t.numel()] == [0, 1, 3]


def test_fused_moe_entry_points_validate_on_host(L):
    ok = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    tab = 0x3000                                       # a (never dereferenced) device table
    # bad rank count, topk, tokens
    assert L.coll_moe_dispatch(0, ok, ok, tab, tab, tab, 4, 2, 8, 0, ok, NULL, NULL) == -1
    assert L.coll_moe_dispatch(2, ok, ok, tab, tab, tab, 4, 0, 8, 0, ok, NULL, NULL) == -1
    assert L.coll_moe_dispatch(2, ok, ok, tab, tab, tab, -1, 2, 8, 0, ok, NULL, NULL) == -1
    # zero tokens / zero hidden: no-op
    assert L.coll_moe_dispatch(2, ok, ok, tab, tab, tab, 0, 2, 8, 0, ok, NULL, NULL) == 0
    assert L.coll_moe_dispatch(2, ok, ok, tab, tab, tab, 4, 2, 0, 0, ok, NULL, NULL) == 0
    # missing layout tables or buffers
    assert L.coll_moe_dispatch(2, ok, ok, NULL, tab, tab, 4, 2, 8, 0, ok, NULL, NULL) == -1
    assert L.coll_moe_dispatch(2, ok, ok, tab, tab, NULL, 4, 2, 8, 0, ok, NULL, NULL) == -1
    assert L.coll_moe_dispatch(2, NULL, ok, tab, tab, tab, 4, 2, 8, 0, ok, NULL, NULL) == -1
    assert L.coll_moe_dispatch(2, ok, ok, tab, tab, tab, 4, 2, 8, 0, NULL, NULL, NULL) == -1
    # T*K must stay below 2^31
    assert L.coll_moe_dispatch(2, ok, ok, tab, tab, tab, 1 << 28, 8, 8, 0, ok, NULL, NULL) == -1

    def cr(R=2, recv=ok, pos=ok, sc=tab, w=ok, ids=NULL, T=4, K=2, H=8, dt=0, out=ok, rows=NULL):
        return L.coll_moe_combine_recv(R, recv, pos, sc, tab, tab, w, ids, T, K, H, dt, out, rows,
                                       NULL)
    assert cr(R=17) == -1
    assert cr(K=0) == -1
    assert cr(dt=2) == -2                              # bf16 only
    assert cr(T=0) == 0 and cr(H=0) == 0
    assert cr(sc=NULL) == -1
    assert cr(w=NULL) == -1
    assert cr(out=NULL) == -1
    assert cr(pos=NULL) == -1
    half = (ctypes.c_void_p * 2)(0x1000, 0)
    assert cr(ids=half) == -1                          # ids given: every rank needs them
    # receive rows: a negative entry is rejected, any non-negative one accepted
    assert cr(rows=(ctypes.c_int64 * 2)(5, -1)) == -1
    assert L.coll_moe_dispatch(2, ok, ok, tab, tab, tab, 4, 2, 8, 0, ok,
                               (ctypes.c_int64 * 2)(-3, 0), NULL) == -1


def test_prepare_rejects_a_non_collective():
    with pytest.raises(TypeError):
        coll.prepare(lambda: 3)


def test_plan_keeps_the_arguments_it_was_made_from():
    """A prepared call owns its arguments: tensors created inline for the call
    (whose raw pointers the plan re-issues) stay alive with the plan."""
    import gc
    import weakref
    import torch

    fake = coll.Plan(lambda *a: 0, (), "fake")
    t = torch.empty(4)
    ref = weakref.ref(t)

    def call(x):
        return fake

    plan = coll.prepare(call, t)
    del t
    gc.collect()
    assert ref() is not None and plan is fake
    del plan, fake
    gc.collect()
    assert ref() is None


def test_moe_expert_split_validation(L):
    """coll_moe_expert_scale_build / _apply: the row-descriptor path must
    apply (16-byte rows and buffers, a nonzero capacity, R*E <= 8192, a
    workspace that holds the descriptors); the apply checks its workspace
    against the full size.  Nothing is launched in any of these cases."""
    t = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    cap = 16
    full = L.coll_moe_expert_workspace_bytes(2, 4, cap)
    table = L.coll_moe_expert_workspace_bytes(2, 4, 0)
    assert full > table > 0
    b = L.coll_moe_expert_scale_build
    a = L.coll_moe_expert_scale_apply
    # the path does not apply: no capacity, rows of 5 bf16, a workspace of the
    # tables alone, a buffer off 16-byte alignment
    assert b(2, t, 0x100, 0x200, 4, 8, 0, 0, NULL, 0x1000, full, NULL) == -2
    assert b(2, t, 0x100, 0x200, 4, 5, 0, cap, NULL, 0x1000, full, NULL) == -2
    assert b(2, t, 0x100, 0x200, 4, 8, 0, cap, NULL, 0x1000, table, NULL) == -2
    m = (ctypes.c_void_p * 2)(0x1000, 0x2008)
    assert b(2, m, 0x100, 0x200, 4, 8, 0, cap, NULL, 0x1000, full, NULL) == -2
    assert a(2, t, 4, 8, 0, 0, 0x1000, full, NULL) == -2
    assert a(2, t, 4, 5, 0, cap, 0x1000, full, NULL) == -2
    assert a(2, m, 4, 8, 0, cap, 0x1000, full, NULL) == -2
    # R * E above the LDS table (16 x 1024 entries)
    t16 = (ctypes.c_void_p * 16)(*[0x100000 * (r + 1) for r in range(16)])
    big = L.coll_moe_expert_workspace_bytes(16, 1024, cap)
    assert b(16, t16, 0x100, 0x200, 1024, 8, 0, cap, NULL, 0x1000, big, NULL) == -2
    assert a(16, t16, 1024, 8, 0, cap, 0x1000, big, NULL) == -2
    # bf16 only
    assert b(2, t, 0x100, 0x200, 4, 8, 2, cap, NULL, 0x1000, full, NULL) == -2
    assert a(2, t, 4, 8, 2, cap, 0x1000, full, NULL) == -2
    # workspace NULL, misaligned or below the size; the apply needs the full size
    assert b(2, t, 0x100, 0x200, 4, 8, 0, cap, NULL, NULL, full, NULL) == -1
    assert b(2, t, 0x100, 0x200, 4, 8, 0, cap, NULL, 0x1010, full, NULL) == -1
    assert a(2, t, 4, 8, 0, cap, NULL, full, NULL) == -1
    assert a(2, t, 4, 8, 0, cap, 0x1010, full, NULL) == -1
    assert a(2, t, 4, 8, 0, cap, 0x1000, full - 1, NULL) == -1
    # bad ranks or experts; NULL tables (build) or receive buffers
    assert b(17, t, 0x100, 0x200, 4, 8, 0, cap, NULL, 0x1000, full, NULL) == -1
    assert a(2, t, 3, 8, 0, cap, 0x1000, full, NULL) == -1
    assert b(2, t, NULL, 0x200, 4, 8, 0, cap, NULL, 0x1000, full, NULL) == -1
    assert b(2, t, 0x100, NULL, 4, 8, 0, cap, NULL, 0x1000, full, NULL) == -1
    z = (ctypes.c_void_p * 2)(0x1000, None)
    assert b(2, z, 0x100, 0x200, 4, 8, 0, cap, NULL, 0x1000, full, NULL) == -1
    assert a(2, z, 4, 8, 0, cap, 0x1000, full, NULL) == -1
    # negative receive rows
    neg = (ctypes.c_int64 * 2)(4, -1)
    assert b(2, t, 0x100, 0x200, 4, 8, 0, cap, neg, 0x1000, full, NULL) == -1


def test_a2av_split_descriptor_form_validation(L):
    """coll_all_to_all_v_ws_build / _reverse_build / _ws_copy: the form must
    apply (capacity from the descriptor threshold up, 16-byte rows), and the
    copy checks its workspace as the one-call form does.  Nothing is launched
    in any of these cases."""
    K = (192 << 20) // 16                                   # rows of 8 bf16: the threshold
    need = L.coll_all_to_all_v_workspace_bytes(2, K, 8, 0)
    assert need > 0
    t = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    # below the threshold, or rows of 10 bytes: no descriptor form
    assert L.coll_all_to_all_v_ws_build(2, t, 0x100, 0x200, t, 0x300, 8, 0, K - 1, NULL, NULL,
                                        0x1000, need, NULL) == -2
    assert L.coll_all_to_all_v_ws_build(2, t, 0x100, 0x200, t, 0x300, 5, 0, K, NULL, NULL,
                                        0x1000, need, NULL) == -2
    assert L.coll_all_to_all_v_reverse_build(2, t, 0x100, 0x200, t, 0x300, 8, 0, K - 1, NULL,
                                             NULL, 0x1000, need, NULL) == -2
    assert L.coll_all_to_all_v_ws_copy(2, 8, 0, K - 1, 0x1000, need, NULL) == -2
    assert L.coll_all_to_all_v_ws_copy(2, 5, 0, K, 0x1000, need, NULL) == -2
    # workspace NULL, misaligned or small; bad ranks; NULL tables
    assert L.coll_all_to_all_v_ws_build(2, t, 0x100, 0x200, t, 0x300, 8, 0, K, NULL, NULL,
                                        NULL, need, NULL) == -1
    assert L.coll_all_to_all_v_ws_copy(2, 8, 0, K, NULL, need, NULL) == -1
    assert L.coll_all_to_all_v_ws_copy(2, 8, 0, K, 0x1010, need, NULL) == -1
    assert L.coll_all_to_all_v_ws_copy(2, 8, 0, K, 0x1000, need - 1, NULL) == -1
    assert L.coll_all_to_all_v_ws_copy(17, 8, 0, K, 0x1000, need, NULL) == -1
    assert L.coll_all_to_all_v_ws_build(2, t, NULL, 0x200, t, 0x300, 8, 0, K, NULL, NULL,
                                        0x1000, need, NULL) == -1
