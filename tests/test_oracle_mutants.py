"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source -- a dropped
term, a wrong index or sign, a transposed operand, a wrong rounding -- builds
it, and runs the pin tests against that build.  At least one pin must fail
for every planted mistake; the unmodified source must pass them all.
"""
import pytest

import oracle
import test_oracle_collectives as C
import test_oracle_formats as F

# (name, snippet in coll_oracle.c, replacement, pins that should catch it)
MUTANTS = [
    ("bf16 rounds half up, not to even",
     "u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0x8000u;",
     [lambda: F.test_bf16_round_matches_torch_on_every_low_half()]),
    ("bf16 truncates",
     "u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0u;",
     [lambda: F.test_bf16_round_matches_torch_on_every_low_half()]),
    ("fp16 subnormal quantum off by one binade",
     "double r = rint(a * ldexp(1.0, 24));", "double r = rint(a * ldexp(1.0, 23));",
     [lambda: F.test_f16_round_matches_numpy()]),
    ("fp16 mantissa rounding drops the tie rule",
     "double r = rint(a * ldexp(1.0, 10 - e));   /* in [1024, 2048] */",
     "double r = floor(a * ldexp(1.0, 10 - e) + 0.5);",
     [lambda: F.test_f16_round_matches_numpy()]),
    ("reduction drops rank 1",
     "for (int r = 1; r < R; r++)\n        acc = apply_fp(op, acc, load_fp(in[r], i, dt));",
     "for (int r = 2; r < R; r++)\n        acc = apply_fp(op, acc, load_fp(in[r], i, dt));",
     [lambda: C.test_allreduce_small_integers_exact("bf16", 3),
      lambda: C.test_allreduce_within_error_bound_of_exact_sum("bf16", 2.0 ** -8, 4)]),
    ("reduction folds in descending rank order",
     "float acc = load_fp(in[0], i, dt);\n    for (int r = 1; r < R; r++)\n        acc = apply_fp(op, acc, load_fp(in[r], i, dt));",
     "float acc = load_fp(in[R - 1], i, dt);\n    for (int r = R - 2; r >= 0; r--)\n        acc = apply_fp(op, acc, load_fp(in[r], i, dt));",
     [lambda: C.test_allreduce_rank_order_is_ascending(),
      lambda: C.test_allreduce_brute_force_tiny(3, 17)]),
    ("sum subtracts",
     "case O_SUM:  return acc + x;", "case O_SUM:  return acc - x;",
     [lambda: C.test_allreduce_small_integers_exact("fp32", 3)]),
    ("max and min swapped",
     "case O_MAX:  return fmax_def(acc, x);", "case O_MAX:  return fmin_def(acc, x);",
     [lambda: C.test_allreduce_max_min_match_numpy("bf16")]),
    ("max ignores a NaN operand (IEEE 754-2008 maxNum)",
     "static float fmax_def(float a, float b)\n{\n    if (isnan(a) || isnan(b)) return bits_to_f32(0x7FC00000u);",
     "static float fmax_def(float a, float b)\n{\n    if (isnan(a)) return b;\n    if (isnan(b)) return a;",
     [lambda: C.test_allreduce_max_min_propagate_nan_like_numpy()]),
    ("max of equal zeros keeps the first operand",
     "if (a == b) return signbit(a) ? b : a;", "if (a == b) return a;",
     [lambda: C.test_allreduce_max_min_special_values_follow_ieee754_2019(
         "fp32", [-0.0, +0.0], +0.0, -0.0)]),
    ("min of equal zeros keeps the first operand",
     "if (a == b) return signbit(a) ? a : b;", "if (a == b) return a;",
     [lambda: C.test_allreduce_max_min_special_values_follow_ieee754_2019(
         "fp32", [+0.0, -0.0], +0.0, -0.0)]),
    ("ReduceScatter chunk index transposed",
     "reduce_element(R, in, (size_t)r * recvcount + i, out[r], i, dt, op);",
     "reduce_element(R, in, i * (size_t)R + (size_t)r, out[r], i, dt, op);",
     [lambda: C.test_allreduce_equals_allgather_of_reducescatter("bf16", 4),
      lambda: C.test_four_segment_owner_layout()]),
    ("AllGather copies the receiver's own shard",
     "memcpy((char *)out[r] + (size_t)q * n, in[q], n);",
     "memcpy((char *)out[r] + (size_t)q * n, in[r], n);",
     [lambda: C.test_sequence_parallel_worked_example()]),
    ("Gather concatenates along the first axis",
     "memcpy((char *)out_root + (o * (size_t)R + (size_t)q) * n,",
     "memcpy((char *)out_root + ((size_t)q * outer + o) * n,",
     [lambda: C.test_gather_is_last_axis_concatenate(8, 16, 19)]),
    ("Scatter sends chunk 0 to everyone",
     "memcpy(out[r], (const char *)in_root + (size_t)r * n, n);",
     "memcpy(out[r], (const char *)in_root, n);",
     [lambda: C.test_gather_of_scatter_is_identity()]),
    ("Broadcast skips rank 0",
     "for (int r = 0; r < R; r++)\n        if (out[r] != in_root)",
     "for (int r = 1; r < R; r++)\n        if (out[r] != in_root)",
     [lambda: C.test_broadcast_every_rank_equals_root(),
      lambda: C.test_broadcast_equals_owner_slice_of_padded_allgather()]),
    ("A2A-v reads the receive displacement transposed",
     "memcpy((char *)recv[d] + (size_t)(rdispls[d * R + s] + j) * row_bytes,",
     "memcpy((char *)recv[d] + (size_t)(rdispls[s * R + d] + j) * row_bytes,",
     [lambda: C.test_a2av_three_rank_figure(),
      lambda: C.test_a2av_exhaustive_two_rank_counts()]),
    ("A2A-v drops the last row of each block",
     "for (int64_t j = 0; j < counts[s * R + d]; j++)",
     "for (int64_t j = 0; j + 1 < counts[s * R + d]; j++)",
     [lambda: C.test_a2av_transposed_counts_restore_input(3)]),
    ("MoE slots ignore earlier entries of the same expert",
     "pos[s][i] = (int32_t)(off[e] + seen[e]);\n            seen[e]++;",
     "pos[s][i] = (int32_t)(off[e] + seen[e]);",
     [lambda: C.test_moe_layout_is_stable_argsort(4, 16, 33, 3)]),
    ("MoE receive displacements scanned over destinations",
     "for (int s = 0; s < R; s++) { rdispls[d * R + s] = acc; acc += sendcounts[s * R + d]; }",
     "for (int s = 0; s < R; s++) { rdispls[d * R + s] = acc; acc += sendcounts[d * R + s]; }",
     [lambda: C.test_moe_layout_is_stable_argsort(4, 16, 33, 3)]),
    ("MoE expert placement interleaved instead of contiguous",
     "for (int e = d * per; e < (d + 1) * per; e++) c += cnt[e];",
     "for (int e = d; e < E; e += R) c += cnt[e];",
     [lambda: C.test_moe_two_rank_four_expert_example(),
      lambda: C.test_moe_layout_is_stable_argsort(4, 16, 33, 3)]),
    ("test expert scales by e/128",
     "float scale = 1.0f + (float)e / 256.0f;", "float scale = 1.0f + (float)e / 128.0f;",
     [lambda: C.test_moe_expert_scale_exact_product()]),
    ("combine drops the last k",
     "for (int k = 0; k < K; k++) {\n                    size_t i = (size_t)t * K + k;",
     "for (int k = 0; k + 1 < K; k++) {\n                    size_t i = (size_t)t * K + k;",
     [lambda: C.test_moe_combine_closed_form_bound()]),
    ("combine ignores the gate weight",
     "float prod = w[s][i] * oracle_bf16_to_f32(row[c]);",
     "float prod = oracle_bf16_to_f32(row[c]);",
     [lambda: C.test_moe_round_trip_one_hot_on_expert_zero()]),
    ("all-to-all takes chunk s instead of chunk d",
     "memcpy((char *)out[d] + (size_t)s * b, (const char *)in[s] + (size_t)d * b, b);",
     "memcpy((char *)out[d] + (size_t)s * b, (const char *)in[s] + (size_t)s * b, b);",
     [lambda: C.test_uniform_all_to_all_is_block_transpose(3)]),
    ("re-shard mixes head and rank order",
     "size_t xi = (t * H + (size_t)d * HR + hh) * D + c;",
     "size_t xi = (t * H + hh * (size_t)R + (size_t)d) * D + c;",
     [lambda: C.test_ulysses_matches_concat_and_head_slice(4, 5, 8, 16)]),
    ("LSE merge forgets to normalise the weights",
     "acc += (e[r] / s) * (double)load_fp(o_parts[r], i * D + c, dt);",
     "acc += e[r] * (double)load_fp(o_parts[r], i * D + c, dt);",
     [lambda: C.test_lse_merge_reproduces_full_attention(4, 100)]),
    ("LSE merge drops the max shift in L",
     "L = m + log(s);", "L = log(s);",
     [lambda: C.test_lse_merge_reproduces_full_attention(4, 100)]),
    ("LSE merge rounds through fp32 before bf16 (two roundings)",
     "((uint16_t *)o_out[r])[i * D + c] = oracle_f64_to_bf16(acc);",
     "((uint16_t *)o_out[r])[i * D + c] = oracle_f32_to_bf16((float)acc);",
     [lambda: C.test_lse_merge_bf16_rounds_the_exact_mean_once()]),
    ("fp64 -> bf16 subnormal quantum off by one binade",
     "double r = rint(a * ldexp(1.0, 133));", "double r = rint(a * ldexp(1.0, 132));",
     [lambda: F.test_f64_to_bf16_matches_a_search_of_the_value_grid()]),
    ("fp64 -> bf16 rounds ties away from zero",
     "double r = rint(a * ldexp(1.0, 7 - e));    /* in [128, 256] */",
     "double r = floor(a * ldexp(1.0, 7 - e) + 0.5);",
     [lambda: F.test_f64_to_bf16_matches_a_search_of_the_value_grid()]),
]


def _caught(checks):
    for chk in checks:
        try:
            chk()
        except (AssertionError, oracle.OracleError):
            return True
    return False


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def test_unmodified_source_passes_the_pins(workdir):
    path = oracle.compile_variant(oracle.source_text(), str(workdir / "clean.so"))
    with oracle.using_library(path):
        for _, _, _, checks in MUTANTS:
            assert not _caught(checks)


@pytest.mark.parametrize("idx", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(idx, workdir):
    name, old, new, checks = MUTANTS[idx]
    src = oracle.source_text()
    assert src.count(old) == 1, f"snippet for '{name}' must occur exactly once"
    path = oracle.compile_variant(src.replace(old, new), str(workdir / f"m{idx}.so"))
    with oracle.using_library(path):
        assert _caught(checks), f"planted mistake not caught: {name}"
