/*
 * coll_oracle.c -- plain, slow CPU definitions of the collectives computed by
 * the collective_communication_amd library.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may call,
 * link or load this file: it is used by the tests, by the smoke check and by
 * the CPU-baseline leg of the benchmark.  It shares no code, header, table or
 * helper with the HIP path.
 *
 * Build: gcc -std=c99 -O2 -ffp-contract=off -fPIC -shared (no fast-math, no
 * -march=native), so every float operation below is one IEEE-754 binary32
 * operation with round-to-nearest-even, in exactly the order written.
 *
 * Sources (cited by page title and section):
 *   [Tut]  "Collective primitives tutorial" (gsyq.cn, news 307221): abstract
 *          and sections 1 Broadcast, 2 Gather, 3 Reduce, 4 Scatter,
 *          5 ReduceScatter, 6 AllReduce, 7 AllGather, 8 All-to-All.
 *   [IPC]  "From NCCL Ring LL to PCIe IPC AllReduce" (hjcheng0602 blog),
 *          section "Pro5000 ?": the four-segment (A-D) owner layout.
 *   [A2A]  sglang PR 27492 digest, all_to_all_single: world size 1 is a copy.
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes):
 *   - sums run in ascending rank order, accumulator seeded with rank 0's value;
 *   - bf16/fp16 inputs are widened exactly to fp32, accumulated in fp32 and
 *     rounded once to the output type, round-to-nearest-even;
 *   - A2A-v uses explicit per-pair row counts and displacements (MPI style),
 *     receive blocks grouped by ascending source rank;
 *   - MoE: experts placed on ranks in contiguous blocks, one dispatched row per
 *     (token, k) pair, rows ordered stably by (expert, token, k), expert op
 *     y = x * (1 + e/256), combine = sum over k ascending of w * y with the
 *     accumulator seeded by the k = 0 product and one final rounding.
 *
 * Parity status: every function here is pinned by CPU tests against closed
 * forms, library routines (numpy / torch casts, concatenate, argsort),
 * invariants from the pages (AllReduce = AllGather after ReduceScatter, Gather
 * after Scatter = identity, A2A-v with transposed counts = identity) and brute
 * force on tiny inputs.  The pages fix no MAX/MIN semantics for NaN and
 * signed zero; these follow the maximum / minimum operations of IEEE 754-2019
 * (a NaN operand gives NaN, -0 orders below +0), pinned to that standard's
 * special cases.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype / op codes: the oracle's own numbering (the tests map names to
 * these; nothing is shared with the library header). */
enum { O_BF16 = 0, O_FP16 = 1, O_FP32 = 2, O_INT32 = 3 };
enum { O_SUM = 0, O_PROD = 1, O_MAX = 2, O_MIN = 3 };

enum { O_OK = 0, O_EINVAL = -1, O_EUNSUP = -2 };

/* ------------------------------------------------------------------ */
/* Number formats, written from the IEEE-754 / bfloat16 definitions.  */
/* ------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16 is the top half of a binary32: widening is exact. */
float oracle_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even.  Adding 0x7FFF plus
 * the lowest kept bit to the full pattern carries into the kept half exactly
 * when the dropped half is above one half ulp, or equal to it with an odd kept
 * part.  Overflow carries into the exponent and lands on +-inf.  NaN is kept
 * NaN (quiet bit forced) since the carry could otherwise turn it into inf. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u = f32_to_bits(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* binary64 -> bfloat16, round to nearest, ties to even, in one step (the
 * LSE merge accumulates in binary64; going through binary32 first would round
 * twice).  From the format's definition: bfloat16 keeps 8 significant bits
 * with binary32's exponent range, so scale |x| until one unit is the
 * bfloat16 quantum of its binade, round that to an integer (rint: ties to
 * even in the default mode) and re-encode.  The scalings are exact. */
uint16_t oracle_f64_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    if (isinf(x))
        return (uint16_t)(sign | 0x7F80u);
    double a = fabs(x);
    if (a < ldexp(1.0, -126)) {
        /* subnormal range: quantum 2^-133; r == 128 encodes the smallest
         * normal (exponent field 1, fraction 0), which is the same pattern */
        double r = rint(a * ldexp(1.0, 133));
        return (uint16_t)(sign | (uint16_t)r);
    }
    int ex;
    frexp(a, &ex);                 /* a = mant * 2^ex, mant in [0.5, 1) */
    int e = ex - 1;                /* a in [2^e, 2^(e+1)) */
    double r = rint(a * ldexp(1.0, 7 - e));    /* in [128, 256] */
    if (r == 256.0) { r = 128.0; e += 1; }
    if (e + 127 >= 255)
        return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | (uint16_t)((e + 127) << 7) | (uint16_t)(r - 128.0));
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);               /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? bits_to_f32(0x7FC00000u) : INFINITY;
    else
        v = ldexpf((float)(1024 + m), e - 25);   /* (1.m) * 2^(e-15) */
    return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even, from the definition:
 * scale |f| so that one unit is the binary16 quantum at its binade, round
 * that to an integer (rint: ties to even in the default mode), re-encode. */
uint16_t oracle_f32_to_f16(float f)
{
    uint16_t sign = (uint16_t)((f32_to_bits(f) >> 16) & 0x8000u);
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00u);
    double a = fabs((double)f);
    if (isinf(f))
        return (uint16_t)(sign | 0x7C00u);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; r == 1024 encodes the smallest
         * normal (exponent field 1, fraction 0), which is the same pattern */
        double r = rint(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)r);
    }
    int ex;
    frexp(a, &ex);                 /* a = mant * 2^ex, mant in [0.5, 1) */
    int e = ex - 1;                /* a in [2^e, 2^(e+1)) */
    double r = rint(a * ldexp(1.0, 10 - e));   /* in [1024, 2048] */
    if (r == 2048.0) { r = 1024.0; e += 1; }
    if (e + 15 >= 31)
        return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(r - 1024.0));
}

/* ------------------------------------------------------------------ */
/* Element access and the reduction operator ([Tut] 3: SUM/MAX/MIN/PROD) */
/* ------------------------------------------------------------------ */

static size_t dtype_size(int dt)
{
    switch (dt) {
    case O_BF16: case O_FP16: return 2;
    case O_FP32: case O_INT32: return 4;
    default: return 0;
    }
}

/* widen element i of a buffer of floating dtype to fp32 (exact) */
static float load_fp(const void *p, size_t i, int dt)
{
    if (dt == O_BF16) return oracle_bf16_to_f32(((const uint16_t *)p)[i]);
    if (dt == O_FP16) return oracle_f16_to_f32(((const uint16_t *)p)[i]);
    return ((const float *)p)[i];
}

static void store_fp(void *p, size_t i, int dt, float v)
{
    if (dt == O_BF16) ((uint16_t *)p)[i] = oracle_f32_to_bf16(v);
    else if (dt == O_FP16) ((uint16_t *)p)[i] = oracle_f32_to_f16(v);
    else ((float *)p)[i] = v;
}

/* MAX/MIN: NaN if either operand is NaN; -0 orders below +0. */
static float fmax_def(float a, float b)
{
    if (isnan(a) || isnan(b)) return bits_to_f32(0x7FC00000u);
    if (a == b) return signbit(a) ? b : a;
    return a > b ? a : b;
}
static float fmin_def(float a, float b)
{
    if (isnan(a) || isnan(b)) return bits_to_f32(0x7FC00000u);
    if (a == b) return signbit(a) ? a : b;
    return a < b ? a : b;
}

static float apply_fp(int op, float acc, float x)
{
    switch (op) {
    case O_SUM:  return acc + x;
    case O_PROD: return acc * x;
    case O_MAX:  return fmax_def(acc, x);
    default:     return fmin_def(acc, x);
    }
}

/* int32: two's-complement wrap-around for SUM and PROD */
static int32_t apply_int(int op, int32_t acc, int32_t x)
{
    switch (op) {
    case O_SUM:  return (int32_t)((uint32_t)acc + (uint32_t)x);
    case O_PROD: return (int32_t)((uint32_t)acc * (uint32_t)x);
    case O_MAX:  return acc > x ? acc : x;
    default:     return acc < x ? acc : x;
    }
}

/* One reduced element: ranks folded in ascending order, seeded with rank 0.
 * Writes result element j of `out` from element i of every input. */
static void reduce_element(int R, const void *const *in, size_t i,
                           void *out, size_t j, int dt, int op)
{
    if (dt == O_INT32) {
        int32_t acc = ((const int32_t *)in[0])[i];
        for (int r = 1; r < R; r++)
            acc = apply_int(op, acc, ((const int32_t *)in[r])[i]);
        ((int32_t *)out)[j] = acc;
        return;
    }
    float acc = load_fp(in[0], i, dt);
    for (int r = 1; r < R; r++)
        acc = apply_fp(op, acc, load_fp(in[r], i, dt));
    store_fp(out, j, dt, acc);
}

static int check_common(int R, int dt, int op)
{
    if (R < 1 || R > 64) return O_EINVAL;
    if (dtype_size(dt) == 0) return O_EUNSUP;
    if (op < O_SUM || op > O_MIN) return O_EUNSUP;
    return O_OK;
}

/* ------------------------------------------------------------------ */
/* The primitives                                                      */
/* ------------------------------------------------------------------ */

/* AllReduce ([Tut] 6; owner layout of [IPC]): every rank receives the same
 * full reduction.  The owner-per-segment split only decides who computes an
 * element, never the value, so the definition is elementwise.  Outputs must
 * not alias inputs here (the oracle writes out[r] while still reading). */
int oracle_allreduce(int R, const void *const *in, void *const *out,
                     size_t count, int dt, int op)
{
    int rc = check_common(R, dt, op);
    if (rc) return rc;
    size_t es = dtype_size(dt);
    for (size_t i = 0; i < count; i++) {
        reduce_element(R, in, i, out[0], i, dt, op);
        for (int r = 1; r < R; r++)
            memcpy((char *)out[r] + i * es, (const char *)out[0] + i * es, es);
    }
    return O_OK;
}

/* Reduce ([Tut] 3): the full reduction lands on `root` only. */
int oracle_reduce(int R, const void *const *in, void *out_root, int root,
                  size_t count, int dt, int op)
{
    int rc = check_common(R, dt, op);
    if (rc) return rc;
    if (root < 0 || root >= R) return O_EINVAL;
    for (size_t i = 0; i < count; i++)
        reduce_element(R, in, i, out_root, i, dt, op);
    return O_OK;
}

/* ReduceScatter ([Tut] 5): rank r keeps the r-th of R equal chunks of the
 * global reduction.  Each input holds R*recvcount elements. */
int oracle_reduce_scatter(int R, const void *const *in, void *const *out,
                          size_t recvcount, int dt, int op)
{
    int rc = check_common(R, dt, op);
    if (rc) return rc;
    for (int r = 0; r < R; r++)
        for (size_t i = 0; i < recvcount; i++)
            reduce_element(R, in, (size_t)r * recvcount + i, out[r], i, dt, op);
    return O_OK;
}

/* AllGather ([Tut] 7): concatenation in rank order, on every rank. */
int oracle_all_gather(int R, const void *const *in, void *const *out,
                      size_t sendcount, size_t elem_size)
{
    if (R < 1 || R > 64 || elem_size == 0) return O_EINVAL;
    size_t n = sendcount * elem_size;
    for (int r = 0; r < R; r++)
        for (int q = 0; q < R; q++)
            memcpy((char *)out[r] + (size_t)q * n, in[q], n);
    return O_OK;
}

/* Gather ([Tut] 2, 2.2.1): each rank's [outer, inner] block is concatenated
 * along the last axis onto the root, giving [outer, R*inner].  Nothing is
 * written for the other ranks. */
int oracle_gather(int R, const void *const *in, void *out_root, int root,
                  size_t outer, size_t inner, size_t elem_size)
{
    if (R < 1 || R > 64 || elem_size == 0) return O_EINVAL;
    if (root < 0 || root >= R) return O_EINVAL;
    size_t n = inner * elem_size;
    for (size_t o = 0; o < outer; o++)
        for (int q = 0; q < R; q++)
            memcpy((char *)out_root + (o * (size_t)R + (size_t)q) * n,
                   (const char *)in[q] + o * n, n);
    return O_OK;
}

/* Scatter ([Tut] 4): root's buffer cut into R equal chunks, chunk r to rank r. */
int oracle_scatter(int R, const void *in_root, void *const *out, int root,
                   size_t recvcount, size_t elem_size)
{
    if (R < 1 || R > 64 || elem_size == 0) return O_EINVAL;
    if (root < 0 || root >= R) return O_EINVAL;
    size_t n = recvcount * elem_size;
    for (int r = 0; r < R; r++)
        memcpy(out[r], (const char *)in_root + (size_t)r * n, n);
    return O_OK;
}

/* Broadcast ([Tut] 1): every rank ends with root's data, bit for bit.  A rank
 * whose output is the root's own buffer is left as is. */
int oracle_broadcast(int R, const void *in_root, void *const *out, int root,
                     size_t count, size_t elem_size)
{
    if (R < 1 || R > 64 || elem_size == 0) return O_EINVAL;
    if (root < 0 || root >= R) return O_EINVAL;
    for (int r = 0; r < R; r++)
        if (out[r] != in_root)
            memcpy(out[r], in_root, count * elem_size);
    return O_OK;
}

/* All-to-All-v ([Tut] 8.1, 8.2; [A2A]): rank s sends count[s][d] rows to rank
 * d, read at row sdispl[s][d] of its send buffer and written at row
 * rdispl[d][s] of d's receive buffer.  Matrices are row-major R x R:
 * counts and sdispls indexed [s*R + d], rdispls indexed [d*R + s].
 * send_rows[s] / recv_rows[d] are the buffer capacities in rows; every block
 * must lie inside them and no two blocks may overlap in a receive buffer. */
int oracle_all_to_all_v(int R, const void *const *send, const int64_t *counts,
                        const int64_t *sdispls, void *const *recv,
                        const int64_t *rdispls, size_t row_bytes,
                        const int64_t *send_rows, const int64_t *recv_rows)
{
    if (R < 1 || R > 64 || row_bytes == 0) return O_EINVAL;
    for (int s = 0; s < R; s++)
        for (int d = 0; d < R; d++) {
            int64_t c = counts[s * R + d];
            int64_t so = sdispls[s * R + d], ro = rdispls[d * R + s];
            if (c < 0 || so < 0 || ro < 0) return O_EINVAL;
            if (so + c > send_rows[s] || ro + c > recv_rows[d]) return O_EINVAL;
        }
    /* receive blocks of one destination must be disjoint */
    for (int d = 0; d < R; d++)
        for (int s1 = 0; s1 < R; s1++)
            for (int s2 = s1 + 1; s2 < R; s2++) {
                int64_t c1 = counts[s1 * R + d], c2 = counts[s2 * R + d];
                int64_t a1 = rdispls[d * R + s1], a2 = rdispls[d * R + s2];
                if (c1 > 0 && c2 > 0 && a1 < a2 + c2 && a2 < a1 + c1)
                    return O_EINVAL;
            }
    for (int s = 0; s < R; s++)
        for (int d = 0; d < R; d++)
            for (int64_t j = 0; j < counts[s * R + d]; j++)
                memcpy((char *)recv[d] + (size_t)(rdispls[d * R + s] + j) * row_bytes,
                       (const char *)send[s] + (size_t)(sdispls[s * R + d] + j) * row_bytes,
                       row_bytes);
    return O_OK;
}

/* ------------------------------------------------------------------ */
/* MoE dispatch / combine ([Tut] 8.4)                                  */
/* ------------------------------------------------------------------ */

/* Layout.  For source rank s with ids[s][t*K + k] in [0, E):
 *   cnt_s[e]          = number of (t,k) routed to expert e
 *   owner(e)          = e / (E/R)          (contiguous expert blocks)
 *   sendcounts[s][d]  = sum of cnt_s[e] over the experts d owns
 *   sdispls[s][d]     = sum_{d' < d} sendcounts[s][d']
 *   rdispls[d][s]     = sum_{s' < s} sendcounts[s'][d]
 *   expert_counts[s][e] = cnt_s[e]
 *   pos[s][t*K + k]   = (sum_{e' < e} cnt_s[e'])
 *                       + number of earlier flat entries of s with expert e
 * i.e. the slot of (t,k) in s's send buffer sorted stably by expert.
 * An id outside [0, E) names no expert: its pair is skipped -- no slot
 * (pos = -1), counted nowhere, no row moved, no term in the combine.  The
 * pages route only to existing experts; a pair with no expert is read as one
 * that does not exist. */
int oracle_moe_layout(int R, const int32_t *const *ids, int T, int K, int E,
                      int64_t *sendcounts, int64_t *sdispls, int64_t *rdispls,
                      int32_t *expert_counts, int32_t *const *pos)
{
    if (R < 1 || R > 64 || T < 0 || K < 1 || E < 1 || E % R != 0) return O_EINVAL;
    int per = E / R;
    int64_t *off = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    int64_t *seen = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    if (!off || !seen) { free(off); free(seen); return O_EINVAL; }
    for (int s = 0; s < R; s++) {
        int32_t *cnt = expert_counts + (size_t)s * E;
        for (int e = 0; e < E; e++) cnt[e] = 0;
        for (int64_t i = 0; i < (int64_t)T * K; i++) {
            int32_t e = ids[s][i];
            if (e >= 0 && e < E) cnt[e]++;
        }
        for (int d = 0; d < R; d++) {
            int64_t c = 0;
            for (int e = d * per; e < (d + 1) * per; e++) c += cnt[e];
            sendcounts[s * R + d] = c;
        }
        int64_t acc = 0;
        for (int d = 0; d < R; d++) { sdispls[s * R + d] = acc; acc += sendcounts[s * R + d]; }
        acc = 0;
        for (int e = 0; e < E; e++) { off[e] = acc; acc += cnt[e]; seen[e] = 0; }
        for (int64_t i = 0; i < (int64_t)T * K; i++) {
            int32_t e = ids[s][i];
            if (e < 0 || e >= E) { pos[s][i] = -1; continue; }
            pos[s][i] = (int32_t)(off[e] + seen[e]);
            seen[e]++;
        }
    }
    for (int d = 0; d < R; d++) {
        int64_t acc = 0;
        for (int s = 0; s < R; s++) { rdispls[d * R + s] = acc; acc += sendcounts[s * R + d]; }
    }
    free(off);
    free(seen);
    return O_OK;
}

/* Dispatch permute (an indexed write, [Tut] 4.3.2 / 8.4): the row of token t
 * goes to slot pos[s][t*K+k] of s's send buffer, once per k. */
int oracle_moe_permute(int R, const void *const *x, const int32_t *const *pos,
                       int T, int K, size_t row_bytes, void *const *send)
{
    if (R < 1 || R > 64 || T < 0 || K < 1) return O_EINVAL;
    for (int s = 0; s < R; s++)
        for (int t = 0; t < T; t++)
            for (int k = 0; k < K; k++) {
                int32_t p = pos[s][(size_t)t * K + k];
                if (p < 0) continue;                 /* a skipped pair (no expert) */
                memcpy((char *)send[s] + (size_t)p * row_bytes,
                       (const char *)x[s] + (size_t)t * row_bytes, row_bytes);
            }
    return O_OK;
}

/* Test expert, bf16 rows: y = rne(widen(x) * (1 + e/256)).  Rank d's receive
 * buffer holds, for each source s in ascending order starting at row
 * rdispls[d][s], the rows of d's experts in ascending expert order, with
 * expert_counts[s][e] rows each.  The scale has at most 9 significant bits and
 * a bf16 value 8, so the fp32 product is exact and y is unique. */
int oracle_moe_expert_scale(int R, void *const *recv, const int32_t *expert_counts,
                            const int64_t *rdispls, int E, size_t hidden)
{
    if (R < 1 || R > 64 || E < 1 || E % R != 0) return O_EINVAL;
    int per = E / R;
    for (int d = 0; d < R; d++)
        for (int s = 0; s < R; s++) {
            int64_t row = rdispls[d * R + s];
            for (int e = d * per; e < (d + 1) * per; e++) {
                float scale = 1.0f + (float)e / 256.0f;
                for (int32_t j = 0; j < expert_counts[(size_t)s * E + e]; j++, row++) {
                    uint16_t *y = (uint16_t *)recv[d] + (size_t)row * hidden;
                    for (size_t c = 0; c < hidden; c++)
                        y[c] = oracle_f32_to_bf16(oracle_bf16_to_f32(y[c]) * scale);
                }
            }
        }
    return O_OK;
}

/* Combine ([Tut] 8.4: results return to the token's owner): back[s] holds the
 * expert outputs in s's send-slot order; out[s][t] = rne(sum over k of
 * w[s][t,k] * widen(back[s][pos[s][t,k]])), k ascending, accumulator seeded by
 * the k = 0 product, multiply and add rounded separately, one final rounding.
 * A skipped pair (pos < 0) adds no term: the fold runs over the token's other
 * pairs in the same order, seeded by the first of them; none left gives +0. */
int oracle_moe_combine(int R, const void *const *back, const int32_t *const *pos,
                       const float *const *w, int T, int K, size_t hidden,
                       void *const *out)
{
    if (R < 1 || R > 64 || T < 0 || K < 1) return O_EINVAL;
    for (int s = 0; s < R; s++)
        for (int t = 0; t < T; t++)
            for (size_t c = 0; c < hidden; c++) {
                float acc = 0.0f;
                int have = 0;                        /* a term has seeded acc */
                for (int k = 0; k < K; k++) {
                    size_t i = (size_t)t * K + k;
                    if (pos[s][i] < 0) continue;     /* a skipped pair: no term */
                    const uint16_t *row = (const uint16_t *)back[s] + (size_t)pos[s][i] * hidden;
                    float prod = w[s][i] * oracle_bf16_to_f32(row[c]);
                    acc = have ? acc + prod : prod;
                    have = 1;
                }
                ((uint16_t *)out[s])[(size_t)t * hidden + c] = oracle_f32_to_bf16(acc);
            }
    return O_OK;
}

/* ------------------------------------------------------------------ */
/* Array forms of the conversions, for the tests' pins                 */
/* ------------------------------------------------------------------ */

void oracle_f32_to_bf16_n(size_t n, const float *in, uint16_t *out)
{
    for (size_t i = 0; i < n; i++) out[i] = oracle_f32_to_bf16(in[i]);
}
void oracle_bf16_to_f32_n(size_t n, const uint16_t *in, float *out)
{
    for (size_t i = 0; i < n; i++) out[i] = oracle_bf16_to_f32(in[i]);
}
void oracle_f32_to_f16_n(size_t n, const float *in, uint16_t *out)
{
    for (size_t i = 0; i < n; i++) out[i] = oracle_f32_to_f16(in[i]);
}
void oracle_f16_to_f32_n(size_t n, const uint16_t *in, float *out)
{
    for (size_t i = 0; i < n; i++) out[i] = oracle_f16_to_f32(in[i]);
}
void oracle_f64_to_bf16_n(size_t n, const double *in, uint16_t *out)
{
    for (size_t i = 0; i < n; i++) out[i] = oracle_f64_to_bf16(in[i]);
}

/* ------------------------------------------------------------------ */
/* Uniform all-to-all and the sequence <-> heads re-shard              */
/* ------------------------------------------------------------------ */

/* all_to_all_single with equal splits (sglang PR 27492 digest; tutorial
 * 8.1): rank s's buffer is R chunks of n elements, chunk d for rank d;
 * rank d receives them ordered by source: out[d][s*n + i] = in[s][d*n + i]. */
int oracle_all_to_all(int R, const void *const *in, void *const *out, size_t n,
                      size_t elem_size)
{
    if (R < 1 || R > 64 || elem_size == 0) return O_EINVAL;
    size_t b = n * elem_size;
    for (int s = 0; s < R; s++)
        for (int d = 0; d < R; d++)
            memcpy((char *)out[d] + (size_t)s * b, (const char *)in[s] + (size_t)d * b, b);
    return O_OK;
}

/* Sequence-parallel re-shard used for all-to-all sequence parallelism at the
 * model level (sglang PR 27492 digest's motivation): rank s holds its
 * sequence chunk of all heads, x_s[t][h][c] with t < SL, h < H, c < D; after
 * the exchange rank d holds the whole sequence for its head group,
 * y_d[s*SL + t][h'][c] = x_s[t][d*(H/R) + h'][c].  to_heads = 0 is the
 * inverse map (y -> x). */
int oracle_ulysses(int R, const void *const *in, void *const *out, size_t SL, size_t H,
                   size_t D, size_t elem_size, int to_heads)
{
    if (R < 1 || R > 64 || elem_size == 0 || H % (size_t)R != 0) return O_EINVAL;
    size_t HR = H / (size_t)R;
    for (int s = 0; s < R; s++)
        for (size_t t = 0; t < SL; t++)
            for (int d = 0; d < R; d++)
                for (size_t hh = 0; hh < HR; hh++)
                    for (size_t c = 0; c < D; c++) {
                        size_t xi = (t * H + (size_t)d * HR + hh) * D + c;        /* in x_s */
                        size_t yi = (((size_t)s * SL + t) * HR + hh) * D + c;     /* in y_d */
                        if (to_heads)
                            memcpy((char *)out[d] + yi * elem_size,
                                   (const char *)in[s] + xi * elem_size, elem_size);
                        else
                            memcpy((char *)out[s] + xi * elem_size,
                                   (const char *)in[d] + yi * elem_size, elem_size);
                    }
    return O_OK;
}

/* ------------------------------------------------------------------ */
/* Context-parallel merge of partial attention (tutorial 5.4.2, 7.4.3) */
/* ------------------------------------------------------------------ */

/* Each rank holds, per (token, head) row, a partial attention output o_r
 * normalised over its own key chunk and that chunk's log-sum-exp l_r.  The
 * pages: the partial outputs cannot be summed as they are; the LSEs are
 * gathered first and the corrected contributions are then summed.  Written
 * out in fp64:
 *     m = max_r l_r,  e_r = exp(l_r - m),  s = sum_r e_r (r ascending),
 *     L = m + log(s),  o = sum_r (e_r / s) * o_r (r ascending),
 * rounded once to the output type; every rank receives (o, L).  A row whose
 * chunks are all empty (every l_r = -inf) gives o = 0, L = -inf.
 * dt is the dtype of o (bf16 or fp32); lse are fp32. */
int oracle_lse_merge(int R, const void *const *o_parts, const float *const *lse_parts,
                     void *const *o_out, float *const *lse_out, size_t rows, size_t D, int dt)
{
    if (R < 1 || R > 64 || (dt != O_BF16 && dt != O_FP32)) return O_EINVAL;
    for (size_t i = 0; i < rows; i++) {
        double m = -INFINITY;
        for (int r = 0; r < R; r++)
            if ((double)lse_parts[r][i] > m) m = (double)lse_parts[r][i];
        double e[64], s = 0.0, L;
        if (m == -INFINITY) {
            for (int r = 0; r < R; r++) e[r] = 0.0;
            L = -INFINITY;
        } else {
            for (int r = 0; r < R; r++) { e[r] = exp((double)lse_parts[r][i] - m); s += e[r]; }
            L = m + log(s);
        }
        for (size_t c = 0; c < D; c++) {
            double acc = 0.0;
            if (m != -INFINITY)
                for (int r = 0; r < R; r++)
                    acc += (e[r] / s) * (double)load_fp(o_parts[r], i * D + c, dt);
            /* one rounding from binary64 to the output type */
            for (int r = 0; r < R; r++) {
                if (dt == O_BF16)
                    ((uint16_t *)o_out[r])[i * D + c] = oracle_f64_to_bf16(acc);
                else
                    ((float *)o_out[r])[i * D + c] = (float)acc;
            }
        }
        for (int r = 0; r < R; r++)
            if (lse_out && lse_out[r]) lse_out[r][i] = (float)L;
    }
    return O_OK;
}
