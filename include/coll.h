/*
 * coll.h -- C ABI of libcoll.so: collectives over R "virtual ranks" whose
 * buffers all live in one MI355X's HBM, computed by hand-written gfx950 HIP
 * kernels.
 *
 * A rank here is only a set of device pointers: rank r owns sendbufs[r] and
 * recvbufs[r].  Every call takes the pointer arrays in HOST memory, copies
 * them into the kernel arguments before returning, and keeps no reference to
 * them afterwards.  Device buffers and device count arrays must stay valid
 * until the work queued on `stream` has finished.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - nranks R is in [1, COLL_MAX_RANKS]; anything else -> COLL_ERR_INVALID_ARG.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    calls are asynchronous: they enqueue kernels and return without a host
 *    synchronisation.
 *  - A count of 0 returns COLL_OK and launches nothing.
 *  - Host-detectable errors (bad R, root, dtype/op, NULL pointer where data is
 *    needed, a size that overflows) return a negative status and launch
 *    nothing.  A launch failure returns COLL_ERR_HIP.  No C++ exception ever
 *    crosses this boundary.
 *  - The library allocates nothing and holds no state beyond a per-device
 *    cache of the compute-unit count and its tuning knobs (COLL_* environment
 *    variables, read once per process); calls on different streams are
 *    independent.  The MoE layout takes caller-provided workspace.
 *  - Reductions of bf16 / fp16 widen every element exactly to fp32, fold the
 *    ranks in ascending order 0, 1, ..., R-1 with the accumulator seeded by
 *    rank 0's value (no FMA, no reassociation), and round once to the output
 *    type, round-to-nearest-even.  fp32 folds in the same order; int32 wraps.
 *    The result is therefore bit-identical on every rank and across calls.
 *  - Element counts are in elements of `dtype`; A2A-v counts are in rows.
 *
 * Sources: "Collective primitives tutorial" (gsyq.cn news 307221), sections
 * 1-8; "From NCCL Ring LL to PCIe IPC AllReduce" (hjcheng0602 blog), section
 * "Pro5000 ?" for the owner-per-segment AllReduce layout; sglang PR 27492
 * digest (all_to_all_single: output mutated, world size 1 is a copy); sglang
 * PR 33307 digest (broadcast from the owner; no host sync on the path).
 */
#ifndef COLL_H
#define COLL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    COLL_OK = 0,
    COLL_ERR_INVALID_ARG = -1,
    COLL_ERR_UNSUPPORTED = -2,
    COLL_ERR_HIP = -3
} coll_status_t;

typedef enum { COLL_BF16 = 0, COLL_FP16 = 1, COLL_FP32 = 2, COLL_INT32 = 3 } coll_dtype_t;

/* Reduction operators of the tutorial's section 3 (Reduce). */
typedef enum { COLL_SUM = 0, COLL_PROD = 1, COLL_MAX = 2, COLL_MIN = 3 } coll_op_t;

#define COLL_MAX_RANKS 16

/* Human-readable name of a status code (static storage, never NULL). */
const char *coll_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int coll_version(void);

/*
 * Placement of virtual-rank buffers in one device allocation (a "rank
 * arena").  Not an operation of the pages: a layout rule for this one-GPU
 * setting, where the R ranks' buffers share one HBM.  A collective touches
 * all R buffers of a role at the same element offset at the same time; when
 * those buffers start at the same address modulo the interleave of the HBM
 * channels, the R concurrent streams fall on the same channels and the
 * pattern loses up to a fifth of its bandwidth (measured on MI355X, AllReduce
 * of 8 inputs + 8 outputs of 16 MiB: separately allocated buffers vs this
 * placement).  The channel hash takes address bits both below and above
 * 2 MiB, so the rule varies both.
 *
 * Buffer k (k = 0..n-1, in the caller's order) starts at the first multiple
 * of COLL_ARENA_ALIGN (2 MiB) at or after the end of buffer k-1, plus
 * (k mod COLL_ARENA_COLORS) * COLL_ARENA_COLOR_BYTES.  Consecutive buffers
 * thus start at distinct 4 KiB colours within their 2 MiB page, and a 2 MiB
 * boundary lies between any two of them; each wastes less than 2 MiB +
 * 124 KiB.  Order the buffers of one call consecutively (e.g. the R inputs,
 * then the R outputs).
 *
 *   bytes[k]:   size of buffer k (0 allowed); host array of n entries.
 *   offsets[k]: (out) byte offset of buffer k from a base aligned to
 *               COLL_ARENA_ALIGN; host array of n entries.
 *   total:      (out) bytes from that base to the end of the last buffer.
 * The caller allocates total + COLL_ARENA_ALIGN - 1 bytes (or an aligned
 * block of `total`), aligns the base up to COLL_ARENA_ALIGN and places buffer
 * k at base + offsets[k].  Host-only: no HIP call, no allocation.
 * Errors: n < 0, a NULL array with n > 0, NULL total, or a size overflow ->
 * COLL_ERR_INVALID_ARG with the outputs unspecified.  n = 0 gives total 0.
 */
#define COLL_ARENA_COLOR_BYTES 4096u
#define COLL_ARENA_COLORS 32u
#define COLL_ARENA_ALIGN (2u << 20)
int coll_arena_layout(int n, const size_t *bytes, size_t *offsets, size_t *total);

/*
 * AllReduce -- tutorial section 6 (every rank ends with the same full
 * reduction), computed in the owner-per-segment layout of the IPC AllReduce
 * blog ("Pro5000 ?"): the element range is split into tiles; each tile is read
 * once from all R ranks, reduced once, and the result stored to all R outputs
 * (ReduceScatter to the tile's owner fused with AllGather from it).
 *
 *   sendbufs[r], recvbufs[r]: R device pointers, `count` elements each.
 *   recvbufs[r] == sendbufs[r] (in place) is allowed; any other overlap is not.
 *   All ops for all dtypes; MAX/MIN propagate NaN and order -0 below +0.
 */
int coll_allreduce(int nranks, const void *const *sendbufs, void *const *recvbufs,
                   size_t count, coll_dtype_t dtype, coll_op_t op, void *stream);

/*
 * ReduceScatter -- tutorial section 5: reduce, then rank r keeps chunk r.
 *   sendbufs[r]: nranks * recvcount elements; recvbufs[r]: recvcount elements.
 *   recvbufs[r][i] = reduction over q of sendbufs[q][r * recvcount + i].
 *   In place allowed when recvbufs[r] == sendbufs[r] + r * recvcount elements.
 */
int coll_reduce_scatter(int nranks, const void *const *sendbufs, void *const *recvbufs,
                        size_t recvcount, coll_dtype_t dtype, coll_op_t op, void *stream);

/*
 * AllGather -- tutorial section 7: concatenation in rank order on every rank.
 *   sendbufs[q]: sendcount elements; recvbufs[r]: nranks * sendcount elements.
 *   recvbufs[r][q * sendcount + i] = sendbufs[q][i].  A pure copy: any dtype.
 *   In place allowed when sendbufs[r] == recvbufs[r] + r * sendcount elements.
 */
int coll_all_gather(int nranks, const void *const *sendbufs, void *const *recvbufs,
                    size_t sendcount, coll_dtype_t dtype, void *stream);

/*
 * Gather -- tutorial section 2 (2.2.1: vocab-sharded logits collected on dst 0):
 * each rank's row-major [outer, inner] block is concatenated along the LAST
 * axis onto the root, giving [outer, nranks * inner]:
 *   recvbuf_root[o * nranks * inner + q * inner + i] = sendbufs[q][o * inner + i].
 * Only the root's buffer is written (the other ranks receive nothing, as the
 * tutorial's non-dst ranks get None).  recvbuf_root must not overlap any send
 * buffer.  A dim-0 concatenation is outer = 1.
 */
int coll_gather(int nranks, const void *const *sendbufs, void *recvbuf_root, int root,
                size_t outer, size_t inner, coll_dtype_t dtype, void *stream);

/*
 * Reduce -- tutorial section 3: the full reduction lands on `root` only.
 *   sendbufs[r]: `count` elements each; recvbuf_root: `count` elements.
 *   recvbuf_root[i] = reduction over r (ascending) of sendbufs[r][i], with the
 *   same arithmetic as coll_allreduce (so it equals AllReduce's output on the
 *   root bit for bit).  recvbuf_root may be sendbufs[root]; no other overlap.
 */
int coll_reduce(int nranks, const void *const *sendbufs, void *recvbuf_root, int root,
                size_t count, coll_dtype_t dtype, coll_op_t op, void *stream);

/*
 * Scatter -- tutorial section 4: the root's buffer is cut into nranks equal
 * chunks of recvcount elements and chunk r goes to rank r.
 *   recvbufs[r][i] = sendbuf_root[r * recvcount + i].  A pure copy: any dtype.
 *   recvbufs[root] may be NULL or sendbuf_root + root * recvcount (then not
 *   written); no other overlap.
 */
int coll_scatter(int nranks, const void *sendbuf_root, void *const *recvbufs, int root,
                 size_t recvcount, coll_dtype_t dtype, void *stream);

/*
 * Broadcast -- tutorial section 1: every rank ends with root's `count`
 * elements, bit for bit.  recvbufs[r] may equal sendbuf_root for r == root
 * (the owner keeps its own tensor, as in the sglang PR 33307 digest); that
 * buffer is then not written.  recvbufs[r] may be NULL for r == root only.
 */
int coll_broadcast(int nranks, const void *sendbuf_root, void *const *recvbufs, int root,
                   size_t count, coll_dtype_t dtype, void *stream);

/*
 * All-to-All-v -- tutorial sections 8.1-8.2: rank s sends a distinct, variable
 * length block to every rank d; d's receive buffer holds the blocks ordered by
 * source.  Units are rows of `row_elems` elements of `dtype`.
 *   sendcounts[s * R + d]: rows s sends to d            (DEVICE int64, R*R)
 *   sdispls   [s * R + d]: first such row in sendbufs[s] (DEVICE int64, R*R)
 *   rdispls   [d * R + s]: where they land in recvbufs[d] (DEVICE int64, R*R)
 *   recvbufs[d][(rdispls[d*R+s] + j) * row_elems + c]
 *        = sendbufs[s][(sdispls[s*R+d] + j) * row_elems + c],  j < sendcounts[s*R+d].
 * Counts live on the device so a layout kernel can feed this call with no
 * host synchronisation; the host cannot read them.  Instead the kernels bound
 * every block by the buffers' sizes:
 *   send_rows[s], recv_rows[d]: rows the buffers sendbufs[s] and recvbufs[d]
 *   hold (HOST int64 arrays of nranks entries, read during the call; NULL
 *   leaves that side unbounded, and a NULL buffer holds 0 rows).
 * Block (s, d) moves only if its count is positive, both displacements are
 * non-negative and all its rows exist: sdispls[s*R+d] + count <= send_rows[s]
 * and rdispls[d*R+s] + count <= recv_rows[d].  Otherwise it moves nothing and
 * the receive rows it names keep their contents; the other blocks are not
 * affected.  So a wrong table can give a wrong result but never touches
 * memory outside the buffers.  Receive blocks that overlap each other, or
 * send and receive buffers that overlap, are the caller's to avoid.  A rank
 * that sends (or receives) no rows may pass NULL for its buffer; the pointer
 * arrays themselves must not be NULL.
 * The reverse exchange (MoE combine) is coll_all_to_all_v_reverse on the same
 * tables.
 *   recv_rows_capacity: the rows of all receive buffers together, an upper
 *   bound of the rows moved that the host knows without reading the counts.
 *   It only shapes the launch, never the result or the memory addressed.
 *   Above 64 MiB of capacity there is one workgroup per tile of the bound.
 *   Up to 64 MiB, or with 0 (unknown), a resident grid loops over the tiles
 *   (the faster forms on MI355X at those sizes).
 */
int coll_all_to_all_v(int nranks, const void *const *sendbufs, const int64_t *sendcounts,
                      const int64_t *sdispls, void *const *recvbufs, const int64_t *rdispls,
                      size_t row_elems, coll_dtype_t dtype, size_t recv_rows_capacity,
                      const int64_t *send_rows, const int64_t *recv_rows, void *stream);

/*
 * All-to-All-v with a caller workspace -- tutorial sections 8.1-8.2, the same
 * exchange, result and arguments as coll_all_to_all_v, faster for large
 * exchanges.  A first kernel writes the
 * block table and, for every tile of 64 sixteen-byte units (1 KiB) of the
 * receive capacity, the index of the block holding its first unit; the copy
 * kernel then starts each tile with that index and the block's entry instead
 * of building the table.  This descriptor form runs when
 * rows are whole 16-byte units and recv_rows_capacity covers at least 192 MiB
 * (environment variable COLL_A2A_DESC_MIN_BYTES, read once per process; below
 * it the second launch costs more than it saves on MI355X).  Otherwise this
 * call is coll_all_to_all_v, the workspace is not touched and may be NULL, and
 * the size below is 0.  Its size is
 * coll_all_to_all_v_workspace_bytes(nranks, recv_rows_capacity, row_elems,
 * dtype): 32 bytes per block and 2 per tile, the tiles counted in whole
 * groups of 512, rounded up to 256 (7 MiB for a 3.5 GiB exchange).
 * workspace: DEVICE, 256-byte aligned, overwritten; concurrent calls need
 * workspaces of their own.  recv_rows_capacity only sizes the launch: a bound
 * below the rows actually received costs time, not correctness.
 * Errors: as coll_all_to_all_v, plus COLL_ERR_INVALID_ARG for a NULL or
 * misaligned workspace or workspace_bytes below the size when one is needed.
 * send_rows / recv_rows bound the blocks as in coll_all_to_all_v.
 */
size_t coll_all_to_all_v_workspace_bytes(int nranks, size_t recv_rows_capacity, size_t row_elems,
                                        coll_dtype_t dtype);
int coll_all_to_all_v_ws(int nranks, const void *const *sendbufs, const int64_t *sendcounts,
                         const int64_t *sdispls, void *const *recvbufs, const int64_t *rdispls,
                         size_t row_elems, coll_dtype_t dtype, size_t recv_rows_capacity,
                         const int64_t *send_rows, const int64_t *recv_rows, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * The descriptor form of coll_all_to_all_v_ws as two calls, so that its first
 * kernel can run off the critical path: it depends only on the count and
 * displacement tables and on the buffers' addresses, not on the rows, so a
 * caller can issue it (for instance on a second stream) while the send
 * buffers are still being written.
 *   coll_all_to_all_v_ws_build: the arguments of coll_all_to_all_v_ws; writes
 *   the workspace (the block table, with the buffers' addresses, and a block
 *   index per tile) and moves nothing.  Returns COLL_ERR_UNSUPPORTED, with
 *   nothing launched, where coll_all_to_all_v_ws would take the plain form
 *   (coll_all_to_all_v_workspace_bytes is 0 for the call, or the buffers are
 *   not 16-byte aligned): call coll_all_to_all_v_ws then.
 *   coll_all_to_all_v_reverse_build: the same for coll_all_to_all_v_reverse
 *   (its arguments; rows_capacity = its send_rows_capacity).
 *   coll_all_to_all_v_ws_copy: the copy kernel alone, from a workspace that
 *   a build wrote for the same nranks, row size and capacity.  It moves the
 *   rows between the buffers the build was given, as the one-call form
 *   would.  The caller orders it after the build (same stream, or an event)
 *   and after the writes to the send buffers, and does not reuse the
 *   workspace until the copy completes.
 * Errors: as coll_all_to_all_v_ws; the copy returns COLL_ERR_INVALID_ARG for
 * a NULL or misaligned workspace or one below the size, and
 * COLL_ERR_UNSUPPORTED where no descriptor form exists for its sizes.
 */
int coll_all_to_all_v_ws_build(int nranks, const void *const *sendbufs, const int64_t *sendcounts,
                               const int64_t *sdispls, void *const *recvbufs,
                               const int64_t *rdispls, size_t row_elems, coll_dtype_t dtype,
                               size_t recv_rows_capacity, const int64_t *send_rows,
                               const int64_t *recv_rows, void *workspace, size_t workspace_bytes,
                               void *stream);
int coll_all_to_all_v_reverse_build(int nranks, const void *const *recvbufs,
                                    const int64_t *sendcounts, const int64_t *sdispls,
                                    void *const *sendbufs, const int64_t *rdispls,
                                    size_t row_elems, coll_dtype_t dtype,
                                    size_t send_rows_capacity, const int64_t *send_rows,
                                    const int64_t *recv_rows, void *workspace,
                                    size_t workspace_bytes, void *stream);
int coll_all_to_all_v_ws_copy(int nranks, size_t row_elems, coll_dtype_t dtype,
                              size_t rows_capacity, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * The reverse of an All-to-All-v, from that exchange's own tables -- tutorial
 * section 8.4 (after the experts, results return to the token's owner in one
 * more exchange).  With the forward call's sendcounts, sdispls and rdispls:
 *   sendbufs[s][(sdispls[s*R+d] + j) * row_elems + c]
 *        = recvbufs[d][(rdispls[d*R+s] + j) * row_elems + c],  j < sendcounts[s*R+d],
 * i.e. every block goes back to where it came from.  This equals
 * coll_all_to_all_v with the count matrix transposed and the two displacement
 * tables swapped, without building the transposed matrix (no extra launch).
 *   recvbufs: the forward exchange's receive buffers (read here);
 *   sendbufs: the forward exchange's send buffers (written here);
 *   send_rows_capacity: an upper bound of the rows moved, here the rows of
 *   the send buffers together (launch shape only, as recv_rows_capacity);
 *   send_rows / recv_rows: the rows of sendbufs[s] / recvbufs[d], as in the
 *   forward call (HOST, NULL = unbounded); a block moves only if all its rows
 *   exist on both sides, as in coll_all_to_all_v.
 * workspace / workspace_bytes: as coll_all_to_all_v_ws (size from
 * coll_all_to_all_v_workspace_bytes with send_rows_capacity); NULL and 0
 * select the plain form.  Errors as coll_all_to_all_v_ws.
 */
int coll_all_to_all_v_reverse(int nranks, const void *const *recvbufs, const int64_t *sendcounts,
                              const int64_t *sdispls, void *const *sendbufs,
                              const int64_t *rdispls, size_t row_elems, coll_dtype_t dtype,
                              size_t send_rows_capacity, const int64_t *send_rows,
                              const int64_t *recv_rows, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * Uniform all-to-all -- all_to_all_single with equal splits (sglang PR 27492
 * digest; tutorial section 8.1's figure): sendbufs[s] holds nranks chunks of
 * count_per_peer elements, chunk d for rank d; rank d receives them ordered
 * by source: recvbufs[d][s * count_per_peer + i] = sendbufs[s][d * count_per_peer + i].
 * With one rank it is a copy.  Send and receive buffers must not overlap.
 */
int coll_all_to_all(int nranks, const void *const *sendbufs, void *const *recvbufs,
                    size_t count_per_peer, coll_dtype_t dtype, void *stream);

/*
 * Sequence <-> heads re-shard of all-to-all sequence parallelism (the use the
 * sglang PR 27492 digest gives for all_to_all_single): with SL = seq_local,
 * H = heads (a multiple of nranks), HR = H / nranks, D = head_dim,
 *   to_heads = 1:  in[s] is [SL, H, D] (rank s's sequence chunk, all heads);
 *                  out[d] is [nranks*SL, HR, D] (the whole sequence, head group d):
 *                  out[d][s*SL + t][h][c] = in[s][t][d*HR + h][c]
 *   to_heads = 0:  the inverse map (in is [nranks*SL, HR, D] per rank).
 * The strided head groups are gathered in the exchange itself (no packed
 * copy).  Inputs and outputs must not overlap.
 */
int coll_seq_heads_reshard(int nranks, const void *const *in, void *const *out,
                           size_t seq_local, size_t heads, size_t head_dim, coll_dtype_t dtype,
                           int to_heads, void *stream);

/*
 * Context-parallel merge of partial attention -- tutorial sections 5.4.2 and
 * 7.4.3 (the partial outputs cannot be summed as they are: the log-sum-exps
 * are gathered and the corrected contributions summed).  Per row i (a
 * (token, head) pair) with o_parts[r] row i and lse_parts[r][i]:
 *   m = max_r lse, e_r = exp(lse_r - m), s = sum_r e_r, L = m + log(s),
 *   o_out[r][i] = sum_r (e_r / s) * o_parts[r][i]   (fp32, ranks ascending),
 *   lse_out[r][i] = L,   for every rank r (AllReduce of the corrected terms).
 * A row whose lse are all -inf gives 0 and -inf.  o_parts/o_out: [rows,
 * head_dim] of bf16 or fp32; lse: fp32 [rows].  o_out[r] may be o_parts[r]
 * (in place); lse_out (or an entry of it) may be NULL to skip it.  No
 * lse_out[r] may overlap any lse_parts[q] (in-place LSEs are rejected with
 * COLL_ERR_INVALID_ARG: a long row is split over several workgroups, and the
 * one that stores L would race the others' reads).  Each row's weights are
 * formed once, by one lane.  exp/log are the device library's fp32
 * functions: o differs from the exact (fp64) merge rounded once by at most
 * 2 ulps of the output type plus a few fp32 ulps of sum_r w_r |o_r|
 * (cancellation); L by a few fp32 ulps.
 */
int coll_lse_merge(int nranks, const void *const *o_parts, const float *const *lse_parts,
                   void *const *o_out, float *const *lse_out, size_t rows, size_t head_dim,
                   coll_dtype_t dtype, void *stream);

/* ---------------------------------------------------------------------------
 * MoE dispatch / combine over expert parallelism -- tutorial section 8.4.
 * Experts are placed on ranks in contiguous blocks: rank d owns experts
 * [d*E/R, (d+1)*E/R); E must be a multiple of R.  Each (token t, slot k) pair
 * is one dispatched row; rows bound for a rank are ordered stably by
 * (expert, t, k), so within a source's send buffer the rows are sorted by
 * expert.  topk_ids are int32; an id outside [0, E) names no expert and its
 * pair is skipped everywhere: it gets no send slot (pos = -1), is counted in
 * no table, moves no row and adds no term to either combine (the tutorial
 * routes tokens only to existing experts; such a pair is read as one that
 * does not exist).
 * ------------------------------------------------------------------------- */

/* Bytes of device workspace coll_moe_layout needs (0 on invalid sizes). */
size_t coll_moe_workspace_bytes(int nranks, int tokens, int topk, int n_experts);

/*
 * Layout: from R device arrays topk_ids[s] (int32 [tokens, topk]) compute
 *   sendcounts[s*R+d], sdispls[s*R+d], rdispls[d*R+s]  (DEVICE int64, R*R each),
 *   expert_counts[s*E+e]  rows of expert e from source s (DEVICE int32, R*E),
 *   pos[s][t*topk+k]      slot of (t,k) in source s's send buffer, -1 for a
 *                         pair with no expert (DEVICE int32 [tokens*topk]).
 * Uses `workspace` (coll_moe_workspace_bytes, 256-byte aligned, device).
 * Supports n_experts <= 1024 and tokens * topk < 2^31.
 */
int coll_moe_layout(int nranks, const int32_t *const *topk_ids, int tokens, int topk,
                    int n_experts, int64_t *sendcounts, int64_t *sdispls, int64_t *rdispls,
                    int32_t *expert_counts, int32_t *const *pos, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * The layout with no workspace argument, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and errors as coll_moe_layout
 * without workspace/workspace_bytes; its scratch is a device array of
 * COLL_MOE_NOALLOC_MAX_BYTES that the library holds on each GPU it runs on
 * until the process ends (nothing is allocated per call).  Sizes whose
 * coll_moe_workspace_bytes exceeds that maximum return COLL_ERR_INVALID_ARG
 * (it holds e.g. 8 ranks x 65,000 tokens x top-8 of 256 experts).  Every call
 * on one GPU uses the same array: calls that may overlap on a GPU (other
 * streams, other threads) race and must not be issued.  COLL_ERR_HIP if the
 * array's device address cannot be obtained.
 */
#define COLL_MOE_NOALLOC_MAX_BYTES (4u << 20)
int coll_moe_layout_noalloc(int nranks, const int32_t *const *topk_ids, int tokens, int topk,
                            int n_experts, int64_t *sendcounts, int64_t *sdispls,
                            int64_t *rdispls, int32_t *expert_counts, int32_t *const *pos,
                            void *stream);

/*
 * Dispatch permute (an indexed write; the tutorial's 4.3.2 warns it is not the
 * Scatter collective): sendbufs[s][pos[s][t*topk+k]] = x[s][t] for every pair
 * with a slot (pos outside [0, tokens*topk), the layout's -1, is skipped).
 * x[s]: [tokens, hidden]; sendbufs[s]: [tokens*topk, hidden].  Any dtype.
 */
int coll_moe_permute(int nranks, const void *const *x, const int32_t *const *pos,
                     int tokens, int topk, size_t hidden, coll_dtype_t dtype,
                     void *const *sendbufs, void *stream);

/* Bytes of device workspace coll_moe_expert_scale needs (0 on invalid sizes):
 * two int64 tables of nranks * n_experts entries, rounded up to 256 bytes,
 * then 8 bytes per row of recv_rows_capacity (rounded up to 256) for the row
 * descriptors of the faster path.  With recv_rows_capacity = 0 the size is
 * the tables alone, the least any call accepts. */
size_t coll_moe_expert_workspace_bytes(int nranks, int n_experts, size_t recv_rows_capacity);

/*
 * Test expert used to exercise the round trip: each received bf16 row of
 * expert e becomes y = rne(x * (1 + e/256)) in place (the fp32 product is
 * exact, so y is unique).  Row order in recvbufs[d] is: for s ascending,
 * starting at rdispls[d*R+s], the rows of d's experts in ascending expert
 * order, expert_counts[s*E+e] rows each (expert_counts and rdispls: DEVICE
 * arrays, the outputs of coll_moe_layout).
 * workspace: DEVICE, 256-byte aligned, at least
 * coll_moe_expert_workspace_bytes(nranks, n_experts, 0) bytes; it is
 * overwritten (a row-prefix table built on the device, and row descriptors),
 * so calls that may run concurrently need workspaces of their own.  The
 * layout's workspace may be reused once coll_moe_layout has completed on the
 * same stream, if it is large enough.
 * recv_rows_capacity: as for coll_all_to_all_v, an upper bound of the rows
 * received by all ranks together; it only sizes the launch and never
 * addresses memory, so a wrong bound costs time, not correctness.
 * recv_rows[d]: rows recvbufs[d] holds (HOST int64, nranks entries; NULL =
 * unbounded).  A (d, s) block -- the rows s sent to d, every one of d's
 * experts -- with a negative expert count, or whose rows do not all lie
 * inside recvbufs[d], is left as it is, as coll_all_to_all_v bounds its
 * blocks.  Rows whose
 * hidden is a multiple of 8 with 16-byte aligned buffers, a nonzero capacity,
 * a workspace of coll_moe_expert_workspace_bytes(nranks, n_experts,
 * recv_rows_capacity) bytes and nranks * n_experts <= 8192 take the faster
 * path: a pre-kernel writes one descriptor per row of the capacity and one
 * wave per (row, 64-unit segment) scales it.  Otherwise one workgroup per
 * tile of the bound searches the table (0 = unknown: a resident grid).
 * Errors: COLL_ERR_INVALID_ARG for a NULL or misaligned workspace, a smaller
 * workspace_bytes, n_experts outside [1, 1024] or not a multiple of nranks,
 * NULL tables or receive buffers; COLL_ERR_UNSUPPORTED for a dtype other
 * than bf16.
 */
int coll_moe_expert_scale(int nranks, void *const *recvbufs, const int32_t *expert_counts,
                          const int64_t *rdispls, int n_experts, size_t hidden,
                          coll_dtype_t dtype, size_t recv_rows_capacity,
                          const int64_t *recv_rows, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * The faster path of coll_moe_expert_scale as two calls, so that its
 * pre-kernels can run off the critical path: they read only expert_counts,
 * rdispls and the receive buffers' addresses, not the rows, so a caller can
 * issue the build (for instance on a second stream) once coll_moe_layout has
 * completed, while the rows are still being exchanged.
 *   coll_moe_expert_scale_build: the arguments of coll_moe_expert_scale;
 *   writes the workspace (the row-prefix table and one descriptor per row of
 *   recv_rows_capacity, holding the row's address and expert) and touches no
 *   row.  Returns COLL_ERR_UNSUPPORTED, with nothing launched, where
 *   coll_moe_expert_scale would not take the faster path (its conditions
 *   above): call coll_moe_expert_scale then.
 *   coll_moe_expert_scale_apply: scales the rows from a workspace that a
 *   build wrote for the same nranks, n_experts, hidden, receive buffers and
 *   capacity; the rows end as the one-call form leaves them.  The caller
 *   orders it after the build (same stream, or an event) and after the rows
 *   have arrived, and does not reuse the workspace until it completes.
 * Errors: as coll_moe_expert_scale; the apply returns COLL_ERR_INVALID_ARG
 * for NULL receive buffers, a NULL or misaligned workspace or one below
 * coll_moe_expert_workspace_bytes(nranks, n_experts, recv_rows_capacity),
 * and COLL_ERR_UNSUPPORTED where the faster path does not apply.
 */
int coll_moe_expert_scale_build(int nranks, void *const *recvbufs, const int32_t *expert_counts,
                                const int64_t *rdispls, int n_experts, size_t hidden,
                                coll_dtype_t dtype, size_t recv_rows_capacity,
                                const int64_t *recv_rows, void *workspace,
                                size_t workspace_bytes, void *stream);
int coll_moe_expert_scale_apply(int nranks, void *const *recvbufs, int n_experts, size_t hidden,
                                coll_dtype_t dtype, size_t recv_rows_capacity, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Combine (results return to the token's owner and are gate-weighted):
 *   out[s][t] = rne( sum_{k=0..topk-1} w[s][t*topk+k] * widen(back[s][pos[s][t*topk+k]]) )
 * with k ascending, the accumulator seeded by the k = 0 product, multiply and
 * add rounded separately (no FMA) and one final rounding: bit-identical to
 * the fold written out.  A pair whose pos is outside [0, tokens*topk) (the
 * layout's -1) adds no term: the fold runs over the token's other pairs in
 * order, seeded by the first of them, and a token with none left gets +0.
 * back[s]: [tokens*topk, hidden] bf16 in s's send-slot
 * order (the output of the reverse All-to-All-v); w[s]: fp32 [tokens, topk];
 * out[s]: bf16 [tokens, hidden], must not overlap back[s].
 */
int coll_moe_combine(int nranks, const void *const *back, const int32_t *const *pos,
                     const float *const *topk_w, int tokens, int topk, size_t hidden,
                     coll_dtype_t dtype, void *const *out, void *stream);

/*
 * Fused dispatch -- the tutorial's 8.4 dispatch (tokens go to the rank that
 * owns their expert) as one pass: on one GPU the exchange is a store into the
 * destination's buffer, so the permute writes each (t, k) row straight to its
 * receive row instead of a send buffer:
 *   recv[d][rdispls[d*R+s] + p - sdispls[s*R+d]] = x[s][t],  p = pos[s][t*topk+k],
 * where d is the rank whose send block [sdispls[s*R+d], sdispls[s*R+d] +
 * sendcounts[s*R+d]) holds p.  recvbufs end up exactly as after
 * coll_moe_permute followed by coll_all_to_all_v with the same layout.
 *   x[s]: [tokens, hidden]; pos, counts, displacements: the outputs of
 *   coll_moe_layout (device arrays); recvbufs[d]: the receive buffers, NULL
 *   allowed for a rank that receives no rows.  Any dtype (a copy).
 * A slot that no block holds (-1: a pair with no expert) is not written.
 *   recv_rows[d]: rows recvbufs[d] holds (HOST int64, nranks entries; NULL =
 *   unbounded): a block whose receive rows do not all exist holds no slot, so
 *   its rows are not written (as coll_all_to_all_v bounds its blocks).
 */
int coll_moe_dispatch(int nranks, const void *const *x, const int32_t *const *pos,
                      const int64_t *sendcounts, const int64_t *sdispls, const int64_t *rdispls,
                      int tokens, int topk, size_t hidden, coll_dtype_t dtype,
                      void *const *recvbufs, const int64_t *recv_rows, void *stream);

/*
 * Fused combine -- the tutorial's 8.4 combine (results return to the token's
 * owner and are gate-weighted) as one pass: the reverse exchange is a read of
 * the destination's buffer, so each (t, k) row is read where
 * coll_moe_dispatch put it:
 *   out[s][t] = rne( sum_{k ascending} w[s][t*topk+k] * widen(y_k) ),
 *   y_k = recvbufs[d][rdispls[d*R+s] + p - sdispls[s*R+d]]  (p, d as above),
 * with the fold, rounding and no-FMA rule of coll_moe_combine: bit-identical
 * to coll_all_to_all_v_reverse followed by coll_moe_combine.
 * topk_ids != NULL (the routing, [tokens, topk] int32 per rank): the test
 * expert of coll_moe_expert_scale is applied to each row as it is read,
 * y_k = rne(widen(row) * (1 + e/256)) with e = topk_ids[s][t*topk+k], so the
 * expert op, the reverse exchange and the combine are one read of recvbufs
 * (which is not modified).  topk_ids == NULL: the rows are used as they are.
 *   bf16 only; out[s]: [tokens, hidden], must not overlap any recvbufs.
 * A slot that no block holds (the layout's -1 for a pair with no expert)
 * adds no term, as in coll_moe_combine.
 *   recv_rows[d]: rows recvbufs[d] holds (HOST int64, nranks entries; NULL =
 *   unbounded): a block whose receive rows do not all exist holds no slot, so
 *   its rows are not read and add no term.
 */
int coll_moe_combine_recv(int nranks, const void *const *recvbufs, const int32_t *const *pos,
                          const int64_t *sendcounts, const int64_t *sdispls,
                          const int64_t *rdispls, const float *const *topk_w,
                          const int32_t *const *topk_ids, int tokens, int topk, size_t hidden,
                          coll_dtype_t dtype, void *const *out, const int64_t *recv_rows,
                          void *stream);

#ifdef __cplusplus
}
#endif

#endif /* COLL_H */
