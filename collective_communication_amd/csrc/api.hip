// api.hip -- the extern "C" boundary of libcoll.so (declared in include/coll.h).
//
// Every entry point validates its arguments on the host, copies the caller's
// host pointer arrays into by-value kernel arguments, and enqueues the
// kernels on the caller's stream.  Nothing is allocated and nothing is
// synchronised; no C++ exception can escape (the code below throws none and
// every HIP call reports through its return code).
#include <stdlib.h>
#include <string.h>

#include "coll_internal.h"

namespace coll {
namespace {

constexpr int kMaxDevices = 64;
struct DevInfo {
  int ready;
  int num_cus;
};
DevInfo g_dev[kMaxDevices];   // per-device compute-unit count (filled once)

long env_long(const char *name, long dflt) {
  const char *v = getenv(name);
  if (!v || !*v) return dflt;
  char *end = nullptr;
  long x = strtol(v, &end, 10);
  return (end && *end == '\0') ? x : dflt;
}

// Tuning knobs, read from the environment once per process.
struct Knobs {
  int wgs_per_cu;
  size_t nt_bytes, nt_store_bytes;
  int a2a_nt;
  long a2a_grid, ar_grid;
  size_t a2a_desc_bytes;
};
const Knobs &knobs() {
  static const Knobs k = [] {
    Knobs v;
    // persistent grids: 4 workgroups of 256 lanes per CU measured best for
    // the test expert (MI355X, 3.5 GiB in place: 4 -> 5655 GB/s, 8 -> 5575,
    // 2 -> 4460)
    const long w = env_long("COLL_WGS_PER_CU", 4);
    v.wgs_per_cu = (int)(w < 1 ? 1 : (w > 64 ? 64 : w));
    const long nt = env_long("COLL_NT_MIN_BYTES", 32L << 20);
    v.nt_bytes = nt < 0 ? 0 : (size_t)nt;
    // reductions to 1/R of their input: the sums are stored cacheable unless
    // the call writes at least the Infinity Cache's 256 MiB.  MI355X, R = 8,
    // ReduceScatter then AllGather of its output, 32..128 MiB written:
    // cacheable 7-9% faster; 256 / 512 MiB: non-temporal 1-5% faster.
    const long nts = env_long("COLL_NT_STORE_MIN_BYTES", 256L << 20);
    v.nt_store_bytes = nts < 0 ? 0 : (size_t)nts;
    v.a2a_nt = env_long("COLL_A2A_NT", 1) ? 1 : 0;
    const long g = env_long("COLL_A2A_GRID", 0);
    v.a2a_grid = (g > 0 && g < 0x7FFFFFFFL) ? g : 0;
    const long ga = env_long("COLL_AR_GRID", 0);
    v.ar_grid = (ga > 0 && ga < 0x7FFFFFFFL) ? ga : 0;
    // All-to-All-v descriptor form from this receive capacity up.  MI355X,
    // R = 8, graph replay: MoE-shaped 224 MiB 74.2% vs 73.3% for the plain
    // form, 3.5 GiB 80.1% vs 74.2%; below, its second launch costs more than
    // it saves (56 MiB: 25.2 vs 21.7 us; uniform 128 MiB: 49.0 vs 46.4 us).
    const long ad = env_long("COLL_A2A_DESC_MIN_BYTES", 192L << 20);
    v.a2a_desc_bytes = ad < 0 ? 0 : (size_t)ad;
    return v;
  }();
  return k;
}

}  // namespace

Launch launch_ctx(void *stream) {
  Launch L;
  L.stream = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  if (!g_dev[dev].ready) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    g_dev[dev].num_cus = cus;
    g_dev[dev].ready = 1;
  }
  L.num_cus = g_dev[dev].num_cus;
  const Knobs &k = knobs();
  L.wgs_per_cu = k.wgs_per_cu;
  L.nt_bytes = k.nt_bytes;
  L.nt_store_bytes = k.nt_store_bytes;
  L.a2a_nt = k.a2a_nt;
  L.a2a_grid = k.a2a_grid;
  L.ar_grid = k.ar_grid;
  return L;
}

}  // namespace coll

using namespace coll;

namespace {

bool ranks_ok(int R) { return R >= 1 && R <= COLL_MAX_RANKS; }
bool dtype_ok(int dt) { return dt >= COLL_BF16 && dt <= COLL_INT32; }
bool op_ok(int op) { return op >= COLL_SUM && op <= COLL_MIN; }

// count * elem * factor must stay far from size_t overflow (2^56 bytes)
bool bytes_ok(size_t count, size_t elem, size_t factor) {
  const size_t lim = (size_t)1 << 56;
  return count < lim / (elem * (factor ? factor : 1));
}

// Copy R host pointers; false if the array or any entry is NULL.
bool fill_in(int R, const void *const *src, const void **dst) {
  if (!src) return false;
  for (int r = 0; r < R; r++) {
    if (!src[r]) return false;
    dst[r] = src[r];
  }
  return true;
}
bool fill_out(int R, void *const *src, void **dst) {
  if (!src) return false;
  for (int r = 0; r < R; r++) {
    if (!src[r]) return false;
    dst[r] = src[r];
  }
  return true;
}

}  // namespace

extern "C" {

const char *coll_status_string(int status) {
  switch (status) {
    case COLL_OK: return "COLL_OK";
    case COLL_ERR_INVALID_ARG: return "COLL_ERR_INVALID_ARG: invalid argument";
    case COLL_ERR_UNSUPPORTED: return "COLL_ERR_UNSUPPORTED: unsupported dtype, op or size";
    case COLL_ERR_HIP: return "COLL_ERR_HIP: HIP launch or runtime error";
    default: return "unknown coll status";
  }
}

int coll_version(void) { return 1 * 10000 + 1 * 100 + 0; }

int coll_arena_layout(int n, const size_t *bytes, size_t *offsets, size_t *total) {
  if (n < 0 || !total || (n > 0 && (!bytes || !offsets))) return COLL_ERR_INVALID_ARG;
  const size_t page = COLL_ARENA_ALIGN;
  const size_t lim = (size_t)1 << 56;
  size_t end = 0;
  for (int k = 0; k < n; k++) {
    if (bytes[k] >= lim) return COLL_ERR_INVALID_ARG;
    const size_t start = (end + page - 1) / page * page +
                         (size_t)(k % COLL_ARENA_COLORS) * COLL_ARENA_COLOR_BYTES;
    offsets[k] = start;
    end = start + bytes[k];
    if (end >= lim) return COLL_ERR_INVALID_ARG;
  }
  *total = end;
  return COLL_OK;
}

int coll_allreduce(int R, const void *const *sendbufs, void *const *recvbufs, size_t count,
                   coll_dtype_t dtype, coll_op_t op, void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
  if (!op_ok(op)) return COLL_ERR_UNSUPPORTED;
  if (count == 0) return COLL_OK;
  if (!bytes_ok(count, dtype_size(dtype), 2 * (size_t)R)) return COLL_ERR_INVALID_ARG;
  RankPtrs p{};
  if (!fill_in(R, sendbufs, p.in) || !fill_out(R, recvbufs, p.out)) return COLL_ERR_INVALID_ARG;
  return launch_allreduce(launch_ctx(stream), R, p, count, dtype, op);
}

int coll_reduce_scatter(int R, const void *const *sendbufs, void *const *recvbufs,
                        size_t recvcount, coll_dtype_t dtype, coll_op_t op, void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
  if (!op_ok(op)) return COLL_ERR_UNSUPPORTED;
  if (recvcount == 0) return COLL_OK;
  if (!bytes_ok(recvcount, dtype_size(dtype), (size_t)R * (R + 1))) return COLL_ERR_INVALID_ARG;
  RankPtrs p{};
  if (!fill_in(R, sendbufs, p.in) || !fill_out(R, recvbufs, p.out)) return COLL_ERR_INVALID_ARG;
  return launch_reduce_scatter(launch_ctx(stream), R, p, recvcount, dtype, op, R);
}

int coll_reduce(int R, const void *const *sendbufs, void *recvbuf_root, int root, size_t count,
                coll_dtype_t dtype, coll_op_t op, void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype) || root < 0 || root >= R) return COLL_ERR_INVALID_ARG;
  if (!op_ok(op)) return COLL_ERR_UNSUPPORTED;
  if (count == 0) return COLL_OK;
  if (!recvbuf_root || !bytes_ok(count, dtype_size(dtype), (size_t)R + 1))
    return COLL_ERR_INVALID_ARG;
  RankPtrs p{};
  if (!fill_in(R, sendbufs, p.in)) return COLL_ERR_INVALID_ARG;
  p.out[0] = recvbuf_root;
  return launch_reduce_scatter(launch_ctx(stream), R, p, count, dtype, op, 1);
}

int coll_scatter(int R, const void *sendbuf_root, void *const *recvbufs, int root,
                 size_t recvcount, coll_dtype_t dtype, void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype) || root < 0 || root >= R) return COLL_ERR_INVALID_ARG;
  if (recvcount == 0) return COLL_OK;
  if (!sendbuf_root || !recvbufs || !bytes_ok(recvcount, dtype_size(dtype), 2 * (size_t)R))
    return COLL_ERR_INVALID_ARG;
  RankPtrs p{};
  for (int r = 0; r < R; r++) {
    if (!recvbufs[r] && r != root) return COLL_ERR_INVALID_ARG;
    p.out[r] = recvbufs[r];
  }
  return launch_scatter(launch_ctx(stream), R, sendbuf_root, p, recvcount * dtype_size(dtype));
}

int coll_all_gather(int R, const void *const *sendbufs, void *const *recvbufs, size_t sendcount,
                    coll_dtype_t dtype, void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
  if (sendcount == 0) return COLL_OK;
  if (!bytes_ok(sendcount, dtype_size(dtype), (size_t)R * (R + 1))) return COLL_ERR_INVALID_ARG;
  RankPtrs p{};
  if (!fill_in(R, sendbufs, p.in) || !fill_out(R, recvbufs, p.out)) return COLL_ERR_INVALID_ARG;
  return launch_all_gather(launch_ctx(stream), R, p, sendcount * dtype_size(dtype));
}

int coll_gather(int R, const void *const *sendbufs, void *recvbuf_root, int root, size_t outer,
                size_t inner, coll_dtype_t dtype, void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype) || root < 0 || root >= R) return COLL_ERR_INVALID_ARG;
  if (outer == 0 || inner == 0) return COLL_OK;
  if (!recvbuf_root || !bytes_ok(outer, inner * dtype_size(dtype), 2 * (size_t)R))
    return COLL_ERR_INVALID_ARG;
  if (inner > ((size_t)1 << 40) / outer) return COLL_ERR_INVALID_ARG;
  RankPtrs p{};
  if (!fill_in(R, sendbufs, p.in)) return COLL_ERR_INVALID_ARG;
  return launch_gather(launch_ctx(stream), R, p, recvbuf_root, outer, inner * dtype_size(dtype));
}

int coll_broadcast(int R, const void *sendbuf_root, void *const *recvbufs, int root, size_t count,
                   coll_dtype_t dtype, void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype) || root < 0 || root >= R) return COLL_ERR_INVALID_ARG;
  if (count == 0) return COLL_OK;
  if (!sendbuf_root || !recvbufs || !bytes_ok(count, dtype_size(dtype), (size_t)R + 1))
    return COLL_ERR_INVALID_ARG;
  RankPtrs p{};
  for (int r = 0; r < R; r++) {
    if (!recvbufs[r] && r != root) return COLL_ERR_INVALID_ARG;
    p.out[r] = recvbufs[r];
  }
  return launch_broadcast(launch_ctx(stream), R, sendbuf_root, p, count * dtype_size(dtype));
}

// Rows each rank's buffer holds, from the caller's host array (NULL: that
// side is not bounded); a NULL buffer holds no rows whatever the array says.
// false for a negative entry.
static bool fill_rows(int R, const int64_t *rows, const void *const *bufs, RankRows &out) {
  for (int r = 0; r < COLL_MAX_RANKS; r++) out.n[r] = INT64_MAX;
  for (int r = 0; r < R; r++) {
    if (rows) {
      if (rows[r] < 0) return false;
      out.n[r] = rows[r];
    }
    if (!bufs[r]) out.n[r] = 0;
  }
  return true;
}

int coll_all_to_all_v(int R, const void *const *sendbufs, const int64_t *sendcounts,
                      const int64_t *sdispls, void *const *recvbufs, const int64_t *rdispls,
                      size_t row_elems, coll_dtype_t dtype, size_t recv_rows_capacity,
                      const int64_t *send_rows, const int64_t *recv_rows, void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
  if (row_elems == 0) return COLL_OK;
  if (!sendcounts || !sdispls || !rdispls || !bytes_ok(row_elems, dtype_size(dtype), 1))
    return COLL_ERR_INVALID_ARG;
  if (!sendbufs || !recvbufs) return COLL_ERR_INVALID_ARG;
  RankPtrs p{};
  for (int r = 0; r < R; r++) {       // NULL is allowed: a rank that moves no rows
    p.in[r] = sendbufs[r];
    p.out[r] = recvbufs[r];
  }
  if (recv_rows_capacity > ((size_t)1 << 48) / (row_elems * dtype_size(dtype)))
    return COLL_ERR_INVALID_ARG;
  RowLimits lim;
  if (!fill_rows(R, send_rows, sendbufs, lim.in) ||
      !fill_rows(R, recv_rows, reinterpret_cast<const void *const *>(recvbufs), lim.out))
    return COLL_ERR_INVALID_ARG;
  return launch_a2av(launch_ctx(stream), R, p, lim, sendcounts, sdispls, rdispls, 0,
                     row_elems * dtype_size(dtype), recv_rows_capacity);
}

size_t coll_all_to_all_v_workspace_bytes(int R, size_t recv_rows_capacity, size_t row_elems,
                                        coll_dtype_t dtype) {
  if (!ranks_ok(R) || !dtype_ok(dtype) || row_elems == 0) return 0;
  if (!bytes_ok(row_elems, dtype_size(dtype), 1)) return 0;
  const size_t row_bytes = row_elems * dtype_size(dtype);
  if (recv_rows_capacity > ((size_t)1 << 48) / row_bytes) return 0;
  return a2av_workspace_bytes(R, recv_rows_capacity, row_bytes, knobs().a2a_desc_bytes);
}

// The workspace form, forward (ct = 0) or reverse (ct = 1: the tables are the
// forward exchange's, sendbufs are its receive buffers and recvbufs its send
// buffers, sdispls its rdispls and rdispls its sdispls, send_rows the rows
// of its receive buffers and recv_rows those of its send buffers).
// build_only: the first kernel alone (coll_all_to_all_v_ws_build), which
// needs the descriptor form to apply.
static int a2av_ws_call(int R, const void *const *sendbufs, const int64_t *sendcounts,
                        const int64_t *sdispls, void *const *recvbufs, const int64_t *rdispls,
                        int ct, size_t row_elems, coll_dtype_t dtype, size_t recv_rows_capacity,
                        const int64_t *send_rows, const int64_t *recv_rows, void *workspace,
                        size_t workspace_bytes, void *stream, bool build_only = false) {
  if (!ranks_ok(R) || !dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
  if (row_elems == 0) return COLL_OK;
  if (!sendcounts || !sdispls || !rdispls || !bytes_ok(row_elems, dtype_size(dtype), 1))
    return COLL_ERR_INVALID_ARG;
  if (!sendbufs || !recvbufs) return COLL_ERR_INVALID_ARG;
  const size_t row_bytes = row_elems * dtype_size(dtype);
  if (recv_rows_capacity > ((size_t)1 << 48) / row_bytes) return COLL_ERR_INVALID_ARG;
  const size_t need =
      a2av_workspace_bytes(R, recv_rows_capacity, row_bytes, knobs().a2a_desc_bytes);
  if (need > 0 && (!workspace || ((uintptr_t)workspace & 255) != 0 || workspace_bytes < need))
    return COLL_ERR_INVALID_ARG;
  RankPtrs p{};
  for (int r = 0; r < R; r++) {       // NULL is allowed: a rank that moves no rows
    p.in[r] = sendbufs[r];
    p.out[r] = recvbufs[r];
  }
  RowLimits lim;
  if (!fill_rows(R, send_rows, sendbufs, lim.in) ||
      !fill_rows(R, recv_rows, reinterpret_cast<const void *const *>(recvbufs), lim.out))
    return COLL_ERR_INVALID_ARG;
  if (build_only) {
    if (need == 0) return COLL_ERR_UNSUPPORTED;
    return launch_a2av_ws_build(launch_ctx(stream), R, p, lim, sendcounts, sdispls, rdispls, ct,
                                row_bytes, recv_rows_capacity, workspace);
  }
  if (need == 0)
    return launch_a2av(launch_ctx(stream), R, p, lim, sendcounts, sdispls, rdispls, ct,
                       row_bytes, recv_rows_capacity);
  return launch_a2av_ws(launch_ctx(stream), R, p, lim, sendcounts, sdispls, rdispls, ct,
                        row_bytes, recv_rows_capacity, workspace);
}

int coll_all_to_all_v_ws(int R, const void *const *sendbufs, const int64_t *sendcounts,
                         const int64_t *sdispls, void *const *recvbufs, const int64_t *rdispls,
                         size_t row_elems, coll_dtype_t dtype, size_t recv_rows_capacity,
                         const int64_t *send_rows, const int64_t *recv_rows, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return a2av_ws_call(R, sendbufs, sendcounts, sdispls, recvbufs, rdispls, 0, row_elems, dtype,
                      recv_rows_capacity, send_rows, recv_rows, workspace, workspace_bytes,
                      stream);
}

int coll_all_to_all_v_ws_build(int R, const void *const *sendbufs, const int64_t *sendcounts,
                               const int64_t *sdispls, void *const *recvbufs,
                               const int64_t *rdispls, size_t row_elems, coll_dtype_t dtype,
                               size_t recv_rows_capacity, const int64_t *send_rows,
                               const int64_t *recv_rows, void *workspace, size_t workspace_bytes,
                               void *stream) {
  if (row_elems == 0) return COLL_ERR_UNSUPPORTED;
  return a2av_ws_call(R, sendbufs, sendcounts, sdispls, recvbufs, rdispls, 0, row_elems, dtype,
                      recv_rows_capacity, send_rows, recv_rows, workspace, workspace_bytes,
                      stream, true);
}

int coll_all_to_all_v_reverse_build(int R, const void *const *recvbufs,
                                    const int64_t *sendcounts, const int64_t *sdispls,
                                    void *const *sendbufs, const int64_t *rdispls,
                                    size_t row_elems, coll_dtype_t dtype,
                                    size_t send_rows_capacity, const int64_t *send_rows,
                                    const int64_t *recv_rows, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  if (row_elems == 0) return COLL_ERR_UNSUPPORTED;
  return a2av_ws_call(R, recvbufs, sendcounts, rdispls, sendbufs, sdispls, 1, row_elems, dtype,
                      send_rows_capacity, recv_rows, send_rows, workspace, workspace_bytes,
                      stream, true);
}

int coll_all_to_all_v_ws_copy(int R, size_t row_elems, coll_dtype_t dtype,
                              size_t rows_capacity, void *workspace, size_t workspace_bytes,
                              void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype) || row_elems == 0 ||
      !bytes_ok(row_elems, dtype_size(dtype), 1))
    return COLL_ERR_INVALID_ARG;
  const size_t row_bytes = row_elems * dtype_size(dtype);
  if (rows_capacity > ((size_t)1 << 48) / row_bytes) return COLL_ERR_INVALID_ARG;
  const size_t need = a2av_workspace_bytes(R, rows_capacity, row_bytes, knobs().a2a_desc_bytes);
  if (need == 0) return COLL_ERR_UNSUPPORTED;
  if (!workspace || ((uintptr_t)workspace & 255) != 0 || workspace_bytes < need)
    return COLL_ERR_INVALID_ARG;
  return launch_a2av_ws_copy(launch_ctx(stream), R, row_bytes, rows_capacity, workspace);
}

int coll_all_to_all_v_reverse(int R, const void *const *recvbufs, const int64_t *sendcounts,
                              const int64_t *sdispls, void *const *sendbufs,
                              const int64_t *rdispls, size_t row_elems, coll_dtype_t dtype,
                              size_t send_rows_capacity, const int64_t *send_rows,
                              const int64_t *recv_rows, void *workspace, size_t workspace_bytes,
                              void *stream) {
  // data moves from the forward receive buffers back to the forward send
  // buffers: the forward rdispls locate the source rows, sdispls the
  // destination rows, and the counts are read transposed.  No workspace:
  // the plain form.
  if (!workspace && workspace_bytes == 0) {
    if (!ranks_ok(R) || !dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
    if (row_elems == 0) return COLL_OK;
    if (!sendcounts || !sdispls || !rdispls || !bytes_ok(row_elems, dtype_size(dtype), 1))
      return COLL_ERR_INVALID_ARG;
    if (!sendbufs || !recvbufs) return COLL_ERR_INVALID_ARG;
    const size_t row_bytes = row_elems * dtype_size(dtype);
    if (send_rows_capacity > ((size_t)1 << 48) / row_bytes) return COLL_ERR_INVALID_ARG;
    RankPtrs p{};
    for (int r = 0; r < R; r++) {     // NULL is allowed: a rank that moves no rows
      p.in[r] = recvbufs[r];
      p.out[r] = sendbufs[r];
    }
    RowLimits lim;            // rows are read from recvbufs and written to sendbufs
    if (!fill_rows(R, recv_rows, reinterpret_cast<const void *const *>(recvbufs), lim.in) ||
        !fill_rows(R, send_rows, reinterpret_cast<const void *const *>(sendbufs), lim.out))
      return COLL_ERR_INVALID_ARG;
    return launch_a2av(launch_ctx(stream), R, p, lim, sendcounts, rdispls, sdispls, 1, row_bytes,
                       send_rows_capacity);
  }
  return a2av_ws_call(R, reinterpret_cast<const void *const *>(recvbufs), sendcounts, rdispls,
                      sendbufs, sdispls, 1, row_elems, dtype, send_rows_capacity, recv_rows,
                      send_rows, workspace, workspace_bytes, stream);
}

int coll_all_to_all(int R, const void *const *sendbufs, void *const *recvbufs,
                    size_t count_per_peer, coll_dtype_t dtype, void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
  if (count_per_peer == 0) return COLL_OK;
  if (!bytes_ok(count_per_peer, dtype_size(dtype), 2 * (size_t)R * R)) return COLL_ERR_INVALID_ARG;
  RankPtrs p{};
  if (!fill_in(R, sendbufs, p.in) || !fill_out(R, recvbufs, p.out)) return COLL_ERR_INVALID_ARG;
  // one sequence row whose R chunks are the per-peer blocks
  return launch_reshard(launch_ctx(stream), R, p, 1, count_per_peer * dtype_size(dtype), true);
}

int coll_seq_heads_reshard(int R, const void *const *in, void *const *out, size_t seq_local,
                           size_t heads, size_t head_dim, coll_dtype_t dtype, int to_heads,
                           void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype) || heads == 0 || heads % (size_t)R != 0)
    return COLL_ERR_INVALID_ARG;
  if (seq_local == 0 || head_dim == 0) return COLL_OK;
  const size_t chunk = heads / (size_t)R * head_dim;
  if (!bytes_ok(chunk, dtype_size(dtype), 1) ||
      !bytes_ok(seq_local, chunk * dtype_size(dtype), 2 * (size_t)R * R))
    return COLL_ERR_INVALID_ARG;
  RankPtrs p{};
  if (!fill_in(R, in, p.in) || !fill_out(R, out, p.out)) return COLL_ERR_INVALID_ARG;
  return launch_reshard(launch_ctx(stream), R, p, seq_local, chunk * dtype_size(dtype),
                        to_heads != 0);
}

int coll_lse_merge(int R, const void *const *o_parts, const float *const *lse_parts,
                   void *const *o_out, float *const *lse_out, size_t rows, size_t head_dim,
                   coll_dtype_t dtype, void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype)) return COLL_ERR_INVALID_ARG;
  if (dtype != COLL_BF16 && dtype != COLL_FP32) return COLL_ERR_UNSUPPORTED;
  if (rows == 0 || head_dim == 0) return COLL_OK;
  if (!bytes_ok(rows, head_dim * dtype_size(dtype), 2 * (size_t)R)) return COLL_ERR_INVALID_ARG;
  RankPtrs o{};
  PtrTable li{};
  MutPtrTable lo{};
  if (!fill_in(R, o_parts, o.in) || !fill_out(R, o_out, o.out) ||
      !fill_in(R, reinterpret_cast<const void *const *>(lse_parts), li.p))
    return COLL_ERR_INVALID_ARG;
  if (lse_out) {
    // An LSE output may not overlap any LSE input: a row's output is stored
    // while workgroups of other segments of that row may still read its inputs.
    const size_t lb = rows * sizeof(float);
    for (int r = 0; r < R; r++) {
      lo.p[r] = lse_out[r];                                  // NULL entries: not written
      if (!lse_out[r]) continue;
      const uintptr_t a = reinterpret_cast<uintptr_t>(lse_out[r]);
      for (int q = 0; q < R; q++) {
        const uintptr_t b = reinterpret_cast<uintptr_t>(li.p[q]);
        if (a < b + lb && b < a + lb) return COLL_ERR_INVALID_ARG;
      }
    }
  }
  return launch_lse_merge(launch_ctx(stream), R, o, li, lo, rows, head_dim, dtype);
}

size_t coll_moe_workspace_bytes(int R, int tokens, int topk, int n_experts) {
  if (!ranks_ok(R) || tokens < 0 || topk < 1 || n_experts < 1 || n_experts > kMoeMaxExperts ||
      n_experts % R != 0 || (int64_t)tokens * topk >= ((int64_t)1 << 31))
    return 0;
  return moe_workspace_bytes(R, tokens, topk, n_experts);
}

int coll_moe_layout(int R, const int32_t *const *topk_ids, int tokens, int topk, int n_experts,
                    int64_t *sendcounts, int64_t *sdispls, int64_t *rdispls,
                    int32_t *expert_counts, int32_t *const *pos, void *workspace,
                    size_t workspace_bytes, void *stream) {
  size_t need = coll_moe_workspace_bytes(R, tokens, topk, n_experts);
  if (need == 0) return COLL_ERR_INVALID_ARG;
  if (!sendcounts || !sdispls || !rdispls || !expert_counts || !workspace ||
      workspace_bytes < need || ((uintptr_t)workspace & 255u))
    return COLL_ERR_INVALID_ARG;
  PtrTable ids{};
  MutPtrTable ps{};
  if (tokens > 0) {
    if (!fill_in(R, reinterpret_cast<const void *const *>(topk_ids), ids.p) ||
        !fill_out(R, reinterpret_cast<void *const *>(pos), ps.p))
      return COLL_ERR_INVALID_ARG;
  }
  return launch_moe_layout(launch_ctx(stream), R, ids, tokens, topk, n_experts, sendcounts,
                           sdispls, rdispls, expert_counts, ps, workspace);
}

int coll_moe_layout_noalloc(int R, const int32_t *const *topk_ids, int tokens, int topk,
                            int n_experts, int64_t *sendcounts, int64_t *sdispls,
                            int64_t *rdispls, int32_t *expert_counts, int32_t *const *pos,
                            void *stream) {
  const size_t need = coll_moe_workspace_bytes(R, tokens, topk, n_experts);
  if (need == 0 || need > kMoeStaticBytes) return COLL_ERR_INVALID_ARG;
  if (!sendcounts || !sdispls || !rdispls || !expert_counts) return COLL_ERR_INVALID_ARG;
  PtrTable ids{};
  MutPtrTable ps{};
  if (tokens > 0) {
    if (!fill_in(R, reinterpret_cast<const void *const *>(topk_ids), ids.p) ||
        !fill_out(R, reinterpret_cast<void *const *>(pos), ps.p))
      return COLL_ERR_INVALID_ARG;
  }
  void *scratch = moe_static_scratch();
  if (!scratch) return COLL_ERR_HIP;
  return launch_moe_layout(launch_ctx(stream), R, ids, tokens, topk, n_experts, sendcounts,
                           sdispls, rdispls, expert_counts, ps, scratch);
}

int coll_moe_permute(int R, const void *const *x, const int32_t *const *pos, int tokens, int topk,
                     size_t hidden, coll_dtype_t dtype, void *const *sendbufs, void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype) || tokens < 0 || topk < 1) return COLL_ERR_INVALID_ARG;
  if (tokens == 0 || hidden == 0) return COLL_OK;
  if ((int64_t)tokens * topk >= ((int64_t)1 << 31) || !bytes_ok(hidden, dtype_size(dtype), 1))
    return COLL_ERR_INVALID_ARG;
  PtrTable xs{}, ps{};
  MutPtrTable ss{};
  if (!fill_in(R, x, xs.p) || !fill_in(R, reinterpret_cast<const void *const *>(pos), ps.p) ||
      !fill_out(R, sendbufs, ss.p))
    return COLL_ERR_INVALID_ARG;
  return launch_moe_permute(launch_ctx(stream), R, xs, ps, tokens, topk,
                            hidden * dtype_size(dtype), ss);
}

size_t coll_moe_expert_workspace_bytes(int R, int n_experts, size_t recv_rows_capacity) {
  if (!ranks_ok(R) || n_experts < 1 || n_experts > kMoeMaxExperts || n_experts % R != 0) return 0;
  if (recv_rows_capacity > ((size_t)1 << 48)) return 0;
  return moe_expert_workspace_bytes(R, n_experts, recv_rows_capacity);
}

// coll_moe_expert_scale (how = 0), its build (1) or its apply (2; the
// tables and recv_rows are not read).
static int expert_call(int how, int R, void *const *recvbufs, const int32_t *expert_counts,
                       const int64_t *rdispls, int n_experts, size_t hidden, coll_dtype_t dtype,
                       size_t recv_rows_capacity, const int64_t *recv_rows, void *workspace,
                       size_t workspace_bytes, void *stream) {
  if (!ranks_ok(R) || n_experts < 1 || n_experts > kMoeMaxExperts || n_experts % R != 0)
    return COLL_ERR_INVALID_ARG;
  if (dtype != COLL_BF16) return COLL_ERR_UNSUPPORTED;
  if (hidden == 0) return how == 0 ? COLL_OK : COLL_ERR_UNSUPPORTED;
  if ((how != 2 && (!expert_counts || !rdispls)) || hidden >= ((size_t)1 << 31))
    return COLL_ERR_INVALID_ARG;
  const size_t need = how == 2 ? moe_expert_workspace_bytes(R, n_experts, recv_rows_capacity)
                               : moe_expert_table_bytes(R, n_experts);
  if (!workspace || ((uintptr_t)workspace & 255) != 0 || workspace_bytes < need)
    return COLL_ERR_INVALID_ARG;
  MutPtrTable rs{};
  if (!fill_out(R, recvbufs, rs.p)) return COLL_ERR_INVALID_ARG;
  if (recv_rows_capacity > ((size_t)1 << 48) / hidden) return COLL_ERR_INVALID_ARG;
  if (how != 0 && !moe_expert_rows_apply(R, rs, n_experts, hidden, recv_rows_capacity,
                                         workspace_bytes))
    return COLL_ERR_UNSUPPORTED;
  if (how == 2)
    return launch_moe_expert_apply(launch_ctx(stream), R, rs, n_experts, hidden,
                                   recv_rows_capacity, workspace, workspace_bytes);
  RankRows rows;
  if (!fill_rows(R, recv_rows, reinterpret_cast<const void *const *>(recvbufs), rows))
    return COLL_ERR_INVALID_ARG;
  const Launch L = launch_ctx(stream);
  if (how == 1)
    return launch_moe_expert_build(L, R, rs, expert_counts, rdispls, n_experts, hidden,
                                   recv_rows_capacity, workspace, workspace_bytes, rows);
  return launch_moe_expert_scale(L, R, rs, expert_counts, rdispls, n_experts, hidden,
                                 recv_rows_capacity, workspace, workspace_bytes, rows);
}

int coll_moe_expert_scale(int R, void *const *recvbufs, const int32_t *expert_counts,
                          const int64_t *rdispls, int n_experts, size_t hidden,
                          coll_dtype_t dtype, size_t recv_rows_capacity,
                          const int64_t *recv_rows, void *workspace, size_t workspace_bytes,
                          void *stream) {
  return expert_call(0, R, recvbufs, expert_counts, rdispls, n_experts, hidden, dtype,
                     recv_rows_capacity, recv_rows, workspace, workspace_bytes, stream);
}

int coll_moe_expert_scale_build(int R, void *const *recvbufs, const int32_t *expert_counts,
                                const int64_t *rdispls, int n_experts, size_t hidden,
                                coll_dtype_t dtype, size_t recv_rows_capacity,
                                const int64_t *recv_rows, void *workspace,
                                size_t workspace_bytes, void *stream) {
  return expert_call(1, R, recvbufs, expert_counts, rdispls, n_experts, hidden, dtype,
                     recv_rows_capacity, recv_rows, workspace, workspace_bytes, stream);
}

int coll_moe_expert_scale_apply(int R, void *const *recvbufs, int n_experts, size_t hidden,
                                coll_dtype_t dtype, size_t recv_rows_capacity, void *workspace,
                                size_t workspace_bytes, void *stream) {
  return expert_call(2, R, recvbufs, nullptr, nullptr, n_experts, hidden, dtype,
                     recv_rows_capacity, nullptr, workspace, workspace_bytes, stream);
}

int coll_moe_combine(int R, const void *const *back, const int32_t *const *pos,
                     const float *const *topk_w, int tokens, int topk, size_t hidden,
                     coll_dtype_t dtype, void *const *out, void *stream) {
  if (!ranks_ok(R) || tokens < 0 || topk < 1) return COLL_ERR_INVALID_ARG;
  if (dtype != COLL_BF16) return COLL_ERR_UNSUPPORTED;
  if (tokens == 0 || hidden == 0) return COLL_OK;
  if ((int64_t)tokens * topk >= ((int64_t)1 << 31) || hidden >= ((size_t)1 << 31))
    return COLL_ERR_INVALID_ARG;
  PtrTable bs{}, ps{}, ws{};
  MutPtrTable os{};
  if (!fill_in(R, back, bs.p) || !fill_in(R, reinterpret_cast<const void *const *>(pos), ps.p) ||
      !fill_in(R, reinterpret_cast<const void *const *>(topk_w), ws.p) || !fill_out(R, out, os.p))
    return COLL_ERR_INVALID_ARG;
  return launch_moe_combine(launch_ctx(stream), R, bs, ps, ws, tokens, topk, hidden, os);
}

// Receive pointers of the fused MoE calls: NULL only for ranks that receive
// no rows (as in coll_all_to_all_v).
static bool fill_recv(int R, const void *const *src, const void **dst) {
  if (!src) return false;
  for (int r = 0; r < R; r++) dst[r] = src[r];
  return true;
}

int coll_moe_dispatch(int R, const void *const *x, const int32_t *const *pos,
                      const int64_t *sendcounts, const int64_t *sdispls, const int64_t *rdispls,
                      int tokens, int topk, size_t hidden, coll_dtype_t dtype,
                      void *const *recvbufs, const int64_t *recv_rows, void *stream) {
  if (!ranks_ok(R) || !dtype_ok(dtype) || tokens < 0 || topk < 1) return COLL_ERR_INVALID_ARG;
  if (tokens == 0 || hidden == 0) return COLL_OK;
  if ((int64_t)tokens * topk >= ((int64_t)1 << 31) || !bytes_ok(hidden, dtype_size(dtype), 1))
    return COLL_ERR_INVALID_ARG;
  if (!sendcounts || !sdispls || !rdispls) return COLL_ERR_INVALID_ARG;
  PtrTable xs{}, ps{}, rs{};
  if (!fill_in(R, x, xs.p) || !fill_in(R, reinterpret_cast<const void *const *>(pos), ps.p) ||
      !fill_recv(R, reinterpret_cast<const void *const *>(recvbufs), rs.p))
    return COLL_ERR_INVALID_ARG;
  MutPtrTable out{};
  for (int r = 0; r < R; r++) out.p[r] = const_cast<void *>(rs.p[r]);
  RankRows rows;
  if (!fill_rows(R, recv_rows, rs.p, rows)) return COLL_ERR_INVALID_ARG;
  return launch_moe_dispatch(launch_ctx(stream), R, xs, ps, sendcounts, sdispls, rdispls, tokens,
                             topk, hidden * dtype_size(dtype), out, rows);
}

int coll_moe_combine_recv(int R, const void *const *recvbufs, const int32_t *const *pos,
                          const int64_t *sendcounts, const int64_t *sdispls,
                          const int64_t *rdispls, const float *const *topk_w,
                          const int32_t *const *topk_ids, int tokens, int topk, size_t hidden,
                          coll_dtype_t dtype, void *const *out, const int64_t *recv_rows,
                          void *stream) {
  if (!ranks_ok(R) || tokens < 0 || topk < 1) return COLL_ERR_INVALID_ARG;
  if (dtype != COLL_BF16) return COLL_ERR_UNSUPPORTED;
  if (tokens == 0 || hidden == 0) return COLL_OK;
  if ((int64_t)tokens * topk >= ((int64_t)1 << 31) || hidden >= ((size_t)1 << 31))
    return COLL_ERR_INVALID_ARG;
  if (!sendcounts || !sdispls || !rdispls) return COLL_ERR_INVALID_ARG;
  PtrTable rs{}, ps{}, ws{}, is{};
  MutPtrTable os{};
  if (!fill_recv(R, recvbufs, rs.p) ||
      !fill_in(R, reinterpret_cast<const void *const *>(pos), ps.p) ||
      !fill_in(R, reinterpret_cast<const void *const *>(topk_w), ws.p) || !fill_out(R, out, os.p))
    return COLL_ERR_INVALID_ARG;
  if (topk_ids && !fill_in(R, reinterpret_cast<const void *const *>(topk_ids), is.p))
    return COLL_ERR_INVALID_ARG;
  RankRows rows;
  if (!fill_rows(R, recv_rows, rs.p, rows)) return COLL_ERR_INVALID_ARG;
  return launch_moe_combine_recv(launch_ctx(stream), R, rs, ps, sendcounts, sdispls, rdispls, ws,
                                 topk_ids ? &is : nullptr, tokens, topk, hidden, os, rows);
}

}  // extern "C"
