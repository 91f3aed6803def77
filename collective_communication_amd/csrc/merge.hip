// merge.hip -- context-parallel merge of partial attention outputs
// ("Collective primitives tutorial", sections 5.4.2 and 7.4.3: the partial
// outputs of context-parallel attention cannot be summed as they are; the
// log-sum-exps are gathered first and the corrected contributions summed).
//
// Per (token, head) row with partial outputs o_r and log-sum-exps l_r:
//   m = max_r l_r, e_r = exp(l_r - m), s = sum_r e_r, L = m + log s,
//   o = sum_r (e_r / s) * o_r   (ranks ascending, fp32), delivered to every rank.
// On one GPU the LSE "AllGather" is a read.  A one-wave workgroup owns whole
// rows (rw = 64 / units-per-row of them) or, for rows longer than 64 units,
// one 64-unit segment of a row.  Every lane first issues the R loads of its
// unit; meanwhile one lane per row reads the row's R LSEs and forms its
// weights once (R exp, one log, R divisions), which the row's lanes then
// read from LDS to fold their R partial units and store the result R times.
// Staging it like the AllReduce (a workgroup of R waves, wave r streaming
// rank r through LDS, weights and fold after barriers) gave the same bits but
// ran at 62% of the HBM peak against 73% for this form on MI355X (8 ranks x
// 8192 tokens x 32 heads x 128 bf16): the weights then sit between two
// barriers with no load in flight, where here they overlap the data loads.
#include "coll_internal.h"

#pragma clang fp contract(off)

namespace coll {
namespace {

constexpr int kMergeLanes = 64;

// Weights of one row: w[r] = e_r / s and L; a row whose LSEs are all -inf
// gets w = 0 and L = -inf.
__device__ __forceinline__ void row_weights(const PtrTable &lse, int R, uint64_t row, float *w,
                                            float *L) {
  float l[COLL_MAX_RANKS];
  float m = -__builtin_inff();
  // all R loads first, then the max: a use inside the load's own `if` made
  // the compiler wait for each load in turn
#pragma unroll
  for (int r = 0; r < COLL_MAX_RANKS; r++)
    if (r < R) l[r] = reinterpret_cast<const float *>(lse.p[r])[row];
#pragma unroll
  for (int r = 0; r < COLL_MAX_RANKS; r++)
    if (r < R) m = l[r] > m ? l[r] : m;
  if (m == -__builtin_inff()) {
#pragma unroll
    for (int r = 0; r < COLL_MAX_RANKS; r++) w[r] = 0.0f;
    *L = -__builtin_inff();
    return;
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < COLL_MAX_RANKS; r++) {
    if (r < R) {
      w[r] = expf(l[r] - m);
      s = s + w[r];
    }
  }
#pragma unroll
  for (int r = 0; r < COLL_MAX_RANKS; r++)
    if (r < R) w[r] = w[r] / s;
  *L = m + logf(s);
}

// VEC: 16-byte units (8 bf16 or 4 fp32); otherwise one element per unit.
// upr = units per row; rw = rows per workgroup (upr <= 64) or 1 with nseg
// 64-unit segments per row (upr > 64).
template <int DT, bool VEC, bool NT>
__global__ __launch_bounds__(kMergeLanes) void lse_merge_rows(RankPtrs o, PtrTable lse_in,
                                                              MutPtrTable lse_out, int R,
                                                              uint64_t rows, uint32_t upr,
                                                              uint32_t rw, uint32_t nseg) {
  using F = Fmt<DT>;
  using E = typename F::Elem;
  constexpr int VL = VEC ? F::kLanes : 1;
  __shared__ float s_w[kMergeLanes][COLL_MAX_RANKS];
  __shared__ float s_L[kMergeLanes];
  const uint32_t lane = threadIdx.x;
  uint64_t row0;
  uint32_t seg = 0, q, j;
  if (nseg > 1) {
    row0 = blockIdx.x / nseg;
    seg = blockIdx.x - (uint32_t)row0 * nseg;
    q = 0;
    j = seg * kMergeLanes + lane;
  } else {
    row0 = (uint64_t)blockIdx.x * rw;
    q = lane / upr;
    j = lane - q * upr;
  }
  const uint64_t row = row0 + q;
  const bool active = (nseg > 1 ? j < upr : q < rw) && row < rows;
  const uint64_t x = row * upr + j;
  // 1. the unit's R partial loads, issued before the weights are known
  u32x4 v[COLL_MAX_RANKS];
  E ve[COLL_MAX_RANKS];
  if (active) {
#pragma unroll
    for (int r = 0; r < COLL_MAX_RANKS; r++) {
      if (r < R) {
        if constexpr (VEC) v[r] = ld<u32x4, NT>(o.in[r], x);
        else ve[r] = reinterpret_cast<const E *>(o.in[r])[x];
      }
    }
  }
  // 2. one lane per row forms the row's weights
  if (lane < rw && row0 + lane < rows) {
    float w[COLL_MAX_RANKS], L;
    row_weights(lse_in, R, row0 + lane, w, &L);
#pragma unroll
    for (int r = 0; r < COLL_MAX_RANKS; r++)
      if (r < R) s_w[lane][r] = w[r];
    s_L[lane] = L;
    if (seg == 0) {
      for (int r = 0; r < R; r++)
        if (lse_out.p[r]) reinterpret_cast<float *>(lse_out.p[r])[row0 + lane] = L;
    }
  }
  __syncthreads();
  if (!active) return;
  // 3. fold in ascending rank order, round once, store to every rank
  const bool empty = s_L[q] == -__builtin_inff();
  if constexpr (VEC) {
    float acc[VL];
    {
      const float w0 = s_w[q][0];
      typename F::Acc a = F::widen(v[0]);
#pragma unroll
      for (int e = 0; e < VL; e++) acc[e] = w0 * a.v[e];
    }
#pragma unroll
    for (int r = 1; r < COLL_MAX_RANKS; r++) {
      if (r < R) {
        const float wr = s_w[q][r];
        typename F::Acc a = F::widen(v[r]);
#pragma unroll
        for (int e = 0; e < VL; e++) acc[e] = acc[e] + wr * a.v[e];
      }
    }
    typename F::Acc outv;
#pragma unroll
    for (int e = 0; e < VL; e++) outv.v[e] = empty ? 0.0f : acc[e];
    const u32x4 ov = F::narrow(outv);
#pragma unroll
    for (int r = 0; r < COLL_MAX_RANKS; r++)
      if (r < R) st<u32x4, NT>(o.out[r], x, ov);
  } else {
    float acc = s_w[q][0] * F::widen1(ve[0]);
    for (int r = 1; r < R; r++) acc = acc + s_w[q][r] * F::widen1(ve[r]);
    const E ov = F::narrow1(empty ? 0.0f : acc);
    for (int r = 0; r < R; r++) reinterpret_cast<E *>(o.out[r])[x] = ov;
  }
}

}  // namespace

int launch_lse_merge(const Launch &L, int R, const RankPtrs &o, const PtrTable &lse_in,
                     const MutPtrTable &lse_out, size_t rows, size_t D, int dt) {
  const int VL = dt == COLL_BF16 ? 8 : 4;
  bool vec = (D % VL) == 0;
  for (int r = 0; r < R; r++) vec = vec && aligned16(o.in[r]) && aligned16(o.out[r]);
  const size_t es = dtype_size(dt);
  const bool nt = 2 * (uint64_t)R * rows * D * es >= L.nt_bytes;
  const uint64_t upr = vec ? D / VL : D;
  if (upr >= (1ull << 31)) return COLL_ERR_UNSUPPORTED;
  uint32_t rw = 1, nseg = 1;
  uint64_t groups;
  if (upr <= (uint64_t)kMergeLanes) {
    rw = (uint32_t)(kMergeLanes / upr);
    groups = (rows + rw - 1) / rw;
  } else {
    nseg = (uint32_t)((upr + kMergeLanes - 1) / kMergeLanes);
    groups = (uint64_t)rows * nseg;
  }
  if (groups > 0x7FFFFFFFull || (nseg > 1 && rows > 0xFFFFFFFFull)) return COLL_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)groups);
#define COLL_MERGE(DTV, VECV, NTV)                                                           \
  hipLaunchKernelGGL((lse_merge_rows<DTV, VECV, NTV>), grid, dim3(kMergeLanes), 0, L.stream, o, \
                     lse_in, lse_out, R, (uint64_t)rows, (uint32_t)upr, rw, nseg)
  if (dt == COLL_BF16) {
    if (vec && nt) COLL_MERGE(COLL_BF16, true, true);
    else if (vec) COLL_MERGE(COLL_BF16, true, false);
    else COLL_MERGE(COLL_BF16, false, false);
  } else {
    if (vec && nt) COLL_MERGE(COLL_FP32, true, true);
    else if (vec) COLL_MERGE(COLL_FP32, true, false);
    else COLL_MERGE(COLL_FP32, false, false);
  }
#undef COLL_MERGE
  return hip_status();
}

}  // namespace coll
