// merge.hip -- context-parallel merge of partial attention outputs
// ("Collective primitives tutorial", sections 5.4.2 and 7.4.3: the partial
// outputs of context-parallel attention cannot be summed as they are; the
// log-sum-exps are gathered first and the corrected contributions summed).
//
// Per (token, head) row with partial outputs o_r and log-sum-exps l_r:
//   m = max_r l_r, e_r = exp(l_r - m), s = sum_r e_r, L = m + log s,
//   o = sum_r (e_r / s) * o_r   (ranks ascending, fp32), delivered to every rank.
// On one GPU the LSE "AllGather" is a read: each 16-byte unit of a row reads
// the row's R LSEs (one cache line shared by the row's lanes), forms the
// weights in fp32, folds its R partial units and stores the result R times.
#include "coll_internal.h"

#pragma clang fp contract(off)

namespace coll {
namespace {

template <int DT>
__device__ __forceinline__ void row_weights(const PtrTable &lse, int R, uint64_t row,
                                            float *w, float *L) {
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

// Vector path: 16-byte units (8 bf16 or 4 fp32 per unit).
template <int DT, bool NT>
__global__ __launch_bounds__(kCopyBlock) void lse_merge_vec(RankPtrs o, PtrTable lse_in,
                                                        MutPtrTable lse_out, int R,
                                                        uint64_t total, FastDiv64 upr) {
  using F = Fmt<DT>;
  constexpr int VL = F::kLanes;
  const uint64_t stride = (uint64_t)gridDim.x * kCopyBlock;
  for (uint64_t x = (uint64_t)blockIdx.x * kCopyBlock + threadIdx.x; x < total; x += stride) {
    const uint64_t row = fdiv64(x, upr);
    const uint64_t j = x - row * upr.d;
    float w[COLL_MAX_RANKS], L;
    row_weights<DT>(lse_in, R, row, w, &L);
    u32x4 v[COLL_MAX_RANKS];
#pragma unroll
    for (int r = 0; r < COLL_MAX_RANKS; r++)
      if (r < R) v[r] = ld<u32x4, NT>(o.in[r], x);
    float acc[VL];
    {
      typename F::Acc a = F::widen(v[0]);
#pragma unroll
      for (int e = 0; e < VL; e++) acc[e] = w[0] * a.v[e];
    }
#pragma unroll
    for (int r = 1; r < COLL_MAX_RANKS; r++) {
      if (r < R) {
        typename F::Acc a = F::widen(v[r]);
#pragma unroll
        for (int e = 0; e < VL; e++) acc[e] = acc[e] + w[r] * a.v[e];
      }
    }
    typename F::Acc outv;
#pragma unroll
    for (int e = 0; e < VL; e++) outv.v[e] = acc[e];
    const u32x4 ov = F::narrow(outv);
#pragma unroll
    for (int r = 0; r < COLL_MAX_RANKS; r++)
      if (r < R) st<u32x4, NT>(o.out[r], x, ov);
    if (j == 0) {
      for (int r = 0; r < R; r++)
        if (lse_out.p[r]) reinterpret_cast<float *>(lse_out.p[r])[row] = L;
    }
  }
}

// Scalar path: one element per thread (head_dim not a multiple of the
// vector width, or unaligned buffers).
template <int DT>
__global__ __launch_bounds__(kCopyBlock) void lse_merge_scalar(RankPtrs o, PtrTable lse_in,
                                                           MutPtrTable lse_out, int R,
                                                           uint64_t total, FastDiv64 D) {
  using F = Fmt<DT>;
  using E = typename F::Elem;
  const uint64_t stride = (uint64_t)gridDim.x * kCopyBlock;
  for (uint64_t x = (uint64_t)blockIdx.x * kCopyBlock + threadIdx.x; x < total; x += stride) {
    const uint64_t row = fdiv64(x, D);
    const uint64_t c = x - row * D.d;
    float w[COLL_MAX_RANKS], L;
    row_weights<DT>(lse_in, R, row, w, &L);
    float acc = w[0] * F::widen1(reinterpret_cast<const E *>(o.in[0])[x]);
    for (int r = 1; r < R; r++) acc = acc + w[r] * F::widen1(reinterpret_cast<const E *>(o.in[r])[x]);
    const E ov = F::narrow1(acc);
    for (int r = 0; r < R; r++) reinterpret_cast<E *>(o.out[r])[x] = ov;
    if (c == 0) {
      for (int r = 0; r < R; r++)
        if (lse_out.p[r]) reinterpret_cast<float *>(lse_out.p[r])[row] = L;
    }
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
  if (vec) {
    const uint64_t upr = D / VL;
    const uint64_t total = (uint64_t)rows * upr;
    const FastDiv64 f = make_fastdiv64(upr);
    dim3 grid(grid_tiles(total, (size_t)kCopyBlock));
    if (dt == COLL_BF16) {
      if (nt) hipLaunchKernelGGL((lse_merge_vec<COLL_BF16, true>), grid, dim3(kCopyBlock), 0, L.stream, o, lse_in, lse_out, R, total, f);
      else hipLaunchKernelGGL((lse_merge_vec<COLL_BF16, false>), grid, dim3(kCopyBlock), 0, L.stream, o, lse_in, lse_out, R, total, f);
    } else {
      if (nt) hipLaunchKernelGGL((lse_merge_vec<COLL_FP32, true>), grid, dim3(kCopyBlock), 0, L.stream, o, lse_in, lse_out, R, total, f);
      else hipLaunchKernelGGL((lse_merge_vec<COLL_FP32, false>), grid, dim3(kCopyBlock), 0, L.stream, o, lse_in, lse_out, R, total, f);
    }
  } else {
    const uint64_t total = (uint64_t)rows * D;
    const FastDiv64 f = make_fastdiv64(D);
    dim3 grid(grid_tiles(total, (size_t)kCopyBlock));
    if (dt == COLL_BF16)
      hipLaunchKernelGGL((lse_merge_scalar<COLL_BF16>), grid, dim3(kCopyBlock), 0, L.stream, o, lse_in, lse_out, R, total, f);
    else
      hipLaunchKernelGGL((lse_merge_scalar<COLL_FP32>), grid, dim3(kCopyBlock), 0, L.stream, o, lse_in, lse_out, R, total, f);
  }
  return hip_status();
}

}  // namespace coll
