// reduce.hip -- AllReduce and ReduceScatter kernels.
//
// AllReduce follows the owner-per-segment dataflow of the IPC AllReduce blog
// ("From NCCL Ring LL to PCIe IPC AllReduce", section "Pro5000 ?"): each
// segment is gathered from all R ranks by its owner, summed once, and the sum
// is sent back to all R ranks.  On one GPU the owner of a 16-byte tile is the
// lane that holds it: it issues the R loads back to back (R * 16 B in flight
// per lane), folds them in ascending rank order in fp32, narrows once (RNE)
// and issues R stores of the same register tile.  ReduceScatter is the first
// half of that (tutorial section 5): one store, to the owner only.
//
// Every output element has exactly one writer, which reads all of its inputs
// before writing, so AllReduce in place (recv[r] == send[r]) and the
// documented in-place ReduceScatter are race free.
#include "coll_internal.h"

#pragma clang fp contract(off)

namespace coll {
namespace {

// ---------------------------------------------------------------- AllReduce

// Tile shape of the R-way reductions (measured on MI355X, R = 8, 16-64 MiB
// per rank, rank buffers in rank arenas): both do best with one-wave
// workgroups and one 16-byte unit per lane per rank (8 loads in flight per
// lane, many small tiles).  ReduceScatter [8192, 4096] x 8: 100.4 us with
// 256 lanes x 2 units, 95.0 with 64 x 1 (Reduce of 8 x 64 MiB: 99.4 -> 94.0);
// 64 x 2 and 128 x 1 measured the same as 256 x 2.
#ifndef COLL_AR_BLOCK
#define COLL_AR_BLOCK 64
#endif
#ifndef COLL_AR_U_MID
#define COLL_AR_U_MID 1          // units per lane for 3 <= R <= 8
#endif
#ifndef COLL_RS_BLOCK
#define COLL_RS_BLOCK 64
#endif
#ifndef COLL_RS_U_MID
#define COLL_RS_U_MID 1
#endif
constexpr int kArBlock = COLL_AR_BLOCK;
constexpr int kRsBlock = COLL_RS_BLOCK;

template <int R>
constexpr int ar_u() { return R <= 2 ? 4 : (R <= 8 ? COLL_AR_U_MID : 1); }
template <int R>
constexpr int rs_u() { return R <= 2 ? 4 : (R <= 8 ? COLL_RS_U_MID : 1); }

// AllReduce staged through LDS (SUM, kArLdsMinR <= R <= 16): a workgroup of R
// waves owns a tile of 64*U units of every rank, and wave r streams rank r: it
// loads the tile of sendbufs[r] into LDS (U runs of 1 KiB per wave); after a
// barrier, one thread per unit folds the R ranks in ascending order and writes
// the narrowed sum back to LDS; after a second barrier, wave r stores the
// summed tile to recvbufs[r].  Per wave this is a copy-like stream (one
// source, one destination) instead of R loads and R stores whose stores all
// wait for the slowest load.  The tile is picked by size: on MI355X, R = 8
// bf16, median of back-to-back launches, 16 / 32 / 64 MiB per rank reach
// 69.7 / 71.5 / 75.0% of the HBM peak with U = 1 and 68.5 / 70.7 / 76.1% with
// U = 2 (U = 3: 65.3 / 67.3 / 71.3%); a single wave loading and storing all R
// ranks reached 70.3 / 70.5 / 71.9% on the access pattern alone in graph
// replay.  Every unit of a tile is read into LDS before any is stored, so
// in-place calls are safe.
#ifndef COLL_AR_LDS_MIN_R
#define COLL_AR_LDS_MIN_R 4
#endif
#ifndef COLL_AR_LDS_BIG_BYTES
#define COLL_AR_LDS_BIG_BYTES (48u << 20)
#endif
constexpr int kArLdsMinR = COLL_AR_LDS_MIN_R;
constexpr size_t kArLdsBigBytes = COLL_AR_LDS_BIG_BYTES;   // per rank: U = 2 from here

template <int R, int DT, int OP, bool NT, int U>
__global__ __launch_bounds__(64 * R) void ar_lds(RankPtrs p, size_t nvec) {
  using F = Fmt<DT>;
  constexpr int kTile = 64 * U;                   // units per rank per tile
  __shared__ u32x4 s_in[R][kTile];
  __shared__ u32x4 s_sum[kTile];
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // the wave's rank
  const int lane = threadIdx.x & 63;
  for (size_t t0 = (size_t)blockIdx.x * kTile; t0 < nvec; t0 += (size_t)gridDim.x * kTile) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const size_t i = t0 + (size_t)u * 64 + lane;
      if (i < nvec) s_in[w][u * 64 + lane] = ld<u32x4, NT>(p.in[w], i);
    }
    __syncthreads();
    if (threadIdx.x < kTile && t0 + threadIdx.x < nvec) {
      typename F::Acc a = F::widen(s_in[0][threadIdx.x]);
#pragma unroll
      for (int r = 1; r < R; r++) F::template fold_in<OP>(a, s_in[r][threadIdx.x]);
      s_sum[threadIdx.x] = F::narrow(a);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; u++) {
      const size_t i = t0 + (size_t)u * 64 + lane;
      if (i < nvec) st<u32x4, NT>(p.out[w], i, s_sum[u * 64 + lane]);
    }
    __syncthreads();                 // the next tile (if any) reuses the LDS
  }
}

// R known at compile time: all U * R loads of a tile issue back to back.
template <int R, int DT, int OP, bool NT>
__global__ __launch_bounds__(kArBlock) void ar_vec(RankPtrs p, size_t nvec) {
  using F = Fmt<DT>;
  constexpr int U = ar_u<R>();
  const size_t tile = (size_t)kArBlock * U;
  for (size_t base = (size_t)blockIdx.x * tile + threadIdx.x; base < nvec;
       base += (size_t)gridDim.x * tile) {
    u32x4 v[U][R];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const size_t i = base + (size_t)u * kArBlock;
      if (i < nvec) {
#pragma unroll
        for (int r = 0; r < R; r++) v[u][r] = ld<u32x4, NT>(p.in[r], i);
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const size_t i = base + (size_t)u * kArBlock;
      if (i < nvec) {
        typename F::Acc a = F::widen(v[u][0]);
#pragma unroll
        for (int r = 1; r < R; r++) F::template fold_in<OP>(a, v[u][r]);
        const u32x4 o = F::narrow(a);
#pragma unroll
        for (int r = 0; r < R; r++) st<u32x4, NT>(p.out[r], i, o);
      }
    }
  }
}

// Runtime R (ops other than SUM, unusual R): loads predicated on r < R.
template <int DT, int OP, bool NT>
__global__ __launch_bounds__(kBlock) void ar_vec_rt(RankPtrs p, int R, size_t nvec) {
  using F = Fmt<DT>;
  const size_t stride = (size_t)gridDim.x * kBlock;
  for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < nvec; i += stride) {
    u32x4 v[COLL_MAX_RANKS];
#pragma unroll
    for (int r = 0; r < COLL_MAX_RANKS; r++)
      if (r < R) v[r] = ld<u32x4, NT>(p.in[r], i);
    typename F::Acc a = F::widen(v[0]);
#pragma unroll
    for (int r = 1; r < COLL_MAX_RANKS; r++)
      if (r < R) F::template fold_in<OP>(a, v[r]);
    const u32x4 o = F::narrow(a);
#pragma unroll
    for (int r = 0; r < COLL_MAX_RANKS; r++)
      if (r < R) st<u32x4, NT>(p.out[r], i, o);
  }
}

// One element per thread, any alignment: tails and unaligned buffers.
template <int DT, int OP>
__device__ __forceinline__ typename Fmt<DT>::Elem reduce_one(const RankPtrs &p, int R, size_t i) {
  using F = Fmt<DT>;
  using E = typename F::Elem;
  if constexpr (DT == COLL_INT32) {
    int32_t acc = reinterpret_cast<const int32_t *>(p.in[0])[i];
    for (int r = 1; r < R; r++) acc = fold_i<OP>(acc, reinterpret_cast<const int32_t *>(p.in[r])[i]);
    return acc;
  } else {
    float acc = F::widen1(reinterpret_cast<const E *>(p.in[0])[i]);
    for (int r = 1; r < R; r++) acc = fold<OP>(acc, F::widen1(reinterpret_cast<const E *>(p.in[r])[i]));
    return F::narrow1(acc);
  }
}

// Elements [first, first + n) of every rank.
template <int DT, int OP>
__global__ __launch_bounds__(kBlock) void ar_scalar(RankPtrs p, int R, size_t first, size_t n) {
  using E = typename Fmt<DT>::Elem;
  const size_t stride = (size_t)gridDim.x * kBlock;
  for (size_t j = (size_t)blockIdx.x * kBlock + threadIdx.x; j < n; j += stride) {
    const size_t i = first + j;
    const E v = reduce_one<DT, OP>(p, R, i);
    for (int r = 0; r < R; r++) reinterpret_cast<E *>(p.out[r])[i] = v;
  }
}

// ------------------------------------------------------------ ReduceScatter

// blockIdx.y = owner rank r: out[r][i] = fold over q of in[q][r*seg + i].
// NTL / NTS: non-temporal loads / stores.  The output is 1/R of the input, so
// below a size threshold the sums are stored cacheable: a consumer that
// reads them next (the AllGather of sequence parallelism) finds them in the
// Infinity Cache.  On MI355X at R = 8 with 8 MiB outputs this took the
// ReduceScatter + AllGather pair from 225 to 200 us per step.
template <int R, int DT, int OP, bool NTL, bool NTS>
__global__ __launch_bounds__(kRsBlock) void rs_vec(RankPtrs p, size_t nvec_seg) {
  using F = Fmt<DT>;
  constexpr int U = rs_u<R>();
  const int r = blockIdx.y;
  const size_t off = (size_t)r * nvec_seg;
  const size_t tile = (size_t)kRsBlock * U;
  for (size_t base = (size_t)blockIdx.x * tile + threadIdx.x; base < nvec_seg;
       base += (size_t)gridDim.x * tile) {
    u32x4 v[U][R];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const size_t i = base + (size_t)u * kRsBlock;
      if (i < nvec_seg) {
#pragma unroll
        for (int q = 0; q < R; q++) v[u][q] = ld<u32x4, NTL>(p.in[q], off + i);
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const size_t i = base + (size_t)u * kRsBlock;
      if (i < nvec_seg) {
        typename F::Acc a = F::widen(v[u][0]);
#pragma unroll
        for (int q = 1; q < R; q++) F::template fold_in<OP>(a, v[u][q]);
        st<u32x4, NTS>(p.out[r], i, F::narrow(a));
      }
    }
  }
}

template <int DT, int OP, bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void rs_vec_rt(RankPtrs p, int R, size_t nvec_seg) {
  using F = Fmt<DT>;
  const int r = blockIdx.y;
  const size_t off = (size_t)r * nvec_seg;
  const size_t stride = (size_t)gridDim.x * kBlock;
  for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < nvec_seg; i += stride) {
    u32x4 v[COLL_MAX_RANKS];
#pragma unroll
    for (int q = 0; q < COLL_MAX_RANKS; q++)
      if (q < R) v[q] = ld<u32x4, NTL>(p.in[q], off + i);
    typename F::Acc a = F::widen(v[0]);
#pragma unroll
    for (int q = 1; q < COLL_MAX_RANKS; q++)
      if (q < R) F::template fold_in<OP>(a, v[q]);
    st<u32x4, NTS>(p.out[r], i, F::narrow(a));
  }
}

template <int DT, int OP>
__global__ __launch_bounds__(kBlock) void rs_scalar(RankPtrs p, int R, size_t seg) {
  const int r = blockIdx.y;
  const size_t stride = (size_t)gridDim.x * kBlock;
  for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < seg; i += stride)
    reinterpret_cast<typename Fmt<DT>::Elem *>(p.out[r])[i] = reduce_one<DT, OP>(p, R, (size_t)r * seg + i);
}

// ------------------------------------------------------------ dispatchers

template <int R, int DT, int OP, bool NT>
void launch_ar_r(const Launch &L, const RankPtrs &p, size_t nvec) {
  if constexpr (R >= kArLdsMinR) {
    if (nvec * sizeof(u32x4) >= kArLdsBigBytes) {
      dim3 grid(L.ar_grid > 0 ? (unsigned)L.ar_grid : grid_tiles(nvec, (size_t)128));
      hipLaunchKernelGGL((ar_lds<R, DT, OP, NT, 2>), grid, dim3(64 * R), 0, L.stream, p, nvec);
    } else {
      dim3 grid(L.ar_grid > 0 ? (unsigned)L.ar_grid : grid_tiles(nvec, (size_t)64));
      hipLaunchKernelGGL((ar_lds<R, DT, OP, NT, 1>), grid, dim3(64 * R), 0, L.stream, p, nvec);
    }
  } else {
    dim3 grid(L.ar_grid > 0 ? (unsigned)L.ar_grid
                            : grid_tiles(nvec, (size_t)ar_u<R>() * kArBlock));
    hipLaunchKernelGGL((ar_vec<R, DT, OP, NT>), grid, dim3(kArBlock), 0, L.stream, p, nvec);
  }
}

template <int DT, int OP, bool NT>
void ar_vec_dispatch(const Launch &L, int R, const RankPtrs &p, size_t nvec) {
  if constexpr (OP == COLL_SUM) {
    switch (R) {
      case 1: return launch_ar_r<1, DT, OP, NT>(L, p, nvec);
      case 2: return launch_ar_r<2, DT, OP, NT>(L, p, nvec);
      case 3: return launch_ar_r<3, DT, OP, NT>(L, p, nvec);
      case 4: return launch_ar_r<4, DT, OP, NT>(L, p, nvec);
      case 5: return launch_ar_r<5, DT, OP, NT>(L, p, nvec);
      case 6: return launch_ar_r<6, DT, OP, NT>(L, p, nvec);
      case 7: return launch_ar_r<7, DT, OP, NT>(L, p, nvec);
      case 8: return launch_ar_r<8, DT, OP, NT>(L, p, nvec);
      case 16: return launch_ar_r<16, DT, OP, NT>(L, p, nvec);
      default: break;
    }
  }
  hipLaunchKernelGGL((ar_vec_rt<DT, OP, NT>), dim3(grid_for(L, nvec)), dim3(kBlock), 0, L.stream,
                     p, R, nvec);
}

template <int DT, int OP>
int ar_dispatch(const Launch &L, int R, const RankPtrs &p, size_t count) {
  constexpr int VL = Fmt<DT>::kLanes;
  bool aligned = true;
  for (int r = 0; r < R; r++) aligned = aligned && aligned16(p.in[r]) && aligned16(p.out[r]);
  const size_t nvec = aligned ? count / VL : 0;
  const size_t tail0 = nvec * VL;
  const bool nt = 2 * (size_t)R * count * Fmt<DT>::kSize >= L.nt_bytes;
  if (nvec) {
    if (nt) ar_vec_dispatch<DT, OP, true>(L, R, p, nvec);
    else ar_vec_dispatch<DT, OP, false>(L, R, p, nvec);
  }
  if (count > tail0) {
    const size_t n = count - tail0;
    hipLaunchKernelGGL((ar_scalar<DT, OP>), dim3(grid_for(L, n)), dim3(kBlock), 0, L.stream,
                       p, R, tail0, n);
  }
  return hip_status();
}

template <int R, int DT, int OP, bool NTL, bool NTS>
void launch_rs_r(const Launch &L, const RankPtrs &p, size_t nvec, int nout) {
  dim3 grid(grid_tiles(nvec, (size_t)rs_u<R>() * kRsBlock), nout);
  hipLaunchKernelGGL((rs_vec<R, DT, OP, NTL, NTS>), grid, dim3(kRsBlock), 0, L.stream, p, nvec);
}

template <int DT, int OP, bool NTL, bool NTS>
void rs_vec_dispatch(const Launch &L, int R, const RankPtrs &p, size_t nvec, int nout) {
  if constexpr (OP == COLL_SUM) {
    switch (R) {
      case 1: return launch_rs_r<1, DT, OP, NTL, NTS>(L, p, nvec, nout);
      case 2: return launch_rs_r<2, DT, OP, NTL, NTS>(L, p, nvec, nout);
      case 3: return launch_rs_r<3, DT, OP, NTL, NTS>(L, p, nvec, nout);
      case 4: return launch_rs_r<4, DT, OP, NTL, NTS>(L, p, nvec, nout);
      case 5: return launch_rs_r<5, DT, OP, NTL, NTS>(L, p, nvec, nout);
      case 6: return launch_rs_r<6, DT, OP, NTL, NTS>(L, p, nvec, nout);
      case 7: return launch_rs_r<7, DT, OP, NTL, NTS>(L, p, nvec, nout);
      case 8: return launch_rs_r<8, DT, OP, NTL, NTS>(L, p, nvec, nout);
      case 16: return launch_rs_r<16, DT, OP, NTL, NTS>(L, p, nvec, nout);
      default: break;
    }
  }
  hipLaunchKernelGGL((rs_vec_rt<DT, OP, NTL, NTS>), dim3(grid_for(L, nvec), nout), dim3(kBlock), 0,
                     L.stream, p, R, nvec);
}

// nout = R: ReduceScatter (owner r = blockIdx.y writes chunk r);
// nout = 1: Reduce (one output, out[0], of the whole range: seg = count).
template <int DT, int OP>
int rs_dispatch(const Launch &L, int R, const RankPtrs &p, size_t seg, int nout) {
  constexpr int VL = Fmt<DT>::kLanes;
  bool aligned = (seg % VL) == 0;
  for (int r = 0; r < R; r++) aligned = aligned && aligned16(p.in[r]);
  for (int r = 0; r < nout; r++) aligned = aligned && aligned16(p.out[r]);
  const size_t written = (size_t)nout * seg * Fmt<DT>::kSize;
  const bool nt = (size_t)(R + 1) * written >= L.nt_bytes;
  const bool nts = nt && written >= L.nt_store_bytes;
  if (aligned) {
    const size_t nvec = seg / VL;
    if (nts) rs_vec_dispatch<DT, OP, true, true>(L, R, p, nvec, nout);
    else if (nt) rs_vec_dispatch<DT, OP, true, false>(L, R, p, nvec, nout);
    else rs_vec_dispatch<DT, OP, false, false>(L, R, p, nvec, nout);
  } else {
    hipLaunchKernelGGL((rs_scalar<DT, OP>), dim3(grid_for(L, seg), nout), dim3(kBlock), 0,
                       L.stream, p, R, seg);
  }
  return hip_status();
}

template <int DT>
int ar_by_op(const Launch &L, int R, const RankPtrs &p, size_t count, int op) {
  switch (op) {
    case COLL_SUM: return ar_dispatch<DT, COLL_SUM>(L, R, p, count);
    case COLL_PROD: return ar_dispatch<DT, COLL_PROD>(L, R, p, count);
    case COLL_MAX: return ar_dispatch<DT, COLL_MAX>(L, R, p, count);
    case COLL_MIN: return ar_dispatch<DT, COLL_MIN>(L, R, p, count);
  }
  return COLL_ERR_UNSUPPORTED;
}

template <int DT>
int rs_by_op(const Launch &L, int R, const RankPtrs &p, size_t seg, int op, int nout) {
  switch (op) {
    case COLL_SUM: return rs_dispatch<DT, COLL_SUM>(L, R, p, seg, nout);
    case COLL_PROD: return rs_dispatch<DT, COLL_PROD>(L, R, p, seg, nout);
    case COLL_MAX: return rs_dispatch<DT, COLL_MAX>(L, R, p, seg, nout);
    case COLL_MIN: return rs_dispatch<DT, COLL_MIN>(L, R, p, seg, nout);
  }
  return COLL_ERR_UNSUPPORTED;
}

}  // namespace

int launch_allreduce(const Launch &L, int R, const RankPtrs &p, size_t count, int dt, int op) {
  switch (dt) {
    case COLL_BF16: return ar_by_op<COLL_BF16>(L, R, p, count, op);
    case COLL_FP16: return ar_by_op<COLL_FP16>(L, R, p, count, op);
    case COLL_FP32: return ar_by_op<COLL_FP32>(L, R, p, count, op);
    case COLL_INT32: return ar_by_op<COLL_INT32>(L, R, p, count, op);
  }
  return COLL_ERR_UNSUPPORTED;
}

int launch_reduce_scatter(const Launch &L, int R, const RankPtrs &p, size_t seg, int dt, int op,
                          int nout) {
  switch (dt) {
    case COLL_BF16: return rs_by_op<COLL_BF16>(L, R, p, seg, op, nout);
    case COLL_FP16: return rs_by_op<COLL_FP16>(L, R, p, seg, op, nout);
    case COLL_FP32: return rs_by_op<COLL_FP32>(L, R, p, seg, op, nout);
    case COLL_INT32: return rs_by_op<COLL_INT32>(L, R, p, seg, op, nout);
  }
  return COLL_ERR_UNSUPPORTED;
}

}  // namespace coll
