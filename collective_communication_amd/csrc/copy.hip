// copy.hip -- the pure data-movement primitives: AllGather, Gather, Broadcast.
//
// All three read each source byte once and write it once per destination, in
// the widest unit (16 bytes when every pointer and size allows, else 8/4/2/1)
// with consecutive lanes on consecutive units, so both sides of every copy are
// fully coalesced.  Bytes are moved as they are: any dtype works.
//
//   AllGather  (tutorial section 7):  recv[r][q*n + i] = send[q][i]   for all r
//   Gather     (tutorial section 2, 2.2.1: logits concatenated along the vocab
//               axis on dst 0): root[o][q*inner + i] = send[q][o][i]
//   Broadcast  (tutorial section 1):  recv[r][i] = send_root[i]       for all r
#include "coll_internal.h"

namespace coll {
namespace {

// ---------------------------------------------------------------- AllGather
// blockIdx.y = source rank q.  A tile of the shard is loaded once and stored
// to every rank's slot q; a rank whose slot q IS the source (the in-place form
// send[q] == recv[q] + q*n) is skipped, so in place costs R-1 stores.
// AllGather tile: one wave, one 16-byte unit per lane (1 load, R stores);
// measured 3-4% above 256 lanes x 4 units at R = 8, 8 MiB shards (MI355X).
// The shard loads are always temporal (cacheable): each shard is read once
// and often was just written by the producer (a ReduceScatter), so it may
// still be in the Infinity Cache.  On MI355X at R = 8 they beat non-temporal
// loads both there (120 -> 114 us with 8 MiB shards) and cold (64 MiB shards,
// non-temporal stores: 890 vs 915 us); the R-fold stores stay non-temporal
// for large calls.
#ifndef COLL_AG_BLOCK
#define COLL_AG_BLOCK 64
#endif
#ifndef COLL_AG_U
#define COLL_AG_U 1
#endif
constexpr int kAgBlock = COLL_AG_BLOCK;
constexpr int kAgU = COLL_AG_U;

template <int B, bool NT>
__global__ __launch_bounds__(kAgBlock) void ag_kernel(RankPtrs p, int R, size_t nunits) {
  using U = typename UnitT<B>::T;
  constexpr int UN = kAgU;
  const int q = blockIdx.y;
  const void *src = p.in[q];
  const size_t tile = (size_t)kAgBlock * UN;
  for (size_t base = (size_t)blockIdx.x * tile + threadIdx.x; base < nunits;
       base += (size_t)gridDim.x * tile) {
    U v[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const size_t i = base + (size_t)u * kAgBlock;
      if (i < nunits) v[u] = ld<U, false>(src, i);
    }
    for (int r = 0; r < R; r++) {
      U *dst = reinterpret_cast<U *>(p.out[r]) + (size_t)q * nunits;
      if (dst == src) continue;
#pragma unroll
      for (int u = 0; u < UN; u++) {
        const size_t i = base + (size_t)u * kAgBlock;
        if (i < nunits) st<U, NT>(dst, i, v[u]);
      }
    }
  }
}

// ------------------------------------------------------------------ Gather
// Flattened over the root's output in units: j -> (o, q, i) with two fast
// divisions; writes are sequential, reads are runs of `upr` units per rank.
template <int B, bool NT>
__global__ __launch_bounds__(kGatherBlock) void gather_kernel(RankPtrs p, void *out, uint32_t total,
                                                        FastDiv per_row, FastDiv upr) {
  using U = typename UnitT<B>::T;
  constexpr int UN = kCopyU;
  const uint32_t tile = kGatherBlock * UN;
  for (uint32_t base = blockIdx.x * tile + threadIdx.x; base < total; base += gridDim.x * tile) {
    U v[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const uint32_t j = base + u * kGatherBlock;
      if (j < total) {
        const uint32_t o = fdiv(j, per_row);
        const uint32_t rem = j - o * per_row.d;
        const uint32_t q = fdiv(rem, upr);
        const uint32_t i = rem - q * upr.d;
        v[u] = ld<U, NT>(p.in[q], (size_t)o * upr.d + i);
      }
    }
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const uint32_t j = base + u * kGatherBlock;
      if (j < total) st<U, NT>(out, j, v[u]);
    }
  }
}

// The same with 64-bit indices, for outputs of 2^31 units (32 GiB with
// 16-byte units) and more.
template <int B, bool NT>
__global__ __launch_bounds__(kGatherBlock) void gather_kernel64(RankPtrs p, void *out, uint64_t total,
                                                          FastDiv64 per_row, FastDiv64 upr) {
  using U = typename UnitT<B>::T;
  constexpr int UN = kCopyU;
  const uint64_t tile = (uint64_t)kGatherBlock * UN;
  for (uint64_t base = (uint64_t)blockIdx.x * tile + threadIdx.x; base < total;
       base += (uint64_t)gridDim.x * tile) {
    U v[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const uint64_t j = base + (uint64_t)u * kGatherBlock;
      if (j < total) {
        const uint64_t o = fdiv64(j, per_row);
        const uint64_t rem = j - o * per_row.d;
        const uint64_t q = fdiv64(rem, upr);
        const uint64_t i = rem - q * upr.d;
        v[u] = ld<U, NT>(p.in[q], o * upr.d + i);
      }
    }
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const uint64_t j = base + (uint64_t)u * kGatherBlock;
      if (j < total) st<U, NT>(out, j, v[u]);
    }
  }
}

// --------------------------------------------------------------- Broadcast
template <int B, bool NT>
__global__ __launch_bounds__(kCopyBlock) void bcast_kernel(const void *src, RankPtrs p, int R,
                                                       size_t nunits) {
  using U = typename UnitT<B>::T;
  constexpr int UN = kCopyU;
  const size_t tile = (size_t)kCopyBlock * UN;
  for (size_t base = (size_t)blockIdx.x * tile + threadIdx.x; base < nunits;
       base += (size_t)gridDim.x * tile) {
    U v[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const size_t i = base + (size_t)u * kCopyBlock;
      if (i < nunits) v[u] = ld<U, NT>(src, i);
    }
    for (int r = 0; r < R; r++) {
      if (p.out[r] == nullptr || p.out[r] == src) continue;
#pragma unroll
      for (int u = 0; u < UN; u++) {
        const size_t i = base + (size_t)u * kCopyBlock;
        if (i < nunits) st<U, NT>(p.out[r], i, v[u]);
      }
    }
  }
}

// ----------------------------------------------------------------- Scatter
// blockIdx.y = destination rank r: out[r][i] = root[r*n + i] (tutorial 4).
// A rank whose buffer is its own chunk of the root buffer is skipped.
template <int B, bool NT>
__global__ __launch_bounds__(kCopyBlock) void scatter_kernel(const void *src, RankPtrs p,
                                                         size_t nunits) {
  using U = typename UnitT<B>::T;
  constexpr int UN = kCopyU;
  const int r = blockIdx.y;
  const U *s = reinterpret_cast<const U *>(src) + (size_t)r * nunits;
  void *dst = p.out[r];
  if (dst == nullptr || dst == (const void *)s) return;
  const size_t tile = (size_t)kCopyBlock * UN;
  for (size_t base = (size_t)blockIdx.x * tile + threadIdx.x; base < nunits;
       base += (size_t)gridDim.x * tile) {
    U v[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const size_t i = base + (size_t)u * kCopyBlock;
      if (i < nunits) v[u] = ld<U, NT>(s, i);
    }
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const size_t i = base + (size_t)u * kCopyBlock;
      if (i < nunits) st<U, NT>(dst, i, v[u]);
    }
  }
}

}  // namespace

int launch_scatter(const Launch &L, int R, const void *src, const RankPtrs &p, size_t bytes) {
  uintptr_t bits = bytes | (uintptr_t)src;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)p.out[r];
  const int unit = copy_unit(bits);
  const size_t nunits = bytes / unit;
  const bool nt = 2 * (size_t)R * bytes >= L.nt_bytes;
  dim3 grid(grid_tiles(nunits, (size_t)kCopyBlock * kCopyU), R);
  COLL_UNIT_SWITCH_BLOCK(scatter_kernel, unit, nt, grid, kCopyBlock, L.stream, src, p, nunits);
  return hip_status();
}

int launch_all_gather(const Launch &L, int R, const RankPtrs &p, size_t bytes) {
  uintptr_t bits = bytes;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)p.in[r] | (uintptr_t)p.out[r];
  const int unit = copy_unit(bits);
  const size_t nunits = bytes / unit;
  const bool nt = (size_t)(R + 1) * R * bytes >= L.nt_bytes;
  dim3 grid(grid_tiles(nunits, (size_t)kAgBlock * kAgU), R);
  COLL_UNIT_SWITCH_BLOCK(ag_kernel, unit, nt, grid, kAgBlock, L.stream, p, R, nunits);
  return hip_status();
}

int launch_gather(const Launch &L, int R, const RankPtrs &p, void *out, size_t outer,
                  size_t inner_bytes) {
  uintptr_t bits = inner_bytes | (uintptr_t)out;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)p.in[r];
  const int unit = copy_unit(bits);
  const size_t upr = inner_bytes / unit;            // units per rank per row
  const size_t total = outer * R * upr;
  const bool nt = 2 * total * (size_t)unit >= L.nt_bytes;
  dim3 grid(grid_tiles(total, (size_t)kGatherBlock * kCopyU));
  if (total < (1ull << 31)) {                        // 32-bit index space
    const FastDiv f_row = make_fastdiv((uint32_t)(R * upr));
    const FastDiv f_upr = make_fastdiv((uint32_t)upr);
    const uint32_t t = (uint32_t)total;
    COLL_UNIT_SWITCH_BLOCK(gather_kernel, unit, nt, grid, kGatherBlock, L.stream, p, out, t, f_row,
                           f_upr);
  } else {
    const FastDiv64 f_row = make_fastdiv64((uint64_t)R * upr);
    const FastDiv64 f_upr = make_fastdiv64(upr);
    COLL_UNIT_SWITCH_BLOCK(gather_kernel64, unit, nt, grid, kGatherBlock, L.stream, p, out,
                           (uint64_t)total, f_row, f_upr);
  }
  return hip_status();
}

int launch_broadcast(const Launch &L, int R, const void *src, const RankPtrs &p, size_t bytes) {
  uintptr_t bits = bytes | (uintptr_t)src;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)p.out[r];
  const int unit = copy_unit(bits);
  const size_t nunits = bytes / unit;
  const bool nt = (size_t)(R + 1) * bytes >= L.nt_bytes;
  dim3 grid(grid_tiles(nunits, (size_t)kCopyBlock * kCopyU));
  COLL_UNIT_SWITCH_BLOCK(bcast_kernel, unit, nt, grid, kCopyBlock, L.stream, src, p, R, nunits);
  return hip_status();
}

}  // namespace coll
