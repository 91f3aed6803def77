// exchange.hip -- the uniform all-to-all and the sequence <-> heads re-shard.
//
// all_to_all_single with equal splits (sglang PR 27492 digest; tutorial
// section 8.1): rank s's buffer is R chunks, chunk d for rank d; rank d
// receives them ordered by source.  The all-to-all sequence parallelism that
// motivates it re-shards attention inputs between "my sequence chunk, all
// heads" [SL, H, D] and "the whole sequence, my head group" [R*SL, H/R, D].
// Frameworks do that as a transpose into contiguous per-destination chunks
// followed by all_to_all_single; here one kernel gathers the strided chunks
// directly, so no packed copy exists.
//
// Both maps move rows of C = (H/R)*D elements between a source and a
// destination rank:
//   to_heads:  y_d[(s*SL + t)] <- x_s[t] chunk d    (row q = s*SL + t of y_d)
//   to_seq:    x_s[t] chunk d  <- y_d[(s*SL + t)]   (row q = t*R + d of x_s)
// The uniform all-to-all is to_heads with SL = 1.  In the output-major body
// blockIdx.y is the destination rank; its output is streamed in 16-byte units,
// one workgroup per tile, each unit finding its source row with two fast
// divisions.  to_heads with SL > 1 runs input-major instead (blockIdx.y the
// source rank), which on MI355X moves 8 ranks x 4096 tokens x 32 heads x 128
// bf16 at 78.7% of the HBM peak against 72.2% output-major.  The mirror
// image for to_seq (read each y_d in order, write 1 KiB pieces at a stride of
// R pieces) measured 62-68% against 76% output-major: there the strided side
// would be the writes, which cost more than strided reads.
#include "coll_internal.h"

namespace coll {
namespace {

template <int B, bool NT, bool TO_HEADS>
__device__ __forceinline__ void reshard_body(const RankPtrs &p, int R, uint64_t SL,
                                             uint64_t total, const FastDiv64 &cu,
                                             const FastDiv64 &div2) {
  using U = typename UnitT<B>::T;
  constexpr int UN = kCopyU;
  const int y = blockIdx.y;                       // destination rank
  void *dst = p.out[y];
  const uint64_t tile = (uint64_t)kCopyBlock * UN;
  for (uint64_t base = (uint64_t)blockIdx.x * tile + threadIdx.x; base < total;
       base += (uint64_t)gridDim.x * tile) {
    U v[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const uint64_t x = base + (uint64_t)u * kCopyBlock;
      if (x < total) {
        const uint64_t q = fdiv64(x, cu);          // destination row
        const uint64_t j = x - q * cu.d;            // unit within the row
        const uint64_t a = fdiv64(q, div2);
        const uint64_t b = q - a * div2.d;
        const void *src;
        uint64_t at;
        if constexpr (TO_HEADS) {                   // a = source s, b = t
          src = p.in[a];
          at = (b * (uint64_t)R + (uint64_t)y) * cu.d + j;
        } else {                                    // a = t, b = source d
          src = p.in[b];
          at = ((uint64_t)y * SL + a) * cu.d + j;
        }
        v[u] = ld<U, NT>(src, at);
      }
    }
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const uint64_t x = base + (uint64_t)u * kCopyBlock;
      if (x < total) st<U, NT>(dst, x, v[u]);
    }
  }
}

// to_heads, input-major: blockIdx.y is the SOURCE rank s and its input x_s
// ([SL, H, D], rows of R chunks) is read in order; unit x lies in input row
// q = t*R + d, chunk d of token t, and goes to row s*SL + t of y_d.  Reads are
// one contiguous stream per source, writes R streams, each contiguous over t.
// The output-major body above reads each token row in R separate pieces at R
// different times (one per destination pass), C elements each.
template <int B, bool NT>
__global__ __launch_bounds__(kCopyBlock) void to_heads_src_kernel(RankPtrs p, int R, uint64_t SL,
                                                              uint64_t total, FastDiv64 cu,
                                                              FastDiv64 rr) {
  using U = typename UnitT<B>::T;
  constexpr int UN = kCopyU;
  const int s = blockIdx.y;                       // source rank
  const void *src = p.in[s];
  const uint64_t tile = (uint64_t)kCopyBlock * UN;
  for (uint64_t base = (uint64_t)blockIdx.x * tile + threadIdx.x; base < total;
       base += (uint64_t)gridDim.x * tile) {
    U v[UN];
    void *dst[UN];
    uint64_t at[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const uint64_t x = base + (uint64_t)u * kCopyBlock;
      if (x < total) {
        v[u] = ld<U, NT>(src, x);
        const uint64_t q = fdiv64(x, cu);          // input row t*R + d
        const uint64_t j = x - q * cu.d;
        const uint64_t t = fdiv64(q, rr);
        const uint64_t d = q - t * rr.d;
        dst[u] = p.out[d];
        at[u] = ((uint64_t)s * SL + t) * cu.d + j;
      }
    }
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const uint64_t x = base + (uint64_t)u * kCopyBlock;
      if (x < total) st<U, NT>(dst[u], at[u], v[u]);
    }
  }
}

template <int B, bool NT>
__global__ __launch_bounds__(kCopyBlock) void to_heads_kernel(RankPtrs p, int R, uint64_t SL,
                                                          uint64_t total, FastDiv64 cu,
                                                          FastDiv64 sl) {
  reshard_body<B, NT, true>(p, R, SL, total, cu, sl);
}
template <int B, bool NT>
__global__ __launch_bounds__(kCopyBlock) void to_seq_kernel(RankPtrs p, int R, uint64_t SL,
                                                        uint64_t total, FastDiv64 cu,
                                                        FastDiv64 rr) {
  reshard_body<B, NT, false>(p, R, SL, total, cu, rr);
}

}  // namespace

// chunk_bytes = (H/R)*D*elem; seq_local rows per rank.
int launch_reshard(const Launch &L, int R, const RankPtrs &p, size_t seq_local,
                   size_t chunk_bytes, bool to_heads) {
  uintptr_t bits = chunk_bytes;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)p.in[r] | (uintptr_t)p.out[r];
  const int unit = copy_unit(bits);
  const uint64_t cu = chunk_bytes / unit;                 // units per row
  const uint64_t total = (uint64_t)R * seq_local * cu;    // units per destination
  if (total == 0) return COLL_OK;
  const FastDiv64 fcu = make_fastdiv64(cu);
  const bool nt = 2 * (uint64_t)R * total * unit >= L.nt_bytes;
  dim3 grid(grid_tiles(total, (size_t)kCopyBlock * kCopyU), R);
  if (to_heads && seq_local > 1) {
    const FastDiv64 fr = make_fastdiv64((uint64_t)R);
    COLL_UNIT_SWITCH_BLOCK(to_heads_src_kernel, unit, nt, grid, kCopyBlock, L.stream, p, R,
                           (uint64_t)seq_local, total, fcu, fr);
  } else if (to_heads) {
    const FastDiv64 fsl = make_fastdiv64(seq_local);
    COLL_UNIT_SWITCH_BLOCK(to_heads_kernel, unit, nt, grid, kCopyBlock, L.stream, p, R,
                           (uint64_t)seq_local, total, fcu, fsl);
  } else {
    const FastDiv64 fr = make_fastdiv64((uint64_t)R);
    COLL_UNIT_SWITCH_BLOCK(to_seq_kernel, unit, nt, grid, kCopyBlock, L.stream, p, R,
                           (uint64_t)seq_local, total, fcu, fr);
  }
  return hip_status();
}

}  // namespace coll
