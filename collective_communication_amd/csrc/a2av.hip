// a2av.hip -- All-to-All-v (tutorial sections 8.1-8.2): every (source s,
// destination d) pair moves its own block of rows, of a length known only on
// the device.
//
// Each block (s, d) is one contiguous run in s's send buffer and one in d's
// receive buffer, so the exchange is R*R memcpys of skewed sizes (MoE routing
// sends most rows to a few ranks).  Rather than one workgroup per pair, which
// would leave most compute units idle under skew, the work is split by
// position in the concatenation of all blocks: every workgroup first builds
// the table of block extents in LDS (a wavefront-level prefix scan over the
// R*R byte lengths), then walks a grid-stride loop over units of that global
// index space, finding each unit's block by binary search in LDS (cached from
// the previous unit, since consecutive units of a lane usually share it).
// Loads and stores are 16-byte and coalesced whenever the row size and the
// buffers allow it.
#include "coll_internal.h"

namespace coll {
namespace {

template <int B> struct AUnit;
template <> struct AUnit<16> { typedef u32x4 T; };
template <> struct AUnit<8> { typedef u32x2 T; };
template <> struct AUnit<4> { typedef uint32_t T; };
template <> struct AUnit<2> { typedef uint16_t T; };
template <> struct AUnit<1> { typedef uint8_t T; };

constexpr int kMaxBlocks = COLL_MAX_RANKS * COLL_MAX_RANKS;   // 256

// Inclusive prefix sum across one wave64 (Hillis-Steele over lanes).
__device__ __forceinline__ uint64_t wave_incl_scan(uint64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint64_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

template <int B>
__global__ __launch_bounds__(kBlock) void a2av_kernel(RankPtrs p, int R, const int64_t *counts,
                                                      const int64_t *sdispls,
                                                      const int64_t *rdispls, uint64_t row_units,
                                                      int nt) {
  using U = typename AUnit<B>::T;
  __shared__ uint64_t s_end[kMaxBlocks];   // inclusive end of block b in the global unit space
  __shared__ uint64_t s_src[kMaxBlocks];   // src unit address minus block start (in units)
  __shared__ uint64_t s_dst[kMaxBlocks];

  const int nb = R * R;
  // Wave 0 builds the table: lane l owns blocks 4l .. 4l+3 (nb <= 256).
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    uint64_t len[4];
    uint64_t local = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      int b = lane * 4 + j;
      len[j] = 0;
      if (b < nb) {
        int64_t c = counts[b];
        len[j] = c > 0 ? (uint64_t)c * row_units : 0;
      }
      local += len[j];
    }
    uint64_t incl = wave_incl_scan(local);
    uint64_t start = incl - local;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      int b = lane * 4 + j;
      if (b < nb) {
        int s = b / R, d = b - s * R;
        uint64_t so = (uint64_t)sdispls[b] * row_units;
        uint64_t ro = (uint64_t)rdispls[d * R + s] * row_units;
        s_src[b] = reinterpret_cast<uintptr_t>(p.in[s]) / B + so - start;
        s_dst[b] = reinterpret_cast<uintptr_t>(p.out[d]) / B + ro - start;
        start += len[j];
        s_end[b] = start;
      }
    }
  }
  __syncthreads();

  const uint64_t total = s_end[nb - 1];
  int top = 1;
  while (top * 2 <= nb) top *= 2;            // largest power of two <= nb
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  int b = 0;
  for (uint64_t v = (uint64_t)blockIdx.x * kBlock + threadIdx.x; v < total; v += stride) {
    if (v >= s_end[b] || (b > 0 && v < s_end[b - 1])) {
      // b = number of blocks that end at or before v
      int lo = 0;
      for (int step = top; step > 0; step >>= 1) {
        int c = lo + step;
        if (c <= nb && s_end[c - 1] <= v) lo = c;
      }
      b = lo;
    }
    const U *src = reinterpret_cast<const U *>((s_src[b] + v) * B);
    U *dst = reinterpret_cast<U *>((s_dst[b] + v) * B);
    U x = *src;
    if (nt) __builtin_nontemporal_store(x, dst);
    else *dst = x;
  }
}

}  // namespace

int launch_a2av(const Launch &L, int R, const RankPtrs &p, const int64_t *counts,
                const int64_t *sdispls, const int64_t *rdispls, size_t row_bytes) {
  uintptr_t bits = row_bytes;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)p.in[r] | (uintptr_t)p.out[r];
  int unit = copy_unit(bits);
  uint64_t row_units = row_bytes / unit;
  // The total is only known on the device: launch the resident grid and let
  // the grid-stride loop cover whatever the counts say.
  dim3 grid((unsigned)L.num_cus * L.wgs_per_cu);
  int nt = L.a2a_nt;
  switch (unit) {
    case 16: hipLaunchKernelGGL(a2av_kernel<16>, grid, dim3(kBlock), 0, L.stream, p, R, counts, sdispls, rdispls, row_units, nt); break;
    case 8: hipLaunchKernelGGL(a2av_kernel<8>, grid, dim3(kBlock), 0, L.stream, p, R, counts, sdispls, rdispls, row_units, nt); break;
    case 4: hipLaunchKernelGGL(a2av_kernel<4>, grid, dim3(kBlock), 0, L.stream, p, R, counts, sdispls, rdispls, row_units, nt); break;
    case 2: hipLaunchKernelGGL(a2av_kernel<2>, grid, dim3(kBlock), 0, L.stream, p, R, counts, sdispls, rdispls, row_units, nt); break;
    default: hipLaunchKernelGGL(a2av_kernel<1>, grid, dim3(kBlock), 0, L.stream, p, R, counts, sdispls, rdispls, row_units, nt); break;
  }
  return hip_status();
}

}  // namespace coll
