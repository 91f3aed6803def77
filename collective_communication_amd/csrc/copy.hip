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

template <int B> struct UnitT;
template <> struct UnitT<16> { typedef u32x4 T; };
template <> struct UnitT<8> { typedef u32x2 T; };
template <> struct UnitT<4> { typedef uint32_t T; };
template <> struct UnitT<2> { typedef uint16_t T; };
template <> struct UnitT<1> { typedef uint8_t T; };

// ---------------------------------------------------------------- AllGather
// blockIdx.y = source rank q.  The shard unit is loaded once and stored to
// every rank's slot q; a rank whose slot q IS the source (the in-place form
// send[q] == recv[q] + q*n) is skipped, so in place costs R-1 stores.
template <int B>
__global__ __launch_bounds__(kBlock) void ag_kernel(RankPtrs p, int R, size_t nunits, int nt) {
  using U = typename UnitT<B>::T;
  const int q = blockIdx.y;
  const void *src = p.in[q];
  const size_t stride = (size_t)gridDim.x * kBlock;
  for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < nunits; i += stride) {
    U v = ld<U>(src, i);
#pragma unroll 4
    for (int r = 0; r < R; r++) {
      U *dst = reinterpret_cast<U *>(p.out[r]) + (size_t)q * nunits;
      if (dst != src) st<U>(dst, i, v, nt);
    }
  }
}

// ------------------------------------------------------------------ Gather
// Flattened over the root's output in units: j -> (o, q, i) with two fast
// divisions; writes are sequential, reads are runs of `upr` units per rank.
template <int B>
__global__ __launch_bounds__(kBlock) void gather_kernel(RankPtrs p, void *out, uint32_t total,
                                                        FastDiv per_row, FastDiv upr, int nt) {
  using U = typename UnitT<B>::T;
  const uint32_t stride = gridDim.x * kBlock;
  for (uint32_t j = blockIdx.x * kBlock + threadIdx.x; j < total; j += stride) {
    uint32_t o = fdiv(j, per_row);
    uint32_t rem = j - o * per_row.d;
    uint32_t q = fdiv(rem, upr);
    uint32_t i = rem - q * upr.d;
    U v = ld<U>(p.in[q], (size_t)o * upr.d + i);
    st<U>(out, j, v, nt);
  }
}

// --------------------------------------------------------------- Broadcast
template <int B>
__global__ __launch_bounds__(kBlock) void bcast_kernel(const void *src, RankPtrs p, int R,
                                                       size_t nunits, int nt) {
  using U = typename UnitT<B>::T;
  const size_t stride = (size_t)gridDim.x * kBlock;
  for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < nunits; i += stride) {
    U v = ld<U>(src, i);
#pragma unroll 4
    for (int r = 0; r < R; r++)
      if (p.out[r] != nullptr && p.out[r] != src) st<U>(p.out[r], i, v, nt);
  }
}

}  // namespace

int launch_all_gather(const Launch &L, int R, const RankPtrs &p, size_t bytes) {
  uintptr_t bits = bytes;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)p.in[r] | (uintptr_t)p.out[r];
  int unit = copy_unit(bits);
  size_t nunits = bytes / unit;
  int nt = ((size_t)(R + 1) * R * bytes >= L.nt_bytes) ? 1 : 0;
  unsigned gx = (grid_for(L, nunits * R) + R - 1) / R;
  dim3 grid(gx, R);
  switch (unit) {
    case 16: hipLaunchKernelGGL(ag_kernel<16>, grid, dim3(kBlock), 0, L.stream, p, R, nunits, nt); break;
    case 8: hipLaunchKernelGGL(ag_kernel<8>, grid, dim3(kBlock), 0, L.stream, p, R, nunits, nt); break;
    case 4: hipLaunchKernelGGL(ag_kernel<4>, grid, dim3(kBlock), 0, L.stream, p, R, nunits, nt); break;
    case 2: hipLaunchKernelGGL(ag_kernel<2>, grid, dim3(kBlock), 0, L.stream, p, R, nunits, nt); break;
    default: hipLaunchKernelGGL(ag_kernel<1>, grid, dim3(kBlock), 0, L.stream, p, R, nunits, nt); break;
  }
  return hip_status();
}

int launch_gather(const Launch &L, int R, const RankPtrs &p, void *out, size_t outer,
                  size_t inner_bytes) {
  uintptr_t bits = inner_bytes | (uintptr_t)out;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)p.in[r];
  int unit = copy_unit(bits);
  size_t upr = inner_bytes / unit;              // units per rank per row
  size_t total = outer * R * upr;
  if (total >= (1ull << 31)) return COLL_ERR_UNSUPPORTED;   // 32-bit index space
  FastDiv f_row = make_fastdiv((uint32_t)(R * upr));
  FastDiv f_upr = make_fastdiv((uint32_t)upr);
  int nt = (2 * total * (size_t)unit >= L.nt_bytes) ? 1 : 0;
  dim3 grid(grid_for(L, total));
  uint32_t t = (uint32_t)total;
  switch (unit) {
    case 16: hipLaunchKernelGGL(gather_kernel<16>, grid, dim3(kBlock), 0, L.stream, p, out, t, f_row, f_upr, nt); break;
    case 8: hipLaunchKernelGGL(gather_kernel<8>, grid, dim3(kBlock), 0, L.stream, p, out, t, f_row, f_upr, nt); break;
    case 4: hipLaunchKernelGGL(gather_kernel<4>, grid, dim3(kBlock), 0, L.stream, p, out, t, f_row, f_upr, nt); break;
    case 2: hipLaunchKernelGGL(gather_kernel<2>, grid, dim3(kBlock), 0, L.stream, p, out, t, f_row, f_upr, nt); break;
    default: hipLaunchKernelGGL(gather_kernel<1>, grid, dim3(kBlock), 0, L.stream, p, out, t, f_row, f_upr, nt); break;
  }
  return hip_status();
}

int launch_broadcast(const Launch &L, int R, const void *src, const RankPtrs &p, size_t bytes) {
  uintptr_t bits = bytes | (uintptr_t)src;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)p.out[r];
  int unit = copy_unit(bits);
  size_t nunits = bytes / unit;
  int nt = ((size_t)(R + 1) * bytes >= L.nt_bytes) ? 1 : 0;
  dim3 grid(grid_for(L, nunits));
  switch (unit) {
    case 16: hipLaunchKernelGGL(bcast_kernel<16>, grid, dim3(kBlock), 0, L.stream, src, p, R, nunits, nt); break;
    case 8: hipLaunchKernelGGL(bcast_kernel<8>, grid, dim3(kBlock), 0, L.stream, src, p, R, nunits, nt); break;
    case 4: hipLaunchKernelGGL(bcast_kernel<4>, grid, dim3(kBlock), 0, L.stream, src, p, R, nunits, nt); break;
    case 2: hipLaunchKernelGGL(bcast_kernel<2>, grid, dim3(kBlock), 0, L.stream, src, p, R, nunits, nt); break;
    default: hipLaunchKernelGGL(bcast_kernel<1>, grid, dim3(kBlock), 0, L.stream, src, p, R, nunits, nt); break;
  }
  return hip_status();
}

}  // namespace coll
