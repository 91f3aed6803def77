// moe.hip -- MoE dispatch / combine helpers around All-to-All-v (tutorial
// section 8.4, "MoE Dispatch / Combine"): tokens go to the rank that owns
// their expert, the experts run there, and the results return to the token's
// owner to be gate-weighted and summed.
//
// Layout (three small launches, integer only, deterministic):
//   1. moe_hist   one workgroup per (source, 1024-id tile): LDS histogram of
//                 expert ids -> per-tile counts in the workspace.
//   2. moe_scan   one 1024-thread workgroup per source: per expert, an
//                 exclusive scan over tiles (tile offsets); then a block-wide
//                 exclusive scan over experts built from wave64 shuffle scans
//                 -> expert offsets, expert counts, send counts, send displs.
//   3. moe_pos    one workgroup per (source, tile): the stable slot of every
//                 (t, k) = expert offset + tile offset + rank within the tile.
//                 The rank within a wave64 comes from matching lanes with equal
//                 ids (one ballot per id bit) and a popcount below the lane;
//                 earlier waves of the tile are added through LDS counters, so
//                 the order is exactly (expert, t, k).  Block (0, 0) also
//                 writes the receive displacements (a scan over sources).
// Data movement:
//   moe_permute   send[s][pos[t,k]] = x[s][t]: each token row is read once and
//                 written topk times, 16-byte units.
//   moe_expert_scale  the harness's test expert y = rne(x * (1 + e/256)), in
//                 place, one wave per received row.
//   moe_combine   one wave per token: topk rows gathered by pos, fp32
//                 fold k = 0..K-1 of separately rounded products, one RNE.
#include "coll_internal.h"

#pragma clang fp contract(off)

namespace coll {

constexpr int kMoeTile = 1024;        // ids per layout tile (kBlock * 4)
constexpr int kMaxExperts = kMoeMaxExperts;

size_t moe_workspace_bytes(int R, int T, int K, int E) {
  size_t tk = (size_t)T * K;
  size_t ntiles = (tk + kMoeTile - 1) / kMoeTile;
  size_t ints = (size_t)R * ntiles * E + (size_t)R * E;
  return (ints * 4 + 255) & ~(size_t)255;
}

namespace {

__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// ------------------------------------------------------------------ layout

__global__ __launch_bounds__(kBlock) void moe_hist(PtrTable ids, int TK, int E, int ntiles,
                                                   int32_t *hist) {
  __shared__ int h[kMaxExperts];
  const int s = blockIdx.y, tile = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kBlock) h[e] = 0;
  __syncthreads();
  const int32_t *id = reinterpret_cast<const int32_t *>(ids.p[s]);
#pragma unroll
  for (int j = 0; j < kMoeTile / kBlock; j++) {
    int i = tile * kMoeTile + j * kBlock + threadIdx.x;
    if (i < TK) {
      const int e = id[i];
      if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);   // out-of-range ids are dropped
    }
  }
  __syncthreads();
  int32_t *out = hist + ((size_t)s * ntiles + tile) * E;
  for (int e = threadIdx.x; e < E; e += kBlock) out[e] = h[e];
}

// blockDim = 1024 (one thread per expert, E <= 1024), grid = R.
__global__ __launch_bounds__(1024) void moe_scan(int R, int E, int ntiles, int TK,
                                                 int32_t *hist, int32_t *expert_off,
                                                 int32_t *expert_counts, int64_t *sendcounts,
                                                 int64_t *sdispls) {
  __shared__ int wave_tot[16];
  __shared__ int off[kMaxExperts + 1];
  const int s = blockIdx.x, e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    int32_t *h = hist + (size_t)s * ntiles * E + e;
    for (int t = 0; t < ntiles; t++) {
      int c = h[(size_t)t * E];
      h[(size_t)t * E] = cnt;           // tile offset within the expert
      cnt += c;
    }
  }
  // block-wide exclusive scan of cnt over experts
  int incl = wave_incl_scan_i32(cnt);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 63) wave_tot[w] = incl;
  __syncthreads();
  if (w == 0) {
    int t = lane < 16 ? wave_tot[lane] : 0;
    int ti = wave_incl_scan_i32(t);
    if (lane < 16) wave_tot[lane] = ti - t;   // exclusive over waves
  }
  __syncthreads();
  int excl = wave_tot[w] + incl - cnt;
  if (e < E) {
    off[e] = excl;
    expert_off[(size_t)s * E + e] = excl;
    expert_counts[(size_t)s * E + e] = cnt;
  }
  if (e == 0) off[E] = TK;
  __syncthreads();
  if (e < R) {
    const int per = E / R;
    sendcounts[s * R + e] = off[(e + 1) * per] - off[e * per];
    sdispls[s * R + e] = off[e * per];
  }
}

__global__ __launch_bounds__(kBlock) void moe_pos(PtrTable ids, MutPtrTable pos, int R, int TK,
                                                  int E, int nbits, int ntiles,
                                                  const int32_t *hist, const int32_t *expert_off,
                                                  const int64_t *sendcounts, int64_t *rdispls) {
  __shared__ int base[kMaxExperts];
  __shared__ int run[kMaxExperts];
  __shared__ int wcnt[kBlock / 64][kMaxExperts];
  const int s = blockIdx.y, tile = blockIdx.x;
  if (s == 0 && tile == 0) {
    // receive displacements: rdispls[d][s'] = sum_{s'' < s'} sendcounts[s''][d]
    for (int t = threadIdx.x; t < R * R; t += kBlock) {
      int d = t / R, s2 = t - d * R;
      int64_t acc = 0;
      for (int q = 0; q < s2; q++) acc += sendcounts[q * R + d];
      rdispls[d * R + s2] = acc;
    }
  }
  if (tile >= ntiles) return;                  // no ids at all: displacements only
  const int32_t *h = hist + ((size_t)s * ntiles + tile) * E;
  for (int e = threadIdx.x; e < E; e += kBlock) {
    base[e] = expert_off[(size_t)s * E + e] + h[e];
    run[e] = 0;
  }
  const int32_t *id = reinterpret_cast<const int32_t *>(ids.p[s]);
  int32_t *out = reinterpret_cast<int32_t *>(pos.p[s]);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int round = 0; round < kMoeTile / kBlock; round++) {
    for (int x = threadIdx.x; x < E; x += kBlock)
#pragma unroll
      for (int q = 0; q < kBlock / 64; q++) wcnt[q][x] = 0;
    __syncthreads();
    const int i = tile * kMoeTile + round * kBlock + threadIdx.x;
    const int raw = i < TK ? id[i] : -1;
    const bool valid = (unsigned)raw < (unsigned)E;   // out-of-range ids get no slot
    const int e = valid ? raw : 0;
    uint64_t mask = __ballot(valid);
    for (int b = 0; b < nbits; b++) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      mask &= bit ? bal : ~bal;
    }
    const int rank = __popcll(mask & below);
    if (valid && rank == 0) wcnt[w][e] = __popcll(mask);
    __syncthreads();
    if (valid) {
      int before = 0;
      for (int q = 0; q < w; q++) before += wcnt[q][e];
      out[i] = base[e] + run[e] + before + rank;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < E; x += kBlock) {
      int sum = 0;
#pragma unroll
      for (int q = 0; q < kBlock / 64; q++) sum += wcnt[q][x];
      run[x] += sum;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ permute

template <int B> struct MUnit;
template <> struct MUnit<16> { typedef u32x4 T; };
template <> struct MUnit<8> { typedef u32x2 T; };
template <> struct MUnit<4> { typedef uint32_t T; };
template <> struct MUnit<2> { typedef uint16_t T; };
template <> struct MUnit<1> { typedef uint8_t T; };

template <int B>
__global__ __launch_bounds__(kBlock) void moe_permute_kernel(PtrTable x, PtrTable pos,
                                                             MutPtrTable send, uint32_t total,
                                                             FastDiv upr, int K, uint32_t TK) {
  using U = typename MUnit<B>::T;
  const int s = blockIdx.y;
  const U *src = reinterpret_cast<const U *>(x.p[s]);
  const int32_t *ps = reinterpret_cast<const int32_t *>(pos.p[s]);
  U *dst = reinterpret_cast<U *>(send.p[s]);
  const uint32_t stride = gridDim.x * kBlock;
  for (uint32_t j = blockIdx.x * kBlock + threadIdx.x; j < total; j += stride) {
    const uint32_t t = fdiv(j, upr);
    const uint32_t v = j - t * upr.d;
    const U val = src[j];
    const int32_t *pk = ps + (size_t)t * K;
    for (int k = 0; k < K; k++) {
      const int32_t slot = pk[k];
      if ((uint32_t)slot < TK) dst[(size_t)slot * upr.d + v] = val;   // never write outside
    }
  }
}

// ------------------------------------------------------------- test expert

// G = bf16 elements per unit (8: 16-byte vectors; 1: scalar fallback)
template <int G>
__global__ __launch_bounds__(kBlock) void moe_expert_scale_kernel(MutPtrTable recv, int R, int E,
                                                                  const int32_t *expert_counts,
                                                                  const int64_t *rdispls,
                                                                  uint32_t upr) {
  __shared__ uint32_t s_end[kMaxExperts];     // inclusive end (rows) of entry j
  __shared__ int64_t s_base[kMaxExperts];     // receive row = s_base[j] + global row
  const int d = blockIdx.y;
  const int per = E / R;
  // Wave 0: entries j = s*per + el in receive order (source, then expert)
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int chunk = (E + 63) / 64;           // entries per lane (<= 16)
    int local = 0;
    for (int c = 0; c < chunk; c++) {
      int j = lane * chunk + c;
      if (j < E) {
        int s = j / per, el = j - s * per;
        local += expert_counts[(size_t)s * E + d * per + el];
      }
    }
    int incl = wave_incl_scan_i32(local);
    int start = incl - local;
    for (int c = 0; c < chunk; c++) {
      int j = lane * chunk + c;
      if (j < E) {
        int s = j / per, el = j - s * per;
        start += expert_counts[(size_t)s * E + d * per + el];
        s_end[j] = start;
      }
    }
  }
  __syncthreads();
  // s_base needs the global start of each source's first entry
  for (int j = threadIdx.x; j < E; j += kBlock) {
    int s = j / per;
    int first = s * per;
    uint32_t gstart = first == 0 ? 0u : s_end[first - 1];
    s_base[j] = rdispls[d * R + s] - (int64_t)gstart;
  }
  __syncthreads();

  const uint32_t nrows = s_end[E - 1];
  int top = 1;
  while (top * 2 <= E) top *= 2;
  const int lane = threadIdx.x & 63;
  const uint32_t nwaves = gridDim.x * (kBlock / 64);
  uint16_t *y = reinterpret_cast<uint16_t *>(recv.p[d]);
  for (uint32_t g = blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6); g < nrows; g += nwaves) {
    int lo = 0;
    for (int step = top; step > 0; step >>= 1) {
      int c = lo + step;
      if (c <= E && s_end[c - 1] <= g) lo = c;
    }
    const int e = d * per + (lo - (lo / per) * per);
    const float scale = 1.0f + (float)e / 256.0f;
    const size_t row = (size_t)(s_base[lo] + g);
    if constexpr (G == 8) {
      u32x4 *p = reinterpret_cast<u32x4 *>(y + row * upr * 8);
      for (uint32_t u = lane; u < upr; u += 64) {
        u32x4 v = p[u];
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; q++)
          o[q] = pack_bf16(bf16_lo(v[q]) * scale, bf16_hi(v[q]) * scale);
        p[u] = o;
      }
    } else {
      uint16_t *p = y + row * upr;
      for (uint32_t u = lane; u < upr; u += 64)
        p[u] = (uint16_t)(pack_bf16(bf16_lo(p[u]) * scale, 0.0f) & 0xFFFFu);
    }
  }
}

// ------------------------------------------------------------------ combine

// A slot outside [0, T*K) (a caller error) reads row 0 instead of memory
// outside the buffer.
__device__ __forceinline__ uint32_t slot_of(int32_t p, uint32_t TK) {
  return (uint32_t)p < TK ? (uint32_t)p : 0u;
}

template <int G>
__global__ __launch_bounds__(kBlock) void moe_combine_kernel(PtrTable back, PtrTable pos,
                                                             PtrTable wts, MutPtrTable out,
                                                             int T, int K, uint32_t upr) {
  const uint32_t TK = (uint32_t)T * (uint32_t)K;
  constexpr int kChunk = 8;                    // gathered rows in flight per lane
  const int s = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const uint16_t *bk = reinterpret_cast<const uint16_t *>(back.p[s]);
  const int32_t *ps = reinterpret_cast<const int32_t *>(pos.p[s]);
  const float *ws = reinterpret_cast<const float *>(wts.p[s]);
  uint16_t *o = reinterpret_cast<uint16_t *>(out.p[s]);
  const int nwaves = gridDim.x * (kBlock / 64);
  for (int t = blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6); t < T; t += nwaves) {
    const int tu = __builtin_amdgcn_readfirstlane(t);
    const int32_t *pk = ps + (size_t)tu * K;
    const float *wk = ws + (size_t)tu * K;
    for (uint32_t u = lane; u < upr; u += 64) {
      if constexpr (G == 8) {
        float acc[8];
        for (int k0 = 0; k0 < K; k0 += kChunk) {
          u32x4 v[kChunk];
#pragma unroll
          for (int c = 0; c < kChunk; c++)
            if (k0 + c < K)
              v[c] = reinterpret_cast<const u32x4 *>(bk + (size_t)slot_of(pk[k0 + c], TK) * upr * 8)[u];
#pragma unroll
          for (int c = 0; c < kChunk; c++) {
            if (k0 + c < K) {
              const float wgt = wk[k0 + c];
#pragma unroll
              for (int q = 0; q < 4; q++) {
                float lo = wgt * bf16_lo(v[c][q]);
                float hi = wgt * bf16_hi(v[c][q]);
                if (k0 + c == 0) { acc[2 * q] = lo; acc[2 * q + 1] = hi; }
                else { acc[2 * q] = acc[2 * q] + lo; acc[2 * q + 1] = acc[2 * q + 1] + hi; }
              }
            }
          }
        }
        u32x4 r;
#pragma unroll
        for (int q = 0; q < 4; q++) r[q] = pack_bf16(acc[2 * q], acc[2 * q + 1]);
        reinterpret_cast<u32x4 *>(o + (size_t)tu * upr * 8)[u] = r;
      } else {
        float acc = 0.0f;
        for (int k = 0; k < K; k++) {
          float prod = wk[k] * bf16_lo(bk[(size_t)slot_of(pk[k], TK) * upr + u]);
          acc = (k == 0) ? prod : acc + prod;
        }
        o[(size_t)tu * upr + u] = (uint16_t)(pack_bf16(acc, 0.0f) & 0xFFFFu);
      }
    }
  }
}

}  // namespace

// ------------------------------------------------------------------ launchers

int launch_moe_layout(const Launch &L, int R, const PtrTable &ids, int T, int K, int E,
                      int64_t *sendcounts, int64_t *sdispls, int64_t *rdispls,
                      int32_t *expert_counts, const MutPtrTable &pos, void *ws) {
  const int TK = T * K;
  const int ntiles = (TK + kMoeTile - 1) / kMoeTile;
  int32_t *hist = reinterpret_cast<int32_t *>(ws);
  int32_t *expert_off = hist + (size_t)R * ntiles * E;
  int nbits = 0;
  while ((1 << nbits) < E) nbits++;
  if (ntiles > 0)
    hipLaunchKernelGGL(moe_hist, dim3(ntiles, R), dim3(kBlock), 0, L.stream, ids, TK, E, ntiles,
                       hist);
  hipLaunchKernelGGL(moe_scan, dim3(R), dim3(1024), 0, L.stream, R, E, ntiles, TK, hist,
                     expert_off, expert_counts, sendcounts, sdispls);
  hipLaunchKernelGGL(moe_pos, dim3(ntiles > 0 ? ntiles : 1, R), dim3(kBlock), 0, L.stream, ids,
                     pos, R, TK, E, nbits, ntiles, hist, expert_off, sendcounts, rdispls);
  return hip_status();
}

int launch_moe_permute(const Launch &L, int R, const PtrTable &x, const PtrTable &pos, int T,
                       int K, size_t row_bytes, const MutPtrTable &send) {
  uintptr_t bits = row_bytes;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)x.p[r] | (uintptr_t)send.p[r];
  const int unit = copy_unit(bits);
  const size_t upr = row_bytes / unit;
  const size_t total = (size_t)T * upr;
  if (total >= (1ull << 31)) return COLL_ERR_UNSUPPORTED;
  if (total == 0) return COLL_OK;
  FastDiv f = make_fastdiv((uint32_t)upr);
  unsigned gx = (grid_for(L, total * R) + R - 1) / R;
  dim3 grid(gx, R);
  uint32_t t32 = (uint32_t)total;
  switch (unit) {
    case 16: hipLaunchKernelGGL(moe_permute_kernel<16>, grid, dim3(kBlock), 0, L.stream, x, pos, send, t32, f, K, (uint32_t)(T * K)); break;
    case 8: hipLaunchKernelGGL(moe_permute_kernel<8>, grid, dim3(kBlock), 0, L.stream, x, pos, send, t32, f, K, (uint32_t)(T * K)); break;
    case 4: hipLaunchKernelGGL(moe_permute_kernel<4>, grid, dim3(kBlock), 0, L.stream, x, pos, send, t32, f, K, (uint32_t)(T * K)); break;
    case 2: hipLaunchKernelGGL(moe_permute_kernel<2>, grid, dim3(kBlock), 0, L.stream, x, pos, send, t32, f, K, (uint32_t)(T * K)); break;
    default: hipLaunchKernelGGL(moe_permute_kernel<1>, grid, dim3(kBlock), 0, L.stream, x, pos, send, t32, f, K, (uint32_t)(T * K)); break;
  }
  return hip_status();
}

int launch_moe_expert_scale(const Launch &L, int R, const MutPtrTable &recv,
                            const int32_t *expert_counts, const int64_t *rdispls, int E,
                            size_t hidden) {
  bool vec = (hidden % 8) == 0;
  for (int r = 0; r < R; r++) vec = vec && aligned16(recv.p[r]);
  dim3 grid((unsigned)((L.num_cus * L.wgs_per_cu + R - 1) / R), R);
  if (vec)
    hipLaunchKernelGGL(moe_expert_scale_kernel<8>, grid, dim3(kBlock), 0, L.stream, recv, R, E,
                       expert_counts, rdispls, (uint32_t)(hidden / 8));
  else
    hipLaunchKernelGGL(moe_expert_scale_kernel<1>, grid, dim3(kBlock), 0, L.stream, recv, R, E,
                       expert_counts, rdispls, (uint32_t)hidden);
  return hip_status();
}

int launch_moe_combine(const Launch &L, int R, const PtrTable &back, const PtrTable &pos,
                       const PtrTable &w, int T, int K, size_t hidden, const MutPtrTable &out) {
  bool vec = (hidden % 8) == 0;
  for (int r = 0; r < R; r++) vec = vec && aligned16(back.p[r]) && aligned16(out.p[r]);
  unsigned gx = (unsigned)((T + 3) / 4);       // one wave per token
  unsigned cap = (unsigned)((L.num_cus * L.wgs_per_cu + R - 1) / R);
  if (gx > cap) gx = cap;
  if (gx == 0) return COLL_OK;
  dim3 grid(gx, R);
  if (vec)
    hipLaunchKernelGGL(moe_combine_kernel<8>, grid, dim3(kBlock), 0, L.stream, back, pos, w, out,
                       T, K, (uint32_t)(hidden / 8));
  else
    hipLaunchKernelGGL(moe_combine_kernel<1>, grid, dim3(kBlock), 0, L.stream, back, pos, w, out,
                       T, K, (uint32_t)hidden);
  return hip_status();
}

}  // namespace coll
