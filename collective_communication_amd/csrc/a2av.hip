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

constexpr int kMaxBlocks = COLL_MAX_RANKS * COLL_MAX_RANKS;   // 256

// Count of block (s, d) -- the rows source s sends to destination d: entry
// s*R+d of the count table, or d*R+s when the tables are those of the forward
// exchange and this call is its reverse (ct = 1).  The displacements are read
// as sdispls[s*R+d] (source side) and rdispls[d*R+s] (destination side) in
// both cases: the reverse passes the forward rdispls as its sdispls and the
// forward sdispls as its rdispls.
__device__ __forceinline__ int count_index(int ct, int R, int s, int d) {
  return ct ? d * R + s : s * R + d;
}
#ifndef COLL_A2A_U
#define COLL_A2A_U 4
#endif
constexpr int kA2aU = COLL_A2A_U;             // units per lane per tile (one-pass grid)
#ifndef COLL_A2A_RES_U
#define COLL_A2A_RES_U 2
#endif
constexpr int kA2aResU = COLL_A2A_RES_U;      // ... resident grid
#ifndef COLL_A2A_BLOCK
#define COLL_A2A_BLOCK 256
#endif
// lanes per workgroup, one-pass grid (MI355X, the MoE exchange: 256 -> 1247 us,
// 128 -> 1275, 64 -> 1320: the workgroup shares one block-table build)
constexpr int kA2aBlock = COLL_A2A_BLOCK;
// receive capacity up to which the plain form runs a resident grid
#ifndef COLL_A2A_RESIDENT_MAX_BYTES
#define COLL_A2A_RESIDENT_MAX_BYTES (64ull << 20)
#endif
// 1: R <= 8 uses the one-block-per-lane table (a2av_kernel8 / a2av_res_kernel8)
#ifndef COLL_A2A_SMALL
#define COLL_A2A_SMALL 1
#endif
// Resident workgroups per CU of the chunk kernel (the 16-byte kernels keep 4).
// MI355X, R = 8, rows of one bf16, graph replay: 8 / 16 / 32 MiB per rank
// 26.1 / 48.6 / 92.9 us with 4, 25.7 / 47.6 / 91.4 with 5, 25.6 / 47.6 /
// 91.2 with 6, 25.4 / 48.2 / 91.7 with 7; with 8, 12 and 16 the 16 / 32 MiB
// launches took 54.6 / 105.7, 49.7 / 96.2 and 50.0 / 94.8 us.  The 16-byte
// resident kernel lost 4% with 6 (48.0 -> 50.1 us at 16 MiB).
#ifndef COLL_A2A_CHUNK_RES_PER_CU
#define COLL_A2A_CHUNK_RES_PER_CU 6
#endif
// 1: ... and the chunk kernel (rows not in 16-byte units) likewise.  MI355X,
// R = 8, rows of one bf16, graph replay: 8 KiB / 1 MiB / 16 / 64 MiB per
// rank 4.1 / 5.8 / 48.4 / 181.0 us against 5.1 / 6.9 / 49.4 / 184.4 us with
// four blocks per lane
#ifndef COLL_A2A_CHUNK_SMALL
#define COLL_A2A_CHUNK_SMALL 1
#endif

// 1: with at most 64 blocks, waves locate their units with one ballot over
// block ends held in registers (wave_block) instead of a per-lane search.
// MI355X, R = 8, graph replay: uniform 16-byte rows at 32 / 64 MiB per rank
// 91.3 -> 90.4 / 185.6 -> 183.6 us, MoE-shaped plain form (T = 1024 / 4096)
// 322 -> 318 / 1308 -> 1299 us; rows of one bf16 unchanged.  A lane still
// checks that its unit lies in the block so located (blocks are disjoint), so
// a wrong block could only cost a search, never an address.
#ifndef COLL_A2A_WAVE_LOCATE
#define COLL_A2A_WAVE_LOCATE 1
#endif

// The block holding a wave's 64 consecutive units x0 .. x0+63 (x0 the same in
// every lane, the whole wave active), for at most 64 blocks whose inclusive
// ends lane l holds in my_end (UINT64_MAX past the last block).  The ends do
// not decrease, so the blocks ending at or before x0 are a prefix and their
// count is the index of the block holding x0.  true when all 64 units lie in
// it -- every wave but those that straddle a block boundary, which search per
// lane.
__device__ __forceinline__ bool wave_block(uint64_t my_end, uint64_t x0, int &lo) {
  lo = (int)__popcll(__ballot(my_end <= x0));
  if (lo >= 64) return false;
  return x0 + 63 < readlane64(my_end, lo);
}

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


// One tile of a wave: UN units per lane, lane l taking units wbase + l +
// u * BS.  1. locate every unit (registers or LDS), 2. all loads, 3. all
// stores: with the lookups kept out from between the loads, the loads issue
// back to back (measured ~5% faster at the MoE shape).
//
// FULL: every unit lies inside the total, so no load or store sits in a
// branch.  With a bound check around each, the compiler cannot count the
// memory operations issued after a load and waits for all of them (vmcnt(0))
// before each store, so each store also waits for the one before it: one
// store of the wave in flight at a time.  The one-pass grid (4 units per
// lane) runs the whole tiles with FULL (the MoE exchange at 4096 tokens
// 71.8 -> 73.9% of HBM peak by graph replay, 8 x 64 MiB of 16-byte rows
// 74.6 -> 77.7%).  The resident grid (2 units per lane, looping over tiles)
// measured slower that way (8 x 32 MiB: 74.1 -> 72.6%, the MoE exchange at
// 256 tokens 74.0 -> 72.9%) and keeps the checked form, like the permute,
// whose fan-out also runs faster with one slot's stores in flight per wave.
template <int B, bool NT, int UN, int BS, bool FULL>
__device__ __forceinline__ void a2av_tile(uint64_t wbase, int lane, uint64_t total, int nb,
                                          int top, bool wl, uint64_t my_end, uint64_t my_src,
                                          uint64_t my_dst, const uint64_t *s_end,
                                          const uint64_t *s_src, const uint64_t *s_dst,
                                          uint64_t &blo, uint64_t &bhi, uint64_t &sbase,
                                          uint64_t &dbase) {
  using U = typename UnitT<B>::T;
  const uint64_t base = wbase + lane;
  uint64_t sa[UN], da[UN];
#pragma unroll
  for (int u = 0; u < UN; u++) {
    const uint64_t x = base + (uint64_t)u * BS;
    sa[u] = da[u] = 0;
    int wlo;
    if (wl && wave_block(my_end, wbase + (uint64_t)u * BS, wlo)) {
      blo = wlo > 0 ? readlane64(my_end, wlo - 1) : 0;
      bhi = readlane64(my_end, wlo);
      sbase = readlane64(my_src, wlo);
      dbase = readlane64(my_dst, wlo);
    }
    if (FULL || x < total) {
      if (x < blo || x >= bhi) {
        int lo = 0;                           // blocks ending at or before x
        for (int step = top; step > 0; step >>= 1) {
          const int c = lo + step;
          if (c <= nb && s_end[c - 1] <= x) lo = c;
        }
        blo = lo > 0 ? s_end[lo - 1] : 0;
        bhi = s_end[lo];
        sbase = s_src[lo];
        dbase = s_dst[lo];
      }
      sa[u] = (sbase + x) * B;
      da[u] = (dbase + x) * B;
    }
  }
  U v[UN];
#pragma unroll
  for (int u = 0; u < UN; u++) {
    if (FULL || base + (uint64_t)u * BS < total) {
      if constexpr (NT) v[u] = __builtin_nontemporal_load(gconst<U>(sa[u]));
      else v[u] = *gconst<U>(sa[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < UN; u++) {
    if (FULL || base + (uint64_t)u * BS < total) {
      if constexpr (NT) __builtin_nontemporal_store(v[u], gmut<U>(da[u]));
      else *gmut<U>(da[u]) = v[u];
    }
  }
}

// SMALL: R <= 8, so the R * R <= 64 blocks fit one per lane of wave 0 and the
// block search has a fixed depth (measured faster than the general form at
// the MoE exchange; the general form serves R up to 16).
template <int B, bool NT, int UN, int BS, bool SMALL, bool SPLIT>
__device__ __forceinline__ void a2av_body(const RankPtrs &p, const RowLimits &lim, int R,
                                          const int64_t *counts, const int64_t *sdispls,
                                          const int64_t *rdispls, int ct, uint64_t row_units) {
  using U = typename UnitT<B>::T;
  constexpr int kTab = SMALL ? 64 : kMaxBlocks;
  __shared__ uint64_t s_end[kTab];   // inclusive end of block b in the global unit space
  __shared__ uint64_t s_src[kTab];   // src unit address minus block start (in units)
  __shared__ uint64_t s_dst[kTab];

  const int nb = R * R;
  if constexpr (SMALL) {
    // Wave 0 builds the table, lane b owning block b; the three loads are
    // unconditional (clamped index) so they issue together
    if (threadIdx.x < 64) {
      const int b = threadIdx.x;
      const int bb = b < nb ? b : 0;
      const int s = bb / R, d = bb - s * R;
      const int64_t c = counts[count_index(ct, R, s, d)], sdv = sdispls[bb],
                    rdv = rdispls[d * R + s];
      const int64_t lin = rows_from_lane(lane_rows(lim.in), s);
      const int64_t lout = rows_from_lane(lane_rows(lim.out), d);
      const uint64_t len =
          (b < nb && block_fits(c, sdv, rdv, lin, lout)) ? (uint64_t)c * row_units : 0;
      const uint64_t incl = wave_incl_scan(len);
      if (b < nb) {
        const uint64_t start = incl - len;
        s_src[b] = reinterpret_cast<uintptr_t>(p.in[s]) / B + (uint64_t)sdv * row_units - start;
        s_dst[b] = reinterpret_cast<uintptr_t>(p.out[d]) / B + (uint64_t)rdv * row_units - start;
        s_end[b] = incl;
      }
    }
  } else
  // Wave 0 builds the table: lane l owns blocks 4l .. 4l+3 (nb <= 256).
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    uint64_t len[4];
    int64_t cnt[4], sdv[4], rdv[4];
    uint64_t local = 0;
    const int64_t my_in = lane_rows(lim.in), my_out = lane_rows(lim.out);
    // all three tables are loaded before the scan: one round trip to L2.  The
    // loads are unconditional (a lane past the last block reads block 0 and
    // discards it): a load under `if (b < nb)` made the compiler wait for it
    // inside the branch, one round trip per block of the lane.
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int b = lane * 4 + j;
      const int bb = b < nb ? b : 0;
      const int s = bb / R, d = bb - s * R;
      cnt[j] = counts[count_index(ct, R, s, d)];
      sdv[j] = sdispls[bb];
      rdv[j] = rdispls[d * R + s];
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int b = lane * 4 + j;
      const int bb = b < nb ? b : 0;
      const int s = bb / R, d = bb - s * R;
      const bool fits = block_fits(cnt[j], sdv[j], rdv[j], rows_from_lane(my_in, s),
                                   rows_from_lane(my_out, d));
      len[j] = (b < nb && fits) ? (uint64_t)cnt[j] * row_units : 0;
      local += len[j];
    }
    const uint64_t incl = wave_incl_scan(local);
    uint64_t start = incl - local;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int b = lane * 4 + j;
      if (b < nb) {
        const int s = b / R, d = b - s * R;
        const uint64_t so = (uint64_t)sdv[j] * row_units;
        const uint64_t ro = (uint64_t)rdv[j] * row_units;
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
  if constexpr (SMALL) top = 32;             // nb <= 64: six steps
  else
    while (top * 2 <= nb) top *= 2;          // largest power of two <= nb
  const uint64_t tile = (uint64_t)BS * UN;
  // at most 64 blocks: lane l keeps block l's end and bases in registers
  const int lane = threadIdx.x & 63;
  const bool wl = COLL_A2A_WAVE_LOCATE && nb <= 64;
  uint64_t my_end = ~0ull, my_src = 0, my_dst = 0;
  if (wl && lane < nb) {
    my_end = s_end[lane];
    my_src = s_src[lane];
    my_dst = s_dst[lane];
  }
  if constexpr (SPLIT) {
    // a tile whose 64 x UN units all lie inside the total takes the form with
    // no bound checks; the one that reaches the total takes the checked form
    // and ends the loop (a later tile of the wave lies past it).  The loop
    // runs while the wave's first unit is inside the total, so the wave stays
    // whole for its ballots.
    uint64_t blo = 1, bhi = 0, sbase = 0, dbase = 0;
    for (uint64_t wbase = (uint64_t)blockIdx.x * tile + (threadIdx.x - lane); wbase < total;
         wbase += (uint64_t)gridDim.x * tile) {
      if (wbase + 63 + (uint64_t)(UN - 1) * BS < total) {
        a2av_tile<B, NT, UN, BS, true>(wbase, lane, total, nb, top, wl, my_end, my_src, my_dst,
                                       s_end, s_src, s_dst, blo, bhi, sbase, dbase);
      } else {
        a2av_tile<B, NT, UN, BS, false>(wbase, lane, total, nb, top, wl, my_end, my_src,
                                        my_dst, s_end, s_src, s_dst, blo, bhi, sbase, dbase);
        break;
      }
    }
    return;
  }
  // The resident grid: every tile in the checked form, written out here
  // rather than through a2av_tile (the same steps), so that its instructions
  // stay those it was measured with; whole tiles without checks, and the
  // helper's slightly different code, measured slower on this grid.
  // The current block's bounds and address bases live in registers; LDS is
  // read only when a unit falls outside them.  The loop runs while the wave's
  // first unit is inside the total, so the wave stays whole for its ballots.
  uint64_t blo = 1, bhi = 0, sbase = 0, dbase = 0;
  for (uint64_t wbase = (uint64_t)blockIdx.x * tile + (threadIdx.x - lane); wbase < total;
       wbase += (uint64_t)gridDim.x * tile) {
    const uint64_t base = wbase + lane;
    // 1. locate every unit of the tile (registers or LDS), 2. all loads,
    // 3. all stores: with the lookups kept out from between the loads, the
    // loads issue back to back (measured ~5% faster at the MoE shape)
    uint64_t sa[UN], da[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const uint64_t x = base + (uint64_t)u * BS;
      sa[u] = da[u] = 0;
      int wlo;
      if (wl && wave_block(my_end, wbase + (uint64_t)u * BS, wlo)) {
        blo = wlo > 0 ? readlane64(my_end, wlo - 1) : 0;
        bhi = readlane64(my_end, wlo);
        sbase = readlane64(my_src, wlo);
        dbase = readlane64(my_dst, wlo);
      }
      if (x < total) {
        if (x < blo || x >= bhi) {
          int lo = 0;                           // blocks ending at or before x
          for (int step = top; step > 0; step >>= 1) {
            const int c = lo + step;
            if (c <= nb && s_end[c - 1] <= x) lo = c;
          }
          blo = lo > 0 ? s_end[lo - 1] : 0;
          bhi = s_end[lo];
          sbase = s_src[lo];
          dbase = s_dst[lo];
        }
        sa[u] = (sbase + x) * B;
        da[u] = (dbase + x) * B;
      }
    }
    U v[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
      if (base + (uint64_t)u * BS < total) {
        if constexpr (NT) v[u] = __builtin_nontemporal_load(gconst<U>(sa[u]));
        else v[u] = *gconst<U>(sa[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < UN; u++) {
      if (base + (uint64_t)u * BS < total) {
        if constexpr (NT) __builtin_nontemporal_store(v[u], gmut<U>(da[u]));
        else *gmut<U>(da[u]) = v[u];
      }
    }
  }
}

// One-pass grid (large exchanges): kA2aU units per lane per tile.
template <int B, bool NT>
__global__ __launch_bounds__(kA2aBlock) void a2av_kernel(RankPtrs p, RowLimits lim, int R, const int64_t *counts,
                                                      const int64_t *sdispls,
                                                      const int64_t *rdispls, int ct, uint64_t row_units) {
  a2av_body<B, NT, kA2aU, kA2aBlock, false, true>(p, lim, R, counts, sdispls, rdispls, ct, row_units);
}
template <int B, bool NT>
__global__ __launch_bounds__(kA2aBlock) void a2av_kernel8(RankPtrs p, RowLimits lim, int R, const int64_t *counts,
                                                       const int64_t *sdispls,
                                                       const int64_t *rdispls, int ct, uint64_t row_units) {
  a2av_body<B, NT, kA2aU, kA2aBlock, true, true>(p, lim, R, counts, sdispls, rdispls, ct, row_units);
}
// Resident grid (up to 64 MiB of capacity): kA2aResU units per lane per tile.
template <int B, bool NT>
__global__ __launch_bounds__(kBlock) void a2av_res_kernel(RankPtrs p, RowLimits lim, int R,
                                                          const int64_t *counts,
                                                          const int64_t *sdispls,
                                                          const int64_t *rdispls, int ct,
                                                          uint64_t row_units) {
  a2av_body<B, NT, kA2aResU, kBlock, false, false>(p, lim, R, counts, sdispls, rdispls, ct, row_units);
}
template <int B, bool NT>
__global__ __launch_bounds__(kBlock) void a2av_res_kernel8(RankPtrs p, RowLimits lim, int R,
                                                           const int64_t *counts,
                                                           const int64_t *sdispls,
                                                           const int64_t *rdispls, int ct,
                                                           uint64_t row_units) {
  a2av_body<B, NT, kA2aResU, kBlock, true, false>(p, lim, R, counts, sdispls, rdispls, ct, row_units);
}

// One tile of the chunk kernel's all-aligned path on the one-pass grid: UN
// 16-byte chunks per lane, located, loaded, then stored.  FULL: every chunk
// lies inside the total, so no load or store sits in a branch (a2av_tile).
template <bool NT, int UN, bool FULL>
__device__ __forceinline__ void chunk_vec_tile(uint64_t wbase, int lane, uint64_t total, int nb,
                                               int top, bool wl, uint64_t my_end,
                                               uint64_t my_src, uint64_t my_dst,
                                               const uint64_t *s_end, const uint64_t *s_src,
                                               const uint64_t *s_dst, uint64_t &blo,
                                               uint64_t &bhi, uint64_t &sbase, uint64_t &dbase) {
  const uint64_t base = wbase + lane;
  u32x4 v[UN];
  uint64_t da[UN];
#pragma unroll
  for (int u = 0; u < UN; u++) {
    const uint64_t x = base + (uint64_t)u * kBlock;
    int wlo;
    if (wl && wave_block(my_end, wbase + (uint64_t)u * kBlock, wlo)) {
      blo = wlo > 0 ? readlane64(my_end, wlo - 1) : 0;
      bhi = readlane64(my_end, wlo);
      sbase = readlane64(my_src, wlo) - blo * 16;
      dbase = readlane64(my_dst, wlo) - blo * 16;
    }
    if (FULL || x < total) {
      if (x < blo || x >= bhi) {
        int lo = 0;
        for (int step = top; step > 0; step >>= 1) {
          const int c = lo + step;
          if (c <= nb && s_end[c - 1] <= x) lo = c;
        }
        blo = lo > 0 ? s_end[lo - 1] : 0;
        bhi = s_end[lo];
        sbase = s_src[lo] - blo * 16;
        dbase = s_dst[lo] - blo * 16;
      }
      da[u] = dbase + x * 16;
      if constexpr (NT) v[u] = __builtin_nontemporal_load(gconst<u32x4>(sbase + x * 16));
      else v[u] = *gconst<u32x4>(sbase + x * 16);
    }
  }
#pragma unroll
  for (int u = 0; u < UN; u++) {
    const uint64_t x = base + (uint64_t)u * kBlock;
    if (FULL || x < total) {
      if constexpr (NT) __builtin_nontemporal_store(v[u], gmut<u32x4>(da[u]));
      else *gmut<u32x4>(da[u]) = v[u];
    }
  }
}

// Rows whose size or buffers do not allow 16-byte units on every row (the
// host only knows the row size): the index space is 16-byte chunks of each
// block, every block padded to whole chunks, so a chunk never spans two
// blocks.  A chunk whose source and destination are 16-byte aligned and that
// lies wholly inside its block moves as one 16-byte vector; any other chunk
// (a block's tail, or a block whose two ends are misaligned) moves in the
// widest unit that divides both addresses and its length.  With rows of one
// bf16 and equal counts every block is aligned, so this runs at vector speed.
// n (<= 16) bytes in units of T: all loads, then all stores.
template <class T>
__device__ __forceinline__ void copy_pieces(uint64_t src, uint64_t dst, uint32_t n) {
  constexpr int M = 16 / (int)sizeof(T);
  T t[M];
#pragma unroll
  for (int i = 0; i < M; i++)
    if ((uint32_t)(i * sizeof(T)) < n) t[i] = gconst<T>(src)[i];
#pragma unroll
  for (int i = 0; i < M; i++)
    if ((uint32_t)(i * sizeof(T)) < n) gmut<T>(dst)[i] = t[i];
}

__device__ __forceinline__ void copy_chunk_narrow(uint64_t src, uint64_t dst, uint32_t n) {
  const uint32_t a = (uint32_t)(src | dst) | n;
  if ((a & 7) == 0) copy_pieces<uint64_t>(src, dst, n);
  else if ((a & 3) == 0) copy_pieces<uint32_t>(src, dst, n);
  else if ((a & 1) == 0) copy_pieces<uint16_t>(src, dst, n);
  else copy_pieces<uint8_t>(src, dst, n);
}

// BPL: blocks per lane of the table-building wave: 4 (up to 256 blocks) or 1
// (R <= 8: smaller LDS tables, one load round of three words per lane)
template <bool NT, int UN, bool FAST, int BPL>
__global__ __launch_bounds__(kBlock) void a2av_chunk_kernel(RankPtrs p, RowLimits lim, int R,
                                                            const int64_t *counts,
                                                            const int64_t *sdispls,
                                                            const int64_t *rdispls, int ct,
                                                            uint64_t row_bytes) {
  constexpr int kTab = 64 * BPL;
  __shared__ uint64_t s_end[kTab];         // inclusive end of block b, in chunks
  __shared__ uint64_t s_src[kTab];         // source byte address of the block's chunk 0
  __shared__ uint64_t s_dst[kTab];
  __shared__ uint64_t s_len[kTab];         // block length in bytes
  __shared__ int s_allvec;                 // every block moves as whole 16-byte chunks

  const int nb = R * R;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    uint64_t len[BPL], nch[BPL];
    int64_t cnt[BPL], sdv[BPL], rdv[BPL];
    uint64_t local = 0;
    const int64_t my_in = lane_rows(lim.in), my_out = lane_rows(lim.out);
    bool misaligned = false;
    // unconditional loads (clamped index), then the bounds: one round trip
#pragma unroll
    for (int j = 0; j < BPL; j++) {
      const int b = lane * BPL + j;
      const int bb = b < nb ? b : 0;
      const int s = bb / R, d = bb - s * R;
      cnt[j] = counts[count_index(ct, R, s, d)];
      sdv[j] = sdispls[bb];
      rdv[j] = rdispls[d * R + s];
    }
#pragma unroll
    for (int j = 0; j < BPL; j++) {
      const int b = lane * BPL + j;
      const int bb = b < nb ? b : 0;
      const int s = bb / R, d = bb - s * R;
      const bool fits = block_fits(cnt[j], sdv[j], rdv[j], rows_from_lane(my_in, s),
                                   rows_from_lane(my_out, d));
      len[j] = (b < nb && fits) ? (uint64_t)cnt[j] * row_bytes : 0;
      nch[j] = (len[j] + 15) / 16;
      local += nch[j];
    }
    const uint64_t incl = wave_incl_scan(local);
    uint64_t start = incl - local;
#pragma unroll
    for (int j = 0; j < BPL; j++) {
      const int b = lane * BPL + j;
      if (b < nb) {
        const int s = b / R, d = b - s * R;
        s_src[b] = reinterpret_cast<uintptr_t>(p.in[s]) + (uint64_t)sdv[j] * row_bytes;
        s_dst[b] = reinterpret_cast<uintptr_t>(p.out[d]) + (uint64_t)rdv[j] * row_bytes;
        s_len[b] = len[j];
        start += nch[j];
        s_end[b] = start;
        if (len[j] && ((s_src[b] | s_dst[b] | len[j]) & 15)) misaligned = true;
      }
    }
    const uint64_t any_mis = __ballot(misaligned);
    if (lane == 0) s_allvec = any_mis == 0;
  }
  __syncthreads();

  if constexpr (!FAST) {
    if (s_allvec) {
      // The one-pass grid with every block aligned whole chunks: whole tiles
      // without bound checks, then the tile that reaches the total (as in
      // a2av_body's one-pass form).  The resident grid's loop below, with
      // its checks, measured 5% slower than the general loop here.
      const uint64_t total = s_end[nb - 1];
      int top = 1;
      while (top * 2 <= nb) top *= 2;
      const uint64_t tile = (uint64_t)kBlock * UN;
      const int lane = threadIdx.x & 63;
      const bool wl = COLL_A2A_WAVE_LOCATE && nb <= 64;
      uint64_t my_end = ~0ull, my_src = 0, my_dst = 0;
      if (wl && lane < nb) {
        my_end = s_end[lane];
        my_src = s_src[lane];
        my_dst = s_dst[lane];
      }
      uint64_t blo = 1, bhi = 0, sbase = 0, dbase = 0;
      for (uint64_t wbase = (uint64_t)blockIdx.x * tile + (threadIdx.x - lane); wbase < total;
           wbase += (uint64_t)gridDim.x * tile) {
        if (wbase + 63 + (uint64_t)(UN - 1) * kBlock < total) {
          chunk_vec_tile<NT, UN, true>(wbase, lane, total, nb, top, wl, my_end, my_src, my_dst,
                                       s_end, s_src, s_dst, blo, bhi, sbase, dbase);
        } else {
          chunk_vec_tile<NT, UN, false>(wbase, lane, total, nb, top, wl, my_end, my_src,
                                        my_dst, s_end, s_src, s_dst, blo, bhi, sbase, dbase);
          break;
        }
      }
      return;
    }
  }
  if (FAST && s_allvec) {
    // Every block is 16-byte aligned at both ends and a whole number of
    // chunks (e.g. rows of one bf16 with equal counts): plain vector copies
    // (the resident grid; the one-pass grid takes the form above).  The same
    // steps as chunk_vec_tile, written out with their checks: whole tiles
    // without them measured slower on this grid.
    const uint64_t total = s_end[nb - 1];
    int top = 1;
    while (top * 2 <= nb) top *= 2;
    const uint64_t tile = (uint64_t)kBlock * UN;
    // at most 64 blocks: lane l keeps block l's end and bases in registers,
    // and a wave locates its units with one ballot (wave_block)
    const int lane = threadIdx.x & 63;
    const bool wl = COLL_A2A_WAVE_LOCATE && nb <= 64;
    uint64_t my_end = ~0ull, my_src = 0, my_dst = 0;
    if (wl && lane < nb) {
      my_end = s_end[lane];
      my_src = s_src[lane];
      my_dst = s_dst[lane];
    }
    uint64_t blo = 1, bhi = 0, sbase = 0, dbase = 0;
    for (uint64_t wbase = (uint64_t)blockIdx.x * tile + (threadIdx.x - lane); wbase < total;
         wbase += (uint64_t)gridDim.x * tile) {
      const uint64_t base = wbase + lane;
      u32x4 v[UN];
      uint64_t da[UN];
#pragma unroll
      for (int u = 0; u < UN; u++) {
        const uint64_t x = base + (uint64_t)u * kBlock;
        int wlo;
        if (wl && wave_block(my_end, wbase + (uint64_t)u * kBlock, wlo)) {
          blo = wlo > 0 ? readlane64(my_end, wlo - 1) : 0;
          bhi = readlane64(my_end, wlo);
          sbase = readlane64(my_src, wlo) - blo * 16;
          dbase = readlane64(my_dst, wlo) - blo * 16;
        }
        if (x < total) {
          if (x < blo || x >= bhi) {
            int lo = 0;
            for (int step = top; step > 0; step >>= 1) {
              const int c = lo + step;
              if (c <= nb && s_end[c - 1] <= x) lo = c;
            }
            blo = lo > 0 ? s_end[lo - 1] : 0;
            bhi = s_end[lo];
            sbase = s_src[lo] - blo * 16;
            dbase = s_dst[lo] - blo * 16;
          }
          da[u] = dbase + x * 16;
          if constexpr (NT) v[u] = __builtin_nontemporal_load(gconst<u32x4>(sbase + x * 16));
          else v[u] = *gconst<u32x4>(sbase + x * 16);
        }
      }
#pragma unroll
      for (int u = 0; u < UN; u++) {
        const uint64_t x = base + (uint64_t)u * kBlock;
        if (x < total) {
          if constexpr (NT) __builtin_nontemporal_store(v[u], gmut<u32x4>(da[u]));
          else *gmut<u32x4>(da[u]) = v[u];
        }
      }
    }
    return;
  }

  const uint64_t total = s_end[nb - 1];
  int top = 1;
  while (top * 2 <= nb) top *= 2;
  const uint64_t tile = (uint64_t)kBlock * UN;
  uint64_t blo = 1, bhi = 0, sbase = 0, dbase = 0, blen = 0;
  for (uint64_t base = (uint64_t)blockIdx.x * tile + threadIdx.x; base < total;
       base += (uint64_t)gridDim.x * tile) {
    uint64_t sa[UN], da[UN];
    uint32_t n[UN];                 // bytes of the chunk; 0 = no chunk
    bool vec[UN];
    // 1. locate every chunk (LDS only)
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const uint64_t x = base + (uint64_t)u * kBlock;
      n[u] = 0;
      vec[u] = false;
      sa[u] = da[u] = 0;
      if (x < total) {
        if (x < blo || x >= bhi) {
          int lo = 0;
          for (int step = top; step > 0; step >>= 1) {
            const int c = lo + step;
            if (c <= nb && s_end[c - 1] <= x) lo = c;
          }
          blo = lo > 0 ? s_end[lo - 1] : 0;
          bhi = s_end[lo];
          sbase = s_src[lo];
          dbase = s_dst[lo];
          blen = s_len[lo];
        }
        const uint64_t off = (x - blo) * 16;
        const uint64_t rem = blen - off;                 // > 0: x lies inside the block
        n[u] = rem < 16 ? (uint32_t)rem : 16u;
        sa[u] = sbase + off;
        da[u] = dbase + off;
        vec[u] = n[u] == 16 && ((sa[u] | da[u]) & 15) == 0;
      }
    }
    // 2. all 16-byte loads, 3. all 16-byte stores
    u32x4 v[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
      if (vec[u]) {
        if constexpr (NT) v[u] = __builtin_nontemporal_load(gconst<u32x4>(sa[u]));
        else v[u] = *gconst<u32x4>(sa[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < UN; u++) {
      if (vec[u]) {
        if constexpr (NT) __builtin_nontemporal_store(v[u], gmut<u32x4>(da[u]));
        else *gmut<u32x4>(da[u]) = v[u];
      }
    }
    // 4. the rest (block tails, misaligned blocks) in narrower units
#pragma unroll
    for (int u = 0; u < UN; u++)
      if (n[u] && !vec[u]) copy_chunk_narrow(sa[u], da[u], n[u]);
  }
}

// ---------------------------------------------- descriptor form (workspace)
// For large exchanges with a caller workspace: a pre-kernel writes the block
// table once and, per tile of kDescTile units, the index of the block holding
// the tile's first unit (16 bits; 0xFFFF: at or past the total).  A
// workgroup of the main kernel then starts with two scalar loads in a row,
// its tile's index and that block's 32-byte entry (a table of at most 8 KiB
// that stays in the scalar cache), instead of building the table itself.
// 16-byte descriptors holding both addresses (one load, 8x the bytes) measured
// 0.2-0.8% slower at the MoE shape, 32-byte ones slower again.
struct A2aBlk {
  uint64_t sb, db;   // unit addresses of the block's first unit minus its start in the index space
  uint64_t end;      // the block's end in the index space
  uint64_t more;     // 1 when the total runs past the last descriptor's tile (same in every entry)
};

// Lanes per workgroup and units per lane of the descriptor kernel.  MI355X,
// R = 8, graph replay, the 3.5 GiB MoE exchange / 8 x 64 MiB of 16-byte rows
// (with 32-byte descriptors): 64 x 1 6405 / 6224 GB/s; 256 x 1 6347 / 6150;
// 512 x 1 6277 / 6175; 128 x 1 6170 / 6112; 64 x 4 6333 / 6209; 256 x 2
// 5890 / 5877.  Four one-wave workgroups sharing a 4 KiB tile's descriptor on
// one XCD: 6346 / 6126.
#ifndef COLL_DESC_LANES
#define COLL_DESC_LANES 64
#endif
#ifndef COLL_DESC_U
#define COLL_DESC_U 1
#endif
#ifndef COLL_DESC_BUILD_WGS
#define COLL_DESC_BUILD_WGS 4
#endif
constexpr int kDescBuildWgs = COLL_DESC_BUILD_WGS;   // descriptor writers per CU
constexpr int kDescLanes = COLL_DESC_LANES;
constexpr int kDescU = COLL_DESC_U;
constexpr int kDescTile = kDescLanes * kDescU;   // units per tile (and per descriptor)

// Workgroups are handed to the 8 XCDs in turn (workgroup w to XCD w % 8), and
// each XCD has its own L2.  Storing tile t's index at desc_slot(t) puts the
// 64 indices of one 128-byte line on tiles t, t+8, ..., t+504 of one XCD, so
// each line is fetched from HBM once rather than once per XCD (measured with
// 32-byte descriptors in tile order: 117 MB of extra reads on the 3.5 GiB MoE
// exchange, the line count times 128 bytes).  A bijection on each group of
// 512 tiles; desc_tile is its inverse.  The workspace holds whole groups.
constexpr uint64_t kDescGroup = 512;
__device__ __forceinline__ uint64_t desc_slot(uint64_t t) {
  return (t & ~(kDescGroup - 1)) | ((t & 7) << 6) | ((t >> 3) & 63);
}
__device__ __forceinline__ uint64_t desc_tile(uint64_t i) {
  return (i & ~(kDescGroup - 1)) | ((i & 63) << 3) | ((i >> 6) & 7);
}

// General table build (R <= 16, four blocks per lane of wave 0), as in a2av_body.
template <int B>
__device__ __forceinline__ void desc_table(const RankPtrs &p, const RowLimits &lim, int R,
                                           const int64_t *counts,
                                           const int64_t *sdispls, const int64_t *rdispls, int ct,
                                           uint64_t row_units, uint64_t *s_end, uint64_t *s_src,
                                           uint64_t *s_dst) {
  const int nb = R * R;
  const int lane = threadIdx.x;
  uint64_t len[4];
  int64_t cnt[4], sdv[4], rdv[4];
  uint64_t local = 0;
  const int64_t my_in = lane_rows(lim.in), my_out = lane_rows(lim.out);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int b = lane * 4 + j;
    const int bb = b < nb ? b : 0;
    const int s = bb / R, d = bb - s * R;
    cnt[j] = counts[count_index(ct, R, s, d)];
    sdv[j] = sdispls[bb];
    rdv[j] = rdispls[d * R + s];
  }
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int b = lane * 4 + j;
    const int bb = b < nb ? b : 0;
    const int s = bb / R, d = bb - s * R;
    const bool fits = block_fits(cnt[j], sdv[j], rdv[j], rows_from_lane(my_in, s),
                                 rows_from_lane(my_out, d));
    len[j] = (b < nb && fits) ? (uint64_t)cnt[j] * row_units : 0;
    local += len[j];
  }
  const uint64_t incl = wave_incl_scan(local);
  uint64_t start = incl - local;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int b = lane * 4 + j;
    if (b < nb) {
      const int s = b / R, d = b - s * R;
      s_src[b] = reinterpret_cast<uintptr_t>(p.in[s]) / B + (uint64_t)sdv[j] * row_units - start;
      s_dst[b] = reinterpret_cast<uintptr_t>(p.out[d]) / B + (uint64_t)rdv[j] * row_units - start;
      start += len[j];
      s_end[b] = start;
    }
  }
}

// Block holding unit x from the table in the workspace (nb entries): the
// index of the first block ending after x, nb when x is past the total.
__device__ __forceinline__ int desc_find(const A2aBlk *blk, int nb, uint64_t x) {
  int lo = 0;
  for (int step = kMaxBlocks; step > 0; step >>= 1) {
    const int c = lo + step;
    if (c <= nb && blk[c - 1].end <= x) lo = c;
  }
  return lo;
}

// Copies the lane's units x0 + u * kDescLanes of a tile whose first unit lies
// in block (sb, db, end); a unit past the block's end finds its own block in
// the table.  Located, then loaded, then stored.
template <int B, bool NT>
__device__ __forceinline__ void desc_units(uint64_t sb, uint64_t db, uint64_t end,
                                           const A2aBlk *blk, int nb, uint64_t x0) {
  using U = typename UnitT<B>::T;
  uint64_t sa[kDescU], da[kDescU];
#pragma unroll
  for (int u = 0; u < kDescU; u++) {
    const uint64_t x = x0 + (uint64_t)u * kDescLanes;
    uint64_t s = sb, d = db;
    sa[u] = 0;
    if (x >= end) {                             // the tile crosses into later blocks
      const int lo = desc_find(blk, nb, x);
      if (lo >= nb) continue;                   // past the total
      s = blk[lo].sb;
      d = blk[lo].db;
    }
    sa[u] = (s + x) * B;
    da[u] = (d + x) * B;
  }
  U v[kDescU];
#pragma unroll
  for (int u = 0; u < kDescU; u++) {
    if (!sa[u]) continue;
    if constexpr (NT) v[u] = __builtin_nontemporal_load(gconst<U>(sa[u]));
    else v[u] = *gconst<U>(sa[u]);
  }
#pragma unroll
  for (int u = 0; u < kDescU; u++) {
    if (!sa[u]) continue;
    if constexpr (NT) __builtin_nontemporal_store(v[u], gmut<U>(da[u]));
    else *gmut<U>(da[u]) = v[u];
  }
}

// A resident grid: each workgroup builds the block table in LDS once, then
// thread i writes slots 2i and 2i+1 (one 32-bit store; a wave's stores are
// contiguous), i += stride.  Workgroup 0 also writes the table.  MI355X, the
// MoE exchange with 16-byte descriptors: one workgroup per 256 tiles storing
// in tile order 28.6 us; 2 resident workgroups per CU 27.2 us; slot order
// with 4 per CU 21.6 us, and 8, 16 or one per 256 slots within 1% of that.
template <int B>
__global__ __launch_bounds__(kBlock) void a2av_desc_build(RankPtrs p, RowLimits lim, int R, const int64_t *counts,
                                                         const int64_t *sdispls,
                                                         const int64_t *rdispls, int ct,
                                                         uint64_t row_units, uint32_t *idx,
                                                         uint64_t ndesc, A2aBlk *blk) {
  __shared__ uint64_t s_end[kMaxBlocks], s_src[kMaxBlocks], s_dst[kMaxBlocks];
  const int nb = R * R;
  if (threadIdx.x < 64)
    desc_table<B>(p, lim, R, counts, sdispls, rdispls, ct, row_units, s_end, s_src, s_dst);
  __syncthreads();
  const uint64_t total = s_end[nb - 1];
  const uint64_t more = total > ndesc * kDescTile ? 1 : 0;
  if (blockIdx.x == 0)
    for (int b = threadIdx.x; b < nb; b += kBlock) blk[b] = A2aBlk{s_src[b], s_dst[b], s_end[b], more};
  const uint64_t pairs = (ndesc + kDescGroup - 1) / kDescGroup * kDescGroup / 2;
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  for (uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < pairs; i += stride) {
    uint32_t w = 0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint64_t t = desc_tile(2 * i + h);
      uint32_t v = 0xFFFFu;
      const uint64_t x = t * kDescTile;
      if (t < ndesc && x < total) {
        int lo = 0;                             // blocks ending at or before x
        for (int step = kMaxBlocks; step > 0; step >>= 1) {
          const int c = lo + step;
          if (c <= nb && s_end[c - 1] <= x) lo = c;
        }
        v = (uint32_t)lo;
      }
      w |= v << (16 * h);
    }
    idx[i] = w;
  }
}

// One workgroup per tile (the grid is exactly ndesc workgroups).  Both loads
// are made before any store, so they go through the scalar cache: inside a
// grid-stride loop the descriptor became a vector load behind a wait and cost
// 20% (MI355X, the MoE exchange).  When the capacity undercounts the rows,
// the tiles past the last descriptor are looped over from the table.
template <int B, bool NT>
__global__ __launch_bounds__(kDescLanes) void a2av_desc_kernel(const uint32_t *__restrict__ idx,
                                                              const A2aBlk *__restrict__ blk,
                                                              int nb) {
  const uint64_t sl = desc_slot(blockIdx.x);
  uint32_t w = idx[sl >> 1];
  COLL_UNIFORM(w);
  const uint32_t b = (sl & 1) ? (w >> 16) : (w & 0xFFFFu);
  if (b == 0xFFFFu) return;                     // at or past the total
  const A2aBlk e = blk[b];
  uint64_t sb = e.sb, db = e.db, end = e.end, more = e.more;
  COLL_UNIFORM(sb);                             // one scalar load of the entry
  COLL_UNIFORM(db);
  COLL_UNIFORM(end);
  COLL_UNIFORM(more);
  const uint64_t t0 = (uint64_t)blockIdx.x * kDescTile;
  desc_units<B, NT>(sb, db, end, blk, nb, t0 + threadIdx.x);
  if (more == 0) return;
  for (uint64_t t = (uint64_t)blockIdx.x + gridDim.x;; t += gridDim.x) {
    const int lo = desc_find(blk, nb, t * kDescTile);
    if (lo >= nb) return;
    desc_units<B, NT>(blk[lo].sb, blk[lo].db, blk[lo].end, blk, nb, t * kDescTile + threadIdx.x);
  }
}

}  // namespace

int launch_a2av(const Launch &L, int R, const RankPtrs &p, const RowLimits &lim,
                const int64_t *counts, const int64_t *sdispls, const int64_t *rdispls, int ct,
                size_t row_bytes, size_t rows_capacity) {
  uintptr_t bits = row_bytes;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)p.in[r] | (uintptr_t)p.out[r];
  const int unit = copy_unit(bits);
  const uint64_t row_units = row_bytes / unit;
  // The total is only known on the device; the receive capacity bounds it.
  // Large exchanges: one workgroup per tile of the bound (surplus workgroups
  // exit at once).  Up to kResidentMaxBytes, and without a bound: a resident
  // grid of 4 workgroups per CU looping over tiles of kA2aResU units per lane,
  // which builds the block table once per workgroup.  MI355X, R = 8, graph
  // replay, since the one-pass grid's whole tiles lost their bound checks:
  // one-pass 1.5-2 points slower at 4-8 MiB per rank, 0.3-0.7 faster at 16,
  // 2-3 faster at 32, 1 faster at the MoE exchange of 256 tokens (28 MiB).
  constexpr uint64_t kResidentMaxBytes = COLL_A2A_RESIDENT_MAX_BYTES;
  const uint64_t cap_bytes = (uint64_t)rows_capacity * row_bytes;
  const bool resident = rows_capacity == 0 || cap_bytes <= kResidentMaxBytes;
  // (never more workgroups than the one-pass grid would have: small
  // messages stay a handful of workgroups)
  const unsigned g_res = (unsigned)L.num_cus * 4;
  unsigned g = g_res;
  if (unit == 16) {
    if (rows_capacity > 0) {
      const uint64_t units = (uint64_t)rows_capacity * row_units;
      g = resident ? grid_for(L, units, kA2aU) : grid_tiles(units, (uint64_t)kA2aBlock * kA2aU);
      if (resident && g > g_res) g = g_res;
    }
    if (L.a2a_grid > 0) g = (unsigned)L.a2a_grid;
    const bool small = COLL_A2A_SMALL && R <= 8;
    if (resident && small)
      COLL_UNIT_SWITCH(a2av_res_kernel8, unit, L.a2a_nt, dim3(g), L.stream, p, lim, R, counts,
                       sdispls, rdispls, ct, row_units);
    else if (resident)
      COLL_UNIT_SWITCH(a2av_res_kernel, unit, L.a2a_nt, dim3(g), L.stream, p, lim, R, counts,
                       sdispls, rdispls, ct, row_units);
    else if (small)
      COLL_UNIT_SWITCH_BLOCK(a2av_kernel8, unit, L.a2a_nt, dim3(g), kA2aBlock, L.stream, p, lim, R,
                             counts, sdispls, rdispls, ct, row_units);
    else
      COLL_UNIT_SWITCH_BLOCK(a2av_kernel, unit, L.a2a_nt, dim3(g), kA2aBlock, L.stream, p, lim, R,
                             counts, sdispls, rdispls, ct, row_units);
  } else {
    // chunks: at most capacity bytes / 16 plus one partial chunk per block
    const unsigned g_res_c = (unsigned)L.num_cus * COLL_A2A_CHUNK_RES_PER_CU;
    g = g_res_c;
    if (rows_capacity > 0) {
      const unsigned g1 = grid_for(L, (cap_bytes + 15) / 16 + (uint64_t)R * R, kA2aU);
      g = resident ? (g1 < g_res_c ? g1 : g_res_c) : g1;
    }
    if (L.a2a_grid > 0) g = (unsigned)L.a2a_grid;
#define COLL_A2A_CHUNK_B(NTV, UNV, FASTV, BPLV)                                                  \
  hipLaunchKernelGGL((a2av_chunk_kernel<NTV, UNV, FASTV, BPLV>), dim3(g), dim3(kBlock), 0,       \
                     L.stream, p, lim, R, counts, sdispls, rdispls, ct, (uint64_t)row_bytes)
#define COLL_A2A_CHUNK(NTV, UNV, FASTV)                                                          \
  do {                                                                                         \
    if (COLL_A2A_CHUNK_SMALL && R <= 8) COLL_A2A_CHUNK_B(NTV, UNV, FASTV, 1);                    \
    else COLL_A2A_CHUNK_B(NTV, UNV, FASTV, 4);                                                  \
  } while (0)
    if (L.a2a_nt && resident) COLL_A2A_CHUNK(true, kA2aResU, true);
    else if (L.a2a_nt) COLL_A2A_CHUNK(true, kA2aU, false);
    else if (resident) COLL_A2A_CHUNK(false, kA2aResU, true);
    else COLL_A2A_CHUNK(false, kA2aU, false);
#undef COLL_A2A_CHUNK
#undef COLL_A2A_CHUNK_B
  }
  return hip_status();
}

size_t a2av_workspace_bytes(int R, size_t rows_capacity, size_t row_bytes, size_t min_bytes) {
  if (row_bytes % 16 != 0 || rows_capacity == 0) return 0;          // no descriptor form
  if (rows_capacity * row_bytes < min_bytes) return 0;              // the plain form is faster
  const uint64_t cap_units = (uint64_t)rows_capacity * (row_bytes / 16);
  const uint64_t ndesc = (cap_units + kDescTile - 1) / kDescTile;
  const uint64_t slots = (ndesc + kDescGroup - 1) / kDescGroup * kDescGroup;
  return ((size_t)R * R * sizeof(A2aBlk) + slots * sizeof(uint16_t) + 255) & ~(size_t)255;
}

// Tiles of 64 units of the descriptor form for this capacity; 0 when the form
// does not apply (rows not whole 16-byte units on every buffer, no capacity,
// or more tiles than one grid holds).
static uint64_t desc_tiles(int R, const RankPtrs *p, size_t row_bytes, size_t rows_capacity) {
  uintptr_t bits = row_bytes;
  if (p)
    for (int r = 0; r < R; r++) bits |= (uintptr_t)p->in[r] | (uintptr_t)p->out[r];
  if (copy_unit(bits) != 16 || rows_capacity == 0) return 0;
  const uint64_t cap_units = (uint64_t)rows_capacity * (row_bytes / 16);
  const uint64_t ndesc = (cap_units + kDescTile - 1) / kDescTile;
  return ndesc > 0x7FFFFFFFull ? 0 : ndesc;
}

int launch_a2av_ws_build(const Launch &L, int R, const RankPtrs &p, const RowLimits &lim,
                         const int64_t *counts, const int64_t *sdispls, const int64_t *rdispls,
                         int ct, size_t row_bytes, size_t rows_capacity, void *ws) {
  const uint64_t ndesc = desc_tiles(R, &p, row_bytes, rows_capacity);
  if (ndesc == 0) return COLL_ERR_UNSUPPORTED;
  A2aBlk *blk = reinterpret_cast<A2aBlk *>(ws);
  uint32_t *idx = reinterpret_cast<uint32_t *>(blk + (size_t)R * R);   // two indices per word
  // descriptor writers: a resident grid (COLL_DESC_BUILD_WGS per CU), no
  // more workgroups than there are index pairs for their threads
  const uint64_t pairs = (ndesc + kDescGroup - 1) / kDescGroup * kDescGroup / 2;
  const uint64_t gneed = (pairs + kBlock - 1) / kBlock;
  const uint64_t gres = (uint64_t)L.num_cus * kDescBuildWgs;
  hipLaunchKernelGGL((a2av_desc_build<16>), dim3((unsigned)(gneed < gres ? gneed : gres)),
                     dim3(kBlock), 0, L.stream, p, lim, R, counts, sdispls, rdispls, ct,
                     (uint64_t)(row_bytes / 16), idx, ndesc, blk);
  return hip_status();
}

int launch_a2av_ws_copy(const Launch &L, int R, size_t row_bytes, size_t rows_capacity,
                        void *ws) {
  const uint64_t ndesc = desc_tiles(R, nullptr, row_bytes, rows_capacity);
  if (ndesc == 0) return COLL_ERR_UNSUPPORTED;
  A2aBlk *blk = reinterpret_cast<A2aBlk *>(ws);
  uint32_t *idx = reinterpret_cast<uint32_t *>(blk + (size_t)R * R);
  if (L.a2a_nt)
    hipLaunchKernelGGL((a2av_desc_kernel<16, true>), dim3((unsigned)ndesc), dim3(kDescLanes), 0,
                       L.stream, idx, blk, R * R);
  else
    hipLaunchKernelGGL((a2av_desc_kernel<16, false>), dim3((unsigned)ndesc), dim3(kDescLanes), 0,
                       L.stream, idx, blk, R * R);
  return hip_status();
}

int launch_a2av_ws(const Launch &L, int R, const RankPtrs &p, const RowLimits &lim,
                   const int64_t *counts, const int64_t *sdispls, const int64_t *rdispls, int ct,
                   size_t row_bytes, size_t rows_capacity, void *ws) {
  // rows that are not whole 16-byte units, no capacity, or more tiles than a
  // grid holds: the plain form
  if (desc_tiles(R, &p, row_bytes, rows_capacity) == 0)
    return launch_a2av(L, R, p, lim, counts, sdispls, rdispls, ct, row_bytes, rows_capacity);
  const int rc = launch_a2av_ws_build(L, R, p, lim, counts, sdispls, rdispls, ct, row_bytes,
                                      rows_capacity, ws);
  if (rc != COLL_OK) return rc;
  return launch_a2av_ws_copy(L, R, row_bytes, rows_capacity, ws);
}

}  // namespace coll
