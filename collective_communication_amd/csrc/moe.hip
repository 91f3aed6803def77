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
//   moe_expert_scale  the test expert y = rne(x * (1 + e/256)), in
//                 place: a one-workgroup table of row prefixes, then either
//                 one descriptor per received row and one wave per (row,
//                 1 KiB segment) -- a path that also runs as two calls, the
//                 descriptors built ahead from the tables alone -- or one
//                 workgroup per tile of received units searching the table.
//   moe_combine   one wave per (token, 1 KiB segment): topk rows gathered by
//                 pos, fp32 fold k = 0..K-1 of separately rounded products,
//                 one RNE.
#include "coll_internal.h"

#pragma clang fp contract(off)

namespace coll {

constexpr int kMoeTile = 1024;        // ids per layout tile (kBlock * 4)
// 16-byte units per lane of a permute / fused-dispatch wave: one (a wave
// moves a 1 KiB segment of a row to its K slots); measured on MI355X at the
// 4096 x 7168 x top-8 shape: 1 -> 5390 / 5580 GB/s (permute / dispatch),
// 2 -> 4990 / 4900, 4 -> 5000 / 4900, 8 -> 5020 / 4450
#ifndef COLL_PERMUTE_U
#define COLL_PERMUTE_U 1
#endif
// test expert, one-pass tiles of 256 lanes x U units; MI355X, the 3.5 GiB
// in-place MoE shape: U = 2 -> 1655 us, 4 -> 1338, 8 -> 1284, 16 -> 1288 (the
// resident grid it replaced: 1345)
#ifndef COLL_EXPERT_U
#define COLL_EXPERT_U 8
#endif
// combine / fused combine: 16-byte units per lane of a wave (a wave reduces
// 64 * U units of one token from its K rows); MI355X, 4096 x 7168 x top-8:
// combine 1 -> 740 us, 2 -> 764, 4 -> 764; fused combine (which also stages
// its source's send blocks per workgroup and applies the expert) 1 -> 828,
// 2 -> 766, 4 -> 764, 7 -> 1008, 8 -> 1072
#ifndef COLL_COMBINE_U
#define COLL_COMBINE_U 1
#endif
#ifndef COLL_COMBINE_RECV_U
#define COLL_COMBINE_RECV_U 2
#endif
// Row items (one wave each) per workgroup; MI355X, 4096 x 7168 x top-8:
// permute 16 -> 878 us, 8 -> 840, 4 -> 779, 2 -> 810, 1 -> 872; fused dispatch 4 -> 766, 2 -> 761,
// 1 -> 786; combine 4 -> 742, 2 -> 730, 1 -> 718; fused combine 4 -> 763,
// 2 -> 760, 1 -> 744.
#ifndef COLL_PERMUTE_WAVES
#define COLL_PERMUTE_WAVES 4
#endif
#ifndef COLL_COMBINE_WAVES
#define COLL_COMBINE_WAVES 1
#endif
#ifndef COLL_DISPATCH_WAVES
#define COLL_DISPATCH_WAVES 4
#endif
#ifndef COLL_COMBINE_RECV_WAVES
#define COLL_COMBINE_RECV_WAVES 1
#endif
// waves (row items) per workgroup of the row-segment kernels
constexpr int kPermuteWaves = COLL_PERMUTE_WAVES;
constexpr int kCombineWaves = COLL_COMBINE_WAVES;
constexpr int kDispatchWaves = COLL_DISPATCH_WAVES;
constexpr int kCombineRecvWaves = COLL_COMBINE_RECV_WAVES;
constexpr int kPermuteU = COLL_PERMUTE_U;     // 16-byte units per lane, permute
constexpr int kExpertU = COLL_EXPERT_U;       // ... test expert
#ifndef COLL_EXPERT_BLOCK
#define COLL_EXPERT_BLOCK 256
#endif
// lanes per workgroup, test expert (MI355X: 256 -> 1290 us, 128 -> 1300, 64 -> 1307)
constexpr int kExpertBlock = COLL_EXPERT_BLOCK;
constexpr int kCombineU = COLL_COMBINE_U;     // ... combine (each gathers K rows)
constexpr int kCombineRecvU = COLL_COMBINE_RECV_U;   // ... fused combine
constexpr int kMaxExperts = kMoeMaxExperts;
// The fused dispatch and the combines load a token's slots (and weights, ids)
// kSlotChunk at a time, all of a chunk's loads issued together from clamped
// indices before any is used: a load guarded by `k < K` made the compiler
// wait for each one in turn.
constexpr int kSlotChunk = 8;

// The entry tables (two int64 per entry), then one 8-byte descriptor per
// receive row of the capacity (the row-descriptor kernel; 0 rows: none).
size_t moe_expert_table_bytes(int R, int E) {
  return ((size_t)R * E * 2 * sizeof(int64_t) + 255) & ~(size_t)255;
}
size_t moe_expert_workspace_bytes(int R, int E, size_t rows_capacity) {
  return moe_expert_table_bytes(R, E) + ((rows_capacity * sizeof(uint64_t) + 255) & ~(size_t)255);
}

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
  // the tile's ids are loaded together (clamped index; TK > tile * kMoeTile)
  int v[kMoeTile / kBlock];
#pragma unroll
  for (int j = 0; j < kMoeTile / kBlock; j++) {
    const int i = tile * kMoeTile + j * kBlock + threadIdx.x;
    v[j] = id[i < TK ? i : TK - 1];
  }
#pragma unroll
  for (int j = 0; j < kMoeTile / kBlock; j++) {
    const int i = tile * kMoeTile + j * kBlock + threadIdx.x;
    const int e = v[j];
    if (i < TK && (unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);   // out-of-range ids dropped
  }
  __syncthreads();
  int32_t *out = hist + ((size_t)s * ntiles + tile) * E;
  for (int e = threadIdx.x; e < E; e += kBlock) out[e] = h[e];
}

// blockDim = 1024 (one thread per expert, E <= 1024), grid = R.
__global__ __launch_bounds__(1024) void moe_scan(int R, int E, int ntiles, int32_t *hist,
                                                 int32_t *expert_off, int32_t *expert_counts,
                                                 int64_t *sendcounts, int64_t *sdispls) {
  __shared__ int wave_tot[16];
  __shared__ int off[kMaxExperts + 1];
  const int s = blockIdx.x, e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    // 16 tile counts in flight per round trip (a 4096 x top-8 batch has 32
    // tiles), then each replaced by the tile's offset within the expert
    constexpr int kIn = 16;
    int32_t *h = hist + (size_t)s * ntiles * E + e;
    for (int t0 = 0; t0 < ntiles; t0 += kIn) {
      int c[kIn];
#pragma unroll
      for (int j = 0; j < kIn; j++) c[j] = (t0 + j < ntiles) ? h[(size_t)(t0 + j) * E] : 0;
#pragma unroll
      for (int j = 0; j < kIn; j++) {
        if (t0 + j < ntiles) {
          h[(size_t)(t0 + j) * E] = cnt;
          cnt += c[j];
        }
      }
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
  // the rows sent: ids outside [0, E) were not counted, so this can be
  // below T * K
  if (e == E - 1) off[E] = excl + cnt;
  __syncthreads();
  if (e < R) {
    const int per = E / R;
    sendcounts[s * R + e] = off[(e + 1) * per] - off[e * per];
    sdispls[s * R + e] = off[e * per];
  }
}

// An id outside [0, E) gets pos = -1: no slot.
__global__ __launch_bounds__(kBlock) void moe_pos(PtrTable ids, MutPtrTable pos, int R, int TK,
                                                  int E, int nbits, int ntiles,
                                                  const int32_t *hist, const int32_t *expert_off,
                                                  const int64_t *sendcounts, int64_t *rdispls) {
  __shared__ int base[kMaxExperts];
  __shared__ int run[kMaxExperts];
  __shared__ int wcnt[kBlock / 64][kMaxExperts];
  __shared__ int64_t sc[COLL_MAX_RANKS * COLL_MAX_RANKS];
  const int s = blockIdx.y, tile = blockIdx.x;
  if (s == 0 && tile == 0) {
    // receive displacements: rdispls[d][s'] = sum_{s'' < s'} sendcounts[s''][d],
    // from the counts staged in LDS (one load per thread, R * R <= kBlock)
    if ((int)threadIdx.x < R * R) sc[threadIdx.x] = sendcounts[threadIdx.x];
    __syncthreads();
    if ((int)threadIdx.x < R * R) {
      const int t = threadIdx.x, d = t / R, s2 = t - d * R;
      int64_t acc = 0;
      for (int q = 0; q < s2; q++) acc += sc[q * R + d];
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
  // every round's id is loaded up front (clamped index; TK > tile * kMoeTile)
  int ids_r[kMoeTile / kBlock];
#pragma unroll
  for (int round = 0; round < kMoeTile / kBlock; round++) {
    const int i = tile * kMoeTile + round * kBlock + threadIdx.x;
    ids_r[round] = id[i < TK ? i : TK - 1];
  }
#pragma unroll
  for (int round = 0; round < kMoeTile / kBlock; round++) {
    for (int x = threadIdx.x; x < E; x += kBlock)
#pragma unroll
      for (int q = 0; q < kBlock / 64; q++) wcnt[q][x] = 0;
    __syncthreads();
    const int i = tile * kMoeTile + round * kBlock + threadIdx.x;
    const int raw = i < TK ? ids_r[round] : -1;
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
    } else if (i < TK) {
      out[i] = -1;                                 // no expert: no slot
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

// Work item of the token-row kernels: one wave per (source s, token t,
// segment of a row).  Everything that identifies the item is wave-uniform
// and lives in scalar registers, so the token's K slots (and weights) are
// scalar loads and the vector memory pipe carries only row data: a wave
// issues all of its row loads, then all of its stores, and exits (no wave
// ever waits on its own stores, which the in-order vmcnt counter would force
// if it went on to a next item).
struct RowItem {
  int t;            // token
  int seg;          // segment index within the row
  bool valid;
};

template <int WAVES>
__device__ __forceinline__ RowItem row_item(int T, int nseg) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int id = (int)blockIdx.x * WAVES + wave;             // < T * nseg + WAVES - 1
  RowItem it;
  it.t = id / nseg;
  it.seg = id - it.t * nseg;
  it.valid = it.t < T;
  return it;
}

// send[s][pos[s][t,k]] = x[s][t] for every k.  Segment = 64 lanes x UN units.
template <int B, bool NT>
__global__ __launch_bounds__(64 * kPermuteWaves) void moe_permute_kernel(PtrTable x, PtrTable pos,
                                                             MutPtrTable send, int T, int K,
                                                             uint32_t upr, int nseg) {
  using U = typename UnitT<B>::T;
  constexpr int UN = kPermuteU;
  const RowItem it = row_item<kPermuteWaves>(T, nseg);
  if (!it.valid) return;
  const int s = blockIdx.y;
  const uint32_t TK = (uint32_t)T * (uint32_t)K;
  const int lane = threadIdx.x & 63;
  const U *src = reinterpret_cast<const U *>(x.p[s]) + (size_t)it.t * upr;
  const int32_t *pk = reinterpret_cast<const int32_t *>(pos.p[s]) + (size_t)it.t * K;
  U *dst = reinterpret_cast<U *>(send.p[s]);
  const uint32_t u0 = (uint32_t)it.seg * (64 * UN) + lane;
  U v[UN];
#pragma unroll
  for (int u = 0; u < UN; u++) {
    const uint32_t x_u = u0 + u * 64;
    if (x_u < upr) v[u] = NT ? __builtin_nontemporal_load(src + x_u) : src[x_u];
  }
  // One slot at a time, each slot read by a vector load issued after the
  // previous slot's stores.  Vector loads and stores share one in-order
  // counter, so the wave waits for those stores before it stores again: at
  // most one slot (1 KiB) of stores per wave in flight, and the fan-out
  // runs faster that way.  Loading a chunk of slots first (as the other MoE
  // kernels do) measured 9% slower here (848 vs 777 us at the MoE shape), and
  // reading each slot through the scalar cache, which leaves all K slots'
  // stores in flight, 10% slower (855-863 vs 779-783 us).  A row form --
  // one workgroup per token, wave k writing slot k's whole 14 KiB row in one
  // run from cacheable loads of the token row -- measured 835 against 785 us.
  for (int k = 0; k < K; k++) {
    const int32_t slot = __builtin_amdgcn_readfirstlane(pk[k]);
    if ((uint32_t)slot >= TK) continue;                      // never write outside
    U *row = dst + (size_t)slot * upr;
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const uint32_t x_u = u0 + u * 64;
      if (x_u < upr) {
        if constexpr (NT) __builtin_nontemporal_store(v[u], row + x_u);
        else row[x_u] = v[u];
      }
    }
  }
}

// ------------------------------------------------------------- test expert

// Receive-order entries: entry j = d*E + s*per + el (per = E/R) covers the
// rows of expert d*per + el sent by s to d, expert_counts[s*E + d*per + el]
// of them.  Numbering every received row of every rank in entry order (global
// row g) balances the work over ranks however skewed the routing is.
//
// moe_expert_table: one workgroup of kTableThreads writes two int64 tables:
//   s_end[j] = rows in entries 0..j (inclusive prefix), so g is in entry j
//              iff s_end[j-1] <= g < s_end[j];
//   rb[j]    = rdispls[d*R+s] - (rows in entries before (d, s)'s first),
//              so the receive row of g in recv[d] is rb[j] + g.
// A (d, s) block with a negative expert count, or whose rows do not all lie
// inside recv[d] (recv_rows), counts as empty: no row of it is numbered, so
// the kernels that follow never address it and its rows keep their values.
// Inclusive scan over the workgroup's threads (at most 1024; entries in thread
// order); returns the exclusive prefix of the thread's `local`.
__device__ __forceinline__ int64_t table_scan(int64_t local, int64_t *wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int64_t incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int64_t run = incl - local;
  for (int q = 0; q < w; q++) run += wsum[q];
  __syncthreads();                               // wsum is reused by the next scan
  return run;
}

// Entry j = d*E + s*per + el of the receive-order table (a (d, s) block's
// entries are consecutive): its count.
__device__ __forceinline__ int64_t entry_count(const int32_t *expert_counts, int E, int per,
                                               int j) {
  const int d = j / E, rem = j - d * E, s = rem / per, el = rem - s * per;
  return (int64_t)expert_counts[(size_t)s * E + d * per + el];
}

// Threads of the table's one workgroup.  256, the size of the permute's
// workgroups: the table is built on a second stream while the permute fills
// the GPU, and there a 1024-thread workgroup waited for 16 free wave slots on
// one CU for 13 to 612 us (MI355X, the MoE step), where a 256-thread one
// takes the first slot a permute workgroup frees.
#ifndef COLL_EXPERT_TABLE_THREADS
#define COLL_EXPERT_TABLE_THREADS 256
#endif
constexpr int kTableThreads = COLL_EXPERT_TABLE_THREADS;
static_assert(kTableThreads >= COLL_MAX_RANKS * COLL_MAX_RANKS && kTableThreads <= 1024 &&
                  kTableThreads % 64 == 0,
              "one thread per (d, s) block, at most 16 waves");

__global__ __launch_bounds__(kTableThreads) void moe_expert_table(const int32_t *expert_counts,
                                                         const int64_t *rdispls, int R, int E,
                                                         RankRows recv_rows, int64_t *s_end,
                                                         int64_t *rb) {
  // a negative count, in the first scan: above any sum of non-negative int32
  // counts over 2^14 entries (< 2^45), and 2^14 of them still fit in int64
  constexpr int64_t kNeg = (int64_t)1 << 46;
  __shared__ int64_t wsum[16];
  __shared__ int64_t first_end[COLL_MAX_RANKS * COLL_MAX_RANKS];   // rows before (d, s)
  __shared__ int64_t s_b1[COLL_MAX_RANKS * COLL_MAX_RANKS];        // scan after (d, s)
  __shared__ int s_ok[COLL_MAX_RANKS * COLL_MAX_RANKS];
  __shared__ int s_bad;
  const int per = E / R;
  const int N = R * E;
  const int chunk = (N + kTableThreads - 1) / kTableThreads;   // <= 2^14 / kTableThreads
  const int j0 = (int)threadIdx.x * chunk;
  // 1. the scan of the counts (a negative one as kNeg) is the table when every
  //    block fits, the usual case; it also gives each block's total (and
  //    whether it holds a negative count) from the scan before its first and
  //    after its last entry.  Counts are re-read in each loop (L2 hits):
  //    keeping them in registers spilled to scratch at 1024 threads.
  int64_t local = 0;
  for (int c = 0; c < chunk; c++) {
    if (j0 + c >= N) break;
    const int64_t v = entry_count(expert_counts, E, per, j0 + c);
    local += v < 0 ? kNeg : v;
  }
  int64_t run = table_scan(local, wsum);
  for (int c = 0; c < chunk; c++) {
    const int j = j0 + c;
    if (j >= N) break;
    const int d = j / E, rem = j - d * E, s = rem / per, el = rem - s * per;
    if (el == 0) first_end[d * R + s] = run;
    const int64_t v = entry_count(expert_counts, E, per, j);
    run += v < 0 ? kNeg : v;
    s_end[j] = run;
    if (el == per - 1) s_b1[d * R + s] = run;
  }
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  if ((int)threadIdx.x < R * R) {
    const int d = threadIdx.x / R, s = threadIdx.x - d * R;
    const int64_t sum = s_b1[threadIdx.x] - first_end[threadIdx.x];
    const bool ok = sum < kNeg && (sum == 0 || block_fits(sum, 0, rdispls[d * R + s],
                                                          INT64_MAX, pick_rows(recv_rows, d)));
    s_ok[threadIdx.x] = ok;
    if (!ok) s_bad = 1;
  }
  __syncthreads();
  if (s_bad) {
    // 2. a block does not fit: the table again, over the blocks that do
    auto kept = [&](int j) -> int64_t {
      const int d = j / E, s = (j - d * E) / per;
      return s_ok[d * R + s] ? entry_count(expert_counts, E, per, j) : 0;
    };
    local = 0;
    for (int c = 0; c < chunk; c++) {
      if (j0 + c >= N) break;
      local += kept(j0 + c);
    }
    run = table_scan(local, wsum);
    for (int c = 0; c < chunk; c++) {
      const int j = j0 + c;
      if (j >= N) break;
      const int d = j / E, rem = j - d * E, s = rem / per, el = rem - s * per;
      if (el == 0) first_end[d * R + s] = run;
      run += kept(j);
      s_end[j] = run;
    }
    __syncthreads();
  }
  for (int c = 0; c < chunk; c++) {
    const int j = j0 + c;
    if (j >= N) break;
    const int d = j / E, s = (j - d * E) / per;
    rb[j] = rdispls[d * R + s] - first_end[d * R + s];
  }
}

// moe_expert_scale_kernel: one workgroup per tile of kBlock * UN units (G bf16
// elements each: 8 = 16-byte vectors, 1 = scalar fallback), looping when the
// grid is smaller than the work.  Each wave finds the entries of the tile's
// first and last rows with two 64-way searches over s_end, interleaved, one
// ballot per level (log64(N) levels).  The last level also loads each probed
// entry's bounds and receive base, so the winner's come from a lane shuffle:
// two dependent L2 round trips before the data loads, the row total loading
// beside the first.  A unit whose row is past the first entry bisects between
// the two.  Every unit of the tile is located, then all loads issue, then the
// scaled values are stored.
template <int G, bool NT>
__global__ __launch_bounds__(kExpertBlock) void moe_expert_scale_kernel(MutPtrTable recv, int R, int E,
                                                                  const int64_t *s_end,
                                                                  const int64_t *rb, int top,
                                                                  FastDiv64 upr) {
  using U = typename std::conditional<G == 8, u32x4, uint16_t>::type;
  constexpr int UN = kExpertU;
  const int per = E / R;
  const int N = R * E;
  const int lane = threadIdx.x & 63;
  // the row total is loaded on the vector path, so it completes beside the
  // first search level instead of being awaited first (an opaque index keeps
  // the compiler from turning it into a scalar load)
  int last = N - 1;
  COLL_OPAQUE(last);
  const int64_t nrows = s_end[last];
  const uint64_t tile = (uint64_t)kExpertBlock * UN;
  for (uint64_t t0 = (uint64_t)blockIdx.x * tile;; t0 += (uint64_t)gridDim.x * tile) {
    // lo(g) = number of entries with s_end <= g = the entry holding row g;
    // rows past the total search to N and are never used
    const int64_t g_first = (int64_t)fdiv64(t0, upr);
    const int64_t g_last = (int64_t)fdiv64(t0 + tile - 1, upr);
    int lo_f = 0, lo_l = 0;
    // probes past the table read its last entry and are discarded: loads
    // under a condition made the compiler wait for each one separately
    for (int stride = top; stride > 1; stride >>= 6) {
      const int jf = lo_f + (lane + 1) * stride - 1;
      const int jl = lo_l + (lane + 1) * stride - 1;
      const int64_t vf = s_end[jf < N ? jf : N - 1];
      const int64_t vl = s_end[jl < N ? jl : N - 1];
      lo_f += (int)__popcll(__ballot(jf < N && vf <= g_first)) * stride;
      lo_l += (int)__popcll(__ballot(jl < N && vl <= g_last)) * stride;
    }
    const int jf = lo_f + lane, jl = lo_l + lane;
    const int jc = jf < N ? jf : N - 1;
    const int64_t e_f = s_end[jc], p_f = s_end[jc > 0 ? jc - 1 : 0], r_f = rb[jc];
    const int64_t vl = s_end[jl < N ? jl : N - 1];
    const int64_t end_f = jf < N ? e_f : INT64_MAX;
    const int64_t beg_f = (jf < N && jf > 0) ? p_f : 0;
    const int64_t rb_f = jf < N ? r_f : 0;
    const bool inl = jl < N && vl <= g_last;
    // all last-level loads and the row total complete here, in one round
    // trip (without this the compiler sank two of the loads below the exit
    // test and hoisted the total's product, and so its wait, out of the loop)
    int64_t nr = nrows;
    COLL_OPAQUE(nr);
    COLL_KEEP(beg_f);
    COLL_KEEP(rb_f);
    const int cf = (int)__popcll(__ballot(end_f <= g_first));
    lo_l += (int)__popcll(__ballot(inl));
    if (t0 >= (uint64_t)nr * upr.d) break;
    lo_f += cf;                                   // < N: g_first is a real row
    if (lo_l > N - 1) lo_l = N - 1;
    // the lane's current entry, decoded once: rows [glo, ghi), receive row
    // rbase + g of rank d, scaled by `scale`
    int cur = lo_f;
    int64_t glo = __shfl(beg_f, cf, 64), ghi = __shfl(end_f, cf, 64), rbase = __shfl(rb_f, cf, 64);
    int d = cur / E;
    float scale = 1.0f + (float)(d * per + (cur - d * E) % per) / 256.0f;
    const uint64_t total = (uint64_t)nr * upr.d;
    U *at[UN];
    float sc[UN];
#pragma unroll
    for (int u = 0; u < UN; u++) {
      const uint64_t x = t0 + threadIdx.x + (uint64_t)u * kExpertBlock;
      at[u] = nullptr;
      if (x >= total) continue;
      const int64_t g = (int64_t)fdiv64(x, upr);
      if (g < glo || g >= ghi) {
        int a = lo_f, b = lo_l;                   // the entry is in [a, b]
        while (a < b) {
          const int m = (a + b) >> 1;
          if (s_end[m] <= g) a = m + 1;
          else b = m;
        }
        cur = a;
        glo = cur > 0 ? s_end[cur - 1] : 0;
        ghi = s_end[cur];
        rbase = rb[cur];
        d = cur / E;
        scale = 1.0f + (float)(d * per + (cur - d * E) % per) / 256.0f;
      }
      // receive unit = (rbase + g) * upr + (x - g * upr) = rbase * upr + x
      at[u] = reinterpret_cast<U *>(recv.p[d]) + (int64_t)x + rbase * (int64_t)upr.d;
      sc[u] = scale;
    }
    U v[UN];
#pragma unroll
    for (int u = 0; u < UN; u++)
      if (at[u]) v[u] = NT ? __builtin_nontemporal_load(at[u]) : *at[u];
#pragma unroll
    for (int u = 0; u < UN; u++) {
      if (!at[u]) continue;
      if constexpr (G == 8) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; q++)
          o[q] = pack_bf16(bf16_lo(v[u][q]) * sc[u], bf16_hi(v[u][q]) * sc[u]);
        if constexpr (NT) __builtin_nontemporal_store(o, at[u]);
        else *at[u] = o;
      } else {
        *at[u] = (uint16_t)(pack_bf16(bf16_lo((uint32_t)v[u]) * sc[u], 0.0f) & 0xFFFFu);
      }
    }
  }
}

// ------------------------------------------------ test expert, row descriptors
// The path for 16-byte rows with a known capacity.  A resident pre-kernel
// writes one 8-byte descriptor per receive row of the capacity: the unit
// address of the row's first unit (low kRowAddrBits) and its expert (high
// bits); 0 for a row past the total.  The main kernel then runs one wave per
// (row, 64-unit segment), and each wave starts with one scalar load of its
// row's descriptor: no search.  MI355X, the 3.5 GiB MoE receive rows in
// place: one-wave 1 KiB tiles ran at 6.78 TB/s in a standalone probe, against
// 5.42 TB/s for 256 lanes x 8 units.
constexpr int kRowAddrBits = 54;                  // unit addresses: byte addresses below 2^58
constexpr uint64_t kRowAddrMask = (1ull << kRowAddrBits) - 1;
constexpr int kRowTableMax = 8192;                // entries (R * E) staged in LDS: 64 KiB
static_assert(kMoeMaxExperts <= (1 << (64 - kRowAddrBits)), "an expert id must fit its field");

__global__ __launch_bounds__(kBlock) void moe_expert_rows(const int64_t *s_end, const int64_t *rb,
                                                         int R, int E, MutPtrTable recv,
                                                         uint64_t upr, uint64_t cap,
                                                         uint64_t *rdesc) {
  __shared__ int64_t t_end[kRowTableMax];
  const int N = R * E, per = E / R;
  for (int j = threadIdx.x; j < N; j += kBlock) t_end[j] = s_end[j];
  __syncthreads();
  const int64_t total = t_end[N - 1];
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  for (uint64_t g = (uint64_t)blockIdx.x * kBlock + threadIdx.x; g < cap; g += stride) {
    uint64_t dd = 0;
    if ((int64_t)g < total) {
      int lo = 0;                                 // entries ending at or before row g
      for (int step = kRowTableMax; step > 0; step >>= 1) {
        const int c = lo + step;
        if (c <= N && t_end[c - 1] <= (int64_t)g) lo = c;
      }
      const int d = lo / E;
      const int e = d * per + (lo - d * E) % per;
      const uint64_t unit = reinterpret_cast<uintptr_t>(recv.p[d]) / 16 +
                            (uint64_t)(rb[lo] + (int64_t)g) * upr;
      dd = (unit & kRowAddrMask) | ((uint64_t)e << kRowAddrBits);
    }
    rdesc[g] = dd;
  }
}

// y = rne(x * (1 + e/256)) on the 16-byte unit at unit address `unit`.
template <bool NT>
__device__ __forceinline__ void expert_unit(uint64_t unit, int e) {
  const float sc = 1.0f + (float)e / 256.0f;
  u32x4 v;
  if constexpr (NT) v = __builtin_nontemporal_load(gconst<u32x4>(unit * 16));
  else v = *gconst<u32x4>(unit * 16);
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; q++) o[q] = pack_bf16(bf16_lo(v[q]) * sc, bf16_hi(v[q]) * sc);
  if constexpr (NT) __builtin_nontemporal_store(o, gmut<u32x4>(unit * 16));
  else *gmut<u32x4>(unit * 16) = o;
}

// One 64-lane workgroup per (row, segment): the grid is exactly cap * nseg.
// Rows past the capacity (a bound below the rows received) are looped over,
// each located by a binary search of the entry table.
template <bool NT>
__global__ __launch_bounds__(64) void moe_expert_row_kernel(const uint64_t *__restrict__ rdesc,
                                                           const int64_t *__restrict__ s_end,
                                                           const int64_t *__restrict__ rb,
                                                           MutPtrTable recv, int R, int E,
                                                           uint32_t upr, uint32_t nseg,
                                                           FastDiv64 fseg, uint64_t cap) {
  const uint32_t row = (uint32_t)fdiv64(blockIdx.x, fseg);
  const uint32_t seg = blockIdx.x - row * nseg;
  const int N = R * E;
  uint64_t dd = rdesc[row];
  int64_t nrows = s_end[N - 1];
  COLL_UNIFORM(dd);                               // both through the scalar cache, together
  COLL_UNIFORM(nrows);
  if (dd == 0) return;                            // past the total
  const uint32_t u = seg * 64 + threadIdx.x;
  if (u < upr) expert_unit<NT>((dd & kRowAddrMask) + u, (int)(uint32_t)(dd >> kRowAddrBits));
  if ((uint64_t)nrows <= cap) return;
  const int per = E / R;
  for (uint64_t g = row + cap; g < (uint64_t)nrows; g += cap) {
    int lo = 0;                                   // entries ending at or before row g
    for (int step = kRowTableMax * 2; step > 0; step >>= 1) {
      const int c = lo + step;
      if (c <= N && s_end[c - 1] <= (int64_t)g) lo = c;
    }
    const int d = lo / E;
    const int e = d * per + (lo - d * E) % per;
    const uint64_t unit = reinterpret_cast<uintptr_t>(recv.p[d]) / 16 +
                          (uint64_t)(rb[lo] + (int64_t)g) * upr;
    if (u < upr) expert_unit<NT>(unit + u, e);
  }
}

// ------------------------------------------------------------------ combine

// One wave per (token, segment of 64 x UN units); its K slots and weights
// are scalar loads, all K x UN gathered loads issue before the fold.  A slot
// outside [0, T*K) -- the layout's -1 for a pair with no expert -- adds no
// term: the fold runs over the token's other pairs in order, seeded by the
// first of them (+0 if none is left).  Slots are wave-uniform, so this never
// diverges.
template <int G, bool NT>
__global__ __launch_bounds__(64 * kCombineWaves) void moe_combine_kernel(PtrTable back, PtrTable pos,
                                                             PtrTable wts, MutPtrTable out,
                                                             int T, int K, uint32_t upr,
                                                             int nseg) {
  constexpr int kChunk = 8;                    // gathered rows in flight per unit
  constexpr int UN = (G == 8) ? kCombineU : 1;
  const RowItem it = row_item<kCombineWaves>(T, nseg);
  if (!it.valid) return;
  const uint32_t TK = (uint32_t)T * (uint32_t)K;
  const int s = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const uint16_t *bk = reinterpret_cast<const uint16_t *>(back.p[s]);
  const int32_t *pk = reinterpret_cast<const int32_t *>(pos.p[s]) + (size_t)it.t * K;
  const float *wk = reinterpret_cast<const float *>(wts.p[s]) + (size_t)it.t * K;
  uint16_t *o = reinterpret_cast<uint16_t *>(out.p[s]);
  const uint32_t u0 = (uint32_t)it.seg * (64 * UN) + lane;
  if constexpr (G == 8) {
    float acc[UN][8];
    bool have = false;                                   // a term has seeded acc
    for (int k0 = 0; k0 < K; k0 += kChunk) {
      uint32_t slot[kChunk];
      float wgt[kChunk];
      bool live[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; c++) {
        const int kc = k0 + c < K ? k0 + c : K - 1;         // past K: used by nothing
        const int32_t p = __builtin_amdgcn_readfirstlane(pk[kc]);
        live[c] = k0 + c < K && (uint32_t)p < TK;
        slot[c] = live[c] ? (uint32_t)p : 0u;
        wgt[c] = __builtin_bit_cast(
            float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wk[kc])));
      }
      u32x4 v[UN][kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; c++) {
        if (live[c]) {
          const uint16_t *row = bk + (size_t)slot[c] * upr * 8;
#pragma unroll
          for (int uu = 0; uu < UN; uu++) {
            const uint32_t u = u0 + uu * 64;
            if (u < upr) v[uu][c] = ld<u32x4, NT>(row, u);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < kChunk; c++) {
        if (live[c]) {
#pragma unroll
          for (int uu = 0; uu < UN; uu++) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
              const float lo = wgt[c] * bf16_lo(v[uu][c][q]);
              const float hi = wgt[c] * bf16_hi(v[uu][c][q]);
              if (!have) { acc[uu][2 * q] = lo; acc[uu][2 * q + 1] = hi; }
              else { acc[uu][2 * q] = acc[uu][2 * q] + lo; acc[uu][2 * q + 1] = acc[uu][2 * q + 1] + hi; }
            }
          }
          have = true;
        }
      }
    }
#pragma unroll
    for (int uu = 0; uu < UN; uu++) {
      const uint32_t u = u0 + uu * 64;
      if (u < upr) {
        u32x4 r;
#pragma unroll
        for (int q = 0; q < 4; q++)
          r[q] = have ? pack_bf16(acc[uu][2 * q], acc[uu][2 * q + 1]) : 0u;
        st<u32x4, NT>(o + (size_t)it.t * upr * 8, u, r);
      }
    }
  } else {
    const uint32_t u = u0;
    if (u < upr) {
      float acc = 0.0f;
      bool have = false;
      for (int k = 0; k < K; k++) {
        const int32_t p = __builtin_amdgcn_readfirstlane(pk[k]);
        if ((uint32_t)p >= TK) continue;                 // a pair with no expert
        const float prod = wk[k] * bf16_lo(bk[(size_t)p * upr + u]);
        acc = have ? acc + prod : prod;
        have = true;
      }
      o[(size_t)it.t * upr + u] = (uint16_t)(pack_bf16(acc, 0.0f) & 0xFFFFu);
    }
  }
}

// ------------------------------------------------- fused dispatch / combine

// The send blocks of source s (its row of the layout), staged in LDS once per
// workgroup: send slots [lo[d], hi[d]) go to rank d, whose receive rows start
// at rd[d].  A slot's destination is found by a wave-uniform scan over d.
// The fused dispatch (4 waves per workgroup) stages its source's blocks in
// LDS once per workgroup; scanning them per slot measured faster there than
// per-wave lane copies (761 against 807 us at the MoE shape).
struct SrcBlocks {
  int64_t lo[COLL_MAX_RANKS];
  int64_t hi[COLL_MAX_RANKS];
  int64_t rd[COLL_MAX_RANKS];
};

// A block whose receive rows do not all lie inside rank d's buffer (recv_rows)
// is staged empty: its slots are then held by no block and not written.
__device__ __forceinline__ void load_src_blocks(SrcBlocks &b, int R, int s,
                                                const int64_t *sendcounts,
                                                const int64_t *sdispls,
                                                const int64_t *rdispls,
                                                const RankRows &recv_rows) {
  if ((int)threadIdx.x < R) {
    const int d = threadIdx.x;
    const int64_t a = sdispls[s * R + d], c = sendcounts[s * R + d], r = rdispls[d * R + s];
    const bool ok = block_fits(c, a, r, INT64_MAX, pick_rows(recv_rows, d));
    b.lo[d] = ok ? a : 1;
    b.hi[d] = ok ? a + c : 0;
    b.rd[d] = r;
  }
  __syncthreads();
}

// Receive row of send slot `slot` of the staged source; d = -1 when no block
// holds it (only a corrupt layout does that).
__device__ __forceinline__ int64_t recv_row_of(const SrcBlocks &b, int R, int64_t slot, int &d) {
  for (int q = 0; q < R; q++) {
    if (slot >= b.lo[q] && slot < b.hi[q]) {
      d = q;
      return b.rd[q] + (slot - b.lo[q]);
    }
  }
  d = -1;
  return 0;
}

// The fused combine and dispatch: lane q < R of a wave holds block q of
// source s: its send slots [lo, hi), the offset from a slot to its
// receive row (rdispls[q][s] - lo) and rank q's receive buffer; the other
// lanes hold an empty block.  Loaded per wave from clamped indices (no LDS,
// no barrier), so locating a slot is one ballot and two lane reads, with no
// memory access (the LDS scan waited on each read in turn, R reads per slot,
// then loaded the buffer pointer: 751-758 against 741-745 us at the MoE
// shape).
struct SrcLane {
  int64_t lo, hi, off;
  uint64_t base;
};

// (a block whose receive rows do not all lie inside rank q's buffer is held
// empty, as in load_src_blocks)
// 1: the fused dispatch locates slots like the fused combine (lane-held
// blocks, one ballot per slot) instead of scanning blocks staged in LDS
// (MI355X, the MoE shape: 785-787 against 792-800 us)
#ifndef COLL_DISPATCH_LANE
#define COLL_DISPATCH_LANE 1
#endif
#ifndef COLL_SRC_LANE_SCALAR
#define COLL_SRC_LANE_SCALAR 1
#endif
template <class Table>
__device__ __forceinline__ SrcLane load_src_lane(int R, int s, const Table &recv,
                                                 const int64_t *sendcounts,
                                                 const int64_t *sdispls,
                                                 const int64_t *rdispls,
                                                 const RankRows &recv_rows) {
  const int q = threadIdx.x & 63;
  const int qq = q < R ? q : 0;
#if COLL_SRC_LANE_SCALAR
  // The entries are the same for the whole workgroup (its source s): they
  // come in through the scalar cache, entry i pinned in scalar registers
  // (clamped index, so every load is unconditional), and lane q selects
  // entry q.  Loaded per lane, they were a vector round trip before any row
  // could be addressed.
  int64_t a = 0, c = 0, r = 0;
#pragma unroll
  for (int i = 0; i < COLL_MAX_RANKS; i++) {
    const int ii = i < R ? i : 0;
    int64_t ai = sdispls[s * R + ii], ci = sendcounts[s * R + ii], ri = rdispls[ii * R + s];
    COLL_SCALAR(ai);
    COLL_SCALAR(ci);
    COLL_SCALAR(ri);
    a = qq == i ? ai : a;
    c = qq == i ? ci : c;
    r = qq == i ? ri : r;
  }
#else
  const int64_t a = sdispls[s * R + qq], c = sendcounts[s * R + qq], r = rdispls[qq * R + s];
#endif
  const bool ok = q < R && block_fits(c, a, r, INT64_MAX, pick_rows(recv_rows, qq));
  SrcLane b;
  b.lo = ok ? a : 1;
  b.hi = ok ? a + c : 0;
  b.off = r - a;
#if COLL_SRC_LANE_SCALAR
  uint64_t base = 0;
#pragma unroll
  for (int i = 0; i < COLL_MAX_RANKS; i++) {
    uint64_t bi = reinterpret_cast<uintptr_t>(recv.p[i]);
    COLL_SCALAR(bi);
    base = qq == i ? bi : base;
  }
  b.base = base;
#else
  b.base = reinterpret_cast<uintptr_t>(recv.p[qq]);
#endif
  return b;
}


// The receive row of the wave-uniform send slot `slot` and its buffer
// (`base`, 0 for a rank that receives nothing); d = the first block holding
// the slot, -1 when none does (only a corrupt layout).  The whole wave must
// be active.
__device__ __forceinline__ int64_t recv_row_lane(const SrcLane &b, int64_t slot, int &d,
                                                 uint64_t &base) {
  const uint64_t m = __ballot(slot >= b.lo && slot < b.hi);
  if (m == 0) {
    d = -1;
    base = 0;
    return 0;
  }
  d = (int)__builtin_ctzll(m);
  base = readlane64(b.base, d);
  return slot + (int64_t)readlane64((uint64_t)b.off, d);
}

// recv[d][rdispls[d][s] + pos - sdispls[s][d]] = x[s][t] for every k: the
// permute and the exchange in one pass (each token row read once, written K
// times straight into its destination's receive buffer).
template <int B, bool NT>
__global__ __launch_bounds__(64 * kDispatchWaves) void moe_dispatch_kernel(
    PtrTable x, PtrTable pos, MutPtrTable recv, const int64_t *__restrict__ sendcounts,
    const int64_t *__restrict__ sdispls, const int64_t *__restrict__ rdispls, RankRows recv_rows,
    int R, int T, int K, uint32_t upr, int nseg) {
  using U = typename UnitT<B>::T;
  constexpr int UN = kPermuteU;
  const int s = blockIdx.y;
#if COLL_DISPATCH_LANE
  const RowItem it = row_item<kDispatchWaves>(T, nseg);
  if (!it.valid) return;
  const SrcLane bl = load_src_lane(R, s, recv, sendcounts, sdispls, rdispls, recv_rows);
#else
  __shared__ SrcBlocks blk;
  load_src_blocks(blk, R, s, sendcounts, sdispls, rdispls, recv_rows);
  const RowItem it = row_item<kDispatchWaves>(T, nseg);
  if (!it.valid) return;
#endif
  const int lane = threadIdx.x & 63;
  const U *src = reinterpret_cast<const U *>(x.p[s]) + (size_t)it.t * upr;
  const int32_t *pk = reinterpret_cast<const int32_t *>(pos.p[s]) + (size_t)it.t * K;
  const uint32_t u0 = (uint32_t)it.seg * (64 * UN) + lane;
  U v[UN];
#pragma unroll
  for (int u = 0; u < UN; u++) {
    const uint32_t x_u = u0 + u * 64;
    if (x_u < upr) v[u] = NT ? __builtin_nontemporal_load(src + x_u) : src[x_u];
  }
  for (int k0 = 0; k0 < K; k0 += kSlotChunk) {
    int32_t sl[kSlotChunk];
#pragma unroll
    for (int c = 0; c < kSlotChunk; c++)
      // through the scalar cache: 778-781 against 786-789 us with vector loads
      sl[c] = ld_scalar(pk, (size_t)(k0 + c < K ? k0 + c : K - 1));
#pragma unroll
    for (int c = 0; c < kSlotChunk; c++) {
      if (k0 + c >= K) break;
      int d;
#if COLL_DISPATCH_LANE
      uint64_t bp;
      const int64_t row = recv_row_lane(bl, sl[c], d, bp);
      if (d < 0 || bp == 0) continue;     // no block holds the slot / a rank receiving nothing
      U *base = reinterpret_cast<U *>(bp);
#else
      const int64_t row = recv_row_of(blk, R, sl[c], d);
      if (d < 0) continue;                                   // never write outside
      U *base = reinterpret_cast<U *>(recv.p[__builtin_amdgcn_readfirstlane(d)]);
      if (!base) continue;                                   // a rank that receives nothing
#endif
      U *dst = base + (size_t)row * upr;
#pragma unroll
      for (int u = 0; u < UN; u++) {
        const uint32_t x_u = u0 + u * 64;
        if (x_u < upr) {
          if constexpr (NT) __builtin_nontemporal_store(v[u], dst + x_u);
          else dst[x_u] = v[u];
        }
      }
    }
  }
}

// out[s][t] = rne(fold_k w[t,k] * widen(y_k)), y_k the receive row of (s,t,k)
// (the reverse exchange is a read of the destination's buffer).  EXPERT: y_k
// = rne(widen(row) * (1 + e/256)) with e = ids[s][t,k], the test expert applied
// as the row is read.  A slot that no block holds (the layout's -1 for a pair
// with no expert) adds no term, as in the unfused combine.
template <int G, bool NT, bool EXPERT>
__global__ __launch_bounds__(64 * kCombineRecvWaves) void moe_combine_recv_kernel(
    PtrTable recv, PtrTable pos, PtrTable wts, PtrTable ids, MutPtrTable out,
    const int64_t *__restrict__ sendcounts, const int64_t *__restrict__ sdispls,
    const int64_t *__restrict__ rdispls, RankRows recv_rows, int R, int T, int K, uint32_t upr,
    int nseg) {
  constexpr int kChunk = 8;
  constexpr int UN = (G == 8) ? kCombineRecvU : 1;
  const int s = blockIdx.y;
  const RowItem it = row_item<kCombineRecvWaves>(T, nseg);
  if (!it.valid) return;
  const SrcLane bl = load_src_lane(R, s, recv, sendcounts, sdispls, rdispls, recv_rows);
  const int lane = threadIdx.x & 63;
  const int32_t *pk = reinterpret_cast<const int32_t *>(pos.p[s]) + (size_t)it.t * K;
  const float *wk = reinterpret_cast<const float *>(wts.p[s]) + (size_t)it.t * K;
  const int32_t *ek = EXPERT ? reinterpret_cast<const int32_t *>(ids.p[s]) + (size_t)it.t * K
                             : nullptr;
  uint16_t *o = reinterpret_cast<uint16_t *>(out.p[s]);
  const uint32_t u0 = (uint32_t)it.seg * (64 * UN) + lane;
  if constexpr (G == 8) {
    float acc[UN][8];
    bool have = false;                                   // a term has seeded acc
    for (int k0 = 0; k0 < K; k0 += kChunk) {
      const uint16_t *rowp[kChunk];
      float wgt[kChunk], sc[kChunk];
      bool live[kChunk];
      int32_t sl[kChunk], ev[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; c++) {
        const int kc = k0 + c < K ? k0 + c : K - 1;         // past K: used by nothing
        sl[c] = __builtin_amdgcn_readfirstlane(pk[kc]);
        wgt[c] = __builtin_bit_cast(
            float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wk[kc])));
        ev[c] = EXPERT ? __builtin_amdgcn_readfirstlane(ek[kc]) : 0;
      }
#pragma unroll
      for (int c = 0; c < kChunk; c++) {
        rowp[c] = nullptr;
        sc[c] = 1.0f;
        live[c] = false;
        if (k0 + c < K) {
          int d;
          uint64_t bp;
          const int64_t row = recv_row_lane(bl, sl[c], d, bp);
          live[c] = d >= 0 && bp != 0;
          if (live[c]) rowp[c] = reinterpret_cast<const uint16_t *>(bp) + (size_t)row * upr * 8;
          if constexpr (EXPERT) sc[c] = 1.0f + (float)ev[c] / 256.0f;
        } else {
          wgt[c] = 0.0f;
        }
      }
      u32x4 v[UN][kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; c++) {
#pragma unroll
        for (int uu = 0; uu < UN; uu++) {
          const uint32_t u = u0 + uu * 64;
          v[uu][c] = u32x4{0u, 0u, 0u, 0u};
          if (live[c] && u < upr) v[uu][c] = ld<u32x4, NT>(rowp[c], u);
        }
      }
#pragma unroll
      for (int c = 0; c < kChunk; c++) {
        if (live[c]) {
#pragma unroll
          for (int uu = 0; uu < UN; uu++) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
              uint32_t y = v[uu][c][q];
              if constexpr (EXPERT) y = pack_bf16(bf16_lo(y) * sc[c], bf16_hi(y) * sc[c]);
              const float lo = wgt[c] * bf16_lo(y);
              const float hi = wgt[c] * bf16_hi(y);
              if (!have) { acc[uu][2 * q] = lo; acc[uu][2 * q + 1] = hi; }
              else { acc[uu][2 * q] = acc[uu][2 * q] + lo; acc[uu][2 * q + 1] = acc[uu][2 * q + 1] + hi; }
            }
          }
          have = true;
        }
      }
    }
#pragma unroll
    for (int uu = 0; uu < UN; uu++) {
      const uint32_t u = u0 + uu * 64;
      if (u < upr) {
        u32x4 r;
#pragma unroll
        for (int q = 0; q < 4; q++)
          r[q] = have ? pack_bf16(acc[uu][2 * q], acc[uu][2 * q + 1]) : 0u;
        st<u32x4, NT>(o + (size_t)it.t * upr * 8, u, r);
      }
    }
  } else {
    const uint32_t u = u0;
    const bool in = u < upr;
    {
      float acc = 0.0f;
      bool have = false;
      for (int k = 0; k < K; k++) {
        int d;                                     // located with the whole wave active
        uint64_t bp;
        const int64_t row = recv_row_lane(bl, __builtin_amdgcn_readfirstlane(pk[k]), d, bp);
        if (d < 0 || bp == 0) continue;            // no block holds the slot: no term
        uint32_t y = 0u;
        if (in) y = reinterpret_cast<const uint16_t *>(bp)[(size_t)row * upr + u];
        if constexpr (EXPERT) {
          const float sc = 1.0f + (float)__builtin_amdgcn_readfirstlane(ek[k]) / 256.0f;
          y = pack_bf16(bf16_lo(y) * sc, 0.0f) & 0xFFFFu;
        }
        const float prod = wk[k] * bf16_lo(y);
        acc = have ? acc + prod : prod;
        have = true;
      }
      if (in) o[(size_t)it.t * upr + u] = (uint16_t)(pack_bf16(acc, 0.0f) & 0xFFFFu);
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
  hipLaunchKernelGGL(moe_scan, dim3(R), dim3(1024), 0, L.stream, R, E, ntiles, hist,
                     expert_off, expert_counts, sendcounts, sdispls);
  hipLaunchKernelGGL(moe_pos, dim3(ntiles > 0 ? ntiles : 1, R), dim3(kBlock), 0, L.stream, ids,
                     pos, R, TK, E, nbits, ntiles, hist, expert_off, sendcounts, rdispls);
  return hip_status();
}

// ------------------------------------------------- layout without a workspace
// The layout's scratch for callers that cannot allocate: a device array of
// kMoeStaticBytes that each GPU holds for the life of the process.  In host
// code `moe_scratch` names a host-side stand-in, not device memory, so its
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is passed to kernels.  Every
// call on a GPU shares its array: calls that overlap on one GPU race, and
// nothing in it needs clearing (the histogram kernel writes every count the
// later kernels read).
namespace {
static __device__ __align__(256) unsigned char moe_scratch[kMoeStaticBytes];
constexpr int kMaxScratchDevices = 64;
void *g_moe_scratch[kMaxScratchDevices];
}  // namespace

void *moe_static_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  void *p = __atomic_load_n(&g_moe_scratch[dev], __ATOMIC_ACQUIRE);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(moe_scratch)) != hipSuccess || !p) return nullptr;
    __atomic_store_n(&g_moe_scratch[dev], p, __ATOMIC_RELEASE);
  }
  return p;
}

int launch_moe_permute(const Launch &L, int R, const PtrTable &x, const PtrTable &pos, int T,
                       int K, size_t row_bytes, const MutPtrTable &send) {
  uintptr_t bits = row_bytes;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)x.p[r] | (uintptr_t)send.p[r];
  const int unit = copy_unit(bits);
  const uint64_t upr = row_bytes / unit;
  if (T == 0 || upr == 0) return COLL_OK;
  if (upr >= (1ull << 31)) return COLL_ERR_UNSUPPORTED;
  const int nseg = (int)((upr + 64 * kPermuteU - 1) / (64 * kPermuteU));
  const uint64_t items = (uint64_t)T * nseg;
  if (items >= (1ull << 31) - 4) return COLL_ERR_UNSUPPORTED;
  const bool nt = (uint64_t)R * T * upr * unit * (1 + K) >= L.nt_bytes;
  dim3 grid((unsigned)((items + kPermuteWaves - 1) / kPermuteWaves), R);
  COLL_UNIT_SWITCH_BLOCK(moe_permute_kernel, unit, nt, grid, 64 * kPermuteWaves, L.stream, x, pos, send, T, K,
                   (uint32_t)upr, nseg);
  return hip_status();
}

// The row-descriptor path applies: 16-byte units, a known capacity, a
// workspace that holds the descriptors, a table that fits in LDS, buffers
// inside the descriptors' address range and a grid of at most 2^31 - 1
// workgroups.  Sets vec (rows move in 16-byte units), upr (units per row)
// and nseg (64-unit segments per row).
static bool expert_rows_apply(int R, const MutPtrTable &recv, int E, size_t hidden,
                              size_t rows_capacity, size_t ws_bytes, bool &vec, uint64_t &upr,
                              uint64_t &nseg) {
  vec = (hidden % 8) == 0;
  uintptr_t top_addr = 0;
  for (int r = 0; r < R; r++) {
    vec = vec && aligned16(recv.p[r]);
    top_addr |= (uintptr_t)recv.p[r];
  }
  upr = vec ? hidden / 8 : hidden;
  nseg = (upr + 63) / 64;
  return vec && rows_capacity > 0 && ws_bytes >= moe_expert_workspace_bytes(R, E, rows_capacity) &&
         R * E <= kRowTableMax && (top_addr >> (kRowAddrBits + 3)) == 0 &&
         rows_capacity * nseg <= 0x7FFFFFFFull;
}

bool moe_expert_rows_apply(int R, const MutPtrTable &recv, int E, size_t hidden,
                           size_t rows_capacity, size_t ws_bytes) {
  bool vec;
  uint64_t upr, nseg;
  return expert_rows_apply(R, recv, E, hidden, rows_capacity, ws_bytes, vec, upr, nseg);
}

// First half of the row-descriptor path: the row-prefix table, then one
// descriptor per receive row of the capacity.  Reads only the count tables
// and the buffers' addresses, so it may run before the rows arrive.
int launch_moe_expert_build(const Launch &L, int R, const MutPtrTable &recv,
                            const int32_t *expert_counts, const int64_t *rdispls, int E,
                            size_t hidden, size_t rows_capacity, void *ws, size_t ws_bytes,
                            const RankRows &recv_rows) {
  bool vec;
  uint64_t upr, nseg;
  if (!expert_rows_apply(R, recv, E, hidden, rows_capacity, ws_bytes, vec, upr, nseg))
    return COLL_ERR_UNSUPPORTED;
  const int N = R * E;
  int64_t *s_end = reinterpret_cast<int64_t *>(ws);
  int64_t *rb = s_end + N;
  hipLaunchKernelGGL(moe_expert_table, dim3(1), dim3(kTableThreads), 0, L.stream, expert_counts, rdispls,
                     R, E, recv_rows, s_end, rb);
  uint64_t *rdesc =
      reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + moe_expert_table_bytes(R, E));
  const uint64_t gneed = (rows_capacity + kBlock - 1) / kBlock;
  const uint64_t gres = (uint64_t)L.num_cus * 2;   // 64 KiB of LDS each: two per CU
  hipLaunchKernelGGL(moe_expert_rows, dim3((unsigned)(gneed < gres ? gneed : gres)), dim3(kBlock),
                     0, L.stream, s_end, rb, R, E, recv, upr, (uint64_t)rows_capacity, rdesc);
  return hip_status();
}

// Second half: one 64-lane workgroup per (row, segment) of the capacity.
int launch_moe_expert_apply(const Launch &L, int R, const MutPtrTable &recv, int E, size_t hidden,
                            size_t rows_capacity, void *ws, size_t ws_bytes) {
  bool vec;
  uint64_t upr, nseg;
  if (!expert_rows_apply(R, recv, E, hidden, rows_capacity, ws_bytes, vec, upr, nseg))
    return COLL_ERR_UNSUPPORTED;
  const int64_t *s_end = reinterpret_cast<const int64_t *>(ws);
  const int64_t *rb = s_end + R * E;
  const uint64_t *rdesc = reinterpret_cast<const uint64_t *>(static_cast<const char *>(ws) +
                                                             moe_expert_table_bytes(R, E));
  const FastDiv64 fs = make_fastdiv64(nseg);
  const unsigned g = (unsigned)(rows_capacity * nseg);
  if (L.a2a_nt)
    hipLaunchKernelGGL((moe_expert_row_kernel<true>), dim3(g), dim3(64), 0, L.stream, rdesc, s_end,
                       rb, recv, R, E, (uint32_t)upr, (uint32_t)nseg, fs, (uint64_t)rows_capacity);
  else
    hipLaunchKernelGGL((moe_expert_row_kernel<false>), dim3(g), dim3(64), 0, L.stream, rdesc,
                       s_end, rb, recv, R, E, (uint32_t)upr, (uint32_t)nseg, fs,
                       (uint64_t)rows_capacity);
  return hip_status();
}

int launch_moe_expert_scale(const Launch &L, int R, const MutPtrTable &recv,
                            const int32_t *expert_counts, const int64_t *rdispls, int E,
                            size_t hidden, size_t rows_capacity, void *ws, size_t ws_bytes,
                            const RankRows &recv_rows) {
  bool vec;
  uint64_t upr, nseg;
  if (expert_rows_apply(R, recv, E, hidden, rows_capacity, ws_bytes, vec, upr, nseg)) {
    const int rc = launch_moe_expert_build(L, R, recv, expert_counts, rdispls, E, hidden,
                                           rows_capacity, ws, ws_bytes, recv_rows);
    if (rc != COLL_OK) return rc;
    return launch_moe_expert_apply(L, R, recv, E, hidden, rows_capacity, ws, ws_bytes);
  }
  const int N = R * E;
  int64_t *s_end = reinterpret_cast<int64_t *>(ws);
  int64_t *rb = s_end + N;
  hipLaunchKernelGGL(moe_expert_table, dim3(1), dim3(kTableThreads), 0, L.stream, expert_counts, rdispls,
                     R, E, recv_rows, s_end, rb);
  int top = 1;
  while (top * 64 < N) top *= 64;
  // the table-search path: one workgroup per tile of the capacity; with no
  // capacity, a resident grid (the kernel loops over tiles either way)
  const size_t tile = (size_t)kExpertBlock * kExpertU;
  const size_t cap_units = rows_capacity * upr;
  size_t g = rows_capacity ? (cap_units + tile - 1) / tile : grid_resident(L);
  if (g < 1) g = 1;
  if (g > 0x7FFFFFFFu) g = 0x7FFFFFFFu;
  const FastDiv64 f = make_fastdiv64(upr);
  const bool nt = L.a2a_nt != 0;
  if (vec) {
    if (nt)
      hipLaunchKernelGGL((moe_expert_scale_kernel<8, true>), dim3((unsigned)g), dim3(kExpertBlock), 0,
                         L.stream, recv, R, E, s_end, rb, top, f);
    else
      hipLaunchKernelGGL((moe_expert_scale_kernel<8, false>), dim3((unsigned)g), dim3(kExpertBlock), 0,
                         L.stream, recv, R, E, s_end, rb, top, f);
  } else {
    hipLaunchKernelGGL((moe_expert_scale_kernel<1, false>), dim3((unsigned)g), dim3(kExpertBlock), 0,
                       L.stream, recv, R, E, s_end, rb, top, f);
  }
  return hip_status();
}

int launch_moe_combine(const Launch &L, int R, const PtrTable &back, const PtrTable &pos,
                       const PtrTable &w, int T, int K, size_t hidden, const MutPtrTable &out) {
  bool vec = (hidden % 8) == 0;
  for (int r = 0; r < R; r++) vec = vec && aligned16(back.p[r]) && aligned16(out.p[r]);
  if (T == 0) return COLL_OK;
  const uint64_t upr = vec ? hidden / 8 : hidden;
  const int per_seg = vec ? 64 * kCombineU : 64;
  const int nseg = (int)((upr + per_seg - 1) / per_seg);
  const uint64_t items = (uint64_t)T * nseg;
  if (items >= (1ull << 31) - 4) return COLL_ERR_UNSUPPORTED;
  dim3 grid((unsigned)((items + kCombineWaves - 1) / kCombineWaves), R);
  const bool nt = (uint64_t)R * T * (K + 1) * hidden * 2 >= L.nt_bytes;
  if (vec) {
    if (nt)
      hipLaunchKernelGGL((moe_combine_kernel<8, true>), grid, dim3(64 * kCombineWaves), 0, L.stream, back, pos,
                         w, out, T, K, (uint32_t)upr, nseg);
    else
      hipLaunchKernelGGL((moe_combine_kernel<8, false>), grid, dim3(64 * kCombineWaves), 0, L.stream, back,
                         pos, w, out, T, K, (uint32_t)upr, nseg);
  } else {
    hipLaunchKernelGGL((moe_combine_kernel<1, false>), grid, dim3(64 * kCombineWaves), 0, L.stream, back, pos,
                       w, out, T, K, (uint32_t)upr, nseg);
  }
  return hip_status();
}

int launch_moe_dispatch(const Launch &L, int R, const PtrTable &x, const PtrTable &pos,
                        const int64_t *sendcounts, const int64_t *sdispls, const int64_t *rdispls,
                        int T, int K, size_t row_bytes, const MutPtrTable &recv,
                        const RankRows &recv_rows) {
  uintptr_t bits = row_bytes;
  for (int r = 0; r < R; r++) bits |= (uintptr_t)x.p[r] | (uintptr_t)recv.p[r];
  const int unit = copy_unit(bits);
  const uint64_t upr = row_bytes / unit;
  if (T == 0 || upr == 0) return COLL_OK;
  if (upr >= (1ull << 31)) return COLL_ERR_UNSUPPORTED;
  const int nseg = (int)((upr + 64 * kPermuteU - 1) / (64 * kPermuteU));
  const uint64_t items = (uint64_t)T * nseg;
  if (items >= (1ull << 31) - 4) return COLL_ERR_UNSUPPORTED;
  const bool nt = (uint64_t)R * T * upr * unit * (1 + K) >= L.nt_bytes;
  dim3 grid((unsigned)((items + kDispatchWaves - 1) / kDispatchWaves), R);
  COLL_UNIT_SWITCH_BLOCK(moe_dispatch_kernel, unit, nt, grid, 64 * kDispatchWaves, L.stream, x, pos, recv, sendcounts,
                   sdispls, rdispls, recv_rows, R, T, K, (uint32_t)upr, nseg);
  return hip_status();
}

int launch_moe_combine_recv(const Launch &L, int R, const PtrTable &recv, const PtrTable &pos,
                            const int64_t *sendcounts, const int64_t *sdispls,
                            const int64_t *rdispls, const PtrTable &w, const PtrTable *ids, int T,
                            int K, size_t hidden, const MutPtrTable &out,
                            const RankRows &recv_rows) {
  bool vec = (hidden % 8) == 0;
  for (int r = 0; r < R; r++) vec = vec && aligned16(recv.p[r]) && aligned16(out.p[r]);
  if (T == 0) return COLL_OK;
  const uint64_t upr = vec ? hidden / 8 : hidden;
  const int per_seg = vec ? 64 * kCombineRecvU : 64;
  const int nseg = (int)((upr + per_seg - 1) / per_seg);
  const uint64_t items = (uint64_t)T * nseg;
  if (items >= (1ull << 31) - 4) return COLL_ERR_UNSUPPORTED;
  dim3 grid((unsigned)((items + kCombineRecvWaves - 1) / kCombineRecvWaves), R);
  const bool nt = (uint64_t)R * T * (K + 1) * hidden * 2 >= L.nt_bytes;
  const PtrTable none{};
  const PtrTable &idt = ids ? *ids : none;
#define COLL_COMBINE_RECV(G, NTV, EX)                                                              \
  hipLaunchKernelGGL((moe_combine_recv_kernel<G, NTV, EX>), grid, dim3(64 * kCombineRecvWaves), 0, L.stream, recv, \
                     pos, w, idt, out, sendcounts, sdispls, rdispls, recv_rows, R, T, K,          \
                     (uint32_t)upr, nseg)
  if (vec && nt && ids) COLL_COMBINE_RECV(8, true, true);
  else if (vec && nt) COLL_COMBINE_RECV(8, true, false);
  else if (vec && ids) COLL_COMBINE_RECV(8, false, true);
  else if (vec) COLL_COMBINE_RECV(8, false, false);
  else if (ids) COLL_COMBINE_RECV(1, false, true);
  else COLL_COMBINE_RECV(1, false, false);
#undef COLL_COMBINE_RECV
  return hip_status();
}

}  // namespace coll
