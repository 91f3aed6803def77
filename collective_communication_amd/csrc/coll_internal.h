// coll_internal.h -- shared device helpers of libcoll (gfx950 only).
//
// Data model: R virtual ranks are R device pointers per buffer role, passed by
// value in the kernel arguments (RankPtrs).  On one GPU a "rank boundary" is
// only a pointer, so every primitive is a streaming HBM kernel: 16-byte
// (dwordx4) coalesced loads and stores, fp32 accumulation of narrow types in a
// fixed ascending rank order, and a grid-stride loop sized to the compute
// units for large messages or a single pass for small ones.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "coll.h"

namespace coll {

constexpr int kBlock = 256;   // threads per workgroup: 4 wave64s

struct RankPtrs {
  const void *in[COLL_MAX_RANKS];
  void *out[COLL_MAX_RANKS];
};

// Rows each rank's buffer holds, one table per buffer role of the exchange
// (in: read, out: written).  A block of an All-to-All-v moves only when all
// its rows lie inside both of its buffers; INT64_MAX marks a side the caller
// does not bound.  Passed by value (256 bytes), like RankPtrs.
struct RankRows {
  int64_t n[COLL_MAX_RANKS];
};
struct RowLimits {
  RankRows in, out;
};


// Rows [sdv, sdv + c) of a buffer of lin rows and [rdv, rdv + c) of one of
// lout rows all exist, and there is at least one (no sum can overflow:
// lin, lout >= 0).
__host__ __device__ __forceinline__ bool block_fits(int64_t c, int64_t sdv, int64_t rdv,
                                                    int64_t lin, int64_t lout) {
  return c > 0 && sdv >= 0 && rdv >= 0 && sdv <= lin - c && rdv <= lout - c;
}

// One pointer per rank for a single buffer role (MoE helpers).
struct PtrTable {
  const void *p[COLL_MAX_RANKS];
};
struct MutPtrTable {
  void *p[COLL_MAX_RANKS];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ vector memory

// Streaming loads and stores.  NT = non-temporal (the "nt" cache policy):
// data moved once is not kept in the caches, which on MI355X lifts a plain
// copy from ~5.5 to ~6.2 TB/s when BOTH sides are non-temporal.
template <class U, bool NT = false>
__device__ __forceinline__ U ld(const void *base, size_t i) {
  const U *p = reinterpret_cast<const U *>(base) + i;
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <class U, bool NT = false>
__device__ __forceinline__ void st(void *base, size_t i, U v) {
  U *p = reinterpret_cast<U *>(base) + i;
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Work decomposition shared by the streaming kernels: a workgroup owns a tile
// of kBlock * U consecutive units (lane l takes units l, l + kBlock, ...,
// so every load and store instruction of a wave covers 64 consecutive units),
// issues all of the tile's loads before any store, and the grid has one
// workgroup per tile (a single pass: the dispatcher balances the load).
// Units per lane of the copy-family kernels (Gather, Broadcast, Scatter, the
// uniform all-to-all and re-shard).  Measured on MI355X, graph replay, rank
// buffers in an arena: one 16-byte unit per lane (4 KiB tiles) beat four
// (16 KiB tiles) everywhere: plain 1 GiB copy 6.26 -> 6.53 TB/s, all-to-all
// 8 x 64 MiB 6.23 -> 6.45, sequence -> heads re-shard 5.26 -> 5.87.
#ifndef COLL_COPY_U
#define COLL_COPY_U 1
#endif
constexpr int kCopyU = COLL_COPY_U;
// lanes per workgroup of the copy family (Broadcast, Scatter, the uniform
// all-to-all and re-shards, the LSE merge) and of Gather.  MI355X, graph-timed:
// 64 lanes beat 256 on the 1 GiB copy (328.5 -> 319.4 us), Scatter 8 x 64 MiB
// (167 -> 162), seq -> heads (95 -> 92.5) and match it elsewhere; 128 and 512
// were no better.  Gather (fp32 logits to the root) is 2% slower with 64.
#ifndef COLL_COPY_BLOCK
#define COLL_COPY_BLOCK 64
#endif
#ifndef COLL_GATHER_BLOCK
#define COLL_GATHER_BLOCK 256
#endif
constexpr int kCopyBlock = COLL_COPY_BLOCK;
constexpr int kGatherBlock = COLL_GATHER_BLOCK;

// ------------------------------------------------ element formats (exact widening)

// bf16 pair in one dword -> two fp32 (exact: bf16 is the top half of fp32)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// two fp32 -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
// two fp32 -> fp16 pair, round to nearest even (v_cvt_f16_f32 in RNE mode)
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
}

// ------------------------------------------------------- reduction operators

// MAX / MIN: NaN if either operand is NaN; -0 orders below +0.
__device__ __forceinline__ float op_max(float a, float b) {
  if (a != a || b != b) return __builtin_bit_cast(float, 0x7FC00000u);
  if (a == b) return __builtin_signbit(a) ? b : a;
  return a > b ? a : b;
}
__device__ __forceinline__ float op_min(float a, float b) {
  if (a != a || b != b) return __builtin_bit_cast(float, 0x7FC00000u);
  if (a == b) return __builtin_signbit(a) ? a : b;
  return a < b ? a : b;
}

template <int OP>
__device__ __forceinline__ float fold(float acc, float x) {
  if constexpr (OP == COLL_SUM) return acc + x;
  else if constexpr (OP == COLL_PROD) return acc * x;
  else if constexpr (OP == COLL_MAX) return op_max(acc, x);
  else return op_min(acc, x);
}

template <int OP>
__device__ __forceinline__ int32_t fold_i(int32_t acc, int32_t x) {
  if constexpr (OP == COLL_SUM) return (int32_t)((uint32_t)acc + (uint32_t)x);
  else if constexpr (OP == COLL_PROD) return (int32_t)((uint32_t)acc * (uint32_t)x);
  else if constexpr (OP == COLL_MAX) return acc > x ? acc : x;
  else return acc < x ? acc : x;
}

// Per-dtype view of a 16-byte vector as fp32 lanes (int32 stays integer).
//   kLanes: elements per 16 bytes; Acc: accumulator vector.
template <int DT> struct Fmt;

template <> struct Fmt<COLL_BF16> {
  static constexpr int kLanes = 8;
  static constexpr int kSize = 2;
  struct Acc { float v[8]; };
  __device__ static Acc widen(u32x4 w) {
    Acc a;
#pragma unroll
    for (int j = 0; j < 4; j++) { a.v[2 * j] = bf16_lo(w[j]); a.v[2 * j + 1] = bf16_hi(w[j]); }
    return a;
  }
  template <int OP> __device__ static void fold_in(Acc &a, u32x4 w) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      a.v[2 * j] = fold<OP>(a.v[2 * j], bf16_lo(w[j]));
      a.v[2 * j + 1] = fold<OP>(a.v[2 * j + 1], bf16_hi(w[j]));
    }
  }
  __device__ static u32x4 narrow(const Acc &a) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; j++) w[j] = pack_bf16(a.v[2 * j], a.v[2 * j + 1]);
    return w;
  }
  // scalar element path (tails, unaligned buffers)
  typedef uint16_t Elem;
  __device__ static float widen1(Elem e) { return bf16_lo(e); }
  __device__ static Elem narrow1(float f) { return (Elem)(pack_bf16(f, 0.0f) & 0xFFFFu); }
};

template <> struct Fmt<COLL_FP16> {
  static constexpr int kLanes = 8;
  static constexpr int kSize = 2;
  struct Acc { float v[8]; };
  __device__ static Acc widen(u32x4 w) {
    Acc a;
#pragma unroll
    for (int j = 0; j < 4; j++) { a.v[2 * j] = f16_lo(w[j]); a.v[2 * j + 1] = f16_hi(w[j]); }
    return a;
  }
  template <int OP> __device__ static void fold_in(Acc &a, u32x4 w) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      a.v[2 * j] = fold<OP>(a.v[2 * j], f16_lo(w[j]));
      a.v[2 * j + 1] = fold<OP>(a.v[2 * j + 1], f16_hi(w[j]));
    }
  }
  __device__ static u32x4 narrow(const Acc &a) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; j++) w[j] = pack_f16(a.v[2 * j], a.v[2 * j + 1]);
    return w;
  }
  typedef uint16_t Elem;
  __device__ static float widen1(Elem e) { return f16_lo(e); }
  __device__ static Elem narrow1(float f) { return (Elem)(pack_f16(f, 0.0f) & 0xFFFFu); }
};

template <> struct Fmt<COLL_FP32> {
  static constexpr int kLanes = 4;
  static constexpr int kSize = 4;
  struct Acc { float v[4]; };
  // (a vector element is copied to a scalar before __builtin_bit_cast: applied
  // to an ext_vector subscript directly, clang reinterprets element 0)
  __device__ static Acc widen(u32x4 w) {
    Acc a;
#pragma unroll
    for (int j = 0; j < 4; j++) { const uint32_t x = w[j]; a.v[j] = __builtin_bit_cast(float, x); }
    return a;
  }
  template <int OP> __device__ static void fold_in(Acc &a, u32x4 w) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t x = w[j];
      a.v[j] = fold<OP>(a.v[j], __builtin_bit_cast(float, x));
    }
  }
  __device__ static u32x4 narrow(const Acc &a) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; j++) w[j] = __builtin_bit_cast(uint32_t, a.v[j]);
    return w;
  }
  typedef float Elem;
  __device__ static float widen1(Elem e) { return e; }
  __device__ static Elem narrow1(float f) { return f; }
};

template <> struct Fmt<COLL_INT32> {
  static constexpr int kLanes = 4;
  static constexpr int kSize = 4;
  struct Acc { int32_t v[4]; };
  __device__ static Acc widen(u32x4 w) {
    Acc a;
#pragma unroll
    for (int j = 0; j < 4; j++) a.v[j] = (int32_t)w[j];
    return a;
  }
  template <int OP> __device__ static void fold_in(Acc &a, u32x4 w) {
#pragma unroll
    for (int j = 0; j < 4; j++) a.v[j] = fold_i<OP>(a.v[j], (int32_t)w[j]);
  }
  __device__ static u32x4 narrow(const Acc &a) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; j++) w[j] = (uint32_t)a.v[j];
    return w;
  }
  typedef int32_t Elem;
};

// ------------------------------------------------------------ fast division
// Division of n < 2^31 by a runtime constant d >= 1 with one mul-high, add and
// shift (Granlund & Montgomery, "Division by invariant integers using
// multiplication", 1994): q = (umulhi(n, m) + n) >> s with s = ceil(log2 d)
// and m = floor(2^32 (2^s - d) / d) + 1.
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) s++;
  f.s = s;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// The same for 64-bit numerators n < 2^63: m = floor(2^64 (2^s - d) / d) + 1.
struct FastDiv64 {
  uint64_t d, m;
  uint32_t s;
};

inline FastDiv64 make_fastdiv64(uint64_t d) {
  FastDiv64 f;
  f.d = d;
  uint32_t s = 0;
  while (s < 64 && (((unsigned __int128)1) << s) < d) s++;
  f.s = s;
  const unsigned __int128 one = 1;
  f.m = (uint64_t)(((one << 64) * ((one << s) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint64_t fdiv64(uint64_t n, const FastDiv64 &f) {
  return (__umul64hi(n, f.m) + n) >> f.s;
}

// Global-address-space views of an integer address (so the compiler emits
// global_load / global_store rather than flat accesses).
template <class U>
__device__ __forceinline__ const __attribute__((address_space(1))) U *gconst(uint64_t a) {
  return (const __attribute__((address_space(1))) U *)a;
}
template <class U>
__device__ __forceinline__ __attribute__((address_space(1))) U *gmut(uint64_t a) {
  return (__attribute__((address_space(1))) U *)a;
}

// ----------------------------------------------------------- copy units
// Widest power-of-two unit (<= 16 bytes) a copy can use, as a type.
template <int B> struct UnitT;
template <> struct UnitT<16> { typedef u32x4 T; };
template <> struct UnitT<8> { typedef u32x2 T; };
template <> struct UnitT<4> { typedef uint32_t T; };
template <> struct UnitT<2> { typedef uint16_t T; };
template <> struct UnitT<1> { typedef uint8_t T; };

// Launch KERNEL<unit, nt> for a unit size and cache policy chosen at run time.
#define COLL_UNIT_SWITCH_BLOCK(KERNEL, UNIT, NT, GRID, BLOCK, STREAM, ...)                      \
  do {                                                                                         \
    if (NT) {                                                                                  \
      switch (UNIT) {                                                                          \
        case 16: hipLaunchKernelGGL((KERNEL<16, true>), GRID, dim3(BLOCK), 0, STREAM, __VA_ARGS__); break; \
        case 8: hipLaunchKernelGGL((KERNEL<8, true>), GRID, dim3(BLOCK), 0, STREAM, __VA_ARGS__); break;   \
        case 4: hipLaunchKernelGGL((KERNEL<4, true>), GRID, dim3(BLOCK), 0, STREAM, __VA_ARGS__); break;   \
        case 2: hipLaunchKernelGGL((KERNEL<2, true>), GRID, dim3(BLOCK), 0, STREAM, __VA_ARGS__); break;   \
        default: hipLaunchKernelGGL((KERNEL<1, true>), GRID, dim3(BLOCK), 0, STREAM, __VA_ARGS__); break;  \
      }                                                                                        \
    } else {                                                                                   \
      switch (UNIT) {                                                                          \
        case 16: hipLaunchKernelGGL((KERNEL<16, false>), GRID, dim3(BLOCK), 0, STREAM, __VA_ARGS__); break; \
        case 8: hipLaunchKernelGGL((KERNEL<8, false>), GRID, dim3(BLOCK), 0, STREAM, __VA_ARGS__); break;   \
        case 4: hipLaunchKernelGGL((KERNEL<4, false>), GRID, dim3(BLOCK), 0, STREAM, __VA_ARGS__); break;   \
        case 2: hipLaunchKernelGGL((KERNEL<2, false>), GRID, dim3(BLOCK), 0, STREAM, __VA_ARGS__); break;   \
        default: hipLaunchKernelGGL((KERNEL<1, false>), GRID, dim3(BLOCK), 0, STREAM, __VA_ARGS__); break;  \
      }                                                                                        \
    }                                                                                          \
  } while (0)
#define COLL_UNIT_SWITCH(KERNEL, UNIT, NT, GRID, STREAM, ...) \
  COLL_UNIT_SWITCH_BLOCK(KERNEL, UNIT, NT, GRID, kBlock, STREAM, __VA_ARGS__)

// Scheduling fences that emit no instruction.  COLL_OPAQUE(x): x is taken to
// be rewritten in a vector register here, so the optimizer can neither see
// its value (a load through it stays a vector load) nor hoist what depends on
// it above this point.  COLL_KEEP(x): x must be available here, so its load
// is issued and completed before this point.
#ifndef COLL_OPAQUE
#define COLL_OPAQUE(x) asm volatile("" : "+v"(x))
#endif
#ifndef COLL_KEEP
#define COLL_KEEP(x) asm volatile("" ::"v"(x))
#endif
// COLL_UNIFORM(x): x (uniform across the wave) is taken to be rewritten in a
// scalar register here, so its load completes through the scalar cache
// before this point instead of being sunk into a later vector load.
#ifndef COLL_UNIFORM
#define COLL_UNIFORM(x) asm volatile("" : "+s"(x))
#endif
// COLL_SCALAR(x): the same fence for a value uniform by construction (a
// kernel argument), where it may sit under divergent control flow.
#ifndef COLL_SCALAR
#define COLL_SCALAR(x) asm volatile("" : "+s"(x))
#endif

// ld_scalar(p, i): p[i] for an address uniform across the wave, from memory
// the kernel never writes, read through the scalar cache (the constant
// address space).  Vector stores and loads share one in-order counter on
// this GPU, so a vector load issued after stores can only be waited on by
// waiting for those stores too; a scalar load has a counter of its own.
#ifndef COLL_HAVE_LD_SCALAR
template <class T>
__device__ __forceinline__ T ld_scalar(const T *p, size_t i) {
  return ((const __attribute__((address_space(4))) T *)p)[i];
}
#endif

// rows.n[i] for a lane-dependent i: a select chain over the table, which the
// kernel loads through the scalar unit.  Indexed directly, the by-value table
// becomes a vector load from the argument segment per lane, a round trip the
// table-building code then waits on (MoE fused dispatch, MI355X: 825 against
// 776-803 us).
__device__ __forceinline__ int64_t pick_rows(const RankRows &rows, int i) {
  int64_t v = 0;
#pragma unroll
  for (int q = 0; q < COLL_MAX_RANKS; q++) {
    int64_t x = rows.n[q];
    COLL_SCALAR(x);             // kept in a scalar register: no indexed reload
    v = i == q ? x : v;
  }
  return v;
}

// For code where a whole wave looks up the limits of many blocks: lane l
// (l < 16) selects rank l's limit once, and a lane reads rank r's from lane r
// with a shuffle (two 32-bit permutes) instead of its own select chain.
__device__ __forceinline__ int64_t lane_rows(const RankRows &rows) {
  return pick_rows(rows, (int)(threadIdx.x & (COLL_MAX_RANKS - 1)));
}
__device__ __forceinline__ int64_t rows_from_lane(int64_t mine, int r) {
  return __shfl(mine, r, 64);
}

// Lane l's 64-bit x (l the same in every lane).
__device__ __forceinline__ uint64_t readlane64(uint64_t x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// ----------------------------------------------------------- launch helpers

struct Launch {
  hipStream_t stream;
  int num_cus;       // compute units of the current device
  int wgs_per_cu;    // workgroups per CU for persistent (device-sized) kernels
  size_t nt_bytes;   // bytes moved at or above which loads/stores are non-temporal
  size_t nt_store_bytes;  // ReduceScatter / Reduce: bytes written at or above which
                          // their stores are non-temporal too
  int a2a_nt;        // non-temporal loads/stores in All-to-All-v (size unknown on the host)
  long a2a_grid;     // > 0: All-to-All-v launches this many workgroups (tuning)
  long ar_grid;      // > 0: AllReduce launches this many workgroups (tuning)
};

// Device properties and tuning knobs (environment, read once per process:
// COLL_WGS_PER_CU, COLL_NT_MIN_BYTES, COLL_NT_STORE_MIN_BYTES, COLL_A2A_NT,
// COLL_A2A_GRID, COLL_AR_GRID, COLL_A2A_DESC_MIN_BYTES).
Launch launch_ctx(void *stream);

// One workgroup per tile of kBlock * per_thread units (single pass), capped
// at 2^31 - 1 workgroups; kernels still loop in case the cap binds.
inline unsigned grid_for(const Launch &L, size_t work, int per_thread = 1) {
  (void)L;
  size_t per_block = (size_t)kBlock * per_thread;
  size_t need = (work + per_block - 1) / per_block;
  if (need < 1) need = 1;
  if (need > 0x7FFFFFFFu) need = 0x7FFFFFFFu;
  return (unsigned)need;
}

// One workgroup per tile of `tile_units` units (single pass), capped likewise.
inline unsigned grid_tiles(size_t work, size_t tile_units) {
  size_t need = (work + tile_units - 1) / tile_units;
  if (need < 1) need = 1;
  if (need > 0x7FFFFFFFu) need = 0x7FFFFFFFu;
  return (unsigned)need;
}

// Resident grid for kernels whose amount of work is only known on the device.
inline unsigned grid_resident(const Launch &L) {
  return (unsigned)L.num_cus * (unsigned)L.wgs_per_cu;
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Largest power-of-two unit (<= 16 bytes) dividing every pointer and `bytes`.
inline int copy_unit(uintptr_t bits_or) {
  if ((bits_or & 15u) == 0) return 16;
  if ((bits_or & 7u) == 0) return 8;
  if ((bits_or & 3u) == 0) return 4;
  if ((bits_or & 1u) == 0) return 2;
  return 1;
}

inline size_t dtype_size(int dt) {
  switch (dt) {
    case COLL_BF16: case COLL_FP16: return 2;
    case COLL_FP32: case COLL_INT32: return 4;
    default: return 0;
  }
}

inline int hip_status() {
  return hipGetLastError() == hipSuccess ? COLL_OK : COLL_ERR_HIP;
}

// ------------------------------------------------------- internal launchers
int launch_allreduce(const Launch &L, int R, const RankPtrs &p, size_t count, int dt, int op);
int launch_reduce_scatter(const Launch &L, int R, const RankPtrs &p, size_t recvcount, int dt, int op,
                          int nout);
int launch_all_gather(const Launch &L, int R, const RankPtrs &p, size_t bytes_per_rank);
int launch_gather(const Launch &L, int R, const RankPtrs &p, void *out, size_t outer,
                  size_t inner_bytes);
int launch_broadcast(const Launch &L, int R, const void *src, const RankPtrs &p, size_t bytes);
int launch_scatter(const Launch &L, int R, const void *src, const RankPtrs &p, size_t bytes);
int launch_reshard(const Launch &L, int R, const RankPtrs &p, size_t seq_local,
                   size_t chunk_bytes, bool to_heads);
int launch_lse_merge(const Launch &L, int R, const RankPtrs &o, const PtrTable &lse_in,
                     const MutPtrTable &lse_out, size_t rows, size_t D, int dt);
// ct = 1: counts is read transposed (the reverse of the exchange whose
// tables these are; see count_index in a2av.hip)
int launch_a2av(const Launch &L, int R, const RankPtrs &p, const RowLimits &lim,
                const int64_t *counts, const int64_t *sdispls, const int64_t *rdispls, int ct,
                size_t row_bytes, size_t rows_capacity);
size_t a2av_workspace_bytes(int R, size_t rows_capacity, size_t row_bytes, size_t min_bytes);
int launch_a2av_ws(const Launch &L, int R, const RankPtrs &p, const RowLimits &lim,
                   const int64_t *counts, const int64_t *sdispls, const int64_t *rdispls, int ct,
                   size_t row_bytes, size_t rows_capacity, void *ws);
// the two halves of launch_a2av_ws: COLL_ERR_UNSUPPORTED where the descriptor
// form does not apply (nothing launched)
int launch_a2av_ws_build(const Launch &L, int R, const RankPtrs &p, const RowLimits &lim,
                         const int64_t *counts, const int64_t *sdispls, const int64_t *rdispls,
                         int ct, size_t row_bytes, size_t rows_capacity, void *ws);
int launch_a2av_ws_copy(const Launch &L, int R, size_t row_bytes, size_t rows_capacity, void *ws);

constexpr int kMoeMaxExperts = 1024;
// Scratch of coll_moe_layout_noalloc: a device array of this many bytes per
// GPU, and its device address on the current device (NULL on failure).
constexpr size_t kMoeStaticBytes = 4u << 20;
void *moe_static_scratch();
size_t moe_workspace_bytes(int R, int T, int K, int E);
size_t moe_expert_table_bytes(int R, int E);
size_t moe_expert_workspace_bytes(int R, int E, size_t rows_capacity);
int launch_moe_layout(const Launch &L, int R, const PtrTable &ids, int T, int K, int E,
                      int64_t *sendcounts, int64_t *sdispls, int64_t *rdispls,
                      int32_t *expert_counts, const MutPtrTable &pos, void *ws);
int launch_moe_permute(const Launch &L, int R, const PtrTable &x, const PtrTable &pos, int T,
                       int K, size_t row_bytes, const MutPtrTable &send);
int launch_moe_expert_scale(const Launch &L, int R, const MutPtrTable &recv,
                            const int32_t *expert_counts, const int64_t *rdispls, int E,
                            size_t hidden, size_t rows_capacity, void *ws, size_t ws_bytes,
                            const RankRows &recv_rows);
// the row-descriptor path of the test expert in two calls (COLL_ERR_UNSUPPORTED
// where that path does not apply; moe_expert_rows_apply tells on the host)
bool moe_expert_rows_apply(int R, const MutPtrTable &recv, int E, size_t hidden,
                           size_t rows_capacity, size_t ws_bytes);
int launch_moe_expert_build(const Launch &L, int R, const MutPtrTable &recv,
                            const int32_t *expert_counts, const int64_t *rdispls, int E,
                            size_t hidden, size_t rows_capacity, void *ws, size_t ws_bytes,
                            const RankRows &recv_rows);
int launch_moe_expert_apply(const Launch &L, int R, const MutPtrTable &recv, int E, size_t hidden,
                            size_t rows_capacity, void *ws, size_t ws_bytes);
int launch_moe_combine(const Launch &L, int R, const PtrTable &back, const PtrTable &pos,
                       const PtrTable &w, int T, int K, size_t hidden, const MutPtrTable &out);
int launch_moe_dispatch(const Launch &L, int R, const PtrTable &x, const PtrTable &pos,
                        const int64_t *sendcounts, const int64_t *sdispls, const int64_t *rdispls,
                        int T, int K, size_t row_bytes, const MutPtrTable &recv,
                        const RankRows &recv_rows);
int launch_moe_combine_recv(const Launch &L, int R, const PtrTable &recv, const PtrTable &pos,
                            const int64_t *sendcounts, const int64_t *sdispls,
                            const int64_t *rdispls, const PtrTable &w, const PtrTable *ids, int T,
                            int K, size_t hidden, const MutPtrTable &out,
                            const RankRows &recv_rows);

}  // namespace coll
