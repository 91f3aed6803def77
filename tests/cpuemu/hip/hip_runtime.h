// CPU emulation of the HIP device subset the library's kernels use -- TEST
// INFRASTRUCTURE ONLY.  The library's .hip sources compile unchanged against
// this header as plain C++ for the host; kernels then run on the CPU, each
// workgroup's lanes as cooperative fibers grouped in wave64s, so barriers,
// ballots, shuffles and readfirstlane behave as they do on the GPU and every
// memory access goes to host memory, where guard pages catch any access past
// a buffer.  Nothing here is part of the product.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <type_traits>

// ---------------------------------------------------------------- qualifiers
#define __global__
#define __device__
#define __host__
#define __forceinline__ inline __attribute__((always_inline))
#define __launch_bounds__(...)
#define __align__(n) __attribute__((aligned(n)))
// LDS: every __shared__ variable goes to the section emu_lds, which the
// emulator fills with a poison pattern before each workgroup starts, so a
// kernel that reads LDS it did not write first computes garbage.
#define __shared__ __attribute__((section("emu_lds"))) static

// the library's scheduling fences emit nothing on the CPU; COLL_UNIFORM, which
// on the GPU moves its value into a scalar register (lane 0's copy wins if the
// lanes disagree), is checked instead: every active lane must hold the same
// bits, or the run aborts naming the site (see the wave ops below)
#define COLL_OPAQUE(x) ((void)0)
#define COLL_KEEP(x) ((void)0)
#define COLL_SCALAR(x) ((void)0)
// ld_scalar: the GPU reads through the scalar cache, which needs the address
// to be the same in every lane; here it is a plain load, after checking that
// every active lane asks for the same address (defined below emu_uniform_at)
#define COLL_HAVE_LD_SCALAR 1
#define ld_scalar(p, i) emu_ld_scalar((p), (size_t)(i), __FILE__, __LINE__)
#define COLL_UNIFORM(x) emu_uniform_at(emu_bits(x), __FILE__, __LINE__)

// ------------------------------------------------------------- runtime types
typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidConfiguration = 9, hipErrorInvalidValue = 1 };
typedef struct emu_stream *hipStream_t;
typedef int hipDeviceAttribute_t;
enum { hipDeviceAttributeMultiprocessorCount = 1 };

struct dim3 {
  unsigned x, y, z;
  constexpr dim3(unsigned x_ = 1, unsigned y_ = 1, unsigned z_ = 1) : x(x_), y(y_), z(z_) {}
};
struct emu_uint3 {
  unsigned x, y, z;
};

extern "C" {
hipError_t hipGetLastError(void);
hipError_t hipGetDevice(int *dev);
hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t attr, int dev);
// scheduler entry points (emu.cpp)
const emu_uint3 *emu_thread_idx(void);
extern emu_uint3 emu_block_idx, emu_block_dim, emu_grid_dim;
void emu_syncthreads(void);
uint64_t emu_wave_op(int op, uint64_t value, int arg, const char *file, int line);
void emu_run_grid(dim3 grid, dim3 block, void (*body)(void *), void *ctx);
}

#define threadIdx (*emu_thread_idx())
#define blockIdx emu_block_idx
#define blockDim emu_block_dim
#define gridDim emu_grid_dim
#define __syncthreads() emu_syncthreads()

static inline hipError_t hipGetSymbolAddress(void **p, const void *sym) {
  *p = const_cast<void *>(sym);
  return hipSuccess;
}
#define HIP_SYMBOL(x) (&(x))

// --------------------------------------------------------------- wave ops
// Each op is a rendezvous of the wave's active lanes at one source position
// (file, line): the same position however the compiler duplicates its code.
// readfirstlane and COLL_UNIFORM also check that every active lane holds the
// same value: the library uses both only on values it takes to be uniform
// (slots, ranks and descriptors loaded from one address), and a lane that
// disagreed would go on with lane 0's address on the GPU.
enum { EMU_BALLOT = 1, EMU_SHFL = 2, EMU_SHFL_UP = 3, EMU_FIRSTLANE = 4, EMU_READLANE = 5,
       EMU_UNIFORM = 6 };

template <class T>
static inline uint64_t emu_bits(T v) {
  static_assert(sizeof(T) <= 8, "wave op payload");
  uint64_t b = 0;
  memcpy(&b, &v, sizeof(T));
  return b;
}
template <class T>
static inline T emu_from(uint64_t b) {
  T v;
  memcpy(&v, &b, sizeof(T));
  return v;
}

static inline uint64_t emu_ballot_at(int pred, const char *f, int l) {
  return emu_wave_op(EMU_BALLOT, pred ? 1 : 0, 0, f, l);
}
template <class T>
static inline T emu_shfl_at(T v, int src, int width, const char *f, int l) {
  (void)width;
  return emu_from<T>(emu_wave_op(EMU_SHFL, emu_bits(v), src, f, l));
}
template <class T>
static inline T emu_shfl_up_at(T v, unsigned delta, int width, const char *f, int l) {
  (void)width;
  return emu_from<T>(emu_wave_op(EMU_SHFL_UP, emu_bits(v), (int)delta, f, l));
}
static inline int emu_readfirstlane_at(int v, const char *f, int l) {
  return (int)emu_wave_op(EMU_FIRSTLANE, (uint32_t)v, 0, f, l);
}
static inline void emu_uniform_at(uint64_t bits, const char *f, int l) {
  (void)emu_wave_op(EMU_UNIFORM, bits, 0, f, l);
}

template <class T>
static inline T emu_ld_scalar(const T *p, size_t i, const char *f, int l) {
  emu_uniform_at((uint64_t)(uintptr_t)(p + i), f, l);
  return p[i];
}
static inline int emu_readlane_at(int v, int lane, const char *f, int l) {
  return (int)emu_wave_op(EMU_READLANE, (uint32_t)v, lane, f, l);
}

#define __ballot(p) emu_ballot_at((int)(p), __FILE__, __LINE__)
#define __shfl(v, s, w) emu_shfl_at((v), (s), (w), __FILE__, __LINE__)
#define __shfl_up(v, d, w) emu_shfl_up_at((v), (unsigned)(d), (w), __FILE__, __LINE__)
#define __builtin_amdgcn_readfirstlane(v) emu_readfirstlane_at((int)(v), __FILE__, __LINE__)
#define __builtin_amdgcn_readlane(v, l) emu_readlane_at((int)(v), (int)(l), __FILE__, __LINE__)

// ------------------------------------------------------------ integer helpers
static inline int __popcll(unsigned long long x) { return __builtin_popcountll(x); }
static inline int __popc(unsigned x) { return __builtin_popcount(x); }
static inline unsigned __umulhi(unsigned a, unsigned b) {
  return (unsigned)(((unsigned long long)a * b) >> 32);
}
static inline unsigned long long __umul64hi(unsigned long long a, unsigned long long b) {
  return (unsigned long long)(((unsigned __int128)a * b) >> 64);
}
// lanes run one at a time, so a plain read-modify-write is atomic
template <class T>
static inline T atomicAdd(T *p, T v) {
  T old = *p;
  *p = old + v;
  return old;
}

// ------------------------------------------------------------------ launch
template <class Body>
static void emu_trampoline(void *ctx) {
  (*static_cast<Body *>(ctx))();
}

template <class F, class... A>
static void emu_launch(F kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                       A... args) {
  (void)shmem;
  (void)stream;
  auto body = [&]() { kernel(args...); };
  emu_run_grid(grid, block, &emu_trampoline<decltype(body)>, &body);
}

#define hipLaunchKernelGGL(K, G, B, S, ST, ...) emu_launch(K, dim3(G), dim3(B), (S), (ST), __VA_ARGS__)
