// Self-test of the CPU emulation -- TEST INFRASTRUCTURE ONLY.  Each case runs
// one small kernel; with bad = 0 it keeps every rule the emulator enforces,
// with bad = 1 it breaks one, and the emulator must stop the run: a value the
// kernel claims is wave-uniform that is not, a wave operation reached by part
// of a wave, a store one element past a guarded buffer, LDS read before it is
// written (which must come back poisoned, not zero).
#include "hip/hip_runtime.h"

namespace {

__global__ void uniform_kernel(int *out, int bad) {
  int v = bad ? (int)threadIdx.x : (int)blockIdx.x;
  COLL_UNIFORM(v);
  out[blockIdx.x * blockDim.x + threadIdx.x] = v;
}

__global__ void firstlane_kernel(int *out, int bad) {
  const int v = bad ? (int)threadIdx.x : 7 + (int)blockIdx.x;
  out[blockIdx.x * blockDim.x + threadIdx.x] = __builtin_amdgcn_readfirstlane(v);
}

__global__ void divergent_kernel(int *out, int bad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (bad && (threadIdx.x & 1))
    out[i] = (int)__popcll(__ballot(1));
  else
    out[i] = (int)__popcll(__ballot(threadIdx.x < 8));
}

__global__ void store_kernel(int *out, int shift) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  out[i + shift] = i;                   // shift 1: the last lane stores past the end
}

__global__ void lds_kernel(int *out, int bad) {
  __shared__ int s[64];
  if (!bad) s[threadIdx.x] = (int)threadIdx.x;
  __syncthreads();
  out[threadIdx.x] = s[63 - threadIdx.x];
}

}  // namespace

// which: 0 uniform, 1 readfirstlane, 2 divergent ballot, 3 store past the end,
// 4 LDS.  out holds 128 ints (two workgroups of 64 lanes; 64 for case 4).
extern "C" int emu_selftest(int which, int *out, int bad) {
  switch (which) {
    case 0: hipLaunchKernelGGL(uniform_kernel, dim3(2), dim3(64), 0, nullptr, out, bad); break;
    case 1: hipLaunchKernelGGL(firstlane_kernel, dim3(2), dim3(64), 0, nullptr, out, bad); break;
    case 2: hipLaunchKernelGGL(divergent_kernel, dim3(2), dim3(64), 0, nullptr, out, bad); break;
    case 3: hipLaunchKernelGGL(store_kernel, dim3(2), dim3(64), 0, nullptr, out, bad); break;
    case 4: hipLaunchKernelGGL(lds_kernel, dim3(1), dim3(64), 0, nullptr, out, bad); break;
    default: return -1;
  }
  return 0;
}
