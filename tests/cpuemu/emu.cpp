// CPU emulation runtime for the library's kernels -- TEST INFRASTRUCTURE ONLY.
//
// A grid runs one workgroup at a time.  Each lane of the workgroup is a fiber
// (ucontext) with its own stack; lane l belongs to wave l / 64.  A lane runs
// until it finishes, reaches __syncthreads, or reaches a wave operation
// (ballot, shuffle, readfirstlane, readlane).  When no lane can run:
//   - a wave whose blocked lanes wait at wave operations resolves them, with
//     those lanes as the active set (lanes of the wave that finished or wait
//     at the barrier are inactive, as exec-masked lanes are on the GPU); all
//     of them must wait at the same call site, otherwise the kernel used a
//     wave operation under divergent control flow and the run aborts;
//   - otherwise every unfinished lane waits at the barrier, which releases.
// Anything else is a deadlock and aborts.  LDS (the emu_lds section) is
// filled with a poison pattern before each workgroup.
#include <stdio.h>
#include <stdlib.h>
#include <sys/mman.h>
#include <ucontext.h>

#include "hip/hip_runtime.h"

namespace {

constexpr int kMaxLanes = 1024;
constexpr size_t kStack = 64 << 10;

enum State { RUNNABLE = 0, AT_WAVEOP = 1, AT_BARRIER = 2, DONE = 3 };

struct Lane {
  ucontext_t ctx;
  State state;
  emu_uint3 tid;
  int op;
  const char *file;
  int line;
  uint64_t val;
  int arg;
  uint64_t result;
};

Lane g_lanes[kMaxLanes];
char *g_stacks = nullptr;
ucontext_t g_sched;
Lane *g_cur = nullptr;
void (*g_body)(void *) = nullptr;
void *g_ctx = nullptr;
hipError_t g_last_error = hipSuccess;
int g_num_cus = -1;

[[noreturn]] void die(const char *what) {
  fprintf(stderr, "emu: %s (block %u,%u,%u)\n", what, emu_block_idx.x, emu_block_idx.y,
          emu_block_idx.z);
  fflush(stderr);
  abort();
}

void lane_main() {
  g_body(g_ctx);
  g_cur->state = DONE;
  // uc_link returns to the scheduler
}

void yield_to_scheduler() {
  if (swapcontext(&g_cur->ctx, &g_sched) != 0) die("swapcontext failed");
}

void describe_site(const char *who, int lane, const Lane &x) {
  fprintf(stderr, "emu:   %s lane %d: op %d at %s:%d\n", who, lane, x.op, x.file, x.line);
}

bool same_site(const Lane &a, const Lane &b) {
  return a.op == b.op && a.line == b.line && strcmp(a.file, b.file) == 0;
}

void resolve_wave(Lane *w, int n) {
  int op = 0, first_lane = -1;
  uint64_t active = 0;
  for (int l = 0; l < n; l++) {
    if (w[l].state != AT_WAVEOP) continue;
    if (first_lane < 0) {
      op = w[l].op;
      first_lane = l;
    } else if (!same_site(w[l], w[first_lane])) {
      describe_site("first", first_lane, w[first_lane]);
      describe_site("other", l, w[l]);
      die("wave operation under divergent control flow (lanes wait at different sites)");
    }
    active |= 1ull << l;
  }
  int first = __builtin_ctzll(active);
  for (int l = 0; l < n; l++) {
    if (!((active >> l) & 1)) continue;
    Lane &x = w[l];
    switch (op) {
      case EMU_BALLOT: {
        uint64_t m = 0;
        for (int q = 0; q < n; q++)
          if (((active >> q) & 1) && w[q].val) m |= 1ull << q;
        x.result = m;
        break;
      }
      case EMU_SHFL: {
        const int src = x.arg & 63;
        x.result = (src < n && ((active >> src) & 1)) ? w[src].val : 0;
        break;
      }
      case EMU_SHFL_UP: {
        const int src = l - x.arg;
        x.result = (src >= 0 && ((active >> src) & 1)) ? w[src].val : x.val;
        break;
      }
      case EMU_FIRSTLANE:
      case EMU_UNIFORM:
        if (x.val != w[first].val) {
          describe_site("first", first, w[first]);
          describe_site("other", l, x);
          die(op == EMU_UNIFORM ? "COLL_UNIFORM of a value that differs across lanes"
                                : "readfirstlane of a value that differs across lanes");
        }
        x.result = w[first].val;
        break;
      case EMU_READLANE: {
        const int src = x.arg;
        if (src < 0 || src >= n) die("readlane of a lane outside the wave");
        // readlane reads the register whatever the exec mask: an inactive
        // source lane's value is not modelled, so it is an error here
        if (!((active >> src) & 1)) die("readlane of an inactive lane");
        x.result = w[src].val;
        break;
      }
      default:
        die("unknown wave operation");
    }
    x.state = RUNNABLE;
  }
}

}  // namespace

extern "C" {

emu_uint3 emu_block_idx, emu_block_dim, emu_grid_dim;

const emu_uint3 *emu_thread_idx(void) { return &g_cur->tid; }

hipError_t hipGetLastError(void) {
  hipError_t e = g_last_error;
  g_last_error = hipSuccess;
  return e;
}

hipError_t hipGetDevice(int *dev) {
  *dev = 0;
  return hipSuccess;
}

// A small machine by default (resident grids stay small); EMU_CUS overrides.
hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t attr, int dev) {
  (void)dev;
  if (attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  if (g_num_cus < 0) {
    const char *e = getenv("EMU_CUS");
    g_num_cus = e ? atoi(e) : 4;
    if (g_num_cus < 1) g_num_cus = 1;
  }
  *value = g_num_cus;
  return hipSuccess;
}

void emu_syncthreads(void) {
  g_cur->state = AT_BARRIER;
  yield_to_scheduler();
}

uint64_t emu_wave_op(int op, uint64_t value, int arg, const char *file, int line) {
  g_cur->op = op;
  g_cur->val = value;
  g_cur->arg = arg;
  g_cur->file = file;
  g_cur->line = line;
  g_cur->state = AT_WAVEOP;
  yield_to_scheduler();
  return g_cur->result;
}

extern char __start_emu_lds[] __attribute__((weak));
extern char __stop_emu_lds[] __attribute__((weak));

void emu_run_grid(dim3 grid, dim3 block, void (*body)(void *), void *ctx) {
  const uint64_t nthreads = (uint64_t)block.x * block.y * block.z;
  if (grid.x == 0 || grid.y == 0 || grid.z == 0 || grid.x > 0x7FFFFFFFu || grid.y > 65535 ||
      grid.z > 65535 || nthreads == 0 || nthreads > kMaxLanes) {
    g_last_error = hipErrorInvalidConfiguration;
    return;
  }
  if (!g_stacks) {
    g_stacks = (char *)mmap(nullptr, kStack * kMaxLanes, PROT_READ | PROT_WRITE,
                            MAP_PRIVATE | MAP_ANONYMOUS, -1, 0);
    if (g_stacks == MAP_FAILED) die("no memory for lane stacks");
  }
  g_body = body;
  g_ctx = ctx;
  emu_grid_dim = {grid.x, grid.y, grid.z};
  emu_block_dim = {block.x, block.y, block.z};
  const int n = (int)nthreads;
  for (unsigned bz = 0; bz < grid.z; bz++)
    for (unsigned by = 0; by < grid.y; by++)
      for (unsigned bx = 0; bx < grid.x; bx++) {
        emu_block_idx = {bx, by, bz};
        if (__start_emu_lds && __stop_emu_lds > __start_emu_lds)
          memset(__start_emu_lds, 0xA5, (size_t)(__stop_emu_lds - __start_emu_lds));
        for (int l = 0; l < n; l++) {
          Lane &x = g_lanes[l];
          x.state = RUNNABLE;
          x.tid = {(unsigned)(l % block.x), (unsigned)((l / block.x) % block.y),
                   (unsigned)(l / (block.x * block.y))};
          getcontext(&x.ctx);
          x.ctx.uc_stack.ss_sp = g_stacks + (size_t)l * kStack;
          x.ctx.uc_stack.ss_size = kStack;
          x.ctx.uc_link = &g_sched;
          makecontext(&x.ctx, lane_main, 0);
        }
        for (;;) {
          bool ran = false;
          for (int l = 0; l < n; l++) {
            if (g_lanes[l].state != RUNNABLE) continue;
            g_cur = &g_lanes[l];
            if (swapcontext(&g_sched, &g_lanes[l].ctx) != 0) die("swapcontext failed");
            ran = true;
          }
          if (ran) continue;
          int done = 0, waveop = 0;
          for (int l = 0; l < n; l++) {
            done += g_lanes[l].state == DONE;
            waveop += g_lanes[l].state == AT_WAVEOP;
          }
          if (done == n) break;
          if (waveop) {
            for (int w = 0; w * 64 < n; w++) {
              const int m = n - w * 64 < 64 ? n - w * 64 : 64;
              bool any = false;
              for (int l = 0; l < m; l++) any = any || g_lanes[w * 64 + l].state == AT_WAVEOP;
              if (any) resolve_wave(&g_lanes[w * 64], m);
            }
            continue;
          }
          // every unfinished lane waits at the barrier
          for (int l = 0; l < n; l++)
            if (g_lanes[l].state == AT_BARRIER) g_lanes[l].state = RUNNABLE;
        }
      }
  g_cur = nullptr;
}

}  // extern "C"
