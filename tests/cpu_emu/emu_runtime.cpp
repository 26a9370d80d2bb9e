// Runtime of the CPU execution harness (see hip/hip_runtime.h here): workgroups are
// OS threads, lanes are ucontext fibers with round-robin scheduling, barriers count
// the live fibers of the workgroup (or of the wave), and a stuck workgroup (every live
// fiber waiting on a barrier that cannot complete) aborts with a message.
#include <sched.h>
#include <stdio.h>
#include <stdlib.h>
#include <ucontext.h>

#include <atomic>
#include <chrono>
#include <cstring>
#include <thread>
#include <deque>
#include <vector>

#include "hip/hip_runtime.h"

// ThreadSanitizer builds: every lane fiber is a TSan fiber, and the workgroup / wave
// barriers are happens-before edges, so TSan checks the kernels' cross-workgroup
// synchronisation (atomics and fences on global memory) and nothing else.
#if defined(__has_feature)
#if __has_feature(thread_sanitizer)
#define ETC_EMU_TSAN 1
#endif
#endif
#ifdef ETC_EMU_TSAN
extern "C" {
void* __tsan_get_current_fiber(void);
void* __tsan_create_fiber(unsigned flags);
void __tsan_destroy_fiber(void* fiber);
void __tsan_switch_to_fiber(void* fiber, unsigned flags);
void __tsan_acquire(void* addr);
void __tsan_release(void* addr);
}
#define TSAN_SWITCH(f) __tsan_switch_to_fiber((f), 0)
#define TSAN_RELEASE(a) __tsan_release(a)
#define TSAN_ACQUIRE(a) __tsan_acquire(a)
#else
#define TSAN_SWITCH(f) ((void)0)
#define TSAN_RELEASE(a) ((void)0)
#define TSAN_ACQUIRE(a) ((void)0)
#endif

namespace {

constexpr int LANES = 64;

enum State { RUNNABLE = 0, AT_BLOCK = 1, AT_WAVE = 2, DONE = 3 };

// A direct-to-LDS copy in flight (ETC_EMU_DMA_LATE): the 16 bytes were read from global
// memory when the copy was issued and land in LDS at the lane's next wait that counts
// it out, as late as the GPU may deliver them.
struct Dma {
  void* dst;
  unsigned char data[16];
  int size;
};

struct Fiber {
  ucontext_t ctx;
  void* tsan = nullptr;
  std::vector<char> stack;
  int state = RUNNABLE;
  unsigned tid = 0;
  std::deque<Dma> dma;
};

std::atomic<int> g_dma_late{-1};  // -1: not set yet (ETC_EMU_DMA_LATE decides)
bool dma_late() {
  int v = g_dma_late.load(std::memory_order_relaxed);
  if (v < 0) {
    v = getenv("ETC_EMU_DMA_LATE") != nullptr ? 1 : 0;
    g_dma_late.store(v, std::memory_order_relaxed);
  }
  return v != 0;
}
void dma_land(Fiber& f, size_t keep) {
  while (f.dma.size() > keep) {
    const Dma& d = f.dma.front();
    memcpy(d.dst, d.data, d.size);
    f.dma.pop_front();
  }
}

struct Workgroup {
  ucontext_t sched;
  void* tsan_sched = nullptr;
  int block_sync = 0, wave_sync[8] = {0};  // addresses the barrier edges hang on
  std::vector<Fiber> f;
  int cur = 0;
  int live = 0;
  int at_block = 0;
  int nwaves = 0;
  std::vector<int> wave_live, wave_at;
  std::vector<std::vector<unsigned char>> wave_buf;
  unsigned block = 0, grid = 0;
  const std::function<void()>* fn = nullptr;
  unsigned spins = 0;
  int or_flag = 0;
};

thread_local Workgroup* g_wg = nullptr;

size_t stack_bytes() {
  const char* s = getenv("ETC_EMU_STACK_KB");
  return (s ? (size_t)atoi(s) : 512) * 1024;
}

void to_sched(Workgroup& w, Fiber& me) {
  TSAN_SWITCH(w.tsan_sched);
  swapcontext(&me.ctx, &w.sched);
}

void release_block(Workgroup& w) {
  for (auto& f : w.f)
    if (f.state == AT_BLOCK) f.state = RUNNABLE;
  w.at_block = 0;
}
void release_wave(Workgroup& w, int wave) {
  for (int i = wave * LANES; i < (wave + 1) * LANES && i < (int)w.f.size(); ++i)
    if (w.f[i].state == AT_WAVE) w.f[i].state = RUNNABLE;
  w.wave_at[wave] = 0;
}

void fiber_entry() {
  Workgroup& w = *g_wg;
  (*w.fn)();
  Fiber& me = w.f[w.cur];
  dma_land(me, 0);
  me.state = DONE;
  --w.live;
  const int wave = me.tid / LANES;
  --w.wave_live[wave];
  if (w.live > 0 && w.at_block == w.live) release_block(w);
  if (w.wave_live[wave] > 0 && w.wave_at[wave] == w.wave_live[wave]) release_wave(w, wave);
  to_sched(w, me);
}

void run_workgroup(unsigned b, unsigned grid, unsigned block, const std::function<void()>* fn) {
  Workgroup w;
  w.block = b;
  w.grid = grid;
  w.fn = fn;
  w.f.resize(block);
  w.live = block;
  w.nwaves = (block + LANES - 1) / LANES;
  w.wave_live.assign(w.nwaves, 0);
  w.wave_at.assign(w.nwaves, 0);
  w.wave_buf.assign(w.nwaves, std::vector<unsigned char>(LANES * 64));
  g_wg = &w;
#ifdef ETC_EMU_TSAN
  w.tsan_sched = __tsan_get_current_fiber();
#endif
  const size_t sb = stack_bytes();
  for (unsigned i = 0; i < block; ++i) {
    Fiber& f = w.f[i];
    f.tid = i;
    ++w.wave_live[i / LANES];
    f.stack.resize(sb);
    getcontext(&f.ctx);
    f.ctx.uc_stack.ss_sp = f.stack.data();
    f.ctx.uc_stack.ss_size = sb;
    f.ctx.uc_link = nullptr;
    makecontext(&f.ctx, fiber_entry, 0);
#ifdef ETC_EMU_TSAN
    f.tsan = __tsan_create_fiber(0);
#endif
  }
  static const bool shuffle = getenv("ETC_EMU_SHUFFLE") != nullptr;
  unsigned rng = 0x9e3779b9u * (b + 1);
  while (w.live > 0) {
    bool ran = false;
    const unsigned start = shuffle ? (rng = rng * 1664525u + 1013904223u) % block : 0;
    for (unsigned n = 0; n < block; ++n) {
      const unsigned i = (start + n) % block;
      if (w.f[i].state != RUNNABLE) continue;
      w.cur = i;
      TSAN_SWITCH(w.f[i].tsan);
      swapcontext(&w.sched, &w.f[i].ctx);
      ran = true;
    }
    if (!ran) {
      fprintf(stderr, "cpu-emu: workgroup %u stuck: %d live fibers, %d at the block barrier\n", b,
              w.live, w.at_block);
      abort();
    }
  }
#ifdef ETC_EMU_TSAN
  for (auto& f : w.f) __tsan_destroy_fiber(f.tsan);
#endif
  g_wg = nullptr;
}

}  // namespace

EmuDim emu_thread_idx() { return EmuDim{g_wg->f[g_wg->cur].tid, 0, 0}; }
EmuDim emu_block_idx() { return EmuDim{g_wg->block, 0, 0}; }
EmuDim emu_grid_dim() { return EmuDim{g_wg->grid, 1, 1}; }
EmuDim emu_block_dim() { return EmuDim{(unsigned)g_wg->f.size(), 1, 1}; }
int emu_lane() { return g_wg->f[g_wg->cur].tid % LANES; }

// Selects when direct-to-LDS copies land for the following launches (0: at once, 1: at
// the lane's wait); set between launches only.
extern "C" __attribute__((visibility("default"))) void etc_emu_set_dma_late(int late) {
  g_dma_late.store(late ? 1 : 0, std::memory_order_relaxed);
}

// global_load_lds of one lane: lands at once, or (ETC_EMU_DMA_LATE) at the lane's wait
void emu_dma_issue(void* dst, const void* src, int size) {
  if (!dma_late()) {
    memcpy(dst, src, size);
    return;
  }
  Dma d;
  d.dst = dst;
  d.size = size;
  memcpy(d.data, src, size);
  g_wg->f[g_wg->cur].dma.push_back(d);
}
// s_waitcnt: the lane's copies beyond the vector-memory count land (oldest first)
void emu_waitcnt(int imm) {
  const int vm = (imm & 15) | (((imm >> 14) & 3) << 4);
  dma_land(g_wg->f[g_wg->cur], (size_t)vm);
}

void emu_syncthreads() {
  Workgroup& w = *g_wg;
  Fiber& me = w.f[w.cur];
  TSAN_RELEASE(&w.block_sync);
  if (++w.at_block == w.live) {
    release_block(w);
  } else {
    me.state = AT_BLOCK;
    to_sched(w, me);
  }
  TSAN_ACQUIRE(&w.block_sync);
}

// OR of v over the workgroup, returned to every thread (a flag in the workgroup,
// cleared by the last thread through a second barrier)
int emu_syncthreads_or(int v) {
  Workgroup& w = *g_wg;
  emu_syncthreads();
  if (v) w.or_flag = 1;
  emu_syncthreads();
  const int r = w.or_flag;
  emu_syncthreads();
  w.or_flag = 0;
  return r;
}

void emu_wave_barrier() {
  Workgroup& w = *g_wg;
  Fiber& me = w.f[w.cur];
  const int wave = me.tid / LANES;
  TSAN_RELEASE(&w.wave_sync[wave]);
  if (++w.wave_at[wave] == w.wave_live[wave]) {
    release_wave(w, wave);
  } else {
    me.state = AT_WAVE;
    to_sched(w, me);
  }
  TSAN_ACQUIRE(&w.wave_sync[wave]);
}

void* emu_wave_scratch(int bytes_per_lane) {
  Workgroup& w = *g_wg;
  auto& buf = w.wave_buf[w.f[w.cur].tid / LANES];
  if ((int)buf.size() < bytes_per_lane * LANES) buf.resize(bytes_per_lane * LANES);
  return buf.data();
}

void emu_yield() {
  Workgroup& w = *g_wg;
  Fiber& me = w.f[w.cur];
  if ((++w.spins & 63) == 0) sched_yield();  // let other workgroups' threads run
  to_sched(w, me);
}

// The device clock counts at 100 MHz; the harness runs far slower than a GPU, so its
// clock is divided by ETC_EMU_CLOCK_DIV (default 1000) to keep the kernels' wait limits
// meaningful.
uint64_t emu_realtime() {
  using namespace std::chrono;
  static const uint64_t div = getenv("ETC_EMU_CLOCK_DIV") ? atoll(getenv("ETC_EMU_CLOCK_DIV")) : 1000;
  return (uint64_t)duration_cast<nanoseconds>(steady_clock::now().time_since_epoch()).count() / 10 / div;
}

// ---- wave-collective MFMA
struct MfmaBf16Slot {
  emu_bf16x8 a[LANES], b[LANES];
};
struct MfmaF32Slot {
  float a[LANES], b[LANES];
};

emu_f32x4 emu_mfma_bf16(emu_bf16x8 a, emu_bf16x8 b, emu_f32x4 c) {
  auto* s = static_cast<MfmaBf16Slot*>(emu_wave_scratch(sizeof(MfmaBf16Slot) / LANES + 1));
  const int lane = emu_lane();
  s->a[lane] = a;
  s->b[lane] = b;
  emu_wave_barrier();
  emu_f32x4 d = c;
  const int j = lane % 16;
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * (lane / 16) + r;
    float acc = 0.f;
    for (int k = 0; k < 32; ++k)
      acc += (float)s->a[i + 16 * (k / 8)][k % 8] * (float)s->b[j + 16 * (k / 8)][k % 8];
    d[r] = c[r] + acc;
  }
  emu_wave_barrier();
  return d;
}

emu_f32x4 emu_mfma_f32(float a, float b, emu_f32x4 c) {
  auto* s = static_cast<MfmaF32Slot*>(emu_wave_scratch(sizeof(MfmaF32Slot) / LANES + 1));
  const int lane = emu_lane();
  s->a[lane] = a;
  s->b[lane] = b;
  emu_wave_barrier();
  emu_f32x4 d = c;
  const int j = lane % 16;
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * (lane / 16) + r;
    float acc = 0.f;
    for (int k = 0; k < 4; ++k) acc += s->a[i + 16 * k] * s->b[j + 16 * k];
    d[r] = c[r] + acc;
  }
  emu_wave_barrier();
  return d;
}

// ---- host API
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipGetDeviceProperties(hipDeviceProp_t* p, int) {
  memset(p, 0, sizeof(*p));
  strcpy(p->gcnArchName, "gfx950:sramecc+:xnack-");
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  const char* s = getenv("ETC_EMU_CUS");
  *v = s ? atoi(s) : 4;
  return hipSuccess;
}
hipError_t hipMemsetAsync(void* p, int v, size_t n, hipStream_t) {
  memset(p, v, n);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* d, const void* s, size_t n, hipMemcpyKind, hipStream_t) {
  memcpy(d, s, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipGetLastError() { return hipSuccess; }

void emu_launch(unsigned grid, unsigned block, std::function<void()> fn) {
  std::vector<std::thread> th;
  th.reserve(grid);
  for (unsigned b = 0; b < grid; ++b) th.emplace_back(run_workgroup, b, grid, block, &fn);
  for (auto& t : th) t.join();
}
