// Device-side building blocks shared by the persistent kernels: storage types,
// bfloat16 conversion, the event-counter primitives (signal / wait with a watchdog)
// and wave-level reductions.  gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#define ETC_DEV __device__ __forceinline__
#define ETC_INLINE __attribute__((always_inline))  // for lambdas

namespace etc {

constexpr int NT = 256;  // default threads per workgroup of a persistent kernel (4 waves)
constexpr int WAVE = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 raw bytes as a native vector: copies are register moves, never memcpy through memory
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct bf16 {
  uint16_t bits;
};

// ------------------------------------------------------------------ conversions

ETC_DEV float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even; NaN stays NaN (quiet).
// float -> bfloat16 bits, round to nearest even (gfx950 converts in hardware, two values
// per v_cvt_pk_bf16_f32)
ETC_DEV uint32_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two values in one v_cvt_pk_bf16_f32 (converting them one at a time costs a conversion
// each plus the shifts and ORs that pack them)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
ETC_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

template <typename TE>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int BYTES = 4;
  ETC_DEV static float load(const float* p, long i) { return p[i]; }
  ETC_DEV static void store(float* p, long i, float v) { p[i] = v; }
};
template <>
struct Elem<bf16> {
  static constexpr int BYTES = 2;
  ETC_DEV static float load(const bf16* p, long i) { return bf16_bits_to_f32(p[i].bits); }
  ETC_DEV static void store(bf16* p, long i, float v) { p[i].bits = (uint16_t)f32_to_bf16_bits(v); }
};

// 16 bytes of a row, expanded to floats (8 bf16 or 4 f32 values)
ETC_DEV void expand16(const uint4& v, float* out8, const bf16*) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out8[2 * i] = __uint_as_float(w[i] << 16);
    out8[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
ETC_DEV void expand16(const uint4& v, float* out4, const float*) {
  out4[0] = __uint_as_float(v.x);
  out4[1] = __uint_as_float(v.y);
  out4[2] = __uint_as_float(v.z);
  out4[3] = __uint_as_float(v.w);
}
ETC_DEV void expand16(const u32x4& v, float* out8, const bf16* tag) {
  expand16(make_uint4(v.x, v.y, v.z, v.w), out8, tag);
}
ETC_DEV void expand16(const u32x4& v, float* out4, const float* tag) {
  expand16(make_uint4(v.x, v.y, v.z, v.w), out4, tag);
}

// ------------------------------------------------------------------ global memory
//
// Pointers reach the task bodies through an LDS copy of the kernel arguments, so the
// compiler cannot tell that they address global memory and would access them with FLAT
// instructions.  Those count against the LDS wait counter as well, so every wait for an
// LDS read would also wait for every global load and store still in flight, and a wait
// for one of several loads could only wait for all of them.  Every access to global
// memory therefore goes through a pointer in address space 1.
#ifndef ETC_GLOBAL
#define ETC_GLOBAL __attribute__((address_space(1)))
#endif
#ifndef ETC_LDS
#define ETC_LDS __attribute__((address_space(3)))
#endif
template <typename T>
ETC_DEV ETC_GLOBAL T* gp(T* p) { return (ETC_GLOBAL T*)p; }
template <typename T>
ETC_DEV const ETC_GLOBAL T* gp(const T* p) { return (const ETC_GLOBAL T*)p; }
// a V (e.g. a 16-byte vector) read from global memory at p
template <typename V, typename T>
ETC_DEV V gld(const T* p) { return *(const ETC_GLOBAL V*)p; }
// relaxed device-scope float addition without a result (the atomic combine)
ETC_DEV void red_add(float* p, float v) {
  __hip_atomic_fetch_add(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ event counters
//
// An event counter is an int32 in global memory.  A producer first makes its own
// results visible to the whole device, then adds to the counter with release
// semantics at agent scope; a consumer reads the counter with acquire semantics at
// agent scope until it reaches its target.  On gfx950 the agent-scope release writes
// back this XCD's L2 and the acquire invalidates the reader's caches, so data written
// on one XCD is seen on another.  Only one lane of a workgroup touches a counter; the
// rest of the workgroup is ordered by barriers around it.

ETC_DEV int ev_load(const int* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
ETC_DEV int ev_load_relaxed(const int* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
ETC_DEV int ev_add(int* p, int v) {
  return __hip_atomic_fetch_add(gp(p), v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
ETC_DEV int ev_add_acquire(int* p, int v) {
  return __hip_atomic_fetch_add(gp(p), v, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
ETC_DEV int ev_add_relaxed(int* p, int v) {
  return __hip_atomic_fetch_add(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A relaxed addition whose result nobody reads: it goes out as an atomic without a
// return, so the signalling wave does not wait for the round trip.
ETC_DEV void ev_signal(int* p, int v) {
  (void)__hip_atomic_fetch_add(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
ETC_DEV void ev_store(int* p, int v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
ETC_DEV void ev_store_relaxed(int* p, int v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
ETC_DEV long long q_load(const long long* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
ETC_DEV long long q_load_relaxed(const long long* p) {
  return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
ETC_DEV void q_store(long long* p, long long v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
ETC_DEV void q_store_relaxed(long long* p, long long v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
ETC_DEV void fence_release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
ETC_DEV void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Shared results.  Every store of data that another workgroup reads after an event
// goes through these: agent-scope atomic stores, which reach the point of coherence
// of all XCDs by themselves.  An event then needs no release (on this GPU an
// agent-scope release writes back the whole L2 of the XCD, several microseconds):
// publish_shared() waits until this workgroup's stores have completed, and the signal
// that follows is a relaxed atomic.  Readers still acquire (invalidating their L2), so
// no stale line from an earlier call or layer is read.
ETC_DEV void st_shared(uint32_t* p, uint32_t v) {
  __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
ETC_DEV void st_shared(int* p, int v) { __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
ETC_DEV void st_shared(float* p, float v) { st_shared(reinterpret_cast<uint32_t*>(p), __float_as_uint(v)); }
ETC_DEV void st_shared8(void* p, uint64_t v) {
  __hip_atomic_store(gp(static_cast<uint64_t*>(p)), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes at byte offset off (16-byte aligned, per lane, below 2^31) from the wave-uniform
// base, as
// one buffer_store_dwordx4 with the same device-scope policy (sc1).  Two 8-byte stores
// would leave every 16-byte piece half written by each instruction: byte-masked partial
// writes of the cache lines, which cost far more than whole 64-byte pieces.
constexpr int BUF_DESC_WORD3 = 0x00020000;  // raw 32-bit buffer access (gfx9 family)
constexpr int CPOL_SC1 = 16;
ETC_DEV void st_shared16(void* base, uint32_t off, const u32x4& v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0x7fffffff, BUF_DESC_WORD3);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, CPOL_SC1);
}

// Every thread's stores have completed (so every shared result of the workgroup has
// reached the point of coherence), then the workgroup meets.
ETC_DEV void publish_shared() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Direct copy of 16 bytes per lane from global memory into LDS (gfx950
// global_load_lds_dwordx4): lane l of the wave writes lds_wave_base + 16 * l, so
// lds_wave_base must be the same in every lane of the wave.  The copy completes
// asynchronously; it counts as an outstanding vector-memory operation of the wave
// until the data is in LDS (see vm_wait_barrier).
ETC_DEV void lds_dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding (and all
// of its LDS operations are done), then meet the workgroup at a barrier.  Nothing moves
// across it: the compiler-only fences keep memory operations in place, the scheduling
// barriers keep every other instruction (MFMAs above all) on its side.
template <int N>
ETC_DEV void vm_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  // s_waitcnt fields: vmcnt [3:0] and [15:14], expcnt [6:4] (7: no wait), lgkmcnt [11:8]
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until this wave's LDS reads (and scalar loads) have completed; vector-memory
// operations may stay outstanding.
ETC_DEV void lgkm_wait_all() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // vmcnt 63, expcnt 7, lgkmcnt 0
}

// Every thread waits until all of its own memory operations have completed, then the
// workgroup meets at a barrier: after this, one thread's agent-scope release covers
// the stores of the whole workgroup.
ETC_DEV void wg_publish() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

ETC_DEV uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }  // 100 MHz

// Control words shared by all workgroups of one call (in the workspace).
enum SchedWord {
  W_TICKET = 0,   // static: next ticket
  W_EXIT = 5,     // workgroups that have left the task loop
  W_STATUS = 7,   // 0 ok, else an etc_status; survives the end-of-call reset
  W_AUX = 8,      // debug: where the abort came from
  W_TRACE = 9,    // trace records written so far in this call
  W_TRACE_LAST = 10,  // trace records of the last traced call (survives the reset)
  // Words that many workgroups touch at once sit in 128-byte lines of their own.  A read
  // of a line that a stream of atomics is updating waits behind those atomics (a
  // workgroup that read the abort flag before every task, in the line of the ticket
  // counter, spent most of its time on that read).
  W_ABORT = 32,   // set when a wait times out: every workgroup leaves
  W_XTICKET = 64, // static: next ticket of XCD queue q at W_XTICKET + q * W_LINE
  // The dynamic queue's words: every claimer adds to the head, every producer to the
  // tail, and idle claimers read the total and the planned-layer count, so each of the
  // three groups has a line of its own.
  W_QHEAD = 320,   // dynamic: next queue slot to take (dedicated: scheduler progress)
  W_QTAIL = 352,   // dynamic: queue slots handed out to producers
  W_QTOTAL = 384,  // dynamic: tasks that will ever be queued (grows as layers plan)
  W_PLANNED = 385, // dynamic: layers whose task counts are final
  W_LINE = 32,     // words per 128-byte line
  W_NWORDS = 416
};
constexpr int MAX_XCD_QUEUES = 8;  // MI355X: 8 XCDs of 32 CUs, each with its own L2

// Static tickets through per-XCD queues (thread 0 of a workgroup calls these).  A fixed
// task order is cut into chunks of G = workers / Q consecutive tasks, chunk c belonging
// to queue c mod Q (Q = min(8, workers)); workgroup b draws the next ticket of queue
// b mod Q.  The dispatcher places workgroup b on XCD b mod 8, so with Q = 8 each chunk
// runs on one XCD and tasks that are adjacent in the order share that XCD's L2.  Each
// queue hands out its tickets in the global order and has at least one workgroup, so a
// waiting task's producers, which come earlier in the order, are always claimed by
// workgroups that can run them: the order stays deadlock-free.
//
// The i-th ticket drawn from queue q.  Every ticket, the first included, comes from the
// queue's counter: a ticket is only ever held by a workgroup that is running, so the
// order stays deadlock-free even when some workgroups of the grid start late (another
// kernel holding their compute units).
ETC_DEV int xcd_ticket_of(int q, int i) {
  const int nwg = (int)gridDim.x;
  const int Q = nwg < MAX_XCD_QUEUES ? nwg : MAX_XCD_QUEUES;
  const int G = nwg / Q;
  return ((i / G) * Q + q) * G + i % G;
}

// The next value of a ticket counter (relaxed, agent scope).  An increment that wraps at
// 2^32 - 1 is a plain increment here; unlike an atomic add it is left alone by the
// compiler's wave-level atomic aggregation, which reads the result back at once (a wait
// for every memory operation issued before the atomic) to spread it over the lanes.
ETC_DEV int ticket_inc(int* counter) {
  return (int)__builtin_amdgcn_atomic_inc32((unsigned*)gp(counter), 0xffffffffu, __ATOMIC_RELAXED, "agent");
}

// A ticket in two steps: the draw (the atomic) and its mapping, so that a caller can
// keep the atomic in flight and map the result only where it needs the ticket.
ETC_DEV int xcd_ticket_draw(int* sched) {
  const int nwg = (int)gridDim.x;
  const int Q = nwg < MAX_XCD_QUEUES ? nwg : MAX_XCD_QUEUES;
  return ticket_inc(sched + W_XTICKET + ((int)blockIdx.x % Q) * W_LINE);
}
ETC_DEV int xcd_ticket_map(int drawn) {
  const int nwg = (int)gridDim.x;
  const int Q = nwg < MAX_XCD_QUEUES ? nwg : MAX_XCD_QUEUES;
  return xcd_ticket_of((int)blockIdx.x % Q, drawn);
}
ETC_DEV int xcd_ticket(int* sched) { return xcd_ticket_map(xcd_ticket_draw(sched)); }

// Waits poll with relaxed loads (no cache invalidation per poll: an agent-scope acquire
// invalidates this CU's L1 and the XCD's L2 lines, which would keep evicting the operands
// of the tiles running beside the waiter) and, once the condition holds, take an
// agent-scope acquire fence: the relaxed load that saw the producers' additions plus
// the fence synchronise with them, and the fence only invalidates this reader's caches,
// where a second (acquire) load would cost another round trip to the counter.
//
// Watchdog.  A wait gives up when what it watches has made no progress for `patience`
// ticks of the 100 MHz real-time clock: the limit starts when the wait begins and starts
// again whenever the polled value changes, so a long call whose counters keep moving is
// never cut short.  It also gives up after SPIN_MAX_ITERS polls without progress, so a
// wait ends even if the clock did not advance.  Giving up records ETC_ERR_TIMEOUT and
// the wait's site in the control words and raises the abort flag; every other wait
// sees the flag at its next check and returns false as well, so every workgroup leaves.
constexpr int SPIN_MAX_ITERS = 1 << 24;
constexpr int WATCH_EVERY = 16;  // polls between two checks of the clock and the abort flag

struct Watchdog {
  uint64_t limit;
  int seen, quiet;
  ETC_DEV void start(uint64_t patience, int value) {
    limit = now_ticks() + patience;
    seen = value;
    quiet = 0;
  }
  // Called every WATCH_EVERY polls with the value the wait currently sees.  True when
  // the call is aborted (by this wait or by another workgroup).
  ETC_DEV bool expired(int* sched, uint64_t patience, int value, int where) {
    if (ev_load_relaxed(sched + W_ABORT)) return true;
    if (value != seen) {
      start(patience, value);
      return false;
    }
    quiet += WATCH_EVERY;
    if (now_ticks() > limit || quiet >= SPIN_MAX_ITERS) {
      ev_store_relaxed(sched + W_STATUS, 5 /* ETC_ERR_TIMEOUT */);
      ev_store_relaxed(sched + W_AUX, where);
      ev_store(sched + W_ABORT, 1);
      return true;
    }
    return false;
  }
};

// Spin (one lane) until *ctr >= target.  Returns false if the call was aborted, by
// this wait giving up or by another workgroup.
ETC_DEV bool spin_until_geq(const int* ctr, int target, int* sched, uint64_t patience,
                            int where) {
  Watchdog wd;
  for (int it = 0;; ++it) {
    const int v = ev_load_relaxed(ctr);
    if (v >= target) {
      fence_acquire_agent();  // everything released before the counter reached v
      return true;
    }
    if (it == 0) wd.start(patience, v);
    else if (it % WATCH_EVERY == 0 && wd.expired(sched, patience, v, where)) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// ------------------------------------------------------------------ wave helpers

// Lane exchanges inside rows of 16 lanes through DPP (no LDS round trip): swap with the
// neighbour (lane ^ 1), swap pairs (lane ^ 2), mirror each half row (lane i <-> 7 - i)
// and mirror the row (lane i <-> 15 - i).  Applied in that order with a commutative
// operation they form a butterfly, so every lane of the row ends with the same result,
// bit for bit.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

template <int CTRL>
ETC_DEV int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
ETC_DEV float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

// The sum over each row of 16 lanes, identical in every lane of the row.
ETC_DEV float row16_sum(float v) {
  v += dpp_f<DPP_XOR1>(v);
  v += dpp_f<DPP_XOR2>(v);
  v += dpp_f<DPP_HALF_MIRROR>(v);
  v += dpp_f<DPP_MIRROR>(v);
  return v;
}

ETC_DEV float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return v;
}

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled: register arrays indexed
// inside stay indexed by compile-time constants
template <typename F, int... I>
ETC_DEV void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
ETC_DEV void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace etc
