// CPU stand-in for <hip/hip_runtime.h>, used only to compile the library's HIP sources
// unchanged as host C++ for the CPU execution harness in tests/ (never for the GPU).
//
// Model: a kernel launch runs every workgroup as an OS thread; the lanes of a
// workgroup are cooperative fibers on that thread.  __syncthreads is a barrier over
// the workgroup's fibers; shuffles and MFMA are wave-collective (the 64 lanes of a
// wave deposit their operands, meet, compute, meet again); global-memory atomics are
// host atomics; s_sleep yields.  The MFMA lane layouts are the ones the kernels assume
// (and that an on-GPU probe confirmed): lane l holds row / column l % 16 and k values
// 8*(l/16)..+7 (bf16 16x16x32) or k = l/16 (f32 16x16x4); result element r of lane l is
// row 4*(l/16) + r, column l % 16.
#pragma once

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <functional>

#define __global__
#define __device__
#define __align__(n) __attribute__((aligned(n)))
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
// __shared__ objects are per-workgroup: one OS thread runs each workgroup.
#define __shared__ static thread_local

typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
typedef struct ihipStream_t* hipStream_t;
enum hipMemcpyKind { hipMemcpyHostToDevice = 1, hipMemcpyDeviceToHost = 2, hipMemcpyDeviceToDevice = 3 };
enum hipDeviceAttribute_t { hipDeviceAttributeMultiprocessorCount = 1 };

struct hipDeviceProp_t {
  char gcnArchName[256];
};

struct dim3 {
  unsigned x, y, z;
  dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
struct uint2 { unsigned x, y; };
struct uint4 { unsigned x, y, z, w; };
struct float4 { float x, y, z, w; };
inline uint2 make_uint2(unsigned a, unsigned b) { return uint2{a, b}; }
inline uint4 make_uint4(unsigned a, unsigned b, unsigned c, unsigned d) { return uint4{a, b, c, d}; }
inline float4 make_float4(float a, float b, float c, float d) { return float4{a, b, c, d}; }

typedef __bf16 emu_bf16x8 __attribute__((ext_vector_type(8)));
typedef float emu_f32x4 __attribute__((ext_vector_type(4)));

struct EmuDim { unsigned x, y, z; };
EmuDim emu_thread_idx();
EmuDim emu_block_idx();
EmuDim emu_grid_dim();
EmuDim emu_block_dim();
#define threadIdx emu_thread_idx()
#define blockIdx emu_block_idx()
#define gridDim emu_grid_dim()
#define blockDim emu_block_dim()

void emu_syncthreads();
void emu_wave_barrier();
void emu_yield();
void* emu_wave_scratch(int bytes_per_lane);  // this wave's exchange buffer (64 lanes)
int emu_lane();
uint64_t emu_realtime();
#define __syncthreads() emu_syncthreads()
int emu_syncthreads_or(int v);
#define __syncthreads_or(v) emu_syncthreads_or(v)
#define __expf(x) expf(x)

template <typename T>
inline T emu_exchange(T v, int src) {
  unsigned char* buf = static_cast<unsigned char*>(emu_wave_scratch(sizeof(T)));
  const int lane = emu_lane();
  memcpy(buf + lane * sizeof(T), &v, sizeof(T));
  emu_wave_barrier();
  T out;
  memcpy(&out, buf + src * sizeof(T), sizeof(T));
  emu_wave_barrier();
  return out;
}
template <typename T>
inline T __shfl_xor(T v, int mask, int width = 64) {
  const int lane = emu_lane();
  const int base = lane & ~(width - 1);
  return emu_exchange(v, base + ((lane - base) ^ mask) % width);
}
template <typename T>
inline T __shfl_up(T v, unsigned delta, int width = 64) {
  const int lane = emu_lane();
  const int base = lane & ~(width - 1);
  const int src = lane - (int)delta;
  return emu_exchange(v, src < base ? lane : src);
}

// lane 0's value; every use in the kernels passes a wave-uniform value, which is checked
inline int emu_readfirstlane(int v) {
  const int first = emu_exchange(v, 0);
  if (first != v) {
    fprintf(stderr, "readfirstlane of a non-uniform value\n");
    abort();
  }
  return first;
}
#define __builtin_amdgcn_readfirstlane(x) emu_readfirstlane(x)

// bit l set when lane l's predicate holds (every lane of the wave takes part)
inline unsigned long long emu_ballot(int pred) {
  unsigned char* buf = static_cast<unsigned char*>(emu_wave_scratch(1));
  const int lane = emu_lane();
  buf[lane] = pred ? 1 : 0;
  emu_wave_barrier();
  unsigned long long m = 0;
  for (int i = 0; i < 64; ++i)
    if (buf[i]) m |= 1ull << i;
  emu_wave_barrier();
  return m;
}
#define __ballot(x) emu_ballot(x)

// Transposed 16-bit LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, value r of
// lane i is value i % 4 at the address given by lane 4r + i / 4 of the group.
typedef short emu_s16x4 __attribute__((ext_vector_type(4)));
inline emu_s16x4 emu_read_tr16(const void* p) {
  const int lane = emu_lane(), grp = lane & ~15, i = lane & 15;
  emu_s16x4 out;
  for (int r = 0; r < 4; ++r) {
    const uintptr_t a = emu_exchange((uintptr_t)p, grp + 4 * r + i / 4);
    out[r] = reinterpret_cast<const short*>(a)[i % 4];
  }
  return out;
}
#define __builtin_amdgcn_ds_read_tr16_b64_v4i16(p) emu_read_tr16((const void*)(p))
#define __builtin_amdgcn_wave_barrier() emu_wave_barrier()
inline int __popcll(unsigned long long v) { return __builtin_popcountll(v); }

template <typename T>
inline T min(T a, T b) { return b < a ? b : a; }
template <typename T>
inline T max(T a, T b) { return a < b ? b : a; }

inline float __uint_as_float(unsigned u) { float f; memcpy(&f, &u, 4); return f; }
inline unsigned __float_as_uint(float f) { unsigned u; memcpy(&u, &f, 4); return u; }
inline float __int_as_float(int u) { float f; memcpy(&f, &u, 4); return f; }
inline int __float_as_int(float f) { int u; memcpy(&u, &f, 4); return u; }

// DPP moves used by the kernels: quad permutations and the two row mirrors
inline int emu_update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask, bool bc) {
  (void)old; (void)row_mask; (void)bank_mask; (void)bc;
  const int lane = emu_lane();
  int from;
  if (ctrl < 0x100) from = (lane & ~3) | ((ctrl >> (2 * (lane & 3))) & 3);
  else if (ctrl == 0x140) from = (lane & ~15) | (15 - (lane & 15));
  else if (ctrl == 0x141) from = (lane & ~7) | (7 - (lane & 7));
  else {
    fprintf(stderr, "unsupported DPP control 0x%x\n", ctrl);
    abort();
  }
  return emu_exchange(src, from);
}
#define __builtin_amdgcn_update_dpp(old, src, ctrl, rm, bm, bc) emu_update_dpp((old), (src), (ctrl), (rm), (bm), (bc))

inline int atomicAdd(int* p, int v) { return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST); }
// increment that wraps to 0 past lim (the device's atomic_inc)
inline unsigned emu_atomic_inc32(unsigned* p, unsigned lim) {
  unsigned old = __atomic_load_n(p, __ATOMIC_RELAXED);
  while (!__atomic_compare_exchange_n(p, &old, old >= lim ? 0u : old + 1u, false, __ATOMIC_SEQ_CST,
                                      __ATOMIC_RELAXED)) {
  }
  return old;
}
#define __builtin_amdgcn_atomic_inc32(p, lim, order, scope) emu_atomic_inc32((unsigned*)(p), (lim))
inline unsigned atomicOr(unsigned* p, unsigned v) { return __atomic_fetch_or(p, v, __ATOMIC_SEQ_CST); }
inline int __popc(unsigned v) { return __builtin_popcount(v); }
inline float atomicAdd(float* p, float v) {
  unsigned* u = reinterpret_cast<unsigned*>(p);
  unsigned old = __atomic_load_n(u, __ATOMIC_RELAXED);
  while (true) {
    const unsigned nw = __float_as_uint(__uint_as_float(old) + v);
    if (__atomic_compare_exchange_n(u, &old, nw, false, __ATOMIC_SEQ_CST, __ATOMIC_RELAXED))
      return __uint_as_float(old);
  }
}

#define __HIP_MEMORY_SCOPE_AGENT 3
// host memory has one address space
#define ETC_GLOBAL
#define ETC_LDS
// ThreadSanitizer builds treat every device-scope atomic as sequentially consistent.  On
// the GPU a signal is a relaxed atomic issued after the workgroup's shared stores have
// completed (publish_shared), so it orders those stores before it at the point of
// coherence; a host memory model has no such completion wait, and only ordered atomics
// carry the edge.  What TSan checks is then that every read of another workgroup's data
// is ordered after the writes by some chain of atomics (a signal, a mailbox word).
#ifdef ETC_EMU_SC_ATOMICS
#define EMU_ORDER(order) __ATOMIC_SEQ_CST
#else
#define EMU_ORDER(order) (order)
#endif
#define __hip_atomic_load(p, order, scope) __atomic_load_n((p), EMU_ORDER(order))
#define __hip_atomic_store(p, v, order, scope) __atomic_store_n((p), (v), EMU_ORDER(order))
#define __hip_atomic_fetch_add(p, v, order, scope) __atomic_fetch_add((p), (v), EMU_ORDER(order))
#define __builtin_amdgcn_fence(order, scope) __atomic_thread_fence(order)
void emu_waitcnt(int imm);
#define __builtin_amdgcn_s_waitcnt(x) emu_waitcnt(x)
#define __builtin_amdgcn_s_sleep(x) emu_yield()
#define __builtin_amdgcn_s_memrealtime() emu_realtime()

// global_load_lds: lane l writes 16 bytes at the wave's LDS base + 16 * l.  By default
// the copy lands at once (a copy that overwrites LDS still being read then shows up as a
// wrong result); with ETC_EMU_DMA_LATE it lands only at the lane's s_waitcnt whose
// vector-memory count excludes it, oldest first (a read of LDS before its wait then
// shows up).  Only these copies are counted, so a wait lands no more of them than the
// GPU's count, which also includes the other vector-memory operations, would.
void emu_dma_issue(void* dst, const void* src, int size);
inline void emu_global_load_lds(const void* src, void* lds_base, int size, int off) {
  emu_dma_issue(static_cast<char*>(lds_base) + off + emu_lane() * size, src, size);
}
#define __builtin_amdgcn_global_load_lds(src, dst, size, off, aux) \
  emu_global_load_lds((const void*)(src), (void*)(dst), (size), (off))
#define __builtin_amdgcn_s_barrier() emu_syncthreads()
// raw buffer stores: the resource is the base address; the 16 bytes go out as two
// 8-byte atomic stores (device-scope stores are atomic in this stand-in as well)
typedef char* __amdgpu_buffer_rsrc_t;
#define __builtin_amdgcn_make_buffer_rsrc(p, stride, num, flags) ((char*)(p))
template <typename V>
inline void emu_buffer_store16(const V& v, char* base, int off, int soff) {
  uint64_t w[2];
  memcpy(w, &v, 16);
  uint64_t* d = reinterpret_cast<uint64_t*>(base + off + soff);
  __atomic_store_n(d, w[0], EMU_ORDER(__ATOMIC_RELAXED));
  __atomic_store_n(d + 1, w[1], EMU_ORDER(__ATOMIC_RELAXED));
}
#define __builtin_amdgcn_raw_buffer_store_b128(v, r, off, soff, aux) emu_buffer_store16((v), (r), (off), (soff))
#define __builtin_amdgcn_sched_barrier(mask) ((void)0)
#define __builtin_amdgcn_sched_group_barrier(mask, n, id) ((void)0)

emu_f32x4 emu_mfma_bf16(emu_bf16x8 a, emu_bf16x8 b, emu_f32x4 c);
emu_f32x4 emu_mfma_f32(float a, float b, emu_f32x4 c);
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, x, y, z) emu_mfma_bf16((a), (b), (c))
#define __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, x, y, z) emu_mfma_f32((a), (b), (c))

// ---- host API
hipError_t hipGetDevice(int* d);
hipError_t hipGetDeviceProperties(hipDeviceProp_t* p, int d);
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t a, int d);
hipError_t hipMemsetAsync(void* p, int v, size_t n, hipStream_t s);
hipError_t hipMemcpyAsync(void* d, const void* s, size_t n, hipMemcpyKind k, hipStream_t st);
hipError_t hipStreamSynchronize(hipStream_t s);
hipError_t hipGetLastError();
template <typename F>
hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* v, F, int, size_t) {
  *v = 1;
  return hipSuccess;
}
void emu_launch(unsigned grid, unsigned block, std::function<void()> fn);
// a device variable's address is its host address here
#define HIP_SYMBOL(x) (x)
template <typename T>
hipError_t hipGetSymbolAddress(void** p, T& sym) {
  *p = (void*)&sym;
  return hipSuccess;
}
#define hipLaunchKernelGGL(kernel, grid, block, shm, stream, ...) \
  emu_launch((grid).x, (block).x, [=]() { kernel(__VA_ARGS__); })
