// Split-K GEMM driven by event counters, as one persistent kernel.
//
// The podcast episode page "Prompt Boundary-Aware Scheduling with Event Tensors for
// Dynamic Kernels" (summary) illustrates waiting on true data dependencies with a
// split-K summation: C = A B with the K range cut into S slices; each (tile, slice)
// task produces a partial tile, and the tile's sum starts as soon as its S partials
// exist instead of after a kernel boundary.  Here the event tensor is ev[tile], one
// int32 per output tile with target S.
//
// Tasks, for T_out = ceil(M/64) * N/128 output tiles of 64 x 128:
//   P(tile, s)  float32 partial of slice s (K/S columns of A): 4 waves, each 64 rows x
//               32 columns of bf16 MFMA 16x16x32, A and B staged through LDS; publishes
//               the partial, then ev[tile] += 1.
//   R(tile, c)  waits ev[tile] >= S (acquire); rows 8c..8c+7 of the tile are
//               C = P_0 + P_1 + ... + P_{S-1}.
// Static mode: tickets 0 .. S*T_out-1 are the partials (slice-major), then 8 reduction
// tickets per tile.  Dynamic mode: only partial tasks are handed out; the partial whose
// add returns S-1 runs the tile's reduction itself (last arriver).
//
// Operands go from global memory straight into LDS (16 bytes per lane per copy) through
// a ring of six stages of 64 k values: the copies run five stages ahead of the MFMAs
// (120 KiB in flight per CU), which is what it takes to stream B at HBM rate when every
// CU streams at once.  A stage holds the
// A block [64 rows][64 k] (rows of 128 bytes, chunks swizzled as in mfma.hpp) and the B
// block [64 k][128 n] (rows of 256 bytes).  B is N-contiguous while the MFMA wants 8
// consecutive k per lane, so a lane's B fragment comes from two transposed LDS reads
// (gfx950 ds_read_b64_tr_b16, 4 k each; see lds_read_tr16_x8).  The 16-byte chunk c of B
// row r sits at position c ^ bsw(r) with bsw(r) = 2 * ((r % 4) + 4 * ((r / 8) % 2)): the
// 16 rows one transposed read touches fall on 8 different chunk pairs, two rows each,
// which is as few bank conflicts as 512 bytes per read allow.
#include <mutex>

#include "common.hpp"
#include "host.hpp"
#include "mfma.hpp"

namespace etc {
namespace splitk {

constexpr int TM = 64, TN = 128, BK = 64;
// Each tile's counter has a 128-byte line of its own: the reductions waiting on one tile
// poll its line while the partials of the other tiles signal theirs.  With all counters
// in one line, the polls held up those signals (static split-K 37 -> 32 us when the
// counters moved apart).
constexpr int EV_STRIDE = W_LINE;
constexpr int A_STAGE = TM * 128;                    // bytes (64 rows x 64 bf16)
constexpr int B_STAGE = BK * TN * 2;                 // bytes (64 k-rows x 128 bf16)
constexpr int STAGE = A_STAGE + B_STAGE;             // 24 KiB
constexpr int NSTAGE = 6;
constexpr int AHEAD = NSTAGE - 1;                    // stages in flight beyond the current
constexpr int RCHUNKS = 8;                           // row chunks of a tile's reduction
constexpr int A_LOADS = TM * 8 / NT;                 // 16-byte copies per thread: 2
constexpr int B_LOADS = BK * (TN / 8) / NT;          // 4
constexpr int LOADS = A_LOADS + B_LOADS;

struct Args {
  int M, N, K, S;
  int tiles_m, tiles_n, tiles;
  int mode;
  uint32_t flags;
  const bf16* A;
  const bf16* B;
  float* C;
  float* part;   // [tiles][S][TM][TN]
  int* sched;    // control words
  int* ev;       // [tiles] counters, EV_STRIDE words apart
  int* status;   // or null: the last workgroup out copies the status word here
  uint64_t timeout_ticks;
};

struct Smem {
  alignas(16) char stage[NSTAGE][STAGE];
  int task;  // broadcast slot
  int flag;
};

ETC_DEV int bsw(int krow) { return 2 * ((krow & 3) + 4 * ((krow >> 3) & 1)); }

// Eight transposed reads of 16-bit values (gfx950 ds_read_b64_tr_b16) at base + off[i].
// In each group of 16 lanes, lane j gives the address of 4 consecutive values (8 bytes);
// lanes 4r..4r+3 of the group thus give row r (r = 0..3) of a 4 x 16 block, and lane i
// of the group receives column i: value r of lane i is value i % 4 at the address of
// lane 4r + i / 4 (layout checked on the device with a probe of known values).
// The device code issues them as one block that waits for its own results: through the
// builtin, the compiler waits for every outstanding direct-to-LDS copy (vmcnt(0))
// before each such read, which would drain the copy ring every stage; here the ring's
// explicit waits already order the reads after the copies of their stage.  Results are
// early-clobber, so no result register shares a register with an address.
ETC_DEV void lds_read_tr16_x8(u32x2 (&o)[8], const char* base, const uint32_t (&off)[8]) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t b = (uint32_t)(uintptr_t)(const ETC_LDS char*)base;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(b + off[0]), "v"(b + off[1]), "v"(b + off[2]), "v"(b + off[3]), "v"(b + off[4]),
        "v"(b + off[5]), "v"(b + off[6]), "v"(b + off[7])
      : "memory");
#else  // host passes: the builtin (the CPU harness supplies it)
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  for (int i = 0; i < 8; ++i) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ETC_LDS s16x4*)(base + off[i]));
    __builtin_memcpy(&o[i], &v, sizeof(v));
  }
#endif
}

// The partial of (tile, s).  Thread 0 draws the workgroup's next ticket with `draw`
// right after the first copies go out, so that the atomic's round trip overlaps the
// stream (it is older than every later copy, so the ring's counted waits stay upper
// bounds), and maps the result with `map` only at the end: a use of the result inside
// the stream would make the wave wait for every copy issued before the atomic.  The
// ticket is in sm.task when the partial returns.
template <typename Draw, typename Map>
ETC_DEV void partial_task(const Args& p, Smem& sm, int tile, int s, Draw draw, Map map) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tm = tile / p.tiles_n, tn = tile % p.tiles_n;
  const int m0 = tm * TM, n0 = tn * TN;
  const int ks = p.K / p.S, kbeg = s * ks;
  const int nk = ks / BK, last = nk - 1;

  // copy sources: A rows 8w + 32i + lane/8 at the chunk its swizzled LDS position holds
  // (rows past M repeat row M-1; their results are not stored); B k-rows 16i + 4w +
  // lane/16 at chunk (lane % 16) ^ bsw(row)
  const char* asrc[A_LOADS];
  const char* bsrc[B_LOADS];
  const int lca = (lane & 7) ^ ((4 * w + (lane >> 4)) & 7);
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int m = min(m0 + 8 * w + 32 * i + (lane >> 3), p.M - 1);
    asrc[i] = reinterpret_cast<const char*>(p.A + (size_t)m * p.K + kbeg) + lca * 16;
  }
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int r = 16 * i + 4 * w + (lane >> 4);
    const int c = (lane & 15) ^ bsw(r);
    bsrc[i] = reinterpret_cast<const char*>(p.B + (size_t)(kbeg + r) * p.N + n0) + c * 16;
  }
  const size_t bstep = (size_t)BK * p.N * 2;  // bytes of B per stage

  auto issue = [&](int kt) ETC_INLINE {
    const int st = min(kt, last);  // past the last stage: re-read it into an unread slot
    char* slot = sm.stage[kt % NSTAGE];
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) lds_dma16(asrc[i] + (size_t)st * 128, slot + (8 * w + 32 * i) * 128);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i)
      lds_dma16(bsrc[i] + (size_t)st * bstep, slot + A_STAGE + (16 * i + 4 * w) * 256);
  };

  f32x4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i < AHEAD; ++i) issue(i);
  int next = 0;
  if (tid == 0) next = draw();
  for (int kt = 0; kt < nk; ++kt) {
    // this thread's copies of stage kt have landed (those of the next AHEAD-1 stages may
    // not), then every wave's have, and every wave has finished reading slot
    // (kt-1) mod NSTAGE, which stage kt+AHEAD overwrites
    vm_wait_barrier<(AHEAD - 1) * LOADS>();
    issue(kt + AHEAD);
    const char* base = sm.stage[kt % NSTAGE];
    // B fragments of the stage: lane i16 of k group g gives k-row kk*32 + 8g + 4h + i16/4,
    // columns n .. n+3 with n = w*32 + j*16 + 4*(i16 % 4); it receives column
    // w*32 + j*16 + i16 of k-rows kk*32 + 8g + 4h .. +3, so the reads h = 0, 1 hold its
    // 8 consecutive k of block (kk, j)
    const int g = lane >> 4, i16 = lane & 15;
    uint32_t boff[8];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int n = w * 32 + j * 16 + 4 * (i16 & 3);
          const int r = kk * 32 + 8 * g + 4 * hh + (i16 >> 2);
          boff[kk * 4 + j * 2 + hh] = A_STAGE + r * 256 + (((n >> 3) ^ bsw(r)) << 4) + ((n & 4) << 1);
        }
    u32x2 bt[8];
    lds_read_tr16_x8(bt, base, boff);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = lds_chunk_v(base, i * 16 + i16, kk * 4 + g);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x2 lo = bt[kk * 4 + j * 2], hi = bt[kk * 4 + j * 2 + 1];
        b[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma16(acc[i][j], a[i], b[j], (const bf16*)nullptr);
    }
  }
  // the last copies (re-reads past the last stage) land before LDS is reused
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
  __syncthreads();

  // The partial is read by another workgroup: agent-scope stores (see st_shared), 16
  // bytes each, so the tile goes through LDS first (the ring is free now; row stride
  // TN + 4 floats keeps the four row groups of a write in different banks and the rows
  // 16-byte aligned).
  constexpr int PSTR = TN + 4;
  static_assert(TM * PSTR * 4 <= (int)sizeof(sm.stage), "staged partial fits the ring");
  float* pt = reinterpret_cast<float*>(&sm.stage[0][0]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        pt[(i * 16 + (lane >> 4) * 4 + r) * PSTR + w * 32 + j * 16 + (lane & 15)] = acc[i][j][r];
  __syncthreads();
  float* dst = p.part + ((long)tile * p.S + s) * (TM * TN);
  for (int q = tid; q < TM * TN / 4; q += NT) {
    const int row = q / (TN / 4), c = (q % (TN / 4)) * 4;
    const f32x4 v = *reinterpret_cast<const f32x4*>(pt + row * PSTR + c);
    st_shared16(dst, (uint32_t)((row * TN + c) * sizeof(float)),
                u32x4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)});
  }
  if (tid == 0) sm.task = map(next);
}

// Rows [rc*TM/RCHUNKS, ...) of a C tile = partials summed in slice order.  Every thread
// owns one float4 of the chunk and has all of its S loads in flight together.
ETC_DEV void reduce_task(const Args& p, int tile, int rc) {
  constexpr int ROWS = TM / RCHUNKS, F4 = ROWS * TN / 4;  // 8 rows: 256 float4
  static_assert(F4 == NT, "one float4 per thread");
  const int tm = tile / p.tiles_n, tn = tile % p.tiles_n;
  const int e4 = threadIdx.x, row = rc * ROWS + (e4 * 4) / TN, col = (e4 * 4) % TN;
  const float* src = p.part + (long)tile * p.S * (TM * TN) + row * TN + col;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < p.S; s0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = (s0 + u < p.S) ? *reinterpret_cast<const float4*>(src + (long)(s0 + u) * TM * TN)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      sum.x += v[u].x; sum.y += v[u].y; sum.z += v[u].z; sum.w += v[u].w;
    }
  }
  const int m = tm * TM + row;
  if (m < p.M) *reinterpret_cast<float4*>(p.C + (long)m * p.N + tn * TN + col) = sum;
}

// Rows [rc0*TM/RCHUNKS, (rc0+NC)*TM/RCHUNKS) of a C tile = partials summed in slice
// order.  Every thread owns one float4 of each of the NC row chunks and has the loads of
// up to 8 slices of all NC chunks in flight together.
template <int NC>
ETC_DEV void reduce_chunks(const Args& p, int tile, int rc0) {
  constexpr int ROWS = TM / RCHUNKS, F4 = ROWS * TN / 4;  // 8 rows: 256 float4
  static_assert(F4 == NT, "one float4 per thread");
  const int tm = tile / p.tiles_n, tn = tile % p.tiles_n;
  const int e4 = threadIdx.x, r = (e4 * 4) / TN, col = (e4 * 4) % TN;
  const float* src = p.part + (long)tile * p.S * (TM * TN) + (rc0 * ROWS + r) * TN + col;
  float4 sum[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) sum[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < p.S; s0 += 8) {
    float4 v[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[c][u] = (s0 + u < p.S)
                      ? *reinterpret_cast<const float4*>(src + (long)(s0 + u) * TM * TN + c * ROWS * TN)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        sum[c].x += v[c][u].x; sum[c].y += v[c][u].y; sum[c].z += v[c][u].z; sum[c].w += v[c][u].w;
      }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int m = tm * TM + (rc0 + c) * ROWS + r;
    if (m < p.M) *reinterpret_cast<float4*>(p.C + (long)m * p.N + tn * TN + col) = sum[c];
  }
}

__global__ __launch_bounds__(NT) void splitk_kernel(Args p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int nparts = p.tiles * p.S;
  // static: the partials, then RCHUNKS reduction tickets per tile
  const bool stat = p.mode == ETC_SCHED_STATIC;
  const int total = stat ? nparts + p.tiles * RCHUNKS : nparts;
  // Static: partial tickets are slice-major, so a chunk of consecutive tickets (one XCD
  // queue's share) holds the tiles of one slice, which share its A block.  Dynamic: one
  // counter.  A workgroup draws its next ticket while its current task runs.  (No check
  // of the abort flag here: partial tasks never wait, and a reduction's wait sees the
  // flag and gives up, so every workgroup still leaves after an abort.)
  auto draw = [&]() ETC_INLINE {
    return stat ? xcd_ticket_draw(p.sched) : ticket_inc(p.sched + W_QHEAD);
  };
  auto map = [&](int drawn) ETC_INLINE { return stat ? xcd_ticket_map(drawn) : drawn; };
  if (tid == 0) sm.task = map(draw());
  __syncthreads();
  int t = sm.task;
  __syncthreads();

  while (t < total) {
    if (t < nparts) {
      const int tile = t % p.tiles, s = t / p.tiles;
      partial_task(p, sm, tile, s, draw, map);  // leaves the next ticket in sm.task
      publish_shared();
      if (tid == 0) {
        if (stat) {
          // nothing waits on the result: the atomic goes out without a return
          ev_signal(p.ev + EV_STRIDE * tile, 1);
          sm.flag = 0;
        } else {
          // the last arriver reduces, so its signal acquires every other partial
          sm.flag = ev_add_acquire(p.ev + EV_STRIDE * tile, 1) == p.S - 1 ? 1 : 0;
        }
      }
      __syncthreads();
      if (sm.flag)  // last arriver: the whole tile, a quarter of it per round trip
        for (int rc = 0; rc < RCHUNKS; rc += RCHUNKS / 4) reduce_chunks<RCHUNKS / 4>(p, tile, rc);
    } else {
      const int tile = (t - nparts) / RCHUNKS, rc = (t - nparts) % RCHUNKS;
      if (tid == 0) {
        const int next = draw();  // in flight during the wait
        sm.flag = spin_until_geq(p.ev + EV_STRIDE * tile, p.S, p.sched, p.timeout_ticks, 1) ? 1 : 0;
        sm.task = map(next);
      }
      __syncthreads();
      if (sm.flag) reduce_task(p, tile, rc);
    }
    t = sm.task;
    __syncthreads();  // every thread has read sm.task before the next task rewrites it
  }

  // the last workgroup out clears the counters for the next call
  wg_publish();
  if (tid == 0) sm.flag = (atomicAdd(p.sched + W_EXIT, 1) == (int)gridDim.x - 1) ? 1 : 0;
  __syncthreads();
  if (sm.flag && tid == 0 && p.status) gp(p.status)[0] = ev_load_relaxed(p.sched + W_STATUS);
  if (sm.flag && !(p.flags & ETC_FLAG_KEEP_COUNTERS)) {
    for (int i = tid; i < p.tiles; i += NT) ev_store_relaxed(p.ev + EV_STRIDE * i, 0);
    for (int i = tid; i < W_NWORDS; i += NT)
      if (i != W_STATUS && i != W_AUX) ev_store_relaxed(p.sched + i, 0);
  }
}

// Clears n int32 words at p: the control words and counters of a scratch buffer that
// an earlier call may have left dirty (a fill kernel rather than a memset, so that the
// clear can sit inside a captured graph).
__global__ __launch_bounds__(NT) void clear_words(int* p, int n) {
  for (int i = blockIdx.x * NT + threadIdx.x; i < n; i += gridDim.x * NT) p[i] = 0;
}

struct Layout {
  size_t sched, ev, part, total;
  int tiles;
};

inline Layout layout(int M, int N, int S) {
  Layout L;
  L.tiles = cdiv(M, TM) * (N / TN);
  host::Carve c;
  L.sched = c.take(W_NWORDS * sizeof(int));
  L.ev = c.take((size_t)L.tiles * EV_STRIDE * sizeof(int));
  L.part = c.take((size_t)L.tiles * S * TM * TN * sizeof(float));
  L.total = c.off;
  return L;
}

// Scratch of the allocation-free entry point: one array per device, held until the
// process ends.  Host code never uses this name as an address (in host code it is a
// stand-in); it uses the device address recorded by scratch_ptr().
constexpr size_t SCRATCH_BYTES = (size_t)16 << 20;
static __device__ __align__(256) char scratch[SCRATCH_BYTES];

// Device address of `scratch` on device dev (current), looked up once per device.
void* scratch_ptr(int dev) {
  static std::mutex mu;
  static void* ptr[host::MAX_DEVICES] = {nullptr};
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

}  // namespace splitk
}  // namespace etc

using namespace etc;

int splitk_default_workers(int dev);

static int splitk_occupancy(int dev) {
  static int occ[host::MAX_DEVICES] = {0};
  if (occ[dev] == 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, splitk::splitk_kernel, NT, 0) != hipSuccess || v < 1)
      v = 1;
    occ[dev] = v;
  }
  return occ[dev];
}

int splitk_default_workers(int dev) { return host::device_cus(dev) * splitk_occupancy(dev); }

static bool splitk_shape_ok(int32_t M, int32_t N, int32_t K, int32_t S) {
  return M >= 1 && N >= 1 && K >= 1 && S >= 1 && S <= 64 && N % splitk::TN == 0 &&
         K % (splitk::BK * S) == 0;
}

ETC_API size_t etc_splitk_workspace_size(int32_t M, int32_t N, int32_t split_k) {
  if (M < 1 || N < 1 || N % splitk::TN || split_k < 1 || split_k > 64) return 0;
  return splitk::layout(M, N, split_k).total;
}

static etc_status splitk_launch(int32_t M, int32_t N, int32_t K, int32_t split_k, const void* A,
                                const void* B, float* C, void* workspace, size_t workspace_bytes,
                                etc_sched_mode mode, uint32_t flags, int32_t workers, void* stream,
                                bool clear_first, int32_t* status);

ETC_API etc_status etc_splitk_gemm(int32_t M, int32_t N, int32_t K, int32_t split_k,
                                   const void* A, const void* B, float* C, void* workspace,
                                   size_t workspace_bytes, etc_sched_mode mode, uint32_t flags,
                                   int32_t workers, void* stream) {
  return splitk_launch(M, N, K, split_k, A, B, C, workspace, workspace_bytes, mode, flags, workers, stream,
                       false, nullptr);
}

ETC_API etc_status etc_splitk_gemm_noalloc(int32_t M, int32_t N, int32_t K, int32_t split_k, const void* A,
                                           const void* B, float* C, int32_t* status, etc_sched_mode mode,
                                           uint32_t flags, int32_t workers, void* stream) {
  if (M < 1 || N < 1 || K < 1 || split_k < 1) return ETC_ERR_INVALID_ARG;
  if (!A || !B || !C) return ETC_ERR_INVALID_ARG;
  if (status && (reinterpret_cast<uintptr_t>(status) & 3u)) return ETC_ERR_INVALID_ARG;
  if (!splitk_shape_ok(M, N, K, split_k)) return ETC_ERR_UNSUPPORTED;
  if (splitk::layout(M, N, split_k).total > splitk::SCRATCH_BYTES) return ETC_ERR_WORKSPACE;
  const int dev = host::current_gfx950_device();
  if (dev < 0) return ETC_ERR_NO_DEVICE;
  void* ws = splitk::scratch_ptr(dev);
  if (!ws) return ETC_ERR_HIP;
  return splitk_launch(M, N, K, split_k, A, B, C, ws, splitk::SCRATCH_BYTES, mode, flags, workers, stream,
                       true, status);
}

static etc_status splitk_launch(int32_t M, int32_t N, int32_t K, int32_t split_k, const void* A,
                                const void* B, float* C, void* workspace, size_t workspace_bytes,
                                etc_sched_mode mode, uint32_t flags, int32_t workers, void* stream,
                                bool clear_first, int32_t* status) {
  if (M < 1 || N < 1 || K < 1 || split_k < 1) return ETC_ERR_INVALID_ARG;
  if (!A || !B || !C) return ETC_ERR_INVALID_ARG;
  if (mode != ETC_SCHED_STATIC && mode != ETC_SCHED_DYNAMIC) return ETC_ERR_INVALID_ARG;
  if (!host::aligned16(A) || !host::aligned16(B) || !host::aligned16(C)) return ETC_ERR_INVALID_ARG;
  if (!splitk_shape_ok(M, N, K, split_k)) return ETC_ERR_UNSUPPORTED;
  const splitk::Layout L = splitk::layout(M, N, split_k);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < L.total)
    return ETC_ERR_WORKSPACE;
  const int dev = host::current_gfx950_device();
  if (dev < 0) return ETC_ERR_NO_DEVICE;

  splitk::Args p;
  p.M = M; p.N = N; p.K = K; p.S = split_k;
  p.tiles_m = cdiv(M, splitk::TM);
  p.tiles_n = N / splitk::TN;
  p.tiles = L.tiles;
  p.mode = mode;
  p.flags = flags;
  p.A = static_cast<const bf16*>(A);
  p.B = static_cast<const bf16*>(B);
  p.C = C;
  char* ws = static_cast<char*>(workspace);
  p.sched = reinterpret_cast<int*>(ws + L.sched);
  p.ev = reinterpret_cast<int*>(ws + L.ev);
  p.part = reinterpret_cast<float*>(ws + L.part);
  p.status = status;
  p.timeout_ticks = 500000000ull;  // 5 s without progress, on the 100 MHz real-time clock

  const int grid = host::grid_size(workers, host::device_cus(dev), splitk_occupancy(dev));
  if (clear_first) {
    // the shared scratch keeps the last call's contents: its control words and counters
    // (everything before the partials, including the status word) start at zero
    const int words = (int)(L.part / sizeof(int));
    hipLaunchKernelGGL(splitk::clear_words, dim3(cdiv(words, NT)), dim3(NT), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<int*>(workspace), words);
    if (hipGetLastError() != hipSuccess) return ETC_ERR_HIP;
  }
  hipLaunchKernelGGL(splitk::splitk_kernel, dim3(grid), dim3(NT), 0, static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? ETC_OK : ETC_ERR_HIP;
}
