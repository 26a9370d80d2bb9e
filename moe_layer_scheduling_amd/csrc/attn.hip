// Variable-context decode attention with split-KV partials merged through event
// counters, as one persistent kernel.
//
// The tutorial chapter "5 · Event Tensor et le dynamisme" names the context length of
// each request as a source of shape dynamism (§5.1) and notes that when the number of
// producer tasks depends on such a length, the counter targets are computed at run time
// on the GPU before anyone waits (§5.5 Obstacle 1).  The podcast episode page "Prompt
// Boundary-Aware Scheduling with Event Tensors for Dynamic Kernels" (summary) uses
// split-K summation as its example of waiting on true data dependencies.  Here the key
// and value cache of request b (L_b tokens) is cut into n_b = ceil(L_b / CH) chunks; each
// (request, KV head, chunk) task writes a partial (max score, sum of weights, weighted
// value sum) per query head and adds 1 to ev[b][kv head]; the head's output is merged
// once that counter reaches n_b, a target that depends on the request's length.  The
// lengths are device data: every workgroup derives n_b and the task numbering from them
// at the start of the call, so one compiled kernel serves any mix of lengths.
//
// Per query head h = g*G + i (G query heads share KV head g), with s_t = scale * q . k_t:
//   partial of chunk c:  m_c = max s_t, l_c = sum exp(s_t - m_c), o_c = sum exp(s_t - m_c) v_t
//   merge:               M = max m_c, L = sum l_c exp(m_c - M), out = sum o_c exp(m_c - M) / L
//
// Tasks (256 threads, four waves):
//   P(b, g, c)  the chunk's 256 tokens (contiguous rows of head g's cache, which is
//               stored head-major: [H_kv][rows][128]): wave w takes tokens 64w .. 64w+63.  Scores come
//               from bf16 MFMA 16x16x32 (the G query heads padded to 16 rows as the A
//               operand, 16 tokens per block as the B operand, K read straight into
//               registers in the MFMA layout); the chunk's max and weight sum per head
//               from the scores staged in LDS; the weighted value sum on the vector ALUs
//               with V rows in registers (16 lanes per token row, 8 dims per lane).  All
//               of a lane's key and value loads go out before the first MFMA.
//   M(b, g)     waits ev[b][g] >= n_b; merges the n_b partials of each of the G heads.
// Static mode: tickets 0 .. NP-1 are the partials, then one merge ticket per (b, g).
// Dynamic mode: only partials are handed out; the partial whose add completes the
// counter runs the merge (last arriver).
#include <float.h>
#include <math.h>

#include "common.hpp"
#include "host.hpp"
#include "mfma.hpp"

namespace etc {
namespace attn {

constexpr int HD = 128;          // head dimension
constexpr int CH = 256;          // tokens per partial task
constexpr int MAXG = 8;          // query heads per KV head
constexpr int MAXB = 2048;       // requests per call
constexpr int REC = HD + 4;      // floats per partial record and head: o[HD], m, l, pad
constexpr int TPW = CH / 4;      // tokens per wave: 64
// each (request, KV head) counter has a 128-byte line of its own, so that merges polling
// one counter do not hold up the partials signalling the others
constexpr int EV_STRIDE = W_LINE;

struct Args {
  int B, HKV, G;
  int mode;
  uint32_t flags;
  float scale;
  const int* lens;      // [B] context lengths (device)
  const int* kv_start;  // [B] first cache row of each request (device)
  int kv_rows;
  const bf16* q;        // [B][HKV*G][HD]
  const bf16* k;        // [HKV][kv_rows][HD]
  const bf16* v;        // [HKV][kv_rows][HD]
  float* out;           // [B][HKV*G][HD]
  float* part;          // [cap][G][REC]
  int cap;              // partial records the workspace holds
  long long max_total;  // the workspace's capacity in tokens over all requests
  int* sched;
  int* ev;              // [B][HKV] counters, EV_STRIDE words apart
  uint64_t timeout_ticks;
};

struct Smem {
  int pbase[MAXB + 1];  // first partial ticket of each request (exclusive scan of HKV * n_b)
  int nsplit[MAXB];
  int len[MAXB];        // the requests' lengths and first cache rows, read once per call
  int start[MAXB];
  int tmp[8];
  long long ltmp[4];
  alignas(16) float s[MAXG][CH];  // scores, then weights exp(s - m); 16-byte views in the merge
  float ml[MAXG][2];        // per head: chunk max, weight sum
  float o[4][MAXG][HD];     // per wave partial weighted value sums
  int task;
  int flag;
  int next;  // a ticket drawn during the previous partial task (-1: none), thread 0
};

// Every thread: the call's plan from the device arrays: n_b = ceil(L_b / CH), the
// exclusive scan of HKV * n_b, and checks of the lengths and cache rows.  Returns the
// number of partial tasks, -1 if a request's length or rows are out of range, or -2 if
// the lengths sum to more tokens than the workspace was sized for.
ETC_DEV int make_plan(const Args& p, Smem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int bad = 0;
  long long lsum = 0;
  for (int b = tid; b < p.B; b += NT) {
    const int L = gp(p.lens)[b], st = gp(p.kv_start)[b];
    const bool ok = L >= 1 && st >= 0 && (long long)st + L <= (long long)p.kv_rows;
    bad |= ok ? 0 : 1;
    lsum += ok ? L : 0;
    sm.nsplit[b] = ok ? cdiv(L, CH) : 0;
    sm.len[b] = L;
    sm.start[b] = st;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, WAVE);
  if (lane == 0) sm.ltmp[w] = lsum;
  bad = __syncthreads_or(bad);
  if (!bad && sm.ltmp[0] + sm.ltmp[1] + sm.ltmp[2] + sm.ltmp[3] > p.max_total) return -2;
  // exclusive scan of HKV * n_b over b, in chunks of NT requests
  int carry = 0;
  for (int b0 = 0; b0 < p.B; b0 += NT) {
    const int b = b0 + tid;
    const int v = b < p.B ? p.HKV * sm.nsplit[b] : 0;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, WAVE);
      if (lane >= off) x += y;
    }
    if (lane == 63) sm.tmp[w] = x;
    __syncthreads();
    int before = carry;
    for (int i = 0; i < w; ++i) before += sm.tmp[i];
    const int total = sm.tmp[0] + sm.tmp[1] + sm.tmp[2] + sm.tmp[3];
    if (b < p.B) sm.pbase[b] = before + x - v;
    __syncthreads();
    carry += total;
  }
  if (tid == 0) sm.pbase[p.B] = carry;
  __syncthreads();
  return bad ? -1 : carry;
}

// Request owning partial ticket t: the largest b with pbase[b] <= t.
ETC_DEV int owner(const Smem& sm, int B, int t) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sm.pbase[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

ETC_DEV void partial_task(const Args& p, Smem& sm, int b, int g, int c, int rec) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G, HQ = p.HKV * G;
  const int L = sm.len[b];
  const int t0 = c * CH, n = min(CH, L - t0);
  // head g's rows of the chunk are contiguous: [g][kv_start[b] + t0 + t][HD]
  const size_t row0 = (size_t)g * p.kv_rows + (size_t)sm.start[b] + t0;
  constexpr int rstride = HD;
  const bf16* kb = p.k + row0 * rstride;
  const bf16* vb = p.v + row0 * rstride;
  const int q16 = lane & 15, grp = lane >> 4;

  // every load of this lane goes out first: q (A operand, head q16, dims 32kk + 8grp),
  // K (B operand, token 16j + q16 of the wave's 64, same dims), V (token 4i + grp, dims
  // 8*q16); tokens past the chunk's end repeat its last token (their scores are masked)
  u32x4 qa[4], kf[4][4], vr[16];
  const bf16* qrow = p.q + ((size_t)b * HQ + (size_t)g * G + min(q16, G - 1)) * HD;
  static_for<4>([&](auto kk) ETC_INLINE { qa[kk] = gld<u32x4>(qrow + 32 * kk + 8 * grp); });
  static_for<4>([&](auto j) ETC_INLINE {
    const int t = min(w * TPW + 16 * j + q16, n - 1);
    static_for<4>([&](auto kk) ETC_INLINE { kf[j][kk] = gld<u32x4>(kb + t * rstride + 32 * kk + 8 * grp); });
  });
  static_for<16>([&](auto i) ETC_INLINE {
    const int t = min(w * TPW + 4 * i + grp, n - 1);
    vr[i] = gld<u32x4>(vb + t * rstride + 8 * q16);
  });
  // the workgroup's next ticket, drawn while this chunk's loads are in flight (a later
  // ticket than the running one, so the order stays deadlock-free: every partial ticket
  // precedes every merge ticket, and a partial never waits); it is read back only at the
  // end of the task, since a wait for it would also wait for every load issued before it
  int drawn = 0;
  if (tid == 0) drawn = ticket_inc(p.sched + W_TICKET);

  // scores of the wave's 64 tokens: block j holds heads 4*grp + r (rows) x tokens
  // 16j + q16 (columns)
  static_for<4>([&](auto j) ETC_INLINE {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    static_for<4>([&](auto kk) ETC_INLINE { mma16(acc, qa[kk], kf[j][kk], (const bf16*)nullptr); });
    const int tl = w * TPW + 16 * j + q16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * grp + r;
      if (h < G) sm.s[h][tl] = tl < n ? p.scale * acc[r] : -INFINITY;
    }
  });
  __syncthreads();

  // per head: chunk max and weights, 16 threads (one DPP row) per head.  Rows past the
  // last head repeat it and store nothing, so every lane of a wave takes part in the row
  // reductions.
  {
    const int h = tid >> 4, j = tid & 15, hh = min(h, G - 1);
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < CH / 16; ++k) m = fmaxf(m, sm.s[hh][j + 16 * k]);
    m = fmaxf(m, dpp_f<DPP_XOR1>(m));
    m = fmaxf(m, dpp_f<DPP_XOR2>(m));
    m = fmaxf(m, dpp_f<DPP_HALF_MIRROR>(m));
    m = fmaxf(m, dpp_f<DPP_MIRROR>(m));
    float e[CH / 16], l = 0.f;
#pragma unroll
    for (int k = 0; k < CH / 16; ++k) {
      e[k] = __expf(sm.s[hh][j + 16 * k] - m);
      l += e[k];
    }
    l = row16_sum(l);
    __syncthreads();  // every row has read its head's scores before any is overwritten
    if (h < G) {
#pragma unroll
      for (int k = 0; k < CH / 16; ++k) sm.s[h][j + 16 * k] = e[k];
      if (j == 0) {
        sm.ml[h][0] = m;
        sm.ml[h][1] = l;
      }
    }
  }
  __syncthreads();

  // weighted value sums: lane (grp, q16) accumulates dims 8*q16 .. +7 over tokens
  // 4i + grp of the wave, for every head
  float o[MAXG][8];
#pragma unroll
  for (int h = 0; h < MAXG; ++h)
#pragma unroll
    for (int d = 0; d < 8; ++d) o[h][d] = 0.f;
  static_for<16>([&](auto i) ETC_INLINE {
    float vv[8];
    expand16(vr[i], vv, (const bf16*)nullptr);
    const int tl = w * TPW + 4 * i + grp;
#pragma unroll
    for (int h = 0; h < MAXG; ++h) {
      if (h < G) {
        const float e = sm.s[h][tl];
#pragma unroll
        for (int d = 0; d < 8; ++d) o[h][d] = fmaf(e, vv[d], o[h][d]);
      }
    }
  });
  // the four token groups of the wave, then the four waves
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
    if (h < G) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        float x = o[h][d];
        x += __shfl_xor(x, 16, WAVE);
        x += __shfl_xor(x, 32, WAVE);
        o[h][d] = x;
      }
      if (grp == 0) {
#pragma unroll
        for (int d = 0; d < 8; ++d) sm.o[w][h][8 * q16 + d] = o[h][d];
      }
    }
  }
  __syncthreads();
  // the partial record of every head, read by the merge on any XCD: agent-scope stores
  float* dst = p.part + (size_t)rec * G * REC;
  // four dims per 16-byte store (a record is REC floats, a multiple of 4)
  for (int e = tid; e < G * (HD / 4); e += NT) {
    const int h = e / (HD / 4), d = (e % (HD / 4)) * 4;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = sm.o[0][h][d + i] + sm.o[1][h][d + i] + sm.o[2][h][d + i] + sm.o[3][h][d + i];
    st_shared16(dst, (uint32_t)((h * REC + d) * sizeof(float)),
                u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
  }
  if (tid < G) {
    st_shared(dst + tid * REC + HD, sm.ml[tid][0]);
    st_shared(dst + tid * REC + HD + 1, sm.ml[tid][1]);
  }
  if (tid == 0) sm.next = drawn;
}

// Output of the G query heads of (b, g) from the n_b partial records starting at rec0
// (every thread of the workgroup).  Pass 1: M = max m_c per head, each thread over every
// NT-th record, then across the workgroup.  Pass 2, CH records at a time: each thread
// turns one record's m into the weight exp(m_c - M) per head (LDS) and adds l_c times
// that weight to its share of L; then thread (s, h, d4) adds weight times o_c[d4..d4+3]
// over every NS-th record of the chunk (NS = NT / (32 G) threads per output, their loads
// unrolled so that several records are in flight).  Last, the NS shares of O and the
// shares of L are summed and out = O / L.
ETC_DEV void merge_task(const Args& p, Smem& sm, int b, int g, int rec0, int nb) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = p.G, HQ = p.HKV * G;
  const float* base = p.part + (size_t)rec0 * G * REC;
  float mloc[MAXG], lloc[MAXG];
#pragma unroll
  for (int h = 0; h < MAXG; ++h) { mloc[h] = -INFINITY; lloc[h] = 0.f; }
  for (int c = tid; c < nb; c += NT) {
#pragma unroll
    for (int h = 0; h < MAXG; ++h)
      if (h < G) mloc[h] = fmaxf(mloc[h], gp(base)[((size_t)c * G + h) * REC + HD]);
  }
  // workgroup max per head: the wave's lanes, then the four waves through LDS
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
    if (h < G) {
      float m = mloc[h];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, WAVE));
      if (lane == 0) sm.o[w][h][0] = m;
    }
  }
  __syncthreads();
  if (tid < G) sm.ml[tid][0] = fmaxf(fmaxf(sm.o[0][tid][0], sm.o[1][tid][0]), fmaxf(sm.o[2][tid][0], sm.o[3][tid][0]));
  __syncthreads();
  const int NS = NT / (32 * G);  // threads per output chunk of 4 dims (1, 2 or 8)
  const int item = tid % (32 * G), sidx = tid / (32 * G);
  const int oh = item / 32, d4 = (item % 32) * 4;
  const bool active = sidx < NS;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nb; c0 += CH) {
    const int c = c0 + tid;
#pragma unroll
    for (int h = 0; h < MAXG; ++h) {
      if (h < G) {
        float f = 0.f;
        if (c < nb) {
          const float* r = base + ((size_t)c * G + h) * REC;
          f = __expf(gp(r)[HD] - sm.ml[h][0]);
          lloc[h] = fmaf(gp(r)[HD + 1], f, lloc[h]);
        }
        sm.s[h][tid] = f;
      }
    }
    __syncthreads();
    const int n = min(CH, nb - c0);
    if (active) {
      const float* r0 = base + ((size_t)c0 * G + oh) * REC + d4;
#pragma unroll 8
      for (int k = sidx; k < n; k += NS) {
        const f32x4 ov = gld<f32x4>(r0 + (size_t)k * G * REC);
        const float f = sm.s[oh][k];
        acc.x = fmaf(ov.x, f, acc.x);
        acc.y = fmaf(ov.y, f, acc.y);
        acc.z = fmaf(ov.z, f, acc.z);
        acc.w = fmaf(ov.w, f, acc.w);
      }
    }
    __syncthreads();  // the weights of the chunk are read before the next chunk's
  }
  // L per head: the wave's lanes, then the waves
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
    if (h < G) {
      float l = lloc[h];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off, WAVE);
      if (lane == 0) sm.o[w][h][1] = l;
    }
  }
  __syncthreads();
  if (tid < G) sm.ml[tid][1] = (sm.o[0][tid][1] + sm.o[1][tid][1]) + (sm.o[2][tid][1] + sm.o[3][tid][1]);
  __syncthreads();
  // the NS shares of each output chunk (staged in the weight area: NS * 32 G * 4 floats
  // = 4 NT floats)
  float* stage = &sm.s[0][0];
  if (active && NS > 1) *reinterpret_cast<f32x4*>(stage + 4 * tid) = acc;
  __syncthreads();
  if (sidx == 0) {
    if (NS > 1) {
      for (int s2 = 1; s2 < NS; ++s2) {
        const f32x4 o2 = *reinterpret_cast<const f32x4*>(stage + 4 * (s2 * 32 * G + item));
        acc.x += o2.x; acc.y += o2.y; acc.z += o2.z; acc.w += o2.w;
      }
    }
    const float inv = 1.0f / sm.ml[oh][1];
    *reinterpret_cast<ETC_GLOBAL f32x4*>(gp(p.out + ((size_t)b * HQ + (size_t)g * G + oh) * HD + d4)) =
        f32x4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  }
  __syncthreads();
}

__global__ __launch_bounds__(NT) void attn_kernel(Args p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int np = make_plan(p, sm);
  // np <= cap follows from the token capacity (every request adds less than one chunk
  // per KV head beyond L_b / CH); it is checked anyway, since the records are indexed by it
  const bool valid = np >= 0 && np <= p.cap;
  if (!valid) {
    // a length or a cache row out of range, or more tokens than the workspace holds:
    // nothing runs; workgroup 0 reports it
    if (blockIdx.x == 0 && tid == 0)
      ev_store_relaxed(p.sched + W_STATUS, np == -1 ? 1 /* ETC_ERR_INVALID_ARG */ : 3 /* ETC_ERR_WORKSPACE */);
  }
  const int nmerge = p.B * p.HKV;
  const int total = !valid ? 0 : (p.mode == ETC_SCHED_STATIC ? np + nmerge : np);

  if (tid == 0) sm.next = -1;
  while (true) {
    if (tid == 0) {
      // (no check of the abort flag here: partial tasks never wait, and a merge's wait
      // sees the flag and gives up, so every workgroup still leaves after an abort)
      const int t = sm.next >= 0 ? sm.next : ticket_inc(p.sched + W_TICKET);
      sm.next = -1;
      sm.task = t;
    }
    __syncthreads();
    const int t = sm.task;
    __syncthreads();
    if (t >= total) break;

    if (t < np) {
      const int b = owner(sm, p.B, t);
      const int nb = sm.nsplit[b];
      const int loc = t - sm.pbase[b];
      const int g = loc / nb, c = loc % nb;
      partial_task(p, sm, b, g, c, t);
      publish_shared();
      if (tid == 0) {
        int* ctr = p.ev + EV_STRIDE * (b * p.HKV + g);
        if (p.mode == ETC_SCHED_DYNAMIC) {
          // the last arriver merges, so its signal acquires every other partial
          sm.flag = ev_add_acquire(ctr, 1) == nb - 1 ? 1 : 0;
        } else {
          // nothing waits on the result: the atomic goes out without a return
          ev_signal(ctr, 1);
          sm.flag = 0;
        }
      }
      __syncthreads();
      if (sm.flag) merge_task(p, sm, b, g, sm.pbase[b] + g * nb, nb);
      __syncthreads();
    } else {
      const int bg = t - np, b = bg / p.HKV, g = bg % p.HKV;
      const int nb = sm.nsplit[b];
      if (tid == 0) sm.flag = spin_until_geq(p.ev + EV_STRIDE * bg, nb, p.sched, p.timeout_ticks, 30) ? 1 : 0;
      __syncthreads();
      if (sm.flag) merge_task(p, sm, b, g, sm.pbase[b] + g * nb, nb);
      __syncthreads();
    }
  }

  // the last workgroup out clears the counters for the next call
  wg_publish();
  if (tid == 0) sm.flag = (atomicAdd(p.sched + W_EXIT, 1) == (int)gridDim.x - 1) ? 1 : 0;
  __syncthreads();
  if (sm.flag && !(p.flags & ETC_FLAG_KEEP_COUNTERS)) {
    for (int i = tid; i < p.B * p.HKV; i += NT) ev_store_relaxed(p.ev + EV_STRIDE * i, 0);
    for (int i = tid; i < W_NWORDS; i += NT)
      if (i != W_STATUS && i != W_AUX) ev_store_relaxed(p.sched + i, 0);
  }
}

struct Layout {
  size_t sched, ev, part, total;
  int cap;
};

// Partial records for up to B requests whose contexts sum to at most max_total_tokens:
// every request contributes ceil(L_b / CH) <= L_b / CH + 1 chunks per KV head.  The
// layout depends only on the workspace's capacity, so calls with fewer requests share it.
inline Layout layout(int B, int HKV, int G, long max_total_tokens) {
  Layout Y;
  Y.cap = (int)((max_total_tokens / CH + B) * HKV);
  host::Carve c;
  Y.sched = c.take(W_NWORDS * sizeof(int));
  Y.ev = c.take((size_t)B * HKV * EV_STRIDE * sizeof(int));
  Y.part = c.take((size_t)Y.cap * G * REC * sizeof(float));
  Y.total = c.off;
  return Y;
}

}  // namespace attn
}  // namespace etc

using namespace etc;

static int attn_occupancy(int dev) {
  static int occ[host::MAX_DEVICES] = {0};
  if (occ[dev] == 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, attn::attn_kernel, NT, 0) != hipSuccess || v < 1) v = 1;
    occ[dev] = v;
  }
  return occ[dev];
}

static etc_status attn_shape_check(int32_t B, int32_t HKV, int32_t G, int32_t D, int64_t max_total) {
  if (B < 1 || HKV < 1 || G < 1 || D < 1 || max_total < 1) return ETC_ERR_INVALID_ARG;
  if (D != attn::HD || G > attn::MAXG || B > attn::MAXB) return ETC_ERR_UNSUPPORTED;
  if ((max_total / attn::CH + B) * (int64_t)HKV > (int64_t)1 << 30) return ETC_ERR_UNSUPPORTED;
  return ETC_OK;
}

ETC_API size_t etc_decode_attention_workspace_size(int32_t max_batch, int32_t kv_heads, int32_t group,
                                                   int32_t head_dim, int64_t max_total_tokens) {
  if (attn_shape_check(max_batch, kv_heads, group, head_dim, max_total_tokens) != ETC_OK) return 0;
  return attn::layout(max_batch, kv_heads, group, max_total_tokens).total;
}

ETC_API etc_status etc_decode_attention(int32_t batch, int32_t kv_heads, int32_t group, int32_t head_dim,
                                        const int32_t* context_lens, const int32_t* kv_start,
                                        int32_t kv_rows, float scale,
                                        const void* q, const void* k_cache, const void* v_cache, float* out,
                                        void* workspace, size_t workspace_bytes, int32_t max_batch,
                                        int64_t max_total_tokens, etc_sched_mode mode, uint32_t flags,
                                        int32_t workers, void* stream) {
  etc_status st = attn_shape_check(max_batch, kv_heads, group, head_dim, max_total_tokens);
  if (st != ETC_OK) return st;
  if (batch < 1 || batch > max_batch || kv_rows < 1 || !(scale == scale)) return ETC_ERR_INVALID_ARG;
  if (!context_lens || !kv_start || !q || !k_cache || !v_cache || !out) return ETC_ERR_INVALID_ARG;
  if (mode != ETC_SCHED_STATIC && mode != ETC_SCHED_DYNAMIC) return ETC_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(context_lens) & 3u) || (reinterpret_cast<uintptr_t>(kv_start) & 3u) ||
      !host::aligned16(q) || !host::aligned16(k_cache) || !host::aligned16(v_cache) || !host::aligned16(out))
    return ETC_ERR_INVALID_ARG;
  const attn::Layout Y = attn::layout(max_batch, kv_heads, group, max_total_tokens);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < Y.total)
    return ETC_ERR_WORKSPACE;
  const int dev = host::current_gfx950_device();
  if (dev < 0) return ETC_ERR_NO_DEVICE;

  attn::Args p;
  p.B = batch;
  p.HKV = kv_heads;
  p.G = group;
  p.mode = mode;
  p.flags = flags;
  p.scale = scale;
  p.lens = context_lens;
  p.kv_start = kv_start;
  p.kv_rows = kv_rows;
  p.q = static_cast<const bf16*>(q);
  p.k = static_cast<const bf16*>(k_cache);
  p.v = static_cast<const bf16*>(v_cache);
  p.out = out;
  char* ws = static_cast<char*>(workspace);
  p.sched = reinterpret_cast<int*>(ws + Y.sched);
  p.ev = reinterpret_cast<int*>(ws + Y.ev);
  p.part = reinterpret_cast<float*>(ws + Y.part);
  p.cap = Y.cap;
  p.max_total = max_total_tokens;
  p.timeout_ticks = 500000000ull;  // 5 s without progress, on the 100 MHz real-time clock
  const int grid = host::grid_size(workers, host::device_cus(dev), attn_occupancy(dev));
  hipLaunchKernelGGL(attn::attn_kernel, dim3(grid), dim3(NT), 0, static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? ETC_OK : ETC_ERR_HIP;
}
