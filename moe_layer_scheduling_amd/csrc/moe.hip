// The event-tensor MoE layer: one persistent kernel per call.
//
// What the pages fix.  The podcast episode page "Prompt Boundary-Aware Scheduling with
// Event Tensors for Dynamic Kernels" (summary) describes MoE routing handled through
// event counters whose values and task triggers are computed from the router's output,
// a symbolic batch size that avoids recompiling, and static versus dynamic scheduling.
// The OpenAlex record of "Event Tensor: A Unified Abstraction for Compiling Dynamic
// Megakernel" (abstract) has the event tensor encode dependencies between tiled tasks of
// one persistent kernel.  The chapter "5 · Event Tensor et le dynamisme" adds that the
// counter targets depend on how many producer tasks the routing creates and are computed
// on the GPU before anyone waits (§5.5 Obstacle 1), and that unpredictable task sizes
// call for online scheduling through atomics (§5.5 Obstacle 3).
//
// Tasks of layer l (BT = 16 tokens per routing tile, BM = 128 rows per expert row tile,
// BN1 = 128 ffn columns per gate/up tile, BN2 = 256 hidden columns per down tile):
//   R(tau)         RMSNorm, router logits, top-k, softmax for 16 tokens; ranks of their
//                  (token, slot) pairs inside the tile and the tile's expert histogram
//                  -> ev_route[l] += 1.  For l > 0 it waits ev_done[l-1][tau] >= 1.
//   S              run by the R task whose signal brings ev_route[l] to n_rt: counts,
//                  exclusive scan, row tiles per expert, first sorted row of every
//                  (routing tile, expert) block; sizes the down split (nS chunks of GPC
//                  gate/up tiles) from the actual number of row tiles; -> ev_scan[l] = 1.
//                  With at most PERM_INLINE_RT routing tiles it also scatters the
//                  permutation (there are no P tasks) -> ev_perm[l] = n_rt.
//   P(tau)         waits ev_scan[l] >= 1: places the (token, slot) pairs of routing
//                  tile tau in the permutation -> ev_perm[l] += 1.
//   GU(e, m, n)    waits ev_perm[l] >= n_rt: gate/up tile of expert e rows m*128.. and
//                  ffn columns n*128..; h = silu(G) * U -> ev_gu[l][rt(e,m)][n / GPC] += 1.
//   D(e, m, n2, s) down tile over ffn chunk s; waits ev_gu[l][rt][s] >= tiles in chunk s;
//                  adds gate * y into the float32 accumulator (or stores y) ->
//                  ev_comb[l][tau] += its rows in tau, per routing tile tau it touches.
//   F(tau)         waits ev_comb[l][tau] >= rows(tau) * k * n2 * nS; writes the layer
//                  output rows -> ev_done[l][tau] = 1.
// Static mode: workgroups draw tickets of the order [R.. P.. GU.. D.. F..] per layer
// and spin on each task's counter.  Dynamic mode: a queue of ready tasks; the R tasks of
// the first layer are implicit in slots 0..n_rt-1, S enqueues the P tasks (or the GU
// tasks when it scattered the permutation itself), the last P enqueues the GU tasks,
// and whichever signal completes a counter enqueues the tasks it releases.
// The token count T is a kernel argument; nothing in the code depends on its value.
#include <float.h>
#include <algorithm>
#include <string.h>

#include "common.hpp"
#include "host.hpp"
#include "ktile.hpp"

namespace etc {
namespace moe {

constexpr int MAXL = 4, MAXE = 256, MAXK = 16;
constexpr int BT = 16, BM = 128, BN1 = 128, BN2 = 256;
// workgroup of the persistent kernel: 8 waves, two per SIMD, so that one wave's MFMAs
// run while the other waits on LDS
constexpr int MNT = 512, NWAVE = MNT / 64;
// H: whole 16-byte chunks in each of the router's four K slices; F: whole 64-value chunks
// (tiles along F and H are masked at the edge)
constexpr int H_ALIGN = 128, F_ALIGN = 64;
constexpr int MAX_WORKERS = 2048;
constexpr int MAX_TOKENS = 262143;  // task fields are 14 bits
// Up to this many routing tiles (T <= 64) the scan task also scatters the permutation
// (at most 64 * k pairs): separate P tasks would only add a hand-off to a short path.
constexpr int PERM_INLINE_RT = 4;
// Router slices: with few routing tiles for the workers, the router of a tile is split
// along K into Q slice tasks (Q <= RQ_MAX) whose partial logits go through the
// workspace; the slice whose report completes its tile's counter finishes the tile
// (sum, top-k, ranks).  At most NRQ_CAP slice records per call.
constexpr int RQ_MAX = 8, NRQ_CAP = 256;

// Task bodies are separate functions: each gets its own register allocation instead of
// sharing one with the scheduler loop and every other task (inlined together they spill
// inside the GEMM loop).  A call per task costs nothing next to the task itself.
#define ETC_TASK __device__ __attribute__((noinline))
// The short tasks (routing, scan, permutation, finalize) are inlined into the task loop:
// as calls they would save and restore the callee-saved registers they use (about 90 per
// lane) on every call, for a task that runs only once or twice per workgroup.
#define ETC_SMALL_TASK __device__ __attribute__((always_inline))

enum Kind { K_NONE = 0, K_R = 1, K_S = 2, K_GU = 3, K_D = 4, K_F = 5, K_P = 6 };
enum PlanWord { PL_RT = 0, PL_NGU, PL_ND, PL_NF, PL_NS, PL_GPC, PL_NEXTBASE, PL_Q, PL_WORDS = 8 };

struct Task {
  int kind, layer, a, b, c, d;
};

ETC_DEV long long enc(const Task& t) {
  unsigned long long v = (unsigned long long)t.kind | ((unsigned long long)t.layer << 4) |
                         ((unsigned long long)t.a << 8) | ((unsigned long long)t.b << 22) |
                         ((unsigned long long)t.c << 36) | ((unsigned long long)t.d << 50);
  return (long long)v;
}
ETC_DEV Task dec(long long sv) {
  unsigned long long v = (unsigned long long)sv;
  Task t;
  t.kind = v & 15;
  t.layer = (v >> 4) & 15;
  t.a = (v >> 8) & 0x3fff;
  t.b = (v >> 22) & 0x3fff;
  t.c = (v >> 36) & 0x3fff;
  t.d = (v >> 50) & 0x3fff;
  return t;
}

struct LayerArgs {
  const float* gamma;
  const void* w_router;
  const float* bias;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* in;
  void* out;
  int* topk_idx;       // [T][k]
  float* topk_w;       // [T][k]
  int* lrank;          // [T][k] rank of the pair among its tile's pairs for the same expert
  int* hist;           // [n_rt][E]
  int* tile_off;       // [n_rt][E] first sorted row of tile tau's pairs for expert e
  int* counts;         // [E]
  int* offsets;        // [E+1]
  int* rt_base;        // [E+1] first row tile of each expert
  int* sorted_assign;  // [T*k]
  int* pos;            // [T][k]
  int* plan;           // [PL_WORDS]
  int* ev_route;       // 1
  int* ev_rq;          // [n_rt] router slices of each tile that have reported
  int* ev_scan;        // 1
  int* ev_perm;        // 1
  int* ev_gu;          // [max_rt][n1]
  int* ev_comb;        // [n_rt]
  int* ev_done;        // [n_rt]
};

struct Args {
  int T, H, E, K, F, L;
  float eps;
  int mode, combine;
  unsigned flags;
  int n_rt, n1, n2, workers, max_rt, n_rt_cap, queue_len;
  int n_perm;  // P tasks per layer: n_rt, or 0 when S scatters the permutation itself
  int Q, n_rq; // router slices per routing tile, R tasks per layer (n_rt * Q)
  uint64_t timeout_ticks;  // watchdog: a wait without progress for this long gives up
  void* xq;        // [T][H] normalised input in storage precision
  void* hbuf;      // [T*k][F] SwiGLU output, rows in sorted order
  float* out_acc;  // [T][H] atomic-combine accumulator
  float* ybuf;     // [T*k][H] ordered-combine rows
  float* rpart;    // [NRQ_CAP][BT][E] partial logits of router slices
  long long* queue;
  int* sched;
  unsigned long long* trace;  // ETC_FLAG_TRACE records, 4 words each
  int trace_cap;
  LayerArgs layer[MAXL];
};

// The workgroup's LDS copy of the kernel arguments, seen as LDS by the task bodies (a
// generic reference would make every field read a FLAT load).
typedef const ETC_LDS Args KArgs;
typedef const ETC_LDS LayerArgs KLayer;

struct RouteSmem {
  static constexpr int GCHUNK = 16384;  // gamma values staged at a time
  float part[BT * 512];  // [KS][BT][E] partial logits, KS * E <= 512
  float lg[BT][MAXE];
  alignas(16) float gam[GCHUNK];
  float rs[BT];
  unsigned emask[MAXE];  // tokens of the tile that selected each expert
  float bias[MAXE];
  int soff[MAXE + 1];    // single-tile scan: first sorted row of each expert
  int stmp[2 * NWAVE];
  int sel[BT][MAXK];
};
struct ScanSmem {
  static constexpr int HIST_LDS = 16384;  // histogram entries staged in LDS
  alignas(16) int hs[HIST_LDS];            // hist, then tile_off in place
  int off[MAXE + 1];
  int tmp[2 * NWAVE];
  int part[MNT];  // per-thread partial counts over a chunk of routing tiles
};
struct TileSmem {
  alignas(16) char gemm[KTile<float, MNT>::LDS_BYTES];  // 16-byte LDS reads and copies
  int row_tok[BM];
  float row_gate[BM];
};
static_assert(PERM_INLINE_RT * MAXE <= ScanSmem::HIST_LDS, "the inline scatter reads staged offsets");
union SmemU {
  RouteSmem r;
  ScanSmem s;
  TileSmem t;
};
// The plan, row-tile bases, counts and offsets of one layer, copied into LDS by the
// whole workgroup before its first gate/up, down or finalize task of that layer: ticket
// decoding (a binary search over the row-tile bases), dependency targets and the tiles'
// row ranges then read LDS instead of making dependent global round trips per task.
struct LayerCache {
  int layer;  // -1: nothing cached
  int plan[PL_WORDS];
  int rtb[MAXE + 1];
  int off[MAXE + 1];
  int cnt[MAXE];
};

struct Smem {
  SmemU u;
  Task task;
  int flag;
  int need_cache;
  // layers whose ev_scan / ev_perm this workgroup has already acquired at their targets
  // (bit l): later waits on them return at once (static mode, thread 0)
  unsigned scan_seen, perm_seen;
  // static mode: the ticket a gate/up or down task drew for the workgroup's next claim
  // while its epilogue ran (-1: none), so the claim's atomic round trip overlaps the
  // task instead of sitting between tasks (thread 0)
  int next_ticket;
  // static mode: first ticket of layer l's successor once known (-1: not yet), so the
  // claims of later layers skip earlier layers without reading their plans (thread 0)
  int lbase[MAXL + 1];
  int ibuf[4];
  LayerCache lc;
};

template <typename TE>
ETC_DEV u32x4 pack16(const float* v);
template <>
ETC_DEV u32x4 pack16<bf16>(const float* v) {
  return u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
               pack_bf16x2(v[6], v[7])};
}
template <>
ETC_DEV u32x4 pack16<float>(const float* v) {
  return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
}

ETC_DEV int tile_rows(KArgs& p, int tau) { return min(BT, p.T - tau * BT); }

// Largest e in [0, E) with rt_base[e] * mult <= idx: the expert owning task idx.
template <typename RtBase>
ETC_DEV int owner_expert_by(RtBase rt_base, int E, int idx, int mult) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (rt_base(mid) * mult <= idx) lo = mid; else hi = mid;
  }
  return lo;
}
ETC_DEV int owner_expert(const int* rt_base, int E, int idx, int mult) {
  return owner_expert_by([&](int i) ETC_INLINE { return gp(rt_base)[i]; }, E, idx, mult);
}

// ------------------------------------------------------------------ R: routing tile
//
// One task routes a tile of BT tokens: RMSNorm, router logits, top-k with softmax, the
// tile's per-expert ranks and histogram (the counts that set the event targets come from
// here: tutorial chapter "5 · Event Tensor et le dynamisme", §5.5 Obstacle 1).
//
// Router precision.  logits[t][e] = rs_t * sum_h v[t][h] * W_r[e][h] (+ b[e]) with
// v = x * gamma in float32 and rs_t = 1/sqrt(mean_h x[t][h]^2 + eps), which is
// sum_h xn[t][h] W_r[e][h] for xn = x * rs * gamma up to float32 rounding.  On the matrix
// cores v is split into three bfloat16 parts (hi = bf16(v), mid = bf16(v - hi),
// lo = bf16(v - hi - mid)); the product of each part with a bfloat16 weight is exact in
// float32 and the parts accumulate separately, so the dot product keeps float32 accuracy.
// Float32 layers use the float32 MFMA on v directly.
//
// Work split.  NB = ceil(E/16) blocks of 16 experts; a wave owns NBW of them (the next
// power of two >= NB, at most 4) over one of KS = 8 / ceil(NB/NBW) K slices, so every
// wave has exactly one item.  A wave loads its x rows once per K step for all its expert
// blocks; the waves of the first expert group also store xn in storage precision (xq,
// the experts' input).

template <int NSPLIT>
struct RouterSplit;
template <>
struct RouterSplit<3> {  // bfloat16 layers: three parts per value
  ETC_DEV static void run(const float* v, u32x4 (&a)[3]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = v[2 * i], x1 = v[2 * i + 1];
      const uint32_t h = pack_bf16x2(x0, x1);
      const float r0 = x0 - __uint_as_float(h << 16), r1 = x1 - __uint_as_float(h & 0xffff0000u);
      const uint32_t m = pack_bf16x2(r0, r1);
      const float q0 = r0 - __uint_as_float(m << 16), q1 = r1 - __uint_as_float(m & 0xffff0000u);
      a[0][i] = h;
      a[1][i] = m;
      a[2][i] = pack_bf16x2(q0, q1);
    }
  }
};
template <>
struct RouterSplit<1> {  // float32 layers: the values themselves
  ETC_DEV static void run(const float* v, u32x4 (&a)[1]) {
    a[0] = u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                 __float_as_uint(v[3])};
  }
};

// Wave item: expert blocks g*NBW .. g*NBW+NBW-1 over the wave's share of every K chunk,
// on v = x * gamma (the 1/rms factor of each token is applied to its logits).
// gamma is staged in LDS one chunk of GCHUNK values at a time (every wave calls this with
// the same NBW, so the barriers around the staging are reached by the whole workgroup).
// Writes the partial logits of its K slice to R.part[ks][t][e].
template <typename TE, int NBW>
ETC_DEV void router_item(KArgs& p, KLayer& L, RouteSmem& R, int t0, int nt, int g, int ks,
                         int KS, int k_lo, int k_hi) {
  constexpr int EPC = 16 / (int)sizeof(TE);  // values per 16-byte chunk
  constexpr int KSTEP = 4 * EPC;              // K per MFMA step (four lane groups)
  constexpr int NSPLIT = sizeof(TE) == 2 ? 3 : 1;
  constexpr int U = NBW <= 2 ? 8 : 4;         // K steps whose loads are in flight together
  const int tid = threadIdx.x, lane = tid & 63, row = lane & 15, grp = lane >> 4;
  const int H = p.H, E = p.E;
  // rows past the tile's tokens repeat its last token and experts past E repeat the last
  // expert, so every load is unconditional; those results are never used
  const int tr = row < nt ? row : nt - 1;
  const TE* xrow = static_cast<const TE*>(L.in) + (size_t)(t0 + tr) * H + grp * EPC;
  const TE* wbase = static_cast<const TE*>(L.w_router) + grp * EPC;
  // the first expert group also writes xn = v * rs in storage precision (xq); rows past
  // the tile's tokens write their copy of the last token's values to its row
  TE* xqtile = static_cast<TE*>(p.xq) + (size_t)t0 * H;
  const uint32_t xqoff = (uint32_t)((tr * H + grp * EPC) * (int)sizeof(TE));
  const bool put = g == 0;
  const float rs = R.rs[tr];
  int woff[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b) woff[b] = min((g * NBW + b) * 16 + row, E - 1) * H;
  f32x4 acc[NBW][NSPLIT];
#pragma unroll
  for (int b = 0; b < NBW; ++b)
#pragma unroll
    for (int q = 0; q < NSPLIT; ++q) acc[b][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kc = k_lo; kc < k_hi; kc += RouteSmem::GCHUNK) {
    const int len = min(RouteSmem::GCHUNK, k_hi - kc);
    __syncthreads();  // every wave is done with the previous chunk
    for (int i = tid * 4; i < len; i += MNT * 4)
      *reinterpret_cast<f32x4*>(&R.gam[i]) = gld<f32x4>(L.gamma + kc + i);
    __syncthreads();
    const int nsteps = len / KSTEP;
    const int s0 = ks * nsteps / KS, s1 = (ks + 1) * nsteps / KS;
    auto steps = [&](int s, auto nst) ETC_INLINE {
      constexpr int N = decltype(nst)::value;
      u32x4 xv[N], wv[N][NBW];
      static_for<N>([&](auto u) ETC_INLINE {
        const int k = kc + (s + u) * KSTEP;
        xv[u] = gld<u32x4>(xrow + k);
        static_for<NBW>([&](auto b) ETC_INLINE { wv[u][b] = gld<u32x4>(wbase + woff[b] + k); });
      });
      static_for<N>([&](auto u) ETC_INLINE {
        const int kl = (s + u) * KSTEP + grp * EPC;  // within the chunk
        float v[EPC];
        expand16(xv[u], v, (const TE*)nullptr);
        static_for<EPC / 4>([&](auto q) ETC_INLINE {
          const f32x4 gq = *reinterpret_cast<const f32x4*>(&R.gam[kl + 4 * q]);
          v[4 * q] *= gq.x;
          v[4 * q + 1] *= gq.y;
          v[4 * q + 2] *= gq.z;
          v[4 * q + 3] *= gq.w;
        });
        if (put) {
          float xn[EPC];
#pragma unroll
          for (int i = 0; i < EPC; ++i) xn[i] = v[i] * rs;
          st_shared16(xqtile, xqoff + (uint32_t)((kc + (s + u) * KSTEP) * (int)sizeof(TE)), pack16<TE>(xn));
        }
        u32x4 a[NSPLIT];
        RouterSplit<NSPLIT>::run(v, a);
        static_for<NBW>([&](auto b) ETC_INLINE {
          static_for<NSPLIT>([&](auto q) ETC_INLINE { mma16(acc[b][q], a[q], wv[u][b], (const TE*)nullptr); });
        });
      });
    };
    int s = s0;
    for (; s + U <= s1; s += U) steps(s, std::integral_constant<int, U>{});
    for (; s < s1; ++s) steps(s, std::integral_constant<int, 1>{});
  }

  // result element (token grp*4+i, expert block column row) of each block
#pragma unroll
  for (int b = 0; b < NBW; ++b) {
    const int e = (g * NBW + b) * 16 + row;
    f32x4 sum = acc[b][0];
    if constexpr (NSPLIT == 3) sum = (acc[b][2] + acc[b][1]) + acc[b][0];
    if (e < E) {
#pragma unroll
      for (int i = 0; i < 4; ++i) R.part[(ks * BT + grp * 4 + i) * E + e] = sum[i];
    }
  }
}

// Router on the vector ALUs for a tile of at most NTOK (1 or 2) tokens and at most 16
// experts (decode-sized batches), where the 16-row MFMA path would split 16 rows for one
// or two real tokens.  Thread tid takes chunks tid, tid + MNT, ... of the rows; for every token
// and expert it accumulates v . W_r[e] over its chunks in float32 (fused multiply-add),
// then every wave sums its lanes and writes R.part[w][t][e] (KS = NWAVE slices).  It also
// writes xq = dtype(v * rs) for the tile's tokens (16 bytes per lane, rows contiguous).
template <typename TE, int NTOK>
ETC_DEV void router_valu(KArgs& p, KLayer& L, RouteSmem& R, int t0, int nt, int k_lo, int k_hi) {
  constexpr int EPC = 16 / (int)sizeof(TE);
  constexpr int EMAX = 16;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int H = p.H, E = p.E;
  const TE* x = static_cast<const TE*>(L.in) + (size_t)t0 * H;
  const TE* wr = static_cast<const TE*>(L.w_router);
  TE* xq = static_cast<TE*>(p.xq) + (size_t)t0 * H;
  float acc[NTOK][EMAX];
#pragma unroll
  for (int t = 0; t < NTOK; ++t)
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[t][e] = 0.f;
  float rs[NTOK];
#pragma unroll
  for (int t = 0; t < NTOK; ++t) rs[t] = R.rs[min(t, nt - 1)];
  for (int c = k_lo / EPC + tid; c < k_hi / EPC; c += MNT) {
    // rows past the tile's tokens repeat its last token, experts past E the last expert
    u32x4 xv[NTOK], wv[EMAX];
    f32x4 gv[EPC / 4];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) xv[t] = gld<u32x4>(x + (size_t)min(t, nt - 1) * H + c * EPC);
#pragma unroll
    for (int q = 0; q < EPC / 4; ++q) gv[q] = gld<f32x4>(L.gamma + c * EPC + 4 * q);
#pragma unroll
    for (int e = 0; e < EMAX; ++e) wv[e] = gld<u32x4>(wr + (size_t)min(e, E - 1) * H + c * EPC);
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
      float v[EPC];
      expand16(xv[t], v, (const TE*)nullptr);
#pragma unroll
      for (int q = 0; q < EPC / 4; ++q) {
        v[4 * q] *= gv[q].x;
        v[4 * q + 1] *= gv[q].y;
        v[4 * q + 2] *= gv[q].z;
        v[4 * q + 3] *= gv[q].w;
      }
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        float wf[EPC];
        expand16(wv[e], wf, (const TE*)nullptr);
#pragma unroll
        for (int i = 0; i < EPC; ++i) acc[t][e] = fmaf(v[i], wf[i], acc[t][e]);
      }
      if (t < nt) {
        float xn[EPC];
#pragma unroll
        for (int i = 0; i < EPC; ++i) xn[i] = v[i] * rs[t];
        st_shared16(xq, (uint32_t)(((size_t)t * H + c * EPC) * sizeof(TE)), pack16<TE>(xn));
      }
    }
  }
  // every wave's sum of its lanes, per (token, expert)
#pragma unroll
  for (int t = 0; t < NTOK; ++t)
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      float v = row16_sum(acc[t][e]);
      v += __shfl_xor(v, 16, WAVE);
      v += __shfl_xor(v, 32, WAVE);
      if (lane == 0 && t < nt && e < E) R.part[(w * BT + t) * E + e] = v;
    }
}

// Top-k of one token per row of 16 lanes: lane j holds experts j, j+16, ...  k rounds of
// an argmax by (logit desc, expert asc) across the row; lane j keeps the j-th winner.
// Softmax over the k selected logits.  Rows past the tile's tokens compute on unused
// LDS values and store nothing.
template <int VPL>
ETC_DEV void topk_row(KArgs& p, KLayer& L, RouteSmem& R, int t0, int nt) {
  const int tid = threadIdx.x, j = tid & 15, tt = tid >> 4;
  const int E = p.E, K = p.K;
  float v[VPL];
  int id[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = j + 16 * i;
    v[i] = e < E ? R.lg[tt][e] : -FLT_MAX;
    id[i] = e < E ? e : 0x7fffffff;
  }
  float mine = 0.f, top = 0.f;
  int mine_e = 0;
  for (int r = 0; r < K; ++r) {
    float bv = v[0];
    int be = id[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i)
      if (v[i] > bv) { bv = v[i]; be = id[i]; }  // experts ascend with i: ties keep the first
    auto merge = [&](float ov, int oe) ETC_INLINE {
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    };
    merge(dpp_f<DPP_XOR1>(bv), dpp_i<DPP_XOR1>(be));
    merge(dpp_f<DPP_XOR2>(bv), dpp_i<DPP_XOR2>(be));
    merge(dpp_f<DPP_HALF_MIRROR>(bv), dpp_i<DPP_HALF_MIRROR>(be));
    merge(dpp_f<DPP_MIRROR>(bv), dpp_i<DPP_MIRROR>(be));
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (id[i] == be) { v[i] = -FLT_MAX; id[i] = 0x7fffffff; }
    if (r == 0) top = bv;
    if (j == r) { mine = bv; mine_e = be; }
  }
  const float z = j < K ? expf(mine - top) : 0.f;
  const float zsum = row16_sum(z);
  if (tt < nt && j < K) {
    const int t = t0 + tt;
    st_shared(L.topk_idx + t * K + j, mine_e);
    st_shared(L.topk_w + t * K + j, z / zsum);
    R.sel[tt][j] = mine_e;
    atomicOr(&R.emask[mine_e], 1u << tt);
  }
}

// R(a): slice q = a mod Q of routing tile tau = a / Q.  Returns true when the tile's
// routing is complete in this workgroup: always with one slice (Q = 1), else only in the
// slice whose report completed the tile's slice counter.  Every thread calls this and
// gets the same answer.
template <typename TE>
ETC_SMALL_TASK bool route_task(KArgs& p, KLayer& L, int a, Smem& sm) {
  constexpr int EPC = 16 / (int)sizeof(TE);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.H, E = p.E, K = p.K, Q = p.Q;
  const int tau = a / Q, q = a - tau * Q;
  const int t0 = tau * BT, nt = tile_rows(p, tau);
  RouteSmem& R = sm.u.r;

  for (int e = tid; e < E; e += MNT) {
    R.emask[e] = 0u;
    R.bias[e] = L.bias ? gp(L.bias)[e] : 0.f;
  }

  // 1. inverse RMS of each token: 32 lanes per token, each summing the squares of every
  //    32nd chunk of the row (eight chunks in flight), then a butterfly over the 32 lanes
  {
    const int tt = tid >> 5, j = tid & 31;
    float ss = 0.f;
    if (tt < nt) {
      const TE* xr = static_cast<const TE*>(L.in) + (size_t)(t0 + tt) * H;
      const int cpr = H / EPC;
      int c = j;
      for (; c + 7 * 32 < cpr; c += 8 * 32) {
        u32x4 xv[8];
        static_for<8>([&](auto u) ETC_INLINE { xv[u] = gld<u32x4>(xr + (c + 32 * u) * EPC); });
        static_for<8>([&](auto u) ETC_INLINE {
          float f[EPC];
          expand16(xv[u], f, (const TE*)nullptr);
#pragma unroll
          for (int i = 0; i < EPC; ++i) ss += f[i] * f[i];
        });
      }
      for (; c < cpr; c += 32) {
        float f[EPC];
        expand16(gld<u32x4>(xr + c * EPC), f, (const TE*)nullptr);
#pragma unroll
        for (int i = 0; i < EPC; ++i) ss += f[i] * f[i];
      }
    }
    ss = row16_sum(ss);
    ss += __shfl_xor(ss, 16, WAVE);
    if (j == 0) R.rs[tt] = tt < nt ? 1.0f / sqrtf(ss / (float)H + p.eps) : 0.f;
  }
  __syncthreads();

  // 2. partial logits over this slice's K range (whole steps of the MFMA or VALU path):
  //    on the vector ALUs for a few tokens and experts, else per (expert group, K
  //    slice) on the matrix cores, one item per wave
  const int kstep = 4 * EPC, nst = H / kstep;
  const int k_lo = (q * nst / Q) * kstep, k_hi = ((q + 1) * nst / Q) * kstep;
  const int NB = cdiv(E, 16);
  const int NBW = NB <= 1 ? 1 : (NB <= 2 ? 2 : 4);
  int KS = NWAVE / cdiv(NB, NBW);
  if (E <= 16 && nt <= 2) {
    KS = NWAVE;
    if (nt == 1) router_valu<TE, 1>(p, L, R, t0, nt, k_lo, k_hi);
    else router_valu<TE, 2>(p, L, R, t0, nt, k_lo, k_hi);
  } else {
    const int g = w / KS, ks = w % KS;
    if (NBW == 1) router_item<TE, 1>(p, L, R, t0, nt, g, ks, KS, k_lo, k_hi);
    else if (NBW == 2) router_item<TE, 2>(p, L, R, t0, nt, g, ks, KS, k_lo, k_hi);
    else router_item<TE, 4>(p, L, R, t0, nt, g, ks, KS, k_lo, k_hi);
  }
  // clear this slice's share of the tile's accumulator rows for the atomic combine (the
  // 16-byte chunks c_lo .. c_hi-1 of every row): the last global loads of the task are
  // done, so these stores drain while the rest of the task runs
  if (p.combine == ETC_COMBINE_ATOMIC) {
    float* acc = p.out_acc + (size_t)t0 * H;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int cpr = H / 4, c_lo = q * cpr / Q, ncs = (q + 1) * cpr / Q - c_lo;
    for (int i = tid; i < nt * ncs; i += MNT) {
      const int row = i / ncs, c = c_lo + (i - row * ncs);
      st_shared16(acc, (uint32_t)((row * cpr + c) * 16), z);
    }
  }
  __syncthreads();
  if (Q == 1) {
    for (int o = tid; o < nt * E; o += MNT) {
      const int tt = o / E, e = o - tt * E;
      float v = 0.f;
      for (int k = 0; k < KS; ++k) v += R.part[(k * BT + tt) * E + e];
      R.lg[tt][e] = R.rs[tt] * v + R.bias[e];
    }
  } else {
    // the slice's partial logits (before the 1/rms factor and the bias) go out; the
    // slice whose report completes the tile's counter sums them in slice order
    float* mine = p.rpart + (size_t)a * BT * E;
    for (int o = tid; o < nt * E; o += MNT) {
      const int tt = o / E, e = o - tt * E;
      float v = 0.f;
      for (int k = 0; k < KS; ++k) v += R.part[(k * BT + tt) * E + e];
      st_shared(mine + o, v);
    }
    publish_shared();
    if (tid == 0) sm.flag = (ev_add_acquire(L.ev_rq + tau, 1) == Q - 1) ? 1 : 0;  // acquire: the others' slices
    __syncthreads();
    const bool last = sm.flag != 0;
    __syncthreads();
    if (!last) return false;
    // every slice's value of an output is loaded before any is added (one round trip),
    // then they are summed in slice order
    const float* all = p.rpart + (size_t)tau * Q * BT * E;
    for (int o = tid; o < nt * E; o += MNT) {
      const int tt = o / E, e = o - tt * E;
      float part[RQ_MAX];
#pragma unroll
      for (int s2 = 0; s2 < RQ_MAX; ++s2) part[s2] = s2 < Q ? gp(all)[(size_t)s2 * BT * E + o] : 0.f;
      float v = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < RQ_MAX; ++s2) v += part[s2];
      R.lg[tt][e] = R.rs[tt] * v + R.bias[e];
    }
  }
  __syncthreads();

  // 3. top-k and gates: one row of 16 lanes per token (waves 0..3)
  if (tid < BT * 16) {
    const int vpl = cdiv(E, 16);
    if (vpl == 1) topk_row<1>(p, L, R, t0, nt);
    else if (vpl == 2) topk_row<2>(p, L, R, t0, nt);
    else if (vpl <= 4) topk_row<4>(p, L, R, t0, nt);
    else if (vpl <= 8) topk_row<8>(p, L, R, t0, nt);
    else topk_row<16>(p, L, R, t0, nt);
  }
  __syncthreads();

  // 4. rank of each pair among the tile's pairs of its expert (tokens ascending; a token
  //    never holds one expert twice) and the tile's histogram, from the per-expert masks
  //    of the tile's tokens that selected it
  for (int a = tid; a < nt * K; a += MNT) {
    const int tt = a / K, j = a - tt * K;
    st_shared(L.lrank + t0 * K + a, __popc(R.emask[R.sel[tt][j]] & ((1u << tt) - 1u)));
  }
  for (int e = tid; e < E; e += MNT) st_shared(L.hist + tau * E + e, __popc(R.emask[e]));
  return true;
}

// ------------------------------------------------------------------ S: scan and permutation

// Exclusive scans of two values at once over the workgroup (thread order): returns the
// prefixes of a and b and their totals.  One exchange through LDS (tmp: 2 * NWAVE ints).
ETC_DEV void block_exclusive_scan2(int a, int b, int* tmp, int& pa, int& pb, int& ta, int& tb) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int x = a, y = b;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int xs = __shfl_up(x, off, WAVE), ys = __shfl_up(y, off, WAVE);
    if (lane >= off) { x += xs; y += ys; }
  }
  if (lane == 63) { tmp[w] = x; tmp[NWAVE + w] = y; }
  __syncthreads();
  int bx = 0, by = 0;
  ta = 0;
  tb = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) {
    bx += (i < w) ? tmp[i] : 0;
    by += (i < w) ? tmp[NWAVE + i] : 0;
    ta += tmp[i];
    tb += tmp[NWAVE + i];
  }
  __syncthreads();
  pa = bx + x - a;
  pb = by + y - b;
}

// The layer's plan words (thread 0), from its number of row tiles RT.  The down split:
// enough down tasks to give every worker one, when the combine is atomic (partial sums
// over ffn chunks add into the same accumulator).  One round of longer tasks beat two
// rounds of shorter ones on decode-sized batches (fewer pipeline fills and epilogues
// per byte of weights).
ETC_DEV void write_plan(KArgs& p, KLayer& L, int layer, int RT) {
  const int n_rt = p.n_rt;
  int nS = 1;
  if (p.combine == ETC_COMBINE_ATOMIC && RT > 0) {
    const int want = p.workers;
    nS = (RT * p.n2 >= want) ? 1 : min(p.n1, cdiv(want, RT * p.n2));
  }
  const int gpc = cdiv(p.n1, nS);
  nS = cdiv(p.n1, gpc);
  const int ngu = RT * p.n1, nd = RT * p.n2 * nS, nf = n_rt;
  const int base = (layer == 0) ? 0 : gp(p.layer[layer - 1].plan)[PL_NEXTBASE];
  st_shared(L.plan + PL_RT, RT);
  st_shared(L.plan + PL_NGU, ngu);
  st_shared(L.plan + PL_ND, nd);
  st_shared(L.plan + PL_NF, nf);
  st_shared(L.plan + PL_NS, nS);
  st_shared(L.plan + PL_GPC, gpc);
  st_shared(L.plan + PL_NEXTBASE, base + p.n_rq + p.n_perm + ngu + nd + nf);
  st_shared(L.plan + PL_Q, p.Q);
}

// S for a layer of a single routing tile, run by that tile's R task straight from its
// LDS results (the tokens that selected each expert, the selections): counts, scans,
// the tile's offsets, the plan and the permutation, with no global round trip between
// routing and scan.  Every thread calls this.
ETC_DEV void scan_single_tile(KArgs& p, KLayer& L, int layer, Smem& sm) {
  const int tid = threadIdx.x, E = p.E, K = p.K, nt = p.T;
  RouteSmem& R = sm.u.r;
  const int cnt = tid < E ? __popc(R.emask[tid]) : 0;
  int off = 0, rtb = 0, total_rows = 0, RT = 0;
  block_exclusive_scan2(cnt, cdiv(cnt, BM), R.stmp, off, rtb, total_rows, RT);
  if (tid < E) {
    R.soff[tid] = off;
    st_shared(L.counts + tid, cnt);
    st_shared(L.offsets + tid, off);
    st_shared(L.rt_base + tid, rtb);
    st_shared(L.tile_off + tid, off);
  }
  if (tid == 0) {
    st_shared(L.offsets + E, total_rows);
    st_shared(L.rt_base + E, RT);
    write_plan(p, L, layer, RT);
  }
  __syncthreads();
  for (int a = tid; a < nt * K; a += MNT) {
    const int t = a / K, j = a - t * K, e = R.sel[t][j];
    const int r = R.soff[e] + __popc(R.emask[e] & ((1u << t) - 1u));
    st_shared(L.sorted_assign + r, a);
    st_shared(L.pos + a, r);
  }
}

ETC_SMALL_TASK void scan_task(KArgs& p, KLayer& L, int layer, Smem& sm) {
  const int tid = threadIdx.x;
  const int E = p.E, K = p.K, n_rt = p.n_rt;
  ScanSmem& S = sm.u.s;
  const bool inline_perm = p.n_perm == 0;
  // few routing tiles: the inputs of the pairs this thread places (at most 64 tokens, so
  // at most two pairs per thread), loaded first so that their latency overlaps the scan
  const int npairs = inline_perm ? p.T * K : 0;
  int pe[2] = {0, 0}, pr[2] = {0, 0};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int a = min(tid + q * MNT, max(npairs - 1, 0));
    if (inline_perm) {
      pe[q] = gp(L.topk_idx)[a];
      pr[q] = gp(L.lrank)[a];
    }
  }

  // The histogram [n_rt][E] comes into LDS in 16-byte pieces when it fits (the routing
  // tiles' counts are then read from global memory once); larger ones are read in place.
  const bool staged = n_rt * E <= ScanSmem::HIST_LDS;
  if (staged) {
    const int n = n_rt * E;
    for (int i = tid * 4; i < n; i += MNT * 4) {
      if (i + 4 <= n) {
        *reinterpret_cast<u32x4*>(&S.hs[i]) = gld<u32x4>(L.hist + i);
      } else {
        for (int j = i; j < n; ++j) S.hs[j] = gp(L.hist)[j];
      }
    }
    __syncthreads();
  }
  auto hist = [&](int tau, int e) ETC_INLINE { return staged ? S.hs[tau * E + e] : gp(L.hist)[tau * E + e]; };

  // counts per expert: thread (c, e) = (tid / E, tid % E) sums the histogram of expert e
  // over chunk c of the routing tiles (C = MNT / E chunks per expert)
  const int C = MNT / E, e_t = tid % E, c_t = tid / E;
  const bool owner = c_t < C;
  const int span = cdiv(n_rt, C), tau0 = min(n_rt, c_t * span), tau1 = min(n_rt, tau0 + span);
  int part = 0;
  if (owner)
    for (int tau = tau0; tau < tau1; ++tau) part += hist(tau, e_t);
  S.part[tid] = part;
  __syncthreads();
  int cnt = 0;
  if (tid < E)
    for (int c = 0; c < C; ++c) cnt += S.part[c * E + tid];
  int off = 0, rtb = 0, total_rows = 0, RT = 0;
  block_exclusive_scan2(cnt, cdiv(cnt, BM), S.tmp, off, rtb, total_rows, RT);
  if (tid < E) {
    S.off[tid] = off;
    st_shared(L.counts + tid, cnt);
    st_shared(L.offsets + tid, off);
    st_shared(L.rt_base + tid, rtb);
  }
  if (tid == 0) {
    S.off[E] = total_rows;
    st_shared(L.offsets + E, total_rows);
    st_shared(L.rt_base + E, RT);
  }
  __syncthreads();
  // first sorted row of every (routing tile, expert) block: each thread continues the
  // running offset of its expert through its chunk (in place in LDS when staged)
  if (owner) {
    int run = S.off[e_t];
    for (int c = 0; c < c_t; ++c) run += S.part[c * E + e_t];
    for (int tau = tau0; tau < tau1; ++tau) {
      const int v = hist(tau, e_t);
      if (staged) S.hs[tau * E + e_t] = run;
      else st_shared(L.tile_off + tau * E + e_t, run);
      run += v;
    }
  }
  if (tid == 0) write_plan(p, L, layer, RT);
  if (staged) {
    __syncthreads();
    const int n = n_rt * E;
    for (int i = tid * 4; i < n; i += MNT * 4) {
      if (i + 4 <= n) {
        st_shared16(L.tile_off, (uint32_t)(i * 4), *reinterpret_cast<const u32x4*>(&S.hs[i]));
      } else {
        for (int j = i; j < n; ++j) st_shared(L.tile_off + j, S.hs[j]);
      }
    }
  }
  // few routing tiles: the permutation scatter of every tile here (what P(tau) does),
  // from the offsets in LDS (n_rt * E is small, so they are staged)
  if (inline_perm) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int a = tid + q * MNT;
      if (a < npairs) {
        const int r = S.hs[(a / (BT * K)) * E + pe[q]] + pr[q];
        st_shared(L.sorted_assign + r, a);
        st_shared(L.pos + a, r);
      }
    }
  }
}

// P(tau): the (token, slot) pairs of routing tile tau go to their rows of the
// permutation: pair a = t*k + j of expert e lands at tile_off[tau][e] + its rank among
// the tile's pairs of e (tokens ascending), so each expert's rows stay in token order.
ETC_SMALL_TASK void perm_task(KArgs& p, KLayer& L, int tau) {
  const int K = p.K, E = p.E;
  const int a0 = tau * BT * K, npairs = tile_rows(p, tau) * K;
  for (int i = threadIdx.x; i < npairs; i += MNT) {
    const int a = a0 + i;
    const int r = gp(L.tile_off)[tau * E + gp(L.topk_idx)[a]] + gp(L.lrank)[a];
    st_shared(L.sorted_assign + r, a);
    st_shared(L.pos + a, r);
  }
}

// ------------------------------------------------------------------ GU / D / F

// Static mode: the next ticket of this workgroup's XCD queue (see claim_static).
ETC_DEV int static_ticket(KArgs& p) { return xcd_ticket(p.sched); }

// Gate/up rows of a tile: A row r is the token of sorted row r (rows past the expert's
// count read the first row); B row b is in 16-row blocks that alternate gate / up over
// the same 16 ffn columns (columns past F read row F-1).  Their results are never stored.
template <typename TE>
ETC_DEV const char* gateup_row(KArgs& p, KLayer& L, const TileSmem& Ts, int e, int n, int bm,
                               int r, int lc) {
  const int H = p.H, F = p.F;
  if (r < bm) {
    const int tok = Ts.row_tok[r];
    const TE* xq = static_cast<const TE*>(p.xq);
    return reinterpret_cast<const char*>(xq + (size_t)(tok >= 0 ? tok : Ts.row_tok[0]) * H) + lc;
  }
  const int b = r - bm, blk = b >> 4;
  const int f = min(n * BN1 + (blk >> 1) * 16 + (b & 15), F - 1);
  const TE* src = static_cast<const TE*>((blk & 1) ? L.w_up : L.w_gate);
  return reinterpret_cast<const char*>(src + ((size_t)e * F + f) * H) + lc;
}

// SwiGLU of the tile into LDS (float, row stride GU_HSTR): small row tiles.
constexpr int GU_HSTR = BN1 + 1;
template <typename TE, int BMS>
ETC_DEV void gateup_small(KArgs& p, KLayer& L, int e, int n, TileSmem& Ts, float* hs) {
  using Tile = KTileS<TE, BMS, MNT>;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const char* rowp[Tile::LOADS];
  const int lc = Tile::load_chunk(tid) * 16;
#pragma unroll
  for (int i = 0; i < Tile::LOADS; ++i) {
    const int r = Tile::load_row(tid, i);
    rowp[i] = gateup_row<TE>(p, L, Ts, e, n, BMS, r < Tile::ROWS ? r : BMS, lc);
  }
  f32x4 acc[Tile::MI][Tile::NJ];
  Tile::run(Ts.gemm, rowp, p.H, acc);
  // wave w's blocks 0 and 1 are gate and up of ffn columns 16 w .. 16 w + 15
#pragma unroll
  for (int i = 0; i < Tile::MI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float g = acc[i][0][r], u = acc[i][1][r];
      hs[(i * 16 + (lane >> 4) * 4 + r) * GU_HSTR + w * 16 + (lane & 15)] = g / (1.0f + expf(-g)) * u;
    }
}

// The SwiGLU of a 128-row tile into LDS (float, row stride GU_HSTR).
template <typename TE>
ETC_DEV void gateup_large(KArgs& p, KLayer& L, int e, int n, int valid, TileSmem& Ts, float* hs) {
  using Tile = KTile<TE, MNT>;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / Tile::WN, wn = w % Tile::WN;
  const char* rowp[Tile::LOADS];
  const int lc = Tile::load_chunk(tid) * 16;
#pragma unroll
  for (int i = 0; i < Tile::LOADS; ++i) rowp[i] = gateup_row<TE>(p, L, Ts, e, n, BM, Tile::load_row(tid, i), lc);
  f32x4 acc[4][Tile::NJ];
  Tile::run(Ts.gemm, rowp, p.H, valid, acc);
  // column block j of this wave is gate (j even) or up (j odd) for ffn columns
  // n*BN1 + (wn*NJ + j)/2 * 16 ..
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < Tile::NJ / 2; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        const int col = (wn * Tile::NJ / 2 + jj) * 16 + (lane & 15);
        const float g = acc[i][2 * jj][r], u = acc[i][2 * jj + 1][r];
        hs[row * GU_HSTR + col] = g / (1.0f + expf(-g)) * u;
      }
}

// GU(e, m, n): row tile m of expert e against ffn columns n*BN1.. of gate and up.  The
// tile's layout in the workgroup's LDS arena follows its row count: up to 16 or 32 valid
// rows take the four-stage small-M layout, more rows the three-stage 128-row one.
template <typename TE>
ETC_TASK void gateup_task(KArgs& p, KLayer& L, int e, int m, int n, Smem& sm) {
  const int tid = threadIdx.x;
  const int F = p.F, K = p.K;
  TileSmem& Ts = sm.u.t;
  const int r0 = sm.lc.off[e] + m * BM;
  const int valid = min(BM, sm.lc.cnt[e] - m * BM);
  for (int i = tid; i < BM; i += MNT) Ts.row_tok[i] = (i < valid) ? gp(L.sorted_assign)[r0 + i] / K : -1;
  __syncthreads();

  static_assert(BM * GU_HSTR * 4 <= (int)sizeof(Ts.gemm), "staged tile fits the GEMM buffer");
  float* hs = reinterpret_cast<float*>(Ts.gemm);
  // (the tile functions return after a barrier: the arena is free for the staging)
  if (valid <= 16) gateup_small<TE, 16>(p, L, e, n, Ts, hs);
  else if (valid <= 32) gateup_small<TE, 32>(p, L, e, n, Ts, hs);
  else gateup_large<TE>(p, L, e, n, valid, Ts, hs);
  // static mode: draw the next ticket now; its atomic round trip overlaps the epilogue
  // (issued before the tile, it would hold up the tile's first wait for its copies).  The
  // drawn value is mapped to a ticket only after the epilogue: computing with it here
  // would make the wave wait for the atomic, and the barrier below the whole workgroup.
  const bool prefetch = p.mode == ETC_SCHED_STATIC;
  int drawn = 0;
  if (prefetch && tid == 0) drawn = xcd_ticket_draw(p.sched);
  __syncthreads();
  // whole rows out to hbuf, 16 bytes per store: 8 bf16 or 4 float columns (F is a
  // multiple of 64, so a store never straddles the edge).  16-byte stores: coherent
  // 8-byte stores move less than half the bytes per cycle when every CU stores at once.
  constexpr int CPS = 16 / (int)sizeof(TE), SPR = BN1 / CPS;  // columns per store, stores per row
  const int f0 = n * BN1, ncols = min(BN1, F - f0);
  TE* hb = static_cast<TE*>(p.hbuf) + (size_t)r0 * F + f0;  // the tile's first element
  for (int q = tid; q < valid * SPR; q += MNT) {
    const int row = q / SPR, c = (q % SPR) * CPS;
    if (c < ncols) {
      const float* src = hs + row * GU_HSTR + c;
      float v[CPS];
#pragma unroll
      for (int i = 0; i < CPS; ++i) v[i] = src[i];
      st_shared16(hb, (uint32_t)(((size_t)row * F + c) * sizeof(TE)), pack16<TE>(v));
    }
  }
  if (prefetch && tid == 0) sm.next_ticket = xcd_ticket_map(drawn);
}

// Down rows of a tile: A row r is sorted row r0 + r of hbuf from column kb (rows past the
// expert's count read row r0); B row b is row n2i*BN2 + b of the expert's w_down
// (columns past H read row H-1).  Their results are never stored.
template <typename TE>
ETC_DEV const char* down_row(KArgs& p, KLayer& L, int e, int n2i, int r0, int valid, int kb,
                             int bm, int r, int lc) {
  const int H = p.H, F = p.F;
  if (r < bm) {
    const TE* hb = static_cast<const TE*>(p.hbuf);
    return reinterpret_cast<const char*>(hb + (size_t)(r0 + (r < valid ? r : 0)) * F + kb) + lc;
  }
  const int h = min(n2i * BN2 + r - bm, H - 1);
  const TE* wd = static_cast<const TE*>(L.w_down);
  return reinterpret_cast<const char*>(wd + ((size_t)e * H + h) * F + kb) + lc;
}

constexpr int D_CSTR = BN2 + 1;  // row stride of the staged down tile (words)

template <typename TE, int BMS>
ETC_DEV void down_small(KArgs& p, KLayer& L, int e, int n2i, int r0, int valid, int kb, int klen,
                        float* ct) {
  using Tile = KTileS<TE, BMS, MNT>;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const char* rowp[Tile::LOADS];
  const int lc = Tile::load_chunk(tid) * 16;
#pragma unroll
  for (int i = 0; i < Tile::LOADS; ++i) {
    const int r = Tile::load_row(tid, i);
    rowp[i] = down_row<TE>(p, L, e, n2i, r0, valid, kb, BMS, r < Tile::ROWS ? r : BMS, lc);
  }
  f32x4 acc[Tile::MI][Tile::NJ];
  Tile::run(reinterpret_cast<char*>(ct), rowp, klen, acc);
#pragma unroll
  for (int i = 0; i < Tile::MI; ++i)
#pragma unroll
    for (int j = 0; j < Tile::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        ct[(i * 16 + (lane >> 4) * 4 + r) * D_CSTR + w * Tile::WCOLS + j * 16 + (lane & 15)] = acc[i][j][r];
}

template <typename TE>
ETC_DEV void down_large(KArgs& p, KLayer& L, int e, int n2i, int r0, int valid, int kb, int klen,
                        float* ct) {
  using Tile = KTile<TE, MNT>;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / Tile::WN, wn = w % Tile::WN;
  const char* rowp[Tile::LOADS];
  const int lc = Tile::load_chunk(tid) * 16;
#pragma unroll
  for (int i = 0; i < Tile::LOADS; ++i)
    rowp[i] = down_row<TE>(p, L, e, n2i, r0, valid, kb, BM, Tile::load_row(tid, i), lc);
  f32x4 acc[4][Tile::NJ];
  Tile::run(reinterpret_cast<char*>(ct), rowp, klen, valid, acc);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < Tile::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        ct[(wm * 64 + i * 16 + (lane >> 4) * 4 + r) * D_CSTR + wn * Tile::WCOLS + j * 16 + (lane & 15)] =
            acc[i][j][r];
}

// D(e, m, n2i, s): row tile m of expert e, output columns n2i*BN2.., ffn chunk s.  The
// tile's LDS layout follows its row count, as in gateup_task.
template <typename TE>
ETC_TASK void down_task(KArgs& p, KLayer& L, int e, int m, int n2i, int s, int gpc,
                       Smem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int H = p.H, F = p.F, K = p.K;
  TileSmem& Ts = sm.u.t;
  const int r0 = sm.lc.off[e] + m * BM;
  const int valid = min(BM, sm.lc.cnt[e] - m * BM);
  // The operand rows are the tile's rows of the sorted activations, which do not depend
  // on the tokens: the (token, slot) pair of each row is loaded now and used only by the
  // epilogue, so its round trip overlaps the tile instead of preceding the first copy.
  static_assert(BM <= MNT, "one row per thread");
  const int pair = tid < valid ? gp(L.sorted_assign)[r0 + tid] : -1;

  const int kb = s * gpc * BN1;
  const int klen = min(F, kb + gpc * BN1) - kb;
  // The tile goes through LDS first (row stride BN2 + 1 words: both passes free of bank
  // conflicts; the arena is free once the tile has returned), so that the results leave
  // as whole rows: each atomic instruction adds 64 consecutive columns of one token row
  // (two cache lines) rather than 16 columns of four different rows, and the ordered
  // combine writes its rows with 8-byte stores.
  static_assert(BM * D_CSTR * 4 <= (int)sizeof(Ts.gemm), "staged tile fits the GEMM buffer");
  float* ct = reinterpret_cast<float*>(Ts.gemm);
  if (valid <= 16) down_small<TE, 16>(p, L, e, n2i, r0, valid, kb, klen, ct);
  else if (valid <= 32) down_small<TE, 32>(p, L, e, n2i, r0, valid, kb, klen, ct);
  else down_large<TE>(p, L, e, n2i, r0, valid, kb, klen, ct);
  const float gate = pair >= 0 ? gp(L.topk_w)[pair] : 0.f;
  if (tid < BM) {
    Ts.row_tok[tid] = pair >= 0 ? pair / K : -1;
    Ts.row_gate[tid] = gate;
  }
  // the next ticket, as in gateup_task; drawn after the gate loads have returned, so
  // that nothing before the epilogue waits for it
  const bool prefetch = p.mode == ETC_SCHED_STATIC;
  int drawn = 0;
  if (prefetch && tid == 0) drawn = xcd_ticket_draw(p.sched);
  __syncthreads();
  const int c0 = n2i * BN2, ncols = min(BN2, H - c0);
  if (p.combine == ETC_COMBINE_ATOMIC) {
    for (int row = w; row < valid; row += NWAVE) {
      float* dst = p.out_acc + (size_t)Ts.row_tok[row] * H + c0;
      const float g = Ts.row_gate[row];
#pragma unroll
      for (int c = lane; c < BN2; c += 64)
        if (c < ncols) red_add(dst + c, g * ct[row * D_CSTR + c]);
    }
  } else {
    // H is a multiple of 128: four columns never straddle the edge (16-byte stores)
    float* yb = p.ybuf + (size_t)r0 * H + c0;  // the tile's first element
    for (int q = tid; q < valid * (BN2 / 4); q += MNT) {
      const int row = q / (BN2 / 4), c = (q % (BN2 / 4)) * 4;
      if (c < ncols) {
        const float* src = ct + row * D_CSTR + c;
        st_shared16(yb, (uint32_t)(((size_t)row * H + c) * sizeof(float)),
                    u32x4{__float_as_uint(src[0]), __float_as_uint(src[1]), __float_as_uint(src[2]),
                          __float_as_uint(src[3])});
      }
    }
  }
  if (prefetch && tid == 0) sm.next_ticket = xcd_ticket_map(drawn);
}

template <typename TE>
ETC_SMALL_TASK void finalize_task(KArgs& p, KLayer& L, int tau) {
  constexpr int EPC = 16 / (int)sizeof(TE);
  // chunks per thread whose loads are in flight together: the stores of one group are
  // not waited for before the next group's loads go out
  constexpr int U = 4;
  const int tid = threadIdx.x, H = p.H, K = p.K;
  const int t0 = tau * BT, nt = tile_rows(p, tau);
  const int nch = nt * H / EPC;
  TE* out = static_cast<TE*>(L.out);
  for (int cb = tid; cb < nch; cb += U * MNT) {
    float v[U][EPC];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < EPC; ++i) v[u][i] = 0.f;
    if (p.combine == ETC_COMBINE_ATOMIC) {
      f32x4 a[U][EPC / 4];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = min(cb + u * MNT, nch - 1);  // past the end: a repeat, never stored
        const int t = t0 + (c * EPC) / H, h = (c * EPC) % H;
#pragma unroll
        for (int i = 0; i < EPC / 4; ++i) a[u][i] = gld<f32x4>(p.out_acc + (size_t)t * H + h + 4 * i);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < EPC; ++i) v[u][i] = a[u][i / 4][i % 4];
    } else {
      for (int j = 0; j < K; ++j) {  // slot order
        float g[U];
        const float* y[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = min(cb + u * MNT, nch - 1);
          const int t = t0 + (c * EPC) / H, h = (c * EPC) % H;
          g[u] = gp(L.topk_w)[t * K + j];
          y[u] = p.ybuf + (size_t)gp(L.pos)[t * K + j] * H + h;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int i = 0; i < EPC; i += 4) {
            const f32x4 a = gld<f32x4>(y[u] + i);
            v[u][i] += g[u] * a[0]; v[u][i + 1] += g[u] * a[1];
            v[u][i + 2] += g[u] * a[2]; v[u][i + 3] += g[u] * a[3];
          }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = cb + u * MNT;
      if (c < nch) st_shared16(out + (size_t)t0 * H, (uint32_t)(c * 16), pack16<TE>(v[u]));
    }
  }
}

// ------------------------------------------------------------------ scheduling

// Static mode: the fixed task order (per layer: all R, all P, all GU, all D, all F) is cut
// into chunks of G consecutive tasks, chunk c belonging to queue c mod Q; workgroup b
// draws from queue b mod Q.  The dispatcher places workgroup b on XCD b mod 8, so with
// Q = 8 each chunk runs on one XCD: the row tiles that share a weight tile and the
// column tiles that share a token tile are taken together and meet in that XCD's L2
// instead of being fetched once per XCD.  G = workers / Q, one task per CU of the XCD.
// Each queue hands out its tasks in the global order and has at least one workgroup
// (Q <= workers), so the smallest waiting task always has its inputs claimed by
// workgroups that are not waiting on it: the order stays deadlock-free.  A gate/up or
// down task draws its workgroup's next ticket while it runs; that ticket is larger than
// the running task's, so the smallest unfinished ticket is still the current task of
// its workgroup and the argument holds.
//
// Static: the ticket's task (the one drawn during the previous task, if any); waits for
// S of a layer before decoding past it.
ETC_DEV bool claim_static(KArgs& p, Task& t, Smem& sm) {
  const int ticket = sm.next_ticket >= 0 ? sm.next_ticket : static_ticket(p);
  sm.next_ticket = -1;
  int base = 0;
  for (int l = 0; l < p.L; ++l) {
    if (sm.lbase[l + 1] >= 0 && ticket >= sm.lbase[l + 1]) {
      base = sm.lbase[l + 1];
      continue;
    }
    KLayer& L = p.layer[l];
    t.layer = l;
    if (ticket < base + p.n_rq) { t.kind = K_R; t.a = ticket - base; return true; }
    int off = ticket - base - p.n_rq;
    if (off < p.n_perm) { t.kind = K_P; t.a = off; return true; }
    off -= p.n_perm;
    if (!(sm.scan_seen >> l & 1u)) {
      if (!spin_until_geq(L.ev_scan, 1, p.sched, p.timeout_ticks, 10 + l)) return false;
      sm.scan_seen |= 1u << l;
    }
    // the layer's plan from the workgroup's LDS copy when it holds this layer
    const bool cached = sm.lc.layer == l;
    auto plan = [&](int w) ETC_INLINE { return cached ? sm.lc.plan[w] : gp(L.plan)[w]; };
    auto rtb = [&](int e) ETC_INLINE { return cached ? sm.lc.rtb[e] : gp(L.rt_base)[e]; };
    const int ngu = plan(PL_NGU), nd = plan(PL_ND), nf = plan(PL_NF), nS = plan(PL_NS);
    if (off < ngu) {
      const int e = owner_expert_by(rtb, p.E, off, p.n1);
      const int me = rtb(e + 1) - rtb(e);
      const int loc = off - rtb(e) * p.n1;
      t.kind = K_GU; t.a = e; t.b = loc % me; t.c = loc / me;
      return true;
    }
    off -= ngu;
    if (off < nd) {
      const int e = owner_expert_by(rtb, p.E, off, p.n2 * nS);
      const int me = rtb(e + 1) - rtb(e);
      const int loc = off - rtb(e) * p.n2 * nS;
      t.kind = K_D; t.a = e; t.b = loc % me; t.c = (loc / me) % p.n2; t.d = loc / (me * p.n2);
      return true;
    }
    off -= nd;
    if (off < nf) { t.kind = K_F; t.a = off; return true; }
    base = plan(PL_NEXTBASE);
    sm.lbase[l + 1] = base;
  }
  t.kind = K_NONE;
  return true;
}

// Dynamic: the next queue slot; slots below n_rq are the first layer's R tasks.  The
// watchdog counts progress as tasks being pushed anywhere (the queue tail moving).
ETC_DEV bool claim_dynamic(KArgs& p, Task& t) {
  const int slot = ev_add_relaxed(p.sched + W_QHEAD, 1);
  if (slot < p.n_rq) {
    t.kind = K_R; t.layer = 0; t.a = slot;
    return true;
  }
  // every slot below the final queue total is filled exactly once; a workgroup that
  // drew a slot past the end of the array only waits for the total to be known
  const bool in_array = slot < p.queue_len;
  Watchdog wd;
  for (int it = 0;; ++it) {
    if (in_array && q_load_relaxed(p.queue + slot) != 0) {
      const long long v = q_load(p.queue + slot);  // acquire: the task's inputs are ready
      q_store_relaxed(p.queue + slot, 0);           // the slot is clean for the next call
      t = dec(v);
      return true;
    }
    // every WATCH_EVERY polls of the slot: every layer has planned (acquire: their
    // additions to the total are visible) and this slot lies past the final total, or
    // the watchdog.  (Reading those words at every poll would keep their lines busy
    // under the producers' additions.)
    if (it % WATCH_EVERY == 0) {
      if (ev_load_relaxed(p.sched + W_PLANNED) == p.L && ev_load(p.sched + W_PLANNED) == p.L &&
          slot >= ev_load_relaxed(p.sched + W_QTOTAL)) {
        t.kind = K_NONE;
        return true;
      }
      if (it == 0) wd.start(p.timeout_ticks, ev_load_relaxed(p.sched + W_QTAIL));
      else if (wd.expired(p.sched, p.timeout_ticks, ev_load_relaxed(p.sched + W_QTAIL), 2))
        return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Static mode: wait until the task's inputs are complete (thread 0).
ETC_DEV bool wait_deps(KArgs& p, const Task& t, Smem& sm) {
  KLayer& L = p.layer[t.layer];
  switch (t.kind) {
    case K_R:
      if (t.layer == 0) return true;
      return spin_until_geq(p.layer[t.layer - 1].ev_done + t.a / p.Q, 1, p.sched, p.timeout_ticks, 20);
    case K_P:
      return spin_until_geq(L.ev_scan, 1, p.sched, p.timeout_ticks, 24);
    case K_GU:
      if (sm.perm_seen >> t.layer & 1u) return true;
      if (!spin_until_geq(L.ev_perm, p.n_rt, p.sched, p.timeout_ticks, 25)) return false;
      sm.perm_seen |= 1u << t.layer;
      return true;
    case K_D: {
      const int gpc = sm.lc.plan[PL_GPC];
      const int rt = sm.lc.rtb[t.a] + t.b;
      const int need = min(gpc, p.n1 - t.d * gpc);
      return spin_until_geq(L.ev_gu + rt * p.n1 + t.d, need, p.sched, p.timeout_ticks, 22);
    }
    case K_F: {
      const int target = tile_rows(p, t.a) * p.K * p.n2 * sm.lc.plan[PL_NS];
      return spin_until_geq(L.ev_comb + t.a, target, p.sched, p.timeout_ticks, 23);
    }
    default:
      return true;
  }
}

// Every thread of the workgroup: copy layer l's plan, row-tile bases, offsets and counts
// into the LDS cache (the layer's S has completed: its results were acquired with the
// task's claim).
ETC_DEV void load_layer_cache(KArgs& p, int l, Smem& sm) {
  KLayer& L = p.layer[l];
  const int tid = threadIdx.x, E = p.E;
  if (tid < PL_WORDS) sm.lc.plan[tid] = gp(L.plan)[tid];
  for (int i = tid; i <= E; i += MNT) {
    sm.lc.rtb[i] = gp(L.rt_base)[i];
    sm.lc.off[i] = gp(L.offsets)[i];
    if (i < E) sm.lc.cnt[i] = gp(L.counts)[i];
  }
  if (tid == 0) sm.lc.layer = l;
}

// Enqueue n tasks (dynamic mode); every thread of the workgroup calls this.
template <typename Gen>
ETC_DEV void push_many(KArgs& p, Smem& sm, int n, Gen gen) {
  if (threadIdx.x == 0) sm.ibuf[0] = p.n_rq + ev_add_relaxed(p.sched + W_QTAIL, n);
  __syncthreads();
  const int base = sm.ibuf[0];
  // the results these tasks read were published (publish_shared) before the call
  for (int i = threadIdx.x; i < n; i += MNT) q_store_relaxed(p.queue + base + i, enc(gen(i)));
  __syncthreads();
}

// The results the task reads were published (publish_shared) before the call.
ETC_DEV void push_one(KArgs& p, const Task& t) {
  const int slot = p.n_rq + ev_add_relaxed(p.sched + W_QTAIL, 1);
  q_store_relaxed(p.queue + slot, enc(t));
}

// Dynamic mode: every gate/up task of the layer is ready (the permutation is complete).
ETC_DEV void push_gateup(KArgs& p, KLayer& L, int layer, Smem& sm) {
  const int n1 = p.n1, E = p.E;
  push_many(p, sm, gp(L.plan)[PL_NGU], [&](int i) {
    const int e = owner_expert(L.rt_base, E, i, n1);
    const int me = gp(L.rt_base)[e + 1] - gp(L.rt_base)[e];
    const int loc = i - gp(L.rt_base)[e] * n1;
    Task g;
    g.kind = K_GU; g.layer = layer; g.a = e; g.b = loc % me; g.c = loc / me; g.d = 0;
    return g;
  });
}

// After S (run by the last routing task of the layer, in both modes): publish ev_scan,
// and ev_perm as well when S scattered the permutation itself.  Dynamic mode then
// enqueues the P tasks (or, without them, every gate/up task) and adds the layer's task
// count to the queue total.
ETC_DEV void after_scan(KArgs& p, int layer, Smem& sm) {
  KLayer& L = p.layer[layer];
  publish_shared();
  if (threadIdx.x == 0) {
    ev_store_relaxed(L.ev_scan, 1);  // the event tensor is complete
    if (p.n_perm == 0) ev_store_relaxed(L.ev_perm, p.n_rt);
  }
  if (p.mode != ETC_SCHED_DYNAMIC) return;
  if (p.n_perm > 0) {
    push_many(p, sm, p.n_perm, [&](int i) {
      Task t;
      t.kind = K_P; t.layer = layer; t.a = i; t.b = t.c = t.d = 0;
      return t;
    });
  } else {
    push_gateup(p, L, layer, sm);
  }
  if (threadIdx.x == 0) {
    // the plan words are in global memory, written by this thread before publish_shared
    const int added = p.n_perm + gp(L.plan)[PL_NGU] + gp(L.plan)[PL_ND] + gp(L.plan)[PL_NF] +
                      (layer + 1 < p.L ? p.n_rq : 0) + (layer == 0 ? p.n_rq : 0);
    ev_add_relaxed(p.sched + W_QTOTAL, added);
    ev_add(p.sched + W_PLANNED, 1);
  }
}

// One ETC_FLAG_TRACE record: task word, start of its claim, workgroup and ticks spent
// claiming / waiting, ticks running.
ETC_DEV void trace_record(KArgs& p, const Task& t, uint64_t t_claim, uint64_t t_run, uint64_t t_end) {
  const int i = ev_add_relaxed(p.sched + W_TRACE, 1);
  if (i < p.trace_cap) {
    ETC_GLOBAL unsigned long long* r = gp(p.trace) + 4 * (size_t)i;
    r[0] = (unsigned long long)enc(t);
    r[1] = t_claim;
    r[2] = (unsigned long long)blockIdx.x | ((unsigned long long)(uint32_t)(t_run - t_claim) << 32);
    r[3] = (unsigned long long)(uint32_t)(t_end - t_run);
  }
}

// One task of either scheduler: its body, then its signals (and, in dynamic mode, the
// tasks its signal releases).  Every thread of the workgroup calls this.
template <typename TE>
ETC_DEV void run_task(KArgs& p, KLayer& L, const Task& t, Smem& sm) {
  const int tid = threadIdx.x;
  if (t.kind == K_R && p.n_rt == 1) {
    // the layer's only routing tile: S follows on the tile's LDS results, and one
    // publish covers both (in the slice that completed the tile)
    if (!route_task<TE>(p, L, t.a, sm)) return;
    __syncthreads();
    const uint64_t t0 = now_ticks();
    scan_single_tile(p, L, t.layer, sm);
    if (tid == 0) ev_add_relaxed(L.ev_route, 1);
    after_scan(p, t.layer, sm);
    if (tid == 0 && (p.flags & ETC_FLAG_TRACE)) {
      Task st;
      st.kind = K_S; st.layer = t.layer; st.a = st.b = st.c = st.d = 0;
      trace_record(p, st, t0, t0, now_ticks());
    }
  } else if (t.kind == K_R) {
    if (!route_task<TE>(p, L, t.a, sm)) return;  // another slice completes the tile
    publish_shared();
    if (tid == 0) {
      // the last routing tile of the layer runs S, which reads every tile's results
      // (acquire: they were published before the other tiles' signals)
      sm.flag = (ev_add_acquire(L.ev_route, 1) + 1 == p.n_rt) ? 1 : 0;
    }
    __syncthreads();
    if (sm.flag) {
      const uint64_t t0 = now_ticks();
      scan_task(p, L, t.layer, sm);
      after_scan(p, t.layer, sm);
      if (tid == 0 && (p.flags & ETC_FLAG_TRACE)) {  // S keeps a trace record of its own
        Task st;
        st.kind = K_S; st.layer = t.layer; st.a = st.b = st.c = st.d = 0;
        trace_record(p, st, t0, t0, now_ticks());
      }
    }
  } else if (t.kind == K_P) {
    perm_task(p, L, t.a);
    publish_shared();
    if (tid == 0) {
      if (p.mode == ETC_SCHED_DYNAMIC) {
        sm.flag = ev_add_acquire(L.ev_perm, 1) + 1 == p.n_rt ? 1 : 0;
      } else {
        ev_signal(L.ev_perm, 1);
        sm.flag = 0;
      }
    }
    __syncthreads();
    if (sm.flag) push_gateup(p, L, t.layer, sm);  // the permutation is complete
  } else if (t.kind == K_GU) {
    gateup_task<TE>(p, L, t.a, t.b, t.c, sm);
    publish_shared();
    const int gpc = sm.lc.plan[PL_GPC];
    const int s = t.c / gpc;
    if (tid == 0) {
      const int rt = sm.lc.rtb[t.a] + t.b;
      const int need = min(gpc, p.n1 - s * gpc);
      if (p.mode == ETC_SCHED_DYNAMIC) {
        sm.flag = ev_add_acquire(L.ev_gu + rt * p.n1 + s, 1) + 1 == need ? 1 : 0;
      } else {
        ev_signal(L.ev_gu + rt * p.n1 + s, 1);  // static: nothing reads the old value
        sm.flag = 0;
      }
    }
    __syncthreads();
    if (sm.flag) {
      const int layer = t.layer, e = t.a, m = t.b;
      push_many(p, sm, p.n2, [&](int i) {
        Task d;
        d.kind = K_D; d.layer = layer; d.a = e; d.b = m; d.c = i; d.d = s;
        return d;
      });
    }
  } else if (t.kind == K_D) {
    down_task<TE>(p, L, t.a, t.b, t.c, t.d, sm.lc.plan[PL_GPC], sm);
    // The results are published once for the whole task, then one signal goes out per
    // run of rows in the same routing tile (rows are token-sorted; a tile's rows can
    // span dozens of routing tiles).  In dynamic mode the signals acquire, for the last
    // arriver that enqueues the finalize task.
    publish_shared();
    const int valid = min(BM, sm.lc.cnt[t.a] - t.b * BM);
    if (tid < valid) {
      const int tau = sm.u.t.row_tok[tid] / BT;
      if (tid == 0 || sm.u.t.row_tok[tid - 1] / BT != tau) {
        int len = 1;
        while (tid + len < valid && sm.u.t.row_tok[tid + len] / BT == tau) ++len;
        if (p.mode == ETC_SCHED_DYNAMIC) {
          const int old = ev_add_acquire(L.ev_comb + tau, len);
          if (old + len == tile_rows(p, tau) * p.K * p.n2 * sm.lc.plan[PL_NS]) {
            Task f;
            f.kind = K_F; f.layer = t.layer; f.a = tau; f.b = f.c = f.d = 0;
            push_one(p, f);
          }
        } else {
          ev_signal(L.ev_comb + tau, len);  // static: nothing reads the old value
        }
      }
    }
    __syncthreads();
  } else if (t.kind == K_F) {
    finalize_task<TE>(p, L, t.a);
    publish_shared();
    if (tid == 0) {
      ev_store_relaxed(L.ev_done + t.a, 1);
      if (p.mode == ETC_SCHED_DYNAMIC && t.layer + 1 < p.L) {
        // the next layer's router slices of these tokens
        const int slot = p.n_rq + ev_add_relaxed(p.sched + W_QTAIL, p.Q);
        for (int q = 0; q < p.Q; ++q) {
          Task r;
          r.kind = K_R; r.layer = t.layer + 1; r.a = t.a * p.Q + q; r.b = r.c = r.d = 0;
          q_store_relaxed(p.queue + slot + q, enc(r));
        }
      }
    }
    __syncthreads();
  }
}


// ------------------------------------------------------------------ dedicated scheduler
//
// Mode ETC_SCHED_DEDICATED: workgroup 0 schedules and the others work, after the runtime
// the tutorial chapter "5 · Event Tensor et le dynamisme" describes for MPK (Q&A on the
// Cluster Launch Control): scheduler units watch the events and hand ready tasks to
// worker queues.  Workers never wait on a counter.
//
// Worker w owns a two-slot mailbox (words 2w and 2w+1 of the queue region) and takes its
// slots in turn.  It posts the idle word in slot 0 when it starts; then it waits on its
// current slot for a task word, runs the task, signals its counters as in static mode,
// writes the idle word back into the slot and moves to the other slot.  A slot is empty
// when it holds 0 or the idle word.  With two slots the scheduler can queue a ready task
// behind the one a worker is running, so the worker starts it without a round trip
// through the scheduler.
//
// The scheduler is one wavefront.  It walks the static topological order with a window
// of 64 tickets, one per lane: each lane decodes its ticket (once the ticket's layer has
// published its plan) and reads the one counter the task waits on.  Ready tickets go
// out in ticket order, each preferring the XCD that static mode would run it on (chunks
// of workers/8 consecutive tickets per XCD, workgroup w on XCD w mod 8, so tasks that
// share a weight tile meet in one L2): first to idle workers of that XCD, then behind a
// running task there, then to idle workers elsewhere.  Every ticket before the window is
// assigned, so the producers of the window's first ticket are all assigned and it
// becomes ready as they finish: the scheduler keeps making progress.  Only workers that
// have posted the idle word receive tasks, so a workgroup that is not resident yet holds
// none.  Once every ticket is assigned and every worker is idle it writes the exit word
// into each worker's current slot; a worker empties both slots as it leaves.  All the
// mailbox and counter reads of one pass are issued before any is used: one memory round
// trip per pass.

constexpr int K_EXIT = 15;  // mailbox word: leave the task loop
constexpr int K_IDLE = 14;  // mailbox word: the worker waits for a task
constexpr int NXCD = 8;
// The scheduler lane l tracks workers 1 + l + 64 j (j < DED_PER_LANE) in registers; all
// of them sit on XCD (1 + l) mod 8.
constexpr int DED_PER_LANE = 4;
constexpr int DED_MAX_GRID = 1 + DED_PER_LANE * WAVE;

// Per-XCD counts of one scheduler pass.
struct SchedTable {
  unsigned long long ready[NXCD];  // ready tickets preferring x (bit i: i-th ticket in order)
  unsigned long long third[NXCD];  // of those, the ones queued behind a running task
  int n_idle[NXCD], n_b1[NXCD];    // idle workers and workers holding one task on x
  int take[NXCD];                  // idle workers of x that x's own tickets take
  int pool0[NXCD];                 // first pool entry of x's left-over idle workers
  int pool_total;
};

struct SchedSmem {
  SchedTable tab;
  int planned;                  // bit l: layer l's plan and row-tile bases are cached
  int base[MAXL + 1];           // first ticket of each layer (-1: not known yet)
  int plan[MAXL][PL_WORDS];
  int rtb[MAXL][MAXE + 1];
  int word;                     // lane 0's reading, for the whole wave
};
static_assert(sizeof(SchedSmem) <= sizeof(SmemU), "the scheduler's state fits the task area");

// The task of ticket c.  Returns 0 with the task, 1 if a plan it needs is not known yet,
// 2 if c lies past the last ticket (every layer has planned).
ETC_DEV int sched_decode(KArgs& p, const SchedSmem& S, int c, Task& t) {
  t.kind = K_NONE; t.layer = 0; t.a = t.b = t.c = t.d = 0;
  for (int l = 0; l < p.L; ++l) {
    const int base = S.base[l];
    if (base < 0) return 1;
    t.layer = l;
    if (c < base + p.n_rq) { t.kind = K_R; t.a = c - base; return 0; }
    int off = c - base - p.n_rq;
    if (off < p.n_perm) { t.kind = K_P; t.a = off; return 0; }
    off -= p.n_perm;
    if (!(S.planned >> l & 1)) return 1;
    const int* pl = S.plan[l];
    const int* rb = S.rtb[l];
    const int ngu = pl[PL_NGU], nd = pl[PL_ND], nf = pl[PL_NF], nS = pl[PL_NS];
    if (off < ngu) {
      const int e = owner_expert_by([&](int i) ETC_INLINE { return rb[i]; }, p.E, off, p.n1);
      const int me = rb[e + 1] - rb[e], loc = off - rb[e] * p.n1;
      t.kind = K_GU; t.a = e; t.b = loc % me; t.c = loc / me;
      return 0;
    }
    off -= ngu;
    if (off < nd) {
      const int e = owner_expert_by([&](int i) ETC_INLINE { return rb[i]; }, p.E, off, p.n2 * nS);
      const int me = rb[e + 1] - rb[e], loc = off - rb[e] * p.n2 * nS;
      t.kind = K_D; t.a = e; t.b = loc % me; t.c = (loc / me) % p.n2; t.d = loc / (me * p.n2);
      return 0;
    }
    off -= nd;
    if (off < nf) { t.kind = K_F; t.a = off; return 0; }
  }
  return 2;
}

// The counter the task waits on and its target (the same waits as static mode); null
// when the task waits on nothing.
ETC_DEV const int* sched_dep(KArgs& p, const SchedSmem& S, const Task& t, int& target) {
  KLayer& L = p.layer[t.layer];
  switch (t.kind) {
    case K_R:
      target = 1;
      return t.layer == 0 ? nullptr : p.layer[t.layer - 1].ev_done + t.a / p.Q;
    case K_P:
      target = 1;
      return L.ev_scan;
    case K_GU:
      target = p.n_rt;
      return L.ev_perm;
    case K_D: {
      const int gpc = S.plan[t.layer][PL_GPC];
      target = min(gpc, p.n1 - t.d * gpc);
      return L.ev_gu + (S.rtb[t.layer][t.a] + t.b) * p.n1 + t.d;
    }
    case K_F:
      target = tile_rows(p, t.a) * p.K * p.n2 * S.plan[t.layer][PL_NS];
      return L.ev_comb + t.a;
    default:
      target = 0;
      return nullptr;
  }
}

ETC_DEV bool slot_empty(long long v) { return v == 0 || v == K_IDLE; }
ETC_DEV unsigned long long lanes_below(int lane) { return (1ull << lane) - 1ull; }
// lanes whose workers sit on XCD x: (1 + l) mod 8 == x
ETC_DEV unsigned long long xcd_lanes(int x) { return 0x0101010101010101ull << ((x + NXCD - 1) % NXCD); }
ETC_DEV unsigned long long rot_right(unsigned long long m, int s) { return s ? (m >> s) | (m << (64 - s)) : m; }
// position of the r-th set bit (r counted from 0; the mask has more than r set bits)
ETC_DEV int nth_bit(unsigned long long m, int r) {
  int pos = 0;
  for (int width = 32; width >= 1; width >>= 1) {
    const unsigned long long low = m & ((1ull << width) - 1ull);
    const int c = __popcll(low);
    if (r >= c) { r -= c; m >>= width; pos += width; } else { m = low; }
  }
  return pos;
}
// The r-th worker (lane-major within each group of 64, groups in order) among the
// per-group masks restricted to the lanes of XCD x.
ETC_DEV int nth_worker(const unsigned long long (&m)[DED_PER_LANE], unsigned long long xl, int r) {
  int w = -1;
#pragma unroll
  for (int j = 0; j < DED_PER_LANE; ++j) {
    const unsigned long long mj = m[j] & xl;
    const int c = __popcll(mj);
    if (w < 0 && r < c) w = 1 + nth_bit(mj, r) + WAVE * j;
    if (w < 0) r -= c;
  }
  return w;
}

// The scheduler: every lane of wave 0 of workgroup 0.  Returns when every worker has been
// sent the exit word, or when the call is aborted.
//
// Lane l holds the window's ticket c with c = l (mod 64), so a ticket keeps its lane
// until it is assigned and only tickets that enter the window are decoded.  Assignment,
// in ticket order: (1) the idle workers of the ticket's XCD; (2) idle workers of other
// XCDs (XCD by XCD); (3) behind the task of a worker of its XCD that holds one.  Each
// lane also owns the state of its workers (tasks held, oldest slot) and works out from
// the same wave-wide counts whether one of them was given a task.
ETC_DEV void run_scheduler(KArgs& p, Smem& sm) {
  SchedSmem& S = *reinterpret_cast<SchedSmem*>(&sm.u);
  const int lane = threadIdx.x & 63;
  const int W = (int)gridDim.x;    // workers 1 .. W-1
  const int G = max(1, W / NXCD);  // tickets per chunk of one XCD
  const int my_x = (1 + lane) % NXCD;
  const unsigned long long my_xl = xcd_lanes(my_x);
  if (lane <= MAXL) S.base[lane] = lane == 0 ? 0 : -1;
  if (lane == 0) S.planned = 0;
  __builtin_amdgcn_wave_barrier();
  int o[DED_PER_LANE], h[DED_PER_LANE];  // tasks held (-1: not started), oldest slot
#pragma unroll
  for (int j = 0; j < DED_PER_LANE; ++j) { o[j] = -1; h[j] = 0; }
  int next = 0;  // lowest ticket not yet assigned
  int c = lane;  // this lane's ticket
  bool assigned = false;
  Task t;
  int st = 1;  // sched_decode's result for c
  const int* dep = nullptr;
  int target = 0;
  Watchdog wd;
  for (int it = 0;; ++it) {
    // ---- every read of the pass is issued before any is used
    int pend = -1;  // the layer whose plan is awaited (at most one)
    for (int l = 0; l < p.L; ++l)
      if (pend < 0 && S.base[l] >= 0 && !(S.planned >> l & 1)) pend = l;
    if (st == 1) {
      st = sched_decode(p, S, c, t);
      dep = st == 0 ? sched_dep(p, S, t, target) : nullptr;
    }
    // (every lane reads, without a branch, so the wait for it lands with the others)
    const int scan_v = ev_load_relaxed(pend >= 0 ? p.layer[pend].ev_scan : p.sched + W_QHEAD);
    const int dep_v = (st == 0 && !assigned && dep) ? ev_load_relaxed(dep) : 0;
    // (the low word of a slot tells empty, idle and task words apart: a task word's
    // low four bits are its kind, 1 to 6)
    int b0[DED_PER_LANE], b1[DED_PER_LANE];
#pragma unroll
    for (int j = 0; j < DED_PER_LANE; ++j) {
      const int w = 1 + lane + WAVE * j;
      const int* slots = reinterpret_cast<const int*>(p.queue + 2 * w);
      b0[j] = (w < W && o[j] != 0) ? ev_load_relaxed(slots + 2 * h[j]) : 0;
      b1[j] = (w < W && o[j] == 2) ? ev_load_relaxed(slots + 2 * (h[j] ^ 1)) : 0;
    }
    // ---- worker states: started, finished tasks
    unsigned long long I[DED_PER_LANE], B1[DED_PER_LANE], Hm[DED_PER_LANE];
#pragma unroll
    for (int j = 0; j < DED_PER_LANE; ++j) {
      const bool valid = 1 + lane + WAVE * j < W;
      const bool start = valid && o[j] < 0 && b0[j] == K_IDLE;
      const bool fin1 = valid && o[j] > 0 && (b0[j] == 0 || b0[j] == K_IDLE);
      const bool fin2 = fin1 && o[j] == 2 && (b1[j] == 0 || b1[j] == K_IDLE);
      o[j] = start ? 0 : o[j] - (int)fin1 - (int)fin2;
      h[j] ^= (int)fin1 ^ (int)fin2;
      I[j] = __ballot(valid && o[j] == 0);
      B1[j] = __ballot(valid && o[j] == 1);
      Hm[j] = __ballot(h[j] != 0);
    }
    int nidle = 0, started = 0;
#pragma unroll
    for (int j = 0; j < DED_PER_LANE; ++j) {
      nidle += __popcll(I[j]);
      started += __popcll(__ballot(1 + lane + WAVE * j < W && o[j] >= 0));
    }

    // ---- the plan of the awaited layer, once its scan has completed
    if (lane == 0) S.word = pend >= 0 && scan_v >= 1 && ev_load(p.layer[pend].ev_scan) >= 1;  // acquire
    __builtin_amdgcn_wave_barrier();
    if (S.word) {
      KLayer& L = p.layer[pend];
      if (lane < PL_WORDS) S.plan[pend][lane] = gp(L.plan)[lane];
      for (int e = lane; e <= p.E; e += WAVE) S.rtb[pend][e] = gp(L.rt_base)[e];
      __builtin_amdgcn_wave_barrier();
      if (lane == 0) {
        S.base[pend + 1] = S.plan[pend][PL_NEXTBASE];
        S.planned |= 1 << pend;
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- ready tickets to workers.  Wave-wide counts per XCD go to a small LDS table
    // that each lane reads at its ticket's XCD and at its workers' XCD.
    const bool ready = st == 0 && !assigned && (dep == nullptr || dep_v >= target);
    const int xp = (c / G) % NXCD;
    const int sh = next & 63;  // lane of the lowest ticket
    const unsigned long long before = lanes_below((lane - sh) & 63);  // earlier tickets
    SchedTable& X = S.tab;
    {
      int pool = 0;
#pragma unroll
      for (int x = 0; x < NXCD; ++x) {
        const unsigned long long xl = xcd_lanes(x);
        const unsigned long long R = rot_right(__ballot(ready && xp == x), sh);
        int ni = 0, nb = 0;
#pragma unroll
        for (int j = 0; j < DED_PER_LANE; ++j) { ni += __popcll(I[j] & xl); nb += __popcll(B1[j] & xl); }
        const int take = min(__popcll(R), ni);
        if (lane == x) {
          X.ready[x] = R; X.n_idle[x] = ni; X.n_b1[x] = nb; X.take[x] = take; X.pool0[x] = pool;
        }
        pool += ni - take;  // idle workers of x that its own tickets leave
      }
      if (lane == 0) X.pool_total = pool;
    }
    __builtin_amdgcn_wave_barrier();
    const int rank = __popcll(X.ready[xp] & before);
    const int t_nidle = X.n_idle[xp], t_take = X.take[xp];
    const int pool_total = X.pool_total;
    // (1) an idle worker of its own XCD; (2) an idle worker elsewhere: entry srank of the
    // pool, XCD by XCD
    const bool spill = ready && rank >= t_nidle;
    const unsigned long long SP = rot_right(__ballot(spill), sh);
    const int srank = __popcll(SP & before);
    const int n2 = min(__popcll(SP), pool_total);
    int pick_x = xp, pick_r = rank;
    bool pick = ready && rank < t_take, pick_b1 = false;
    if (spill && srank < pool_total) {
      int px = 0;
      for (int x = 1; x < NXCD; ++x)
        if (srank >= X.pool0[x] && X.n_idle[x] > X.take[x]) px = x;
      pick = true;
      pick_x = px;
      pick_r = X.take[px] + (srank - X.pool0[px]);
    }
    // (3) behind the one task a worker of its own XCD holds, once every worker has
    // started (while workers are still starting, a queued task could wait behind a
    // routing task for its whole length)
    const bool third = spill && srank >= pool_total && started == W - 1;
#pragma unroll
    for (int x = 0; x < NXCD; ++x) {
      const unsigned long long Q = rot_right(__ballot(third && xp == x), sh);
      if (lane == x) X.third[x] = Q;
    }
    __builtin_amdgcn_wave_barrier();
    if (third) {
      const int q = __popcll(X.third[xp] & before);
      if (q < X.n_b1[xp]) { pick = true; pick_b1 = true; pick_r = q; }
    }
    int w_to = -1;
    if (pick) {
      unsigned long long m[DED_PER_LANE];
#pragma unroll
      for (int j = 0; j < DED_PER_LANE; ++j) m[j] = pick_b1 ? B1[j] : I[j];
      w_to = nth_worker(m, xcd_lanes(pick_x), pick_r);
      // the slot after the worker's current task (idle: its current slot); the task's
      // inputs reached the point of coherence before the counter did, and the worker
      // acquires its slot before reading them
      const int jw = (w_to - 1) / WAVE, lw = (w_to - 1) % WAVE;
      unsigned long long hm = Hm[0];
#pragma unroll
      for (int j = 1; j < DED_PER_LANE; ++j)
        if (jw == j) hm = Hm[j];
      const int slot = (int)((hm >> lw) & 1ull) ^ (pick_b1 ? 1 : 0);
      q_store_relaxed(p.queue + 2 * w_to + slot, enc(t));
    }
    // this lane's workers that were given a task: its rank among the idle (or one-task)
    // workers of its XCD decides, with the counts every lane saw
    {
      const int o_take = X.take[my_x], o_pool0 = X.pool0[my_x];
      const int o_n3 = min(__popcll(X.third[my_x]), X.n_b1[my_x]);
      int ri = 0, rb = 0;
#pragma unroll
      for (int j = 0; j < DED_PER_LANE; ++j) {
        const unsigned long long mi = I[j] & my_xl, mb = B1[j] & my_xl;
        const int myri = ri + __popcll(mi & lanes_below(lane));
        const int myrb = rb + __popcll(mb & lanes_below(lane));
        const int w = 1 + lane + WAVE * j;
        if (w < W && o[j] == 0) {
          if (myri < o_take || o_pool0 + (myri - o_take) < n2) o[j] = 1;
        } else if (w < W && o[j] == 1) {
          if (myrb < o_n3) o[j] = 2;
        }
        ri += __popcll(mi);
        rb += __popcll(mb);
      }
    }
    __builtin_amdgcn_wave_barrier();
    const unsigned long long gmask = __ballot(w_to >= 0);
    if (gmask && lane == 0) ev_add_relaxed(p.sched + W_QHEAD, 1);  // progress seen by idle workers
    if (w_to >= 0) assigned = true;
    // slide the window past its assigned prefix; the lanes it passes take the tickets
    // that enter it
    const unsigned long long A = rot_right(__ballot(assigned), sh);
    const int done = A == ~0ull ? 64 : __builtin_ctzll(~A);
    next += done;
    if (assigned && c < next) {
      c += WAVE;
      assigned = false;
      st = 1;
    }

    const int total = S.base[p.L];  // -1 until every layer has planned
    if (total >= 0 && next >= total && nidle == W - 1 && gmask == 0) {
#pragma unroll
      for (int j = 0; j < DED_PER_LANE; ++j) {
        const int w = 1 + lane + WAVE * j;
        if (w < W) q_store_relaxed(p.queue + 2 * w + h[j], (long long)K_EXIT);
      }
      return;
    }
    // the watchdog (lane 0) counts a new ticket assigned or a worker finishing as progress
    const int seen = next * 4099 + nidle;
    if (it == 0) {
      if (lane == 0) wd.start(p.timeout_ticks, seen);
    } else if (it % WATCH_EVERY == 0) {
      if (lane == 0) S.word = wd.expired(p.sched, p.timeout_ticks, seen, 40) ? 1 : 0;
      __builtin_amdgcn_wave_barrier();
      const int stop = S.word;
      __builtin_amdgcn_wave_barrier();
      if (stop) return;
    }
  }
}

// A worker's wait on its current mailbox slot (thread 0).  Returns false if the call was
// aborted.
ETC_DEV bool claim_mailbox(KArgs& p, Task& t, int slot) {
  long long* box = p.queue + 2 * blockIdx.x + slot;
  Watchdog wd;
  for (int it = 0;; ++it) {
    if (!slot_empty(q_load_relaxed(box))) {
      const long long v = q_load(box);  // acquire: the task's inputs are complete
      if ((v & 15) == K_EXIT) {
        // both slots empty for the next call
        q_store_relaxed(p.queue + 2 * blockIdx.x, 0);
        q_store_relaxed(p.queue + 2 * blockIdx.x + 1, 0);
        t.kind = K_NONE;
      } else {
        t = dec(v);
      }
      return true;
    }
    if (it == 0) wd.start(p.timeout_ticks, ev_load_relaxed(p.sched + W_QHEAD));
    else if (it % WATCH_EVERY == 0 &&
             wd.expired(p.sched, p.timeout_ticks, ev_load_relaxed(p.sched + W_QHEAD), 41))
      return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

template <typename TE>
__global__ __launch_bounds__(MNT) void moe_kernel(Args pk) {
  __shared__ Smem sm;
  // The task bodies are separate functions that take the arguments by reference; a
  // reference to the kernel argument itself would make every lane copy it to scratch,
  // so the workgroup copies it once into LDS and hands out references to that copy.
  __shared__ Args p_lds;
  const int tid = threadIdx.x;
  static_assert(sizeof(Args) % 4 == 0, "Args copies as words");
  {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(&pk);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&p_lds);
    for (int i = tid; i < (int)(sizeof(Args) / 4); i += MNT) dst[i] = src[i];
  }
  __syncthreads();
  KArgs& p = *(KArgs*)&p_lds;

  const bool tracing = (p.flags & ETC_FLAG_TRACE) != 0;
  uint64_t t_claim = 0, t_run = 0;
  if (tid == 0) {
    sm.lc.layer = -1;
    sm.scan_seen = 0u;
    sm.perm_seen = 0u;
    sm.next_ticket = -1;
    for (int l = 0; l <= MAXL; ++l) sm.lbase[l] = -1;
  }
  const bool dedicated = p.mode == ETC_SCHED_DEDICATED;
  int mslot = 0;  // dedicated mode: the worker's current mailbox slot (thread 0)
  if (dedicated && blockIdx.x != 0 && tid == 0) q_store_relaxed(p.queue + 2 * blockIdx.x, K_IDLE);
  if (dedicated && blockIdx.x == 0) {
    // the scheduler workgroup: wave 0 schedules, the other waves wait at the exit
    if (tid < WAVE) run_scheduler(p, sm);
  } else while (true) {
    // Thread 0 claims a task.  A gate/up, down or finalize task of a layer whose plan the
    // workgroup has not cached yet first has the whole workgroup copy it into LDS; then
    // (static mode) thread 0 waits for the task's inputs.
    if (tid == 0) {
      if (tracing) t_claim = now_ticks();
      Task t;
      t.kind = K_NONE; t.layer = 0; t.a = t.b = t.c = t.d = 0;
      const bool ok = (p.mode == ETC_SCHED_STATIC)    ? claim_static(p, t, sm)
                      : (p.mode == ETC_SCHED_DYNAMIC) ? claim_dynamic(p, t)
                                                      : claim_mailbox(p, t, mslot);
      if (!ok) t.kind = K_NONE;
      const bool gemm_or_f = t.kind == K_GU || t.kind == K_D || t.kind == K_F;
      sm.need_cache = (gemm_or_f && sm.lc.layer != t.layer) ? 1 : 0;
      if (!sm.need_cache && t.kind != K_NONE && p.mode == ETC_SCHED_STATIC &&
          !wait_deps(p, t, sm))
        t.kind = K_NONE;
      sm.task = t;
      if (tracing) t_run = now_ticks();
    }
    __syncthreads();
    Task t = sm.task;
    const bool load_cache = sm.need_cache != 0;
    __syncthreads();
    if (load_cache) {
      load_layer_cache(p, t.layer, sm);
      __syncthreads();
      if (tid == 0) {
        if (p.mode == ETC_SCHED_STATIC && !wait_deps(p, sm.task, sm)) sm.task.kind = K_NONE;
        if (tracing) t_run = now_ticks();
      }
      __syncthreads();
      t = sm.task;
      __syncthreads();
    }
    if (t.kind == K_NONE) break;
    KLayer& L = p.layer[t.layer];
    run_task<TE>(p, L, t, sm);
    if (tracing && tid == 0) trace_record(p, t, t_claim, t_run, now_ticks());
    // dedicated mode: the task's signals have gone out (run_task ends at a barrier after
    // them); the worker is idle again
    if (dedicated && tid == 0) {
      q_store_relaxed(p.queue + 2 * blockIdx.x + mslot, K_IDLE);
      mslot ^= 1;
    }
  }

  // the last workgroup out clears the event counters and control words
  wg_publish();
  if (tid == 0) sm.flag = (ev_add_relaxed(p.sched + W_EXIT, 1) == (int)gridDim.x - 1) ? 1 : 0;
  __syncthreads();
  // dedicated mode: empty mailboxes for the next call (an aborted call can leave task
  // words behind)
  if (sm.flag && dedicated)
    for (int i = tid; i < 2 * (int)gridDim.x; i += MNT) q_store_relaxed(p.queue + i, 0);
  if (sm.flag && !(p.flags & ETC_FLAG_KEEP_COUNTERS)) {
    for (int l = 0; l < p.L; ++l) {
      KLayer& L = p.layer[l];
      if (tid == 0) {
        ev_store_relaxed(L.ev_route, 0);
        ev_store_relaxed(L.ev_scan, 0);
        ev_store_relaxed(L.ev_perm, 0);
      }
      for (int i = tid; i < p.max_rt * p.n1; i += MNT) ev_store_relaxed(L.ev_gu + i, 0);
      for (int i = tid; i < p.n_rt_cap; i += MNT) {
        ev_store_relaxed(L.ev_comb + i, 0);
        ev_store_relaxed(L.ev_done + i, 0);
        ev_store_relaxed(L.ev_rq + i, 0);
      }
    }
    if (tid == 0) ev_store_relaxed(p.sched + W_TRACE_LAST, ev_load_relaxed(p.sched + W_TRACE));
    __syncthreads();
    for (int i = tid; i < W_NWORDS; i += MNT)
      if (i != W_STATUS && i != W_AUX && i != W_TRACE_LAST) ev_store_relaxed(p.sched + i, 0);
  }
}

// ------------------------------------------------------------------ host side

struct Layout {
  size_t sched, queue, trace, xq, hbuf, out_acc, ybuf, act, rpart, total;
  struct {
    size_t topk_idx, topk_w, lrank, hist, tile_off, counts, offsets, rt_base, sorted_assign, pos,
        plan, ev_route, ev_scan, ev_perm, ev_gu, ev_comb, ev_done, ev_rq;
  } l[MAXL];
  int n_rt, max_rt, n1, n2, queue_len;
};

inline Layout layout(int Tm, int H, int E, int K, int F, int nl, int es, bool ordered) {
  Layout Y;
  Y.n_rt = cdiv(Tm, BT);
  Y.max_rt = (Tm * K) / BM + (E < Tm * K ? E : Tm * K);
  Y.n1 = cdiv(F, BN1);
  Y.n2 = cdiv(H, BN2);
  host::Carve c;
  Y.sched = c.take(W_NWORDS * sizeof(int));
  for (int l = 0; l < nl; ++l) {  // counters first: the control region
    Y.l[l].ev_route = c.take(sizeof(int));
    Y.l[l].ev_scan = c.take(sizeof(int));
    Y.l[l].ev_perm = c.take(sizeof(int));
    Y.l[l].ev_gu = c.take((size_t)Y.max_rt * Y.n1 * sizeof(int));
    Y.l[l].ev_comb = c.take((size_t)Y.n_rt * sizeof(int));
    Y.l[l].ev_done = c.take((size_t)Y.n_rt * sizeof(int));
    Y.l[l].ev_rq = c.take((size_t)Y.n_rt * sizeof(int));
    Y.l[l].plan = c.take(PL_WORDS * sizeof(int));
  }
  const long per_layer = (long)Y.n_rt * (4 + RQ_MAX) + (long)Y.max_rt * Y.n1 + 2L * MAX_WORKERS +
                         (long)Y.max_rt * Y.n2 + 64;
  // + room for the one extra slot each worker draws before it sees the end
  Y.queue_len = (int)(Y.n_rt * RQ_MAX + per_layer * nl + 2 * MAX_WORKERS);  // dedicated: two slots per worker
  Y.queue = c.take((size_t)Y.queue_len * sizeof(long long));
  Y.trace = c.take((size_t)Y.queue_len * 32);  // one record per task at most
  for (int l = 0; l < nl; ++l) {
    const size_t pairs = (size_t)Tm * K;
    Y.l[l].topk_idx = c.take(pairs * 4);
    Y.l[l].topk_w = c.take(pairs * 4);
    Y.l[l].lrank = c.take(pairs * 4);
    Y.l[l].hist = c.take((size_t)Y.n_rt * E * 4);
    Y.l[l].tile_off = c.take((size_t)Y.n_rt * E * 4);
    Y.l[l].counts = c.take((size_t)E * 4);
    Y.l[l].offsets = c.take((size_t)(E + 1) * 4);
    Y.l[l].rt_base = c.take((size_t)(E + 1) * 4);
    Y.l[l].sorted_assign = c.take(pairs * 4);
    Y.l[l].pos = c.take(pairs * 4);
  }
  Y.xq = c.take((size_t)Tm * H * es);
  Y.hbuf = c.take((size_t)Tm * K * F * es);
  Y.out_acc = c.take((size_t)Tm * H * 4);
  Y.ybuf = ordered ? c.take((size_t)Tm * K * H * 4) : 0;
  Y.act = c.take((size_t)(nl > 1 ? nl - 1 : 0) * Tm * H * es);
  Y.rpart = c.take((size_t)NRQ_CAP * BT * E * sizeof(float));
  Y.total = c.off;
  return Y;
}

}  // namespace moe
}  // namespace etc

using namespace etc;

static int moe_occupancy(int dev, etc_dtype dt) {
  static int occ[host::MAX_DEVICES][2] = {{0}};
  if (occ[dev][dt] == 0) {
    int v = 0;
    hipError_t e = (dt == ETC_DTYPE_BF16)
                       ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, moe::moe_kernel<bf16>, moe::MNT, 0)
                       : hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, moe::moe_kernel<float>, moe::MNT, 0);
    if (e != hipSuccess || v < 1) v = 1;
    occ[dev][dt] = v;
  }
  return occ[dev][dt];
}

static etc_status moe_shape_check(int32_t Tm, int32_t H, int32_t E, int32_t K, int32_t F, int32_t nl,
                                  etc_dtype dt) {
  if (Tm < 0 || H < 1 || E < 1 || K < 1 || F < 1 || nl < 1) return ETC_ERR_INVALID_ARG;
  if (dt != ETC_DTYPE_F32 && dt != ETC_DTYPE_BF16) return ETC_ERR_INVALID_ARG;
  if (K > E) return ETC_ERR_INVALID_ARG;
  if (H % moe::H_ALIGN || F % moe::F_ALIGN || E > moe::MAXE || K > moe::MAXK || nl > moe::MAXL ||
      Tm > moe::MAX_TOKENS)
    return ETC_ERR_UNSUPPORTED;
  return ETC_OK;
}

ETC_API size_t etc_moe_workspace_size(int32_t max_tokens, int32_t hidden, int32_t experts, int32_t top_k,
                                      int32_t ffn, int32_t num_layers, etc_dtype dtype, etc_combine combine) {
  if (moe_shape_check(max_tokens, hidden, experts, top_k, ffn, num_layers, dtype) != ETC_OK) return 0;
  if (combine != ETC_COMBINE_ATOMIC && combine != ETC_COMBINE_ORDERED) return 0;
  const int es = dtype == ETC_DTYPE_BF16 ? 2 : 4;
  return moe::layout(max_tokens < 1 ? 1 : max_tokens, hidden, experts, top_k, ffn, num_layers, es,
                     combine == ETC_COMBINE_ORDERED)
      .total;
}

ETC_API etc_status etc_moe_workspace_layout(int32_t max_tokens, int32_t hidden, int32_t experts,
                                            int32_t top_k, int32_t ffn, int32_t num_layers, etc_dtype dtype,
                                            etc_combine combine, int32_t layer, int64_t* out) {
  const etc_status st = moe_shape_check(max_tokens, hidden, experts, top_k, ffn, num_layers, dtype);
  if (st != ETC_OK) return st;
  if (!out || layer < 0 || layer >= num_layers) return ETC_ERR_INVALID_ARG;
  const int es = dtype == ETC_DTYPE_BF16 ? 2 : 4;
  const moe::Layout Y = moe::layout(max_tokens < 1 ? 1 : max_tokens, hidden, experts, top_k, ffn, num_layers,
                                    es, combine == ETC_COMBINE_ORDERED);
  out[0] = (int64_t)Y.l[layer].ev_route;
  out[1] = (int64_t)Y.l[layer].ev_scan;
  out[2] = (int64_t)Y.l[layer].ev_gu;
  out[3] = (int64_t)Y.l[layer].ev_comb;
  out[4] = (int64_t)Y.l[layer].ev_done;
  out[5] = (int64_t)Y.l[layer].plan;
  out[6] = Y.max_rt;
  out[7] = Y.n1;
  out[8] = Y.n_rt;
  out[9] = moe::BT;
  out[10] = moe::BM;
  out[11] = moe::BN1;
  out[12] = moe::BN2;
  out[13] = (int64_t)Y.trace;
  out[14] = Y.queue_len;
  out[15] = (int64_t)Y.l[layer].ev_perm;
  out[16] = (int64_t)Y.l[layer].ev_rq;
  return ETC_OK;
}

ETC_API int32_t etc_default_workers(int32_t kind, etc_dtype dtype);

ETC_API etc_status etc_moe_layer(int32_t T, int32_t H, int32_t E, int32_t K, int32_t F, int32_t nl,
                                 etc_dtype dtype, float eps, const etc_moe_weights* weights, const void* x,
                                 void* out, void* layer_out, const etc_moe_routing* routing, void* workspace,
                                 size_t workspace_bytes, int32_t max_tokens, etc_sched_mode mode,
                                 etc_combine combine, uint32_t flags, int32_t workers, void* stream) {
  etc_status st = moe_shape_check(max_tokens, H, E, K, F, nl, dtype);
  if (st != ETC_OK) return st;
  if (T < 0 || T > max_tokens || !(eps >= 0.f)) return ETC_ERR_INVALID_ARG;
  if (mode != ETC_SCHED_STATIC && mode != ETC_SCHED_DYNAMIC && mode != ETC_SCHED_DEDICATED)
    return ETC_ERR_INVALID_ARG;
  if (mode == ETC_SCHED_DEDICATED && workers == 1) return ETC_ERR_INVALID_ARG;  // a scheduler and a worker
  // The dynamic (ready-queue) scheduler runs only when the caller opts in: a run of it on
  // MI355X did not terminate and its cause has not been identified.
  if (mode == ETC_SCHED_DYNAMIC && !(flags & ETC_FLAG_ALLOW_DYNAMIC)) return ETC_ERR_UNSUPPORTED;
  if (combine != ETC_COMBINE_ATOMIC && combine != ETC_COMBINE_ORDERED) return ETC_ERR_INVALID_ARG;
  if (T == 0) return ETC_OK;  // nothing to compute; empty tensors may have null pointers
  if (!weights || !x || !out) return ETC_ERR_INVALID_ARG;
  if (!host::aligned16(x) || !host::aligned16(out) || (layer_out && !host::aligned16(layer_out)))
    return ETC_ERR_INVALID_ARG;
  for (int l = 0; l < nl; ++l) {
    const etc_moe_weights& w = weights[l];
    if (!w.gamma || !w.w_router || !w.w_gate || !w.w_up || !w.w_down) return ETC_ERR_INVALID_ARG;
    if (!host::aligned16(w.w_router) || !host::aligned16(w.w_gate) || !host::aligned16(w.w_up) ||
        !host::aligned16(w.w_down))
      return ETC_ERR_INVALID_ARG;
  }
  if (routing) {
    const void* ps[4] = {routing->topk_idx, routing->topk_w, routing->expert_counts, routing->sorted_assign};
    for (const void* q : ps)
      if (q && (reinterpret_cast<uintptr_t>(q) & 3u)) return ETC_ERR_INVALID_ARG;
  }
  const int es = dtype == ETC_DTYPE_BF16 ? 2 : 4;
  const moe::Layout Y = moe::layout(max_tokens < 1 ? 1 : max_tokens, H, E, K, F, nl, es,
                                    combine == ETC_COMBINE_ORDERED);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < Y.total)
    return ETC_ERR_WORKSPACE;
  const int dev = host::current_gfx950_device();
  if (dev < 0) return ETC_ERR_NO_DEVICE;

  char* ws = static_cast<char*>(workspace);
  moe::Args p;
  memset(&p, 0, sizeof(p));
  p.T = T; p.H = H; p.E = E; p.K = K; p.F = F; p.L = nl;
  p.eps = eps;
  p.mode = mode;
  p.combine = combine;
  p.flags = flags;
  p.n_rt = cdiv(T, moe::BT);
  p.n_perm = p.n_rt <= moe::PERM_INLINE_RT ? 0 : p.n_rt;
  p.n1 = Y.n1;
  p.n2 = Y.n2;
  p.max_rt = Y.max_rt;
  p.queue_len = Y.queue_len;
  p.n_rt_cap = Y.n_rt;
  p.timeout_ticks = 500000000ull;  // 5 s without progress, on the 100 MHz real-time clock
  int grid = host::grid_size(workers, host::device_cus(dev), moe_occupancy(dev, dtype));
  if (grid > moe::MAX_WORKERS) grid = moe::MAX_WORKERS;
  // dedicated: a scheduler and at least one worker; the scheduler tracks up to 256 workers
  if (mode == ETC_SCHED_DEDICATED && grid > moe::DED_MAX_GRID) grid = moe::DED_MAX_GRID;
  if (mode == ETC_SCHED_DEDICATED && grid < 2) return ETC_ERR_INVALID_ARG;
  p.workers = grid;
  // router slices: when the routing tiles leave at least half the workers idle, each
  // tile's router is cut into Q slices along K (at most RQ_MAX, and NRQ_CAP slice records)
  {
    const int wk = mode == ETC_SCHED_DEDICATED ? grid - 1 : grid;
    int Q = 1;
    if (p.n_rt * 2 <= wk) Q = std::min(moe::RQ_MAX, std::min(wk / p.n_rt, moe::NRQ_CAP / p.n_rt));
    p.Q = Q < 1 ? 1 : Q;
    p.n_rq = p.n_rt * p.Q;
  }
  p.xq = ws + Y.xq;
  p.hbuf = ws + Y.hbuf;
  p.out_acc = reinterpret_cast<float*>(ws + Y.out_acc);
  p.ybuf = combine == ETC_COMBINE_ORDERED ? reinterpret_cast<float*>(ws + Y.ybuf) : nullptr;
  p.rpart = reinterpret_cast<float*>(ws + Y.rpart);
  p.queue = reinterpret_cast<long long*>(ws + Y.queue);
  p.trace = reinterpret_cast<unsigned long long*>(ws + Y.trace);
  p.trace_cap = Y.queue_len;
  p.sched = reinterpret_cast<int*>(ws + Y.sched);
  const size_t act_bytes = (size_t)T * H * es;
  for (int l = 0; l < nl; ++l) {
    moe::LayerArgs& L = p.layer[l];
    const etc_moe_weights& w = weights[l];
    L.gamma = w.gamma;
    L.w_router = w.w_router;
    L.bias = w.router_bias;
    L.w_gate = w.w_gate;
    L.w_up = w.w_up;
    L.w_down = w.w_down;
    L.in = (l == 0) ? x : p.layer[l - 1].out;
    if (l == nl - 1) L.out = out;
    else if (layer_out) L.out = static_cast<char*>(layer_out) + (size_t)l * act_bytes;
    else L.out = ws + Y.act + (size_t)l * max_tokens * H * es;
    const size_t pairs = (size_t)T * K;
    L.topk_idx = (routing && routing->topk_idx) ? routing->topk_idx + l * pairs
                                                : reinterpret_cast<int*>(ws + Y.l[l].topk_idx);
    L.topk_w = (routing && routing->topk_w) ? routing->topk_w + l * pairs
                                            : reinterpret_cast<float*>(ws + Y.l[l].topk_w);
    L.counts = (routing && routing->expert_counts) ? routing->expert_counts + (size_t)l * E
                                                   : reinterpret_cast<int*>(ws + Y.l[l].counts);
    L.sorted_assign = (routing && routing->sorted_assign) ? routing->sorted_assign + l * pairs
                                                          : reinterpret_cast<int*>(ws + Y.l[l].sorted_assign);
    L.lrank = reinterpret_cast<int*>(ws + Y.l[l].lrank);
    L.hist = reinterpret_cast<int*>(ws + Y.l[l].hist);
    L.tile_off = reinterpret_cast<int*>(ws + Y.l[l].tile_off);
    L.offsets = reinterpret_cast<int*>(ws + Y.l[l].offsets);
    L.rt_base = reinterpret_cast<int*>(ws + Y.l[l].rt_base);
    L.pos = reinterpret_cast<int*>(ws + Y.l[l].pos);
    L.plan = reinterpret_cast<int*>(ws + Y.l[l].plan);
    L.ev_route = reinterpret_cast<int*>(ws + Y.l[l].ev_route);
    L.ev_scan = reinterpret_cast<int*>(ws + Y.l[l].ev_scan);
    L.ev_perm = reinterpret_cast<int*>(ws + Y.l[l].ev_perm);
    L.ev_gu = reinterpret_cast<int*>(ws + Y.l[l].ev_gu);
    L.ev_comb = reinterpret_cast<int*>(ws + Y.l[l].ev_comb);
    L.ev_done = reinterpret_cast<int*>(ws + Y.l[l].ev_done);
    L.ev_rq = reinterpret_cast<int*>(ws + Y.l[l].ev_rq);
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == ETC_DTYPE_BF16)
    hipLaunchKernelGGL(moe::moe_kernel<bf16>, dim3(grid), dim3(moe::MNT), 0, s, p);
  else
    hipLaunchKernelGGL(moe::moe_kernel<float>, dim3(grid), dim3(moe::MNT), 0, s, p);
  return hipGetLastError() == hipSuccess ? ETC_OK : ETC_ERR_HIP;
}

int splitk_default_workers(int dev);

ETC_API int32_t etc_default_workers(int32_t kind, etc_dtype dtype) {
  const int dev = host::current_gfx950_device();
  if (dev < 0) return 0;
  if (kind == 1) return splitk_default_workers(dev);
  if (dtype != ETC_DTYPE_F32 && dtype != ETC_DTYPE_BF16) return 0;
  int g = host::device_cus(dev) * moe_occupancy(dev, dtype);
  return g > moe::MAX_WORKERS ? moe::MAX_WORKERS : g;
}
