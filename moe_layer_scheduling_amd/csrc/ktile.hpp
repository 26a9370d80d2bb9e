// 128 x 256 output tile over K-contiguous operands on bf16 (or float32) MFMA, computed
// by a workgroup of 4 or 8 waves (NTH = 256 or 512 threads).
//
// Both operands are lists of rows whose K values are contiguous in memory: A rows are
// token activations (gathered through the MoE permutation), B rows are weight rows in
// nn.Linear layout.  The tile stages 384 rows (128 A rows, then 256 B rows) through
// LDS, 128 bytes of K per row per stage (64 bf16 or 32 float values, 48 KiB), in three
// rotating slots (144 KiB).
//
// Operands go from global memory straight into LDS (16 bytes per lane per copy, no
// staging registers).  Thread t makes LOADS = 384 * 8 / NTH copies per stage, copy i
// covering tile row t/8 + RSTEP*i (RSTEP = NTH/8).  For copy i, wave w fills rows
// 8w + RSTEP*i .. +7, one 1 KiB run of LDS: lane l lands at byte 16 l of the run, i.e.
// row 8w + RSTEP*i + l/8 at chunk position l % 8.  The LDS layout is swizzled (chunk c
// of row r sits at position c ^ ((r >> 1) & 7), see mfma.hpp), so lane l fetches the
// global chunk that belongs at its position: c = (l % 8) ^ ((4w + l/16) % 8).  rowp[i]
// is the address of thread t's row at k = 0 plus 16 c.  Every pointer must address a
// readable row: callers point rows past an expert's token count or past the matrix edge
// at a valid row and discard those output rows and columns.
//
// Pipeline: the copies run three stages ahead of the MFMAs, and each half-stage of
// MFMAs (one 16 x 16 x 32 step per fragment pair) overlaps the LDS reads of the next
// half-stage.  In step k the wave reads the second half of stage k, runs the MFMAs of
// the first half (read at the end of step k-1), then waits until only its copies of
// stage k+2 are outstanding and meets the workgroup at a barrier: stage k+1 has landed
// everywhere and every wave's reads of slot k mod 3 have completed, so the copies of
// stage k+3 go into that slot; the wave then reads the first half of stage k+1 and runs
// the MFMAs of the second half of stage k.  Copies past the last stage re-read the last
// stage into a slot no step reads, so every step issues the same copies and the wait
// count is a constant; the run drains them before returning.
//
// Waves form a 2 x WN grid (WN = NTH/128); wave (wm, wn) owns rows wm*64.. and columns
// wn*WCOLS.. (WCOLS = 256/WN) of the tile as 4 x NJ blocks of 16 x 16 (acc[i][j]):
// element r of acc[i][j] in lane l is row wm*64 + 16*i + 4*(l/16) + r, column
// wn*WCOLS + 16*j + (l % 16).  Row blocks past `rows` (the valid row count) skip their
// MFMAs: the count of live blocks is fixed per tile and selects one of five branch-free
// instances of the loop; with at most 64 valid rows a second set of instances also
// drops the copies of A rows 64..127.  Register arrays are indexed through static_for,
// so every index is a compile-time constant.
#pragma once

#include "common.hpp"
#include "mfma.hpp"

namespace etc {

template <typename TE, int NTH = NT>
struct KTile {
  static_assert(NTH == 256 || NTH == 512, "4 or 8 waves");
  static constexpr int BM = 128, BN = 256;
  static constexpr int ROWS = BM + BN;              // 384
  static constexpr int LOADS = ROWS * 8 / NTH;      // 16-byte copies per thread per stage: 12 or 6
  static constexpr int RSTEP = NTH / 8;             // rows between a thread's copies: 32 or 64
  static constexpr int ALOADS = BM / RSTEP;         // copies of A rows: 4 or 2
  static constexpr int STAGE_BYTES = ROWS * 128;    // 48 KiB
  static constexpr int NSTAGE = 3;
  static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;  // 144 KiB
  static constexpr int EPC = 16 / (int)sizeof(TE);  // elements per 16-byte chunk
  static constexpr int BK = 128 / (int)sizeof(TE);  // K per stage
  static constexpr int WN = NTH / 128;              // wave columns: 2 or 4 (2 wave rows)
  static constexpr int WCOLS = BN / WN;             // columns per wave: 128 or 64
  static constexpr int NJ = WCOLS / 16;             // 16-column blocks per wave: 8 or 4

  // The 16-byte chunk of its rows (within each 128-byte stage) that thread tid copies.
  ETC_DEV static int load_chunk(int tid) {
    const int l = tid & 63, w = tid >> 6;
    return (l & 7) ^ ((4 * w + (l >> 4)) & 7);
  }
  // Row of the tile that copy i of thread tid reads (i < ALOADS: A rows, else B rows
  // counted from the first B row).
  ETC_DEV static int load_row(int tid, int i) { return (tid >> 3) + RSTEP * i; }

  // rowp[i]: byte pointer of row load_row(tid, i) (minus BM for B rows) at k = 0, plus
  // load_chunk(tid) * 16.  klen: K values, a positive multiple of BK.  rows: valid A
  // rows (MFMAs of row blocks past it are skipped).  Wave w owns rows (w / WN) * 64 ..
  // +63 and columns (w % WN) * WCOLS .. of the tile; acc[i][j] holds the 16 x 16 block
  // (16 i, 16 j) of that region.
  ETC_DEV static void run(char* smem, const char* const (&rowp)[LOADS], int klen, int rows,
                          f32x4 (&acc)[4][NJ]) {
    static_for<4>([&](auto i) ETC_INLINE {
      static_for<NJ>([&](auto j) ETC_INLINE { acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f}; });
    });
    // the wave index is uniform across the wave: say so, so that per-wave choices become
    // scalar branches instead of exec-masked code
    const int wm = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) / WN;
    const int live = __builtin_amdgcn_readfirstlane(min(4, max(0, cdiv(rows - wm * 64, 16))));
    // At most 64 valid rows (decode batches, the last row tile of an expert): the copies
    // of A rows 64..127 are dropped as well as their MFMAs; those LDS rows are never read.
    if (rows <= 64) {
      switch (live) {
        case 4: pipeline<4, true>(smem, rowp, klen, acc); break;
        case 3: pipeline<3, true>(smem, rowp, klen, acc); break;
        case 2: pipeline<2, true>(smem, rowp, klen, acc); break;
        case 1: pipeline<1, true>(smem, rowp, klen, acc); break;
        default: pipeline<0, true>(smem, rowp, klen, acc); break;
      }
    } else {
      switch (live) {
        case 4: pipeline<4, false>(smem, rowp, klen, acc); break;
        case 3: pipeline<3, false>(smem, rowp, klen, acc); break;
        case 2: pipeline<2, false>(smem, rowp, klen, acc); break;
        case 1: pipeline<1, false>(smem, rowp, klen, acc); break;
        default: pipeline<0, false>(smem, rowp, klen, acc); break;
      }
    }
    // the last copies (re-reads past the last stage) land before LDS is reused
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    __syncthreads();
  }

 private:
  // Operand fragments of one K half-stage (32 bf16 / 16 float values) for this wave.
  struct Half {
    u32x4 a[4], b[NJ];
  };

  template <int LIVE, bool HALF>
  ETC_DEV static void pipeline(char* smem, const char* const (&rowp)[LOADS], int klen,
                               f32x4 (&acc)[4][NJ]) {
    // copies this thread issues per stage: with HALF, those of A rows 64..127 (copy
    // indices ALOADS/2 .. ALOADS-1) are dropped, and every wait counts NL
    constexpr int NL = LOADS - (HALF ? ALOADS / 2 : 0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w / WN, wn = w % WN;
    const int nk = klen / BK, last = nk - 1;
    const TE* tag = nullptr;
    // per-lane LDS byte offsets of the fragment rows within a slot, chunk kk * 4 + l/16
    int aoff[2][4], boff[2][NJ];
    static_for<2>([&](auto kk) ETC_INLINE {
      const int c = kk * 4 + (lane >> 4);
      static_for<4>([&](auto i) ETC_INLINE { aoff[kk][i] = swz(wm * 64 + i * 16 + (lane & 15), c); });
      static_for<NJ>([&](auto j) ETC_INLINE { boff[kk][j] = swz(BM + wn * WCOLS + j * 16 + (lane & 15), c); });
    });

    // The copies of a stage: their sources and slot are formed first (prep, before the
    // step's barrier), so that after the barrier only the copies themselves go out and
    // the MFMAs resume at once.
    auto prep = [&](int kt, const char* (&src)[LOADS], char*& slot) ETC_INLINE {
      const int st = min(kt, last);  // past the last stage: re-read it into an unread slot
      const size_t off = (size_t)st * 128;
      slot = smem + (kt % NSTAGE) * STAGE_BYTES + w * 8 * 128;
      static_for<LOADS>([&](auto i) ETC_INLINE { src[i] = rowp[i] + off; });
    };
    auto go = [&](const char* const (&src)[LOADS], char* slot) ETC_INLINE {
      static_for<LOADS>([&](auto i) ETC_INLINE {
        constexpr int I = decltype(i)::value;
        if constexpr (!(HALF && I >= ALOADS / 2 && I < ALOADS)) lds_dma16(src[i], slot + i * RSTEP * 128);
      });
    };
    auto issue = [&](int kt) ETC_INLINE {
      const char* src[LOADS];
      char* slot;
      prep(kt, src, slot);
      go(src, slot);
    };
    auto read = [&](Half& f, int kt, auto kk) ETC_INLINE {
      const char* base = smem + (kt % NSTAGE) * STAGE_BYTES;
      static_for<NJ>([&](auto j) ETC_INLINE { f.b[j] = *reinterpret_cast<const u32x4*>(base + boff[kk][j]); });
      static_for<LIVE>([&](auto i) ETC_INLINE { f.a[i] = *reinterpret_cast<const u32x4*>(base + aoff[kk][i]); });
    };
    auto mma = [&](const Half& f) ETC_INLINE {
      static_for<LIVE>([&](auto i) ETC_INLINE {
        static_for<NJ>([&](auto j) ETC_INLINE { mma16(acc[i][j], f.a[i], f.b[j], tag); });
      });
    };
    constexpr auto K0 = std::integral_constant<int, 0>{};
    constexpr auto K1 = std::integral_constant<int, 1>{};
    // Issue order within each half-step: the copies and LDS reads are spread over the
    // MFMAs (one memory instruction, then one MFMA) instead of going out in a burst that
    // stalls the wave on a full vector-memory queue before its first MFMA.
    constexpr int NMMA = LIVE * NJ, NRD = NJ + LIVE;
    auto interleave = [&](auto ncopy) ETC_INLINE {
      if constexpr (NMMA >= (int)decltype(ncopy)::value + NRD) {
        static_for<decltype(ncopy)::value>([&](auto) ETC_INLINE {
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // vector-memory read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        });
        static_for<NRD>([&](auto) ETC_INLINE {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        });
        __builtin_amdgcn_sched_group_barrier(0x008, NMMA - decltype(ncopy)::value - NRD, 0);
      }
    };

    Half h0, h1;
    issue(0);
    issue(1);
    issue(2);
    vm_wait_barrier<2 * NL>();  // stage 0 has landed
    read(h0, 0, K0);
    for (int kt = 0; kt < nk; ++kt) {
      // the first-half fragments were read before the previous MFMAs and have arrived;
      // waiting for them here leaves the compiler nothing outstanding that the MFMAs
      // below depend on, so it does not wait for the reads issued next
      lgkm_wait_all();
      read(h1, kt, K1);
      mma(h0);
      interleave(std::integral_constant<int, 0>{});
      // stage kt+1 has landed everywhere, and every wave has finished reading slot
      // kt mod 3 (its reads completed before the barrier): stage kt+3 may overwrite it
      const char* src[LOADS];
      char* slot;
      prep(kt + 3, src, slot);
      vm_wait_barrier<NL>();
      go(src, slot);
      read(h0, kt + 1, K0);  // past the last stage: unused reads of an unused slot
      mma(h1);
      interleave(std::integral_constant<int, NL>{});
    }
  }
};

// Small-M variant: BM_ (16 or 32) x 256 output tile for row tiles with at most BM_ valid
// rows (decode batches, cold experts).  Its A rows take 2 or 4 KiB of each stage instead
// of 16, so four stages fit where the 128-row tile keeps three (34 or 36 KiB each, at
// most 144 KiB): three stages of weight rows are in flight instead of two.  The same
// LDS arena thus takes one of two layouts, chosen per task from the row count.
//
// Copies: tile rows 0..BM_-1 are A rows, BM_..BM_+255 B rows; thread t's copy i covers
// tile row t/8 + 64 i (same lane-to-chunk mapping and swizzle as KTile).  Copies 0..3
// exist in every thread; copy 4 (rows 256..) only in the first BM_/8 waves, so those
// waves count five copies per stage and the others four.  The eight waves split the 256
// columns, 32 each: wave w owns columns 32 w .. 32 w + 31 of every row as BM_/16 x 2
// blocks of 16 x 16 (acc[i][j]: element r in lane l is row 16 i + 4 (l/16) + r, column
// 32 w + 16 j + (l % 16)).  Pipeline: as KTile's, four stages deep (stage k+4 goes into
// the slot of stage k once every wave has read it).
template <typename TE, int BM_, int NTH = 512>
struct KTileS {
  static_assert(NTH == 512 && (BM_ == 16 || BM_ == 32), "8 waves, 16 or 32 rows");
  static constexpr int BM = BM_, BN = 256;
  static constexpr int ROWS = BM + BN;              // 272 or 288
  static constexpr int RSTEP = NTH / 8;             // 64 tile rows per copy index
  static constexpr int FULL = BN / RSTEP;           // copies every thread makes: 4
  static constexpr int LOADS = FULL + 1;            // the last one in the first BM/8 waves
  static constexpr int XWAVES = BM / 8;             // waves that make the last copy
  static constexpr int STAGE_BYTES = ROWS * 128;
  static constexpr int NSTAGE = 4;
  static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;
  static constexpr int BK = 128 / (int)sizeof(TE);  // K per stage
  static constexpr int MI = BM / 16;                // 16-row blocks
  static constexpr int NJ = 2;                      // 16-column blocks per wave
  static constexpr int WCOLS = 32;
  static_assert(LDS_BYTES <= KTile<TE, NTH>::LDS_BYTES, "both layouts fit one arena");

  ETC_DEV static int load_chunk(int tid) { return KTile<TE, NTH>::load_chunk(tid); }
  // Tile row of copy i of thread tid (>= ROWS: the thread makes no such copy).
  ETC_DEV static int load_row(int tid, int i) { return (tid >> 3) + RSTEP * i; }

  // rowp[i]: byte pointer of tile row load_row(tid, i) at k = 0 plus load_chunk(tid) * 16
  // (any readable address where the thread makes no copy i).  klen: a positive multiple
  // of BK.
  ETC_DEV static void run(char* smem, const char* const (&rowp)[LOADS], int klen,
                          f32x4 (&acc)[MI][NJ]) {
    static_for<MI>([&](auto i) ETC_INLINE {
      static_for<NJ>([&](auto j) ETC_INLINE { acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f}; });
    });
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w < XWAVES) pipeline<LOADS>(smem, rowp, klen, acc);
    else pipeline<FULL>(smem, rowp, klen, acc);
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): the last copies landed
    __syncthreads();
  }

 private:
  struct Half {
    u32x4 a[MI], b[NJ];
  };

  template <int NL>
  ETC_DEV static void pipeline(char* smem, const char* const (&rowp)[LOADS], int klen,
                               f32x4 (&acc)[MI][NJ]) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nk = klen / BK, last = nk - 1;
    const TE* tag = nullptr;
    int aoff[2][MI], boff[2][NJ];
    static_for<2>([&](auto kk) ETC_INLINE {
      const int c = kk * 4 + (lane >> 4);
      static_for<MI>([&](auto i) ETC_INLINE { aoff[kk][i] = swz(i * 16 + (lane & 15), c); });
      static_for<NJ>([&](auto j) ETC_INLINE { boff[kk][j] = swz(BM + w * WCOLS + j * 16 + (lane & 15), c); });
    });
    auto prep = [&](int kt, const char* (&src)[NL], char*& slot) ETC_INLINE {
      const size_t off = (size_t)min(kt, last) * 128;  // past the last stage: a re-read
      slot = smem + (kt % NSTAGE) * STAGE_BYTES + w * 8 * 128;
      static_for<NL>([&](auto i) ETC_INLINE { src[i] = rowp[i] + off; });
    };
    auto go = [&](const char* const (&src)[NL], char* slot) ETC_INLINE {
      static_for<NL>([&](auto i) ETC_INLINE { lds_dma16(src[i], slot + i * RSTEP * 128); });
    };
    auto issue = [&](int kt) ETC_INLINE {
      const char* src[NL];
      char* slot;
      prep(kt, src, slot);
      go(src, slot);
    };
    auto read = [&](Half& f, int kt, auto kk) ETC_INLINE {
      const char* base = smem + (kt % NSTAGE) * STAGE_BYTES;
      static_for<NJ>([&](auto j) ETC_INLINE { f.b[j] = *reinterpret_cast<const u32x4*>(base + boff[kk][j]); });
      static_for<MI>([&](auto i) ETC_INLINE { f.a[i] = *reinterpret_cast<const u32x4*>(base + aoff[kk][i]); });
    };
    auto mma = [&](const Half& f) ETC_INLINE {
      static_for<MI>([&](auto i) ETC_INLINE {
        static_for<NJ>([&](auto j) ETC_INLINE { mma16(acc[i][j], f.a[i], f.b[j], tag); });
      });
    };
    constexpr auto K0 = std::integral_constant<int, 0>{};
    constexpr auto K1 = std::integral_constant<int, 1>{};
    Half h0, h1;
    static_for<NSTAGE>([&](auto k) ETC_INLINE { issue(decltype(k)::value); });
    vm_wait_barrier<(NSTAGE - 1) * NL>();  // stage 0 has landed
    read(h0, 0, K0);
    for (int kt = 0; kt < nk; ++kt) {
      lgkm_wait_all();
      read(h1, kt, K1);
      mma(h0);
      // stage kt+1 has landed everywhere and every wave has read slot kt mod 4 (its
      // reads completed before the barrier): stage kt+4 may overwrite it
      const char* src[NL];
      char* slot;
      prep(kt + NSTAGE, src, slot);
      vm_wait_barrier<(NSTAGE - 2) * NL>();
      go(src, slot);
      read(h0, kt + 1, K0);  // past the last stage: unused reads of an unused slot
      mma(h1);
    }
  }
};

}  // namespace etc
