// 128 x 256 output tile over K-contiguous operands on bf16 (or float32) MFMA.
//
// Both operands are lists of rows whose K values are contiguous in memory: A rows are
// token activations (gathered through the MoE permutation), B rows are weight rows in
// nn.Linear layout.  The tile stages 384 rows (i < 4: A rows 32i..32i+31, i >= 4: B rows
// 32(i-4)..) through LDS, 128 bytes of K per row per stage (64 bf16 or 32 float values,
// 48 KiB), in three rotating slots (144 KiB).
//
// Operands go from global memory straight into LDS (16 bytes per lane per copy, no
// staging registers).  For copy i, wave w fills rows 8w + 32i .. +7 of the slot, one
// 1 KiB run of LDS: lane l lands at byte 16 l of the run, i.e. row 8w + 32i + l/8 at
// chunk position l % 8.  The LDS layout is swizzled (chunk c of row r sits at position
// c ^ ((r >> 1) & 7), see mfma.hpp), so lane l fetches the global chunk that belongs at
// its position: c = (l % 8) ^ ((4w + l/16) % 8).  Thread t therefore reads rows
// t/8 + 32i at chunk c(t); rowp[i] is that row's address at k = 0.  Every pointer must
// address a readable row: callers point rows past an expert's token count or past the
// matrix edge at a valid row and discard those output rows and columns.
//
// Pipeline: the copies for stage k+2 are issued right after the barrier of step k and
// run under the MFMAs of stages k and k+1.  Before the barrier of step k each thread
// waits until only its 12 copies of stage k+1 are outstanding (its part of stage k has
// landed); after the barrier every wave's part has landed and every wave has finished
// reading slot (k-1) mod 3, the slot stage k+2 then overwrites.  Past the last stage
// the copies re-read the last stage into a slot no step reads, so every step issues the
// same 12 copies and the wait count is a constant; the run drains them before returning.
//
// Waves form a 2 x 2 grid; wave (wm, wn) owns rows wm*64.. and columns wn*128.. of the
// tile as 4 x 8 blocks of 16 x 16 (acc[i][j]): element r of acc[i][j] in lane l is
// row wm*64 + 16*i + 4*(l/16) + r, column wn*128 + 16*j + (l % 16).  Row blocks past
// `rows` (the valid row count) skip their MFMAs: the count of live blocks is fixed per
// tile and selects one of five branch-free instances of the loop.  Register arrays are
// indexed through static_for, so every index is a compile-time constant.
#pragma once

#include <utility>

#include "common.hpp"
#include "mfma.hpp"

namespace etc {

#define ETC_INLINE __attribute__((always_inline))

template <typename F, int... I>
ETC_DEV void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
ETC_DEV void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <typename TE>
struct KTile {
  static constexpr int BM = 128, BN = 256;
  static constexpr int ROWS = BM + BN;              // 384
  static constexpr int LOADS = ROWS * 8 / NT;       // 16-byte copies per thread per stage: 12
  static constexpr int STAGE_BYTES = ROWS * 128;    // 48 KiB
  static constexpr int NSTAGE = 3;
  static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;  // 144 KiB
  static constexpr int EPC = 16 / (int)sizeof(TE);  // elements per 16-byte chunk
  static constexpr int BK = 128 / (int)sizeof(TE);  // K per stage

  // The 16-byte chunk of its rows (within each 128-byte stage) that thread tid copies.
  ETC_DEV static int load_chunk(int tid) {
    const int l = tid & 63, w = tid >> 6;
    return (l & 7) ^ ((4 * w + (l >> 4)) & 7);
  }

  // rowp[i]: byte pointer of row (tid/8 + 32*i) at k = 0.  klen: K values, a positive
  // multiple of BK.  rows: valid A rows (MFMAs of row blocks past it are skipped).
  ETC_DEV static void run(char* smem, const char* const (&rowp)[LOADS], int klen, int rows,
                          f32x4 (&acc)[4][8]) {
    static_for<4>([&](auto i) ETC_INLINE {
      static_for<8>([&](auto j) ETC_INLINE { acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f}; });
    });
    // the wave index is uniform across the wave: say so, so that per-wave choices become
    // scalar branches instead of exec-masked code
    const int wm = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >> 1;
    const int live = __builtin_amdgcn_readfirstlane(min(4, max(0, cdiv(rows - wm * 64, 16))));
    switch (live) {
      case 4: pipeline<4>(smem, rowp, klen, acc); break;
      case 3: pipeline<3>(smem, rowp, klen, acc); break;
      case 2: pipeline<2>(smem, rowp, klen, acc); break;
      case 1: pipeline<1>(smem, rowp, klen, acc); break;
      default: pipeline<0>(smem, rowp, klen, acc); break;
    }
    // the last copies (re-reads past the last stage) land before LDS is reused
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
    __syncthreads();
  }

 private:
  template <int LIVE>
  ETC_DEV static void pipeline(char* smem, const char* const (&rowp)[LOADS], int klen,
                               f32x4 (&acc)[4][8]) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int nk = klen / BK, last = nk - 1;
    const TE* tag = nullptr;

    auto issue = [&](int kt) ETC_INLINE {
      const size_t off = (size_t)kt * 128;
      char* slot = smem + (kt % NSTAGE) * STAGE_BYTES + w * 8 * 128;
      static_for<LOADS>([&](auto i) ETC_INLINE { lds_dma16(rowp[i] + off, slot + i * 32 * 128); });
    };
    auto compute = [&](int kt) ETC_INLINE {
      const char* base = smem + (kt % NSTAGE) * STAGE_BYTES;
      static_for<2>([&](auto kk) ETC_INLINE {
        const int c = kk * 4 + (lane >> 4);
        u32x4 a[4], b[8];
        static_for<8>([&](auto j) ETC_INLINE {
          b[j] = lds_chunk_v(base, BM + wn * 128 + j * 16 + (lane & 15), c);
        });
        static_for<LIVE>([&](auto i) ETC_INLINE {
          a[i] = lds_chunk_v(base, wm * 64 + i * 16 + (lane & 15), c);
        });
        static_for<LIVE>([&](auto i) ETC_INLINE {
          static_for<8>([&](auto j) ETC_INLINE { mma16(acc[i][j], a[i], b[j], tag); });
        });
      });
    };

    issue(0);
    issue(min(1, last));
    for (int kt = 0; kt < nk; ++kt) {
      vm_wait_barrier<LOADS>();
      issue(min(kt + 2, last));
      compute(kt);
    }
  }
};

}  // namespace etc
