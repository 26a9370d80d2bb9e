// 128 x 256 output tile over K-contiguous operands on bf16 (or float32) MFMA.
//
// Both operands are lists of rows whose K values are contiguous in memory: A rows are
// token activations (gathered through the MoE permutation), B rows are weight rows in
// nn.Linear layout.  Each of the 256 threads always loads 16-byte chunk (tid % 8) of
// rows tid/8 + 32*i, i = 0..11 (i < 4: A rows 0..127, i >= 4: B rows 0..255), so a
// thread needs 12 row pointers; a null pointer stands for a row of zeros (rows past an
// expert's token count, weight rows past the matrix edge).
//
// A stage holds 128 bytes of K (64 bf16 or 32 float values) of each of the 384 rows in
// LDS (48 KiB, swizzled per mfma.hpp).  Three stages rotate through LDS and two sets of
// staging registers hold the stages in flight, so the global loads for stage k+2 are
// issued while the MFMAs consume stage k: two stages of compute (~0.85 us at the MFMA
// rate) cover the load latency.  One barrier per stage: the stage written at the end
// of step k was last read at step k-2.
//
// Waves form a 2 x 2 grid; wave (wm, wn) owns rows wm*64.. and columns wn*128.. of the
// tile as 4 x 8 blocks of 16 x 16 (acc[i][j]): element r of acc[i][j] in lane l is
// row wm*64 + 16*i + 4*(l/16) + r, column wn*128 + 16*j + (l % 16).  Row blocks past
// `rows` (the valid row count) skip their MFMAs.
#pragma once

#include "common.hpp"
#include "mfma.hpp"

namespace etc {

template <typename TE>
struct KTile {
  static constexpr int BM = 128, BN = 256;
  static constexpr int ROWS = BM + BN;              // 384
  static constexpr int LOADS = ROWS * 8 / NT;       // 16-byte chunks per thread per stage: 12
  static constexpr int STAGE_BYTES = ROWS * 128;    // 48 KiB
  static constexpr int NSTAGE = 3;
  static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;  // 144 KiB
  static constexpr int EPC = 16 / (int)sizeof(TE);  // elements per 16-byte chunk
  static constexpr int BK = 128 / (int)sizeof(TE);  // K per stage

  // rowp[i]: byte pointer of row (tid/8 + 32*i) at k = 0 (null = zeros).  klen: K values
  // (a multiple of EPC).  rows: valid A rows (MFMAs of row blocks past it are skipped).
  ETC_DEV static void run(char* smem, const char* const (&rowp)[LOADS], int klen, int rows,
                          f32x4 (&acc)[4][8]) {
    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index is uniform across the wave: say so, so that per-wave choices become
    // scalar branches instead of exec-masked code
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int chunk = tid & 7, row0 = tid >> 3;
    const int nk = cdiv(klen, BK);
    const TE* tag = nullptr;
    // row blocks of this wave that hold at least one valid row
    const int live_blocks = __builtin_amdgcn_readfirstlane(min(4, max(0, cdiv(rows - wm * 64, 16))));

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 sa[LOADS], sb[LOADS];
    auto gload = [&](uint4 (&st)[LOADS], int kt) {
      const int k = kt * BK + chunk * EPC;
      const bool inb = k < klen;
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        st[i] = (inb && rowp[i]) ? *reinterpret_cast<const uint4*>(rowp[i] + (size_t)kt * 128 + chunk * 16)
                                 : zero4();
    };
    auto sstore = [&](const uint4 (&st)[LOADS], int kt) {
      char* base = smem + (kt % NSTAGE) * STAGE_BYTES;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) lds_put_chunk(base, row0 + 32 * i, chunk, st[i]);
    };
    auto compute = [&](int kt) {
      const char* base = smem + (kt % NSTAGE) * STAGE_BYTES;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int c = kk * 4 + (lane >> 4);
        uint4 a[4], b[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = lds_chunk(base, BM + wn * 128 + j * 16 + (lane & 15), c);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = lds_chunk(base, wm * 64 + i * 16 + (lane & 15), c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < live_blocks) {
#pragma unroll
            for (int j = 0; j < 8; ++j) mma16(acc[i][j], a[i], b[j], tag);
          }
        }
      }
    };
    // step kt: prefetch kt+2 into `ld` (whose stage kt is already in LDS), consume kt,
    // move stage kt+1 from `st` into LDS
    auto step = [&](int kt, uint4 (&ld)[LOADS], const uint4 (&st)[LOADS]) {
      if (kt + 2 < nk) gload(ld, kt + 2);
      compute(kt);
      if (kt + 1 < nk) sstore(st, kt + 1);
      __syncthreads();
    };

    gload(sa, 0);
    if (nk > 1) gload(sb, 1);
    sstore(sa, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      step(kt, sa, sb);
      if (kt + 1 < nk) step(kt + 1, sb, sa);
    }
  }
};

}  // namespace etc
