// 128 x 128 output tile over K-contiguous operands on bf16 (or float32) MFMA.
//
// Both operands are lists of rows whose K values are contiguous in memory: A rows are
// token activations (gathered through the MoE permutation), B rows are weight rows in
// nn.Linear layout.  Each of the 256 threads always loads 16-byte chunk (tid % 8) of
// rows tid/8 + 32*i, i = 0..7 (i < 4: A rows, i >= 4: B rows), so a thread needs just
// 8 row pointers; a null pointer stands for a row of zeros (rows past an expert's
// token count).  A stage holds 128 bytes of each of the 256 rows (64 bf16 or 32 float
// values of K) in LDS, swizzled per mfma.hpp; two stages alternate: the global loads
// of stage kt+1 are in flight while the MFMAs consume stage kt.
//
// Waves form a 2 x 2 grid; wave (wm, wn) owns rows wm*64.. and columns wn*64.. of the
// tile as 4 x 4 blocks of 16 x 16 (acc[i][j]): element r of acc[i][j] in lane l is
// row wm*64 + 16*i + 4*(l/16) + r, column wn*64 + 16*j + (l % 16).
#pragma once

#include "common.hpp"
#include "mfma.hpp"

namespace etc {

template <typename TE>
struct KTile {
  static constexpr int ROWS = 256;                  // 128 A rows + 128 B rows
  static constexpr int STAGE_BYTES = ROWS * 128;    // 32 KiB
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES; // 64 KiB
  static constexpr int EPC = 16 / (int)sizeof(TE);  // elements per 16-byte chunk
  static constexpr int BK = 128 / (int)sizeof(TE);  // K per stage

  // rowp[i]: byte pointer of row (tid/8 + 32*i) at k = 0 (null = zeros).  klen: number
  // of K values (a multiple of EPC).  smem: LDS_BYTES, 16-byte aligned.
  ETC_DEV static void run(char* smem, const char* const (&rowp)[8], int klen, f32x4 (&acc)[4][4]) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int chunk = tid & 7, row0 = tid >> 3;
    const int nk = cdiv(klen, BK);
    const TE* tag = nullptr;

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 st[8];
    auto gload = [&](int kt) {
      const int k = kt * BK + chunk * EPC;
      const bool inb = k < klen;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        st[i] = (inb && rowp[i]) ? *reinterpret_cast<const uint4*>(rowp[i] + (size_t)kt * 128 + chunk * 16)
                                 : zero4();
    };
    auto sstore = [&](int buf) {
      char* base = smem + buf * STAGE_BYTES;
#pragma unroll
      for (int i = 0; i < 8; ++i) lds_put_chunk(base, row0 + 32 * i, chunk, st[i]);
    };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) gload(kt + 1);
      const char* base = smem + (kt & 1) * STAGE_BYTES;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint4 a[4], b[4];
        const int c = kk * 4 + (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = lds_chunk(base, wm * 64 + i * 16 + (lane & 15), c);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = lds_chunk(base, 128 + wn * 64 + j * 16 + (lane & 15), c);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) mma16(acc[i][j], a[i], b[j], tag);
      }
      if (kt + 1 < nk) sstore((kt + 1) & 1);
      __syncthreads();
    }
  }
};

}  // namespace etc
