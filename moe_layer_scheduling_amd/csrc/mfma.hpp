// MFMA wrappers and LDS fragment helpers for gfx950.
//
// v_mfma_f32_16x16x32_bf16 multiplies a 16x32 A block by a 32x16 B block into a
// 16x16 float32 block.  Lane l supplies row (l % 16) of A and column (l % 16) of B,
// each as 8 consecutive k values; lane group g = l / 16 covers k = 8g .. 8g+7.
// The result element (row 4*(l/16) + r, column l % 16) sits in lane l, slot r.
// The float32 variant v_mfma_f32_16x16x4_f32 takes one k value per lane (k = l / 16);
// four of them consume a 16-byte chunk of 4 floats per lane, the q-th issue using the
// q-th float, so both element types consume one 16-byte chunk per lane per step and
// A and B always pair the same k.
#pragma once

#include "common.hpp"

namespace etc {

ETC_DEV void mma16(f32x4& c, const uint4& a, const uint4& b, const bf16*) {
  bf16x8 av = __builtin_bit_cast(bf16x8, a);
  bf16x8 bv = __builtin_bit_cast(bf16x8, b);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

ETC_DEV void mma16(f32x4& c, const u32x4& a, const u32x4& b, const bf16*) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                              c, 0, 0, 0);
}

ETC_DEV void mma16(f32x4& c, const u32x4& a, const u32x4& b, const float*) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
}

ETC_DEV void mma16(f32x4& c, const uint4& a, const uint4& b, const float*) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
}

// LDS tile of K-contiguous rows, 128 bytes (8 chunks of 16 B) per row per stage.
// Chunk c of row r is stored at chunk position c ^ ((r >> 1) & 7): the 16 lanes of a
// quarter-wave that read one chunk of 16 consecutive rows then hit 16 distinct
// 4-bank groups.
ETC_DEV int swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

ETC_DEV uint4 lds_chunk(const char* base, int row, int chunk) {
  return *reinterpret_cast<const uint4*>(base + swz(row, chunk));
}
// The same read as a native vector.  Reads of this type are what the compiler can tell
// apart from direct global-to-LDS copies still in flight, so it does not make them wait
// for every outstanding copy (the tile pipeline orders them with explicit waits).
ETC_DEV u32x4 lds_chunk_v(const char* base, int row, int chunk) {
  return *reinterpret_cast<const u32x4*>(base + swz(row, chunk));
}
ETC_DEV void lds_put_chunk(char* base, int row, int chunk, const uint4& v) {
  *reinterpret_cast<uint4*>(base + swz(row, chunk)) = v;
}

ETC_DEV uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

}  // namespace etc
