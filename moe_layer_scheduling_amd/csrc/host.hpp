// Host-side helpers of the C ABI: device checks, workspace carving, launch sizing.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/etc_moe.h"

#define ETC_API extern "C" __attribute__((visibility("default")))

namespace etc {
namespace host {

constexpr int MAX_DEVICES = 64;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Current device if it is a gfx950 part, else -1.  The check runs once per device.
int current_gfx950_device();

// Compute units of `dev` (cached).
int device_cus(int dev);

// Bump allocator over a workspace: offsets are 256-byte aligned.
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  }
};

// Persistent grid size: min(requested or all resident slots, resident slots).
inline int grid_size(int requested, int cus, int occupancy) {
  int slots = cus * (occupancy > 0 ? occupancy : 1);
  if (requested <= 0 || requested > slots) return slots;
  return requested;
}

}  // namespace host
}  // namespace etc
