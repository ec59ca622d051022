// Device helpers shared by the attention kernels (gfx950).
#pragma once

#include "relpos_device.hpp"

namespace relpos {
namespace attn {

constexpr int kD = 64;
constexpr int kTileKeys = 64;
constexpr int kTileRows = 4;
constexpr int kTileCols = 16;
constexpr int kKStride = kD + 8;  // halves per K/V row in LDS (144 B)
constexpr int kTileHalves = kTileKeys * kKStride;
constexpr int kSlots = 4;               // LDS ring depth (power of two)
// MFMA/VALU chunks of a pipeline step between scheduling fences.  8-wave
// workgroups (two waves per SIMD in one workgroup) run faster with the
// interleave fixed chunk by chunk (64x64: 75.9 -> 74.3 us), 4- and 2-wave
// workgroups with the compiler's own order inside the step (122.8 us against
// 126.5 us at 48x80).
template <int NW>
constexpr int chunks_per_fence() {
  return NW >= 8 ? 1 : 8;
}
constexpr float kGrowLimit = 32768.0f;  // 2^15: largest p allowed before m moves

typedef short __attribute__((ext_vector_type(4))) s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// gfx950 LDS transpose read.  Within each 16-lane group, lane i receives
// element (i % 4) of the 4-element row addressed by lane 4*k + i/4, k = 0..3.
__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Logical work index of this workgroup.  Workgroups are dispatched round-robin
// over the 8 XCDs; this maps the blocks that land on one XCD to a contiguous
// range of (head, query tile) work so that a head's K/V stays in one XCD's L2.
__device__ __forceinline__ int xcd_work_index(int G) {
  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int per = G >> 3, rem = G & 7;
  const int start = xcd * per + (xcd < rem ? xcd : rem);
  return start + (L >> 3);
}

struct TilePos {
  int kh, kw;
};

__device__ __forceinline__ TilePos next_tile(TilePos p, int H) {
  p.kh += kTileRows;
  if (p.kh >= H) {
    p.kh = 0;
    p.kw += kTileCols;
  }
  return p;
}

}  // namespace attn
}  // namespace relpos
