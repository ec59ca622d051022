// Host-side launch interface between the C ABI (relpos_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace relpos {

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

struct BuildArgs {
  const void* q;
  const void* rel_pos_h;
  const void* rel_pos_w;
  float* rel_h;
  float* rel_w;
  int BH, H, W;
  bool bf16;
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* rel_h;
  const float* rel_w;
  void* out;
  int BH, H, W;
  float scale;
  bool bf16;
  bool out_f32;
};

hipError_t launch_build(const BuildArgs& a, hipStream_t stream);

// Attention launch configurations:
//   0, 1, 2: 32 queries per wave, 8, 4 or 2 waves per workgroup (default: 0)
//   3: 16 queries per wave, 4 waves per workgroup (64 queries)
//   4: 16 queries per wave, 8 waves per workgroup (128 queries)
int attn_num_configs();
// LDS bytes the attention kernel needs in configuration `cfg`.
size_t attn_lds_bytes(int cfg, int H, int W);
hipError_t launch_attn_fwd(const AttnArgs& a, int cfg, hipStream_t stream);

// The 16-query-per-wave kernel (relpos_attn16.hip).
size_t attn16_lds_bytes();
hipError_t launch_attn16(const AttnArgs& a, int nw, hipStream_t stream);

}  // namespace relpos
