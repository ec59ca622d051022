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
  // Configuration kAttnSplitConfig only: a scratch workspace of
  // attn_split_workspace_bytes(BH, H*W, split_ctas) bytes and the device's
  // CU count.
  void* ws = nullptr;
  int split_ctas = 0;
  // launch_attn_fused only: the tables rel_pos_h [2H-1, 64] and rel_pos_w
  // [2W-1, 64] in the input dtype (rel_h and rel_w are then unused).
  const void* th = nullptr;
  const void* tw = nullptr;
  // LDS bytes a workgroup may use on this device (0: only the K/V ring is
  // used; more lets 8-wave launches keep rel_h rows in LDS).
  int lds_limit = 0;
};

hipError_t launch_build(const BuildArgs& a, hipStream_t stream);

// Attention launch configurations:
//   0, 1: 32 queries per wave, 8 or 4 waves per workgroup, one workgroup
//         per unit of 32*waves queries
//   3: 16 queries per wave, 4 waves per workgroup (64 queries)
//   5: configuration 0 with the key range split over a persistent grid of
//      split_ctas workgroups (needs the workspace)
//   6: 12 waves x 32 queries, even and odd key tiles on separate waves
//      (relpos_attn12.hip)
constexpr int kAttnSplitConfig = 5;
// Fixed cost of one segment of the split launch (pipeline start and drain,
// the piece store, cold K/V tiles at the cut), in key-tile steps, and the
// same for the fused launch, whose segments also compute their bias rows.
// Set by measurement: on the 64x64, 12-head workload (T = 64, k = 3) these
// put the cut at s = 51 and s = 54, the fastest of a sweep of s.
constexpr int kSplitSegmentTiles = 6;
// Fixed cost of splitting a last round beyond its segments (the merge launch),
// in tile steps.  Checked on whole steps (relpos_build, then the attention
// call): at 64x64 the split step is 88.0 us against 93.2 us unsplit, although
// alone the unsplit call is 1 us faster; 48x80 is within 1% either way and
// 96x96 favours the split.
constexpr int kMergeTiles = 4;
constexpr int kFusedPrologueTiles = 12;
// Per-tile cost of the persistent split grid against an unsplit 8-wave
// launch, beyond its segments and merge (per-segment staging of rel_h rows,
// the piece stores; measured: 64x64 split 78.3-78.9 us against 75.4-75.6 us
// unsplit where the tile model alone predicts 0.953 of it; 96x96 0.954 of
// unsplit against a predicted 0.914).
constexpr double kSplitGridFactor = 1.06;

// Last-round split of configuration kAttnSplitConfig.  With `units` query
// units of T key tiles on P workgroups (one per CU), `rounds` = units / P full
// rounds run unsplit; the rest = units % P units of the last round are cut at
// key tile s: their heads [0, s) run on `rest` workgroups and their tails
// [s, T) on the idle ones, k tails each, every head and every tail starting
// at the same tile so a head's K/V tiles are shared in L2.  s = T*k/(k+1)
// balances the two (k = ceil(rest / (P - rest))).  s == T means no tails
// (T < 2): the last round then runs unsplit too.  With a fixed cost of `pro`
// tiles per segment, s = (T*k + (k-1)*pro) / (k+1) balances s + pro against
// k*(T - s + pro).
struct SplitPlan {
  int rounds, rest, k, s;
};
inline SplitPlan split_plan(int64_t units, int T, int P, int pro = 0) {
  SplitPlan p{};
  p.rounds = static_cast<int>(units / P);
  p.rest = static_cast<int>(units - static_cast<int64_t>(p.rounds) * P);
  if (p.rest == 0) return p;
  p.k = (p.rest + (P - p.rest) - 1) / (P - p.rest);
  p.s = static_cast<int>((static_cast<int64_t>(T) * p.k + static_cast<int64_t>(p.k - 1) * pro + (p.k + 1) / 2) /
                         (p.k + 1));
  if (p.s < 1) p.s = 1;
  if (p.s > T - 1) p.s = T < 2 ? T : T - 1;
  return p;
}
size_t attn_split_workspace_bytes(int64_t BH, int64_t N, int ctas);
// The fused path: configuration kAttnSplitConfig's kernel with the bias
// computed in the kernel.  Workspace: the split pieces, then one slot of bias
// rows per workgroup (split_ctas workgroups).
size_t attn_fused_workspace_bytes(int H, int W, int ctas);
hipError_t launch_attn_fused(const AttnArgs& a, hipStream_t stream);
// LDS bytes the attention kernel needs in configuration `cfg`.
size_t attn_lds_bytes(int cfg, int H, int W);
hipError_t launch_attn_fwd(const AttnArgs& a, int cfg, hipStream_t stream);

// The 12-wave kernel (relpos_attn12.hip): 6 query blocks x even/odd key
// tiles per workgroup, three waves per SIMD, no workspace.  Needs at least 6
// query blocks of 32 per head (attn12_fits).
constexpr int kAttn12Config = 6;
size_t attn12_lds_bytes();
bool attn12_fits(int H, int W);
// Whether the kernel runs P.V in bf16 for bf16 inputs on this grid.
bool attn12_bf16_p(int H, int W);
hipError_t launch_attn12(const AttnArgs& a, hipStream_t stream);
// The fused call on the 12-wave kernel: a persistent grid of min(units,
// split_ctas) workgroups, each computing its blocks' bias rows into its slot
// of ws (kBlocks12 * 32 * (H + W) floats) before the key loop.  For bf16
// inputs with W % 32 == 0, H % 4 == 0 and the kernel's bf16-P grids.
bool attn_fused12_ok(int H, int W, bool bf16);
// Grids whose fused units keep their bias rows in LDS (H, W <= 64).
bool attn_fused12_lds_bias(int H, int W);
size_t attn_fused12_workspace_bytes(int64_t BH, int H, int W, int ctas);
hipError_t launch_attn_fused12(const AttnArgs& a, hipStream_t stream);

// The 16-query-per-wave kernel (relpos_attn16.hip).
size_t attn16_lds_bytes();
hipError_t launch_attn16(const AttnArgs& a, hipStream_t stream);
// The fused call on the 16-query kernel, for grids with H, W <= 32 and at
// most 4 key tiles: each workgroup computes its 64 queries' bias rows into
// LDS (attn_fused16_lds_bytes) from the tables th / tw; no workspace.
bool attn_fused16_ok(int H, int W);
size_t attn_fused16_lds_bytes(int H, int W);
hipError_t launch_attn_fused16(const AttnArgs& a, hipStream_t stream);

}  // namespace relpos
