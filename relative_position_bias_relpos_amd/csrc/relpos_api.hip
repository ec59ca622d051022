// C ABI of librelpos: argument validation, operand checks and kernel launch.
// Declared and documented in include/relpos.h.
#include "../../include/relpos.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "relpos_kernels.hpp"

namespace {

constexpr int64_t kMaxSide = 4096;
constexpr int64_t kMaxTokens = int64_t(1) << 24;
constexpr int64_t kMaxHeads = 65535;  // B*heads maps to grid.y
constexpr int kMaxDevices = 64;

struct Operand {
  const void* p;
  size_t bytes;
};

bool overlaps(const Operand& a, const Operand& b) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

relpos_status check_dims(int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D, int64_t* BH) {
  if (D != 64) return RELPOS_E_SHAPE;
  if (B < 0 || heads < 0) return RELPOS_E_SHAPE;
  if (H < 1 || W < 1 || H > kMaxSide || W > kMaxSide || H * W > kMaxTokens) return RELPOS_E_SHAPE;
  if (heads != 0 && B > kMaxHeads / heads) return RELPOS_E_SHAPE;
  *BH = B * heads;
  return RELPOS_OK;
}

bool is_half(relpos_dtype t) { return t == RELPOS_BF16 || t == RELPOS_FP16; }

// The attention kernels fold rel_w / scale into the q.k accumulator, so a
// nonzero scale must keep 1/scale finite with room to spare: 0, or
// 2^-64 <= |scale| < inf.
bool scale_ok(float scale) {
  if (!std::isfinite(scale)) return false;
  return scale == 0.0f || std::fabs(scale) >= 0x1p-64f;
}

relpos_status check_align(const Operand* ops, int n) {
  for (int i = 0; i < n; ++i) {
    if (ops[i].p == nullptr) return RELPOS_E_NULL;
  }
  for (int i = 0; i < n; ++i) {
    if (reinterpret_cast<uintptr_t>(ops[i].p) & 15u) return RELPOS_E_ALIGN;
  }
  return RELPOS_OK;
}

// Every operand must be device memory of the current device, and its
// allocation must hold the whole operand.  Each allocation is queried once:
// an operand inside a range an earlier operand of the same call already
// resolved needs no query (q, k and v cut from one qkv tensor cost one).
// Failed queries leave no sticky HIP error behind.
relpos_status check_device(const Operand* ops, int n) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return RELPOS_E_HIP;
  }
  uintptr_t lo[8], hi[8];
  int known = 0;
  for (int i = 0; i < n; ++i) {
    const uintptr_t p0 = reinterpret_cast<uintptr_t>(ops[i].p);
    const uintptr_t p1 = p0 + ops[i].bytes;
    bool inside = false;
    for (int j = 0; j < known && !inside; ++j) inside = p0 >= lo[j] && p0 < hi[j];
    if (inside) {
      for (int j = 0; j < known; ++j) {
        if (p0 >= lo[j] && p0 < hi[j] && p1 > hi[j]) return RELPOS_E_SHAPE;
      }
      continue;
    }
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, ops[i].p) != hipSuccess) {
      (void)hipGetLastError();
      return RELPOS_E_DEVICE;
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return RELPOS_E_DEVICE;
    if (attr.device != dev) return RELPOS_E_DEVICE;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(ops[i].p)) != hipSuccess) {
      (void)hipGetLastError();
      return RELPOS_E_DEVICE;
    }
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(base);
    if (p1 > b0 + size) return RELPOS_E_SHAPE;
    if (known < 8) {
      lo[known] = b0;
      hi[known] = b0 + size;
      ++known;
    }
  }
  return RELPOS_OK;
}

// Per-device cache of the LDS a workgroup may use and the compute-unit count.
struct DeviceProps {
  int lds_limit;
  int cus;
};
int device_props(DeviceProps* out) {
  static std::once_flag once[kMaxDevices];
  static DeviceProps props[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return -1;
  }
  std::call_once(once[dev], [dev]() {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) {
      (void)hipGetLastError();
      v = 65536;
    }
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) {
      (void)hipGetLastError();
      c = 256;
    }
    props[dev] = DeviceProps{v, c};
  });
  *out = props[dev];
  return 0;
}

// Scratch memory of relpos_attn_fused_noalloc: one array per device (each
// device that loads the library holds its own copy until the process ends).
// Host code never passes `scratch` itself to a kernel (on the host it names a
// stand-in, not device memory); it passes the device address looked up once
// per device by scratch_ptr.
static __device__ __align__(256) unsigned char scratch[RELPOS_SCRATCH_BYTES];

// Device address of the current device's scratch array, or nullptr if the
// lookup fails (the HIP error is cleared).  Looked up on the first call on
// each device, with that device current.
void* scratch_ptr() {
  static std::once_flag once[kMaxDevices];
  static void* ptrs[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::call_once(once[dev], [dev]() {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      p = nullptr;
    }
    ptrs[dev] = p;
  });
  return ptrs[dev];
}

relpos_status fused_impl(const void* q, const void* k, const void* v, const void* rel_pos_h,
                         const void* rel_pos_w, void* out, int64_t B, int64_t heads, int64_t H, int64_t W,
                         int64_t D, float scale, relpos_dtype in_dtype, relpos_dtype out_dtype, void* workspace,
                         int64_t workspace_bytes, bool from_scratch, void* stream);

// Attention configuration for B*heads = BH problems on an H x W grid on `cus`
// compute units: 0 (8-wave workgroups), 1 (4-wave) or, when a workspace is
// available, kAttnSplitConfig.  The cost model is the one documented with
// relpos_attn_config in include/relpos.h; times are in 4-wave rounds.
int attn_auto_config(int64_t BH, int64_t H, int64_t W, bool bf16, int cus, bool allow_split) {
  const int64_t N = H * W;
  const int64_t T = ((H + 3) / 4) * ((W + 15) / 16);  // key tiles per query unit
  // Key loops of at most four tiles: the 16-query kernel (configuration 3),
  // whose two-stage pipeline starts and drains faster and which runs three
  // waves per SIMD, is the fastest (25 windows x 12 heads of 14x14: 17.4 us
  // against 18.9 us for 4-wave and 21.1 us for 8-wave workgroups).
  if (T <= 4) return 3;
  const double a8 = bf16 ? 0.91 : 0.985;
  // Configuration 0 (one workgroup per CU): every started round is a full
  // round.  Configuration 1 (two per CU): a last round with at most one
  // workgroup per CU runs those workgroups alone on their CUs.
  const int64_t g8 = BH * ((N + 255) / 256);
  const int64_t g4 = BH * ((N + 127) / 128);
  const double t8 = a8 * static_cast<double>((g8 + cus - 1) / cus);
  const int64_t full = g4 / (2 * cus), rem = g4 % (2 * cus);
  const double t4 = static_cast<double>(full) + (rem == 0 ? 0.0 : (rem <= cus ? 0.77 : 1.0));
  int best = t8 <= t4 ? 0 : 1;
  double tbest = best == 0 ? t8 : t4;
  // 12-wave kernel (configuration 6), bf16 inputs on grids where it runs
  // P.V in bf16 and so stages V without conversion: one workgroup of 192
  // queries per CU, a round taken as 0.75 * 1.05 of an 8-wave round.  The
  // finer grain fills CUs that 256-query units leave idle.  Measured (us,
  // configuration 6 / 0 / split): 64x64 x 12 heads 67.8 / 73.8 / 75.4, 48x80
  // x 24 heads 116.7 / 142.0 / 124.8, 96x96 x 32 heads 802 / 893 / 841.
  if (bf16 && relpos::attn12_bf16_p(static_cast<int>(H), static_cast<int>(W)) &&
      relpos::attn12_fits(static_cast<int>(H), static_cast<int>(W))) {
    const int64_t g12 = (BH * ((N + 31) / 32) + 5) / 6;
    const double t12 = a8 * 0.75 * 1.05 * static_cast<double>((g12 + cus - 1) / cus);
    if (t12 < tbest) {
      best = relpos::kAttn12Config;
      tbest = t12;
    }
  }
  // Split: the full rounds of 8-wave units, then a last round whose heads
  // and tails (k per idle CU) take max(s + F, k*(T - s + F)) tiles with F =
  // kSplitSegmentTiles per segment, plus the merge, all at kSplitGridFactor
  // times the unsplit per-tile cost; considered when at most 4 tails share a
  // CU.
  if (allow_split) {
    constexpr int F = relpos::kSplitSegmentTiles;
    const relpos::SplitPlan sp = relpos::split_plan(g8, static_cast<int>(T), cus, F);
    if (sp.rest > 0 && sp.s < T && sp.k <= 4) {
      const int64_t head = sp.s + F, tails = static_cast<int64_t>(sp.k) * (T - sp.s + F);
      const int64_t last = head > tails ? head : tails;
      const double ts = a8 * relpos::kSplitGridFactor *
                        (sp.rounds + static_cast<double>(last + relpos::kMergeTiles) / static_cast<double>(T));
      if (ts < tbest) best = relpos::kAttnSplitConfig;
    }
  }
  return best;
}

// Order in which attention configurations are tried when the chosen one does
// not fit the device's LDS.
constexpr int kAttnFallback[] = {0, 1, 3};

bool config_known(int c) {
  return c == 0 || c == 1 || c == 3 || c == relpos::kAttnSplitConfig || c == relpos::kAttn12Config;
}

// Shared body of relpos_attn_fwd, relpos_attn_fwd_ws and relpos_attn_fwd_cfg
// (forced >= 0: that configuration, which must fit the device's LDS).
relpos_status attn_fwd_impl(const void* q, const void* k, const void* v,
                            const float* rel_h, const float* rel_w, void* out,
                            int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                            float scale, relpos_dtype in_dtype, relpos_dtype out_dtype,
                            bool with_ws, void* workspace, int64_t workspace_bytes, void* stream,
                            int forced) {
  int64_t BH = 0;
  relpos_status st = check_dims(B, heads, H, W, D, &BH);
  if (st != RELPOS_OK) return st;
  if (!is_half(in_dtype)) return RELPOS_E_DTYPE;
  if (out_dtype != RELPOS_FP32 && out_dtype != in_dtype) return RELPOS_E_DTYPE;
  if (!scale_ok(scale)) return RELPOS_E_VALUE;
  if (BH == 0) return RELPOS_OK;
  // Workgroup counts (down to 64 queries each) must fit a 1-D grid.
  if (BH * ((H * W + 63) / 64) >= (int64_t(1) << 31)) return RELPOS_E_SHAPE;

  const size_t N = static_cast<size_t>(H * W);
  const size_t in_bytes = BH * N * 64 * 2;
  const size_t out_bytes = BH * N * 64 * (out_dtype == RELPOS_FP32 ? 4 : 2);
  Operand ops[7] = {
      {q, in_bytes}, {k, in_bytes}, {v, in_bytes},
      {rel_h, BH * N * H * 4}, {rel_w, BH * N * W * 4}, {out, out_bytes}, {nullptr, 0},
  };
  if ((st = check_align(ops, 6)) != RELPOS_OK) return st;
  for (int i = 0; i < 5; ++i) {
    if (overlaps(ops[5], ops[i])) return RELPOS_E_ALIAS;
  }

  DeviceProps props{};
  if (device_props(&props) != 0) return RELPOS_E_HIP;
  auto fits = [&](int c) {
    if (c == relpos::kAttn12Config && !relpos::attn12_fits(static_cast<int>(H), static_cast<int>(W))) return false;
    return relpos::attn_lds_bytes(c, static_cast<int>(H), static_cast<int>(W)) <=
           static_cast<size_t>(props.lds_limit);
  };
  const bool bf16 = in_dtype == RELPOS_BF16;
  // The workspace is used (and checked) only when the split is chosen.
  const size_t need = relpos::attn_split_workspace_bytes(BH, H * W, props.cus);
  int cfg = forced;
  if (cfg >= 0 && !fits(cfg)) return RELPOS_E_SHAPE;
  if (cfg < 0) cfg = attn_auto_config(BH, H, W, bf16, props.cus, with_ws);
  if (cfg == relpos::kAttnSplitConfig) {
    if (workspace == nullptr) return RELPOS_E_NULL;
    ops[6] = Operand{workspace, need};
    if ((st = check_align(ops + 6, 1)) != RELPOS_OK) return st;
    if (static_cast<uint64_t>(workspace_bytes) < need) return RELPOS_E_SHAPE;
    for (int i = 0; i < 6; ++i) {
      if (overlaps(ops[6], ops[i])) return RELPOS_E_ALIAS;
    }
  }
  if (!fits(cfg)) {
    cfg = -1;
    for (int cand : kAttnFallback) {
      if (fits(cand)) {
        cfg = cand;
        break;
      }
    }
  }
  if (cfg < 0) return RELPOS_E_SHAPE;
  if ((st = check_device(ops, cfg == relpos::kAttnSplitConfig ? 7 : 6)) != RELPOS_OK) return st;

  relpos::AttnArgs a{q, k, v, rel_h, rel_w, out,
                     static_cast<int>(BH), static_cast<int>(H), static_cast<int>(W), scale,
                     bf16, out_dtype == RELPOS_FP32};
  a.lds_limit = props.lds_limit;
  if (cfg == relpos::kAttnSplitConfig) {
    a.ws = workspace;
    a.split_ctas = props.cus;
  }
  if (relpos::launch_attn_fwd(a, cfg, static_cast<hipStream_t>(stream)) != hipSuccess) return RELPOS_E_LAUNCH;
  return RELPOS_OK;
}

}  // namespace

extern "C" {

int relpos_abi_version(void) { return RELPOS_ABI_VERSION; }

int relpos_attn_config(int64_t B, int64_t heads, int64_t H, int64_t W, relpos_dtype in_dtype,
                       int cu_count, int with_workspace) {
  int64_t BH = 0;
  if (check_dims(B, heads, H, W, 64, &BH) != RELPOS_OK || !is_half(in_dtype) || cu_count < 1) return -1;
  return attn_auto_config(BH, H, W, in_dtype == RELPOS_BF16, cu_count, with_workspace != 0);
}

const char* relpos_status_string(relpos_status s) {
  switch (s) {
    case RELPOS_OK: return "ok";
    case RELPOS_E_NULL: return "a required pointer is NULL";
    case RELPOS_E_SHAPE: return "a size is out of range or an allocation is too small";
    case RELPOS_E_DTYPE: return "unsupported dtype or dtype combination";
    case RELPOS_E_ALIGN: return "a pointer is not 16-byte aligned";
    case RELPOS_E_DEVICE: return "a pointer is not device memory of the current device";
    case RELPOS_E_ALIAS: return "an output overlaps another operand";
    case RELPOS_E_LAUNCH: return "kernel launch failed";
    case RELPOS_E_HIP: return "a HIP runtime call failed";
    case RELPOS_E_VALUE: return "a scalar argument is invalid";
  }
  return "unknown status";
}

relpos_status relpos_build(const void* q, const void* rel_pos_h, const void* rel_pos_w,
                           float* rel_h, float* rel_w,
                           int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                           relpos_dtype in_dtype, void* stream) {
  int64_t BH = 0;
  relpos_status st = check_dims(B, heads, H, W, D, &BH);
  if (st != RELPOS_OK) return st;
  if (!is_half(in_dtype)) return RELPOS_E_DTYPE;
  if (BH == 0) return RELPOS_OK;

  const size_t N = static_cast<size_t>(H * W);
  const Operand ops[5] = {
      {q, BH * N * 64 * 2},
      {rel_pos_h, static_cast<size_t>(2 * H - 1) * 64 * 2},
      {rel_pos_w, static_cast<size_t>(2 * W - 1) * 64 * 2},
      {rel_h, BH * N * H * 4},
      {rel_w, BH * N * W * 4},
  };
  if ((st = check_align(ops, 5)) != RELPOS_OK) return st;
  for (int o = 3; o < 5; ++o) {
    for (int i = 0; i < 5; ++i) {
      if (i != o && overlaps(ops[o], ops[i])) return RELPOS_E_ALIAS;
    }
  }
  if ((st = check_device(ops, 5)) != RELPOS_OK) return st;

  relpos::BuildArgs a{q, rel_pos_h, rel_pos_w, rel_h, rel_w,
                      static_cast<int>(BH), static_cast<int>(H), static_cast<int>(W),
                      in_dtype == RELPOS_BF16};
  if (relpos::launch_build(a, static_cast<hipStream_t>(stream)) != hipSuccess) return RELPOS_E_LAUNCH;
  return RELPOS_OK;
}

relpos_status relpos_attn_fwd(const void* q, const void* k, const void* v,
                              const float* rel_h, const float* rel_w, void* out,
                              int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                              float scale, relpos_dtype in_dtype, relpos_dtype out_dtype,
                              void* stream) {
  return attn_fwd_impl(q, k, v, rel_h, rel_w, out, B, heads, H, W, D, scale, in_dtype, out_dtype,
                       false, nullptr, 0, stream, -1);
}

int64_t relpos_attn_workspace_bytes(int64_t B, int64_t heads, int64_t H, int64_t W, relpos_dtype in_dtype,
                                    int cu_count) {
  int64_t BH = 0;
  if (check_dims(B, heads, H, W, 64, &BH) != RELPOS_OK || !is_half(in_dtype) || cu_count < 1) return -1;
  if (attn_auto_config(BH, H, W, in_dtype == RELPOS_BF16, cu_count, true) != relpos::kAttnSplitConfig) return 0;
  return static_cast<int64_t>(relpos::attn_split_workspace_bytes(BH, H * W, cu_count));
}

int64_t relpos_fused_workspace_bytes(int64_t B, int64_t heads, int64_t H, int64_t W, relpos_dtype in_dtype,
                                     int cu_count) {
  int64_t BH = 0;
  if (check_dims(B, heads, H, W, 64, &BH) != RELPOS_OK || !is_half(in_dtype) || cu_count < 1) return -1;
  if (relpos::attn_fused16_ok(static_cast<int>(H), static_cast<int>(W))) return 0;
  if (relpos::attn_fused12_ok(static_cast<int>(H), static_cast<int>(W), in_dtype == RELPOS_BF16)) {
    return static_cast<int64_t>(
        relpos::attn_fused12_workspace_bytes(BH, static_cast<int>(H), static_cast<int>(W), cu_count));
  }
  return static_cast<int64_t>(relpos::attn_fused_workspace_bytes(static_cast<int>(H), static_cast<int>(W),
                                                                 cu_count));
}

relpos_status relpos_attn_fused(const void* q, const void* k, const void* v,
                                const void* rel_pos_h, const void* rel_pos_w, void* out,
                                int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                                float scale, relpos_dtype in_dtype, relpos_dtype out_dtype,
                                void* workspace, int64_t workspace_bytes, void* stream) {
  return fused_impl(q, k, v, rel_pos_h, rel_pos_w, out, B, heads, H, W, D, scale, in_dtype, out_dtype,
                    workspace, workspace_bytes, false, stream);
}

relpos_status relpos_attn_fused_noalloc(const void* q, const void* k, const void* v,
                                        const void* rel_pos_h, const void* rel_pos_w, void* out,
                                        int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                                        float scale, relpos_dtype in_dtype, relpos_dtype out_dtype,
                                        void* stream) {
  return fused_impl(q, k, v, rel_pos_h, rel_pos_w, out, B, heads, H, W, D, scale, in_dtype, out_dtype,
                    nullptr, 0, true, stream);
}

}  // extern "C"

namespace {

// relpos_attn_fused, with the caller's workspace or (from_scratch) the
// library's per-device scratch array.
relpos_status fused_impl(const void* q, const void* k, const void* v, const void* rel_pos_h,
                         const void* rel_pos_w, void* out, int64_t B, int64_t heads, int64_t H, int64_t W,
                         int64_t D, float scale, relpos_dtype in_dtype, relpos_dtype out_dtype, void* workspace,
                         int64_t workspace_bytes, bool from_scratch, void* stream) {
  int64_t BH = 0;
  relpos_status st = check_dims(B, heads, H, W, D, &BH);
  if (st != RELPOS_OK) return st;
  if (!is_half(in_dtype)) return RELPOS_E_DTYPE;
  if (out_dtype != RELPOS_FP32 && out_dtype != in_dtype) return RELPOS_E_DTYPE;
  if (!scale_ok(scale) || workspace_bytes < 0) return RELPOS_E_VALUE;
  if (BH == 0) return RELPOS_OK;
  if (BH * ((H * W + 63) / 64) >= (int64_t(1) << 31)) return RELPOS_E_SHAPE;

  const size_t N = static_cast<size_t>(H * W);
  const size_t in_bytes = BH * N * 64 * 2;
  const size_t out_bytes = BH * N * 64 * (out_dtype == RELPOS_FP32 ? 4 : 2);
  Operand ops[7] = {
      {q, in_bytes},
      {k, in_bytes},
      {v, in_bytes},
      {rel_pos_h, static_cast<size_t>(2 * H - 1) * 64 * 2},
      {rel_pos_w, static_cast<size_t>(2 * W - 1) * 64 * 2},
      {out, out_bytes},
      {workspace, 0},
  };
  // Three launch forms: the 16-query kernel with the bias rows in LDS (small
  // grids, no workspace), the 12-wave fused kernel where the grid allows it,
  // else the split-grid one.
  const bool f16 = relpos::attn_fused16_ok(static_cast<int>(H), static_cast<int>(W));
  const bool f12 =
      !f16 && relpos::attn_fused12_ok(static_cast<int>(H), static_cast<int>(W), in_dtype == RELPOS_BF16);
  // The scratch array is not the caller's, and the 16-query form takes no
  // workspace: then only the six operands are checked.
  const int nops = from_scratch || f16 ? 6 : 7;
  if ((st = check_align(ops, nops)) != RELPOS_OK) return st;
  for (int i = 0; i < 5; ++i) {
    if (overlaps(ops[5], ops[i])) return RELPOS_E_ALIAS;
  }
  // The workspace size depends on the device's compute-unit count.
  DeviceProps props{};
  if (device_props(&props) != 0) return RELPOS_E_HIP;
  if (f16) {
    if (relpos::attn_fused16_lds_bytes(static_cast<int>(H), static_cast<int>(W)) >
        static_cast<size_t>(props.lds_limit)) {
      return RELPOS_E_SHAPE;
    }
    if ((st = check_device(ops, 6)) != RELPOS_OK) return st;
    relpos::AttnArgs a{q, k, v, nullptr, nullptr, out,
                       static_cast<int>(BH), static_cast<int>(H), static_cast<int>(W), scale,
                       in_dtype == RELPOS_BF16, out_dtype == RELPOS_FP32};
    a.th = rel_pos_h;
    a.tw = rel_pos_w;
    if (relpos::launch_attn_fused16(a, static_cast<hipStream_t>(stream)) != hipSuccess) return RELPOS_E_LAUNCH;
    return RELPOS_OK;
  }
  const size_t need = f12 ? relpos::attn_fused12_workspace_bytes(BH, static_cast<int>(H), static_cast<int>(W), props.cus)
                          : relpos::attn_fused_workspace_bytes(static_cast<int>(H), static_cast<int>(W), props.cus);
  if (from_scratch) {
    if (need > static_cast<size_t>(RELPOS_SCRATCH_BYTES)) return RELPOS_E_SHAPE;
    if ((workspace = scratch_ptr()) == nullptr) return RELPOS_E_HIP;
  } else {
    if (static_cast<uint64_t>(workspace_bytes) < need) return RELPOS_E_SHAPE;
    ops[6].bytes = need;
    for (int i = 0; i < 6; ++i) {
      if (overlaps(ops[6], ops[i])) return RELPOS_E_ALIAS;
    }
  }
  if ((f12 ? relpos::attn12_lds_bytes()
           : relpos::attn_lds_bytes(relpos::kAttnSplitConfig, static_cast<int>(H), static_cast<int>(W))) >
      static_cast<size_t>(props.lds_limit)) {
    return RELPOS_E_SHAPE;
  }
  if ((st = check_device(ops, nops)) != RELPOS_OK) return st;

  relpos::AttnArgs a{q, k, v, nullptr, nullptr, out,
                     static_cast<int>(BH), static_cast<int>(H), static_cast<int>(W), scale,
                     in_dtype == RELPOS_BF16, out_dtype == RELPOS_FP32};
  a.ws = workspace;
  a.split_ctas = props.cus;
  a.th = rel_pos_h;
  a.tw = rel_pos_w;
  a.lds_limit = props.lds_limit;
  const hipError_t err = f12 ? relpos::launch_attn_fused12(a, static_cast<hipStream_t>(stream))
                            : relpos::launch_attn_fused(a, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return RELPOS_E_LAUNCH;
  return RELPOS_OK;
}

}  // namespace

extern "C" {

relpos_status relpos_attn_fwd_ws(const void* q, const void* k, const void* v,
                                 const float* rel_h, const float* rel_w, void* out,
                                 int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                                 float scale, relpos_dtype in_dtype, relpos_dtype out_dtype,
                                 void* workspace, int64_t workspace_bytes, void* stream) {
  if (workspace_bytes < 0) return RELPOS_E_VALUE;
  return attn_fwd_impl(q, k, v, rel_h, rel_w, out, B, heads, H, W, D, scale, in_dtype, out_dtype,
                       true, workspace, workspace_bytes, stream, -1);
}

relpos_status relpos_attn_fwd_cfg(const void* q, const void* k, const void* v,
                                  const float* rel_h, const float* rel_w, void* out,
                                  int64_t B, int64_t heads, int64_t H, int64_t W, int64_t D,
                                  float scale, relpos_dtype in_dtype, relpos_dtype out_dtype,
                                  int config, void* workspace, int64_t workspace_bytes, void* stream) {
  if (workspace_bytes < 0 || (config != -1 && !config_known(config))) return RELPOS_E_VALUE;
  return attn_fwd_impl(q, k, v, rel_h, rel_w, out, B, heads, H, W, D, scale, in_dtype, out_dtype,
                       true, workspace, workspace_bytes, stream, config);
}

}  // extern "C"
