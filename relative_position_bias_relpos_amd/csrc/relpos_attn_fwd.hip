// relpos_attn_fwd kernel: attention over an H x W token grid with the decomposed
// relative-position bias added per tile (PR #55629 page, implementation section,
// item 1: K/V streamed with an online softmax, the bias slices loaded per key
// block, no dense [N, N] bias).
//
// Layout of the work
//   * A workgroup owns BM = 32*NW consecutive queries of one (batch, head); each
//     of its NW waves owns 32 of them.
//   * Keys are visited in 2-D tiles of the key grid: 4 grid rows x 16 grid
//     columns = 64 keys.  Inside a tile, key o (0..63) is grid cell
//     (kh0 + o/16, kw0 + o%16).  Cells outside the grid are masked.
//   * Scores are computed transposed, S^T = K * Q^T, with 32x32x16 MFMA: a lane
//     then holds one query (lane%32) and 32 of the tile's keys, so row max and
//     row sum need a single cross-lane step (lane ^ 32).
//   * For the lane's keys o = 32*st + 8*g + 4*(lane/32) + e the grid offsets are
//     r = o/16 = 2*st + g/2 and c = o%16 = 8*(g%2) + 4*(lane/32) + e, so the
//     bias needs 4 rel_h values and 8 rel_w values per tile, read as three
//     16-byte LDS loads.
//   * O^T = V^T * P^T, again 32x32x16 MFMA, with P in fp16.  V tiles are stored
//     transposed in LDS (d-major) with the keys of each 16-key step permuted so
//     that a lane's eight keys are one 16-byte read.  bf16 V is converted to
//     fp16 while staging (exact for |v| < 65520).
#include "relpos_device.hpp"
#include "relpos_kernels.hpp"

namespace relpos {

namespace {

constexpr int kD = 64;
constexpr int kTileKeys = 64;
constexpr int kTileRows = 4;
constexpr int kTileCols = 16;
constexpr int kKStride = kD + 8;          // halves per K row in LDS (144 B)
constexpr int kVStride = kTileKeys + 8;   // halves per V^T row in LDS (144 B)

// LDS slot of key o inside its tile for the V^T layout: within each 16-key
// group, bit 2 of o selects the lane half and bit 3 the second 4-key run.
__device__ __forceinline__ int v_slot(int o) {
  return (o & ~15) | (((o >> 2) & 1) << 3) | (((o >> 3) & 1) << 2) | (o & 3);
}

template <bool BF16, bool OUT_F32, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ rel_h,
    const float* __restrict__ rel_w, void* __restrict__ out,
    int H, int W, int Hp, int Wp, float c2) {
  constexpr int BM = 32 * NW;
  constexpr int NT = NW * 64;
  const int N = H * W;
  const int WSTR = Wp + 4;
  const int HSTR = Hp + 4;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);         // [2][64][kKStride]
  uint16_t* Vt = Ks + 2 * kTileKeys * kKStride;              // [2][64][kVStride]
  float* rws = reinterpret_cast<float*>(Vt + 2 * kD * kVStride);  // [BM][WSTR]
  float* rhs = rws + BM * WSTR;                                    // [BM][HSTR]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int q0 = blockIdx.x * BM;
  const size_t head = static_cast<size_t>(blockIdx.y) * N;

  // ---- per-workgroup bias rows, in log2 units, padding = -inf -------------
  for (int idx = tid; idx < BM * Wp; idx += NT) {
    const int r = idx / Wp, c = idx - r * Wp;
    const int qi = q0 + r;
    float val = -__builtin_inff();
    if (c < W) val = (qi < N) ? rel_w[(head + qi) * W + c] * kLog2e : 0.f;
    rws[r * WSTR + c] = val;
  }
  for (int idx = tid; idx < BM * Hp; idx += NT) {
    const int r = idx / Hp, c = idx - r * Hp;
    const int qi = q0 + r;
    float val = -__builtin_inff();
    if (c < H) val = (qi < N) ? rel_h[(head + qi) * H + c] * kLog2e : 0.f;
    rhs[r * HSTR + c] = val;
  }

  // ---- this lane's query: Q^T operand fragments (4 k-steps of 16) ---------
  const int qrow = wave * 32 + (lane & 31);
  const int qi = q0 + qrow;
  u32x4 qf[4];
#pragma unroll
  for (int kd = 0; kd < 4; ++kd) {
    qf[kd] = (qi < N) ? *reinterpret_cast<const u32x4*>(q + (head + qi) * kD + 16 * kd + 8 * half)
                      : u32x4{0, 0, 0, 0};
  }

  const int nWt = (W + kTileCols - 1) / kTileCols;
  const int nHt = (H + kTileRows - 1) / kTileRows;
  const int T = nWt * nHt;

  // ---- K/V tile staging: global -> registers -> LDS ------------------------
  constexpr int KCH = (kTileKeys * kD / 8) / NT;   // 16-byte K chunks per thread
  constexpr int VPT = (kTileKeys / 2) * (kD / 8) / NT;  // (key pair, d chunk) tasks per thread
  static_assert(KCH >= 1 && VPT >= 1, "workgroup too large for one tile");
  u32x4 kreg[KCH];
  u32x4 vreg[VPT][2];

  auto key_of = [&](int t, int o, bool& ok) -> int {
    const int kh = (t / nWt) * kTileRows + (o >> 4);
    const int kw = (t % nWt) * kTileCols + (o & 15);
    ok = (kh < H) && (kw < W);
    return kh * W + kw;
  };
  auto load_tile = [&](int t) {
#pragma unroll
    for (int s = 0; s < KCH; ++s) {
      const int cid = tid + s * NT;
      const int o = cid >> 3, ch = cid & 7;
      bool ok;
      const int j = key_of(t, o, ok);
      kreg[s] = ok ? *reinterpret_cast<const u32x4*>(k + (head + j) * kD + 8 * ch) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
      const int task = tid + s * NT;
      const int p = task >> 3, dc = task & 7;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bool ok;
        const int j = key_of(t, 2 * p + u, ok);
        vreg[s][u] = ok ? *reinterpret_cast<const u32x4*>(v + (head + j) * kD + 8 * dc) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* kb = Ks + buf * kTileKeys * kKStride;
    uint16_t* vb = Vt + buf * kD * kVStride;
#pragma unroll
    for (int s = 0; s < KCH; ++s) {
      const int cid = tid + s * NT;
      const int o = cid >> 3, ch = cid & 7;
      *reinterpret_cast<u32x4*>(kb + o * kKStride + 8 * ch) = kreg[s];
    }
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
      const int task = tid + s * NT;
      const int p = task >> 3, dc = task & 7;
      const int slot = v_slot(2 * p);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a = vreg[s][0][w], b = vreg[s][1][w];
        uint32_t lo, hi;  // (key 2p, key 2p+1) pairs for d = 8dc+2w and 8dc+2w+1
        if constexpr (BF16) {
          lo = pack_f16(bf16_lo(a), bf16_lo(b));
          hi = pack_f16(bf16_hi(a), bf16_hi(b));
        } else {
          lo = (a & 0xffffu) | (b << 16);
          hi = (a >> 16) | (b & 0xffff0000u);
        }
        const int d = 8 * dc + 2 * w;
        *reinterpret_cast<uint32_t*>(vb + d * kVStride + slot) = lo;
        *reinterpret_cast<uint32_t*>(vb + (d + 1) * kVStride + slot) = hi;
      }
    }
  };

  load_tile(0);
  store_tile(0);

  f32x16 acc[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) acc[dt] = f32x16{};
  float m = -__builtin_inff();
  float l = 0.f;
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

  for (int t = 0; t < T; ++t) {
    __syncthreads();
    const int buf = t & 1;
    if (t + 1 < T) load_tile(t + 1);
    const uint16_t* kb = Ks + buf * kTileKeys * kKStride;
    const uint16_t* vb = Vt + buf * kD * kVStride;
    const int kh0 = (t / nWt) * kTileRows;
    const int kw0 = (t % nWt) * kTileCols;

    // S^T = K Q^T for the tile's 64 keys (two 32-key halves).
    f32x16 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = f32x16{};
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(kb + (32 * st + (lane & 31)) * kKStride + 16 * kd + 8 * half);
        s[st] = mfma32<BF16>(kf, qf[kd], s[st]);
      }
    }

    // bias, in log2 units: t = s*scale*log2e + rel_h' + rel_w'
    const f32x4 rw0 = *reinterpret_cast<const f32x4*>(rws + qrow * WSTR + kw0 + 4 * half);
    const f32x4 rw1 = *reinterpret_cast<const f32x4*>(rws + qrow * WSTR + kw0 + 8 + 4 * half);
    const f32x4 rh = *reinterpret_cast<const f32x4*>(rhs + qrow * HSTR + kh0);
    float mloc = -__builtin_inff();
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float rhv = rh[2 * st + (g >> 1)];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float rwv = (g & 1) ? rw1[e] : rw0[e];
          const float x = __builtin_fmaf(s[st][4 * g + e], c2, rhv + rwv);
          s[st][4 * g + e] = x;
          mloc = __builtin_fmaxf(mloc, x);
        }
      }
    }
    mloc = __builtin_fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = __builtin_fmaxf(m, mloc);
    const float alpha = exp2_fast(m - m_new);
    m = m_new;

    // p = exp2(t - m), rounded to fp16; the row sum uses the rounded values.
    u32x4 pf[4];
    float lt = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        uint32_t w4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = exp2_fast(s[st][8 * gg + 2 * i] - m_new);
          const float p1 = exp2_fast(s[st][8 * gg + 2 * i + 1] - m_new);
          w4[i] = pack_f16(p0, p1);
          lt = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w4[i]), ones, lt, false);
        }
        pf[2 * st + gg] = u32x4{w4[0], w4[1], w4[2], w4[3]};
      }
    }
    l = l * alpha + lt;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) acc[dt] *= alpha;

    // O^T += V^T P^T: four 16-key steps, two 32-row d tiles.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const u32x4 vf = *reinterpret_cast<const u32x4*>(vb + (32 * dt + (lane & 31)) * kVStride + 16 * ks + 8 * half);
        acc[dt] = mfma32<false>(vf, pf[ks], acc[dt]);
      }
    }

    if (t + 1 < T) store_tile(buf ^ 1);
  }

  // ---- epilogue: combine the two lane halves' row sums, normalise, store ----
  l += __shfl_xor(l, 32);
  if (qi < N) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * half;
        const f32x4 o4 = {acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv,
                          acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv};
        if constexpr (OUT_F32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(out) + (head + qi) * kD + d) = o4;
        } else {
          const u32x2 pk = BF16 ? u32x2{pack_bf16(o4[0], o4[1]), pack_bf16(o4[2], o4[3])}
                                : u32x2{pack_f16(o4[0], o4[1]), pack_f16(o4[2], o4[3])};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + (head + qi) * kD + d) = pk;
        }
      }
    }
  }
}

template <bool BF16, bool OUT_F32, int NW>
hipError_t launch_nw(const AttnArgs& a, size_t lds, hipStream_t stream) {
  auto kern = attn_fwd_kernel<BF16, OUT_F32, NW>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (err != hipSuccess) return err;
  constexpr int BM = 32 * NW;
  dim3 grid(static_cast<unsigned>((a.H * a.W + BM - 1) / BM), static_cast<unsigned>(a.BH));
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.rel_h, a.rel_w, a.out,
                     a.H, a.W, round_up(a.H, kTileRows), round_up(a.W, kTileCols),
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <bool BF16, bool OUT_F32>
hipError_t launch_dt(const AttnArgs& a, int nw, size_t lds, hipStream_t stream) {
  switch (nw) {
    case 4: return launch_nw<BF16, OUT_F32, 4>(a, lds, stream);
    case 2: return launch_nw<BF16, OUT_F32, 2>(a, lds, stream);
    default: return launch_nw<BF16, OUT_F32, 1>(a, lds, stream);
  }
}

}  // namespace

size_t attn_lds_bytes(int nw, int H, int W) {
  const size_t kv = 2 * (size_t)kTileKeys * kKStride * 2 + 2 * (size_t)kD * kVStride * 2;
  const size_t rel = (size_t)32 * nw * ((round_up(W, kTileCols) + 4) + (round_up(H, kTileRows) + 4)) * 4;
  return kv + rel;
}

hipError_t launch_attn_fwd(const AttnArgs& a, int nw, hipStream_t stream) {
  const size_t lds = attn_lds_bytes(nw, a.H, a.W);
  if (a.bf16) {
    return a.out_f32 ? launch_dt<true, true>(a, nw, lds, stream) : launch_dt<true, false>(a, nw, lds, stream);
  }
  return a.out_f32 ? launch_dt<false, true>(a, nw, lds, stream) : launch_dt<false, false>(a, nw, lds, stream);
}

}  // namespace relpos
