// relpos_attn_fwd, 16-query-per-wave kernel (launch configuration 3).
//
// Same method as the 32-query kernel in relpos_attn_fwd.hip (PR #55629 page,
// implementation section, item 1: K/V streamed with an online softmax and the
// rel_h/rel_w slices added per key block), laid out for more waves per SIMD:
//
//   * A wave owns 16 queries; a workgroup of 4 waves owns 64 queries of one
//     (batch, head), and three waves fit per SIMD.  Measured on MI355X it is
//     slower than the 32-query kernel on long key loops (twice the LDS operand
//     traffic per score, and 16x16 MFMAs hide less VALU work); its shorter
//     pipeline wins on units of at most four key tiles (small windows).
//   * S^T = K Q^T on 16x16x32 MFMA.  A lane holds one query (lane%16) and, per
//     64-key tile of the key grid (4 rows x 16 columns), 16 keys
//     o = 16*st + 4*g + j (g = lane/16), i.e. grid row st and grid column
//     4*g + j.  Its bias needs 4 rel_w values per 16-column band and 4 rel_h
//     values per tile.
//   * O^T += V^T P^T on 16x16x32 MFMA with P in fp16.  For the 32-key step ks
//     the lane's 8 P values are keys 32ks + 4g + {0..3} and 32ks + 16 + 4g +
//     {0..3}; the V^T operand is two transpose reads of four consecutive keys.
//   * Two-stage pipeline: step t issues Q.K^T of tile t+1 together with the
//     softmax of tile t, then P.V of tile t.  K lives in a 2-slot LDS ring and
//     V in a 3-slot ring (tile t+2 is staged while t and t+1 are resident).
//   * Online softmax with a lazy reference maximum, as in the 32-query kernel:
//     m moves only on the first tile or when a tile's rounded-p sum exceeds
//     2^15; the row sum adds the rounded fp16 p.
//   * FUSED (relpos_attn_fused on grids with H, W <= 32 and at most four key
//     tiles, e.g. windows of 14x14): the workgroup first computes the rel_h
//     and rel_w rows of its 64 queries into LDS, with relpos_build's
//     small-grid products (both tables have at most 63 rows, so 32 queries'
//     products Q T^T are two 32x32 MFMA tiles per table; waves 0/2 take rel_h,
//     1/3 rel_w, of queries 0-31 / 32-63), and reads its bias from there: no
//     workspace and no rel_h / rel_w tensors.
#include <type_traits>

#include "relpos_attn_common.hpp"
#include "relpos_kernels.hpp"

namespace relpos {

using namespace attn;

namespace {

constexpr int kKSlots16 = 2;
constexpr int kVSlots16 = 3;

constexpr int NW = 4;
constexpr int kGStride16 = 72;  // floats per staged product row (64 used)

// x / d for 0 <= x < 2048 and 1 <= d <= 32, with m = ceil(2^16 / d): the
// error of x*m / 2^16 against x/d is below x/2^16 < 1/32 <= 1/d.
__device__ __forceinline__ int div_small16(int x, uint32_t m) {
  return static_cast<int>((static_cast<uint32_t>(x) * m) >> 16);
}

// Bias rows of `rows` (<= 32) consecutive queries i0 .. of one (b, h) into LDS
// (H, W <= 32): axis 0 writes rel_h [rows][H], axis 1 rel_w [rows][W] at dst,
// row-major.  G = Q T^T over all 2L-1 table rows (2 MFMA tiles), staged in
// `stage` (this wave's 32 x 72 floats), then element (m, c) of the rows is
// G[m, a - c + L - 1] with a the query's grid row (axis 0) or column.  The
// same products and order as relpos_build's small-grid kernel.
template <bool BF16>
__device__ __forceinline__ void bias_rows_lds(const uint16_t* __restrict__ qrows, int rows,
                                              const uint16_t* __restrict__ tab, int axis, int i0, int H, int W,
                                              uint32_t mh, uint32_t mw, float* stage, float* dst, int lane) {
  const int ml = lane & 31, half = lane >> 5;
  const int L = axis == 0 ? H : W;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qrows, static_cast<uint32_t>(rows) * kD * 2);
  const __amdgpu_buffer_rsrc_t rt = make_rsrc(tab, static_cast<uint32_t>(2 * L - 1) * kD * 2);
  const int dchunk = 16 * half;
  u32x4 a[4], b[2][4];
#pragma unroll
  for (int kd = 0; kd < 4; ++kd) a[kd] = buf_load16(rq, ml < rows ? ml * kD * 2 + 32 * kd + dchunk : kOob);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int j = 32 * nt + ml;
    const int off = j < 2 * L - 1 ? j * kD * 2 + dchunk : kOob;
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) b[nt][kd] = buf_load16(rt, off, 32 * kd);
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    f32x16 g{};
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) g = mfma32<BF16>(a[kd], b[nt][kd], g);
#pragma unroll
    for (int r = 0; r < 16; ++r) stage[(8 * (r >> 2) + 4 * half + (r & 3)) * kGStride16 + 32 * nt + ml] = g[r];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint32_t mL = axis == 0 ? mh : mw;
  const int total = rows * L;
  for (int f = lane; f < total; f += 64) {
    const int m = div_small16(f, mL);
    const int c = f - m * L;
    const int i = i0 + m;
    const int qr = div_small16(i, mw);  // grid row of query i
    const int av = axis == 0 ? qr : i - qr * W;
    dst[f] = stage[m * kGStride16 + av - c + L - 1];
  }
}

template <bool BF16, bool OUT_F32, bool FUSED>
__global__ __launch_bounds__(NW * 64, 3) void attn16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ rel_h,
    const float* __restrict__ rel_w, void* __restrict__ out,
    const uint16_t* __restrict__ th, const uint16_t* __restrict__ tw,
    int H, int W, int q_tiles, float c2, uint32_t mh, uint32_t mw) {
  constexpr int BM = 16 * NW;
  constexpr int NT = NW * 64;
  const int N = H * W;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);  // [2][64][kKStride]
  uint16_t* Vs = Ks + kKSlots16 * kTileHalves;       // [3][64][kKStride]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane >> 4;   // lane group: which 4 keys of each 16-key row, which 8 k of an MFMA
  const int col = lane & 15;   // this lane's query within the wave

  const int work = xcd_work_index(static_cast<int>(gridDim.x));
  const int bh = work / q_tiles;
  const int q0 = (work - bh * q_tiles) * BM;
  const size_t head = static_cast<size_t>(bh) * N;

  // ---- FUSED: the bias rows of the workgroup's 64 queries into LDS ------------
  // (rel_h [64][H] then rel_w [64][W] after the K/V ring; the products are
  // staged in the ring's space, which the tiles take only after the barrier)
  float* const bias_h = reinterpret_cast<float*>(smem + (kKSlots16 + kVSlots16) * kTileHalves * 2);
  float* const bias_w = bias_h + BM * H;
  if constexpr (FUSED) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int jb = wv >> 1, axis = wv & 1;
    const int i0 = q0 + 32 * jb;
    const int rows = N - i0 < 32 ? N - i0 : 32;
    if (rows > 0) {
      bias_rows_lds<BF16>(q + (head + i0) * kD, rows, axis == 0 ? th : tw, axis, i0, H, W, mh, mw,
                          reinterpret_cast<float*>(smem) + wv * 32 * kGStride16,
                          axis == 0 ? bias_h + 32 * jb * H : bias_w + 32 * jb * W, lane);
    }
    __syncthreads();
  }

  // ---- Q^T operand fragments: d = 32*kd + 8*grp .. +7 ------------------------
  const int qrow = wave * 16 + col;
  const int qi = q0 + qrow;
  u32x4 qf[2];
#pragma unroll
  for (int kd = 0; kd < 2; ++kd) {
    qf[kd] = (qi < N) ? *reinterpret_cast<const u32x4*>(q + (head + qi) * kD + 32 * kd + 8 * grp)
                      : u32x4{0, 0, 0, 0};
  }

  const int T = ((W + kTileCols - 1) / kTileCols) * ((H + kTileRows - 1) / kTileRows);

  // ---- K/V tile staging: global -> registers -> LDS (row-major, 16 B chunks)
  constexpr int CH = (kTileKeys * kD / 8) / NT;
  static_assert(CH >= 1, "workgroup too large for one tile");
  int ch_r[CH], ch_c[CH], ch_off[CH], ch_lds[CH];
#pragma unroll
  for (int s = 0; s < CH; ++s) {
    const int cid = tid + s * NT;
    const int o = cid >> 3, dc = cid & 7;
    ch_r[s] = o >> 4;
    ch_c[s] = o & 15;
    ch_off[s] = (o >> 4) * W + (o & 15);
    ch_lds[s] = o * kKStride + 8 * dc;
  }
  const int dcol = 8 * (tid & 7);
  u32x4 kreg[CH], vreg[CH];
  const uint32_t head_bytes = static_cast<uint32_t>(N) * kD * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + head * kD, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + head * kD, head_bytes);

  auto load_tile = [&](TilePos p) {
    const int base = p.kh * W + p.kw;
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      const bool ok = (p.kh + ch_r[s] < H) && (p.kw + ch_c[s] < W);
      const int off = ok ? ((base + ch_off[s]) * kD + dcol) * 2 : kOob;
      kreg[s] = buf_load16(krs, off);
      vreg[s] = buf_load16(vrs, off);
    }
  };
  auto store_tile = [&](int kslot, int vslot) {
    uint16_t* kb = Ks + kslot * kTileHalves;
    uint16_t* vb = Vs + vslot * kTileHalves;
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      *reinterpret_cast<u32x4*>(kb + ch_lds[s]) = kreg[s];
      u32x4 x = vreg[s];
      if constexpr (BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) x[w] = pack_f16(bf16_lo(x[w]), bf16_hi(x[w]));
      }
      *reinterpret_cast<u32x4*>(vb + ch_lds[s]) = x;
    }
  };

  // ---- bias: rel_w' for the lane's 4 columns of a band, rel_h' per tile ------
  // The unit's own rows only (at most 64 rows of at most 4096 floats, so the
  // byte range and the offsets stay far inside 32 bits for every grid).
  const int unit_rows = N - q0 < BM ? N - q0 : BM;
  const __amdgpu_buffer_rsrc_t rwrs =
      make_rsrc(FUSED ? nullptr : rel_w + (head + q0) * W,
                static_cast<uint32_t>(unit_rows) * static_cast<uint32_t>(W) * 4);
  const __amdgpu_buffer_rsrc_t rhrs =
      make_rsrc(FUSED ? nullptr : rel_h + (head + q0) * H,
                static_cast<uint32_t>(unit_rows) * static_cast<uint32_t>(H) * 4);
  const int brow = qi < N ? qrow : 0;  // queries past the grid read row 0's bias
  const int rw_off = brow * W * 4;
  const int rh_off = brow * H * 4;
  float rw[4];
  auto load_band = [&](int kw0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = kw0 + 4 * grp + j;
      float x;
      if constexpr (FUSED) {
        x = c < W ? bias_w[brow * W + c] : 0.f;
      } else {
        x = buf_loadf(rwrs, c < W ? rw_off + 4 * c : kOob);
      }
      rw[j] = (c < W) ? x * kLog2e : -__builtin_inff();
    }
  };
  float rhn[4];  // rel_h' of the 4 grid rows of the next tile to process
  auto load_rh = [&](int kh0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x;
      if constexpr (FUSED) {
        x = kh0 + r < H ? bias_h[brow * H + kh0 + r] : 0.f;
      } else {
        x = buf_loadf(rhrs, kh0 + r < H ? rh_off + 4 * (kh0 + r) : kOob);
      }
      rhn[r] = (kh0 + r < H) ? x * kLog2e : -__builtin_inff();
    }
  };

  // ---- compute pieces ------------------------------------------------------
  auto qk = [&](int kslot, f32x4 (&s)[4]) {
    const uint16_t* kb = Ks + kslot * kTileHalves;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4 k0 = *reinterpret_cast<const u32x4*>(kb + (16 * st + col) * kKStride + 8 * grp);
      const u32x4 k1 = *reinterpret_cast<const u32x4*>(kb + (16 * st + col) * kKStride + 32 + 8 * grp);
      s[st] = mfma16<BF16>(k0, qf[0], f32x4{0.f, 0.f, 0.f, 0.f});
      s[st] = mfma16<BF16>(k1, qf[1], s[st]);
    }
  };
  const int jl = col;
  const int tr_row = 4 * grp + (jl >> 2);
  const int tr_col = 4 * (jl & 3);
  f32x4 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto pv = [&](int vslot, const u32x4 (&pf)[2]) {
    const uint16_t* vb = Vs + vslot * kTileHalves;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint16_t* vp = vb + (32 * ks + tr_row) * kKStride + 16 * dt + tr_col;
        const u32x2 lo = ds_read_tr16(vp);
        const u32x2 hi = ds_read_tr16(vp + 16 * kKStride);
        const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
        acc[dt] = mfma16<false>(vf, pf[ks], acc[dt]);
      }
    }
  };

  // ---- prologue: tiles 0 and 1 in LDS, tile 2 in registers ------------------
  const TilePos p0{0, 0};
  const TilePos p1 = next_tile(p0, H);
  const TilePos p2 = next_tile(p1, H);
  load_tile(p0);
  store_tile(0, 0);
  if (T > 1) {
    load_tile(p1);
    store_tile(1, 1);
  }
  if (T > 2) load_tile(p2);
  load_rh(0);
  __syncthreads();

  float m = 0.f, l = 0.f;
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  f32x4 sA[4], sB[4];
  qk(0, sA);

  TilePos pc = p0;                // tile t
  TilePos pl = next_tile(p2, H);  // tile t+3
  int vslot = 0;                  // t % 3

  auto step = [&](int t, auto first_c, auto last_c, f32x4 (&sc)[4], f32x4 (&sn)[4]) {
    constexpr bool kFirst = decltype(first_c)::value;
    constexpr bool kLast = decltype(last_c)::value;
    if (pc.kh == 0) load_band(pc.kw);
    const TilePos pn = next_tile(pc, H);
    if constexpr (!kLast) qk((t + 1) & 1, sn);

    // softmax of tile t against the current reference maximum
    u32x4 pf[2];
    float tsum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const float rhm = rhn[st] - m;
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = __builtin_fmaf(sc[st][j], c2, rw[j] + rhm);
        sc[st][j] = x[j];
      }
      const uint32_t w0 = pack_f16(exp2_fast(x[0]), exp2_fast(x[1]));
      const uint32_t w1 = pack_f16(exp2_fast(x[2]), exp2_fast(x[3]));
      tsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w0), ones, tsum, false);
      tsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w1), ones, tsum, false);
      pf[st >> 1][2 * (st & 1)] = w0;
      pf[st >> 1][2 * (st & 1) + 1] = w1;
    }
    if constexpr (!kLast) load_rh(pn.kh);

    const bool grow = kFirst || !(tsum <= kGrowLimit);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      // Move the reference maximum: exact tile maximum per query (over the
      // four lane groups holding it), rescale O and l, recompute this tile's p.
      // (The empty volatile asm keeps this rare block a real branch.)
      __asm__ volatile("; reference maximum moves" ::);
      float mx = -__builtin_inff();
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = __builtin_fmaxf(mx, sc[st][j]);
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
      float inc;
      if (kFirst) {
        inc = mx;  // O and l are still zero: only set m
      } else {
        inc = __builtin_fmaxf(mx, 0.f);
        const float alpha = exp2_fast(-inc);
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
      }
      m += inc;
      tsum = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint32_t w0 = pack_f16(exp2_fast(sc[st][0] - inc), exp2_fast(sc[st][1] - inc));
        const uint32_t w1 = pack_f16(exp2_fast(sc[st][2] - inc), exp2_fast(sc[st][3] - inc));
        tsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w0), ones, tsum, false);
        tsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w1), ones, tsum, false);
        pf[st >> 1][2 * (st & 1)] = w0;
        pf[st >> 1][2 * (st & 1) + 1] = w1;
      }
    }
    l += tsum;

    pv(vslot, pf);

    // tile t+2 -> K slot (t+2)%2, V slot (t+2)%3; start the loads of tile t+3
    const int vslot2 = (vslot == 0) ? 2 : vslot - 1;  // (t+2) % 3
    // K slot t%2 held tile t, read by Q.K^T(t) in the previous step (or, for
    // t = 0, in the prologue, which no barrier separates from this store).
    if constexpr (kFirst) __syncthreads();
    if (t + 2 < T) store_tile(t & 1, vslot2);
    if (t + 3 < T) load_tile(pl);
    __syncthreads();
    pl = next_tile(pl, H);
    pc = pn;
    vslot = (vslot == 2) ? 0 : vslot + 1;
  };

  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;
  if (T == 1) {
    step(0, True{}, True{}, sA, sB);
  } else {
    step(0, True{}, False{}, sA, sB);
    int t = 1;
    for (; t + 2 < T; t += 2) {
      step(t, False{}, False{}, sB, sA);
      step(t + 1, False{}, False{}, sA, sB);
    }
    if (t + 2 == T) {
      step(t, False{}, False{}, sB, sA);
      step(t + 1, False{}, True{}, sA, sB);
    } else {
      step(t, False{}, True{}, sB, sA);
    }
  }

  // ---- epilogue: sum l over the four lane groups, normalise, store --------
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (qi < N) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int d = 16 * dt + 4 * grp;
      const f32x4 o4 = acc[dt] * inv;
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

template <bool BF16, bool OUT_F32, bool FUSED>
hipError_t launch16(const AttnArgs& a, hipStream_t stream) {
  auto kern = attn16_kernel<BF16, OUT_F32, FUSED>;
  const size_t lds = FUSED ? attn_fused16_lds_bytes(a.H, a.W) : attn16_lds_bytes();
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (err != hipSuccess) return err;
  constexpr int BM = 16 * NW;
  const int q_tiles = (a.H * a.W + BM - 1) / BM;
  dim3 grid(static_cast<unsigned>(q_tiles * a.BH));
  const uint32_t mh = (65536u + a.H - 1) / a.H, mw = (65536u + a.W - 1) / a.W;
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.rel_h, a.rel_w, a.out,
                     static_cast<const uint16_t*>(a.th), static_cast<const uint16_t*>(a.tw),
                     a.H, a.W, q_tiles, a.scale * kLog2e, mh, mw);
  return hipGetLastError();
}

}  // namespace

size_t attn16_lds_bytes() { return static_cast<size_t>(kKSlots16 + kVSlots16) * kTileHalves * 2; }

size_t attn_fused16_lds_bytes(int H, int W) {
  return attn16_lds_bytes() + static_cast<size_t>(16 * NW) * (H + W) * 4;
}

bool attn_fused16_ok(int H, int W) {
  const int T = ((H + kTileRows - 1) / kTileRows) * ((W + kTileCols - 1) / kTileCols);
  return H <= 32 && W <= 32 && T <= 4;
}

hipError_t launch_attn16(const AttnArgs& a, hipStream_t stream) {
  if (a.bf16) {
    return a.out_f32 ? launch16<true, true, false>(a, stream) : launch16<true, false, false>(a, stream);
  }
  return a.out_f32 ? launch16<false, true, false>(a, stream) : launch16<false, false, false>(a, stream);
}

hipError_t launch_attn_fused16(const AttnArgs& a, hipStream_t stream) {
  if (a.bf16) {
    return a.out_f32 ? launch16<true, true, true>(a, stream) : launch16<true, false, true>(a, stream);
  }
  return a.out_f32 ? launch16<false, true, true>(a, stream) : launch16<false, false, true>(a, stream);
}

}  // namespace relpos
