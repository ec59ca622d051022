// relpos_attn_fwd kernel: attention over an H x W token grid with the decomposed
// relative-position bias added per tile (PR #55629 page, implementation section,
// item 1: K/V streamed with an online softmax, the bias slices loaded per key
// block, no dense [N, N] bias).
//
// Work layout
//   * A unit is BM = 32*NW consecutive queries of one (batch, head); each of a
//     workgroup's NW waves owns 32 of them.  Either one workgroup per unit
//     takes all of the unit's key tiles, or (key-range split, SplitPlan) a
//     persistent grid of one workgroup per CU runs whole rounds of units and
//     cuts the units of the last round at one key tile into a head and a
//     tail on different workgroups, merged afterwards by split_merge_kernel.
//   * Bias sources: the rel_h/rel_w tensors written by relpos_build (rel_h
//     rows copied to LDS per segment when they fit beside the ring), or, in
//     the fused launch, rows computed per segment from q and the tables
//     (fused_bias_rows: rel_h to LDS when it fits, rel_w to a workspace slot).
//   * Keys are visited in 2-D tiles of the key grid: 4 grid rows x 16 grid
//     columns = 64 keys, in column bands (kw0 outer, kh0 inner).  Key o
//     (0..63) of a tile is grid cell (kh0 + o/16, kw0 + o%16); cells outside
//     the grid are masked with a -inf bias.
//   * Scores are computed transposed, S^T = K * Q^T, on 32x32x16 MFMA: a lane
//     holds one query (lane%32) and 32 of the tile's keys,
//     o = 32*st + 8*g + 4*(lane/32) + e, i.e. grid offsets r = 2*st + g/2 and
//     c = 8*(g%2) + 4*(lane/32) + e.  Its bias therefore needs 8 rel_w values
//     per column band, which initialise the first Q.K^T MFMA's accumulator,
//     and 4 rel_h values per tile (prefetched one tile ahead).
//   * O^T += V^T * P^T, again 32x32x16 MFMA, with P in fp16.  V tiles are kept
//     row-major in LDS and read with the gfx950 transpose read
//     (ds_read_b64_tr_b16), which hands each lane four consecutive keys of one
//     V column.  bf16 V is converted to fp16 while staging (exact for
//     |v| < 65520).
//
// Pipeline (one barrier per tile)
//   * K/V tiles live in a 4-slot LDS ring.  In step t a wave issues, in one
//     basic block, the Q.K^T MFMAs of tile t+1 (slot (t+1)%4), the softmax of
//     tile t and the P.V MFMAs of tile t-1 (slot (t-1)%4), interleaved so the
//     matrix cores run while the VALU does exp/convert work.  Then it stores
//     the registers holding tile t+2 into slot (t+2)%4 and starts the global
//     loads of tile t+3.  The loop is unrolled by two with the S and P register
//     sets swapping roles, so no copies are made between steps, and by four
//     where registers allow (every LDS slot offset then a constant).
//
// Online softmax (exp2 domain, scores pre-multiplied by log2 e)
//   * Each query row keeps a reference maximum m.  Per tile,
//     p = exp2(fma(s + rel_w*log2e/c2, c2, rel_h*log2e - m)) with c2 =
//     scale*log2e; the fp16 values of p are summed (v_dot2) into l and fed to
//     the P.V MFMA.
//   * m is only moved when it must be: on the first tile (exact tile maximum),
//     and when some p of a tile exceeds 2^15, detected from the per-lane sum of
//     the rounded p.  Then the tile's true maximum is taken, O and l are
//     rescaled by exp2(m_old - m_new), and the tile's p are recomputed.  Between
//     such events no rescale of O is needed; p stays <= 2^15 (finite in fp16)
//     and the row's first maximum keeps l >= 1.
#include <algorithm>
#include <type_traits>

#include "relpos_attn_common.hpp"
#include "relpos_kernels.hpp"

namespace relpos {

namespace {

using namespace attn;

// LDS row of a V tile.  8-wave workgroups (one per CU) use 96 halves (48
// dwords): the four rows a 16-lane group of the transpose read touches then
// start 0, 16, 32 and 48 banks apart and two such groups (32 lanes) cover the
// 64 banks once; with K's 72 halves the second group's rows fall on the first
// group's banks.  Smaller workgroups keep 72 halves so that two of them still
// fit a CU's LDS.
// The plain launches copy a unit's rel_h rows to LDS with at most this many
// 16-byte chunks per lane: 32 rows x H/4 chunks over 64 lanes, so H <= 72.
constexpr int kRhLdsMaxChunks = 9;
constexpr int kRhLdsMaxH = kRhLdsMaxChunks * 64 * 4 / 32;

template <int NW>
constexpr int v_stride() {
  return NW >= 8 ? 96 : kKStride;
}
template <int NW>
constexpr size_t attn32_lds_bytes() {
  return kSlots * static_cast<size_t>(kTileKeys) * (kKStride + v_stride<NW>()) * 2;
}
// LDS of the fused launch's rel_h rows: 256 queries x (rows padded to whole
// tiles + 4) floats.
inline size_t fused_rh_lds_bytes(int H) {
  return 256 * static_cast<size_t>((H + kTileRows - 1) / kTileRows * kTileRows + 4) * sizeof(float);
}

// ---- bias computed in the attention kernel ----------------------------------
// One axis of the bias for the 32 queries of a wave: out[j][x] = q_j . T[a_j + L
// - 1 - x] for x in [0, L), with a_j the query's coordinate along the axis
// (qh for rel_h, qw for rel_w) and T the table of 2L - 1 rows (PR #55629 page,
// key source snippet: add_decomposed_rel_pos on the unscaled q).  The products
// C[j][r] = q_j . T[r] are taken on MFMA for 32 table rows at a time over the
// rows [r_lo, r_hi] the wave's queries use, with A = the wave's Q fragments and
// B = T^T; a lane then holds table row r for 16 queries and writes each value
// to its diagonal position x = a_j + L - 1 - r.  For one query the 32 lanes of
// a half write 32 consecutive floats.  Stores outside [0, L) are dropped by the
// buffer range check (offset kOob), or skipped when the rows are in LDS.
//
// The queries' coordinates: query j_i = 8*(i/4) + 4*half + i%4 (the row of
// result register i) is gq0 + min(j_i, jmax) with grid column t = qw0 + min(j_i,
// jmax) < W + 32 past the wave's first grid row qh0; floor(t / W) is exact from
// the float product (the quotient is at least 0.5/W from the next integer).
template <bool BF16, bool AXIS_W, bool TO_LDS>
__device__ __forceinline__ void bias_axis(const u32x4 (&qf)[4], const uint16_t* __restrict__ tab, int L,
                                          int qh0, int qw0, int jmax, int W, float rcp_w, int r_lo, int r_hi,
                                          float* dst, int Ls, int lane) {
  // The empty asm makes the lane index opaque, so the per-register offsets
  // below are recomputed here rather than hoisted out of the workgroup's
  // loop over segments (where they would only take registers from it).
  __asm__ volatile("" : "+v"(lane));
  const int half = lane >> 5;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(dst, static_cast<uint32_t>(32 * Ls) * 4);
  int xa[16];  // a_i + L - 1: the position x of table row r = 0
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int j = 8 * (i >> 2) + 4 * half + (i & 3);
    const int t = qw0 + (j < jmax ? j : jmax);
    const int d = static_cast<int>((static_cast<float>(t) + 0.5f) * rcp_w);
    xa[i] = (AXIS_W ? t - d * W : qh0 + d) + L - 1;
  }
  auto load_rows = [&](int rb, u32x4 (&tf)[4]) {
    const int r = rb + (lane & 31);
    const bool ok = r <= 2 * L - 2;
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) {
      tf[kd] = ok ? *reinterpret_cast<const u32x4*>(tab + static_cast<size_t>(r) * kD + 16 * kd + 8 * half)
                  : u32x4{0, 0, 0, 0};
    }
  };
  u32x4 tf[4], tn[4];
  load_rows(r_lo, tf);
  for (int rb = r_lo; rb <= r_hi; rb += 32) {
    const int r = rb + (lane & 31);
    if (rb + 32 <= r_hi) load_rows(rb + 32, tn);  // the next block's rows load under this block's work
    f32x16 c = {};
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) c = mfma32<BF16>(qf[kd], tf[kd], c);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int x = xa[i] - r;
      const int row = 8 * (i >> 2) + 4 * half + (i & 3);
      if constexpr (TO_LDS) {
        if (static_cast<unsigned>(x) < static_cast<unsigned>(L)) dst[row * Ls + x] = c[i];
      } else {
        const int off = static_cast<unsigned>(x) < static_cast<unsigned>(L) ? 4 * (row * Ls + x) : kOob;
        __builtin_amdgcn_raw_buffer_store_b32(as_uint(c[i]), rs, off, 0, 0);
      }
    }
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) tf[kd] = tn[kd];
  }
}

// rel_h and rel_w rows of the wave's 32 queries gq0 .. gq0+31 (clamped to the
// last query, so rows of queries past the grid hold finite copies), written to
// sh[j][0..H) and sw[j][kw_lo..W) with row strides hstride and Ws; the columns
// [H, Hs) and [W, Ws) are set to -inf (keys outside the grid).  rel_w columns
// below kw_lo (key columns a segment starting past them never visits) are left
// unwritten.  RH_LDS: sh is in LDS.  gq0 is wave-uniform.
template <bool BF16, bool RH_LDS>
__device__ __forceinline__ void fused_bias_rows(const u32x4 (&qf)[4], const uint16_t* __restrict__ th,
                                                const uint16_t* __restrict__ tw, float* sh, float* sw,
                                                int H, int W, int Hs, int hstride, int Ws, int gq0, int N,
                                                int kw_lo, int lane) {
  const int half = lane >> 5;
  const int ga = gq0 < N - 1 ? gq0 : N - 1;
  const int gb = gq0 + 31 < N - 1 ? gq0 + 31 : N - 1;
  const int qh0 = ga / W, qw0 = ga - qh0 * W;
  const int qh1 = gb / W, qw1 = gb - qh1 * W;
  const float rcp_w = 1.0f / static_cast<float>(W);
  bias_axis<BF16, false, RH_LDS>(qf, th, H, qh0, qw0, gb - ga, W, rcp_w, qh0, qh1 + H - 1, sh, hstride, lane);
  // A wave that wraps to a new grid row holds every qw.  Columns x >= kw_lo
  // need table rows r = qw + W - 1 - x <= max qw + W - 1 - kw_lo.
  const int rw_lo = qh0 == qh1 ? qw0 : 0, rw_hi = (qh0 == qh1 ? qw1 : W - 1) + W - 1 - kw_lo;
  bias_axis<BF16, true, false>(qf, tw, W, qh0, qw0, gb - ga, W, rcp_w, rw_lo, rw_hi, sw, Ws, lane);
  const int j = lane & 31;
  for (int p = H + half; p < Hs; p += 2) sh[j * hstride + p] = -__builtin_inff();
  for (int p = W + half; p < Ws; p += 2) sw[j * Ws + p] = -__builtin_inff();
}

// A piece: a workgroup's partial result for one unit -- O / l in fp16 (BM x
// 64 halves, in the first half of the BM x 64 floats the slot reserves), then
// the reference maximum m and the row sum l of each query (fp32).  O / l is a
// weighted mean of V rows, so it is within V's fp16 range; the merge takes a
// convex combination of the two pieces' O / l, so their fp16 rounding (2^-11
// relative) bounds its error.  Unit i of the split last round keeps its head in
// slot 2i, its tail in 2i+1.
template <int BM>
constexpr int64_t piece_floats() {
  return static_cast<int64_t>(BM) * kD + 2 * BM;
}

// Floats of one query's bias rows when computed in the kernel: rel_h padded
// to whole 4-row tiles, rel_w to whole 16-column tiles.
__host__ __device__ constexpr int fused_row_floats(int H, int W) {
  return (H + kTileRows - 1) / kTileRows * kTileRows + (W + kTileCols - 1) / kTileCols * kTileCols;
}

// One segment: tiles [t0, t0 + nt) of unit `unit`.  A full segment (nt == T)
// writes the normalised output; otherwise the segment is one piece of a split
// unit (see SplitPlan), written to workspace slot `slot`.  FUSED: the bias rows
// are computed from q and the tables th/tw into `bias_slot` (the workgroup's
// BM * (Hs + Ws) floats) instead of being read from rel_h/rel_w.  RH_LDS: the
// unit's rel_h rows live in LDS after the K/V ring (row stride Hs + 4 floats,
// so the 16-byte reads of 16 lanes cover the 64 banks once): computed there
// when FUSED, else copied there from rel_h once per segment (tile-aligned
// grids only, whose rows are 16-byte aligned).
template <bool BF16, bool OUT_F32, int NW, bool ALIGNED, bool SPLIT, bool FUSED, bool RH_LDS = false>
__device__ __forceinline__ void attn_segment(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ rel_h,
    const float* __restrict__ rel_w, void* __restrict__ out,
    int H, int W, int q_tiles, float c2, float rw_mul, bool zero_q,
    float* __restrict__ ws, int unit, int t0, int nt, int slot,
    const uint16_t* __restrict__ th, const uint16_t* __restrict__ tw, float* bias_slot) {
  constexpr int BM = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int kVStride = v_stride<NW>();
  constexpr int kVTileHalves = kTileKeys * kVStride;
  const int N = H * W;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);  // [kSlots][64][kKStride]
  uint16_t* Vs = Ks + kSlots * kTileHalves;          // [kSlots][64][kVStride]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;

  const int bh = unit / q_tiles;
  const int q0 = (unit - bh * q_tiles) * BM;
  const size_t head = static_cast<size_t>(bh) * N;

  // ---- this lane's query: Q^T operand fragments (4 k-steps of 16) ----------
  const int qi = q0 + wave * 32 + (lane & 31);
  const bool qok = qi < N;
  u32x4 qf[4];
#pragma unroll
  for (int kd = 0; kd < 4; ++kd) {
    qf[kd] = qok ? *reinterpret_cast<const u32x4*>(q + (head + qi) * kD + 16 * kd + 8 * half)
                 : u32x4{0, 0, 0, 0};
  }

  const int T = nt;  // tiles of this segment

  // ---- K/V tile staging: global -> registers -> LDS (row-major, 16 B chunks)
  constexpr int CH = (kTileKeys * kD / 8) / NT;  // 16-byte chunks of K (and of V) per thread
  static_assert(CH >= 1, "workgroup too large for one tile");
  int ch_r[CH], ch_c[CH], ch_voff[CH], ch_lds[CH], ch_vlds[CH];
#pragma unroll
  for (int s = 0; s < CH; ++s) {
    const int cid = tid + s * NT;
    const int o = cid >> 3, dc = cid & 7;
    ch_r[s] = o >> 4;
    ch_c[s] = o & 15;
    ch_voff[s] = ((o >> 4) * W + (o & 15)) * (kD * 2) + 16 * dc;  // bytes from the tile origin
    ch_lds[s] = o * kKStride + 8 * dc;
    ch_vlds[s] = o * kVStride + 8 * dc;
  }
  u32x4 kreg[CH], vreg[CH];
  const uint32_t head_bytes = static_cast<uint32_t>(N) * kD * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + head * kD, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + head * kD, head_bytes);

  auto load_tile = [&](TilePos p) {
    if constexpr (ALIGNED) {
      // Every cell of a tile lies in the grid; the tile origin goes in the
      // scalar offset.  Past the last tile (kw >= W) tile 0 is re-read: the
      // slot it is stored to is never read again.
      const int org = (p.kw < W ? p.kh * W + p.kw : 0) * (kD * 2);
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        kreg[s] = buf_load16(krs, ch_voff[s], org);
        vreg[s] = buf_load16(vrs, ch_voff[s], org);
      }
    } else {
      const int org = (p.kh * W + p.kw) * (kD * 2);
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        const bool ok = (p.kh + ch_r[s] < H) && (p.kw + ch_c[s] < W);
        const int off = ok ? org + ch_voff[s] : kOob;
        kreg[s] = buf_load16(krs, off);
        vreg[s] = buf_load16(vrs, off);
      }
    }
  };
  auto store_tile = [&](int slot) {
    uint16_t* kb = Ks + slot * kTileHalves;
    uint16_t* vb = Vs + slot * kVTileHalves;
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      *reinterpret_cast<u32x4*>(kb + ch_lds[s]) = kreg[s];
      u32x4 x = vreg[s];
      if constexpr (BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) x[w] = pack_f16(bf16_lo(x[w]), bf16_hi(x[w]));
      }
      *reinterpret_cast<u32x4*>(vb + ch_vlds[s]) = x;
    }
  };

  // ---- bias ------------------------------------------------------------------
  // rel_w enters through the Q.K^T MFMA: the first MFMA of each 32-key half
  // accumulates onto rwc, which holds rel_w * log2(e) / c2 for the key column
  // of each accumulator register (the same 8 columns repeat in both halves and
  // in both grid rows of a half), so after the multiply by c2 below the score
  // already carries its rel_w term.  rel_h (4 grid rows per tile) is
  // prefetched one tile ahead and added with the running maximum in one fma.
  // The unit's bias rows (queries q0 .. q0+BM-1) have row strides hs and wst
  // floats.  They are padded (whole tiles, 16-byte rows) when the grid is
  // tile-aligned or when they are computed here (-inf columns past the grid):
  // then each load is one 16-byte load without a mask.
  constexpr bool kPadded = FUSED || ALIGNED;
  int hs = H, wst = W;
  const float* rh_rows;
  const float* rw_rows;
  int rows;
  if constexpr (FUSED) {
    hs = (H + kTileRows - 1) / kTileRows * kTileRows;
    wst = (W + kTileCols - 1) / kTileCols * kTileCols;
    rh_rows = bias_slot;
    rw_rows = bias_slot + BM * hs;
    rows = BM;
  } else {
    rh_rows = rel_h + (head + q0) * H;
    rw_rows = rel_w + (head + q0) * W;
    rows = N - q0 < BM ? N - q0 : BM;
  }
  const __amdgpu_buffer_rsrc_t rwrs = make_rsrc(rw_rows, static_cast<uint32_t>(rows * wst) * 4);
  const __amdgpu_buffer_rsrc_t rhrs = make_rsrc(rh_rows, static_cast<uint32_t>(rows * hs) * 4);
  const int ql = wave * 32 + (lane & 31);  // query within the unit
  const int qrow = FUSED || qok ? ql : 0;
  const int rw_lane = (qrow * wst + 4 * half) * 4;  // bytes: this lane's row, column 4*half
  const int rh_lane = qrow * hs * 4;
  const int hs_l = hs + 4;  // LDS row stride of rel_h (RH_LDS)
  float* rh_lds = reinterpret_cast<float*>(smem + kSlots * static_cast<size_t>(kTileHalves + kVTileHalves) * 2);
  f32x16 rwc;
  auto load_band = [&](int kw0) {
    float x[8];
    if constexpr (kPadded) {
      const u32x4 a0 = buf_load16(rwrs, rw_lane, 4 * kw0);
      const u32x4 a1 = buf_load16(rwrs, rw_lane + 32, 4 * kw0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = as_float(a0[i]) * rw_mul;
        x[4 + i] = as_float(a1[i]) * rw_mul;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int dc = 8 * (i >> 2) + (i & 3);  // column offset beyond 4*half
        const int c = kw0 + dc + 4 * half;
        const float y = buf_loadf(rwrs, c < W ? rw_lane + 4 * (kw0 + dc) : kOob);
        // The mask is scaled with the values: rw_mul has the sign of the
        // scale, and the product with c2 below turns it back into -inf.
        x[i] = (c < W ? y : -__builtin_inff()) * rw_mul;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) rwc[r] = x[4 * ((r >> 2) & 1) + (r & 3)];
  };
  float rhn[4];  // rel_h of the next tile's 4 grid rows (-inf outside the grid)
  auto load_rh = [&](int kh0) {
    if constexpr (RH_LDS) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(rh_lds + ql * hs_l + kh0);
#pragma unroll
      for (int r = 0; r < 4; ++r) rhn[r] = a[r];
    } else if constexpr (kPadded) {
      const u32x4 a = buf_load16(rhrs, rh_lane, 4 * kh0);
#pragma unroll
      for (int r = 0; r < 4; ++r) rhn[r] = as_float(a[r]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float y = buf_loadf(rhrs, kh0 + r < H ? rh_lane + 4 * (kh0 + r) : kOob);
        rhn[r] = kh0 + r < H ? y : -__builtin_inff();
      }
    }
  };

  // ---- tile compute pieces -----------------------------------------------
  // S^T = K Q^T (+ rel_w term) for the tile in `slot`, two 32-key halves.
  auto qk = [&](int slot, f32x16 (&s)[2]) {
    const uint16_t* kb = Ks + slot * kTileHalves;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(kb + (32 * st + (lane & 31)) * kKStride + 16 * kd + 8 * half);
        s[st] = mfma32<BF16>(kf, qf[kd], kd == 0 ? rwc : s[st]);
      }
    }
  };
  // transpose-read lane addressing for the V^T operand
  const int grp = lane >> 4, jl = lane & 15;
  const int tr_row = 4 * (grp >> 1) + (jl >> 2);
  const int tr_col = 16 * (grp & 1) + 4 * (jl & 3);
  f32x16 acc[2];
  // O^T += V^T P^T for the tile in `slot`: four 16-key steps, two 32-row d tiles.
  auto pv = [&](int slot, const u32x4 (&pf)[4]) {
    const uint16_t* vb = Vs + slot * kVTileHalves;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const uint16_t* vp = vb + (16 * ks + tr_row) * kVStride + 32 * dt + tr_col;
        const u32x2 lo = ds_read_tr16(vp);
        const u32x2 hi = ds_read_tr16(vp + 8 * kVStride);
        const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
        acc[dt] = mfma32<false>(vf, pf[ks], acc[dt]);
      }
    }
  };

  // ---- prologue: the segment's tiles 0 and 1 in LDS, tile 2 in registers,
  // S of tile 0.  Tile t0 of the key walk (column bands of ceil(H/4) tiles).
  const int band_tiles = (H + kTileRows - 1) / kTileRows;
  const TilePos p0{(t0 % band_tiles) * kTileRows, (t0 / band_tiles) * kTileCols};
  const TilePos p1 = next_tile(p0, H);
  const TilePos p2 = next_tile(p1, H);
  if constexpr (!FUSED && RH_LDS) {
    static_assert(ALIGNED, "rel_h rows are copied in 16-byte chunks");
    // This wave's 32 rel_h rows, contiguous in memory: 16-byte chunk c = lane
    // + 64*j is row c / (H/4), chunk c % (H/4) of it; at most kRhLdsMaxChunks
    // per lane (H <= 72 on this path).  All loads are issued before the first
    // LDS store.  Rows past the grid get zeros (their outputs are not
    // written).  The wave reads back only its own rows.
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int row0 = q0 + wu * 32;
    const int cpr = H / 4;
    const int nch = (N - row0 < 32 ? N - row0 : 32) * cpr;  // chunks inside the grid (<= 0: none)
    // An opaque copy of the lane index keeps the per-chunk offsets from being
    // hoisted out of the persistent kernel's loop over segments, where they
    // would hold registers through the key loop.
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    const float* src = rel_h + (head + row0) * H;
    const float rcp = 1.0f / static_cast<float>(cpr);
    u32x4 x[kRhLdsMaxChunks];
#pragma unroll
    for (int j = 0; j < kRhLdsMaxChunks; ++j) {
      const int c = ln + 64 * j;
      x[j] = c < nch ? *reinterpret_cast<const u32x4*>(src + 4 * c) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < kRhLdsMaxChunks; ++j) {
      const int c = ln + 64 * j;
      // c / cpr from the float product: (c + 0.5) / cpr is at least 1/(2 cpr)
      // from the nearest integer, far more than the product's rounding error.
      const int row = static_cast<int>((static_cast<float>(c) + 0.5f) * rcp);
      if (c < 32 * cpr) *reinterpret_cast<u32x4*>(rh_lds + (wu * 32 + row) * hs_l + 4 * (c - row * cpr)) = x[j];
    }
  }
  if constexpr (FUSED) {
    load_tile(p0);
    // This wave's 32 bias rows; the wave reads back only its own rows, so
    // waiting for its stores (vmcnt also counts stores) is enough.
    const int wu = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: scalar addresses
    float* sh = RH_LDS ? rh_lds + wu * 32 * hs_l : bias_slot + wu * 32 * hs;
    fused_bias_rows<BF16, RH_LDS>(qf, th, tw, sh, bias_slot + BM * hs + wu * 32 * wst, H, W, hs,
                                  RH_LDS ? hs_l : hs, wst, q0 + wu * 32, N, p0.kw, lane);
    store_tile(0);
    load_tile(p1);
    store_tile(1);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    load_band(p0.kw);
    load_tile(p2);
    load_rh(p0.kh);
  } else {
    load_band(p0.kw);
    load_tile(p0);
    store_tile(0);
    load_tile(p1);  // tiles past the segment's last one are staged too and never used
    store_tile(1);
    load_tile(p2);
    load_rh(p0.kh);
  }
  __syncthreads();

  acc[0] = f32x16{};
  acc[1] = f32x16{};
  float m = 0.f, l = 0.f;
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

  // scale == 0: the scores are the bias alone.  The launch then passes c2 =
  // log2(e) and rw_mul = 1 and the q.k products are taken against zero Q
  // fragments (after the fused bias rows, which need the real q).
  if (zero_q) {
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) qf[kd] = u32x4{0, 0, 0, 0};
  }

  f32x16 sA[2], sB[2];
  u32x4 pA[4], pB[4];
  qk(0, sA);

  TilePos pc = p0;                // tile t
  TilePos pl = next_tile(p2, H);  // tile t+3, the next one to load

  // One pipeline step for tile t: Q.K^T of tile t+1 (into sn), softmax of
  // tile t (sc -> pcur) and P.V of tile t-1 (pprev), all in one basic block so
  // the MFMA and VALU streams interleave; then the rare maximum move, the
  // staging of tile t+2 and one barrier.  The last step also multiplies the
  // slot after the last tile (data staged from outside the grid) and drops
  // the result: one code path for every step keeps register pressure low.
  auto step = [&](int t, auto first_c, f32x16 (&sc)[2], f32x16 (&sn)[2],
                  u32x4 (&pprev)[4], u32x4 (&pcur)[4]) {
    constexpr bool kFirst = decltype(first_c)::value;
    const TilePos pn = next_tile(pc, H);
    if (pn.kh == 0 && pn.kw < W) load_band(pn.kw);  // tile t+1 opens a new column band

    // Operands of this step's MFMAs: K^T fragments of tile t+1 and V^T
    // fragments of tile t-1, read from LDS two chunks ahead of their use.
    const uint16_t* kb = Ks + ((t + 1) & (kSlots - 1)) * kTileHalves;
    const uint16_t* vb = Vs + ((t - 1) & (kSlots - 1)) * kVTileHalves;
    auto read_k = [&](int i) -> u32x4 {
      const int st = i & 1, kd = i >> 1;
      return *reinterpret_cast<const u32x4*>(kb + (32 * st + (lane & 31)) * kKStride + 16 * kd + 8 * half);
    };
    auto read_v = [&](int i) -> u32x4 {
      const int dt = i & 1, ks = i >> 1;
      const uint16_t* vp = vb + (16 * ks + tr_row) * kVStride + 32 * dt + tr_col;
      const u32x2 lo = ds_read_tr16(vp);
      const u32x2 hi = ds_read_tr16(vp + 8 * kVStride);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 kf[8], vf[8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      kf[i] = read_k(i);
      if constexpr (!kFirst) vf[i] = read_v(i);
    }
    __builtin_amdgcn_sched_barrier(0);

    // Eight chunks, each: one Q.K^T MFMA of tile t+1, one P.V MFMA of tile
    // t-1 and the softmax of four of tile t's scores.  The fences keep this
    // order so the matrix cores run under the VALU work.
    float tsum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i + 2 < 8) {
        kf[i + 2] = read_k(i + 2);
        if constexpr (!kFirst) vf[i + 2] = read_v(i + 2);
      }
      {
        const int st = i & 1, kd = i >> 1;
        sn[st] = mfma32<BF16>(kf[i], qf[kd], kd == 0 ? rwc : sn[st]);
      }
      if constexpr (!kFirst) {
        const int dt = i & 1, ks = i >> 1;
        acc[dt] = mfma32<false>(vf[i], pprev[ks], acc[dt]);
      }
      // scores 4*i .. 4*i+3 of the lane: st = i/4, g = i%4, grid row 2*st + g/2
      const int st = i >> 2, g = i & 3;
      const float rhm = __builtin_fmaf(rhn[2 * st + (g >> 1)], kLog2e, -m);
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = __builtin_fmaf(sc[st][4 * g + e], c2, rhm);
        sc[st][4 * g + e] = x[e];
      }
      const uint32_t w0 = pack_f16(exp2_fast(x[0]), exp2_fast(x[1]));
      const uint32_t w1 = pack_f16(exp2_fast(x[2]), exp2_fast(x[3]));
      tsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w0), ones, tsum, false);
      tsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w1), ones, tsum, false);
      // registers 8*gg + 2*j of S half st map to P operand (2*st + gg), word j
      pcur[2 * st + (g >> 1)][2 * (g & 1)] = w0;
      pcur[2 * st + (g >> 1)][2 * (g & 1) + 1] = w1;
      if ((i + 1) % chunks_per_fence<NW>() == 0) __builtin_amdgcn_sched_barrier(0);
    }
    load_rh(pn.kh);  // rel_h of tile t+1 (this tile's values are used); row 0 past the grid

    // tile t+2: registers -> LDS slot (t+2)%4 (last read in iteration t-1);
    // then start the global loads of tile t+3.  Both run unconditionally so the
    // step stays one basic block (a branch here lets the compiler sink the
    // softmax below it, away from the MFMAs): past the last tile the slot
    // written is never read again.
    store_tile((t + 2) & (kSlots - 1));
    load_tile(pl);
    const bool grow = kFirst || !(tsum <= kGrowLimit);

    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      // Move the reference maximum: exact tile maximum per query, then
      // rescale O (which already holds tiles < t) and l, and recompute this
      // tile's p against the new m.  (The empty volatile asm keeps this rare
      // block a real branch instead of code speculated on every tile.)
      __asm__ volatile("; reference maximum moves" ::);
      float mx = -__builtin_inff();
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sc[st][r]);
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
      float inc;
      if (kFirst) {
        inc = mx;  // O and l are still zero: only set m
      } else {
        inc = __builtin_fmaxf(mx, 0.f);
        const float alpha = exp2_fast(-inc);
        l *= alpha;
        acc[0] *= alpha;
        acc[1] *= alpha;
      }
      m += inc;
      float ts = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          uint32_t w4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            w4[i] = pack_f16(exp2_fast(sc[st][8 * gg + 2 * i] - inc),
                             exp2_fast(sc[st][8 * gg + 2 * i + 1] - inc));
            ts = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w4[i]), ones, ts, false);
          }
          pcur[2 * st + gg] = u32x4{w4[0], w4[1], w4[2], w4[3]};
        }
      }
      tsum = ts;
    }
    l += tsum;

    __syncthreads();
    pl = next_tile(pl, H);
    pc = pn;
  };

  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;
  const int slot_last = (T - 1) & (kSlots - 1);
  step(0, True{}, sA, sB, pB, pA);
  int t = 1;
  if constexpr (!SPLIT || (ALIGNED && !FUSED)) {
    // Unrolled by four: with t = 1 (mod 4) at each iteration every LDS slot
    // of the four steps is a compile-time offset (no per-step address
    // arithmetic; 64x64: 74.3 -> 71.2 us).  The persistent kernels on ragged
    // grids and the fused kernels keep the two-step loop: unrolled by four
    // they spill registers (in the key loop, resp. 2-4 outside it).
    for (; t + 3 < T; t += 4) {
      step(t, False{}, sB, sA, pA, pB);
      step(t + 1, False{}, sA, sB, pB, pA);
      step(t + 2, False{}, sB, sA, pA, pB);
      step(t + 3, False{}, sA, sB, pB, pA);
    }
  }
  for (; t + 1 < T; t += 2) {
    step(t, False{}, sB, sA, pA, pB);
    step(t + 1, False{}, sA, sB, pB, pA);
  }
  if (t < T) {  // an even number of tiles: one step left
    step(t, False{}, sB, sA, pA, pB);
    pv(slot_last, pB);
  } else {
    pv(slot_last, pA);
  }

  // ---- epilogue: combine the two lane halves' row sums, normalise, store ----
  const float lt = l + __shfl_xor(l, 32);
  float inv = 1.0f / lt;
  if constexpr (SPLIT) {
    const int unit_tiles = band_tiles * ((W + kTileCols - 1) / kTileCols);
    if (nt != unit_tiles) {
      // One piece of a split unit: O / l (fp16), m and l go to the
      // workspace; split_merge_kernel combines the pieces after this launch.
      float* pw = ws + static_cast<int64_t>(slot) * piece_floats<BM>();
      uint16_t* po = reinterpret_cast<uint16_t*>(pw);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * dt + 8 * g + 4 * half;
          *reinterpret_cast<u32x2*>(po + ql * kD + d) =
              u32x2{pack_f16(acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv),
                    pack_f16(acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv)};
        }
      if (half == 0) {
        pw[BM * kD + ql] = m;
        pw[BM * kD + BM + ql] = lt;
      }
      return;
    }
  }
  if (!qok) return;
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

// Without SPLIT: one workgroup per unit, all of its tiles.  With SPLIT: a
// persistent grid following SplitPlan: full rounds of units, then the split
// last round.

// Merges the head and tail pieces of each unit of the split last round (head
// first, so results are reproducible) and writes the normalised output.
// Sixteen workgroups per unit, one thread per (query, 4-float chunk of d).
template <bool BF16, bool OUT_F32>
__global__ __launch_bounds__(256) void split_merge_kernel(const float* __restrict__ ws, void* __restrict__ out,
                                                          int N, int q_tiles, int first_unit) {
  constexpr int BM = 256;
  const int ui = blockIdx.x >> 4;  // unit of the last round
  const int unit = first_unit + ui;
  const int it = ((blockIdx.x & 15) << 8) + threadIdx.x;  // 0 .. 4095
  const int ql = it >> 4, c = 4 * (it & 15);
  const int bh = unit / q_tiles;
  const int qi = (unit - bh * q_tiles) * BM + ql;
  if (qi >= N) return;
  const float* ph = ws + (2 * static_cast<int64_t>(ui)) * piece_floats<BM>();
  const float* pt = ph + piece_floats<BM>();
  const float mh = ph[BM * kD + ql], mt = pt[BM * kD + ql];
  const float lh = ph[BM * kD + BM + ql], lt = pt[BM * kD + BM + ql];
  const u32x2 xh = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(ph) + ql * kD + c);
  const u32x2 xt = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(pt) + ql * kD + c);
  const float mx = __builtin_fmaxf(mh, mt);
  // The pieces' weights: l * exp2(m - max), normalised to sum to one.
  const float wh0 = lh * exp2_fast(mh - mx), wt0 = lt * exp2_fast(mt - mx);
  const float inv = 1.0f / (wh0 + wt0);
  const float wh = wh0 * inv, wt = wt0 * inv;
  f32x4 o4;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const f32x2 a = unpack_f16(xh[e]);
    const f32x2 b = unpack_f16(xt[e]);
    o4[2 * e] = a[0] * wh + b[0] * wt;
    o4[2 * e + 1] = a[1] * wh + b[1] * wt;
  }
  const size_t row = static_cast<size_t>(bh) * N + qi;
  if constexpr (OUT_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + row * kD + c) = o4;
  } else {
    const u32x2 pk = BF16 ? u32x2{pack_bf16(o4[0], o4[1]), pack_bf16(o4[2], o4[3])}
                          : u32x2{pack_f16(o4[0], o4[1]), pack_f16(o4[2], o4[3])};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + row * kD + c) = pk;
  }
}

// FUSED (always with SPLIT): the bias is computed per segment from q and the
// tables th/tw; workgroup b keeps its bias rows in the workspace after the
// 2 * P split pieces, at bias slot b.
template <bool BF16, bool OUT_F32, int NW, bool ALIGNED, bool SPLIT, bool FUSED, bool RH_LDS>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ rel_h,
    const float* __restrict__ rel_w, void* __restrict__ out,
    int H, int W, int q_tiles, float c2, float rw_mul, int zero_q,
    float* __restrict__ ws, SplitPlan plan,
    const uint16_t* __restrict__ th, const uint16_t* __restrict__ tw) {
  static_assert(!FUSED || SPLIT, "the fused bias needs the persistent grid");
  constexpr int BM = 32 * NW;
  const int T = ((W + kTileCols - 1) / kTileCols) * ((H + kTileRows - 1) / kTileRows);
  const int L = xcd_work_index(static_cast<int>(gridDim.x));
  float* bias_slot = nullptr;
  if constexpr (FUSED) {
    const int64_t slot_floats = static_cast<int64_t>(BM) * (fused_row_floats(H, W));
    bias_slot = ws + 2 * static_cast<int64_t>(gridDim.x) * piece_floats<BM>() + blockIdx.x * slot_floats;
  }
  if constexpr (!SPLIT) {
    attn_segment<BF16, OUT_F32, NW, ALIGNED, false, false, RH_LDS>(q, k, v, rel_h, rel_w, out, H, W, q_tiles, c2,
                                                           rw_mul, zero_q != 0, ws, L, 0, T, 0, th, tw, bias_slot);
  } else {
    const int P = static_cast<int>(gridDim.x);
    for (int i = 0; i < plan.rounds; ++i) {
      attn_segment<BF16, OUT_F32, NW, ALIGNED, true, FUSED, RH_LDS>(q, k, v, rel_h, rel_w, out, H, W, q_tiles, c2,
                                                            rw_mul, zero_q != 0, ws, i * P + L, 0, T, 0, th, tw, bias_slot);
      __syncthreads();  // the next segment reuses the LDS ring
    }
    const int base = plan.rounds * P;
    if (L < plan.rest) {
      attn_segment<BF16, OUT_F32, NW, ALIGNED, true, FUSED, RH_LDS>(q, k, v, rel_h, rel_w, out, H, W, q_tiles, c2,
                                                            rw_mul, zero_q != 0, ws, base + L, 0, plan.s, 2 * L, th, tw,
                                                            bias_slot);
    } else if (plan.s < T) {
      for (int j = 0; j < plan.k; ++j) {
        const int ui = (L - plan.rest) * plan.k + j;
        if (ui >= plan.rest) break;
        attn_segment<BF16, OUT_F32, NW, ALIGNED, true, FUSED, RH_LDS>(q, k, v, rel_h, rel_w, out, H, W, q_tiles, c2,
                                                              rw_mul, zero_q != 0, ws, base + ui, plan.s, T - plan.s,
                                                              2 * ui + 1, th, tw, bias_slot);
        __syncthreads();
      }
    }
  }
}

// Split workspace: two piece slots per workgroup.
int64_t split_piece_bytes(int ctas) {
  return 2 * static_cast<int64_t>(ctas) * piece_floats<256>() * static_cast<int64_t>(sizeof(float));
}

template <bool BF16, bool OUT_F32, int NW, bool ALIGNED, bool SPLIT, bool FUSED = false, bool RH_LDS = false>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t stream) {
  const size_t lds = attn32_lds_bytes<NW>() + (RH_LDS ? fused_rh_lds_bytes(a.H) : 0);
  auto kern = attn_fwd_kernel<BF16, OUT_F32, NW, ALIGNED, SPLIT, FUSED, RH_LDS>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (err != hipSuccess) return err;
  constexpr int BM = 32 * NW;
  const int q_tiles = (a.H * a.W + BM - 1) / BM;
  const int64_t units = static_cast<int64_t>(q_tiles) * a.BH;
  const int64_t T = static_cast<int64_t>((a.W + kTileCols - 1) / kTileCols) * ((a.H + kTileRows - 1) / kTileRows);
  float* ws = nullptr;
  unsigned grid = static_cast<unsigned>(units);
  SplitPlan plan{};
  if constexpr (SPLIT) {
    ws = static_cast<float*>(a.ws);
    const int pro = FUSED ? kFusedPrologueTiles : kSplitSegmentTiles;
    plan = split_plan(units, static_cast<int>(T), a.split_ctas, pro);
    if (FUSED && plan.rest > 0 && plan.s < T) {
      // The fused launch has no unsplit alternative: keep the last round
      // whole when its split would not be faster (many tails per CU).
      const int64_t last = std::max<int64_t>(plan.s + pro, static_cast<int64_t>(plan.k) * (T - plan.s + pro));
      if (last + kMergeTiles >= T + pro) plan.s = static_cast<int>(T);
    }
    grid = static_cast<unsigned>(a.split_ctas);
  }
  // Scores are s * c2 + rel_h * log2(e) - m with s = q.k + rel_w * rw_mul
  // (rel_w enters through the MFMA accumulator), so rw_mul = log2(e) / c2.
  // scale == 0 has no such fold: Q is zeroed in the kernel instead, and s =
  // rel_w times c2 = log2(e) gives the bias alone.
  const bool zero_q = a.scale == 0.0f;
  const float c2 = zero_q ? kLog2e : a.scale * kLog2e;
  const float rw_mul = zero_q ? 1.0f : kLog2e / c2;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), lds, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.rel_h, a.rel_w, a.out,
                     a.H, a.W, q_tiles, c2, rw_mul, zero_q ? 1 : 0, ws, plan,
                     static_cast<const uint16_t*>(a.th), static_cast<const uint16_t*>(a.tw));
  if constexpr (SPLIT) {
    if (plan.rest > 0 && plan.s < T) {
      err = hipGetLastError();
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL((split_merge_kernel<BF16, OUT_F32>), dim3(static_cast<unsigned>(plan.rest) * 16),
                         dim3(256), 0, stream, static_cast<const float*>(ws), a.out, a.H * a.W, q_tiles,
                         plan.rounds * a.split_ctas);
    }
  }
  return hipGetLastError();
}

template <bool BF16, bool OUT_F32, int NW, bool SPLIT, bool FUSED = false, bool RH_LDS = false>
hipError_t launch_nw(const AttnArgs& a, hipStream_t stream) {
  // Grids whose sides are multiples of the 4 x 16 key tile need no masking.
  const bool aligned = a.H % kTileRows == 0 && a.W % kTileCols == 0;
  if constexpr (NW == 8 && !FUSED) {
    // rel_h rows in LDS when they fit beside the ring (one workgroup per CU).
    if (aligned && a.H <= kRhLdsMaxH &&
        attn32_lds_bytes<8>() + fused_rh_lds_bytes(a.H) <= static_cast<size_t>(a.lds_limit)) {
      return launch_cfg<BF16, OUT_F32, NW, true, SPLIT, false, true>(a, stream);
    }
  }
  return aligned ? launch_cfg<BF16, OUT_F32, NW, true, SPLIT, FUSED, RH_LDS>(a, stream)
                 : launch_cfg<BF16, OUT_F32, NW, false, SPLIT, FUSED, RH_LDS>(a, stream);
}

template <bool BF16, bool OUT_F32>
hipError_t launch_dt(const AttnArgs& a, int cfg, hipStream_t stream) {
  switch (cfg) {
    case 0: return launch_nw<BF16, OUT_F32, 8, false>(a, stream);
    case 1: return launch_nw<BF16, OUT_F32, 4, false>(a, stream);
    default: return launch_nw<BF16, OUT_F32, 8, true>(a, stream);  // kAttnSplitConfig
  }
}



}  // namespace

size_t attn_split_workspace_bytes(int64_t BH, int64_t N, int ctas) {
  (void)BH;
  (void)N;
  return static_cast<size_t>(split_piece_bytes(ctas));
}

size_t attn_fused_workspace_bytes(int H, int W, int ctas) {
  return static_cast<size_t>(split_piece_bytes(ctas)) +
         static_cast<size_t>(ctas) * 256 * static_cast<size_t>(fused_row_floats(H, W)) * sizeof(float);
}

template <bool RH_LDS>
hipError_t launch_fused_rh(const AttnArgs& a, hipStream_t stream) {
  if (a.bf16) {
    return a.out_f32 ? launch_nw<true, true, 8, true, true, RH_LDS>(a, stream)
                     : launch_nw<true, false, 8, true, true, RH_LDS>(a, stream);
  }
  return a.out_f32 ? launch_nw<false, true, 8, true, true, RH_LDS>(a, stream)
                   : launch_nw<false, false, 8, true, true, RH_LDS>(a, stream);
}

hipError_t launch_attn_fused(const AttnArgs& a, hipStream_t stream) {
  // rel_h rows in LDS when they fit beside the K/V ring (up to H = 68 on a
  // 160 KB LDS), else in the workspace slot like rel_w.
  const bool rh_lds = attn32_lds_bytes<8>() + fused_rh_lds_bytes(a.H) <= static_cast<size_t>(a.lds_limit);
  return rh_lds ? launch_fused_rh<true>(a, stream) : launch_fused_rh<false>(a, stream);
}

size_t attn_lds_bytes(int cfg, int H, int W) {
  (void)H;
  (void)W;
  switch (cfg) {
    case 1: return attn32_lds_bytes<4>();
    case 3: return attn16_lds_bytes();
    case kAttn12Config: return attn12_lds_bytes();
    default: return attn32_lds_bytes<8>();  // 0 and kAttnSplitConfig
  }
}

hipError_t launch_attn_fwd(const AttnArgs& a, int cfg, hipStream_t stream) {
  if (cfg == 3) return launch_attn16(a, stream);
  if (cfg == kAttn12Config) return launch_attn12(a, stream);
  if (a.bf16) {
    return a.out_f32 ? launch_dt<true, true>(a, cfg, stream) : launch_dt<true, false>(a, cfg, stream);
  }
  return a.out_f32 ? launch_dt<false, true>(a, cfg, stream) : launch_dt<false, false>(a, cfg, stream);
}

}  // namespace relpos
