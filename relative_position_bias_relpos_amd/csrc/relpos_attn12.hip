// relpos_attn_fwd, 12-wave kernel (launch configuration 6).
//
// Same method as the 32-query kernel in relpos_attn_fwd.hip (PR #55629 page,
// implementation section, item 1: K/V streamed with an online softmax, the
// rel_h/rel_w slices added per key block, no dense [N, N] bias), with the work
// cut so that every SIMD of every compute unit gets the same share:
//
//   * A workgroup owns 6 query blocks of 32 consecutive queries (192 queries;
//     block b of the workgroup is global block 6*unit + b in (b*heads,
//     query) order, so a workgroup may span the end of one head and the start
//     of the next).  Each block is worked by two waves: the even one takes the
//     even key tiles, the odd one the odd tiles.  12 waves, three per SIMD.
//     On the 64x64 grid with 12 heads that is 256 workgroups, one per CU.
//   * The two waves of a block keep their own online-softmax state (O, m, l)
//     and merge through LDS at the end; each writes half of the block's
//     output columns.  No workspace.
//   * Per step the workgroup stages one tile pair (the next even and odd tile)
//     per head it spans, all by LDS-direct 16-byte buffer loads that pass no
//     data through registers, at the top of step t into the slot step t+1
//     reads (two LDS slots).  Waves 8..11, the third wave of each SIMD, load
//     K and V; waves 0..7 load V only where it is converted, and run the key
//     loop at wave priority 1.  P.V runs on bf16 MFMA with P rounded to bf16
//     for bf16 inputs on grids of >= 2048 keys, so V is staged as loaded;
//     fp16 inputs likewise in fp16.  Otherwise (bf16, fewer keys) P is fp16,
//     and bf16 V lands in a raw area first and each of waves 0..7 converts
//     its own 16 bytes per lane to fp16 at the end of the step.  Tiles are
//     unpadded (8 KB) with XOR-swizzled 16-byte chunks so the MFMA operand
//     reads hit every LDS bank once.
//   * Inside a wave a step is plain: S^T = K Q^T (32x32x16 MFMA, rel_w in the
//     accumulator's initial value), exp2 softmax with a lazy reference maximum,
//     O^T += V^T P^T.  The three waves of a SIMD overlap one another's MFMA
//     and VALU work.
//   * The fused call (relpos_attn_fused) runs the same unit on a persistent
//     grid, each unit first forming its blocks' bias rows on MFMA: into LDS
//     for units inside one head on grids with H, W <= 64, else into a
//     workspace slot (fused_bias_lds_phase1/2, fused_bias_slot_phase2,
//     fused_bias_rows below).
//
// Lane layouts (S, P, the V transpose read) are the 32-query kernel's; only
// the LDS addressing differs (swizzle instead of padding).
#include <type_traits>

#include "relpos_attn_common.hpp"
#include "relpos_kernels.hpp"

namespace relpos {

namespace {

using namespace attn;

constexpr int kBlocks12 = 6;                       // query blocks per workgroup
constexpr int kWaves12 = 2 * kBlocks12;            // even and odd tile waves
constexpr int kThreads12 = 64 * kWaves12;
constexpr int kTileBytes12 = kTileKeys * kD * 2;   // one K or V tile, 8 KB
constexpr int kPairBytes12 = 4 * kTileBytes12;     // K even, K odd, V even, V odd
constexpr int kSlotBytes12 = 2 * kPairBytes12;     // one pair per head spanned
constexpr int kRawBytes12 = 2 * 2 * kTileBytes12;   // V of a pair as loaded, per head (before conversion)
constexpr int kLds12 = 2 * kSlotBytes12 + kRawBytes12;  // two slots + the raw V area: 160 KB
constexpr int kMergeStride12 = 64 * 16 * 4 + 2 * 32 * 4;  // per wave: 16 accumulators per lane, m, l
// Output staging after the merge, per wave: its 32 queries x 32 d (fp32), rows
// padded to 36 floats; placed after the 12 merge areas.
constexpr int kOutStride12 = 36;
constexpr int kOutBase12 = kWaves12 * kMergeStride12;
static_assert(kOutBase12 + kWaves12 * 32 * kOutStride12 * 4 <= kLds12, "output staging must fit the LDS");
// bf16 inputs with at least this many keys run P.V in bf16.  Rounding p to
// bf16 (8 significant bits) adds to each output an error that averages out
// over the keys; emulated in float64 on the workloads here, its mean over
// the outputs is 3.4e-5 at N = 4096 and 2.3e-5 at N = 9216 (1.2e-4 at N =
// 256; measured 6.8e-5 at N = 1024), against a 1e-4 bar, and it falls as
// 1/sqrt(N).  Smaller grids keep fp16 P.
constexpr int kBf16PMinKeys = 2048;

// Byte offset of K chunk c (16 bytes, d = 8c .. 8c+7) of tile row o: rows of
// 128 bytes, chunk index XOR-ed with bits 1..3 of the row, so that the 16
// rows a 16-lane group of the Q.K^T operand read touches fall on 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int k_off(int o, int c) { return o * 128 + 16 * (c ^ ((o >> 1) & 7)); }
// Byte offset of V chunk c of row o: 8-byte units XOR-ed with 8 * bit 1 of
// the row, so that the four rows of a transpose-read lane group and the two
// groups of a 32-lane pass cover the 64 banks once.
__device__ __forceinline__ int v_off(int o, int c) { return o * 128 + 16 * (c ^ (4 * ((o >> 1) & 1))); }

// Bias rows of one block of 32 queries (m0 .. m0+31 of grid row qh, W % 32 ==
// 0) for the fused call, computed by one wave on 32x32x16 MFMA: axis 0 writes
// rel_h [32][H] at dst, axis 1 rel_w [32][W] (the same products as
// relpos_build: rel_h against the reversed window of T_h, rel_w through the
// 96 columns of q . T_w its 64-column chunks reach, read back along the
// diagonal).  `a` holds the block's Q fragments.  `stage` is this wave's LDS
// area (32 x 104 floats, LDS byte address stage_lds); each chunk's table
// window (64 rows of T_h or 96 of T_w, contiguous in the table) is first
// staged there by LDS-direct loads of 8 rows each (8 cache lines per load,
// against 32 when each lane loads its own row), rows of 128 bytes with chunk
// c at c ^ (row % 8), and the operands are read from it before the products
// are staged over it.  Rows outside the table read zeros.
template <bool BF16>
__device__ __forceinline__ void fused_bias_rows(const u32x4 (&a)[4], const uint16_t* __restrict__ th,
                                                const uint16_t* __restrict__ tw, float* __restrict__ dst,
                                                int axis, int qh, int m0, int H, int W, float* stage,
                                                uint32_t stage_lds, int lane) {
  constexpr int kHS = 72, kGS = 104;  // staging row strides (floats)
  const int ml = lane & 31, half = lane >> 5;
  auto out_row = [&](int r) { return 8 * (r >> 2) + 4 * half + (r & 3); };
  const int sc = 4 * (lane & 15), sr = lane >> 4;
  const unsigned char* const win = reinterpret_cast<const unsigned char*>(stage);
  auto window = [&](const sgpr4& rs, int t0, int pieces) {
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's reads of the area are done
    for (int p = 0; p < pieces; ++p) {
      const int r = 8 * p + (lane >> 3);
      lds_load16(rs, (t0 + r) * kD * 2 + 16 * ((lane & 7) ^ (r & 7)), 0, stage_lds + 1024 * p);
    }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  auto wread = [&](int r, int c) { return *reinterpret_cast<const u32x4*>(win + r * 128 + 16 * (c ^ (r & 7))); };
  if (axis == 0) {
    const sgpr4 rt = rsrc_words(th, static_cast<uint32_t>(2 * H - 1) * kD * 2);
    for (int n0 = 0; n0 < H; n0 += 64) {
      // kh = n0 + j takes table row qh - kh + H - 1: window row 63 - j
      window(rt, qh + H - 1 - n0 - 63, 8);
      u32x4 b[2][4];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int kd = 0; kd < 4; ++kd) b[nt][kd] = wread(63 - 32 * nt - ml, 2 * kd + half);
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x16 acc{};
#pragma unroll
        for (int kd = 0; kd < 4; ++kd) acc = mfma32<BF16>(a[kd], b[nt][kd], acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) stage[out_row(r) * kHS + 32 * nt + ml] = acc[r];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = sr + 4 * i, n = n0 + sc;
        const f32x4 x = *reinterpret_cast<const f32x4*>(stage + m * kHS + sc);
        if (n < H) *reinterpret_cast<f32x4*>(dst + m * H + n) = x;  // H % 4 == 0 here
      }
    }
  } else {
    const sgpr4 rt = rsrc_words(tw, static_cast<uint32_t>(2 * W - 1) * kD * 2);
    for (int n0 = 0; n0 < W; n0 += 64) {
      // G column j takes table row tlo + j: window row j
      window(rt, m0 - n0 - 63 + W - 1, 12);
      u32x4 b[3][4];
#pragma unroll
      for (int gt = 0; gt < 3; ++gt) {
#pragma unroll
        for (int kd = 0; kd < 4; ++kd) b[gt][kd] = wread(32 * gt + ml, 2 * kd + half);
      }
#pragma unroll
      for (int gt = 0; gt < 3; ++gt) {
        f32x16 g{};
#pragma unroll
        for (int kd = 0; kd < 4; ++kd) g = mfma32<BF16>(a[kd], b[gt][kd], g);
#pragma unroll
        for (int r = 0; r < 16; ++r) stage[out_row(r) * kGS + 32 * gt + ml] = g[r];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = sr + 4 * i, n = n0 + sc;
        const float* gp = stage + m * kGS + m - sc + 63;  // G[m, m - (sc + e) + 63]
        const f32x4 x{gp[0], gp[-1], gp[-2], gp[-3]};
        if (n < W) *reinterpret_cast<f32x4*>(dst + 32 * H + m * W + n) = x;  // W % 32 == 0 here
      }
    }
  }
}
static_assert(12 * 1024 <= 32 * 104 * 4, "a T_w window must fit a wave's staging area");

// Bias rows kept in LDS (the fused call, single-head units, H <= 64 and W <=
// 64, bf16 P): a workgroup spanning one head uses one 32 KB pair of each
// slot and not the raw-V area, which leaves three 32 KB regions free; block
// b's rel_h rows go to region b/2 at (b%2) * 16 KB, its rel_w rows 8 KB
// further.  A row is 64 floats (256 B) whose 16-byte chunk c sits at chunk c
// ^ (row % 16), so that the 32 rows a key-loop read touches at one column
// cover the 64 banks twice.
constexpr int kLbMaxSide = 64;  // LDS bias rows are 64 floats
__device__ __forceinline__ int lb_block_off(int b) {
  return (b < 2 ? kPairBytes12 : b < 4 ? kSlotBytes12 + kPairBytes12 : 2 * kSlotBytes12) + (b & 1) * 16384;
}
__device__ __forceinline__ int lb_off(int row, int col) {
  return row * 256 + 16 * ((col >> 2) ^ (row & 15)) + 4 * (col & 3);
}
static_assert(2 * kSlotBytes12 + 32768 <= kLds12, "the third bias region must fit the LDS");

// The tables staged once per workgroup for the LDS-resident bias: T_h and T_w
// (2L - 1 <= 127 rows of 128 bytes each, zeros past the last row) in the
// pair area of slot 1, which pair 1's loads first use in step 0; row t's
// 16-byte chunk c at chunk c ^ (t % 8), so that the 32 rows an MFMA operand
// read touches at one chunk spread over all banks.
constexpr int kTabBytes12 = 16384;
__device__ __forceinline__ int tab_off(int t, int c) { return t * 128 + 16 * (c ^ (t & 7)); }

// The bias rows of one block of 32 queries (m0 .. m0+31 of grid row qh) for
// the LDS rows above, by one wave on 32x32x16 MFMA, in two phases around a
// workgroup barrier (the same products, same order, as relpos_build), with
// the block's Q fragments `a` and the tables staged in LDS (`tabs`).
//   Phase 1.  axis 0: acc = the product against the reversed window of T_h,
//     rel_h[m, kh] = q[m] . T_h[qh - kh + H - 1] (kept in registers).
//     axis 1: G[m, j] = q[m] . T_w[tlo + j] over the 95 table rows tlo = m0 -
//     63 + W - 1 .. the block reaches, staged in the block's 16 KB region
//     (rows of 104 floats) and read back along the diagonal, rel_w[m, n] =
//     G[m, m - n + 63], into wr (lane: rows lane/16 + 4i, columns 4*(lane%16)
//     .. +3).  Columns past H (W) get values that are never read; table
//     rows outside [0, 127] are clamped into the staged area for the same
//     reason.
//   Phase 2 (after the barrier, once the odd wave of every block has read its
//     staged G back): the rows are written to their swizzled places.
struct BiasRegs {
  f32x16 acc[2];
  f32x4 wr[8];
};

template <bool BF16>
__device__ __forceinline__ void fused_bias_lds_phase1(const u32x4 (&a)[4], const unsigned char* tabs,
                                                      unsigned char* region, int axis, int qh, int m0, int H,
                                                      int W, int lane, BiasRegs& br) {
  constexpr int kGS = 104;  // staging row stride (floats): the two 32-lane halves on disjoint banks
  const int ml = lane & 31, half = lane >> 5;
  auto out_row = [&](int r) { return 8 * (r >> 2) + 4 * half + (r & 3); };
  auto clamp_row = [](int t) { return t < 0 ? 0 : (t > 127 ? 127 : t); };
  if (axis == 0) {
    u32x4 b[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int t = clamp_row(qh - (32 * nt + ml) + H - 1);
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) b[nt][kd] = *reinterpret_cast<const u32x4*>(tabs + tab_off(t, 2 * kd + half));
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x16 acc{};
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) acc = mfma32<BF16>(a[kd], b[nt][kd], acc);
      br.acc[nt] = acc;
    }
  } else {
    const unsigned char* const tw = tabs + kTabBytes12;
    const int tlo = m0 - 63 + W - 1;
    u32x4 b[3][4];
#pragma unroll
    for (int gt = 0; gt < 3; ++gt) {
      const int t = clamp_row(tlo + 32 * gt + ml);
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) b[gt][kd] = *reinterpret_cast<const u32x4*>(tw + tab_off(t, 2 * kd + half));
    }
    float* const stage = reinterpret_cast<float*>(region);
#pragma unroll
    for (int gt = 0; gt < 3; ++gt) {
      f32x16 g{};
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) g = mfma32<BF16>(a[kd], b[gt][kd], g);
#pragma unroll
      for (int r = 0; r < 16; ++r) stage[out_row(r) * kGS + 32 * gt + ml] = g[r];
    }
    // read back by this wave only
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int sc = 4 * (lane & 15), sr = lane >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = sr + 4 * i;
      const float* gp = stage + m * kGS + m - sc + 63;  // G[m, m - (sc + e) + 63]
      br.wr[i] = f32x4{gp[0], gp[-1], gp[-2], gp[-3]};
    }
  }
}

__device__ __forceinline__ void fused_bias_lds_phase2(unsigned char* region, int axis, int lane,
                                                      const BiasRegs& br) {
  const int ml = lane & 31, half = lane >> 5;
  if (axis == 0) {
    // element (m, kh), m = 8*(r/4) + 4*half + r%4, kh = 32*nt + ml: chunk
    // (kh/4) ^ (m % 16) of row m, and m % 16 = c_r | 4*half with c_r =
    // 8*((r/4) % 2) + r%4, so the lane's chunk is ((kh/4) ^ 4*half) ^ c_r.
    // Columns kh >= H hold zeros (the table loads there read zeros) and lie
    // inside the 64-float rows; they are never read.
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int kh = 32 * nt + ml;
      const int xl = (kh >> 2) ^ (4 * half);
      unsigned char* const base = region + half * 4 * 256 + 4 * (kh & 3);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int cr = 8 * ((r >> 2) & 1) + (r & 3);
        const int mrow = 8 * (r >> 2) + (r & 3);  // m without the 4*half part
        *reinterpret_cast<float*>(base + mrow * 256 + 16 * (xl ^ cr)) = br.acc[nt][r];
      }
    }
  } else {
    const int sc = 4 * (lane & 15), sr = lane >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = sr + 4 * i;
      *reinterpret_cast<f32x4*>(region + 8192 + lb_off(m, sc)) = br.wr[i];
    }
  }
}

// Phase 2 for a unit whose bias rows go to its workspace slot instead (units
// spanning two heads, or a partial last unit, on grids with H, W <= 64):
// rel_h [32][H] at dst through `stage` (rows of 72 floats; the phase-1
// staging of this block, read back before the barrier), rel_w [32][W] at dst
// + 32 * H from the registers, as 16-byte stores of whole rows.
__device__ __forceinline__ void fused_bias_slot_phase2(float* __restrict__ dst, float* stage, int axis, int H,
                                                       int W, int lane, const BiasRegs& br) {
  constexpr int kHS = 72;
  const int ml = lane & 31, half = lane >> 5;
  const int sc = 4 * (lane & 15), sr = lane >> 4;
  if (axis == 0) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) stage[(8 * (r >> 2) + 4 * half + (r & 3)) * kHS + 32 * nt + ml] = br.acc[nt][r];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = sr + 4 * i;
      const f32x4 x = *reinterpret_cast<const f32x4*>(stage + m * kHS + sc);
      if (sc < H) *reinterpret_cast<f32x4*>(dst + m * H + sc) = x;  // H % 4 == 0 here
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = sr + 4 * i;
      if (sc < W) *reinterpret_cast<f32x4*>(dst + 32 * H + m * W + sc) = br.wr[i];  // W % 32 == 0 here
    }
  }
}

// Phase-1 staging area of block b for fused_bias_slot_phase2's units: free
// LDS before pair 0 is loaded (slot 0) and outside the staged tables (slot 1's
// first 32 KB): 13 KB each in [0, 64 KB) and [96, 128 KB).
__device__ __forceinline__ int s2_stage_off(int b) { return b < 4 ? b * 13312 : 3 * kPairBytes12 + (b - 4) * 13312; }
static_assert(3 * 13312 + 13312 <= 2 * kPairBytes12 && 3 * kPairBytes12 + 2 * 13312 <= 2 * kSlotBytes12,
              "staging areas must fit beside the tables");

// One unit (6 blocks of 32 queries) of the 12-wave kernel.
// PB (bf16 inputs only): P.V runs in bf16 (P rounded to bf16, V staged as
// loaded); otherwise in fp16 (bf16 V converted to fp16 while staged).
// FUSED: the bias rows of the unit's blocks are computed first into this
// workgroup's slot of `ws` (block b: rel_h [32][H] then rel_w [32][W] at
// b * 32 * (H + W) floats) and read from there instead of rel_h / rel_w;
// with LB (units within one head, H, W <= 64, bf16 P) into LDS instead;
// with S2 (the other units on such grids) into the slot, formed from the
// tables staged in LDS.
template <bool BF16, bool OUT_F32, bool ALIGNED, bool PB, bool FUSED, bool LB = false, bool S2 = false>
__device__ __forceinline__ void attn12_unit(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ rel_h,
    const float* __restrict__ rel_w, void* __restrict__ out,
    const uint16_t* __restrict__ th, const uint16_t* __restrict__ tw, float* __restrict__ ws,
    int H, int W, int nblk, int total_blocks, float c2, float rw_mul, int zero_q, int unit) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int N = H * W;
  // In the fused call's unit loop: opaque to the compiler, so that the
  // lane-derived addresses below are recomputed per unit rather than kept
  // live across the whole loop (which would spill).
  int tid = static_cast<int>(threadIdx.x);
  if constexpr (FUSED) __asm__ volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int blk = wave >> 1, par = wave & 1;

  // ---- this workgroup's blocks and heads -------------------------------------
  const int gb0 = unit * kBlocks12;
  const int gb_last = gb0 + kBlocks12 - 1 < total_blocks - 1 ? gb0 + kBlocks12 - 1 : total_blocks - 1;
  const int bhA = gb0 / nblk;
  const bool two = gb_last / nblk != bhA;  // the workgroup spans two heads
  const bool bvalid = gb0 + blk < total_blocks;
  const int gb = bvalid ? gb0 + blk : total_blocks - 1;
  const int bh = gb / nblk;
  const int q0 = (gb - bh * nblk) * 32;
  const int hs = bh - bhA;  // head slot of this wave's block
  const size_t head = static_cast<size_t>(bh) * N;

  // ---- the fused call: this block's bias rows into the workgroup's slot ---------
  // The even wave of the block writes rel_h, the odd one rel_w, each staging
  // through its own 13 KB of LDS (free until pair 0 is staged below).
  const float* rh_rows = rel_h + (head + q0) * H;
  const float* rw_rows = rel_w + (head + q0) * W;
  static_assert(!LB || (FUSED && PB), "bias rows in LDS only in the fused call with bf16 P");
  static_assert(!S2 || (FUSED && PB && !LB), "two-phase slot rows only in the fused call with bf16 P");
  // S2 units have one slot each, one per b*heads when there are at most as
  // many as workgroups: a unit spanning heads bhA and bhA + 1 slot bhA (each
  // head boundary lies in one unit), a partial last unit inside one head
  // slot B*heads - 1; else the workgroup's own slot.
  const int n_bh = total_blocks / nblk;
  const int s2_slot = n_bh <= static_cast<int>(gridDim.x) ? (two ? bhA : n_bh - 1) : static_cast<int>(blockIdx.x);
  float* const s2_rows = ws + (static_cast<size_t>(s2_slot) * kBlocks12 + blk) * 32 * (H + W);
  if constexpr (S2) {
    rh_rows = s2_rows;
    rw_rows = s2_rows + 32 * H;
  }
  // ---- Q^T operand fragments of this wave's 32 queries -----------------------
  const int ql = lane & 31;
  const int qi = q0 + ql;
  const bool qok = qi < N;
  u32x4 qf[4];
#pragma unroll
  for (int kd = 0; kd < 4; ++kd) {
    qf[kd] = (qok && zero_q == 0) ? *reinterpret_cast<const u32x4*>(q + (head + qi) * kD + 16 * kd + 8 * half)
                                  : u32x4{0, 0, 0, 0};
  }

  if constexpr (FUSED && !LB && !S2) {
    float* brow = ws + (static_cast<size_t>(blockIdx.x) * kBlocks12 + blk) * 32 * (H + W);
    if (bvalid) {
      // the block's Q fragments (reloaded when scale == 0 zeroed them)
      u32x4 qa[4];
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) {
        qa[kd] = zero_q == 0 ? qf[kd] : *reinterpret_cast<const u32x4*>(q + (head + qi) * kD + 16 * kd + 8 * half);
      }
      const uint32_t stage_lds = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(
          reinterpret_cast<size_t>((__attribute__((address_space(3))) unsigned char*)smem)))) + wave * 32 * 104 * 4;
      fused_bias_rows<BF16>(qa, th, tw, brow, par, q0 / W, q0 % W, H, W,
                            reinterpret_cast<float*>(smem) + wave * 32 * 104, stage_lds, lane);
    }
    // the rows are read back by this wave only (through the same L1)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    rh_rows = brow;
    rw_rows = brow + 32 * H;
  }

  const int band_tiles = (H + kTileRows - 1) / kTileRows;
  const int T = band_tiles * ((W + kTileCols - 1) / kTileCols);
  const int steps = (T + 1) / 2;

  // ---- staging ------------------------------------------------------------------
  // Every load is an LDS-direct 16-byte buffer load: waves 8..11 bring in K
  // and V (4 of each tile's 1-KB row blocks each, per head spanned), except
  // that V to be converted (bf16 inputs with fp16 P) comes in on waves 0..7
  // (2 row blocks each).
  const bool v_wave = wave < 8;
  const uint32_t head_bytes = static_cast<uint32_t>(N) * kD * 2;
  const sgpr4 krs0 = rsrc_words(k + static_cast<size_t>(bhA) * N * kD, head_bytes);
  const sgpr4 krs1 = rsrc_words(k + static_cast<size_t>(bhA + 1) * N * kD, head_bytes);
  const sgpr4 vrs0 = rsrc_words(v + static_cast<size_t>(bhA) * N * kD, head_bytes);
  const sgpr4 vrs1 = rsrc_words(v + static_cast<size_t>(bhA + 1) * N * kD, head_bytes);

  // V to convert: wave w < 8 loads row blocks rb = 2*(w&3) + j (j = 0, 1) of tile w>>2
  // of a pair into the raw area (lane L: row 8*rb + L/8, chunk L%8, as in
  // memory), and at the end of the step converts exactly those 16 bytes per
  // lane (bf16 -> fp16) into the slot's swizzled V tile.  No barrier is
  // needed between the two: each lane reads back what its own load wrote,
  // after waiting for it.
  const int v_tile = (wave >> 2) & 1;
  int v_goff[2], v_lds[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int o = 8 * (2 * (wave & 3) + j) + (lane >> 3);
    v_goff[j] = ((o >> 4) * W + (o & 15)) * (kD * 2) + 16 * (lane & 7);
    v_lds[j] = (2 + v_tile) * kTileBytes12 + v_off(o, lane & 7);
  }
  unsigned char* raw = smem + 2 * kSlotBytes12;
  // LDS byte address of smem (wave-uniform): the LDS-direct loads take their
  // destination as a scalar
  const uint32_t lds0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(
      reinterpret_cast<size_t>((__attribute__((address_space(3))) unsigned char*)smem))));
  auto raw_off = [&](int e, int j) { return e * 2 * kTileBytes12 + v_tile * kTileBytes12 + (2 * (wave & 3) + j) * 1024; };
  auto tile_org = [&](TilePos p) { return (p.kh * W + p.kw) * (kD * 2); };
  // V to convert (bf16 inputs with fp16 P): into the raw area, converted
  // later; otherwise straight into the slot's swizzled V tile (lane L then
  // loads logical chunk (L%8) ^ (4*bit 1 of the row), as K does).
  // pair_off: the pair's LDS offset.
  constexpr bool kConvertV = BF16 && !PB;
  auto v_dma = [&](int e, const sgpr4& rs, TilePos pe, int pair_off) {
    const TilePos p = v_tile == 0 ? pe : next_tile(pe, H);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int o = 8 * (2 * (wave & 3) + j) + (lane >> 3);
      const int gchunk = kConvertV ? 0 : 16 * (((lane & 7) ^ (4 * ((o >> 1) & 1))) - (lane & 7));
      int voff, soff;
      if constexpr (ALIGNED) {
        voff = v_goff[j] + gchunk;
        soff = p.kw < W ? tile_org(p) : 0;
      } else {
        const bool ok = p.kh + (o >> 4) < H && p.kw + (o & 15) < W;
        voff = ok ? tile_org(p) + v_goff[j] + gchunk : kOob;
        soff = 0;
      }
      const uint32_t dst = kConvertV ? lds0 + 2 * kSlotBytes12 + raw_off(e, j)
                                     : lds0 + pair_off + (2 + v_tile) * kTileBytes12 + (2 * (wave & 3) + j) * 1024;
      lds_load16(rs, voff, soff, dst);
    }
  };
  // bf16 V for fp16 P, after this wave's loads are complete: raw -> fp16 -> slot
  auto v_convert = [&](int e, unsigned char* pair) {
    if constexpr (!kConvertV) return;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 x = *reinterpret_cast<const u32x4*>(raw + raw_off(e, j) + 16 * lane);
      if constexpr (BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) x[w] = pack_f16(bf16_lo(x[w]), bf16_hi(x[w]));
      }
      *reinterpret_cast<u32x4*>(pair + v_lds[j]) = x;
    }
  };
  // K: wave 8 + kw issues row blocks rb = 4*(kw&1) + i of tile kw>>1 (even,
  // odd).  Lane L of a row block writes LDS bytes 16L..16L+15 of it: row o =
  // 8*rb + L/8, swizzled chunk L%8, i.e. logical chunk (L%8) ^ ((o>>1)&7).
  const int kwv = wave - 8;
  const int k_tile = kwv >> 1;
  int k_goff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = 8 * (4 * (kwv & 1) + i) + (lane >> 3);
    const int c = (lane & 7) ^ ((o >> 1) & 7);
    k_goff[i] = ((o >> 4) * W + (o & 15)) * (kD * 2) + 16 * c;
  }
  // pair_off: byte offset of the pair in LDS
  auto k_dma = [&](const sgpr4& rs, TilePos pe, int pair_off) {
    const TilePos p = k_tile == 0 ? pe : next_tile(pe, H);
    const uint32_t dst = lds0 + pair_off + k_tile * kTileBytes12 + 4 * (kwv & 1) * 1024;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int voff, soff;
      if constexpr (ALIGNED) {
        voff = k_goff[i];
        soff = p.kw < W ? tile_org(p) : 0;
      } else {
        const int o = 8 * (4 * (kwv & 1) + i) + (lane >> 3);
        const bool ok = p.kh + (o >> 4) < H && p.kw + (o & 15) < W;
        voff = ok ? tile_org(p) + k_goff[i] : kOob;
        soff = 0;
      }
      lds_load16(rs, voff, soff, dst + i * 1024);
    }
  };
  // V row blocks without conversion (bf16 P, or fp16 inputs): loaded by the
  // K waves too, each its K blocks' (tile, rb), so that waves 0..7 issue no
  // staging load.  Waves 8..11 are the third wave of their SIMDs, the last
  // in the issue order, and have the slack: at 64x64 with 12 heads 63.3-63.4
  // against 65.0-65.4 us with V on waves 0..7, 48x80 111.4 against 115.8-119.3
  // us (spreading the loads over all 12 waves instead was slower: 119 us at
  // 48x80).
  auto v_dma_k = [&](const sgpr4& rs, TilePos pe, int pair_off) {
    const TilePos p = k_tile == 0 ? pe : next_tile(pe, H);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = 8 * (4 * (kwv & 1) + i) + (lane >> 3);
      const int goff = ((o >> 4) * W + (o & 15)) * (kD * 2) + 16 * ((lane & 7) ^ (4 * ((o >> 1) & 1)));
      int voff, soff;
      if constexpr (ALIGNED) {
        voff = goff;
        soff = p.kw < W ? tile_org(p) : 0;
      } else {
        const bool ok = p.kh + (o >> 4) < H && p.kw + (o & 15) < W;
        voff = ok ? tile_org(p) + goff : kOob;
        soff = 0;
      }
      lds_load16(rs, voff, soff, lds0 + pair_off + (2 + k_tile) * kTileBytes12 + (4 * (kwv & 1) + i) * 1024);
    }
  };
  // The loads of one pair (per head spanned) into the pair area at pair_off.
  auto stage_pair = [&](int e, const sgpr4& krs, const sgpr4& vrs, TilePos pe, int pair_off) {
    if (v_wave) {
      if constexpr (kConvertV) v_dma(e, vrs, pe, pair_off);
    } else {
      k_dma(krs, pe, pair_off);
      if constexpr (!kConvertV) v_dma_k(vrs, pe, pair_off);
    }
  };
  auto slot_ptr = [&](int s) { return smem + s * kSlotBytes12; };

  // ---- bias ---------------------------------------------------------------------
  // rel_w through the Q.K^T accumulator (rwc = rel_w * rw_mul per register's
  // key column, reloaded per 16-column band), rel_h and the reference maximum
  // in one fma per score (as in the 32-query kernel).
  const int rows = N - q0 < 32 ? N - q0 : 32;
  const __amdgpu_buffer_rsrc_t rwrs = make_rsrc(rw_rows, static_cast<uint32_t>(rows * W) * 4);
  const __amdgpu_buffer_rsrc_t rhrs = make_rsrc(rh_rows, static_cast<uint32_t>(rows * H) * 4);
  const int qrow = qok ? ql : 0;
  const int rw_lane = (qrow * W + 4 * half) * 4;
  const int rh_lane = qrow * H * 4;
  f32x16 rwc;
  const unsigned char* const lb_rows = smem + lb_block_off(blk);
  auto load_band = [&](int kw0) {
    float x[8];
    if constexpr (LB) {
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(lb_rows + 8192 + lb_off(qrow, kw0 + 4 * half));
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(lb_rows + 8192 + lb_off(qrow, kw0 + 4 * half + 8));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = as_float(a0[i]) * rw_mul;
        x[4 + i] = as_float(a1[i]) * rw_mul;
      }
    } else if constexpr (ALIGNED) {
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
        const int dc = 8 * (i >> 2) + (i & 3);
        const int c = kw0 + dc + 4 * half;
        const float y = buf_loadf(rwrs, c < W ? rw_lane + 4 * (kw0 + dc) : kOob);
        x[i] = (c < W ? y : -__builtin_inff()) * rw_mul;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) rwc[r] = x[4 * ((r >> 2) & 1) + (r & 3)];
  };
  float rh[4], rh_next[4];  // rel_h of the step's tile; of the next step's, prefetched
  auto load_rh = [&](int kh0) {
    if constexpr (LB) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(lb_rows + lb_off(qrow, kh0));
#pragma unroll
      for (int r = 0; r < 4; ++r) rh_next[r] = as_float(a[r]);
    } else if constexpr (ALIGNED) {
      const u32x4 a = buf_load16(rhrs, rh_lane, 4 * kh0);
#pragma unroll
      for (int r = 0; r < 4; ++r) rh_next[r] = as_float(a[r]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float y = buf_loadf(rhrs, kh0 + r < H ? rh_lane + 4 * (kh0 + r) : kOob);
        rh_next[r] = kh0 + r < H ? y : -__builtin_inff();
      }
    }
  };

  // ---- operand read addressing (bytes within a pair) --------------------------
  // K^T fragment (st, kd): row 32*st + ql, chunk 2*kd + half, swizzled.
  int k_rd[4];
#pragma unroll
  for (int kd = 0; kd < 4; ++kd) k_rd[kd] = par * kTileBytes12 + k_off(ql, 2 * kd + half);
  // V^T fragment (ks, dt): transpose reads of rows 16*ks + tr_row (+8) at 8-byte
  // unit 8*dt + 4*(grp&1) + (jl&3), units XOR-ed with 8 when bit 1 of the row
  // (bit 3 of jl) is set.
  const int grp = lane >> 4, jl = lane & 15;
  const int tr_row = 4 * (grp >> 1) + (jl >> 2);
  const int vsw = 8 * ((jl >> 3) & 1);
  int v_rd[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
    v_rd[dt] = (2 + par) * kTileBytes12 + tr_row * 128 + 8 * ((8 * dt + 4 * (grp & 1) + (jl & 3)) ^ vsw);

  // ---- prologue: pair 0 in slot 0 ---------------------------------------------
  // Tables of the LDS-formed bias: once per workgroup into slot 1's first pair
  // area (1 KB pieces, 16 per table, spread over the waves).
  auto stage_tables = [&]() {
    const sgpr4 trs_h = rsrc_words(th, static_cast<uint32_t>(2 * H - 1) * kD * 2);
    const sgpr4 trs_w = rsrc_words(tw, static_cast<uint32_t>(2 * W - 1) * kD * 2);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int piece = wave + 12 * i;
      if (piece < 32) {
        const int tr = 8 * (piece & 15) + (lane >> 3);
        lds_load16(piece < 16 ? trs_h : trs_w, tr * 128 + 16 * ((lane & 7) ^ (tr & 7)), 0,
                   lds0 + kSlotBytes12 + (piece >> 4) * kTabBytes12 + (piece & 15) * 1024);
      }
    }
  };
  // The block's Q fragments for the bias products (reloaded when scale == 0
  // zeroed them).
  auto bias_q = [&](u32x4 (&qa)[4]) {
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) {
      qa[kd] = zero_q == 0 ? qf[kd] : *reinterpret_cast<const u32x4*>(q + (head + qi) * kD + 16 * kd + 8 * half);
    }
  };
  if constexpr (S2) {
    // Units spanning two heads (or partial) on grids with H, W <= 64: the
    // rows are formed as for LB, from LDS, before pair 0 is staged (the
    // staging areas lie in its slot), and written to the workspace slot.
    stage_tables();
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    u32x4 qa[4];
    bias_q(qa);
    BiasRegs br;
    float* const stage = reinterpret_cast<float*>(smem + s2_stage_off(blk));
    if (bvalid) {
      fused_bias_lds_phase1<BF16>(qa, smem + kSlotBytes12, reinterpret_cast<unsigned char*>(stage), par, q0 / W,
                                  q0 % W, H, W, lane, br);
    }
    __syncthreads();
    if (bvalid) fused_bias_slot_phase2(s2_rows, stage, par, H, W, lane, br);
    // the rows are read back by this wave only (through the same L1); the
    // staging areas are free again before pair 0 lands in slot 0
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  const TilePos p0{0, 0};
  stage_pair(0, krs0, vrs0, p0, 0);
  if (two) stage_pair(1, krs1, vrs1, p0, kPairBytes12);
  if constexpr (LB) stage_tables();  // beside pair 0's loads
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (v_wave) {
    v_convert(0, slot_ptr(0));
    if (two) v_convert(1, slot_ptr(0) + kPairBytes12);
  }
  if constexpr (LB) {
    // Every block valid and in the one head: the even wave forms rel_h, the
    // odd one rel_w (staging in the block's region), from the block's Q
    // fragments (reloaded when scale == 0 zeroed them) and the staged tables;
    // then both write their rows into the region once every odd wave has read
    // its staging back.
    __syncthreads();  // tables and pair 0 in LDS
    u32x4 qa[4];
    bias_q(qa);
    BiasRegs br;
    unsigned char* const region = smem + lb_block_off(blk);
    fused_bias_lds_phase1<BF16>(qa, smem + kSlotBytes12, region, par, q0 / W, q0 % W, H, W, lane, br);
    __syncthreads();
    fused_bias_lds_phase2(region, par, lane, br);
    __syncthreads();  // the block's rows of both waves written
  }
  TilePos pc = par ? next_tile(p0, H) : p0;  // this wave's tile of the current step
  int band_kw = pc.kw;
  load_band(pc.kw);
  load_rh(pc.kh);
  if constexpr (!LB) __syncthreads();

  f32x16 acc[2];
  acc[0] = f32x16{};
  acc[1] = f32x16{};
  float m = 0.f, l = 0.f;
  bool first = true;
  // p packing and the row sum of the rounded p, in P's type
  auto pack_p = [](float a, float b) -> uint32_t {
    if constexpr (PB) {
      return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
    } else {
      return pack_f16(a, b);
    }
  };
  auto sum_p = [](uint32_t w, float acc_) -> float {
    if constexpr (PB) {
      return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), bf16x2{(__bf16)1.0f, (__bf16)1.0f},
                                             acc_, false);
    } else {
      return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), f16x2{(_Float16)1.0f, (_Float16)1.0f}, acc_,
                                    false);
    }
  };

  TilePos pk = next_tile(next_tile(p0, H), H);  // even tile of pair t+1 (staged during step t)

  // This wave's tile of the step, from the pair in `pair` (rel_h already
  // loaded), as two halves of 32 keys (grid rows 2*st, 2*st+1 of the tile),
  // each S^T = K Q^T + rel_w term, softmax, O^T += V^T P^T; the first half's
  // P.V MFMAs are interleaved with the second half's Q.K^T MFMAs (independent
  // accumulators), so only one half's scores are held at a time.
  auto compute = [&](const unsigned char* pair, auto&& tail) {
    const unsigned char* kb = pair + hs * kPairBytes12;
    auto read_k = [&](int st, u32x4 (&kf)[4]) {
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) kf[kd] = *reinterpret_cast<const u32x4*>(kb + k_rd[kd] + st * 32 * 128);
    };
    auto read_v = [&](int st, u32x4 (&vf)[4]) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const unsigned char* vp = kb + v_rd[dt] + (2 * st + kk) * 16 * 128;
          const u32x2 lo = ds_read_tr16(reinterpret_cast<const uint16_t*>(vp));
          const u32x2 hi = ds_read_tr16(reinterpret_cast<const uint16_t*>(vp + 8 * 128));
          vf[2 * kk + dt] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      }
    };
    // Softmax of scores 4g..4g+3 of one half (grid row g/2 of the half):
    // x = s*c2 + rel_h*log2(e) - m, p = 2^x rounded to fp16 (l sums the
    // rounded p).
    auto softmax_chunk = [&](int st, int g, f32x16& sc, u32x4 (&pf)[2], float& tsum) {
      const float rhm = __builtin_fmaf(rh[2 * st + (g >> 1)], kLog2e, -m);
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = __builtin_fmaf(sc[4 * g + e], c2, rhm);
        sc[4 * g + e] = x[e];
      }
      const uint32_t w0 = pack_p(exp2_fast(x[0]), exp2_fast(x[1]));
      const uint32_t w1 = pack_p(exp2_fast(x[2]), exp2_fast(x[3]));
      tsum = sum_p(w0, tsum);
      tsum = sum_p(w1, tsum);
      pf[g >> 1][2 * (g & 1)] = w0;
      pf[g >> 1][2 * (g & 1) + 1] = w1;
    };
    // After a half's softmax: move the reference maximum when it must (the
    // first half-tile, or a p above 2^15): the exact maximum of these scores
    // per query, O and l rescaled, p recomputed.
    auto settle = [&](f32x16& sc, u32x4 (&pf)[2], float tsum) {
      const bool grow = first || !(tsum <= kGrowLimit);
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        __asm__ volatile("; reference maximum moves" ::);
        float mx = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sc[r]);
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
        // an idle step's scores are all -inf: no maximum to take, p = 0
        const bool empty = !(mx > -__builtin_inff());
        const float inc = empty ? 0.f : (first ? mx : __builtin_fmaxf(mx, 0.f));
        if (!first && !empty) {
          const float alpha = exp2_fast(-inc);
          l *= alpha;
          acc[0] *= alpha;
          acc[1] *= alpha;
        }
        m += inc;
        float ts = 0.f;
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          uint32_t w4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            w4[i] = pack_p(exp2_fast(sc[8 * gg + 2 * i] - inc), exp2_fast(sc[8 * gg + 2 * i + 1] - inc));
            ts = sum_p(w4[i], ts);
          }
          pf[gg] = u32x4{w4[0], w4[1], w4[2], w4[3]};
        }
        tsum = ts;
        if (!empty) first = false;
      }
      l += tsum;
    };

    // half 0's Q.K^T; then four chunks of (one Q.K^T MFMA of half 1, the
    // softmax of four of half 0's scores); then four chunks of (one P.V MFMA
    // of half 0, the softmax of four of half 1's scores); then half 1's P.V.
    u32x4 kf[4], vf[4];
    u32x4 p0[2], p1[2];
    f32x16 s0, s1;
    read_k(0, kf);
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) s0 = mfma32<BF16>(kf[kd], qf[kd], kd == 0 ? rwc : s0);
    // half 1's K fragments are read one chunk ahead of their MFMA
    auto k1 = [&](int kd) { return *reinterpret_cast<const u32x4*>(kb + k_rd[kd] + 32 * 128); };
    u32x4 ka = k1(0), kn;
    __builtin_amdgcn_sched_barrier(0);
    float ts0 = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (g < 3) kn = k1(g + 1);
      s1 = mfma32<BF16>(ka, qf[g], g == 0 ? rwc : s1);
      softmax_chunk(0, g, s0, p0, ts0);
      ka = kn;
      __builtin_amdgcn_sched_barrier(0);
    }
    read_v(0, vf);
    settle(s0, p0, ts0);
    __builtin_amdgcn_sched_barrier(0);
    float ts1 = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      acc[g & 1] = mfma32<PB>(vf[g], p0[g >> 1], acc[g & 1]);
      softmax_chunk(1, g, s1, p1, ts1);
      __builtin_amdgcn_sched_barrier(0);
    }
    read_v(1, vf);
    settle(s1, p1, ts1);
    __builtin_amdgcn_sched_barrier(0);
    // the step's staging tail (V conversion) runs beside the last P.V MFMAs
    tail();
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[g & 1] = mfma32<PB>(vf[g], p1[g >> 1], acc[g & 1]);
  };

  // One step: the loads of pair t+1 (K straight into the other slot, V into
  // the raw area) are issued first, then this wave's tile of pair t is
  // computed from slot t%2; V of pair t+1 is converted into the other slot
  // beside the tile's last MFMAs; barrier.
  auto step = [&](int t, auto slot_c) {
    constexpr int cs = decltype(slot_c)::value;  // t % 2
    unsigned char* nxt = slot_ptr(cs ^ 1);
    const bool active = 2 * t + par < T;
    // This step's rel_h (loaded a step ago) and, at a new column band, its
    // rel_w are waited for before the staging loads are issued: the compiler
    // does not count those, so a wait it inserted later for an older load
    // would also wait for them.  Then the next step's rel_h is prefetched.
    // An idle step (the odd wave's last one when T is odd) runs the same code
    // with rel_h = -inf: every score is -inf, every p 0, and O, l, m stay as
    // they are (a branch around the tile would make the compiler copy O).
#pragma unroll
    for (int r = 0; r < 4; ++r) rh[r] = active ? rh_next[r] : -__builtin_inff();
    __asm__ volatile("" ::"v"(rh[0]), "v"(rh[1]), "v"(rh[2]), "v"(rh[3]));
    if (active && pc.kw != band_kw) {
      band_kw = pc.kw;
      load_band(pc.kw);
      __asm__ volatile("" ::"v"(rwc[0]), "v"(rwc[4]));
    }
    {
      const TilePos pn = next_tile(next_tile(pc, H), H);
      if (pn.kw < W) load_rh(pn.kh);
    }
    // The loads of pair t+1 (issued right away: their latency is hidden by
    // this step's compute).
    auto stage = [&]() {
      stage_pair(0, krs0, vrs0, pk, (cs ^ 1) * kSlotBytes12);
      if (two) stage_pair(1, krs1, vrs1, pk, (cs ^ 1) * kSlotBytes12 + kPairBytes12);
    };
    stage();
    compute(slot_ptr(cs), [&]() {
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (v_wave) {
        v_convert(0, nxt);
        if (two) v_convert(1, nxt + kPairBytes12);
      }
    });
    __syncthreads();
    pc = next_tile(next_tile(pc, H), H);
    pk = next_tile(next_tile(pk, H), H);
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // Waves 0..7, which issue no staging load (unless V is converted), take
  // precedence over the staging waves 8..11 in the issue arbitration through
  // the key loop: 62.2 against 62.5 us at 64x64 on one box, 64.1-64.2
  // against 64.4 on another (the staging waves first: 65.7 us).
  if (v_wave) __builtin_amdgcn_s_setprio(1);
  int t = 0;
  for (; t + 1 < steps; t += 2) {
    step(t, S0{});
    step(t + 1, S1{});
  }
  if (t < steps) step(t, S0{});
  __builtin_amdgcn_s_setprio(0);

  // ---- merge the two waves of each block through LDS, store ---------------------
  const float lt = l + __shfl_xor(l, 32);
  if (lt == 0.0f) m = -__builtin_inff();  // a wave with no key (odd wave, T == 1) carries no weight
  float* mine = reinterpret_cast<float*>(smem + wave * kMergeStride12);
  const float* theirs = reinterpret_cast<const float*>(smem + (wave ^ 1) * kMergeStride12);
  // the partner finalises output columns 32*(1-par) .. : it needs acc[1-par]
#pragma unroll
  for (int r = 0; r < 16; ++r) mine[r * 64 + lane] = par ? acc[0][r] : acc[1][r];
  if (half == 0) {
    mine[16 * 64 + ql] = m;
    mine[16 * 64 + 32 + ql] = lt;
  }
  __syncthreads();
  const float mp = theirs[16 * 64 + ql];
  const float lp = theirs[16 * 64 + 32 + ql];
  const float mx = __builtin_fmaxf(m, mp);
  const float wa = exp2_fast(m - mx), wb = exp2_fast(mp - mx);
  const float inv = 1.0f / (lt * wa + lp * wb);
  const float ca = wa * inv, cb = wb * inv;
  // This wave's output columns 32*par .. 32*par + 31 of its 32 queries go
  // through LDS (query-major) so that every store writes whole rows of 32
  // values: 128-byte (fp32) or 64-byte (half) pieces, not 16- or 8-byte ones
  // that would reach memory as partial lines.
  float* ostage = reinterpret_cast<float*>(smem + kOutBase12) + wave * 32 * kOutStride12;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    f32x4 o4;
#pragma unroll
    for (int e = 0; e < 4; ++e) o4[e] = (par ? acc[1][4 * g + e] : acc[0][4 * g + e]) * ca + theirs[(4 * g + e) * 64 + lane] * cb;
    *reinterpret_cast<f32x4*>(ostage + ql * kOutStride12 + 8 * g + 4 * half) = o4;
  }
  // the rows are read back by other lanes of this wave only
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (!bvalid) return;
  const int rows_here = N - q0 < 32 ? N - q0 : 32;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * i + (lane >> 3);  // query row of the block
    const int c = 4 * (lane & 7);       // first of this lane's 4 columns
    const f32x4 o4 = *reinterpret_cast<const f32x4*>(ostage + r * kOutStride12 + c);
    if (r < rows_here) {
      const size_t at = (head + q0 + r) * kD + 32 * par + c;
      if constexpr (OUT_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + at) = o4;
      } else {
        const u32x2 pk2 = BF16 ? u32x2{pack_bf16(o4[0], o4[1]), pack_bf16(o4[2], o4[3])}
                               : u32x2{pack_f16(o4[0], o4[1]), pack_f16(o4[2], o4[3])};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + at) = pk2;
      }
    }
  }
}

// Unit `it`-th of this workgroup in a persistent grid over `units` units:
// XCD x (workgroups with blockIdx % 8 == x) takes a contiguous range of units,
// its workgroups every n_x-th of them; `units` when there is none left.
__device__ __forceinline__ int persistent_unit(int it, int units) {
  const int P = static_cast<int>(gridDim.x);
  const int x = static_cast<int>(blockIdx.x) & 7;
  const int per = units >> 3, rem = units & 7;
  const int start = x * per + (x < rem ? x : rem);
  const int cnt = per + (x < rem ? 1 : 0);
  const int nx = (P >> 3) + ((P & 7) > x ? 1 : 0);
  const int li = (static_cast<int>(blockIdx.x) >> 3) + it * nx;
  return li < cnt ? start + li : units;
}

template <bool BF16, bool OUT_F32, bool ALIGNED, bool PB, bool FUSED>
__global__ __launch_bounds__(kThreads12, 1) void attn12_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ rel_h,
    const float* __restrict__ rel_w, void* __restrict__ out,
    const uint16_t* __restrict__ th, const uint16_t* __restrict__ tw, float* __restrict__ ws,
    int H, int W, int nblk, int total_blocks, int units, float c2, float rw_mul, int zero_q) {
  if constexpr (FUSED) {
    // one workgroup per compute unit, each with its own bias slot, over all units
    // Units inside one head keep their bias rows in LDS where they fit (H, W
    // <= 64); units spanning two heads stage two heads' K/V per slot and use
    // the workspace slot (formed from the tables staged in LDS on such grids).
    const bool lds_fits = PB && H <= kLbMaxSide && W <= kLbMaxSide;
    for (int it = 0;; ++it) {
      const int unit = persistent_unit(it, units);
      if (unit >= units) break;
      const int gb0 = unit * kBlocks12;
      const int gb_last = gb0 + kBlocks12 - 1;
      if constexpr (PB) {
        if (lds_fits) {
          if (gb_last < total_blocks && gb_last / nblk == gb0 / nblk) {
            attn12_unit<BF16, OUT_F32, ALIGNED, PB, true, true>(q, k, v, rel_h, rel_w, out, th, tw, ws, H, W, nblk,
                                                                total_blocks, c2, rw_mul, zero_q, unit);
          } else {
            attn12_unit<BF16, OUT_F32, ALIGNED, PB, true, false, true>(q, k, v, rel_h, rel_w, out, th, tw, ws, H,
                                                                       W, nblk, total_blocks, c2, rw_mul, zero_q,
                                                                       unit);
          }
          __syncthreads();  // the next unit reuses the LDS and the slot
          continue;
        }
      }
      attn12_unit<BF16, OUT_F32, ALIGNED, PB, true>(q, k, v, rel_h, rel_w, out, th, tw, ws, H, W, nblk,
                                                    total_blocks, c2, rw_mul, zero_q, unit);
      __syncthreads();  // the next unit reuses the LDS and the slot
    }
  } else {
    attn12_unit<BF16, OUT_F32, ALIGNED, PB, false>(q, k, v, rel_h, rel_w, out, th, tw, ws, H, W, nblk,
                                                   total_blocks, c2, rw_mul, zero_q,
                                                   xcd_work_index(static_cast<int>(gridDim.x)));
  }
}

template <bool BF16, bool OUT_F32, bool ALIGNED, bool PB, bool FUSED>
hipError_t launch12(const AttnArgs& a, hipStream_t stream) {
  auto kern = attn12_kernel<BF16, OUT_F32, ALIGNED, PB, FUSED>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds12);
  if (err != hipSuccess) return err;
  const int N = a.H * a.W;
  const int nblk = (N + 31) / 32;
  const int total = nblk * a.BH;
  const int units = (total + kBlocks12 - 1) / kBlocks12;
  const bool zero_q = a.scale == 0.0f;
  const float c2 = zero_q ? kLog2e : a.scale * kLog2e;
  const float rw_mul = zero_q ? 1.0f : kLog2e / c2;
  const int grid = FUSED ? (units < a.split_ctas ? units : a.split_ctas) : units;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kThreads12), kLds12, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.rel_h, a.rel_w, a.out,
                     static_cast<const uint16_t*>(a.th), static_cast<const uint16_t*>(a.tw),
                     static_cast<float*>(a.ws), a.H, a.W, nblk, total, units, c2, rw_mul, zero_q ? 1 : 0);
  return hipGetLastError();
}

template <bool BF16, bool OUT_F32, bool PB>
hipError_t launch12_al(const AttnArgs& a, hipStream_t stream) {
  const bool aligned = a.H % kTileRows == 0 && a.W % kTileCols == 0;
  return aligned ? launch12<BF16, OUT_F32, true, PB, false>(a, stream)
                 : launch12<BF16, OUT_F32, false, PB, false>(a, stream);
}

}  // namespace

size_t attn12_lds_bytes() { return kLds12; }

bool attn12_bf16_p(int H, int W) { return H * W >= kBf16PMinKeys; }

bool attn12_fits(int H, int W) {
  // A workgroup's 6 blocks must span at most two heads.
  return (H * W + 31) / 32 >= kBlocks12;
}

hipError_t launch_attn12(const AttnArgs& a, hipStream_t stream) {
  if (a.bf16) {
    if (attn12_bf16_p(a.H, a.W))
      return a.out_f32 ? launch12_al<true, true, true>(a, stream) : launch12_al<true, false, true>(a, stream);
    return a.out_f32 ? launch12_al<true, true, false>(a, stream) : launch12_al<true, false, false>(a, stream);
  }
  return a.out_f32 ? launch12_al<false, true, false>(a, stream) : launch12_al<false, false, false>(a, stream);
}

}  // namespace relpos

namespace relpos {

bool attn_fused12_lds_bias(int H, int W) { return H <= kLbMaxSide && W <= kLbMaxSide; }

bool attn_fused12_ok(int H, int W, bool bf16) {
  // whole-row blocks (each block of 32 queries inside one grid row), whole
  // 4 x 16 key tiles, bf16 P
  return bf16 && W % 32 == 0 && H % 4 == 0 && attn12_fits(H, W) && attn12_bf16_p(H, W);
}

size_t attn_fused12_workspace_bytes(int64_t BH, int H, int W, int ctas) {
  // One slot per workgroup of the persistent grid of min(units, ctas); with
  // H, W <= 64 only the units spanning two heads or partial use one, so
  // min(B*heads, workgroups) slots.
  const int64_t units = (BH * ((static_cast<int64_t>(H) * W + 31) / 32) + kBlocks12 - 1) / kBlocks12;
  int64_t slots = units < ctas ? units : ctas;
  if (attn_fused12_lds_bias(H, W) && BH < slots) slots = BH;
  return static_cast<size_t>(slots) * kBlocks12 * 32 * (H + W) * 4;
}

hipError_t launch_attn_fused12(const AttnArgs& a, hipStream_t stream) {
  // H % 4 == 0 and W % 32 == 0 (attn_fused12_ok): the aligned tile path
  return a.out_f32 ? launch12<true, true, true, true, true>(a, stream)
                   : launch12<true, false, true, true, true>(a, stream);
}

}  // namespace relpos
