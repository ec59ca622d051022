// relpos_build kernel: per-query relative-position logits along each grid axis
// (PR #55629 page, key source snippet, the add_decomposed_rel_pos call on the
// unscaled q; table index qh - kh + H - 1, resp. qw - kw + W - 1).
//
// The kernel writes 8 bytes of bias per byte of q it reads (D = 64, H + W
// fp32 values per query against 64 bf16/fp16 values), so it is bound by HBM
// writes.  Each q row is read once for both axes, and every output goes out
// in 16-byte stores over contiguous rows.
//
// A workgroup is one wave and owns a unit of up to 32 consecutive queries of
// one grid row qh (columns qw = m0 .. m0 + 31):
//   * rel_h: all queries of the unit use the same table rows, reversed:
//     rel_h[m, kh] = q[m] . T_h[qh - kh + H - 1], a [32 x 64] x [64 x H]
//     product on 32x32x16 MFMA (bf16/fp16 products are exact in fp32,
//     accumulation is fp32), 64 columns at a time.
//   * rel_w: the table row depends on qw - kw, so for 64 output columns
//     kw = n0 .. n0 + 63 the wave forms G[m', j] = q[m0 + m'] . T_w[tlo + j]
//     over the 95 table rows tlo .. tlo + 94 those columns reach (tlo = m0 -
//     n0 - 63 + W - 1), i.e. 96 columns of MFMA output, and reads the output
//     back along the diagonal: rel_w[m0 + m', n0 + n'] = G[m', m' - n' + 63].
// Either product is staged in LDS (row strides of 72 and 104 floats, which
// put the two 32-lane halves of an MFMA result store on disjoint banks) and
// stored as rows of 16-byte pieces.  All loads are branch-free raw buffer
// loads (zeros past a tensor's end), so a chunk's q and table loads are in
// flight together and the next chunk's are issued before this one's stores.
//
// Grid: B*heads * H * ceil(W/32) units, 1-D and XCD-matched to the attention
// kernels' query blocks.  Written on another XCD than the one whose L2 had
// just read them in the attention call, the rows took 15.4-17.5 us at 64x64
// with 12 heads (right after that call) against 9.6 us now.  Grids of more
// than 2^26 units fall back to x = units of one (b, h), y = B*heads.
//
// Small grids (H, W <= 32, e.g. windows of 14x14) take a second kernel: there
// a unit of the kernel above covers one grid row of W < 32 queries and a
// 64-column MFMA product of which it uses H or W columns, and its rows of H
// or W floats are too short for 16-byte stores.  Instead a unit is 32
// consecutive queries of one (b, h) in token order; both tables have at most
// 63 rows, so the unit forms the full products Gh = Q T_h^T and Gw = Q T_w^T
// (2 x 32 columns each), stages them in LDS and writes its rel_h and rel_w
// rows, which are contiguous in memory, as one run of 16-byte pieces each:
// element f of the run is row m = f / H (f / W), column c of query i = i0 + m,
// taken from Gh[m, qh - c + H - 1] (Gw[m, qw - c + W - 1]).
#include "relpos_attn_common.hpp"
#include "relpos_device.hpp"
#include "relpos_kernels.hpp"

namespace relpos {

namespace {

constexpr int kD = 64;
constexpr int kHStride = 72;   // floats per staged rel_h row (64 used)
constexpr int kGStride = 104;  // floats per staged G row (95 used)
// Table windows staged in LDS by build_kernel: 64 rows of T_h (8 KB) then 96
// rows of T_w (12 KB), 128-byte rows whose 16-byte chunk c sits at chunk c ^
// (row % 8).
constexpr int kWinH = 0, kWinW = 8192, kWinBytes = 20480;
static_assert(32 * kGStride * 4 <= kWinBytes, "the product staging must fit the window area");
__device__ __forceinline__ int win_off(int r, int c) { return r * 128 + 16 * (c ^ (r & 7)); }

// Cache policy of the row stores of build_kernel: sc1 (device scope: written
// through to memory, so the kernel ends with no dirty L2 lines of rows to
// write back) and nt (streaming).  Back to back: 9.1-9.2 against 9.6 us at
// 64x64 with 12 heads, 54.7-55.1 against 56.8 us at 96x96 with 32 heads,
// 25.5 against 24.5 us for 4 x 12 heads of 64x64 (nt alone: the previous
// figures; plain stores 10.9-11.3 us at 64x64).  The small-grid kernel keeps
// plain non-temporal stores (its 14x14 windows: 7.3-7.5 against 8.4-8.6 us
// written through).
constexpr int kRowStorePolicy = 16 | 2;

// 16 bytes of output: 4 consecutive floats of one row from column n (a
// multiple of 4) on, the part below `cols` (a row's length) written; one
// 16-byte buffer store where the rows keep 16-byte alignment (cols % 4 == 0,
// the tensors being 16-byte aligned), else one 4-byte store per float.  `rs`
// covers the unit's rows, `off` is the byte offset of the row in it.
__device__ __forceinline__ void store_row4(__amdgpu_buffer_rsrc_t rs, int off, int n, int cols, f32x4 v) {
  if ((cols & 3) == 0) {
    if (n < cols) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off + 4 * n, 0, kRowStorePolicy);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (n + e < cols) {
        __builtin_amdgcn_raw_buffer_store_b32(as_uint(v[e]), rs, off + 4 * (n + e), 0, kRowStorePolicy);
      }
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(64) void build_kernel(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ th,
                                                   const uint16_t* __restrict__ tw,
                                                   float* __restrict__ rel_h,
                                                   float* __restrict__ rel_w, int H, int W, int mtn) {
  // 20 KB: the table windows the wave's MFMA operands come from (T_h rows at
  // 0, T_w rows at 8 KB), then, once those operands are in registers, the
  // staging area of both products (13 KB; the rel_h pass ends with a barrier
  // before the rel_w pass writes).  8 one-wave workgroups per CU.
  __shared__ __attribute__((aligned(16))) float stage[kWinBytes / 4];
  float* const stage_h = stage;
  float* const stage_g = stage;
  const int lane = threadIdx.x;
  const int ml = lane & 31, half = lane >> 5;
  // Units in (b*heads, grid row, 32-query chunk) order.  On the 1-D grid the
  // workgroups dispatched to one XCD take a contiguous range of them, as the
  // attention kernels do with their query blocks, so each XCD writes the rows
  // it reads in the attention call (and read in the previous one).
  int bhi, u;
  const int per_head = H * mtn;
  if (gridDim.y == 1) {
    const int unit = attn::xcd_work_index(static_cast<int>(gridDim.x));
    bhi = unit / per_head;
    u = unit - bhi * per_head;
  } else {
    bhi = blockIdx.y;
    u = blockIdx.x;
  }
  const int qh = u / mtn;
  const int m0 = (u - qh * mtn) * 32;
  const int rows = W - m0 < 32 ? W - m0 : 32;
  const size_t row0 = static_cast<size_t>(bhi) * H * W + static_cast<size_t>(qh) * W + m0;

  // Every load is a raw buffer load whose out-of-range offsets read zeros:
  // no branch, so all of a chunk's loads are in flight together.
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + row0 * kD, static_cast<uint32_t>(rows) * kD * 2);
  const int dchunk = 16 * half;  // byte offset of this lane's 8 d values within a 16-wide slice
  // the unit's rel_h and rel_w rows (store targets)
  const __amdgpu_buffer_rsrc_t rsh =
      make_rsrc(rel_h + row0 * H, static_cast<uint32_t>(rows) * static_cast<uint32_t>(H) * 4);
  const __amdgpu_buffer_rsrc_t rsw =
      make_rsrc(rel_w + row0 * W, static_cast<uint32_t>(rows) * static_cast<uint32_t>(W) * 4);

  // A operand: query m0 + ml, d = 16*kd + 8*half .. +7
  u32x4 a[4];
#pragma unroll
  for (int kd = 0; kd < 4; ++kd) a[kd] = buf_load16(rq, ml < rows ? ml * kD * 2 + 32 * kd + dchunk : kOob);

  // B operands: table row per output column (rel_h) or per G column (rel_w).
  // Each chunk's rows form one contiguous window of the table, staged in LDS
  // by LDS-direct loads of 1 KB (8 rows) each: the 64 lanes of a load touch 8
  // cache lines, where loading the operands straight from the table touches
  // 32 (one row per lane), which made the CU's vector-memory path the limit
  // of the kernel's first microseconds (loads landed 3.6 us after the start
  // at 64x64 with 12 heads).  Rows outside the table read zeros (negative
  // offsets are out of range as unsigned offsets too).
  const uint32_t lds0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(
      reinterpret_cast<size_t>((__attribute__((address_space(3))) float*)stage))));
  const sgpr4 wth = rsrc_words(th, static_cast<uint32_t>(2 * H - 1) * kD * 2);
  const sgpr4 wtw = rsrc_words(tw, static_cast<uint32_t>(2 * W - 1) * kD * 2);
  // window of `rows8` pieces of 8 rows from table row t0 at LDS byte `at`
  auto stage_window = [&](const sgpr4& rs, int t0, int rows8, int at) {
    for (int p = 0; p < rows8; ++p) {
      const int r = 8 * p + (lane >> 3);
      lds_load16(rs, (t0 + r) * kD * 2 + 16 * ((lane & 7) ^ (r & 7)), 0, lds0 + at + 1024 * p);
    }
  };
  // chunk n0 of rel_h: kh = n0 + j (j < 64) takes table row qh - kh + H - 1,
  // window row 63 - j of the window from row qh + H - 1 - n0 - 63
  auto window_h = [&](int n0) { stage_window(wth, qh + H - 1 - n0 - 63, 8, kWinH); };
  // chunk n0 of rel_w: G column j (< 96) takes table row tlo + j
  auto window_w = [&](int n0) { stage_window(wtw, m0 - n0 - 63 + W - 1, 12, kWinW); };
  const unsigned char* const win = reinterpret_cast<const unsigned char*>(stage);
  u32x4 bh[2][4], bw[3][4];
  auto read_h = [&]() {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int kd = 0; kd < 4; ++kd)
        bh[nt][kd] = *reinterpret_cast<const u32x4*>(win + kWinH + win_off(63 - 32 * nt - ml, 2 * kd + half));
    }
  };
  auto read_w = [&]() {
#pragma unroll
    for (int gt = 0; gt < 3; ++gt) {
#pragma unroll
      for (int kd = 0; kd < 4; ++kd)
        bw[gt][kd] = *reinterpret_cast<const u32x4*>(win + kWinW + win_off(32 * gt + ml, 2 * kd + half));
    }
  };
  // before the windows are staged again over the product staging: this
  // wave's reads of it are complete
  auto lds_idle = [&]() { __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
  window_h(0);
  window_w(0);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  read_h();
  read_w();

  // MFMA output register r of this lane: row 8*(r/4) + 4*half + r%4, column ml.
  auto out_row = [&](int r) { return 8 * (r >> 2) + 4 * half + (r & 3); };
  // Store pass: lane covers columns sc .. sc+3 of rows lane/16 + 4i.
  const int sc = 4 * (lane & 15);
  const int sr = lane >> 4;

  // ---- rel_h --------------------------------------------------------------------
  for (int n0 = 0; n0 < H; n0 += 64) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x16 acc{};
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) acc = mfma32<BF16>(a[kd], bh[nt][kd], acc);
#pragma unroll
      for (int r = 0; r < 16; ++r) stage_h[out_row(r) * kHStride + 32 * nt + ml] = acc[r];
    }
    __syncthreads();
    f32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const f32x4*>(stage_h + (sr + 4 * i) * kHStride + sc);
    if (n0 + 64 < H) {
      lds_idle();
      window_h(n0 + 64);
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      read_h();
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = sr + 4 * i;
      if (m < rows) store_row4(rsh, m * H * 4, n0 + sc, H, v[i]);
    }
    __syncthreads();
  }

  // ---- rel_w --------------------------------------------------------------------
  for (int n0 = 0; n0 < W; n0 += 64) {
#pragma unroll
    for (int gt = 0; gt < 3; ++gt) {
      f32x16 g{};
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) g = mfma32<BF16>(a[kd], bw[gt][kd], g);
#pragma unroll
      for (int r = 0; r < 16; ++r) stage_g[out_row(r) * kGStride + 32 * gt + ml] = g[r];
    }
    __syncthreads();
    // columns n0 + sc + e of row m take G[m, m - sc - e + 63]
    f32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = sr + 4 * i;
      const float* gp = stage_g + m * kGStride + m - sc + 63;
      v[i] = f32x4{gp[0], gp[-1], gp[-2], gp[-3]};
    }
    if (n0 + 64 < W) {
      lds_idle();
      window_w(n0 + 64);
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      read_w();
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = sr + 4 * i;
      if (m < rows) store_row4(rsw, m * W * 4, n0 + sc, W, v[i]);
    }
    __syncthreads();
  }
}

// x / d for 0 <= x < 2048 and 1 <= d <= 32, with m = ceil(2^16 / d): the
// error of x*m / 2^16 against x/d is below x/2^16 < 1/32 <= 1/d.
__device__ __forceinline__ int div_small(int x, uint32_t m) { return static_cast<int>((static_cast<uint32_t>(x) * m) >> 16); }

template <bool BF16>
__global__ __launch_bounds__(64) void build_small_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ th,
                                                         const uint16_t* __restrict__ tw,
                                                         float* __restrict__ rel_h,
                                                         float* __restrict__ rel_w, int H, int W, int upb,
                                                         uint32_t mh, uint32_t mw) {
  // The products gh, gw (32 rows of 72 floats each); before them, the two
  // tables (rows of 128 bytes, chunk c of row r at chunk c ^ (r % 8); T_h at
  // 0, T_w at 8 KB), staged by LDS-direct loads and read into registers.
  __shared__ __attribute__((aligned(16))) float gsm[2 * 32 * kHStride];
  static_assert(2 * 32 * kHStride * 4 >= 16384, "both tables must fit the product area");
  float* const gh = gsm;
  float* const gw = gsm + 32 * kHStride;
  const int lane = threadIdx.x;
  const int ml = lane & 31, half = lane >> 5;
  // units in (b*heads, 32-query block) order, XCD-matched like the kernel above
  const int unit = attn::xcd_work_index(static_cast<int>(gridDim.x));
  const int bhi = unit / upb;
  const int i0 = (unit - bhi * upb) * 32;
  const int N = H * W;
  const int rows = N - i0 < 32 ? N - i0 : 32;
  const size_t row0 = static_cast<size_t>(bhi) * N + i0;

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + row0 * kD, static_cast<uint32_t>(rows) * kD * 2);
  const int dchunk = 16 * half;
  u32x4 a[4], bh[2][4], bw[2][4];
#pragma unroll
  for (int kd = 0; kd < 4; ++kd) a[kd] = buf_load16(rq, ml < rows ? ml * kD * 2 + 32 * kd + dchunk : kOob);
  // B operands: table row j = 32*nt + ml (both tables have at most 63 rows,
  // zeros past the last).  The tables go to LDS by LDS-direct loads of 8 rows
  // each (8 cache lines per load, against 32 when each lane loads its own
  // row), as in the kernel above; rows past the staged pieces hold whatever
  // LDS held, and only feed product columns past 2L - 2, which are not read.
  {
    const uint32_t lds0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(
        reinterpret_cast<size_t>((__attribute__((address_space(3))) float*)gsm))));
    const sgpr4 wth = rsrc_words(th, static_cast<uint32_t>(2 * H - 1) * kD * 2);
    const sgpr4 wtw = rsrc_words(tw, static_cast<uint32_t>(2 * W - 1) * kD * 2);
    const int ph = (2 * H - 1 + 7) / 8, pw = (2 * W - 1 + 7) / 8;
    for (int p = 0; p < 8; ++p) {
      const int r = 8 * p + (lane >> 3);
      const int off = r * kD * 2 + 16 * ((lane & 7) ^ (r & 7));
      if (p < ph) lds_load16(wth, off, 0, lds0 + 1024 * p);
      if (p < pw) lds_load16(wtw, off, 0, lds0 + 8192 + 1024 * p);
    }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const unsigned char* const tb = reinterpret_cast<const unsigned char*>(gsm);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int j = 32 * nt + ml;  // table row
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) {
        const int off = j * 128 + 16 * ((2 * kd + half) ^ (j & 7));
        bh[nt][kd] = *reinterpret_cast<const u32x4*>(tb + off);
        bw[nt][kd] = *reinterpret_cast<const u32x4*>(tb + 8192 + off);
      }
    }
  }
  auto out_row = [&](int r) { return 8 * (r >> 2) + 4 * half + (r & 3); };
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    f32x16 ch{}, cw{};
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) {
      ch = mfma32<BF16>(a[kd], bh[nt][kd], ch);
      cw = mfma32<BF16>(a[kd], bw[nt][kd], cw);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      gh[out_row(r) * kHStride + 32 * nt + ml] = ch[r];
      gw[out_row(r) * kHStride + 32 * nt + ml] = cw[r];
    }
  }
  __syncthreads();

  // One run per table: rows*L floats from element (row0 * L) on; 16-byte
  // stores where the run starts 16-byte aligned, else one store per float.
  auto emit = [&](float* __restrict__ dst, const float* g, int L, uint32_t mL, bool is_h) {
    const int total = rows * L;
    const bool al = ((row0 * static_cast<size_t>(L)) & 3) == 0;
    float* run = dst + row0 * L;
    for (int f0 = 4 * lane; f0 < total; f0 += 256) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = f0 + e < total ? f0 + e : total - 1;
        const int m = div_small(f, mL);
        const int c = f - m * L;
        const int i = i0 + m;
        const int qr = div_small(i, mw);  // grid row of query i
        const int a_ = is_h ? qr : i - qr * W;
        v[e] = g[m * kHStride + a_ - c + L - 1];
      }
      if (al && f0 + 3 < total) {
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(run + f0));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (f0 + e < total) run[f0 + e] = v[e];
        }
      }
    }
  };
  emit(rel_h, gh, H, mh, true);
  emit(rel_w, gw, W, mw, false);
}

}  // namespace

hipError_t launch_build(const BuildArgs& a, hipStream_t stream) {
  const int64_t upb = (static_cast<int64_t>(a.H) * a.W + 31) / 32;
  if (a.H <= 32 && a.W <= 32 && upb * a.BH <= INT32_MAX) {
    const uint32_t mh = (65536u + a.H - 1) / a.H, mw = (65536u + a.W - 1) / a.W;
    const dim3 grid(static_cast<unsigned>(upb * a.BH));
    if (a.bf16) {
      hipLaunchKernelGGL(build_small_kernel<true>, grid, dim3(64), 0, stream,
                         static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.rel_pos_h),
                         static_cast<const uint16_t*>(a.rel_pos_w), a.rel_h, a.rel_w, a.H, a.W,
                         static_cast<int>(upb), mh, mw);
    } else {
      hipLaunchKernelGGL(build_small_kernel<false>, grid, dim3(64), 0, stream,
                         static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.rel_pos_h),
                         static_cast<const uint16_t*>(a.rel_pos_w), a.rel_h, a.rel_w, a.H, a.W,
                         static_cast<int>(upb), mh, mw);
    }
    return hipGetLastError();
  }
  const int mtn = (a.W + 31) / 32;
  // 1-D (XCD-matched) up to 2^26 workgroups; beyond that x = units of one
  // (b, h), y = B*heads.
  const int64_t units = static_cast<int64_t>(a.H) * mtn;
  const bool flat = units * a.BH <= (int64_t(1) << 26);
  const dim3 grid = flat ? dim3(static_cast<unsigned>(units * a.BH))
                         : dim3(static_cast<unsigned>(units), static_cast<unsigned>(a.BH));
  if (a.bf16) {
    hipLaunchKernelGGL(build_kernel<true>, grid, dim3(64), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.rel_pos_h),
                       static_cast<const uint16_t*>(a.rel_pos_w), a.rel_h, a.rel_w, a.H, a.W, mtn);
  } else {
    hipLaunchKernelGGL(build_kernel<false>, grid, dim3(64), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.rel_pos_h),
                       static_cast<const uint16_t*>(a.rel_pos_w), a.rel_h, a.rel_w, a.H, a.W, mtn);
  }
  return hipGetLastError();
}

}  // namespace relpos
