// relpos_build kernel: per-query relative-position logits along each grid axis
// (PR #55629 page, key source snippet, the add_decomposed_rel_pos call on the
// unscaled q; table index qh - kh + H - 1, resp. qw - kw + W - 1).
//
// For a fixed query grid row qh the W queries of that row all use the same
// window of H table rows, reversed: rel_h[qh*W + m, n] = q[qh*W + m] . T_h[qh - n + H - 1].
// That is a [W x 64] x [64 x H] product, done here with 32x32x16 MFMA (bf16 or
// fp16 products are exact in fp32, accumulation is fp32).  rel_w is the same
// with the roles of the axes swapped: for a fixed grid column qw, the H queries
// m*W + qw against T_w[qw - n + W - 1].
//
// Grid: x = H + W (one workgroup per grid row, then per grid column), y = B*heads.
// The waves of a workgroup share out its 32x32 output tiles.
#include "relpos_device.hpp"
#include "relpos_kernels.hpp"

namespace relpos {

namespace {

constexpr int kD = 64;

template <bool BF16>
__global__ __launch_bounds__(256) void build_kernel(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ th,
                                                    const uint16_t* __restrict__ tw,
                                                    float* __restrict__ rel_h,
                                                    float* __restrict__ rel_w, int H, int W) {
  const int N = H * W;
  const size_t head = static_cast<size_t>(blockIdx.y) * N;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;

  // Problem for this workgroup: rows m < M are queries (base + m*stride),
  // columns n < NC index the output axis, table row = tbase - n.
  int M, NC, base, stride, tbase, ldo;
  const uint16_t* tab;
  float* dst;
  if (static_cast<int>(blockIdx.x) < H) {
    const int qh = blockIdx.x;
    M = W; NC = H; base = qh * W; stride = 1; tbase = qh + H - 1; tab = th; dst = rel_h; ldo = H;
  } else {
    const int qw = blockIdx.x - H;
    M = H; NC = W; base = qw; stride = W; tbase = qw + W - 1; tab = tw; dst = rel_w; ldo = W;
  }
  const int mt_n = (M + 31) / 32, nt_n = (NC + 31) / 32;

  for (int tile = wave; tile < mt_n * nt_n; tile += 4) {
    const int mt = tile / nt_n, nt = tile - mt * nt_n;
    const int m = mt * 32 + (lane & 31);
    const int n = nt * 32 + (lane & 31);
    const bool mok = m < M, nok = n < NC;
    const uint16_t* qrow = q + (head + base + static_cast<size_t>(m) * stride) * kD;
    const uint16_t* trow = tab + static_cast<size_t>(nok ? tbase - n : 0) * kD;
    f32x16 acc{};
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) {
      const u32x4 a = mok ? *reinterpret_cast<const u32x4*>(qrow + 16 * kd + 8 * half) : u32x4{0, 0, 0, 0};
      const u32x4 b = nok ? *reinterpret_cast<const u32x4*>(trow + 16 * kd + 8 * half) : u32x4{0, 0, 0, 0};
      acc = mfma32<BF16>(a, b, acc);
    }
    if (nok) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mr = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (mr < M) dst[(head + base + static_cast<size_t>(mr) * stride) * ldo + n] = acc[r];
      }
    }
  }
}

}  // namespace

hipError_t launch_build(const BuildArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(a.H + a.W), static_cast<unsigned>(a.BH));
  if (a.bf16) {
    hipLaunchKernelGGL(build_kernel<true>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.rel_pos_h),
                       static_cast<const uint16_t*>(a.rel_pos_w), a.rel_h, a.rel_w, a.H, a.W);
  } else {
    hipLaunchKernelGGL(build_kernel<false>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.rel_pos_h),
                       static_cast<const uint16_t*>(a.rel_pos_w), a.rel_h, a.rel_w, a.H, a.W);
  }
  return hipGetLastError();
}

}  // namespace relpos
