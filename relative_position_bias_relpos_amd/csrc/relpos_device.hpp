// Device-side types and helpers shared by the librelpos kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace relpos {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;

// One 32x32x16 MFMA, C += A(32x16) * B(16x32), fp32 accumulate.  Each lane
// holds 8 consecutive-k elements of A (row lane%32) and of B (column lane%32);
// the lane half (lane/32) selects which 8 of the 16 k.  The two operands share
// the same k assignment, so any contraction laid out the same way on both is
// summed completely.  C: lane holds column lane%32, rows 8*(r/4)+4*(lane/32)+r%4.
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Bit casts through a by-value argument.  Apply these (not __builtin_bit_cast)
// to an element of an ext_vector: this compiler lowers a bit cast of a vector
// element expression as a read of the vector's first element.
__device__ __forceinline__ float as_float(uint32_t w) { return __builtin_bit_cast(float, w); }
__device__ __forceinline__ uint32_t as_uint(float x) { return __builtin_bit_cast(uint32_t, x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Packed fp16 pair -> two fp32 (exact).
__device__ __forceinline__ f32x2 unpack_f16(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
}

// Two fp32 -> packed fp16 pair (round to nearest even; overflow gives inf).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// Two fp32 -> packed bf16 pair, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  uint32_t a = __builtin_bit_cast(uint32_t, lo), b = __builtin_bit_cast(uint32_t, hi);
  a += 0x7fffu + ((a >> 16) & 1u);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (a >> 16) | (b & 0xffff0000u);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer loads: an offset at or past the resource's byte size returns
// zeros in hardware, which masks grid cells outside the tile without branches.
constexpr uint32_t kBufFlags = 0x00020000u;  // gfx9 raw-buffer descriptor word 3
constexpr int kOob = 0x7ffffff0;             // any offset past every resource used here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                          static_cast<int>(kBufFlags));
}
// `soff` is a wave-uniform byte offset (scalar register); callers that rely
// on the zero fill keep it 0 and put the whole offset in `off`.
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int off, int soff = 0) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
__device__ __forceinline__ float buf_loadf(__amdgpu_buffer_rsrc_t r, int off, int soff = 0) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
}

typedef uint32_t __attribute__((ext_vector_type(4))) sgpr4;

// Raw buffer descriptor words (base, no stride, `bytes` records, raw-buffer
// flags) for the LDS-direct load below; wave-uniform.
__device__ __forceinline__ sgpr4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32))) & 0xffffu;
  return sgpr4{lo, hi, bytes, kBufFlags};
}

// One LDS-direct 16-byte buffer load per lane: lane L's 16 bytes at byte
// offset voff + soff of the buffer land at LDS byte lds + 16*L (offsets past
// the buffer's size read zeros).  Written as asm because the compiler, which
// cannot tell LDS written this way from the LDS other instructions read,
// otherwise waits for every outstanding vector load before each LDS read and
// barrier that follows.  Nothing is returned in registers: the data is only
// read after an explicit vmcnt(0) wait of the loading wave (and a workgroup
// barrier where other waves read it).
__device__ __forceinline__ void lds_load16(sgpr4 rs, int voff, int soff, uint32_t lds) {
  __asm__ volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rs), "s"(soff), "s"(lds)
      : "memory", "m0");
}

}  // namespace relpos

namespace relpos {

// One 16x16x32 MFMA, C += A(16x32) * B(32x16), fp32 accumulate.  Each lane
// holds 8 consecutive-k elements of A (row lane%16) and of B (column lane%16);
// the lane group (lane/16) selects which 8 of the 32 k.  C: lane holds column
// lane%16, rows 4*(lane/16) + 0..3.
template <bool BF16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

}  // namespace relpos
