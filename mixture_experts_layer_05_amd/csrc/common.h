// Internal helpers shared by the library's kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront
constexpr int kGroup = 128;        // fp8 scale group along the contraction dim
constexpr int kMxBlock = 32;       // MX (microscaling) block along the contraction dim
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 16;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte loads: plain (cached) and streaming (non-temporal, for weights read once).
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v.x, v.y, v.z, v.w};
}

// Raw buffer loads: a scalar resource (base, size in bytes) plus a 32-bit
// per-lane offset and a scalar offset.  Loads past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float silu_f32(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }
__device__ __forceinline__ float sigmoid_f32(float a) { return 1.0f / (1.0f + __expf(-a)); }

// ---------------------------------------------------------------- MFMA wrappers

// D(16x16,f32) += A(16x32,bf16) * B(32x16,bf16).  Lane l supplies row (A) / column
// (B) l%16 and eight contraction elements of lane group l/16; both operands use
// the same contraction placement, so any consistent assignment of k to
// (lane group, element) computes the same sum.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(16x16,f32) = A(16x128,e4m3) * B(128x16,e4m3) + C, 32 codes per lane.  The
// block-scale operands are set to the E8M0 encoding of 1.0 (127), so this is
// the plain fp8 product; group scales are applied by the caller in float32.
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// D(16x16,f32) += A(16x128, MXFP8 e4m3 codes) * B(128x16, MXFP4 e2m1 codes), both
// scaled by E8M0 block scales in the matrix core.  Lane l supplies A row / B column
// l%16.  A uses the 8-bit operand layout (lane group g = l/16 holds contraction
// elements [16g, +16) in bytes 0..15 and [64+16g, +16) in bytes 16..31); B the
// 4-bit layout (lane group g holds elements [32g, +32), element 2i in the low
// nibble of byte i, upper four dwords unused).  sa / sb: the E8M0 code of
// contraction block g (elements [32g, +32)) of the lane's row / column.
__device__ __forceinline__ f32x4 mfma_mxfp8_mxfp4_16x16x128(i32x8 a, i32x8 b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, sb);
}

// Output placement of the 16x16 MFMAs: lane l, element i -> row 4*(l/16)+i, column l%16.
__device__ __forceinline__ int mfma16_row(int lane, int i) { return 4 * (lane >> 4) + i; }
__device__ __forceinline__ int mfma16_col(int lane) { return lane & 15; }

// ---------------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ---------------------------------------------------------------- misc

__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr inline size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

}  // namespace moe
