// Device helpers shared by the gfx950 (CDNA4) kernels of libgqa.
//
// Lane layouts used throughout (wave64, checked on gfx950 with known inputs):
//  * v_mfma_f32_32x32x16_bf16: A lane l holds row l%32, B lane l holds column
//    l%32, each with 8 bf16 of the reduction dimension (the same k positions
//    in A and B for the same lane and element); the 16 fp32 results of lane l
//    are D[(i/4)*8 + 4*(l/32) + i%4][l%32], i = 0..15.
//  * v_mfma_f32_16x16x32_bf16: A row l%16, B column l%16, 8 bf16 each; the 4
//    results of lane l are D[4*(l/16) + i][l%16], i = 0..3.
//  * ds_read_b64_tr_b16: in each group of 16 lanes, lane s supplies the address
//    of 4 consecutive 16-bit values M[s][0..3]; lane i receives
//    M[4j + i/4][i%4] for j = 0..3. If lane s = 4a + b points at
//    X[r0 + a][c0 + 4b] of a row-major 16-bit matrix, lane i receives the
//    column X[r0 .. r0+3][c0 + i]: a 4 x 16 block comes back transposed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes, kept in registers

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 of a pair (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<uint4*>(w));
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two transposing LDS reads joined into one 8-element MFMA operand. p0 and p1
// point into __shared__ memory (8-byte aligned).
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const uint16_t* p0, const uint16_t* p1) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Number of `unit`-sized pieces covering n (n >= 0).
__host__ __device__ __forceinline__ int div_up(int n, int unit) { return (n + unit - 1) / unit; }

}  // namespace gqa
