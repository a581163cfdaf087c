// Device-side helpers shared by the LC-VQ kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LCVQ_LDS __attribute__((address_space(3)))
// Constant address space: uniform reads through such a pointer become scalar loads.
#define LCVQ_CONST __attribute__((address_space(4)))

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// "R16" word: 16 consecutive 2-bit codes c0..c15 (along the contraction) stored so
// that each pair (c2p, c2p+1) expands to a bf16 pair with one shift and one
// and-or. A code c is represented in the GEMM operand by v(c) = 2 + c/2, whose bf16
// bit pattern is 0x4000 | c << 5 (exact); the callers undo the map c = 2 v - 4 in
// their other operand and in a per-row correction term.
//   W = place8(c0..c7) | rotl(place8(c8..c15), 8),
//   place8(a) = sum_p a[2p] << (5 + 2p) | a[2p+1] << (21 + 2p),  p = 0..3.
__host__ __device__ __forceinline__ uint32_t r16_place8(const uint32_t* a) {
  uint32_t w = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) w |= (a[2 * p] << (5 + 2 * p)) | (a[2 * p + 1] << (21 + 2 * p));
  return w;
}
__host__ __device__ __forceinline__ uint32_t r16_encode(const uint32_t c[16]) {
  const uint32_t hi = r16_place8(c + 8);
  return r16_place8(c) | (hi << 8) | (hi >> 24);
}

}  // namespace lcvq
