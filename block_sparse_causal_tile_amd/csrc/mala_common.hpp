// Shared device helpers for the MALA HIP kernels (gfx950 / CDNA4).
//
// Everything here is plumbing: vector types, 16-byte loads and stores, bf16
// packing, and the lane layout of the 32x32x16 bf16 MFMA. The attention
// arithmetic lives in the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mala_internal.hpp"

namespace mala {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}
__device__ __forceinline__ u32x4_t zero16() { return u32x4_t{0u, 0u, 0u, 0u}; }

// Two floats -> two bf16 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// D = A * B + C on a 32x32x16 bf16 matrix core op. Lane l supplies
//   A[l % 32][8 * (l / 32) + 0..7]  and  B[8 * (l / 32) + 0..7][l % 32],
// and holds C/D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32] in register r.
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Row (within a 32-row MFMA block) of accumulator register r in lane half hh.
__device__ __forceinline__ constexpr int acc_row(int r, int hh) {
  return 8 * (r >> 2) + 4 * hh + (r & 3);
}

__device__ __forceinline__ float wave_max_halves(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum_halves(float x) { return x + __shfl_xor(x, 32); }

}  // namespace mala
