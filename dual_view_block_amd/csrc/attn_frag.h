// Register and LDS fragment helpers of the bf16 MFMA attention kernels
// (shared by the streaming attention and the training backward).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orthrus {
namespace frag {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // plain vector: stays in registers
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS layouts of the K and V tiles (and of q): the 16-byte chunks of a row are
// permuted by an XOR with a row-dependent value so that the read patterns hit
// distinct banks.  K (and q) rows are read 16 lanes per row index apart, so
// 16 consecutive rows get 16 different chunk offsets.  V is read through the
// transposing LDS read, where 16 lanes take 4 consecutive rows x 2 adjacent
// chunks; XOR with 4 * (row mod 4) gives those 4 rows disjoint chunk quads.
template <int DCH>
__device__ __forceinline__ int swz_k(int row, int chunk) {
  if constexpr (DCH == 16) return chunk ^ (row & 15);
  else return chunk ^ ((row >> 1) & 7);
}
template <int DCH>
__device__ __forceinline__ int swz_v(int row, int chunk) {
  if constexpr (DCH == 16) return chunk ^ (4 * (row & 3));
  else return chunk ^ (2 * (row & 3));
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// lane `src`'s value of x, for the whole wave (the builtin moves 32-bit ints)
__device__ __forceinline__ float readlane_f(float x, int src) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(x), src));
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

}  // namespace frag
}  // namespace orthrus
