// Order-preserving 64-bit keys for arg-max style reductions whose result
// must not depend on the reduction order (shared by the consensus, top-M and
// tree kernels).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orthrus {
namespace keys {

// Unsigned key with the order of the float: -inf < ... < -0 == +0 < ... < +inf
// < NaN (every NaN ranks above every number).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) return 0xFFFFFFFFu;  // NaN ranks above every number
  if (x == 0.0f) u = 0u;           // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long pack_key(float x, uint32_t idx) {
  return ((unsigned long long)order_key(x) << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

__device__ __forceinline__ unsigned long long wave_max64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = umax64(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ unsigned long long wave_sum64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// The float of an order_key (NaN keys give a NaN).
__device__ __forceinline__ float key_value(uint32_t k) {
  if (k == 0xFFFFFFFFu) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

}  // namespace keys
}  // namespace orthrus
