// Shared pieces of the W4G128 kernels: vector types and the int4 -> fp16
// dequantization used by both the small-batch and the large-batch linear.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace paro {
namespace w4 {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Eight 4-bit codes (k0 in bits 0..3, ..., k7 in bits 28..31) -> eight fp16
// values (q - z) * s in k order.
__device__ __forceinline__ h8 dequant8(uint32_t w, h2 zz, h2 ss) {
  const uint32_t lo = w & 0x0F0F0F0Fu;         // q0 q2 q4 q6 (one per byte)
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // q1 q3 q5 q7
  uint32_t p[4];
  p[0] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x64006400u;
  p[1] = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x64006400u;
  p[2] = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x64006400u;
  p[3] = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x64006400u;
  h8 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h2 v = __builtin_bit_cast(h2, p[i]);
    v = (v - zz) * ss;
    out[2 * i] = v.x;
    out[2 * i + 1] = v.y;
  }
  return out;
}

__device__ __forceinline__ h2 splat2(_Float16 v) { return h2{v, v}; }
__device__ __forceinline__ float half_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
__device__ __forceinline__ uint32_t half_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

}  // namespace w4
}  // namespace paro
