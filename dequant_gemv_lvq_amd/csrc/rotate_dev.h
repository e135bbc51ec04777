// Device helpers of the activation rotation (H kron Q)(S x), shared by the
// standalone rotation kernel and the GEMV that rotates x in LDS.
#pragma once

#include "common.h"

namespace lvq {

__device__ __forceinline__ float rot_half(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// the sign bits of 8 consecutive coordinates (bits 0..7) onto fp16 sign bits
__device__ __forceinline__ uint4 rot_apply_signs(uint4 v, uint32_t s8) {
  auto two = [](uint32_t w, uint32_t b2) {
    return w ^ (((b2 & 1u) << 15) | ((b2 & 2u) << 30));
  };
  return make_uint4(two(v.x, s8), two(v.y, s8 >> 2), two(v.z, s8 >> 4), two(v.w, s8 >> 6));
}

__device__ __forceinline__ uint16_t rot_sign_bit(const uint32_t* signs, int j) {
  return signs ? (uint16_t)(((signs[j >> 5] >> (j & 31)) & 1u) << 15) : (uint16_t)0;
}

__device__ __forceinline__ uint16_t rot_out(float v, float scale) {
  return __builtin_bit_cast(uint16_t, (_Float16)(v * scale));
}

// Stages 0-2 of 8 values in registers, in the order h = 1, 2, 4.
__device__ __forceinline__ void rot_reg_stages(float (&v)[8], int cw) {
#pragma unroll
  for (int e = 0; e < 3; ++e) {
    const int h = 1 << e;
    if (h >= cw) break;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t & h) continue;
      const float lo = v[t], hi = v[t + h];
      v[t] = lo + hi;
      v[t + h] = lo - hi;
    }
  }
}

// Radix-2^R butterflies of one set: v[t] at coordinates base + t 2^s.
template <int R>
__device__ __forceinline__ void rot_set_stages(float (&v)[1 << R]) {
  constexpr int kR = 1 << R;
#pragma unroll
  for (int e = 0; e < R; ++e) {
    const int h = 1 << e;
#pragma unroll
    for (int t = 0; t < kR; ++t) {
      if (t & h) continue;
      const float lo = v[t], hi = v[t + h];
      v[t] = lo + hi;
      v[t + h] = lo - hi;
    }
  }
}

}  // namespace lvq
