// E4M3 / E8M0 helpers shared by the MX conversion kernels and GEMM epilogues.
// Rule (OCP MX v1.0): X = floor(log2 amax) - 8 clamped to [-127, 127] (-127 for an
// all-zero block); element = RNE_E4M3(clamp(v / 2^X, +-448)), input sign kept.
#pragma once

#include "common.hpp"

namespace moe {

MOE_DEV float to_f32(bf16_t v) { return bf16_to_f32(v); }
MOE_DEV float to_f32(float v) { return v; }

MOE_DEV void load32(const bf16_t* p, float* v) {
  const uint4* q = (const uint4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack8(q[i], v + 8 * i);
}
MOE_DEV void load32(const float* p, float* v) {
  const float4* q = (const float4*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 a = q[i];
    v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
  }
}

// Scale exponent X of a block whose largest magnitude is amax.
MOE_DEV int mx_exp_of_amax(float amax) {
  if (!(amax > 0.0f)) return -127;
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127;  // floor(log2) for normals
  const int X = e - 8;                                               // subnormal amax: e = -127
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

MOE_DEV int mx_scale_exp(const float* v) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  return mx_exp_of_amax(amax);
}

// E4M3 code of v / 2^X: scaling by a power of two is exact, then round to
// nearest even on the integer bits of the fp32 value.
MOE_DEV uint32_t e4m3_code(float v, int X) {
  const float a0 = ldexpf(fabsf(v), -X);
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  const float a = fminf(a0, 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: multiples of 2^-9
    code = (uint32_t)rintf(a * 512.0f);      // exact scaling; rintf ties to even
  } else {
    const uint32_t u = __float_as_uint(a);
    int E = (int)(u >> 23) - 127;            // 2^-6 <= a <= 448: -6 <= E <= 8
    uint32_t m = (u >> 20) & 7u;
    const uint32_t rem = u & 0xfffffu, half = 0x80000u;
    if (rem > half || (rem == half && (m & 1u))) ++m;
    if (m == 8u) {
      m = 0u;
      ++E;
    }
    code = ((uint32_t)(E + 7) << 3) | m;
  }
  return code | sign;
}

// 32 values -> 32 codes (little-endian bytes in lo, hi)
MOE_DEV void mx_encode32(const float* v, int X, uint4& lo, uint4& hi) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = e4m3_code(v[4 * i], X) | (e4m3_code(v[4 * i + 1], X) << 8) |
           (e4m3_code(v[4 * i + 2], X) << 16) | (e4m3_code(v[4 * i + 3], X) << 24);
  lo = make_uint4(w[0], w[1], w[2], w[3]);
  hi = make_uint4(w[4], w[5], w[6], w[7]);
}

// 8 values -> 8 codes
MOE_DEV uint2 mx_encode8(const float* v, int X) {
  uint32_t w[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    w[i] = e4m3_code(v[4 * i], X) | (e4m3_code(v[4 * i + 1], X) << 8) |
           (e4m3_code(v[4 * i + 2], X) << 16) | (e4m3_code(v[4 * i + 3], X) << 24);
  return make_uint2(w[0], w[1]);
}

}  // namespace moe
