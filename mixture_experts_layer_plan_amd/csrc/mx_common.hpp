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

// v / 2^X clamped to +-448 (scaling by a power of two is exact)
MOE_DEV float e4m3_scaled(float v, int X) {
  return fminf(fmaxf(ldexpf(v, -X), -448.0f), 448.0f);
}

// E4M3 codes of four values in one word (byte i: the code of the i-th) by the gfx950
// conversion v_cvt_pk_fp8_f32 (OCP E4M3, round to nearest even, sign kept).  On
// inputs clamped to +-448 its codes are the rule's: compared on MI355X with a
// software encoder of the rule (the fp32 bits rounded to three mantissa bits,
// multiples of 2^-9 below 2^-6) for every fp32 value of magnitude below 2^10, both
// signs, with no difference.
MOE_DEV uint32_t e4m3_pack4(float a, float b, float c, float d, int X) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_scaled(a, X), e4m3_scaled(b, X), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_scaled(c, X), e4m3_scaled(d, X), w, true);
  return (uint32_t)w;
}

// 32 values -> 32 codes (little-endian bytes in lo, hi)
MOE_DEV void mx_encode32(const float* v, int X, uint4& lo, uint4& hi) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = e4m3_pack4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], X);
  lo = make_uint4(w[0], w[1], w[2], w[3]);
  hi = make_uint4(w[4], w[5], w[6], w[7]);
}

// 8 values -> 8 codes
MOE_DEV uint2 mx_encode8(const float* v, int X) {
  return make_uint2(e4m3_pack4(v[0], v[1], v[2], v[3], X), e4m3_pack4(v[4], v[5], v[6], v[7], X));
}

}  // namespace moe
