// The fixed-order combine of one token's 16-byte chunk, shared by the combine and
// reverse-dispatch kernels (move.hip) and the combine phase of the persistent forward
// (gemm_big.hip), so that both give the same bits: out = round( sum_j w_j Y[pos_j] +
// shared ), fp32 from zero, j ascending, the shared row last (sebask.de,
// "Mixture-of-Kittens: Cursors Open-Source-Ansatz für effizientes MoE-Training auf
// NVL72", § Push oder Pull; stamatios.com, "Cursor abre código de megakernel MoE para
// GPUs NVL72", § Outras características).
#pragma once

#include "common.hpp"

namespace moe {

// 16 bytes at p; COHERENT: read at device scope (two 8-byte loads that miss any line
// of this XCD's L2 older than a store another XCD wrote through in the same launch),
// else a non-temporal load (each Y row is read once)
template <bool COHERENT>
MOE_DEV uint4 load_chunk(const uint4* p) {
  if (COHERENT) {
    const uint64_t lo = __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load((const uint64_t*)p + 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    return make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
  }
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)p));
}

// Chunk c (8 values) of token t: Y rows pos_t[j] (< 0: no row), weights w_t[j]
// (WEIGHTED = false: weight 1), shared_t the token's shared row (NULL: none), out_t
// the token's output row; pos_t and w_t are read through the constant address space
// (wave-uniform, not written by the launch).  COHERENT: Y and the shared row were
// written earlier in the same launch (load_chunk).
template <bool WEIGHTED, bool COHERENT = false>
MOE_DEV void combine_chunk(const uint4* __restrict__ Y, const int32_t* pos_t, const float* w_t,
                           const uint4* shared_t, uint4* out_t, int k, int row_chunks, int c) {
  typedef const __attribute__((address_space(4))) int32_t* cpos_t;
  typedef const __attribute__((address_space(4))) float* cw_t;
  const cpos_t s_pos = (cpos_t)pos_t;
  const cw_t s_w = WEIGHTED ? (cw_t)w_t : nullptr;
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += 8) {
    const bool last = j0 + 8 >= k;
    int rr[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) rr[jj] = s_pos[min(j0 + jj, k - 1)];  // issued together
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      if (j0 + jj >= k) rr[jj] = -1;
    uint4 raw[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      raw[jj] = rr[jj] >= 0 ? load_chunk<COHERENT>(Y + (size_t)rr[jj] * row_chunks + c) : z;
    const uint4 sh = shared_t && last
                         ? (COHERENT ? load_chunk<true>(shared_t + c) : shared_t[c])
                         : z;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = j0 + jj;
      if (rr[jj] < 0) continue;
      float v[8];
      unpack8(raw[jj], v);
      if (WEIGHTED) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(s_w[j], v[i], acc[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
      }
    }
    if (shared_t && last) {
      float v[8];
      unpack8(sh, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
  }
  if (shared_t && k == 0) {
    float v[8];
    unpack8(COHERENT ? load_chunk<true>(shared_t + c) : shared_t[c], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, pack8(acc)), (u32x4_t*)(out_t + c));
}

}  // namespace moe
