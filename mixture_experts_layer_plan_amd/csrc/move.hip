// Row movement of the four operations on one GPU, plus the fixed-order reduction
// of the router-weight-gradient partials.
//
// Dispatch and reverse-combine pull rows by the plan's source list; combine and
// reverse-dispatch sum a token's k rows in ascending slot order so that the token
// order is kept and the floating-point order never changes (sebask.de,
// "Mixture-of-Kittens: Cursors Open-Source-Ansatz für effizientes MoE-Training
// auf NVL72", § Push oder Pull; stamatios.com, "Cursor abre código de megakernel
// MoE para GPUs NVL72", § Escolha da direção de comunicação and § Outras
// características).  All are HBM-bound streams: 16-byte vector accesses, one
// workgroup per destination row.
#include "common.hpp"
#include "internal.hpp"
#include "move_common.hpp"

namespace moe {

// 16-byte non-temporal store: the gathered rows (R rows, larger than the Infinity
// Cache at the bench shape) are read back by a later launch, not from cache
// (measured on MI355X: 0.141 -> 0.137 ms per gather at T = 4096, k = 8, H = 7168).
__device__ inline void nts(uint4* p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), (u32x4_t*)p);
}

// dst[r, :] = src[src_token[r], :] for r < n_valid; row_bytes is a multiple of 16.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ src,
                                                          uint4* __restrict__ dst,
                                                          const int32_t* __restrict__ src_token,
                                                          const int32_t* __restrict__ n_valid,
                                                          int row_chunks) {
  const int r = blockIdx.x;
  if (r >= n_valid[0]) return;
  const uint4* s = src + (size_t)src_token[r] * row_chunks;
  uint4* d = dst + (size_t)r * row_chunks;
  int c = threadIdx.x;
  for (; c + 3 * 256 < row_chunks; c += 4 * 256) {
    const uint4 v0 = s[c], v1 = s[c + 256], v2 = s[c + 512], v3 = s[c + 768];
    nts(d + c, v0); nts(d + c + 256, v1); nts(d + c + 512, v2); nts(d + c + 768, v3);
  }
  for (; c < row_chunks; c += 256) nts(d + c, s[c]);
}

// The same copy walked by source token: dst[pos[t, j], :] = src[t, :] for every pair
// with pos[t, j] >= 0 (the rows r < n_valid, each written once), so that each source
// row is read once and written to its k rows.  One workgroup per token; the token's
// slots are wave-uniform reads through the constant address space.
__global__ __launch_bounds__(256) void scatter_rows_kernel(const uint4* __restrict__ src,
                                                           uint4* __restrict__ dst,
                                                           const int32_t* __restrict__ pos, int k,
                                                           int row_chunks) {
  const int t = blockIdx.x;
  typedef const __attribute__((address_space(4))) int32_t* cpos_t;
  const cpos_t s_pos = (cpos_t)(pos + (size_t)t * k);
  const uint4* s = src + (size_t)t * row_chunks;
  for (int c0 = 0; c0 < row_chunks; c0 += 4 * 256) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * 256 + (int)threadIdx.x;
      if (c < row_chunks) v[u] = s[c];
    }
    for (int j = 0; j < k; ++j) {
      const int r = s_pos[j];
      if (r < 0) continue;
      uint4* d = dst + (size_t)r * row_chunks;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * 256 + (int)threadIdx.x;
        if (c < row_chunks) nts(d + c, v[u]);
      }
    }
  }
}

// y[t, :] = round( sum_j w[t, j] * Y[pos[t, j], :] + shared[t, :] ), fp32 from zero,
// j ascending, shared last.  WEIGHTED = false sums with weight 1 (reverse-dispatch).
// One 128-thread workgroup per (token, slice of 128 16-byte chunks); each thread
// issues the loads of up to 8 slots and of the shared row together, then adds them
// in slot order.
constexpr int CMB_THREADS = 128;
template <bool WEIGHTED>
__global__ __launch_bounds__(CMB_THREADS) void combine_bf16_kernel(
    const uint4* __restrict__ Y, const int32_t* __restrict__ pos, const float* __restrict__ w,
    const uint4* __restrict__ shared, uint4* __restrict__ y, int k, int row_chunks, int slices) {
  const int t = blockIdx.x / slices;
  const int c = (blockIdx.x - t * slices) * CMB_THREADS + threadIdx.x;
  if (c >= row_chunks) return;
  combine_chunk<WEIGHTED>(Y, pos + (size_t)t * k, WEIGHTED ? w + (size_t)t * k : nullptr,
                          shared ? shared + (size_t)t * row_chunks : nullptr,
                          y + (size_t)t * row_chunks, k, row_chunks, c);
}

template <bool WEIGHTED>
__global__ __launch_bounds__(256) void combine_f32_kernel(const float4* __restrict__ Y,
                                                          const int32_t* __restrict__ pos,
                                                          const float* __restrict__ w,
                                                          const float4* __restrict__ shared,
                                                          float4* __restrict__ y, int k,
                                                          int row_chunks) {
  const int t = blockIdx.x;
  __shared__ int s_pos[MOE_MAX_K];
  __shared__ float s_w[MOE_MAX_K];
  if (threadIdx.x < k) {
    s_pos[threadIdx.x] = pos[(size_t)t * k + threadIdx.x];
    s_w[threadIdx.x] = WEIGHTED ? w[(size_t)t * k + threadIdx.x] : 1.0f;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < row_chunks; c += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int r = s_pos[j];
      if (r < 0) continue;
      const float4 v = Y[(size_t)r * row_chunks + c];
      if (WEIGHTED) {
        acc.x = fmaf(s_w[j], v.x, acc.x); acc.y = fmaf(s_w[j], v.y, acc.y);
        acc.z = fmaf(s_w[j], v.z, acc.z); acc.w = fmaf(s_w[j], v.w, acc.w);
      } else {
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
    }
    if (shared) {
      const float4 v = shared[(size_t)t * row_chunks + c];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    y[(size_t)t * row_chunks + c] = acc;
  }
}

// d_topk_w[p] = sum_{n ascending} dgp[pos[p], n]; 0 for pairs left out of the plan.
__global__ __launch_bounds__(256) void dg_reduce_kernel(const float* __restrict__ dgp,
                                                        const int32_t* __restrict__ pos, int R,
                                                        int n_parts, float* __restrict__ out) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= R) return;
  const int r = pos[p];
  float s = 0.0f;
  if (r >= 0)
    for (int n = 0; n < n_parts; ++n) s += dgp[(size_t)r * n_parts + n];
  out[p] = s;
}

hipError_t launch_gather_rows(const void* src, void* dst, const int32_t* src_token,
                              const int32_t* n_valid, int R, int row_bytes, hipStream_t s) {
  if (R == 0) return hipSuccess;
  return MOE_LAUNCH("gather_rows", s,
                    gather_rows_kernel<<<R, 256, 0, s>>>((const uint4*)src, (uint4*)dst,
                                                         src_token, n_valid, row_bytes / 16));
}

hipError_t launch_scatter_rows(const void* src, void* dst, const int32_t* pos, int T, int k,
                               int row_bytes, hipStream_t s) {
  if (T == 0) return hipSuccess;
  return MOE_LAUNCH("gather_rows", s,
                    scatter_rows_kernel<<<T, 256, 0, s>>>((const uint4*)src, (uint4*)dst, pos, k,
                                                          row_bytes / 16));
}

hipError_t launch_combine_bf16(const void* Y, const int32_t* pos, const float* w,
                               const void* shared, void* y, int T, int k, int H, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int chunks = H / 8, slices = (chunks + CMB_THREADS - 1) / CMB_THREADS;
  if ((long)T * slices > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const unsigned grid = (unsigned)((long)T * slices);
  if (w)
    return MOE_LAUNCH("combine_bf16", s,
                      combine_bf16_kernel<true><<<grid, CMB_THREADS, 0, s>>>(
                          (const uint4*)Y, pos, w, (const uint4*)shared, (uint4*)y, k, chunks,
                          slices));
  return MOE_LAUNCH("reverse_dispatch_bf16", s,
                    combine_bf16_kernel<false><<<grid, CMB_THREADS, 0, s>>>(
                        (const uint4*)Y, pos, nullptr, (const uint4*)shared, (uint4*)y, k, chunks,
                        slices));
}

hipError_t launch_combine_f32(const float* Y, const int32_t* pos, const float* w,
                              const float* shared, float* y, int T, int k, int H, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (w)
    return MOE_LAUNCH("combine_f32", s,
                      combine_f32_kernel<true><<<T, 256, 0, s>>>(
                          (const float4*)Y, pos, w, (const float4*)shared, (float4*)y, k, H / 4));
  return MOE_LAUNCH("reverse_dispatch_f32", s,
                    combine_f32_kernel<false><<<T, 256, 0, s>>>((const float4*)Y, pos, nullptr,
                                                               (const float4*)shared, (float4*)y,
                                                               k, H / 4));
}

hipError_t launch_dg_reduce(const float* dgp, const int32_t* pos, int R, int n_parts,
                            float* d_topk_w, hipStream_t s) {
  if (R == 0) return hipSuccess;
  return MOE_LAUNCH("dg_reduce", s,
                    dg_reduce_kernel<<<(R + 255) / 256, 256, 0, s>>>(dgp, pos, R, n_parts,
                                                                      d_topk_w));
}

}  // namespace moe
