// Router kernels: top-k selection with softmax gates, its backward, and the fp32
// router GEMM of the tiny workload.  One 64-lane wavefront per token.
//
// The router distributes tokens to a selection of experts (sebask.de,
// "Mixture-of-Kittens: Cursors Open-Source-Ansatz für effizientes MoE-Training auf
// NVL72", introduction).  Selection order: logit descending, expert id ascending;
// gates: softmax over the k selected logits.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int ROUTE_MAX_PER_LANE = MOE_MAX_E / 64;

// Order-preserving map of fp32 to uint32 (larger float -> larger integer); -0.0
// is first turned into +0.0 so that the two tie.
MOE_DEV uint32_t ordered_bits(float v) {
  uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

MOE_DEV float from_ordered_bits(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

// key = ordered logit in the high word, (0xffffffff - expert) in the low word, so
// the largest key is the largest logit and, among equal logits, the lowest id.
// 0 marks "taken / absent" (no finite logit maps to it).
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* L = logits + (size_t)t * E;
  unsigned long long key[ROUTE_MAX_PER_LANE];
#pragma unroll
  for (int i = 0; i < ROUTE_MAX_PER_LANE; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? (((unsigned long long)ordered_bits(L[e]) << 32) |
                        (unsigned long long)(0xffffffffu - (uint32_t)e))
                     : 0ull;
  }
  float my_logit = 0.0f, top_logit = 0.0f;
  for (int j = 0; j < k; ++j) {
    unsigned long long m = 0ull;
#pragma unroll
    for (int i = 0; i < ROUTE_MAX_PER_LANE; ++i) m = key[i] > m ? key[i] : m;
    m = wave_max_u64(m);
    const int e = (int)(0xffffffffu - (uint32_t)(m & 0xffffffffu));
    const float lg = from_ordered_bits((uint32_t)(m >> 32));
    if (j == 0) top_logit = lg;
    if (lane == j) my_logit = lg;
#pragma unroll
    for (int i = 0; i < ROUTE_MAX_PER_LANE; ++i)
      if (lane + 64 * i == e) key[i] = 0ull;
    if (lane == 0) topk_idx[(size_t)t * k + j] = e;
  }
  const float z = (lane < k) ? expf(my_logit - top_logit) : 0.0f;
  const float s = wave_sum_f32(z);
  if (lane < k) topk_w[(size_t)t * k + lane] = z / s;
}

// d_logits[t, e_j] = w_j (dw_j - sum_i w_i dw_i); 0 for unselected experts.
__global__ __launch_bounds__(256) void route_backward_kernel(const int32_t* __restrict__ topk_idx,
                                                             const float* __restrict__ topk_w,
                                                             const float* __restrict__ d_topk_w,
                                                             int T, int E, int k,
                                                             float* __restrict__ d_logits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_e = -1;
  float wj = 0.0f, dj = 0.0f;
  if (lane < k) {
    my_e = topk_idx[(size_t)t * k + lane];
    wj = topk_w[(size_t)t * k + lane];
    dj = d_topk_w[(size_t)t * k + lane];
  }
  const float s = wave_sum_f32(wj * dj);
  const float val = wj * (dj - s);
  float* out = d_logits + (size_t)t * E;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    float v = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int ej = __shfl(my_e, j, 64);
      const float vj = __shfl(val, j, 64);
      if (ej == e) v = vj;
    }
    if (e < E) out[e] = v;
  }
}

// logits[t, e] = sum_h x[t, h] w_r[e, h]: lane partial sums in ascending h, then a
// fixed butterfly; one wave per token.  Meant for small E and H.
__global__ __launch_bounds__(256) void router_logits_f32_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ wr,
                                                                int T, int H, int E,
                                                                float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* xr = x + (size_t)t * H;
  for (int e = 0; e < E; ++e) {
    const float* w = wr + (size_t)e * H;
    float acc = 0.0f;
    for (int h = lane; h < H; h += 64) acc = fmaf(xr[h], w[h], acc);
    acc = wave_sum_f32(acc);
    if (lane == 0) logits[(size_t)t * E + e] = acc;
  }
}

// dw_r[e, h] = sum_t dL[t, e] x[t, h], ascending t; one thread per (e, h).
__global__ __launch_bounds__(256) void router_dw_f32_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ dL, int T,
                                                            int H, int E, float* __restrict__ dwr) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)E * H) return;
  const int e = (int)(idx / H), h = (int)(idx % H);
  float acc = 0.0f;
  for (int t = 0; t < T; ++t) acc = fmaf(dL[(size_t)t * E + e], x[(size_t)t * H + h], acc);
  dwr[idx] = acc;
}

// dx[t, h] += sum_e dL[t, e] w_r[e, h], ascending e; one thread per (t, h).
__global__ __launch_bounds__(256) void router_dx_f32_kernel(const float* __restrict__ wr,
                                                            const float* __restrict__ dL, int T,
                                                            int H, int E, float* __restrict__ dx) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)T * H) return;
  const int t = (int)(idx / H), h = (int)(idx % H);
  float acc = 0.0f;
  for (int e = 0; e < E; ++e) acc = fmaf(dL[(size_t)t * E + e], wr[(size_t)e * H + h], acc);
  dx[idx] += acc;
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  return MOE_LAUNCH("route", s, route_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, idx, w));
}

hipError_t launch_route_backward(const int32_t* idx, const float* w, const float* dw, int T, int E,
                                 int k, float* dL, hipStream_t s) {
  if (T == 0) return hipSuccess;
  return MOE_LAUNCH("route_backward", s,
                    route_backward_kernel<<<(T + 3) / 4, 256, 0, s>>>(idx, w, dw, T, E, k, dL));
}

hipError_t launch_router_logits_f32(const float* x, const float* wr, int T, int H, int E,
                                    float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  return MOE_LAUNCH("router_logits_f32", s,
                    router_logits_f32_kernel<<<(T + 3) / 4, 256, 0, s>>>(x, wr, T, H, E, logits));
}

hipError_t launch_router_backward_f32(const float* x, const float* wr, const float* dL, int T,
                                      int H, int E, float* dwr, float* dx, hipStream_t s) {
  const long n1 = (long)E * H;
  hipError_t err = MOE_LAUNCH(
      "router_dw_f32", s,
      router_dw_f32_kernel<<<(unsigned)((n1 + 255) / 256), 256, 0, s>>>(x, dL, T, H, E, dwr));
  if (err != hipSuccess || T == 0) return err;
  const long n2 = (long)T * H;
  return MOE_LAUNCH(
      "router_dx_f32", s,
      router_dx_f32_kernel<<<(unsigned)((n2 + 255) / 256), 256, 0, s>>>(wr, dL, T, H, E, dx));
}

}  // namespace moe
