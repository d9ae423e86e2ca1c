// Sort-free schedule table ("plan") built on the GPU from the routing indices.
//
// The pull schedule is a list of sources whose order follows from the routing,
// built entirely on the GPU (sebask.de, "Mixture-of-Kittens: Cursors
// Open-Source-Ansatz für effizientes MoE-Training auf NVL72", § Das Scheduling);
// it is built once, reused by the four movement operations and needs no sorting
// (stamatios.com, "Cursor abre código de megakernel MoE para GPUs NVL72",
// § Escolha da direção de comunicação).
//
// A counting sort in three launches:
//   1. plan_hist: each wavefront owns a chunk of PLAN_CHUNK consecutive pairs and
//      counts them per expert.  64 pairs at a time, lanes holding the same expert
//      are found with one ballot per expert-id bit; the lowest such lane adds the
//      group's popcount to the chunk's LDS counter (no atomics).
//   2. plan_scan: one workgroup reduces the chunk histograms to counts, takes the
//      exclusive prefix over experts (offsets) and over chunks (each chunk's first
//      row per expert), writes the GEMM tile list, the list of experts that
//      received rows, and the error flag.
//   3. plan_scatter: each wavefront replays its chunk in pair order; a pair's row
//      is its chunk base + the number of earlier same-expert pairs, so rows of an
//      expert keep ascending pair order (stable) and the result does not depend on
//      the launch shape.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int PLAN_WAVES = 4;  // wavefronts (chunks) per workgroup

struct MbPlanPtrs {
  const int32_t* counts[MX_MAX_MB];
  const int32_t* offsets[MX_MAX_MB];
  const int32_t* tiles[MX_MAX_MB];
  const int32_t* n_tiles[MX_MAX_MB];
  const int32_t* src_token[MX_MAX_MB];
  int n_mb;
};
constexpr int PLAN_STEPS = PLAN_CHUNK / 64;

// Lanes whose expert id equals mine (only meaningful for lanes with ok == true).
MOE_DEV unsigned long long match_expert(int e, bool ok, int nbits) {
  unsigned long long mask = ballot64(ok);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const unsigned long long bb = ballot64(ok && bit);
    mask &= bit ? bb : ~bb;
  }
  return mask;
}

MOE_DEV void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(256) void plan_hist_kernel(const int32_t* __restrict__ idx, int R,
                                                        int E, int nbits, int n_chunks,
                                                        int32_t* __restrict__ hist,
                                                        int32_t* __restrict__ chunk_invalid) {
  extern __shared__ int32_t cnt_all[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * PLAN_WAVES + w;
  if (c >= n_chunks) return;
  int32_t* cnt = cnt_all + w * E;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  wave_sync_lds();
  int invalid = 0;
  for (int st = 0; st < PLAN_STEPS; ++st) {
    const int p = c * PLAN_CHUNK + st * 64 + lane;
    const bool in = p < R;
    const int e = in ? idx[p] : -1;
    const bool ok = in && e >= 0 && e < E;
    invalid += (in && !ok) ? 1 : 0;
    const unsigned long long m = match_expert(e, ok, nbits);
    const bool leader = ok && (lane == __ffsll((long long)m) - 1);
    if (leader) cnt[e] += __popcll(m);
    wave_sync_lds();
  }
  for (int e = lane; e < E; e += 64) hist[(size_t)c * E + e] = cnt[e];
  const int inv = (int)wave_sum_f32((float)invalid);  // <= 512, exact in fp32
  if (lane == 0) chunk_invalid[c] = inv;
}

// One workgroup of 1024 threads; E <= 1024 so each thread owns at most one expert.
__global__ __launch_bounds__(1024) void plan_scan_kernel(
    int32_t* __restrict__ hist, const int32_t* __restrict__ chunk_invalid, int n_chunks, int E,
    int R, int tile_m, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles, int32_t* __restrict__ err_flag,
    int32_t* __restrict__ src_token, int32_t* __restrict__ src_slot,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active,
    int32_t* __restrict__ tile_first, int wtile_m, int32_t* __restrict__ wtiles,
    int32_t* __restrict__ n_wtiles) {
  __shared__ int32_t s_rows[1];
  __shared__ int32_t s_wave[4][16];
  __shared__ int32_t s_bad;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) s_bad = 0;
  int n = 0;
  if (tid < E)
    for (int c = 0; c < n_chunks; ++c) n += hist[(size_t)c * E + tid];
  const int nt = (n + tile_m - 1) / tile_m;
  const int nw = (n + wtile_m - 1) / wtile_m;
  const int act = n > 0 ? 1 : 0;
  // inclusive scans inside each wavefront (Hillis-Steele over shuffles)
  int a = n, b = nt, c3 = act, d = nw;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ua = __shfl_up(a, o, 64), ub = __shfl_up(b, o, 64), uc = __shfl_up(c3, o, 64);
    const int ud = __shfl_up(d, o, 64);
    if (lane >= o) { a += ua; b += ub; c3 += uc; d += ud; }
  }
  if (lane == 63) { s_wave[0][wv] = a; s_wave[1][wv] = b; s_wave[2][wv] = c3; s_wave[3][wv] = d; }
  __syncthreads();
  int base_a = 0, base_b = 0, base_c = 0, base_d = 0;
  for (int i = 0; i < wv; ++i) {
    base_a += s_wave[0][i]; base_b += s_wave[1][i]; base_c += s_wave[2][i]; base_d += s_wave[3][i];
  }
  const int excl_rows = base_a + a - n, excl_tiles = base_b + b - nt, excl_act = base_c + c3 - act;
  const int excl_w = base_d + d - nw;
  if (tid < E) {
    counts[tid] = n;
    tile_first[tid] = excl_tiles;
    if (act) active[excl_act] = tid;
    offsets[tid] = excl_rows;
    // first row of each chunk for this expert
    int run = excl_rows;
    for (int c = 0; c < n_chunks; ++c) {
      const int h = hist[(size_t)c * E + tid];
      hist[(size_t)c * E + tid] = run;
      run += h;
    }
    for (int m = 0; m < nt; ++m) {
      tiles[2 * (excl_tiles + m)] = tid;
      tiles[2 * (excl_tiles + m) + 1] = excl_rows + m * tile_m;
    }
    for (int m = 0; m < nw; ++m) {
      wtiles[2 * (excl_w + m)] = tid;
      wtiles[2 * (excl_w + m) + 1] = excl_rows + m * wtile_m;
    }
  }
  if (tid == E - 1) {
    offsets[E] = excl_rows + n;
    n_tiles[0] = excl_tiles + nt;
    n_wtiles[0] = excl_w + nw;
    n_active[0] = excl_act + act;
    tile_first[E] = excl_tiles + nt;
    s_rows[0] = excl_rows + n;
  }
  for (int c = tid; c < n_chunks; c += 1024)
    if (chunk_invalid[c]) s_bad = 1;  // benign same-value race on LDS
  __syncthreads();
  if (tid == 0) err_flag[0] = s_bad;
  for (int r = s_rows[0] + tid; r < R; r += 1024) {
    src_token[r] = -1;
    src_slot[r] = -1;
  }
}

__global__ __launch_bounds__(256) void plan_scatter_kernel(const int32_t* __restrict__ idx, int R,
                                                           int E, int k, int nbits, int n_chunks,
                                                           const int32_t* __restrict__ chunk_base,
                                                           int32_t* __restrict__ src_token,
                                                           int32_t* __restrict__ src_slot,
                                                           int32_t* __restrict__ pos) {
  extern __shared__ int32_t cur_all[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * PLAN_WAVES + w;
  if (c >= n_chunks) return;
  int32_t* cur = cur_all + w * E;
  for (int e = lane; e < E; e += 64) cur[e] = chunk_base[(size_t)c * E + e];
  wave_sync_lds();
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int st = 0; st < PLAN_STEPS; ++st) {
    const int p = c * PLAN_CHUNK + st * 64 + lane;
    const bool in = p < R;
    const int e = in ? idx[p] : -1;
    const bool ok = in && e >= 0 && e < E;
    const unsigned long long m = match_expert(e, ok, nbits);
    const int base = ok ? cur[e] : 0;
    if (ok) {
      const int row = base + __popcll(m & below);
      src_token[row] = p / k;
      src_slot[row] = p - (p / k) * k;
      pos[p] = row;
    } else if (in) {
      pos[p] = -1;
    }
    wave_sync_lds();
    if (ok && lane == __ffsll((long long)m) - 1) cur[e] = base + __popcll(m);
    wave_sync_lds();
  }
}

hipError_t launch_plan(const int32_t* topk_idx, int T, int k, int E, const PlanPtrs& p,
                       hipStream_t s) {
  const int R = T * k;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int blocks = (p.n_chunks + PLAN_WAVES - 1) / PLAN_WAVES;
  const size_t lds = (size_t)PLAN_WAVES * E * sizeof(int32_t);
  if (p.n_chunks > 0) {
    hipError_t err = MOE_LAUNCH("plan_hist", s,
                                plan_hist_kernel<<<blocks, 256, lds, s>>>(
                                    topk_idx, R, E, nbits, p.n_chunks, p.chunk_hist,
                                    p.chunk_invalid));
    if (err != hipSuccess) return err;
  }
  hipError_t err = MOE_LAUNCH("plan_scan", s,
                              plan_scan_kernel<<<1, 1024, 0, s>>>(
                                  p.chunk_hist, p.chunk_invalid, p.n_chunks, E, R, GEMM_TILE_M,
                                  p.counts, p.offsets, p.tiles, p.n_tiles, p.err_flag,
                                  p.src_token, p.src_slot, p.active, p.n_active,
                                  p.tile_first, GEMM_WTILE_M, p.wtiles, p.n_wtiles));
  if (err != hipSuccess || p.n_chunks == 0) return err;
  return MOE_LAUNCH("plan_scatter", s,
                    plan_scatter_kernel<<<blocks, 256, lds, s>>>(topk_idx, R, E, k, nbits,
                                                                 p.n_chunks, p.chunk_hist,
                                                                 p.src_token, p.src_slot, p.pos));
}

}  // namespace moe

namespace moe {

// The weight gradients' token axis over the minibatches of one macro batch (one
// workgroup of 1024 threads; thread e owns expert e).  Expert e's rows of all
// minibatches, in token order, are its global rows goff[e] .. goff[e + 1] - 1
// (minibatch m's segment starts at goff[e] + cum[m * E + e]); on the packed token
// axis they take the byte columns kpos[e] .. kpos[e] + n_e - 1, kpos advancing by
// n_e rounded up to 32 (the MX blocks run from each expert's first row); gtiles lists
// (expert, first global row) per 128 global rows of each expert.
MOE_DEV int block_excl_scan(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int c = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(c, o, 64);
    if (lane >= o) c += u;
  }
  __syncthreads();  // s_wave free from a previous scan
  if (lane == 63) s_wave[wv] = c;
  __syncthreads();
  int base = 0;
  total = 0;
  for (int i = 0; i < nw; ++i) {
    if (i < wv) base += s_wave[i];
    total += s_wave[i];
  }
  return base + c - v;
}

__global__ __launch_bounds__(1024) void mb_union_kernel(MbPlanPtrs mc, int E,
                                                        int32_t* __restrict__ counts_all,
                                                        int32_t* __restrict__ active,
                                                        int32_t* __restrict__ n_active,
                                                        int32_t* __restrict__ cum,
                                                        int32_t* __restrict__ kpos,
                                                        int32_t* __restrict__ goff,
                                                        int32_t* __restrict__ gtiles,
                                                        int32_t* __restrict__ n_gtiles) {
  __shared__ int s_wave[16];
  const int tid = threadIdx.x;
  int n = 0;
  if (tid < E)
    for (int m = 0; m < mc.n_mb; ++m) {
      cum[m * E + tid] = n;
      n += mc.counts[m][tid];
    }
  const int act = n > 0 ? 1 : 0, ntile = (n + 127) / 128;
  int tot_act, tot_k, tot_n, tot_t;
  const int e_act = block_excl_scan(act, s_wave, tot_act);
  const int e_k = block_excl_scan((n + 31) & ~31, s_wave, tot_k);
  const int e_n = block_excl_scan(n, s_wave, tot_n);
  const int e_t = block_excl_scan(ntile, s_wave, tot_t);
  if (tid < E) {
    counts_all[tid] = n;
    if (act) active[e_act] = tid;
    kpos[tid] = e_k;
    goff[tid] = e_n;
    for (int i = 0; i < ntile; ++i) {
      gtiles[2 * (e_t + i)] = tid;
      gtiles[2 * (e_t + i) + 1] = e_n + 128 * i;
    }
  }
  if (tid == 0) {
    n_active[0] = tot_act;
    kpos[E] = tot_k;
    goff[E] = tot_n;
    n_gtiles[0] = tot_t;
  }
}

// Global row p of a macro batch (see mb_union_kernel) of minibatch m's plan row r:
// grow[p] = m * R_mb + r (rows of per-minibatch arrays stored one minibatch after
// the other) and gtok[p] = m * T_mb + src_token_m[r] (its token).  One workgroup of
// 128 threads per (plan tile, minibatch).
__global__ __launch_bounds__(128) void mb_rows_kernel(MbPlanPtrs mc, int E, int R_mb, int T_mb,
                                                      const int32_t* __restrict__ cum,
                                                      const int32_t* __restrict__ goff,
                                                      int32_t* __restrict__ grow,
                                                      int32_t* __restrict__ gtok) {
  const int m = blockIdx.y, t = blockIdx.x;
  if (m >= mc.n_mb || t >= mc.n_tiles[m][0]) return;
  const int e = mc.tiles[m][2 * t], row = mc.tiles[m][2 * t + 1] + (int)threadIdx.x;
  const int32_t* off = mc.offsets[m];
  if (row >= off[e + 1]) return;
  const int p = goff[e] + cum[m * E + e] + (row - off[e]);
  grow[p] = m * R_mb + row;
  gtok[p] = m * T_mb + mc.src_token[m][row];
}

static MbPlanPtrs mb_ptrs(const MbPlanViews& v) {
  MbPlanPtrs mc = {};
  mc.n_mb = v.n_mb;
  for (int m = 0; m < v.n_mb && m < MX_MAX_MB; ++m) {
    mc.counts[m] = v.counts[m];
    mc.offsets[m] = v.offsets[m];
    mc.tiles[m] = v.tiles[m];
    mc.n_tiles[m] = v.n_tiles[m];
    mc.src_token[m] = v.src_token[m];
  }
  return mc;
}

hipError_t launch_mb_union(const MbPlanViews& v, int E, const MbAxis& ax, hipStream_t s) {
  return MOE_LAUNCH("mb_union", s,
                    mb_union_kernel<<<1, 1024, 0, s>>>(mb_ptrs(v), E, ax.counts_all, ax.active,
                                                       ax.n_active, ax.cum, ax.kpos, ax.goff,
                                                       ax.gtiles, ax.n_gtiles));
}

hipError_t launch_mb_rows(const MbPlanViews& v, int E, int max_tiles, int R_mb, int T_mb,
                          const MbAxis& ax, hipStream_t s) {
  if (max_tiles == 0 || v.n_mb == 0) return hipSuccess;
  return MOE_LAUNCH("mb_rows", s,
                    mb_rows_kernel<<<dim3(max_tiles, v.n_mb), 128, 0, s>>>(
                        mb_ptrs(v), E, R_mb, T_mb, ax.cum, ax.goff, ax.grow, ax.gtok));
}

}  // namespace moe
