// Launch functions of the gfx950 kernels, called by the C-ABI layer (api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define MOE_MAX_E 1024
#define MOE_MAX_K 32

struct moe_trace;

namespace moe {

// Optional per-thread kernel timing (moe_trace_set in the C-ABI).
extern thread_local ::moe_trace* tls_trace;
void trace_before(hipStream_t s, const char* name);
void trace_after(hipStream_t s);

// Compute units that persistent launches size their grids for: the current
// device's CU count, capped by the calling thread's moe_set_cu_budget.
int device_cus();

// Enqueue one kernel launch between trace events; evaluates to hipGetLastError().
#define MOE_LAUNCH(name, stream, ...)   \
  (::moe::trace_before((stream), (name)), (__VA_ARGS__), ::moe::trace_after(stream), \
   hipGetLastError())

// plan construction
constexpr int PLAN_CHUNK = 512;      // pairs per wavefront chunk
constexpr int GEMM_TILE_M = 128;     // rows per grouped-GEMM tile (plan tile list)
constexpr int GEMM_WTILE_M = 256;    // rows per wide tile (second plan tile list)

// router
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                        hipStream_t s);
hipError_t launch_route_backward(const int32_t* idx, const float* w, const float* dw, int T,
                                 int E, int k, float* dL, hipStream_t s);
hipError_t launch_router_logits_f32(const float* x, const float* wr, int T, int H, int E,
                                    float* logits, hipStream_t s);
hipError_t launch_router_backward_f32(const float* x, const float* wr, const float* dL, int T,
                                      int H, int E, float* dwr, float* dx, hipStream_t s);

// plan
struct PlanPtrs {
  int32_t* counts;
  int32_t* offsets;
  int32_t* src_token;
  int32_t* src_slot;
  int32_t* pos;
  int32_t* tiles;
  int32_t* n_tiles;
  int32_t* err_flag;
  int32_t* active;         // [E] experts with rows, ascending
  int32_t* n_active;
  int32_t* tile_first;     // [E + 1] first tile of each expert in the tile list
  int32_t* wtiles;         // wide-tile list and its length
  int32_t* n_wtiles;
  int32_t* chunk_hist;     // [n_chunks, E]
  int32_t* chunk_invalid;  // [n_chunks]
  int n_chunks;
  int max_tiles;
};
hipError_t launch_plan(const int32_t* topk_idx, int T, int k, int E, const PlanPtrs& p,
                       hipStream_t s);

// row movement
hipError_t launch_gather_rows(const void* src, void* dst, const int32_t* src_token,
                              const int32_t* n_valid, int R, int row_bytes, hipStream_t s);
// the same rows written from the source side: dst[pos[t, j]] = src[t] (pos < 0 skipped)
hipError_t launch_scatter_rows(const void* src, void* dst, const int32_t* pos, int T, int k,
                               int row_bytes, hipStream_t s);
hipError_t launch_combine_bf16(const void* Y, const int32_t* pos, const float* w,
                               const void* shared, void* y, int T, int k, int H, hipStream_t s);
hipError_t launch_combine_f32(const float* Y, const int32_t* pos, const float* w,
                              const float* shared, float* y, int T, int k, int H, hipStream_t s);
hipError_t launch_dg_reduce(const float* dgp, const int32_t* pos, int R, int n_parts,
                            float* d_topk_w, hipStream_t s);

// grouped GEMMs (gemm.hip); `dt` 0 = fp32, 1 = bf16
struct GroupInfo {
  const int32_t* tiles;      // rows-grouped: plan tile list (NULL: dense over dense_rows)
  const int32_t* n_tiles;
  const int32_t* offsets;    // expert row offsets [E+1] (NULL: dense)
  const int32_t* src_token;  // token of each row (NULL: rows are tokens)
  const int32_t* src_slot;
  const int32_t* active;     // K-grouped: experts with rows (NULL: dense)
  const int32_t* n_active;
  const int32_t* counts;     // rows per expert (zero-fill of empty experts)
  const int32_t* wtiles;     // rows-grouped, wide kernels: 256-row tile list
  const int32_t* n_wtiles;
  int max_tiles;             // grid bound for rows-grouped launches
  int max_wtiles;
  int dense_rows;            // row count in dense mode
  int E;
  // K-grouped 128 x 128 wgrads: experts with >= hot_rows rows are left to the
  // large-tile kernel (INT_MAX: this kernel takes every expert)
  int hot_rows;
};

// bf16 large-tile kernels (gemm_big.hip) behind the launch_gemm_* entry points
hipError_t launch_big_up_swiglu(const GroupInfo& g, const void* x, const void* wg, const void* wu,
                                int H, int I, void* Z, void* h, hipStream_t s);
hipError_t launch_big_down(const GroupInfo& g, const void* h, const void* wd, int H, int I,
                           void* Y, hipStream_t s);
// The bf16 forward after the plan in one persistent launch: GEMM1 + SwiGLU and GEMM2
// of the routed and the shared experts and the combine, with device-counter hand-off
// between them (gemm_big.hip); outputs bitwise those of the separate launches.
struct FusedForwardArgs {
  GroupInfo g;                      // routed rows; needs the plan's wide-tile list
  GroupInfo gs;                     // the shared expert: dense over the T tokens
  int T, k, H, I, Is;               // Is = 0: no shared expert (sg, su, sd, Zs, hs, ys unused)
  const void *x, *wg, *wu, *wd;     // bf16 tokens and routed weights
  const void *sg, *su, *sd;         // bf16 shared expert weights
  void *Z, *h, *Y;                  // routed pre-activations (fp32), h and Y (bf16)
  void *Zs, *hs, *ys;               // the shared expert's
  const int32_t* pos;               // [T, k] plan inverse
  const float* w;                   // [T, k] combine weights
  void* y;                          // [T, H] bf16 output
  int32_t* ready;                   // fused_counters(g.max_wtiles, T) int32 of workspace
  int32_t* err;                     // the plan's err flag: bit 2 set if a wait gave up
};
inline int fused_counters(int max_wtiles, int T) { return max_wtiles + (T + 255) / 256 + 1 + 8; }
// hipErrorNotSupported (nothing enqueued) without the plan's wide-tile list
hipError_t launch_big_forward_fused(const FusedForwardArgs& a, hipStream_t s);
// MXFP8 GEMM2 and dgrad-up on the 256 x 256 core (gemm_big.hip); hipErrorNotSupported
// (nothing enqueued) unless H and I are multiples of 512 and the plan has its
// wide-tile list, and the launch_mx_* entry points then use the 128 x 128 kernels
hipError_t launch_big_mx_down(const GroupInfo& g, const uint8_t* hq, const uint8_t* hs,
                              const uint8_t* wd8, const uint8_t* wds, int H, int I, void* Y,
                              hipStream_t s);
hipError_t launch_big_mx_dgrad_up(const GroupInfo& g, const uint8_t* dZ8, const uint8_t* dZs,
                                  const uint8_t* wgT8, const uint8_t* wgTs, const uint8_t* wuT8,
                                  const uint8_t* wuTs, int H, int I, void* dX, hipStream_t s);
hipError_t launch_big_dgrad_up(const GroupInfo& g, const void* dZ, const void* wg, const void* wu,
                               int H, int I, void* dX, hipStream_t s);
// bf16 wgrads of the experts with >= hot_rows rows on the large tiles;
// hipErrorNotSupported (nothing enqueued) for shapes the large tiles do not cover
hipError_t launch_big_wgrad_up_hot(const GroupInfo& g, const void* dZ, const void* X, int H,
                                   int I, void* dwg, void* dwu, int hot_rows, hipStream_t s);
hipError_t launch_big_wgrad_down_hot(const GroupInfo& g, const void* dYu, const void* gh, int H,
                                     int I, void* dwd, int hot_rows, hipStream_t s);

// GEMM1 + SwiGLU: Z (fp32) [:, i] = A, Z[:, I + i] = B, h = silu(A) * B, with
// A = X W_g[e]^T, B = X W_u[e]^T and X rows gathered from x through src_token.
hipError_t launch_gemm_up_swiglu(int dt, const GroupInfo& g, const void* x, const void* wg,
                                 const void* wu, int H, int I, void* Z, void* h, hipStream_t s);
// GEMM2: Y = h W_d[e]^T
hipError_t launch_gemm_down(int dt, const GroupInfo& g, const void* h, const void* wd, int H,
                            int I, void* Y, hipStream_t s);
// dgrad-down + SwiGLU backward + router-weight-gradient partials; dYu = rows of dy
// in expert order (dy itself in dense mode)
hipError_t launch_gemm_dgrad_down(int dt, const GroupInfo& g, const void* dYu, const void* wd,
                                  const void* Z, const float* topk_w, int H, int I, int k,
                                  void* dZ, void* gh, float* dgp, hipStream_t s);
// dgrad-up: dX = dZ[:, :I] W_g[e] + dZ[:, I:] W_u[e]
hipError_t launch_gemm_dgrad_up(int dt, const GroupInfo& g, const void* dZ, const void* wg,
                                const void* wu, int H, int I, void* dX, hipStream_t s);
// wgrad-down: dW_d[e] = sum_r dYu[r] (x) gh[r]
hipError_t launch_gemm_wgrad_down(int dt, const GroupInfo& g, const void* dYu, const void* gh,
                                  int H, int I, void* dwd, hipStream_t s);
// wgrad-up: dW_g[e] = sum_r dZ[r, :I] (x) X[r], dW_u[e] likewise with dZ[r, I:]
hipError_t launch_gemm_wgrad_up(int dt, const GroupInfo& g, const void* dZ, const void* X,
                                int H, int I, void* dwg, void* dwu, hipStream_t s);

// ------------------------------------------------------------------ MXFP8
#define MX_MAX_MB 8  // minibatches per macro batch in the MX path
// MX wgrads: experts whose packed token range (their rows of all minibatches, padded
// to 32) has at least this many bytes run on the 256 x 256 core
constexpr int MX_WGRAD_HOT_BYTES = 256;

// Row quantisation: q[r] = E4M3 of src[gather ? gather[r] : r] (cols values) with
// one scale per 32; rows r < min(n_rows, *n_rows_dev) (n_rows_dev may be NULL).
hipError_t launch_quant_rows(int dt, const void* src, const int32_t* gather,
                             const int32_t* n_rows_dev, int n_rows, int cols, uint8_t* q,
                             uint8_t* sc, hipStream_t s);
// The same rows written from the source side (the dispatch of tokens into expert
// rows): q[pos[t, j]] = Q(src[t]) for t < n_tok, j < k, pos >= 0.
hipError_t launch_quant_scatter_rows(int dt, const void* src, const int32_t* pos, int n_tok, int k,
                                     int cols, uint8_t* q, uint8_t* sc, hipStream_t s);
// Column quantisation of batch x [rows, cols] into batch x [cols, rows] (blocks along rows).
hipError_t launch_quant_cols(int dt, const void* src, int batch, int rows, int cols, uint8_t* q,
                             uint8_t* sc, hipStream_t s);
// Token quantisation into the transposed token axis of the wgrads (dt 1: bf16
// source, 0: fp32 source) over a tile list of 128-row tiles (expert, first row) of
// a row space with expert offsets `offsets`.  Expert e's rows go to columns
// kpos[e] + (kseg ? kseg[e] : 0) + (row - offsets[e]), in blocks of 32 rows from
// its first row (the last block zero-padded); blocks without a row are not written.
// Row r is read from src row gather ? gather[r] : r.  kpad_total: the axis length
// (row pitch of q).
hipError_t launch_quant_tokens(int dt, const void* src, const int32_t* gather, int ld,
                               const int32_t* tiles, const int32_t* n_tiles,
                               const int32_t* offsets, const int32_t* kpos,
                               const int32_t* kseg, int max_tiles, int cols, size_t kpad_total,
                               uint8_t* q, uint8_t* sc, hipStream_t s);

// The minibatch plans of one macro batch (device pointers into the plan buffer).
struct MbPlanViews {
  int n_mb;
  const int32_t* counts[MX_MAX_MB];
  const int32_t* offsets[MX_MAX_MB];
  const int32_t* tiles[MX_MAX_MB];
  const int32_t* n_tiles[MX_MAX_MB];
  const int32_t* src_token[MX_MAX_MB];
};

// The wgrads' token axis over all minibatches (device arrays in the workspace):
// expert e's rows of the macro batch in token order are its global rows
// [goff[e], goff[e + 1]) (minibatch m's segment from goff[e] + cum[m * E + e]) and
// take the packed columns [kpos[e], kpos[e] + n_e), kpos advancing by n_e rounded
// up to 32; gtiles / n_gtiles: (expert, first global row) per 128 global rows;
// grow / gtok: per global row, its row in the per-minibatch arrays stored one
// minibatch after the other (m * R_mb + r) and its token.
struct MbAxis {
  int32_t* counts_all;
  int32_t* active;
  int32_t* n_active;
  int32_t* cum;     // [n_mb * E]
  int32_t* kpos;    // [E + 1]
  int32_t* goff;    // [E + 1]
  int32_t* gtiles;  // [max_gtiles * 2]
  int32_t* n_gtiles;
  int32_t* grow;    // [T * k]
  int32_t* gtok;    // [T * k]
};

// What the wgrad kernels read of the axis.
struct MbPlans {
  int n_mb;
  const int32_t* kpos;       // [E + 1]
  const int32_t* active;     // union over minibatches of the experts with rows
  const int32_t* n_active;
};

hipError_t launch_mb_union(const MbPlanViews& v, int E, const MbAxis& ax, hipStream_t s);
hipError_t launch_mb_rows(const MbPlanViews& v, int E, int max_tiles, int R_mb, int T_mb,
                          const MbAxis& ax, hipStream_t s);

hipError_t launch_mx_up_swiglu(const GroupInfo& g, const uint8_t* X8, const uint8_t* Xs,
                               const uint8_t* wg8, const uint8_t* wgs, const uint8_t* wu8,
                               const uint8_t* wus, int H, int I, float* Z, uint8_t* hq,
                               uint8_t* hs, hipStream_t s);
hipError_t launch_mx_down(const GroupInfo& g, const uint8_t* hq, const uint8_t* hs,
                          const uint8_t* wd8, const uint8_t* wds, int H, int I, void* Y,
                          hipStream_t s);
hipError_t launch_mx_dgrad_down(const GroupInfo& g, const uint8_t* dYu8, const uint8_t* dYus,
                                const uint8_t* wdT8, const uint8_t* wdTs, const float* Z,
                                const float* topk_w, int H, int I, int k, void* dZ, uint8_t* dZ8,
                                uint8_t* dZs, void* gh, float* dgp, hipStream_t s);
hipError_t launch_mx_dgrad_up(const GroupInfo& g, const uint8_t* dZ8, const uint8_t* dZs,
                              const uint8_t* wgT8, const uint8_t* wgTs, const uint8_t* wuT8,
                              const uint8_t* wuTs, int H, int I, void* dX, hipStream_t s);
// experts whose packed range has >= hot_bytes bytes are skipped (0: none)
hipError_t launch_mx_wgrad(const char* name, const MbPlans& mp, int E, const uint8_t* A8,
                           const uint8_t* As, const uint8_t* B8, const uint8_t* Bs, int M, int N,
                           int split, size_t Kp, void* out0, void* out1, int hot_bytes,
                           hipStream_t s);
// The same wgrads for the experts whose packed range has >= hot_bytes bytes on the
// 256 x 256 core (zeroes the operands' bytes past kpos[E] first); hipErrorNotSupported
// (nothing enqueued) for shapes the 256-tiles do not cover.
hipError_t launch_mx_wgrad_hot(const char* name, const MbPlans& mp, int E, uint8_t* A8,
                               const uint8_t* As, uint8_t* B8, const uint8_t* Bs, int M, int N,
                               int split, size_t Kp, void* out0, void* out1, int hot_bytes,
                               hipStream_t s);

}  // namespace moe
