// C-ABI of the MoE layer (include/moe.h): argument checks, buffer layouts and the
// enqueue sequences of the forward and backward passes.  Nothing here allocates device
// memory or synchronises with the host.  Every kernel goes onto the caller's stream,
// except in moe_forward_bf16 and the bf16 and MXFP8 backwards, which fork independent
// GEMMs onto a second stream of their own and join it back before returning (see
// SideStream).
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "internal.hpp"

using namespace moe;

typedef uint16_t bf16_t_host;  // bfloat16 bits on the host side

namespace moe {

thread_local ::moe_trace* tls_trace = nullptr;
thread_local int tls_cu_budget = 0;

int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (cus <= 0) cus = 256;
  return tls_cu_budget > 0 && tls_cu_budget < cus ? tls_cu_budget : cus;
}

void trace_before(hipStream_t s, const char* name) {
  moe_trace* t = tls_trace;
  if (!t || t->count >= t->capacity) return;
  t->names[t->count] = name;
  (void)hipEventRecord(t->events[2 * t->count], s);
}

void trace_after(hipStream_t s) {
  moe_trace* t = tls_trace;
  if (!t || t->count >= t->capacity) return;
  (void)hipEventRecord(t->events[2 * t->count + 1], s);
  ++t->count;
}

}  // namespace moe

namespace {

// A second stream (default priority) per host thread and device, for the part of one
// call's work that does not depend on the rest. fork() makes it wait for all that the
// caller's stream holds so far; join() makes the caller's stream wait for all that it
// holds. Everything a call enqueues thus stays ordered with the caller's stream
// before and after it, as if it had all gone onto that stream. side_stream() returns
// null where the stream or its events cannot be made; the caller then enqueues all
// its work on its own stream. Made on first use, kept until the process ends.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
  hipError_t fork(hipStream_t from) {
    hipError_t e = hipEventRecord(fork_ev, from);
    return e != hipSuccess ? e : hipStreamWaitEvent(s, fork_ev, 0);
  }
  hipError_t join(hipStream_t to) {
    hipError_t e = hipEventRecord(join_ev, s);
    return e != hipSuccess ? e : hipStreamWaitEvent(to, join_ev, 0);
  }
};

SideStream* side_stream() {
  constexpr int MAX_DEV = 64;
  thread_local SideStream tab[MAX_DEV];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return nullptr;
  SideStream& x = tab[dev];
  if (x.s) return &x;
  hipStream_t s = nullptr;
  hipEvent_t a = nullptr, b = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess &&
      hipEventCreateWithFlags(&a, hipEventDisableTiming) == hipSuccess &&
      hipEventCreateWithFlags(&b, hipEventDisableTiming) == hipSuccess) {
    x.fork_ev = a;
    x.join_ev = b;
    x.s = s;
    return &x;
  }
  if (b) (void)hipEventDestroy(b);
  if (a) (void)hipEventDestroy(a);
  if (s) (void)hipStreamDestroy(s);
  return nullptr;
}

constexpr size_t ALIGN = 256;

size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Carves consecutive 256-byte-aligned regions out of one buffer.
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += up(bytes);
    return o;
  }
};

// The bf16 GEMMs address activation rows and one expert's weights with 32-bit
// byte offsets from a base: every such operand must be smaller than 4 GiB.
bool bf16_offsets_fit(const moe_shape* s) {
  const uint64_t R = (uint64_t)s->T * s->k;
  const uint64_t w = std::max<uint64_t>({(uint64_t)s->H, 2ull * s->I, 2ull * s->I_shared});
  const uint64_t lim = 1ull << 32;
  return R * w * 2 < lim && (uint64_t)s->I * s->H * 2 < lim &&
         (uint64_t)s->I_shared * s->H * 2 < lim;
}

moe_status check_shape(const moe_shape* s, bool need_gemm_dims) {
  if (!s) return MOE_E_NULL;
  if (s->T < 0 || s->E < 1 || s->E > MOE_MAX_E || s->k < 1 || s->k > s->E || s->k > MOE_MAX_K)
    return MOE_E_SHAPE;
  if ((int64_t)s->T * s->k >= (int64_t)1 << 31) return MOE_E_SHAPE;
  if (s->H < 128 || s->H % 128) return MOE_E_SHAPE;
  if (s->flags & ~(MOE_REPLAY | MOE_FUSED_FORWARD)) return MOE_E_SHAPE;
  if (need_gemm_dims) {
    if (s->I < 128 || s->I % 128) return MOE_E_SHAPE;
    if (s->I_shared < 0 || s->I_shared % 128) return MOE_E_SHAPE;
    if (s->T_minibatch < 0) return MOE_E_SHAPE;
  }
  return MOE_OK;
}

// Minibatches: T_minibatch in (0, T) splits the tokens into ceil(T / T_minibatch)
// consecutive minibatches, each with its own plan; otherwise one minibatch of T.
int n_minibatches(const moe_shape* s) {
  if (s->T_minibatch <= 0 || s->T_minibatch >= s->T) return 1;
  return (s->T + s->T_minibatch - 1) / s->T_minibatch;
}
int minibatch_tokens(const moe_shape* s) { return n_minibatches(s) > 1 ? s->T_minibatch : s->T; }

// Layout of one minibatch plan (sized for minibatch_tokens(s) tokens).
moe_plan_layout plan_layout(const moe_shape* s) {
  moe_plan_layout L;
  memset(&L, 0, sizeof(L));
  const int64_t R = (int64_t)minibatch_tokens(s) * s->k;
  L.tile_m = GEMM_TILE_M;
  L.max_tiles = (int32_t)(R / GEMM_TILE_M + (R < s->E ? R : s->E) + 1);
  L.wtile_m = GEMM_WTILE_M;
  L.max_wtiles = (int32_t)(R / GEMM_WTILE_M + (R < s->E ? R : s->E) + 1);
  L.chunk_pairs = PLAN_CHUNK;
  L.n_chunks = (int32_t)((R + PLAN_CHUNK - 1) / PLAN_CHUNK);
  Carve c;
  L.counts = c.take(sizeof(int32_t) * s->E);
  L.offsets = c.take(sizeof(int32_t) * (s->E + 1));
  L.src_token = c.take(sizeof(int32_t) * R);
  L.src_slot = c.take(sizeof(int32_t) * R);
  L.pos = c.take(sizeof(int32_t) * R);
  L.tiles = c.take(sizeof(int32_t) * 2 * (size_t)L.max_tiles);
  L.n_tiles = c.take(sizeof(int32_t));
  L.err_flag = c.take(sizeof(int32_t));
  L.active = c.take(sizeof(int32_t) * s->E);
  L.n_active = c.take(sizeof(int32_t));
  L.tile_first = c.take(sizeof(int32_t) * (s->E + 1));
  L.wtiles = c.take(sizeof(int32_t) * 2 * (size_t)L.max_wtiles);
  L.n_wtiles = c.take(sizeof(int32_t));
  L.scratch = c.take(sizeof(int32_t) * ((size_t)L.n_chunks * s->E + L.n_chunks));
  L.sub_plan_bytes = c.off;
  L.n_minibatch = n_minibatches(s);
  L.T_minibatch = minibatch_tokens(s);
  L.total_bytes = L.sub_plan_bytes * L.n_minibatch;
  return L;
}

template <typename P>
P* at(void* base, size_t off) {
  return (P*)((char*)base + off);
}
template <typename P>
const P* at(const void* base, size_t off) {
  return (const P*)((const char*)base + off);
}

struct PlanView {
  const int32_t *counts, *offsets, *src_token, *src_slot, *pos, *tiles, *n_tiles, *active,
      *n_active, *tile_first, *wtiles, *n_wtiles;
  int max_tiles, max_wtiles;
};

// View of minibatch m's plan.
PlanView view_plan(const moe_shape* s, const void* plan_all, int m = 0) {
  const moe_plan_layout L = plan_layout(s);
  const void* plan = (const char*)plan_all + (size_t)m * L.sub_plan_bytes;
  PlanView v;
  v.counts = at<int32_t>(plan, L.counts);
  v.offsets = at<int32_t>(plan, L.offsets);
  v.src_token = at<int32_t>(plan, L.src_token);
  v.src_slot = at<int32_t>(plan, L.src_slot);
  v.pos = at<int32_t>(plan, L.pos);
  v.tiles = at<int32_t>(plan, L.tiles);
  v.n_tiles = at<int32_t>(plan, L.n_tiles);
  v.active = at<int32_t>(plan, L.active);
  v.n_active = at<int32_t>(plan, L.n_active);
  v.tile_first = at<int32_t>(plan, L.tile_first);
  v.wtiles = at<int32_t>(plan, L.wtiles);
  v.n_wtiles = at<int32_t>(plan, L.n_wtiles);
  v.max_tiles = L.max_tiles;
  v.max_wtiles = L.max_wtiles;
  return v;
}

GroupInfo grouped(const moe_shape* s, const PlanView& v) {
  GroupInfo g;
  g.tiles = v.tiles;
  g.n_tiles = v.n_tiles;
  g.offsets = v.offsets;
  g.src_token = v.src_token;
  g.src_slot = v.src_slot;
  g.active = v.active;
  g.n_active = v.n_active;
  g.counts = v.counts;
  g.wtiles = v.wtiles;
  g.n_wtiles = v.n_wtiles;
  g.max_tiles = v.max_tiles;
  g.max_wtiles = v.max_wtiles;
  g.dense_rows = 0;
  g.E = s->E;
  g.hot_rows = INT_MAX;
  return g;
}

GroupInfo dense(int rows) {
  GroupInfo g;
  memset(&g, 0, sizeof(g));
  g.dense_rows = rows;
  g.E = 1;
  g.hot_rows = INT_MAX;
  return g;
}

size_t esize(moe_dtype dt) { return dt == MOE_F32 ? 4 : 2; }

// saved: Z fp32 [R, 2I] then Zs fp32 [T, 2 Is] (gate | up pre-activations)
struct SavedLayout {
  size_t Z, Zs, total;
};
SavedLayout saved_layout(const moe_shape* s, moe_dtype) {
  const size_t R = (size_t)s->T * s->k;
  Carve c;
  SavedLayout L;
  L.Z = c.take(R * 2 * s->I * sizeof(float));
  L.Zs = c.take((size_t)s->T * 2 * s->I_shared * sizeof(float));
  L.total = c.off;
  return L;
}

// forward workspace: h [R, I], Y [R, H], hs [T, Is], ys [T, H], and the row-tile
// counters of the fused forward
struct FwdWs {
  size_t h, Y, hs, ys, ready, total;
};
FwdWs fwd_ws(const moe_shape* s, moe_dtype dt) {
  const size_t R = (size_t)s->T * s->k, es = esize(dt), T = s->T;
  Carve c;
  FwdWs L;
  L.h = c.take(R * s->I * es);
  L.Y = c.take(R * s->H * es);
  L.hs = c.take(T * s->I_shared * es);
  L.ys = c.take(s->I_shared ? T * s->H * es : 0);
  L.ready = c.take((s->flags & MOE_FUSED_FORWARD)
                       ? sizeof(int32_t) * fused_counters(plan_layout(s).max_wtiles, s->T)
                       : 0);
  L.total = c.off;
  return L;
}

// backward workspace: dZ [R, 2I], gh [R, I], dgp fp32 [R, I/128], dX [R, H],
// X [R, H] and dYu [R, H] (replayed gathers), dZs [T, 2Is], hs [T, Is], dxs [T, H]
struct BwdWs {
  size_t dZ, gh, dgp, dX, X, dYu, dZs, hs, dxs, total;
};
BwdWs bwd_ws(const moe_shape* s, moe_dtype dt) {
  const size_t R = (size_t)s->T * s->k, es = esize(dt), T = s->T;
  Carve c;
  BwdWs L;
  L.dZ = c.take(R * 2 * s->I * es);
  L.gh = c.take(R * s->I * es);
  L.dgp = c.take(R * (s->I / 128) * sizeof(float));
  L.dX = c.take(R * s->H * es);
  L.X = c.take(R * s->H * es);
  L.dYu = c.take(R * s->H * es);
  L.dZs = c.take(T * 2 * s->I_shared * es);
  L.hs = c.take(T * s->I_shared * es);
  L.dxs = c.take(s->I_shared ? T * s->H * es : 0);
  L.total = c.off;
  return L;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_HIP; }

#define MOE_TRY(expr)                         \
  do {                                        \
    const hipError_t e_ = (expr);             \
    if (e_ != hipSuccess) return MOE_E_HIP;   \
  } while (0)

bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned16(p)) return false;
  return true;
}

bool any_null(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return true;
  return false;
}

// Arrays whose size is a multiple of T may be NULL when T == 0.
bool any_null_rows(const moe_shape* s, std::initializer_list<const void*> ps) {
  return s->T > 0 && any_null(ps);
}

moe_status forward_impl(moe_dtype dt, const moe_shape* s, const void* plan, const void* x,
                        const float* topk_w, const void* wg, const void* wu, const void* wd,
                        const void* sg, const void* su, const void* sd, void* y, void* saved,
                        void* ws, size_t ws_bytes, hipStream_t st,
                        bool may_fork = false) {
  moe_status rc = check_shape(s, true);
  if (rc != MOE_OK) return rc;
  if (n_minibatches(s) != 1) return MOE_E_UNSUPPORTED;
  if (dt == MOE_BF16 && !bf16_offsets_fit(s)) return MOE_E_UNSUPPORTED;
  if (any_null({plan, wg, wu, wd}) || any_null_rows(s, {x, topk_w, y, saved, ws}))
    return MOE_E_NULL;
  if (s->I_shared && any_null({sg, su, sd})) return MOE_E_NULL;
  if (!all_aligned({plan, x, topk_w, wg, wu, wd, sg, su, sd, y, saved, ws})) return MOE_E_ALIGN;
  const FwdWs W = fwd_ws(s, dt);
  if (ws_bytes < W.total) return MOE_E_WORKSPACE;
  if (s->T == 0) return MOE_OK;
  const int d = dt == MOE_BF16 ? 1 : 0;
  const PlanView v = view_plan(s, plan);
  const SavedLayout S = saved_layout(s, dt);
  const GroupInfo g = grouped(s, v);
  void* Z = at<char>(saved, S.Z);
  void* h = at<char>(ws, W.h);
  void* Y = at<char>(ws, W.Y);
  void* ys = s->I_shared ? at<char>(ws, W.ys) : nullptr;
  if (d && (s->flags & MOE_FUSED_FORWARD)) {
    const moe_plan_layout P = plan_layout(s);
    FusedForwardArgs a;
    a.g = g;
    a.gs = dense(s->T);
    a.T = s->T;
    a.k = s->k;
    a.H = s->H;
    a.I = s->I;
    a.Is = s->I_shared;
    a.x = x;
    a.wg = wg;
    a.wu = wu;
    a.wd = wd;
    a.sg = sg;
    a.su = su;
    a.sd = sd;
    a.Z = Z;
    a.h = h;
    a.Y = Y;
    a.Zs = s->I_shared ? at<char>(saved, S.Zs) : nullptr;
    a.hs = s->I_shared ? at<char>(ws, W.hs) : nullptr;
    a.ys = ys;
    a.pos = v.pos;
    a.w = topk_w;
    a.y = y;
    a.ready = at<int32_t>(ws, W.ready);
    a.err = (int32_t*)((char*)const_cast<void*>(plan) + P.err_flag);
    const hipError_t fe = launch_big_forward_fused(a, st);
    if (fe == hipSuccess) return MOE_OK;
    if (fe != hipErrorNotSupported) return MOE_E_HIP;
  }
  // In the bf16 pass of moe_forward_bf16 the shared expert's two GEMMs, which read only
  // x, run on the side stream beside the routed ones (not while a kernel trace is set,
  // so that each kernel's events time it alone); joined on every return path.
  SideStream* side = d && may_fork && s->I_shared && !tls_trace ? side_stream() : nullptr;
  const hipStream_t sx = side ? side->s : st;
#define HIP_TRY(expr)                    \
  do {                                   \
    const hipError_t e_ = (expr);        \
    if (e_ != hipSuccess) return e_;     \
  } while (0)
  const auto enqueue = [&]() -> hipError_t {
    if (s->I_shared) {
      const GroupInfo gs = dense(s->T);
      void* Zs = at<char>(saved, S.Zs);
      void* hs = at<char>(ws, W.hs);
      HIP_TRY(launch_gemm_up_swiglu(d, gs, x, sg, su, s->H, s->I_shared, Zs, hs, sx));
      HIP_TRY(launch_gemm_down(d, gs, hs, sd, s->H, s->I_shared, ys, sx));
    }
    HIP_TRY(launch_gemm_up_swiglu(d, g, x, wg, wu, s->H, s->I, Z, h, st));
    HIP_TRY(launch_gemm_down(d, g, h, wd, s->H, s->I, Y, st));
    return hipSuccess;
  };
#undef HIP_TRY
  if (side) MOE_TRY(side->fork(st));
  hipError_t e = enqueue();
  if (side) {
    const hipError_t j = side->join(st);
    if (e == hipSuccess) e = j;
  }
  MOE_TRY(e);
  if (d)
    MOE_TRY(launch_combine_bf16(Y, v.pos, topk_w, ys, y, s->T, s->k, s->H, st));
  else
    MOE_TRY(launch_combine_f32((const float*)Y, v.pos, topk_w, (const float*)ys, (float*)y, s->T,
                               s->k, s->H, st));
  return MOE_OK;
}

moe_status backward_impl(moe_dtype dt, const moe_shape* s, const void* plan, const void* x,
                         const float* topk_w, const void* wg, const void* wu, const void* wd,
                         const void* sg, const void* su, const void* sd, const void* saved,
                         const void* dy, void* dx, void* dwg, void* dwu, void* dwd, void* dsg,
                         void* dsu, void* dsd, float* d_topk_w, void* ws, size_t ws_bytes,
                         hipStream_t st) {
  moe_status rc = check_shape(s, true);
  if (rc != MOE_OK) return rc;
  if (n_minibatches(s) != 1) return MOE_E_UNSUPPORTED;
  if (dt == MOE_BF16 && !bf16_offsets_fit(s)) return MOE_E_UNSUPPORTED;
  if (any_null({plan, wg, wu, wd, dwg, dwu, dwd}) ||
      any_null_rows(s, {x, topk_w, saved, dy, dx, d_topk_w, ws}))
    return MOE_E_NULL;
  if (s->I_shared && any_null({sg, su, sd, dsg, dsu, dsd})) return MOE_E_NULL;
  if (!all_aligned({plan, x, topk_w, wg, wu, wd, sg, su, sd, saved, dy, dx, dwg, dwu, dwd, dsg, dsu,
                    dsd, d_topk_w, ws}))
    return MOE_E_ALIGN;
  const BwdWs W = bwd_ws(s, dt);
  if (ws_bytes < W.total) return MOE_E_WORKSPACE;
  const int d = dt == MOE_BF16 ? 1 : 0;
  const PlanView v = view_plan(s, plan);
  const SavedLayout S = saved_layout(s, dt);
  const GroupInfo g = grouped(s, v);
  const int H = s->H, I = s->I, R = s->T * s->k;
  const void* Z = at<char>(saved, S.Z);
  void* dZ = at<char>(ws, W.dZ);
  void* gh = at<char>(ws, W.gh);
  float* dgp = at<float>(ws, W.dgp);
  void* dX = at<char>(ws, W.dX);
  void* X = at<char>(ws, W.X);
  void* dYu = at<char>(ws, W.dYu);
  const int es = d ? 2 : 4;
  // In the bf16 pass the dispatch replay of x and the up-projection wgrads, which only
  // wgrad-up reads or writes, run on a side stream beside the rest: the GEMMs after
  // dgrad-down are independent of one another, and each alone leaves the chip's
  // memory system partly idle. Both streams are joined before the combine.
  // (not while a kernel trace is set: each kernel's events then time it alone)
  SideStream* side = d && !tls_trace ? side_stream() : nullptr;
  const hipStream_t sx = side ? side->s : st;
  void* dxs = s->I_shared ? at<char>(ws, W.dxs) : nullptr;
#define HIP_TRY(expr)                    \
  do {                                   \
    const hipError_t e_ = (expr);        \
    if (e_ != hipSuccess) return e_;     \
  } while (0)
  // the shared expert's backward: it reads only dy, x and its saved activations
  const auto shared_expert = [&](hipStream_t ss) -> hipError_t {
    if (!s->I_shared) return hipSuccess;
    const int Is = s->I_shared;
    const GroupInfo gs = dense(s->T);
    const void* Zs = at<char>(saved, S.Zs);
    void* dZs = at<char>(ws, W.dZs);
    void* hs = at<char>(ws, W.hs);
    HIP_TRY(launch_gemm_dgrad_down(d, gs, dy, sd, Zs, nullptr, H, Is, 1, dZs, hs, nullptr, ss));
    HIP_TRY(launch_gemm_wgrad_down(d, gs, dy, hs, H, Is, dsd, ss));
    HIP_TRY(launch_gemm_dgrad_up(d, gs, dZs, sg, su, H, Is, dxs, ss));
    HIP_TRY(launch_gemm_wgrad_up(d, gs, dZs, x, H, Is, dsg, dsu, ss));
    return hipSuccess;
  };
  // the side stream is joined on every return path, failed launches included
  const auto enqueue = [&]() -> hipError_t {
    // reverse-combine: pull dy rows into expert order; replay the dispatch of x
    HIP_TRY(launch_scatter_rows(dy, dYu, v.pos, s->T, s->k, H * es, st));
    HIP_TRY(launch_scatter_rows(x, X, v.pos, s->T, s->k, H * es, sx));
    // dgrad-down + SwiGLU backward + router-weight-gradient partials
    HIP_TRY(launch_gemm_dgrad_down(d, g, dYu, wd, Z, topk_w, H, I, s->k, dZ, gh, dgp, st));
    HIP_TRY(launch_dg_reduce(dgp, v.pos, R, I / 128, d_topk_w, st));
    if (side) HIP_TRY(side->fork(st));  // dZ is written
    // the wgrads also write the zero gradients of experts without rows
    HIP_TRY(launch_gemm_wgrad_up(d, g, dZ, X, H, I, dwg, dwu, sx));
    HIP_TRY(launch_gemm_wgrad_down(d, g, dYu, gh, H, I, dwd, st));
    HIP_TRY(launch_gemm_dgrad_up(d, g, dZ, wg, wu, H, I, dX, st));
    HIP_TRY(shared_expert(st));
#undef HIP_TRY
    return hipSuccess;
  };
  if (side) MOE_TRY(side->fork(st));
  hipError_t e = enqueue();
  if (side) {
    const hipError_t j = side->join(st);
    if (e == hipSuccess) e = j;
  }
  MOE_TRY(e);
  if (d)
    MOE_TRY(launch_combine_bf16(dX, v.pos, nullptr, dxs, dx, s->T, s->k, H, st));
  else
    MOE_TRY(launch_combine_f32((const float*)dX, v.pos, nullptr, (const float*)dxs, (float*)dx,
                               s->T, s->k, H, st));
  return MOE_OK;
}

moe_status plan_one(const moe_shape* s, const moe_plan_layout& L, int T_m,
                           const int32_t* topk_idx, void* plan, hipStream_t st) {
  PlanPtrs p;
  p.counts = at<int32_t>(plan, L.counts);
  p.offsets = at<int32_t>(plan, L.offsets);
  p.src_token = at<int32_t>(plan, L.src_token);
  p.src_slot = at<int32_t>(plan, L.src_slot);
  p.pos = at<int32_t>(plan, L.pos);
  p.tiles = at<int32_t>(plan, L.tiles);
  p.n_tiles = at<int32_t>(plan, L.n_tiles);
  p.err_flag = at<int32_t>(plan, L.err_flag);
  p.active = at<int32_t>(plan, L.active);
  p.n_active = at<int32_t>(plan, L.n_active);
  p.tile_first = at<int32_t>(plan, L.tile_first);
  p.wtiles = at<int32_t>(plan, L.wtiles);
  p.n_wtiles = at<int32_t>(plan, L.n_wtiles);
  p.chunk_hist = at<int32_t>(plan, L.scratch);
  p.chunk_invalid = p.chunk_hist + (size_t)L.n_chunks * s->E;
  p.n_chunks = (int)(((int64_t)T_m * s->k + PLAN_CHUNK - 1) / PLAN_CHUNK);
  p.max_tiles = L.max_tiles;
  return hip_status(launch_plan(topk_idx, T_m, s->k, s->E, p, st));
}


// ------------------------------------------------------------------ MXFP8
// Quantised weights: forward orientation (blocks along each GEMM's K) and the
// transposed backward orientation, each an E4M3 array plus its scale bytes.
//   wg, wu [E, I, H] along H;  wd [E, H, I] along I;
//   wdT [E, I, H] = W_d^T along H;  wgT, wuT [E, H, I] = W_g^T, W_u^T along I.
struct MxWeights {
  size_t wg8, wgs, wu8, wus, wd8, wds, wdT8, wdTs, wgT8, wgTs, wuT8, wuTs, total;
};
MxWeights mx_weights_layout(const moe_shape* s) {
  const size_t n = (size_t)s->E * s->I * s->H, ns = n / 32;
  Carve c;
  MxWeights L;
  L.wg8 = c.take(n); L.wgs = c.take(ns);
  L.wu8 = c.take(n); L.wus = c.take(ns);
  L.wd8 = c.take(n); L.wds = c.take(ns);
  L.wdT8 = c.take(n); L.wdTs = c.take(ns);
  L.wgT8 = c.take(n); L.wgTs = c.take(ns);
  L.wuT8 = c.take(n); L.wuTs = c.take(ns);
  L.total = c.off;
  return L;
}

// Saved by the MX forward: Z fp32 of every minibatch (minibatch m's rows at
// m * R_mb; with MOE_REPLAY the last minibatch's only) and Zs fp32 [T, 2 Is].
struct MxSaved {
  size_t Z, Zs, total;
};
bool mx_replay(const moe_shape* s) { return (s->flags & MOE_REPLAY) && n_minibatches(s) > 1; }

MxSaved mx_saved_layout(const moe_shape* s) {
  const size_t R_mb = (size_t)minibatch_tokens(s) * s->k;
  const size_t n_saved = mx_replay(s) ? 1 : (size_t)n_minibatches(s);
  Carve c;
  MxSaved L;
  L.Z = c.take(n_saved * R_mb * 2 * s->I * sizeof(float));
  L.Zs = c.take((size_t)s->T * 2 * s->I_shared * sizeof(float));
  L.total = c.off;
  return L;
}

// Forward workspace: the ring of two minibatch slots of dispatched MX rows, the
// quantised h, Y, and the shared expert's h and output of one minibatch.
struct MxFwdWs {
  size_t ring8[2], rings[2], hq, hs, Y, hs_sh, ys, Zr, total;
};
MxFwdWs mx_fwd_ws(const moe_shape* s) {
  const size_t Tm = minibatch_tokens(s), R = Tm * s->k, H = s->H, I = s->I;
  Carve c;
  MxFwdWs L;
  for (int i = 0; i < 2; ++i) {
    L.ring8[i] = c.take(R * H);
    L.rings[i] = c.take(R * H / 32);
  }
  L.hq = c.take(R * I);
  L.hs = c.take(R * I / 32);
  L.Y = c.take(R * H * 2);
  // the shared expert runs once over all T tokens: h_s and its output for every token
  L.hs_sh = c.take((size_t)s->T * s->I_shared * 2);
  L.ys = c.take(s->I_shared ? (size_t)s->T * H * 2 : 0);
  // with MOE_REPLAY: Z of the minibatches before the last (not kept)
  L.Zr = c.take(mx_replay(s) ? R * 2 * I * sizeof(float) : 0);
  L.total = c.off;
  return L;
}

// Backward workspace: per-minibatch buffers (dYu ring, dZ MX, dg partials, dX), the
// fp32 dZ and g h of every minibatch (minibatch m's rows at m * R_mb), the
// token-quantised wgrad operands on the packed token axis of the macro batch (Kp
// bytes per row: each expert's rows of all minibatches padded to 32, plus at least
// 128 bytes of tail that the large-tile wgrad may read past the last expert) and the
// arrays that map that axis to the minibatch plans.
struct MxBwdWs {
  size_t ring8[2], rings[2], dZ, dZ8, dZs, gh, dgp, dX;
  size_t dYuT8, dYuTs, ghT8, ghTs, dZT8, dZTs, XT8, XTs;
  size_t counts_all, active, n_active, cum, kpos, goff, gtiles, n_gtiles, grow, gtok;
  size_t rX8, rXs, rZ, rhq, rhs;  // MOE_REPLAY: replayed dispatch, Z and (unused) h
  size_t dZs_sh, hs_sh, dxs, total;
  size_t Kp;
  int max_gtiles;
};
size_t mx_token_axis_bytes(const moe_shape* s) {
  const size_t R = (size_t)s->T * s->k;
  return (R + 32 * (size_t)std::min<size_t>(s->E, R) + 127) / 128 * 128 + 128;
}
MxBwdWs mx_bwd_ws(const moe_shape* s) {
  const size_t Tm = minibatch_tokens(s), R = Tm * s->k, H = s->H, I = s->I, T = s->T;
  const size_t nmb = n_minibatches(s), Rall = nmb * R, Rtot = T * s->k;
  const size_t Kp = mx_token_axis_bytes(s);
  Carve c;
  MxBwdWs L;
  for (int i = 0; i < 2; ++i) {
    L.ring8[i] = c.take(R * H);
    L.rings[i] = c.take(R * H / 32);
  }
  L.dZ = c.take(Rall * 2 * I * sizeof(float));
  L.dZ8 = c.take(R * 2 * I);
  L.dZs = c.take(R * 2 * I / 32);
  L.gh = c.take(Rall * I * sizeof(float));
  L.dgp = c.take(R * (I / 128) * sizeof(float));
  L.dX = c.take(R * H * 2);
  L.dYuT8 = c.take(H * Kp); L.dYuTs = c.take(H * Kp / 32);
  L.ghT8 = c.take(I * Kp); L.ghTs = c.take(I * Kp / 32);
  L.dZT8 = c.take(2 * I * Kp); L.dZTs = c.take(2 * I * Kp / 32);
  L.XT8 = c.take(H * Kp); L.XTs = c.take(H * Kp / 32);
  L.max_gtiles = (int)(Rtot / 128 + std::min<size_t>(s->E, Rtot) + 1);
  L.counts_all = c.take(sizeof(int32_t) * s->E);
  L.active = c.take(sizeof(int32_t) * s->E);
  L.n_active = c.take(sizeof(int32_t));
  L.cum = c.take(sizeof(int32_t) * nmb * s->E);
  L.kpos = c.take(sizeof(int32_t) * (s->E + 1));
  L.goff = c.take(sizeof(int32_t) * (s->E + 1));
  L.gtiles = c.take(sizeof(int32_t) * 2 * (size_t)L.max_gtiles);
  L.n_gtiles = c.take(sizeof(int32_t));
  L.grow = c.take(sizeof(int32_t) * Rtot);
  L.gtok = c.take(sizeof(int32_t) * Rtot);
  const size_t rp = mx_replay(s) ? 1 : 0;
  L.rX8 = c.take(rp * R * H);
  L.rXs = c.take(rp * R * H / 32);
  L.rZ = c.take(rp * R * 2 * I * sizeof(float));
  L.rhq = c.take(rp * R * I);
  L.rhs = c.take(rp * R * I / 32);
  L.dZs_sh = c.take(T * 2 * s->I_shared * 2);
  L.hs_sh = c.take(T * s->I_shared * 2);
  L.dxs = c.take(s->I_shared ? T * H * 2 : 0);
  L.total = c.off;
  L.Kp = Kp;
  return L;
}

// The MX GEMMs address a minibatch's E4M3 activation rows with 32-bit signed
// products row * width (width = H or 2I bytes), the wgrads a packed token-axis row
// with 32-bit offsets below 256 rows * Kp, and the shared expert's bf16 GEMMs run
// densely over all T tokens with the 32-bit byte offsets of the bf16 kernels.
bool mx_offsets_fit(const moe_shape* s) {
  const uint64_t R = (uint64_t)minibatch_tokens(s) * s->k;
  const uint64_t w = std::max<uint64_t>((uint64_t)s->H, 2ull * s->I);
  if (R * w >= (1ull << 31)) return false;
  const uint64_t ws = std::max<uint64_t>((uint64_t)s->H, 2ull * s->I_shared);
  if ((uint64_t)s->T * ws * 2 >= (1ull << 32) || (uint64_t)s->I_shared * s->H * 2 >= (1ull << 32))
    return false;
  return 256 * (uint64_t)mx_token_axis_bytes(s) < (1ull << 32);
}

moe_status check_mx(const moe_shape* s) {
  moe_status rc = check_shape(s, true);
  if (rc != MOE_OK) return rc;
  if (n_minibatches(s) > MX_MAX_MB) return MOE_E_SHAPE;
  if (!mx_offsets_fit(s)) return MOE_E_UNSUPPORTED;
  return MOE_OK;
}

moe_status forward_mx_impl(const moe_shape* s, const void* plan, const void* x,
                           const float* topk_w, const void* wq, const void* sg, const void* su,
                           const void* sd, void* y, void* saved, void* ws, size_t ws_bytes,
                           hipStream_t st) {
  moe_status rc = check_mx(s);
  if (rc != MOE_OK) return rc;
  if (any_null({plan, wq}) || any_null_rows(s, {x, topk_w, y, saved, ws})) return MOE_E_NULL;
  if (s->I_shared && any_null({sg, su, sd})) return MOE_E_NULL;
  if (!all_aligned({plan, x, topk_w, wq, sg, su, sd, y, saved, ws})) return MOE_E_ALIGN;
  const MxFwdWs W = mx_fwd_ws(s);
  if (ws_bytes < W.total) return MOE_E_WORKSPACE;
  if (s->T == 0) return MOE_OK;
  const MxWeights Q = mx_weights_layout(s);
  const MxSaved S = mx_saved_layout(s);
  const int H = s->H, I = s->I, k = s->k, nmb = n_minibatches(s), Tmb = minibatch_tokens(s);
  const uint8_t* q = (const uint8_t*)wq;
  // the shared expert (bf16, dense, per token) once over all tokens: 256-row tiles of
  // the whole batch fill the chip where a 2048-token minibatch gives 128 workgroups
  const bf16_t_host* ys_all = nullptr;
  if (s->I_shared) {
    const GroupInfo gs = dense(s->T);
    MOE_TRY(launch_gemm_up_swiglu(1, gs, x, sg, su, H, s->I_shared, at<float>(saved, S.Zs),
                                  at<char>(ws, W.hs_sh), st));
    MOE_TRY(launch_gemm_down(1, gs, at<char>(ws, W.hs_sh), sd, H, s->I_shared,
                             at<char>(ws, W.ys), st));
    ys_all = at<bf16_t_host>(ws, W.ys);
  }
  for (int m = 0; m < nmb; ++m) {
    const int T_m = std::min(Tmb, s->T - m * Tmb);
    const PlanView v = view_plan(s, plan, m);
    const GroupInfo g = grouped(s, v);
    const bf16_t_host* xm = (const bf16_t_host*)x + (size_t)m * Tmb * H;
    uint8_t* X8 = at<uint8_t>(ws, W.ring8[m & 1]);
    uint8_t* Xs = at<uint8_t>(ws, W.rings[m & 1]);
    float* Z = !mx_replay(s) ? at<float>(saved, S.Z) + (size_t)m * Tmb * k * 2 * I
                             : (m == nmb - 1 ? at<float>(saved, S.Z) : at<float>(ws, W.Zr));
    uint8_t* hq = at<uint8_t>(ws, W.hq);
    uint8_t* hs = at<uint8_t>(ws, W.hs);
    void* Y = at<char>(ws, W.Y);
    // dispatch into the ring slot, quantised along H on the way
    MOE_TRY(launch_quant_scatter_rows(1, xm, v.pos, T_m, k, H, X8, Xs, st));
    MOE_TRY(launch_mx_up_swiglu(g, X8, Xs, q + Q.wg8, q + Q.wgs, q + Q.wu8, q + Q.wus, H, I, Z,
                                hq, hs, st));
    MOE_TRY(launch_mx_down(g, hq, hs, q + Q.wd8, q + Q.wds, H, I, Y, st));
    const void* ys = ys_all ? ys_all + (size_t)m * Tmb * H : nullptr;
    MOE_TRY(launch_combine_bf16(Y, v.pos, topk_w + (size_t)m * Tmb * k, ys,
                                (bf16_t_host*)y + (size_t)m * Tmb * H, T_m, k, H, st));
  }
  return MOE_OK;
}

moe_status backward_mx_impl(const moe_shape* s, const void* plan, const void* x,
                            const float* topk_w, const void* wq, const void* sg, const void* su,
                            const void* sd, const void* saved, const void* dy, void* dx,
                            void* dwg, void* dwu, void* dwd, void* dsg, void* dsu, void* dsd,
                            float* d_topk_w, void* ws, size_t ws_bytes, hipStream_t st) {
  moe_status rc = check_mx(s);
  if (rc != MOE_OK) return rc;
  if (any_null({plan, wq, dwg, dwu, dwd}) || any_null_rows(s, {x, topk_w, saved, dy, dx, d_topk_w, ws}))
    return MOE_E_NULL;
  if (s->I_shared && any_null({sg, su, sd, dsg, dsu, dsd})) return MOE_E_NULL;
  if (!all_aligned({plan, x, topk_w, wq, sg, su, sd, saved, dy, dx, dwg, dwu, dwd, dsg, dsu, dsd,
                    d_topk_w, ws}))
    return MOE_E_ALIGN;
  const MxBwdWs W = mx_bwd_ws(s);
  if (ws_bytes < W.total) return MOE_E_WORKSPACE;
  const MxWeights Q = mx_weights_layout(s);
  const MxSaved S = mx_saved_layout(s);
  const moe_plan_layout P = plan_layout(s);
  const int H = s->H, I = s->I, k = s->k, nmb = n_minibatches(s), Tmb = minibatch_tokens(s);
  const uint8_t* q = (const uint8_t*)wq;
  // shared expert (bf16, dense over all tokens)
  void* dxs = nullptr;
  if (s->I_shared) {
    const int Is = s->I_shared;
    const GroupInfo gs = dense(s->T);
    const float* Zs = at<float>(saved, S.Zs);
    void* dZs = at<char>(ws, W.dZs_sh);
    void* hsh = at<char>(ws, W.hs_sh);
    dxs = at<char>(ws, W.dxs);
    MOE_TRY(launch_gemm_dgrad_down(1, gs, dy, sd, Zs, nullptr, H, Is, 1, dZs, hsh, nullptr, st));
    MOE_TRY(launch_gemm_wgrad_down(1, gs, dy, hsh, H, Is, dsd, st));
    MOE_TRY(launch_gemm_dgrad_up(1, gs, dZs, sg, su, H, Is, dxs, st));
    MOE_TRY(launch_gemm_wgrad_up(1, gs, dZs, x, H, Is, dsg, dsu, st));
  }
  // the wgrads' token axis over all minibatches: each expert's rows of the macro batch
  // in token order (global rows), their packed columns and plan rows
  MbPlanViews pv;
  memset(&pv, 0, sizeof(pv));
  pv.n_mb = nmb;
  for (int m = 0; m < nmb; ++m) {
    const PlanView v = view_plan(s, plan, m);
    pv.counts[m] = v.counts;
    pv.offsets[m] = v.offsets;
    pv.tiles[m] = v.tiles;
    pv.n_tiles[m] = v.n_tiles;
    pv.src_token[m] = v.src_token;
  }
  MbAxis ax;
  ax.counts_all = at<int32_t>(ws, W.counts_all);
  ax.active = at<int32_t>(ws, W.active);
  ax.n_active = at<int32_t>(ws, W.n_active);
  ax.cum = at<int32_t>(ws, W.cum);
  ax.kpos = at<int32_t>(ws, W.kpos);
  ax.goff = at<int32_t>(ws, W.goff);
  ax.gtiles = at<int32_t>(ws, W.gtiles);
  ax.n_gtiles = at<int32_t>(ws, W.n_gtiles);
  ax.grow = at<int32_t>(ws, W.grow);
  ax.gtok = at<int32_t>(ws, W.gtok);
  MOE_TRY(launch_mb_union(pv, s->E, ax, st));
  MOE_TRY(launch_mb_rows(pv, s->E, P.max_tiles, Tmb * k, Tmb, ax, st));
  MbPlans mp;
  mp.n_mb = nmb;
  mp.kpos = ax.kpos;
  mp.active = ax.active;
  mp.n_active = ax.n_active;
  for (int m = nmb - 1; m >= 0; --m) {
    const int T_m = std::min(Tmb, s->T - m * Tmb), R_m = T_m * k;
    const PlanView v = view_plan(s, plan, m);
    if (T_m <= 0) continue;
    const GroupInfo g = grouped(s, v);
    const size_t tok0 = (size_t)m * Tmb;
    const bf16_t_host* dym = (const bf16_t_host*)dy + tok0 * H;
    uint8_t* dYu8 = at<uint8_t>(ws, W.ring8[m & 1]);
    uint8_t* dYus = at<uint8_t>(ws, W.rings[m & 1]);
    const float* Z = at<float>(saved, S.Z) + tok0 * k * 2 * I;
    if (mx_replay(s)) {
      if (m == nmb - 1) {
        Z = at<float>(saved, S.Z);
      } else {
        // replay this minibatch's dispatch and up/gate GEMM for its pre-activations
        const bf16_t_host* xm = (const bf16_t_host*)x + tok0 * H;
        uint8_t* X8 = at<uint8_t>(ws, W.rX8);
        uint8_t* Xs = at<uint8_t>(ws, W.rXs);
        float* rZ = at<float>(ws, W.rZ);
        MOE_TRY(launch_quant_scatter_rows(1, xm, v.pos, T_m, k, H, X8, Xs, st));
        MOE_TRY(launch_mx_up_swiglu(g, X8, Xs, q + Q.wg8, q + Q.wgs, q + Q.wu8, q + Q.wus, H, I,
                                    rZ, at<uint8_t>(ws, W.rhq), at<uint8_t>(ws, W.rhs), st));
        Z = rZ;
      }
    }
    float* dZ = at<float>(ws, W.dZ) + tok0 * k * 2 * I;
    uint8_t* dZ8 = at<uint8_t>(ws, W.dZ8);
    uint8_t* dZsc = at<uint8_t>(ws, W.dZs);
    float* gh = at<float>(ws, W.gh) + tok0 * k * I;
    float* dgp = at<float>(ws, W.dgp);
    void* dX = at<char>(ws, W.dX);
    // reverse-combine into the ring slot, quantised along H
    MOE_TRY(launch_quant_scatter_rows(1, dym, v.pos, T_m, k, H, dYu8, dYus, st));
    MOE_TRY(launch_mx_dgrad_down(g, dYu8, dYus, q + Q.wdT8, q + Q.wdTs, Z, topk_w + tok0 * k, H,
                                 I, k, dZ, dZ8, dZsc, gh, dgp, st));
    MOE_TRY(launch_dg_reduce(dgp, v.pos, R_m, I / 128, d_topk_w + tok0 * k, st));
    MOE_TRY(launch_mx_dgrad_up(g, dZ8, dZsc, q + Q.wgT8, q + Q.wgTs, q + Q.wuT8, q + Q.wuTs, H, I,
                               dX, st));
    MOE_TRY(launch_combine_bf16(dX, v.pos, nullptr,
                                dxs ? (const bf16_t_host*)dxs + tok0 * H : nullptr,
                                (bf16_t_host*)dx + tok0 * H, T_m, k, H, st));
  }
  // wgrad operands of the macro batch, quantised along each expert's tokens (blocks
  // from its first row, spanning minibatches): dy and x pulled by token, g h and dZ
  // from the rows the minibatches stored
  MOE_TRY(launch_quant_tokens(1, dy, ax.gtok, H, ax.gtiles, ax.n_gtiles, ax.goff, ax.kpos, nullptr,
                              W.max_gtiles, H, W.Kp, at<uint8_t>(ws, W.dYuT8),
                              at<uint8_t>(ws, W.dYuTs), st));
  MOE_TRY(launch_quant_tokens(1, x, ax.gtok, H, ax.gtiles, ax.n_gtiles, ax.goff, ax.kpos, nullptr,
                              W.max_gtiles, H, W.Kp, at<uint8_t>(ws, W.XT8),
                              at<uint8_t>(ws, W.XTs), st));
  MOE_TRY(launch_quant_tokens(0, at<float>(ws, W.gh), ax.grow, I, ax.gtiles, ax.n_gtiles, ax.goff,
                              ax.kpos, nullptr, W.max_gtiles, I, W.Kp, at<uint8_t>(ws, W.ghT8),
                              at<uint8_t>(ws, W.ghTs), st));
  MOE_TRY(launch_quant_tokens(0, at<float>(ws, W.dZ), ax.grow, 2 * I, ax.gtiles, ax.n_gtiles,
                              ax.goff, ax.kpos, nullptr, W.max_gtiles, 2 * I, W.Kp,
                              at<uint8_t>(ws, W.dZT8), at<uint8_t>(ws, W.dZTs), st));
  // Experts with a long packed token range run on the 256-tile kernel; the 128-tile
  // kernel takes the others and stores the zero gradients of experts without rows.
  // The two projections' weight gradients are independent: the up-projection pair runs
  // on the side stream beside the down-projection pair (not while a kernel trace is
  // set, so that each kernel's events time it alone); joined on every return path.
  SideStream* side = tls_trace ? nullptr : side_stream();
  const hipStream_t sx = side ? side->s : st;
  const auto down = [&]() -> hipError_t {
    int hot = MX_WGRAD_HOT_BYTES;
    hipError_t e = launch_mx_wgrad_hot("mx_gemm_wgrad_down_hot", mp, s->E,
                                       at<uint8_t>(ws, W.dYuT8), at<uint8_t>(ws, W.dYuTs),
                                       at<uint8_t>(ws, W.ghT8), at<uint8_t>(ws, W.ghTs), H, I, H,
                                       W.Kp, dwd, nullptr, hot, st);
    if (e == hipErrorNotSupported) hot = 0;
    else if (e != hipSuccess) return e;
    return launch_mx_wgrad("mx_gemm_wgrad_down", mp, s->E, at<uint8_t>(ws, W.dYuT8),
                           at<uint8_t>(ws, W.dYuTs), at<uint8_t>(ws, W.ghT8),
                           at<uint8_t>(ws, W.ghTs), H, I, H, W.Kp, dwd, nullptr, hot, st);
  };
  const auto up = [&]() -> hipError_t {
    int hot = MX_WGRAD_HOT_BYTES;
    hipError_t e = launch_mx_wgrad_hot("mx_gemm_wgrad_up_hot", mp, s->E, at<uint8_t>(ws, W.dZT8),
                                       at<uint8_t>(ws, W.dZTs), at<uint8_t>(ws, W.XT8),
                                       at<uint8_t>(ws, W.XTs), 2 * I, H, I, W.Kp, dwg, dwu, hot,
                                       sx);
    if (e == hipErrorNotSupported) hot = 0;
    else if (e != hipSuccess) return e;
    return launch_mx_wgrad("mx_gemm_wgrad_up", mp, s->E, at<uint8_t>(ws, W.dZT8),
                           at<uint8_t>(ws, W.dZTs), at<uint8_t>(ws, W.XT8), at<uint8_t>(ws, W.XTs),
                           2 * I, H, I, W.Kp, dwg, dwu, hot, sx);
  };
  if (side) MOE_TRY(side->fork(st));
  hipError_t e = up();
  if (e == hipSuccess) e = down();
  if (side) {
    const hipError_t j = side->join(st);
    if (e == hipSuccess) e = j;
  }
  MOE_TRY(e);
  return MOE_OK;
}

// Workspace of moe_forward_bf16_noalloc: one static device array per GPU (each
// device that loads the library holds its own copy until the process ends).  In
// host code `scratch` names a host-side stand-in, not the device address: the
// address comes from hipGetSymbolAddress, once per device with that device current.
__device__ __attribute__((aligned(256))) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

moe_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MOE_E_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_E_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

void moe_trace_set(moe_trace* trace) { moe::tls_trace = trace; }

void moe_set_cu_budget(int32_t cus) { moe::tls_cu_budget = cus > 0 ? cus : 0; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_E_NULL: return "a required pointer is NULL";
    case MOE_E_SHAPE: return "shape out of range or not a supported multiple";
    case MOE_E_ALIGN: return "pointer not 16-byte aligned";
    case MOE_E_WORKSPACE: return "workspace too small";
    case MOE_E_UNSUPPORTED: return "valid request that the library does not implement";
    case MOE_E_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

moe_status moe_plan_layout_of(const moe_shape* shape, moe_plan_layout* out) {
  if (!out) return MOE_E_NULL;
  const moe_status rc = check_shape(shape, false);
  if (rc != MOE_OK) return rc;
  *out = plan_layout(shape);
  return MOE_OK;
}

size_t moe_plan_bytes(const moe_shape* shape) {
  if (check_shape(shape, false) != MOE_OK) return 0;
  return plan_layout(shape).total_bytes;
}

size_t moe_saved_bytes(const moe_shape* shape, moe_dtype dtype) {
  if (check_shape(shape, true) != MOE_OK) return 0;
  if (dtype == MOE_MXFP8) return check_mx(shape) == MOE_OK ? mx_saved_layout(shape).total : 0;
  return saved_layout(shape, dtype).total;
}

size_t moe_workspace_bytes(const moe_shape* shape, moe_dtype dtype, int backward) {
  if (check_shape(shape, true) != MOE_OK) return 0;
  if (dtype == MOE_MXFP8) {
    if (check_mx(shape) != MOE_OK) return 0;
    return backward ? mx_bwd_ws(shape).total : mx_fwd_ws(shape).total;
  }
  return backward ? bwd_ws(shape, dtype).total : fwd_ws(shape, dtype).total;
}

size_t moe_mx_weights_bytes(const moe_shape* shape) {
  if (check_shape(shape, true) != MOE_OK) return 0;
  return mx_weights_layout(shape).total;
}

moe_status moe_quantize_weights_mxfp8(const moe_shape* s, const void* w_gate, const void* w_up,
                                      const void* w_down, void* wq, hipStream_t st) {
  moe_status rc = check_shape(s, true);
  if (rc != MOE_OK) return rc;
  if (any_null({w_gate, w_up, w_down, wq})) return MOE_E_NULL;
  if (!all_aligned({w_gate, w_up, w_down, wq})) return MOE_E_ALIGN;
  const MxWeights L = mx_weights_layout(s);
  uint8_t* q = (uint8_t*)wq;
  const int E = s->E, H = s->H, I = s->I;
  MOE_TRY(launch_quant_rows(1, w_gate, nullptr, nullptr, E * I, H, q + L.wg8, q + L.wgs, st));
  MOE_TRY(launch_quant_rows(1, w_up, nullptr, nullptr, E * I, H, q + L.wu8, q + L.wus, st));
  MOE_TRY(launch_quant_rows(1, w_down, nullptr, nullptr, E * H, I, q + L.wd8, q + L.wds, st));
  MOE_TRY(launch_quant_cols(1, w_down, E, H, I, q + L.wdT8, q + L.wdTs, st));
  MOE_TRY(launch_quant_cols(1, w_gate, E, I, H, q + L.wgT8, q + L.wgTs, st));
  MOE_TRY(launch_quant_cols(1, w_up, E, I, H, q + L.wuT8, q + L.wuTs, st));
  return MOE_OK;
}

static moe_status quantize_mxfp8(int dt, const void* src, int64_t rows, int64_t cols, int axis,
                                 uint8_t* q, uint8_t* scales, hipStream_t st) {
  if (any_null({src, q, scales}) && rows * cols > 0) return MOE_E_NULL;
  if (!all_aligned({src, q})) return MOE_E_ALIGN;
  if (rows < 0 || cols < 0 || rows > INT32_MAX || cols > INT32_MAX) return MOE_E_SHAPE;
  if (rows * cols == 0) return MOE_OK;
  if (axis == 1) {
    if (cols % 32) return MOE_E_SHAPE;
    return hip_status(launch_quant_rows(dt, src, nullptr, nullptr, (int)rows, (int)cols, q, scales, st));
  }
  if (axis == 0) {
    if (rows % 32) return MOE_E_SHAPE;
    return hip_status(launch_quant_cols(dt, src, 1, (int)rows, (int)cols, q, scales, st));
  }
  return MOE_E_SHAPE;
}

moe_status moe_quantize_mxfp8(const void* src, int64_t rows, int64_t cols, int axis, uint8_t* q,
                              uint8_t* scales, hipStream_t st) {
  return quantize_mxfp8(1, src, rows, cols, axis, q, scales, st);
}

moe_status moe_quantize_mxfp8_f32(const float* src, int64_t rows, int64_t cols, int axis,
                                  uint8_t* q, uint8_t* scales, hipStream_t st) {
  return quantize_mxfp8(0, src, rows, cols, axis, q, scales, st);
}

moe_status moe_forward_mxfp8(const moe_shape* s, const void* plan, const void* x,
                             const float* topk_w, const void* wq, const void* s_gate,
                             const void* s_up, const void* s_down, void* y, void* saved, void* ws,
                             size_t ws_bytes, hipStream_t st) {
  return forward_mx_impl(s, plan, x, topk_w, wq, s_gate, s_up, s_down, y, saved, ws, ws_bytes, st);
}

moe_status moe_backward_mxfp8(const moe_shape* s, const void* plan, const void* x,
                              const float* topk_w, const void* wq, const void* s_gate,
                              const void* s_up, const void* s_down, const void* saved,
                              const void* dy, void* dx, void* dw_gate, void* dw_up, void* dw_down,
                              void* ds_gate, void* ds_up, void* ds_down, float* d_topk_w, void* ws,
                              size_t ws_bytes, hipStream_t st) {
  return backward_mx_impl(s, plan, x, topk_w, wq, s_gate, s_up, s_down, saved, dy, dx, dw_gate,
                          dw_up, dw_down, ds_gate, ds_up, ds_down, d_topk_w, ws, ws_bytes, st);
}

moe_status moe_router_logits_f32(const moe_shape* s, const float* x, const float* w_router,
                                 float* logits, hipStream_t st) {
  moe_status rc = check_shape(s, false);
  if (rc != MOE_OK) return rc;
  if (!w_router || any_null_rows(s, {x, logits})) return MOE_E_NULL;
  if (!all_aligned({x, w_router, logits})) return MOE_E_ALIGN;
  return hip_status(launch_router_logits_f32(x, w_router, s->T, s->H, s->E, logits, st));
}

moe_status moe_route(const moe_shape* s, const float* logits, int32_t* topk_idx, float* topk_w,
                     hipStream_t st) {
  moe_status rc = check_shape(s, false);
  if (rc != MOE_OK) return rc;
  if (any_null_rows(s, {logits, topk_idx, topk_w})) return MOE_E_NULL;
  if (!all_aligned({logits, topk_idx, topk_w})) return MOE_E_ALIGN;
  return hip_status(launch_route(logits, s->T, s->E, s->k, topk_idx, topk_w, st));
}

moe_status moe_route_backward(const moe_shape* s, const int32_t* topk_idx, const float* topk_w,
                              const float* d_topk_w, float* d_logits, hipStream_t st) {
  moe_status rc = check_shape(s, false);
  if (rc != MOE_OK) return rc;
  if (any_null_rows(s, {topk_idx, topk_w, d_topk_w, d_logits})) return MOE_E_NULL;
  if (!all_aligned({topk_idx, topk_w, d_topk_w, d_logits})) return MOE_E_ALIGN;
  return hip_status(
      launch_route_backward(topk_idx, topk_w, d_topk_w, s->T, s->E, s->k, d_logits, st));
}

moe_status moe_router_backward_f32(const moe_shape* s, const float* x, const float* w_router,
                                   const float* d_logits, float* dw_router, float* dx,
                                   hipStream_t st) {
  moe_status rc = check_shape(s, false);
  if (rc != MOE_OK) return rc;
  if (any_null({w_router, dw_router}) || any_null_rows(s, {x, d_logits, dx})) return MOE_E_NULL;
  if (!all_aligned({x, w_router, d_logits, dw_router, dx})) return MOE_E_ALIGN;
  return hip_status(
      launch_router_backward_f32(x, w_router, d_logits, s->T, s->H, s->E, dw_router, dx, st));
}

moe_status moe_plan(const moe_shape* s, const int32_t* topk_idx, void* plan, hipStream_t st) {
  moe_status rc = check_shape(s, false);
  if (rc != MOE_OK) return rc;
  if (!plan || any_null_rows(s, {topk_idx})) return MOE_E_NULL;
  if (!all_aligned({topk_idx, plan})) return MOE_E_ALIGN;
  const moe_plan_layout L = plan_layout(s);
  if (L.n_minibatch > MX_MAX_MB) return MOE_E_SHAPE;
  for (int m = 0; m < L.n_minibatch; ++m) {
    const int T_m = std::min(L.T_minibatch, s->T - m * L.T_minibatch);
    void* sub = (char*)plan + (size_t)m * L.sub_plan_bytes;
    const moe_status rc = plan_one(s, L, T_m, topk_idx + (size_t)m * L.T_minibatch * s->k, sub, st);
    if (rc != MOE_OK) return rc;
  }
  return MOE_OK;
}

static moe_status gather_impl(const moe_shape* s, const void* plan, const void* src, void* dst,
                              size_t es, hipStream_t st) {
  moe_status rc = check_shape(s, false);
  if (rc != MOE_OK) return rc;
  if (!plan || any_null_rows(s, {src, dst})) return MOE_E_NULL;
  if (!all_aligned({plan, src, dst})) return MOE_E_ALIGN;
  const PlanView v = view_plan(s, plan);
  return hip_status(launch_gather_rows(src, dst, v.src_token, v.offsets + s->E, s->T * s->k,
                                       (int)(s->H * es), st));
}

moe_status moe_dispatch_bf16(const moe_shape* s, const void* plan, const void* x, void* X,
                             hipStream_t st) {
  return gather_impl(s, plan, x, X, 2, st);
}
moe_status moe_dispatch_f32(const moe_shape* s, const void* plan, const float* x, float* X,
                            hipStream_t st) {
  return gather_impl(s, plan, x, X, 4, st);
}
moe_status moe_reverse_combine_bf16(const moe_shape* s, const void* plan, const void* dy,
                                    void* dYu, hipStream_t st) {
  return gather_impl(s, plan, dy, dYu, 2, st);
}

moe_status moe_combine_bf16(const moe_shape* s, const void* plan, const void* Y,
                            const float* topk_w, const void* shared_out, void* y,
                            hipStream_t st) {
  moe_status rc = check_shape(s, false);
  if (rc != MOE_OK) return rc;
  if (!plan || any_null_rows(s, {Y, topk_w, y})) return MOE_E_NULL;
  if (!all_aligned({plan, Y, topk_w, shared_out, y})) return MOE_E_ALIGN;
  const PlanView v = view_plan(s, plan);
  return hip_status(launch_combine_bf16(Y, v.pos, topk_w, shared_out, y, s->T, s->k, s->H, st));
}

moe_status moe_combine_f32(const moe_shape* s, const void* plan, const float* Y,
                           const float* topk_w, const float* shared_out, float* y,
                           hipStream_t st) {
  moe_status rc = check_shape(s, false);
  if (rc != MOE_OK) return rc;
  if (!plan || any_null_rows(s, {Y, topk_w, y})) return MOE_E_NULL;
  if (!all_aligned({plan, Y, topk_w, shared_out, y})) return MOE_E_ALIGN;
  const PlanView v = view_plan(s, plan);
  return hip_status(launch_combine_f32(Y, v.pos, topk_w, shared_out, y, s->T, s->k, s->H, st));
}

moe_status moe_reverse_dispatch_bf16(const moe_shape* s, const void* plan, const void* dX,
                                     const void* shared_dx, void* dx, hipStream_t st) {
  moe_status rc = check_shape(s, false);
  if (rc != MOE_OK) return rc;
  if (!plan || any_null_rows(s, {dX, dx})) return MOE_E_NULL;
  if (!all_aligned({plan, dX, shared_dx, dx})) return MOE_E_ALIGN;
  const PlanView v = view_plan(s, plan);
  return hip_status(launch_combine_bf16(dX, v.pos, nullptr, shared_dx, dx, s->T, s->k, s->H, st));
}

moe_status moe_forward_bf16(const moe_shape* s, const void* plan, const void* x,
                            const float* topk_w, const void* w_gate, const void* w_up,
                            const void* w_down, const void* s_gate, const void* s_up,
                            const void* s_down, void* y, void* saved, void* ws, size_t ws_bytes,
                            hipStream_t st) {
  return forward_impl(MOE_BF16, s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, y,
                      saved, ws, ws_bytes, st, true);
}

moe_status moe_forward_bf16_noalloc(const moe_shape* s, const void* plan, const void* x,
                                    const float* topk_w, const void* w_gate, const void* w_up,
                                    const void* w_down, const void* s_gate, const void* s_up,
                                    const void* s_down, void* y, void* saved, hipStream_t st) {
  moe_status rc = check_shape(s, true);
  if (rc != MOE_OK) return rc;
  if (fwd_ws(s, MOE_BF16).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_E_WORKSPACE;
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != MOE_OK) return rc;
  return forward_impl(MOE_BF16, s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, y,
                      saved, ws, MOE_NOALLOC_SCRATCH_BYTES, st);
}

moe_status moe_forward_f32(const moe_shape* s, const void* plan, const float* x,
                           const float* topk_w, const float* w_gate, const float* w_up,
                           const float* w_down, const float* s_gate, const float* s_up,
                           const float* s_down, float* y, void* saved, void* ws, size_t ws_bytes,
                           hipStream_t st) {
  return forward_impl(MOE_F32, s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, y,
                      saved, ws, ws_bytes, st);
}

moe_status moe_backward_bf16(const moe_shape* s, const void* plan, const void* x,
                             const float* topk_w, const void* w_gate, const void* w_up,
                             const void* w_down, const void* s_gate, const void* s_up,
                             const void* s_down, const void* saved, const void* dy, void* dx,
                             void* dw_gate, void* dw_up, void* dw_down, void* ds_gate,
                             void* ds_up, void* ds_down, float* d_topk_w, void* ws,
                             size_t ws_bytes, hipStream_t st) {
  return backward_impl(MOE_BF16, s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down,
                       saved, dy, dx, dw_gate, dw_up, dw_down, ds_gate, ds_up, ds_down, d_topk_w,
                       ws, ws_bytes, st);
}

moe_status moe_backward_f32(const moe_shape* s, const void* plan, const float* x,
                            const float* topk_w, const float* w_gate, const float* w_up,
                            const float* w_down, const float* s_gate, const float* s_up,
                            const float* s_down, const void* saved, const float* dy, float* dx,
                            float* dw_gate, float* dw_up, float* dw_down, float* ds_gate,
                            float* ds_up, float* ds_down, float* d_topk_w, void* ws,
                            size_t ws_bytes, hipStream_t st) {
  return backward_impl(MOE_F32, s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down,
                       saved, dy, dx, dw_gate, dw_up, dw_down, ds_gate, ds_up, ds_down, d_topk_w,
                       ws, ws_bytes, st);
}

}  // extern "C"
