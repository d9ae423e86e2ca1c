/*
 * moe.h — C-ABI of the deterministic MoE layer on one MI355X (gfx950).
 *
 * The layer, as the pages state the problem: a router sends each token to a
 * selection of experts, each a small feed-forward net with up, gate and down
 * projections (sebask.de, "Mixture-of-Kittens: Cursors Open-Source-Ansatz für
 * effizientes MoE-Training auf NVL72", introduction), the experts are SwiGLU
 * (stamatios.com, "Cursor abre código de megakernel MoE para GPUs NVL72",
 * § Outras características); tokens are dispatched to their experts and the
 * results combined back (sebask.de, § Das Kernproblem); one schedule table, built
 * on the GPU without sorting, serves all four movement operations (forward
 * dispatch and combine, backward reverse-combine and reverse-dispatch)
 * (sebask.de, § Push oder Pull; stamatios.com, § Escolha da direção de
 * comunicação); the operation order is fixed so that outputs are bitwise
 * reproducible (sebask.de, § Determinismus und MXFP8-Unterstützung;
 * stamatios.com, § Outras características).
 *
 * Conventions for every entry point
 *  - Every array pointer is a DEVICE pointer owned by the caller.  The library
 *    allocates no device memory, keeps no state between calls (apart from
 *    the optional per-thread timing trace below, and the side stream of
 *    moe_forward_bf16, moe_backward_bf16 and moe_backward_mxfp8), never
 *    synchronises the host and enqueues all work on
 *    `stream` (NULL = the null stream), or orders it with `stream` as if it
 *    were enqueued there.  Outputs are valid once the caller has synchronised
 *    the stream.
 *  - Matrices are row-major and contiguous.  Per-expert weights are stacked
 *    [E, out, in] (nn.Linear layout): w_gate, w_up [E, I, H]; w_down [E, H, I].
 *    Shared-expert weights: s_gate, s_up [I_shared, H]; s_down [H, I_shared].
 *  - "bf16" data is passed as `void*` (IEEE bfloat16, 2 bytes), fp32 as float*.
 *  - Every pointer must be 16-byte aligned.  With T == 0, arrays whose size is a
 *    multiple of T may be NULL (weights, weight gradients and the plan may not;
 *    the backward still overwrites the weight gradients with zeros).
 *  - Arguments are checked on the host before anything is enqueued; a failed
 *    check returns a status other than MOE_OK and enqueues nothing.
 *  - A data error that only the device can see (an expert id outside [0, E))
 *    sets the plan's err_flag: the pair is left out of the plan (its pos is -1)
 *    and the layer runs on the remaining pairs.
 *  - Calls on one stream are ordered; concurrent calls sharing output or
 *    workspace buffers on different streams race.
 *  - Results are bitwise identical across repeated calls with the same inputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_E_NULL = 1,        /* a required pointer is NULL */
  MOE_E_SHAPE = 2,       /* a size is out of range or not a supported multiple */
  MOE_E_ALIGN = 3,       /* a pointer is not 16-byte aligned */
  MOE_E_WORKSPACE = 4,   /* workspace smaller than moe_workspace_bytes() */
  MOE_E_UNSUPPORTED = 5, /* valid request that the library does not implement */
  MOE_E_HIP = 6          /* a HIP launch failed (hipGetLastError) */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP8 = 2 } moe_dtype;

/* T tokens, H hidden, I expert intermediate, E experts, k experts per token,
 * I_shared intermediate of the always-on shared expert (0 = none),
 * T_minibatch tokens per minibatch (0 = T).
 * Limits: 0 <= T, T*k < 2^31, 1 <= E <= 1024, 1 <= k <= min(E, 32);
 * H, I and I_shared multiples of 128 for the expert GEMMs; the bf16 and fp32
 * layer calls take one minibatch (T_minibatch 0 or >= T), the MXFP8 calls at
 * most 8.  The bf16 layer calls also need T*k*max(H, 2I, 2 I_shared)*2 bytes and
 * I*H*2, I_shared*H*2 bytes below 4 GiB (MOE_E_UNSUPPORTED otherwise).  The MXFP8
 * layer calls need T_minibatch*k*max(H, 2I) below 2^31 (T*k when T_minibatch is 0),
 * T*max(H, 2 I_shared)*2 and I_shared*H*2 below 2^32, and 256 times the packed
 * token-axis length (n_minibatch * max_tiles * 128, see moe_plan_layout) below 2^32
 * (MOE_E_UNSUPPORTED otherwise; the size queries then return 0). */
typedef struct {
  int32_t T, H, I, E, k;
  int32_t I_shared;
  int32_t T_minibatch;
  int32_t flags; /* MOE_REPLAY | MOE_FUSED_FORWARD or 0; other bits: MOE_E_SHAPE */
} moe_shape;

/* MXFP8 calls with several minibatches: the forward keeps the pre-activations of
 * the last minibatch only (the one still in the ring when the forward ends, which
 * the backward, walking the minibatches in reverse, needs first) and the backward
 * replays the dispatch and the up/gate GEMM of the others (stamatios.com, § Ring
 * token buffers: a reverse ring in the forward keeps the activation replay of the
 * backward small).  Outputs are bitwise the same as without it; moe_saved_bytes
 * shrinks by a factor of n_minibatch for the routed experts.  No effect on the bf16
 * and fp32 calls (one minibatch). */
#define MOE_REPLAY 1

/* bf16 forward: everything after the plan (the up/gate GEMMs with SwiGLU and the
 * down GEMMs of the routed and the shared experts, and the combine) runs as one
 * persistent kernel; each down-GEMM tile starts as soon as the up/gate tiles of its
 * rows have signalled through a device counter, and the combine once every down-GEMM
 * tile has (stamatios.com, § Granularidade do overlap and § Outras características:
 * one kernel whose units signal each other through counters).  Outputs are bitwise
 * the same as without it.
 * A tile gives up waiting after about two seconds, which can only happen when other
 * work keeps the GPU's compute units from the kernel that long; bit 1 (value 2) of
 * the plan's err_flag is then set and y is not valid. */
#define MOE_FUSED_FORWARD 2

/* Where each array of the schedule table sits inside the plan buffer (byte
 * offsets from its start; all 256-byte aligned).  With R = T*k:
 *   counts    int32 [E]      rows routed to each expert
 *   offsets   int32 [E+1]    exclusive prefix of counts; offsets[E] = valid rows
 *   src_token int32 [R]      pull list: token of row r (-1 past offsets[E])
 *   src_slot  int32 [R]      pull list: slot j of row r (-1 past offsets[E])
 *   pos       int32 [T, k]   inverse: row of pair (t, j), -1 if left out
 *   tiles     int32 [max_tiles, 2]  (expert, first row) per tile_m rows of each
 *                            expert, experts in id order; n_tiles entries valid
 *   n_tiles   int32 [1]
 *   err_flag  int32 [1]      bit 0: some expert id was outside [0, E); bit 1: a
 *                            MOE_FUSED_FORWARD wait gave up (see there)
 *   active    int32 [E]      ids of the experts with rows, ascending; n_active valid
 *   n_active  int32 [1]
 *   tile_first int32 [E+1]   index of each expert's first entry in `tiles`
 *   wtiles    int32 [max_wtiles, 2]  the same list for wtile_m-row tiles (the
 *                            wide-tile bf16 GEMMs); n_wtiles entries valid
 *   n_wtiles  int32 [1]
 *   scratch   per-chunk histograms used while building the plan
 * With T_minibatch in (0, T) the tokens form n_minibatch = ceil(T / T_minibatch)
 * consecutive minibatches and the plan buffer holds one such table per minibatch
 * (sized for T_minibatch tokens; minibatch m at byte m * sub_plan_bytes, covering
 * tokens m * T_minibatch ..); R above is then T_minibatch * k.  Otherwise there is
 * one table and T_minibatch reads T. */
typedef struct {
  size_t counts, offsets, src_token, src_slot, pos, tiles, n_tiles, err_flag, active, n_active,
      tile_first, wtiles, n_wtiles, scratch;
  size_t sub_plan_bytes, total_bytes;
  int32_t tile_m, max_tiles, chunk_pairs, n_chunks, n_minibatch, T_minibatch;
  int32_t wtile_m, max_wtiles;
} moe_plan_layout;

const char* moe_status_str(moe_status s);

/* Per-kernel timing.  While a trace is set on a host thread, every kernel that a
 * call from that thread enqueues is bracketed by events[2 i] (before) and
 * events[2 i + 1] (after), recorded on the stream the kernel runs on (the call's
 * stream or the side stream of the backwards), and names[i] is set to
 * the kernel's name (a static string); i runs from the trace's `count`, which the
 * library increments, up to `capacity` (later kernels are not recorded).  The
 * caller creates the 2 * capacity events and reads them with hipEventElapsedTime
 * after synchronising.  moe_trace_set(NULL) stops tracing.  Apart from the side
 * stream of the backwards, this is the only state the library keeps; both are
 * per host thread. */
typedef struct moe_trace {
  hipEvent_t* events;
  const char** names;
  int32_t capacity;
  int32_t count;
} moe_trace;

void moe_trace_set(moe_trace* trace);

/* Compute units that the persistent kernels of calls from this host thread size
 * their grids for (the weight-gradient kernels run a fixed number of workgroups
 * that walk their work items): 0 (the default) = every CU of the device, otherwise
 * min(cus, the device's CUs).  For callers that keep CUs busy with other work on
 * another stream, as the pages partition SMs in software between communication and
 * computation (stamatios.com, § Granularidade do overlap).  Outputs do not depend
 * on it: every output element is produced by one workgroup with a fixed K order
 * (sebask.de, § Determinismus und MXFP8-Unterstützung).  Per host thread, like the
 * trace. */
void moe_set_cu_budget(int32_t cus);

/* Layout and size of the plan buffer for `shape` (T, k, E are used). */
moe_status moe_plan_layout_of(const moe_shape* shape, moe_plan_layout* out);
size_t moe_plan_bytes(const moe_shape* shape);

/* Bytes of activations the forward keeps for the backward (`saved`):
 * Z = (A | B) fp32 [T*k, 2I] (gate and up pre-activations of every routed row)
 * followed by Zs fp32 [T, 2*I_shared] for the shared expert.  They stay fp32 in
 * every variant: the SwiGLU backward multiplies by silu'(A), which magnifies a
 * rounding of A near its zero. */
size_t moe_saved_bytes(const moe_shape* shape, moe_dtype dtype);

/* Scratch bytes of moe_forward_* (backward = 0) or moe_backward_* (backward = 1). */
size_t moe_workspace_bytes(const moe_shape* shape, moe_dtype dtype, int backward);

/* ---------------------------------------------------------------- router */

/* Router scores of the fp32 workload: logits [T, E] = x [T, H] * w_router[E, H]^T.
 * (sebask.de, introduction: a router distributes tokens to experts.) */
moe_status moe_router_logits_f32(const moe_shape* shape, const float* x, const float* w_router,
                                 float* logits, hipStream_t stream);

/* Top-k routing (sebask.de, introduction).  For each token the k experts with
 * the largest logits are taken in order (logit descending, expert id ascending;
 * -0.0 ties with +0.0), and topk_w holds the softmax of the k selected logits.
 *   logits   fp32 [T, E]   in
 *   topk_idx int32 [T, k]  out
 *   topk_w   fp32 [T, k]   out
 * NaN logits are not supported. */
moe_status moe_route(const moe_shape* shape, const float* logits, int32_t* topk_idx,
                     float* topk_w, hipStream_t stream);

/* Gradient of the logits from the gradient of the gates: for selected experts
 * d_logits[t, e_j] = w_j (d_w_j - sum_i w_i d_w_i), 0 elsewhere.
 *   d_topk_w fp32 [T, k] in; d_logits fp32 [T, E] out (overwritten). */
moe_status moe_route_backward(const moe_shape* shape, const int32_t* topk_idx,
                              const float* topk_w, const float* d_topk_w, float* d_logits,
                              hipStream_t stream);

/* Backward of moe_router_logits_f32: dw_router [E, H] = d_logits^T x
 * (overwritten) and dx [T, H] += d_logits w_router (accumulated in place). */
moe_status moe_router_backward_f32(const moe_shape* shape, const float* x,
                                   const float* w_router, const float* d_logits,
                                   float* dw_router, float* dx, hipStream_t stream);

/* ------------------------------------------------------------------ plan */

/* Build the schedule table from the routing (sebask.de, § Das Scheduling: the
 * pull schedule is a list of sources whose order follows from the routing and
 * is built entirely on the GPU; stamatios.com, § Escolha da direção: built once,
 * reused by the four operations, no sorting).  A counting sort: rows of expert
 * e are its pairs in ascending t*k + j.  `plan` is a buffer of
 * moe_plan_bytes(shape) bytes laid out as moe_plan_layout_of() reports.
 *   topk_idx int32 [T, k] in. */
moe_status moe_plan(const moe_shape* shape, const int32_t* topk_idx, void* plan,
                    hipStream_t stream);

/* ---------------------------------------------------- row movement (bf16/f32)
 * Building blocks of the four movement operations, one GPU's share.  The
 * layer entry points fuse dispatch and reverse-combine into the loaders of the
 * expert GEMMs; these exported forms are the same gathers, materialised. */

/* Dispatch, pull form (sebask.de, § Push oder Pull: dispatch pulls):
 * X[r, :] = x[src_token[r], :] for the valid rows r < offsets[E].
 * x [T, H] in; X [T*k, H] out (rows past offsets[E] untouched). */
moe_status moe_dispatch_bf16(const moe_shape* shape, const void* plan, const void* x, void* X,
                             hipStream_t stream);
moe_status moe_dispatch_f32(const moe_shape* shape, const void* plan, const float* x, float* X,
                            hipStream_t stream);

/* Combine in token order (sebask.de, § Push oder Pull: combine keeps the token
 * order; stamatios.com, § Outras características: fixed order):
 * y[t, :] = round( sum_{j=0..k-1} topk_w[t, j] * Y[pos[t, j], :]  + shared_out[t, :] ),
 * accumulated in fp32 from zero in ascending j, the shared term added last,
 * one rounding to the output type.  Y [T*k, H] in; shared_out [T, H] in or NULL;
 * y [T, H] out. */
moe_status moe_combine_bf16(const moe_shape* shape, const void* plan, const void* Y,
                            const float* topk_w, const void* shared_out, void* y,
                            hipStream_t stream);
moe_status moe_combine_f32(const moe_shape* shape, const void* plan, const float* Y,
                           const float* topk_w, const float* shared_out, float* y,
                           hipStream_t stream);

/* Reverse-combine, pull form (stamatios.com, § Escolha da direção: pull for the
 * backward reverse-combine): dYu[r, :] = dy[src_token[r], :].  Same gather as
 * dispatch; dy [T, H] in, dYu [T*k, H] out. */
moe_status moe_reverse_combine_bf16(const moe_shape* shape, const void* plan, const void* dy,
                                    void* dYu, hipStream_t stream);

/* Reverse-dispatch in fixed order (sebask.de, § Push oder Pull: the four
 * operations): dx[t, :] = round( sum_{j ascending} dX[pos[t, j], :] + shared_dx[t, :] )
 * in fp32.  dX [T*k, H] in; shared_dx [T, H] in or NULL; dx [T, H] out. */
moe_status moe_reverse_dispatch_bf16(const moe_shape* shape, const void* plan, const void* dX,
                                     const void* shared_dx, void* dx, hipStream_t stream);

/* ------------------------------------------------------------ layer, bf16 */

/* Forward of the expert part of the layer (sebask.de, introduction; stamatios.com,
 * § Outras características: SwiGLU experts, shared expert):
 *   per routed row r of expert e:  A = X_r W_g[e]^T, B = X_r W_u[e]^T,
 *   h = silu(A) * B, Y_r = h W_d[e]^T, with X_r = x[src_token[r]] gathered in the
 *   GEMM loader; shared expert S(x) = (silu(x S_g^T) * (x S_u^T)) S_d^T;
 *   y = combine(Y) + S(x) as in moe_combine_bf16.
 * bf16 operands, fp32 accumulation; A and B are kept in fp32 (`saved`), h is
 * formed from them in fp32 and rounded to bf16, as is Y.
 *   plan   from moe_plan on the same topk_idx
 *   x [T, H], topk_w fp32 [T, k], weights as in the conventions
 *   s_gate, s_up, s_down: NULL when shape->I_shared == 0
 *   y [T, H] out; saved [moe_saved_bytes] out; ws [ws_bytes >= moe_workspace_bytes(.., 0)].
 * T_minibatch must be 0 or T in this variant.  The shared expert's two GEMMs run on
 * the side stream described at moe_backward_bf16, under the same rules (not in
 * moe_forward_bf16_noalloc, nor with MOE_FUSED_FORWARD). */
moe_status moe_forward_bf16(const moe_shape* shape, const void* plan, const void* x,
                            const float* topk_w, const void* w_gate, const void* w_up,
                            const void* w_down, const void* s_gate, const void* s_up,
                            const void* s_down, void* y, void* saved, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): moe_forward_bf16 with its workspace in a
 * static device array of the library instead of a caller buffer.  It allocates
 * nothing and calls no allocating routine; the caller passes inputs and outputs as
 * for moe_forward_bf16 (y, saved).  The array holds MOE_NOALLOC_SCRATCH_BYTES per
 * GPU, from the library's first use of a GPU until the process ends; shapes whose
 * forward workspace, moe_workspace_bytes(shape, MOE_BF16, 0), is larger return
 * MOE_E_WORKSPACE (at H = 7168, I = I_shared = 2048, k = 8: up to 404 tokens).
 * Every call on one GPU uses that GPU's one array: calls that overlap on a GPU (on
 * different streams, or from different threads without ordering) race.  Nothing
 * in the array needs to start at zero: every workspace element the forward reads
 * it has written earlier in the same call. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_bf16_noalloc(const moe_shape* shape, const void* plan, const void* x,
                                    const float* topk_w, const void* w_gate, const void* w_up,
                                    const void* w_down, const void* s_gate, const void* s_up,
                                    const void* s_down, void* y, void* saved, hipStream_t stream);

/* Backward, the mirror of the forward (sebask.de, § Push oder Pull: reverse-combine
 * and reverse-dispatch; stamatios.com, § Outras características: router-weight
 * gradient fused into the SwiGLU backward):
 *   dh' = dy[src_token[r]] W_d[e]       (reverse-combine gathered in the loader)
 *   d_topk_w[t, j] = <dh'_r, h_r>       (= <dy_t, Y_r>), reduced in fixed order
 *   dh = w dh'; dA = dh B silu'(A); dB = dh silu(A)   (h, A, B from `saved`)
 *   dW_d[e] = sum_r dy_r (x) (w h)_r;  dW_g[e] = dA^T X_e;  dW_u[e] = dB^T X_e
 *   dX_r = dA W_g[e] + dB W_u[e];  dx = reverse-dispatch(dX) + shared dx
 * Outputs are overwritten: dx [T, H]; dw_* like the weights (experts with no
 * rows get zeros); ds_* like the shared weights (NULL without a shared expert);
 * d_topk_w fp32 [T, k] (0 for pairs left out of the plan).
 * ws [ws_bytes >= moe_workspace_bytes(.., 1)].
 * The dispatch replay of x and the up-projection weight gradients run on a second
 * stream of default priority that the library makes, once per host thread and
 * device, on the first call; it waits for the work enqueued on `stream` before the
 * call, and `stream` waits for it before the call's last kernel, also when a launch
 * fails. Where that stream cannot be made, and while a kernel trace is set on the
 * calling thread (so that each kernel's events time it alone), all the work goes
 * onto `stream`. A caller that captures the backward into a HIP graph makes one
 * uncaptured call on that thread and device first, so that the stream and its
 * events exist before the capture. */
moe_status moe_backward_bf16(const moe_shape* shape, const void* plan, const void* x,
                             const float* topk_w, const void* w_gate, const void* w_up,
                             const void* w_down, const void* s_gate, const void* s_up,
                             const void* s_down, const void* saved, const void* dy, void* dx,
                             void* dw_gate, void* dw_up, void* dw_down, void* ds_gate,
                             void* ds_up, void* ds_down, float* d_topk_w, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------- layer, fp32
 * The same computation with fp32 operands and outputs (fp32 MFMA, fp32
 * intermediates); arguments as the bf16 forms with float pointers. */
moe_status moe_forward_f32(const moe_shape* shape, const void* plan, const float* x,
                           const float* topk_w, const float* w_gate, const float* w_up,
                           const float* w_down, const float* s_gate, const float* s_up,
                           const float* s_down, float* y, void* saved, void* ws,
                           size_t ws_bytes, hipStream_t stream);
moe_status moe_backward_f32(const moe_shape* shape, const void* plan, const float* x,
                            const float* topk_w, const float* w_gate, const float* w_up,
                            const float* w_down, const float* s_gate, const float* s_up,
                            const float* s_down, const void* saved, const float* dy, float* dx,
                            float* dw_gate, float* dw_up, float* dw_down, float* ds_gate,
                            float* ds_up, float* ds_down, float* d_topk_w, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ layer, MXFP8
 * MXFP8 training with the conversion inside the kernels and the shared expert in
 * BF16 (sebask.de, § Determinismus und MXFP8-Unterstützung; stamatios.com,
 * § Outras características).  Every operand of the six expert GEMMs is E4M3 with
 * one E8M0 scale per 32 elements along that GEMM's K (OCP MX v1.0 rule: scale
 * exponent floor(log2 amax) - 8, elements rounded to nearest even and saturated):
 * x and dy along H (quantised while they are gathered into the ring of minibatch
 * slots), h along I, dZ = (dA | dB) along 2I, the weights along H or I (both
 * orientations, from moe_quantize_weights_mxfp8), and the wgrad operands along
 * the tokens of each expert: its rows of the whole call in token order, in blocks
 * of 32 from its first row (zero-padded), whatever the minibatch size, so that the
 * weight gradients are bitwise the same for every T_minibatch (sebask.de,
 * § Determinismus und MXFP8-Unterstützung).  Tokens run in minibatches of
 * shape->T_minibatch (at most 8 per call; 0 = one minibatch) through a ring of two
 * slots of T_minibatch * k dispatched rows (stamatios.com, § Ring token buffers
 * and § Granularidade do overlap); the plan must come from moe_plan with the same
 * shape.  Weight gradients are summed over all minibatches in one pass. */

/* Bytes of the quantised expert weights (both orientations, codes and scales). */
size_t moe_mx_weights_bytes(const moe_shape* shape);

/* Quantise w_gate, w_up [E, I, H] and w_down [E, H, I] (bf16) into `wq`: w_gate
 * and w_up along H, w_down along I (forward), w_down along H and w_gate, w_up along
 * I (backward, stored transposed). */
moe_status moe_quantize_weights_mxfp8(const moe_shape* shape, const void* w_gate,
                                      const void* w_up, const void* w_down, void* wq,
                                      hipStream_t stream);

/* Quantise a bf16 matrix src [rows, cols].  axis = 1: blocks of 32 along cols,
 * q [rows, cols], scales [rows, cols / 32].  axis = 0: blocks of 32 along rows,
 * written transposed: q [cols, rows], scales [cols, rows / 32]. */
moe_status moe_quantize_mxfp8(const void* src, int64_t rows, int64_t cols, int axis, uint8_t* q,
                              uint8_t* scales, hipStream_t stream);

/* The same for an fp32 matrix, as the MXFP8 backward quantises its fp32
 * intermediates (dZ and g h along the tokens): the rule applied to the fp32 value. */
moe_status moe_quantize_mxfp8_f32(const float* src, int64_t rows, int64_t cols, int axis,
                                  uint8_t* q, uint8_t* scales, hipStream_t stream);

/* As moe_forward_bf16 with the expert weights replaced by `wq`; the shared-expert
 * weights s_* stay bf16.  saved: moe_saved_bytes(shape, MOE_MXFP8); ws:
 * moe_workspace_bytes(shape, MOE_MXFP8, 0). */
moe_status moe_forward_mxfp8(const moe_shape* shape, const void* plan, const void* x,
                             const float* topk_w, const void* wq, const void* s_gate,
                             const void* s_up, const void* s_down, void* y, void* saved, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* As moe_backward_bf16 with the expert weights replaced by `wq`; weight gradients
 * are bf16 and overwritten. ws: moe_workspace_bytes(shape, MOE_MXFP8, 1).  The
 * up-projection weight gradients run on the side stream described at
 * moe_backward_bf16, beside the down-projection ones, under the same rules. */
moe_status moe_backward_mxfp8(const moe_shape* shape, const void* plan, const void* x,
                              const float* topk_w, const void* wq, const void* s_gate,
                              const void* s_up, const void* s_down, const void* saved,
                              const void* dy, void* dx, void* dw_gate, void* dw_up, void* dw_down,
                              void* ds_gate, void* ds_up, void* ds_down, float* d_topk_w, void* ws,
                              size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
