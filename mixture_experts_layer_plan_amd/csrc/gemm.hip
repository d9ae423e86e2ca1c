// Grouped expert GEMMs on MFMA (gfx950), with the layer's epilogues fused.
//
// The experts are SwiGLU feed-forward nets (up, gate, down projections) run as
// grouped GEMMs over all experts at once (sebask.de, "Mixture-of-Kittens: Cursors
// Open-Source-Ansatz für effizientes MoE-Training auf NVL72", introduction;
// stamatios.com, "Cursor abre código de megakernel MoE para GPUs NVL72",
// § Granularidade do overlap and § Outras características: SwiGLU, router-weight
// gradient fused into the SwiGLU backward).
//
// One workgroup (256 threads = 4 wavefronts in 2 x 2) computes a 128 x 128 output
// tile; each wavefront owns 64 x 64 = 2 x 2 blocks of the 32 x 32 MFMA
// (v_mfma_f32_32x32x16_bf16 for bf16, 8 x v_mfma_f32_32x32x2_f32 per 16-deep step
// for fp32).  Operands are staged through LDS as 128 rows x 128 bytes (64 bf16 or
// 32 fp32 of K per row), 16-byte chunks XOR-swizzled by row so that the MFMA
// fragment reads and the staging writes spread over the banks; two LDS buffers
// and a register prefetch overlap the next tile's global loads with the current
// tile's MFMAs.  An operand stored K-contiguous ("K-major") is copied chunk by
// chunk; one stored with K as the outer dimension ("MN-major": the wgrad operands
// and the weights of the dgrad GEMMs) is stored into LDS as it lies in memory and
// read back with the transposing LDS read ds_read_b64_tr_b16 (bf16), or loaded as
// 4 x VEC blocks and transposed in registers on its way into LDS (fp32).
//
// Grouping: a "rows-grouped" GEMM (forward GEMMs and dgrads) walks the plan's
// tile list (expert, first row) so a tile never mixes experts; a "K-grouped" GEMM
// (wgrads) is persistent: its workgroups walk (expert, output tile) items over all
// E experts and run K over that expert's rows; the items of experts without rows
// store zero tiles, interleaved with the multiplying items.  The dispatch gather of
// x happens in the A loader of GEMM1 through the plan's src_token list (X is not
// written in the forward); the backward replays the gathers of x and dy once into
// row-major buffers so that the K rows of the wgrad operands are plain strided
// addresses.  Every output
// element is produced by one workgroup with a fixed K order: results are bitwise
// reproducible and independent of the grid.
//
// Epilogues stage the fp32 accumulator tile in LDS (64 KiB, swizzled) and then
// work on rows of 8 consecutive columns with 16-byte global accesses.
#include <type_traits>

#include "gemm_common.hpp"

namespace moe {

// ------------------------------------------------ DMA-fed loop (bf16 wgrads, dgrad-down)
// The K-grouped wgrad operands and dgrad-down's operands reach LDS by the direct-to-LDS load
// (buffer_load_dwordx4 ... lds: lane L's 16 bytes land at the wavefront's LDS base +
// 16 L), so no registers stage them.  A ring of 32-deep K stages of 16 KiB (two operand
// tiles of 32 K rows x 256 bytes each, the same swizzled layout as the register-staged
// tiles): dgrad-down keeps three stages in flight while a fourth is multiplied (64 KiB,
// two workgroups per CU); the wgrad remainders, short K loops bound by their output
// writes, keep two in flight (48 KiB) so that three workgroups fit per CU.  The loads
// go through a buffer resource whose range is the expert's segment: K rows past it lie
// out of range and load as zeros, so they add exactly zero and never leave the
// operands.

namespace wdma {
constexpr int BK = 32;          // K rows per stage
constexpr int OPB = BK * 256;   // bytes of one operand tile in a stage
constexpr int STB = 2 * OPB;    // stage bytes
static_assert(4 * STB == LDS_BYTES, "the ring fills the LDS of the staged C tile");


// MN-major operand: K row k = row seg0 + k of a row-major bf16 matrix, columns
// c0 .. c0 + 127.  Instruction q (0, 1) of wavefront w fills K rows 8 w + 4 q ..
// + 3 of a stage: lane L brings K row r = 8 w + 4 q + L / 16 into physical chunk
// L % 16, i.e. its logical chunk (L % 16) ^ mn_swz(r).
struct Opnd {
  rsrc_t rs;         // element (seg0, c0); range: the segment's rows
  uint32_t ldb;      // row stride, bytes
  int r[2];
  uint32_t col[2];
  MOE_DEV void set(const bf16_t* b, size_t ld, int rows) {
    ldb = (uint32_t)(ld * 2);
    rs = make_rsrc(b, (uint32_t)rows * ldb);
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      r[q] = 8 * w + 4 * q + (L >> 4);
      col[q] = (uint32_t)(((L & 15) ^ mn_swz(r[q])) << 4);
    }
  }
  MOE_DEV void issue(int kt, char* tile) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < 2; ++q)  // K rows past the segment lie past the range: zeros
      dma16_buf(rs, (uint32_t)(kt * BK + r[q]) * ldb + col[q], 0u,
                tile + (8 * w + 4 * q) * 256);
  }
};

// K-major operand (dgrad-down's rows of dYu, K = H along each row): 128 rows x 32 K
// per stage, 64-byte rows, chunk c (K values 8 c .. 8 c + 7) of row r at r * 64 +
// 16 (c ^ ((r >> 2) & 3)), so that the 16 lanes of a fragment read that share a chunk
// index hit 16 different 16-byte bank groups.  Instruction q of wavefront w fills rows
// 16 (2 w + q) .. + 15: lane L brings row 16 (2 w + q) + L / 4, physical chunk L % 4.
MOE_DEV int km_chunk(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }
struct KOpnd {
  rsrc_t rs;  // row 0 of the tile; range: its valid rows (rows past them load zeros)
  uint32_t off[2];
  MOE_DEV void set(const bf16_t* rows, size_t ld, int nrows) {
    const uint32_t ldb = (uint32_t)(ld * 2);
    rs = make_rsrc(rows, (uint32_t)nrows * ldb);
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = 16 * (2 * w + q) + (L >> 2);
      off[q] = (uint32_t)r * ldb + (uint32_t)(((L & 3) ^ ((r >> 2) & 3)) << 4);
    }
  }
  MOE_DEV void issue(int kt, char* tile) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      dma16_buf(rs, off[q], (uint32_t)(kt * BK * 2), tile + (2 * w + q) * 1024);
  }
};

// The MFMAs of one 32-deep stage (two 16-deep steps) on two MN-major tiles.  The
// transposing LDS reads are issued from inline assembly: for the
// ds_read_b64_tr_b16 builtin the compiler waits for every outstanding
// direct-to-LDS load first (vmcnt(0)), which would drain the ring on every stage.
// Each step's eight reads and their lgkmcnt(0) wait form one asm block, so no
// fragment register is used before its data is in.
MOE_DEV uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
MOE_DEV uint32_t mn_frag_addr(const char* t, int c0, int ks, int lane) {
  const int g = lane >> 4, a = lane & 3, j = (lane >> 2) & 3;
  const int k = 16 * ks + 8 * (g >> 1) + j;  // K row k + 4 has the same swizzle
  const int col = c0 + 16 * (g & 1) + 4 * a;
  return lds_addr(t + k * 256 + (((col >> 3) ^ mn_swz(k)) << 4) + (col & 7) * 2);
}
MOE_DEV bf16x8_t join_tr(const s16x4_t& lo, const s16x4_t& hi) {
  return __builtin_bit_cast(bf16x8_t, (s16x8_t)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5,
                                                                        6, 7));
}
// A K-major (KOpnd): its two fragments are plain 16-byte reads.
MOE_DEV void mma_stage_km(const char* ta, const char* tb, f32x16_t (&acc)[2][2], int arow,
                          const int (&brow)[2], int lane) {
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int ch = 2 * ks + (lane >> 5);
    const uint32_t pa0 = lds_addr(ta + km_chunk(arow + (lane & 31), ch));
    const uint32_t pa1 = lds_addr(ta + km_chunk(arow + 32 + (lane & 31), ch));
    const uint32_t pb0 = mn_frag_addr(tb, brow[0], ks, lane);
    const uint32_t pb1 = mn_frag_addr(tb, brow[1], ks, lane);
    s16x8_t a0, a1;
    s16x4_t b0l, b0h, b1l, b1h;
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b64_tr_b16 %2, %8\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:1024\n\t"
        "ds_read_b64_tr_b16 %4, %9\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(b0l), "=&v"(b0h), "=&v"(b1l), "=&v"(b1h)
        : "v"(pa0), "v"(pa1), "v"(pb0), "v"(pb1)
        : "memory");
    const bf16x8_t fa0 = __builtin_bit_cast(bf16x8_t, a0), fa1 = __builtin_bit_cast(bf16x8_t, a1);
    const bf16x8_t b0 = join_tr(b0l, b0h), b1 = join_tr(b1l, b1h);
    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, b0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, b1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, b0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, b1, acc[1][1], 0, 0, 0);
  }
}

MOE_DEV void mma_stage(const char* ta, const char* tb, f32x16_t (&acc)[2][2], int arow,
                       const int (&brow)[2], int lane) {
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const uint32_t pa0 = mn_frag_addr(ta, arow, ks, lane), pa1 = mn_frag_addr(ta, arow + 32, ks, lane);
    const uint32_t pb0 = mn_frag_addr(tb, brow[0], ks, lane);
    const uint32_t pb1 = mn_frag_addr(tb, brow[1], ks, lane);
    s16x4_t a0l, a0h, a1l, a1h, b0l, b0h, b1l, b1h;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:1024\n\t"
        "ds_read_b64_tr_b16 %2, %9\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:1024\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:1024\n\t"
        "ds_read_b64_tr_b16 %6, %11\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0l), "=&v"(a0h), "=&v"(a1l), "=&v"(a1h), "=&v"(b0l), "=&v"(b0h), "=&v"(b1l),
          "=&v"(b1h)
        : "v"(pa0), "v"(pa1), "v"(pb0), "v"(pb1)
        : "memory");
    const bf16x8_t a0 = join_tr(a0l, a0h), a1 = join_tr(a1l, a1h);
    const bf16x8_t b0 = join_tr(b0l, b0h), b1 = join_tr(b1l, b1h);
    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
  }
}

// Wait until at most `ahead` stages of this wavefront's loads (4 instructions each)
// are outstanding and its LDS reads are done, then meet the workgroup.
MOE_DEV void ring_wait(int ahead) {
  if (ahead >= 2) __builtin_amdgcn_s_waitcnt(0x0078);       // vmcnt(8) lgkmcnt(0)
  else if (ahead == 1) __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) lgkmcnt(0)
  else __builtin_amdgcn_s_waitcnt(0x0070);                  // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// OA: Opnd (MN-major A, the wgrads) or KOpnd (K-major A, dgrad-down); n: K.  NS: ring
// stages (NS - 1 in flight): 4 (64 KiB) for dgrad-down, 3 (48 KiB) for the wgrad
// remainders, which run three workgroups per CU.
template <int NS = 4, class OA>
MOE_DEV void main_loop(char* lds, const OA& A, const Opnd& B, int n, f32x16_t (&acc)[2][2],
                       int arow, const int (&brow)[2], int lane) {
  static_assert(NS == 3 || NS == 4, "ring depth");
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  const int nk = (n + BK - 1) / BK;
  for (int s = 0; s < NS - 1 && s < nk; ++s) {
    A.issue(s, lds + s * STB);
    B.issue(s, lds + s * STB + OPB);
  }
  int slot = 0;  // kt % NS
  for (int kt = 0; kt < nk; ++kt) {
    ring_wait(min(NS - 2, nk - 1 - kt));  // stage kt is in; stage kt - 1 is no longer read
    if (kt + NS - 1 < nk) {  // into the slot of stage kt - 1
      char* st = lds + (slot == 0 ? NS - 1 : slot - 1) * STB;
      A.issue(kt + NS - 1, st);
      B.issue(kt + NS - 1, st + OPB);
    }
    const char* cur = lds + slot * STB;
    slot = slot == NS - 1 ? 0 : slot + 1;
    if constexpr (std::is_same<OA, KOpnd>::value) mma_stage_km(cur, cur + OPB, acc, arow, brow, lane);
    else mma_stage(cur, cur + OPB, acc, arow, brow, lane);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);
  __builtin_amdgcn_s_barrier();  // every wavefront is done with the ring
}
}  // namespace wdma

// ------------------------------------------------------------------ kernels
// GEMM1 + SwiGLU.  Tile n covers i in [64 n, 64 n + 64): B-tile rows 0..63 are
// W_g[e] rows, 64..127 the W_u[e] rows of the same i.  The pre-activations A and B
// are kept in fp32 (Z) for the backward; h = silu(A) * B is formed from them in
// fp32 and rounded once to T.
template <typename T>
__global__ __launch_bounds__(NTHR, 2) void k_up_swiglu(GroupInfo g, const T* __restrict__ x,
                                                       const T* __restrict__ wg,
                                                       const T* __restrict__ wu, int H, int I,
                                                       float* __restrict__ Z, T* __restrict__ hout) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  RowTile t;
  int nt;
  if (!rows_tile(g, I / 64, t, nt)) return;
  const int i0 = nt * 64;
  const size_t wofs = (size_t)t.e * I * H;
  KLoad<T> la, lb;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int rr = (threadIdx.x >> 3) + 32 * s;
    const int r = t.row0 + rr;
    const bool ok = r < t.row_end;
    la.set(s, ok ? x + (size_t)token_of(g, r) * H : nullptr, ok);
    lb.set(s, rr < 64 ? wg + wofs + (size_t)(i0 + rr) * H : wu + wofs + (size_t)(i0 + rr - 64) * H,
           true);
  }
  int arow, brow[2];
  wave_coords(arow, brow, true);
  const int lane = threadIdx.x & 63;
  f32x16_t acc[2][2];
  gemm_main<T>(lds, la, lb, H / Tr<T>::BK, acc, arow, brow, lane);
  float* C = (float*)lds;
  stage_acc(C, acc, arow, brow, lane);
  __syncthreads();
  const int nrows = t.row_end - t.row0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int r = (threadIdx.x >> 3) + 32 * s, c = threadIdx.x & 7;
    if (r < nrows) {
      float a[8], b[8], h[8];
      read8(C, r, 8 * c, a);
      read8(C, r, 64 + 8 * c, b);
#pragma unroll
      for (int q = 0; q < 8; ++q) h[q] = silu_f(a[q]) * b[q];
      float* zr = Z + (size_t)(t.row0 + r) * (2 * I);
      store8(zr + i0 + 8 * c, a);
      store8(zr + I + i0 + 8 * c, b);
      store8(hout + (size_t)(t.row0 + r) * I + i0 + 8 * c, h);
    }
  }
}

// GEMM2: Y[r, n] = sum_i h[r, i] W_d[e][n, i]
template <typename T>
__global__ __launch_bounds__(NTHR, 2) void k_down(GroupInfo g, const T* __restrict__ h,
                                                  const T* __restrict__ wd, int H, int I,
                                                  T* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  RowTile t;
  int nt;
  if (!rows_tile(g, H / TN, t, nt)) return;
  const int n0 = nt * TN;
  const size_t wofs = (size_t)t.e * H * I;
  KLoad<T> la, lb;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int rr = (threadIdx.x >> 3) + 32 * s;
    const int r = t.row0 + rr;
    la.set(s, h + (size_t)r * I, r < t.row_end);
    lb.set(s, wd + wofs + (size_t)(n0 + rr) * I, true);
  }
  int arow, brow[2];
  wave_coords(arow, brow, false);
  const int lane = threadIdx.x & 63;
  f32x16_t acc[2][2];
  gemm_main<T>(lds, la, lb, I / Tr<T>::BK, acc, arow, brow, lane);
  float* C = (float*)lds;
  stage_acc(C, acc, arow, brow, lane);
  __syncthreads();
  auto out = [&](int r) { return Y + (size_t)(t.row0 + r) * H + n0; };
  epi_store<T>(C, out, t.row_end - t.row0);
}

// dgrad-down: dh'[r, i] = sum_n dYu[r, n] W_d[e][n, i] with dYu[r] = dy[tok(r)] (the
// reverse-combined rows); epilogue: SwiGLU backward and the router-weight-gradient
// partial of this tile's 128 columns.  bf16 runs K through the direct-to-LDS ring
// (dYu rows K-major, W_d MN-major; three 32-deep stages in flight); fp32 through the
// register-staged loop.
template <typename T>
__global__ __launch_bounds__(NTHR, 2) void k_dgrad_down(GroupInfo g, const T* __restrict__ dYu,
                                                        const T* __restrict__ wd,
                                                        const float* __restrict__ Z,
                                                        const float* __restrict__ topk_w, int H,
                                                        int I, int k, T* __restrict__ dZ,
                                                        T* __restrict__ gh,
                                                        float* __restrict__ dgp) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  RowTile t;
  int nt;
  if (!rows_tile(g, I / TN, t, nt)) return;
  const int i0 = nt * TN;
  int arow, brow[2];
  wave_coords(arow, brow, false);
  const int lane = threadIdx.x & 63;
  f32x16_t acc[2][2];
  if constexpr (sizeof(T) == 2) {  // the direct-to-LDS ring
    wdma::KOpnd la;
    la.set(dYu + (size_t)t.row0 * H, (size_t)H, t.row_end - t.row0);
    wdma::Opnd lb;
    lb.set(wd + (size_t)t.e * H * I + i0, (size_t)I, H);
    wdma::main_loop(lds, la, lb, H, acc, arow, brow, lane);
  } else {
    KLoad<T> la;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = t.row0 + (threadIdx.x >> 3) + 32 * s;
      la.set(s, dYu + (size_t)r * H, r < t.row_end);
    }
    MNLoad<T, KRowPlain<T>> lb{{wd + (size_t)t.e * H * I + i0, (size_t)I}};
    gemm_main<T>(lds, la, lb, H / Tr<T>::BK, acc, arow, brow, lane);
  }
  float* C = (float*)lds;
  stage_acc(C, acc, arow, brow, lane);
  __syncthreads();
  const int nrows = t.row_end - t.row0;
  const int n_parts = I / TN;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int r = (threadIdx.x >> 4) + 16 * s, c = threadIdx.x & 15;
    const bool ok = r < nrows;
    float part = 0.0f;
    if (ok) {
      const int row = t.row0 + r;
      const float gate = g.src_token ? topk_w[(size_t)g.src_token[row] * k + g.src_slot[row]] : 1.0f;
      float d[8], a[8], b[8], da[8], db[8], gh8[8];
      read8(C, r, 8 * c, d);
      const float* zr = Z + (size_t)row * (2 * I);
      load8(zr + i0 + 8 * c, a);
      load8(zr + I + i0 + 8 * c, b);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float sg = 1.0f / (1.0f + expf(-a[q]));
        const float sl = a[q] * sg;
        const float hv = sl * b[q];
        part = fmaf(d[q], hv, part);
        const float dh = gate * d[q];
        da[q] = dh * b[q] * (sg * (1.0f + a[q] * (1.0f - sg)));
        db[q] = dh * sl;
        gh8[q] = gate * hv;
      }
      T* dzr = dZ + (size_t)row * (2 * I);
      store8(dzr + i0 + 8 * c, da);
      store8(dzr + I + i0 + 8 * c, db);
      store8(gh + (size_t)row * I + i0 + 8 * c, gh8);
    }
    // fixed-order sum over the 16 lanes holding this row's 128 columns
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
    if (ok && c == 0 && dgp) dgp[(size_t)(t.row0 + r) * n_parts + nt] = part;
  }
}

// dgrad-up: dX[r, n] = sum_{k < 2I} dZ[r, k] Wcat[k, n]
template <typename T>
__global__ __launch_bounds__(NTHR, 2) void k_dgrad_up(GroupInfo g, const T* __restrict__ dZ,
                                                      const T* __restrict__ wg,
                                                      const T* __restrict__ wu, int H, int I,
                                                      T* __restrict__ dX) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  RowTile t;
  int nt;
  if (!rows_tile(g, H / TN, t, nt)) return;
  const int n0 = nt * TN;
  const size_t wofs = (size_t)t.e * I * H + n0;
  KLoad<T> la;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int r = t.row0 + (threadIdx.x >> 3) + 32 * s;
    la.set(s, dZ + (size_t)r * (2 * I), r < t.row_end);
  }
  MNLoad<T, KRowCat<T>> lb{{wg + wofs, wu + wofs, I, H}};
  int arow, brow[2];
  wave_coords(arow, brow, false);
  const int lane = threadIdx.x & 63;
  f32x16_t acc[2][2];
  gemm_main<T>(lds, la, lb, (2 * I) / Tr<T>::BK, acc, arow, brow, lane);
  float* C = (float*)lds;
  stage_acc(C, acc, arow, brow, lane);
  __syncthreads();
  auto out = [&](int r) { return dX + (size_t)(t.row0 + r) * H + n0; };
  epi_store<T>(C, out, t.row_end - t.row0);
}


// stage_acc inside the persistent item loops: the wave's row and column bases are
// made opaque per item, so that the 64 staging offsets are computed in each item and
// not once before the loop and held across it (64 registers)
MOE_DEV void stage_acc_item(float* C, const f32x16_t (&acc)[2][2], int arow,
                            const int (&brow)[2], int lane) {
  int r = arow, b[2] = {brow[0], brow[1]};
  asm volatile("" : "+v"(r), "+v"(b[0]), "+v"(b[1]));
  stage_acc(C, acc, r, b, lane);
}

// The wgrad remainders' epilogue through 32 KiB: the C tile in two halves of 64 rows
// (the wavefronts of row half hf stage theirs at C rows 0..63, then all threads store
// those rows), so that the LDS is the 48 KiB ring.
template <typename T, class RowPtr>
MOE_DEV void epi_halves(float* C, const f32x16_t (&acc)[2][2], int arow, const int (&brow)[2],
                        int lane, const RowPtr& out_row) {
#pragma unroll 1
  for (int hf = 0; hf < 2; ++hf) {
    if (arow == 64 * hf) stage_acc_item(C, acc, 0, brow, lane);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = (threadIdx.x >> 4) + 16 * s, c = threadIdx.x & 15;
      float f[8];
      read8(C, r, 8 * c, f);
      store8_nt(out_row(64 * hf + r) + 8 * c, f);
    }
    __syncthreads();
  }
}

// wgrad-down: dW_d[e][m, n] = sum_r dYu[r, m] gh[r, n]  (M = H, N = I, K = rows of e).
// Persistent: each workgroup walks work items blockIdx.x, + gridDim.x, ...; the
// tiles of experts without rows are stored as zeros.
template <typename T>
__global__ __launch_bounds__(NTHR, sizeof(T) == 2 ? 3 : 2) void k_wgrad_down(GroupInfo g, const T* __restrict__ dYu,
                                                        const T* __restrict__ gh, int H, int I,
                                                        T* __restrict__ dwd) {
  __shared__ __attribute__((aligned(16))) char lds[sizeof(T) == 2 ? 3 * wdma::STB : LDS_BYTES];
  const int MT = H / TM, NT = I / TN;
  const int total = k_work_items(g, MT, NT);
  int arow, brow[2];
  wave_coords(arow, brow, false);
  const int lane = threadIdx.x & 63;
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const KTile t = k_tile(g, w, MT, NT, true);
    const int kind = k_item_kind(g, t.e);
    if (kind == 2) {
      w = k_skip_expert(w, t.e, MT * NT);
      continue;
    }
    if (kind == 1) {
      zero_span<T>(dwd + (size_t)t.e * H * I + ((size_t)(t.m0 / TM) * NT + t.n0 / TN) * (TM * TN));
      continue;
    }
    int seg0, seg1;
    k_segment(g, t.e, seg0, seg1);
    f32x16_t acc[2][2];
    if constexpr (sizeof(T) == 2) {
      wdma::Opnd la, lb;
      la.set(dYu + (size_t)seg0 * H + t.m0, (size_t)H, seg1 - seg0);
      lb.set(gh + (size_t)seg0 * I + t.n0, (size_t)I, seg1 - seg0);
      wdma::main_loop<3>(lds, la, lb, seg1 - seg0, acc, arow, brow, lane);
    } else {
      MNSeg<T> la, lb;
      la.set(dYu + (size_t)seg0 * H + t.m0, (size_t)H, seg1 - seg0);
      lb.set(gh + (size_t)seg0 * I + t.n0, (size_t)I, seg1 - seg0);
      const int nk = (seg1 - seg0 + Tr<T>::BK - 1) / Tr<T>::BK;
      gemm_main<T, 1>(lds, la, lb, nk, acc, arow, brow, lane);
    }
    float* C = (float*)lds;
    T* base = dwd + (size_t)t.e * H * I + (size_t)t.m0 * I + t.n0;
    auto out = [&](int r) { return base + (size_t)r * I; };
    if constexpr (sizeof(T) == 2) {
      epi_halves<T>(C, acc, arow, brow, lane, out);
    } else {
      stage_acc_item(C, acc, arow, brow, lane);
      __syncthreads();
      epi_store<T, true>(C, out, TM);
      __syncthreads();
    }
  }
}

// wgrad-up: [dW_g; dW_u][e][m, n] = sum_r dZ[r, m] X[r, n] with X[r] = x[tok(r)] (the
// dispatched rows, replayed)  (M = 2I, N = H); persistent, zeros for experts
// without rows.
template <typename T>
__global__ __launch_bounds__(NTHR, sizeof(T) == 2 ? 3 : 2) void k_wgrad_up(GroupInfo g, const T* __restrict__ dZ,
                                                      const T* __restrict__ X, int H, int I,
                                                      T* __restrict__ dwg, T* __restrict__ dwu) {
  __shared__ __attribute__((aligned(16))) char lds[sizeof(T) == 2 ? 3 * wdma::STB : LDS_BYTES];
  const int MT = (2 * I) / TM, NT = H / TN;
  const int total = k_work_items(g, MT, NT);
  int arow, brow[2];
  wave_coords(arow, brow, false);
  const int lane = threadIdx.x & 63;
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const KTile t = k_tile(g, w, MT, NT, false);
    const int kind = k_item_kind(g, t.e);
    if (kind == 2) {
      w = k_skip_expert(w, t.e, MT * NT);
      continue;
    }
    if (kind == 1) {
      const int mg = t.m0 < I ? t.m0 : t.m0 - I;  // row tile within dW_g or dW_u
      zero_span<T>((t.m0 < I ? dwg : dwu) + (size_t)t.e * I * H +
                   ((size_t)(mg / TM) * NT + t.n0 / TN) * (TM * TN));
      continue;
    }
    int seg0, seg1;
    k_segment(g, t.e, seg0, seg1);
    f32x16_t acc[2][2];
    if constexpr (sizeof(T) == 2) {
      wdma::Opnd la, lb;
      la.set(dZ + (size_t)seg0 * (2 * I) + t.m0, (size_t)(2 * I), seg1 - seg0);
      lb.set(X + (size_t)seg0 * H + t.n0, (size_t)H, seg1 - seg0);
      wdma::main_loop<3>(lds, la, lb, seg1 - seg0, acc, arow, brow, lane);
    } else {
      MNSeg<T> la, lb;
      la.set(dZ + (size_t)seg0 * (2 * I) + t.m0, (size_t)(2 * I), seg1 - seg0);
      lb.set(X + (size_t)seg0 * H + t.n0, (size_t)H, seg1 - seg0);
      const int nk = (seg1 - seg0 + Tr<T>::BK - 1) / Tr<T>::BK;
      gemm_main<T, 1>(lds, la, lb, nk, acc, arow, brow, lane);
    }
    float* C = (float*)lds;
    T* base = (t.m0 < I ? dwg + (size_t)t.e * I * H + (size_t)t.m0 * H
                        : dwu + (size_t)t.e * I * H + (size_t)(t.m0 - I) * H) + t.n0;
    auto out = [&](int r) { return base + (size_t)r * H; };
    if constexpr (sizeof(T) == 2) {
      epi_halves<T>(C, acc, arow, brow, lane, out);
    } else {
      stage_acc_item(C, acc, arow, brow, lane);
      __syncthreads();
      epi_store<T, true>(C, out, TM);
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ launchers
static unsigned row_tiles(const GroupInfo& g) {
  return g.tiles ? (unsigned)g.max_tiles : (unsigned)((g.dense_rows + TM - 1) / TM);
}

template <typename T>
static hipError_t up_swiglu_t(const GroupInfo& g, const void* x, const void* wg, const void* wu,
                              int H, int I, void* Z, void* h, hipStream_t s) {
  const unsigned ty = row_tiles(g);
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH(g.tiles ? "gemm_up_swiglu" : "gemm_up_swiglu_shared", s,
                    k_up_swiglu<T><<<ty * (I / 64), NTHR, 0, s>>>(
                        g, (const T*)x, (const T*)wg, (const T*)wu, H, I, (float*)Z, (T*)h));
}

template <typename T>
static hipError_t down_t(const GroupInfo& g, const void* h, const void* wd, int H, int I, void* Y,
                         hipStream_t s) {
  const unsigned ty = row_tiles(g);
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH(g.tiles ? "gemm_down" : "gemm_down_shared", s,
                    k_down<T><<<ty * (H / TN), NTHR, 0, s>>>(g, (const T*)h, (const T*)wd, H,
                                                                 I, (T*)Y));
}

template <typename T>
static hipError_t dgrad_down_t(const GroupInfo& g, const void* dy, const void* wd, const void* Z,
                               const float* topk_w, int H, int I, int k, void* dZ, void* gh,
                               float* dgp, hipStream_t s) {
  const unsigned ty = row_tiles(g);
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH(g.tiles ? "gemm_dgrad_down" : "gemm_dgrad_down_shared", s,
                    k_dgrad_down<T><<<ty * (I / TN), NTHR, 0, s>>>(
                        g, (const T*)dy, (const T*)wd, (const float*)Z, topk_w, H, I, k, (T*)dZ,
                        (T*)gh, dgp));
}

template <typename T>
static hipError_t dgrad_up_t(const GroupInfo& g, const void* dZ, const void* wg, const void* wu,
                             int H, int I, void* dX, hipStream_t s) {
  const unsigned ty = row_tiles(g);
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH(g.tiles ? "gemm_dgrad_up" : "gemm_dgrad_up_shared", s,
                    k_dgrad_up<T><<<ty * (H / TN), NTHR, 0, s>>>(
                        g, (const T*)dZ, (const T*)wg, (const T*)wu, H, I, (T*)dX));
}

template <typename T>
static hipError_t wgrad_down_t(const GroupInfo& g, const void* dy, const void* gh, int H, int I,
                               void* dwd, hipStream_t s) {
  const unsigned grid = persistent_grid((long)g.E * (H / TM) * (I / TN), sizeof(T) == 2 ? 3 : 2);
  return MOE_LAUNCH(g.offsets ? "gemm_wgrad_down" : "gemm_wgrad_down_shared", s,
                    k_wgrad_down<T><<<grid, NTHR, 0, s>>>(g, (const T*)dy, (const T*)gh, H, I,
                                                          (T*)dwd));
}

template <typename T>
static hipError_t wgrad_up_t(const GroupInfo& g, const void* dZ, const void* x, int H, int I,
                             void* dwg, void* dwu, hipStream_t s) {
  const unsigned grid = persistent_grid((long)g.E * ((2 * I) / TM) * (H / TN), sizeof(T) == 2 ? 3 : 2);
  return MOE_LAUNCH(g.offsets ? "gemm_wgrad_up" : "gemm_wgrad_up_shared", s,
                    k_wgrad_up<T><<<grid, NTHR, 0, s>>>(g, (const T*)dZ, (const T*)x, H, I,
                                                        (T*)dwg, (T*)dwu));
}

hipError_t launch_gemm_up_swiglu(int dt, const GroupInfo& g, const void* x, const void* wg,
                                 const void* wu, int H, int I, void* Z, void* h, hipStream_t s) {
  return dt ? launch_big_up_swiglu(g, x, wg, wu, H, I, Z, h, s)
            : up_swiglu_t<float>(g, x, wg, wu, H, I, Z, h, s);
}
hipError_t launch_gemm_down(int dt, const GroupInfo& g, const void* h, const void* wd, int H,
                            int I, void* Y, hipStream_t s) {
  if (dt) return launch_big_down(g, h, wd, H, I, Y, s);
  return dt ? down_t<bf16_t>(g, h, wd, H, I, Y, s) : down_t<float>(g, h, wd, H, I, Y, s);
}
hipError_t launch_gemm_dgrad_down(int dt, const GroupInfo& g, const void* dy, const void* wd,
                                  const void* Z, const float* topk_w, int H, int I, int k,
                                  void* dZ, void* gh, float* dgp, hipStream_t s) {
  return dt ? dgrad_down_t<bf16_t>(g, dy, wd, Z, topk_w, H, I, k, dZ, gh, dgp, s)
            : dgrad_down_t<float>(g, dy, wd, Z, topk_w, H, I, k, dZ, gh, dgp, s);
}
hipError_t launch_gemm_dgrad_up(int dt, const GroupInfo& g, const void* dZ, const void* wg,
                                const void* wu, int H, int I, void* dX, hipStream_t s) {
  return dt ? launch_big_dgrad_up(g, dZ, wg, wu, H, I, dX, s)
            : dgrad_up_t<float>(g, dZ, wg, wu, H, I, dX, s);
}
// Grouped bf16 wgrads: the experts with at least WGRAD_HOT_ROWS rows run on the
// 256 x 256 core; the 128 x 128 kernel takes the experts with fewer rows (short K,
// bound by their output writes) and stores the zero gradients of the experts
// without rows.  A dense operand pair (the shared expert) with at least that many
// rows runs on the 256 x 256 core alone.
constexpr int WGRAD_HOT_ROWS = 256;

hipError_t launch_gemm_wgrad_down(int dt, const GroupInfo& g, const void* dy, const void* gh,
                                  int H, int I, void* dwd, hipStream_t s) {
  if (!dt) return wgrad_down_t<float>(g, dy, gh, H, I, dwd, s);
  if (!g.offsets && g.dense_rows < WGRAD_HOT_ROWS)  // a short dense operand
    return wgrad_down_t<bf16_t>(g, dy, gh, H, I, dwd, s);
  const hipError_t e = launch_big_wgrad_down_hot(g, dy, gh, H, I, dwd, WGRAD_HOT_ROWS, s);
  if (e == hipErrorNotSupported) return wgrad_down_t<bf16_t>(g, dy, gh, H, I, dwd, s);
  if (e != hipSuccess || !g.offsets) return e;
  GroupInfo rest = g;
  rest.hot_rows = WGRAD_HOT_ROWS;
  return wgrad_down_t<bf16_t>(rest, dy, gh, H, I, dwd, s);
}
hipError_t launch_gemm_wgrad_up(int dt, const GroupInfo& g, const void* dZ, const void* x,
                                int H, int I, void* dwg, void* dwu, hipStream_t s) {
  if (!dt) return wgrad_up_t<float>(g, dZ, x, H, I, dwg, dwu, s);
  if (!g.offsets && g.dense_rows < WGRAD_HOT_ROWS)  // a short dense operand
    return wgrad_up_t<bf16_t>(g, dZ, x, H, I, dwg, dwu, s);
  const hipError_t e = launch_big_wgrad_up_hot(g, dZ, x, H, I, dwg, dwu, WGRAD_HOT_ROWS, s);
  if (e == hipErrorNotSupported) return wgrad_up_t<bf16_t>(g, dZ, x, H, I, dwg, dwu, s);
  if (e != hipSuccess || !g.offsets) return e;
  GroupInfo rest = g;
  rest.hot_rows = WGRAD_HOT_ROWS;
  return wgrad_up_t<bf16_t>(rest, dZ, x, H, I, dwg, dwu, s);
}

}  // namespace moe
