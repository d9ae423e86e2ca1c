// Large-tile grouped GEMMs for gfx950 (MI355X): bf16 GEMM1 + SwiGLU, GEMM2 and
// dgrad-up with their epilogues fused, MXFP8 GEMM2 and dgrad-up, and the weight
// gradients (bf16 and MXFP8) of the experts with many rows.
//
// The experts are SwiGLU feed-forward nets run as grouped GEMMs over all experts
// at once (sebask.de, "Mixture-of-Kittens: Cursors Open-Source-Ansatz für
// effizientes MoE-Training auf NVL72", introduction; stamatios.com, "Cursor abre
// código de megakernel MoE para GPUs NVL72", § Outras características).
//
// Core (chosen from measurements on MI355X): one workgroup of eight wavefronts
// (two per SIMD) computes a 256 x 256 output tile; wavefront (wm, wn) owns rows
// 128 wm .. +127 and columns 64 wn .. +63 as 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16.  Both operands travel global -> LDS by the gfx950
// direct-to-LDS load (buffer_load_dwordx4 ... lds through a buffer resource: each
// lane's 16 bytes land at the wavefront's LDS base + 16 * lane; the scale bytes and
// zero-row tails keep the global_load_lds form), so no registers stage them; two LDS stages of
// 64 KiB each: the next K tile (64 deep) streams in while the current one is
// multiplied.  MFMA fragments are read one 16-deep step ahead, and the tile
// barrier sits before the last step's MFMAs so that the next tile's first
// fragments load underneath them.  Against a 128 x 128 tile with register-staged
// loads this halves LDS traffic per flop (32 flops per LDS byte) and frees the
// registers that made the loop wait on every fragment read.  (dgrad-down, and the
// wgrads of experts with few rows and of experts without rows, stay on the 128 x 128
// kernels of gemm.hip: short-K, write-heavy items overlap better two workgroups per
// CU, and dgrad-down's 256-wide column tiles are too few.)
//
// Operand layouts in LDS (one stage = 32 KiB per operand):
//  * K-major (rows of K-contiguous data: tokens, and the weights of the forward
//    GEMMs): 256 rows x 128 bytes, 16-byte chunks XOR-swizzled by row; fragments
//    by 16-byte reads.
//  * MN-major (K is the outer dimension: the weights of dgrad-up, both bf16 wgrad
//    operands): 64 K rows x 512 bytes as stored in memory, 16-byte chunks
//    XOR-swizzled by K row; fragments by the gfx950 transposing LDS read
//    ds_read_b64_tr_b16 (within each 16-lane group, lane 4a + b receives element b
//    of the 8-byte rows addressed by lanes a, a + 4, a + 8, a + 12), two reads per
//    fragment.  No register transpose, no bank conflicts.
//  * MXFP8 operands (wgrads, and the row-grouped GEMM2 and dgrad-up): K-major,
//    128-byte K pieces (128 E4M3 values) in the K-major layout above.
//
// Grouping: the kernels walk the plan's 256-row tile list (expert, first row); a
// wavefront skips the MFMAs of 32-row blocks that lie past the expert's rows and
// the token loads skip whole 64-row groups past them, so a tile of a small expert
// costs what its rows need and is bound by its weight reads.  Such a tile (at most
// 64 or 128 rows) runs K through a deeper ring whose stages hold only the A rows
// that exist, so more of its weight panel is in flight.  Every output element
// is produced by one workgroup with a fixed K order: bitwise reproducible and
// independent of the grid.
#include "gemm_common.hpp"
#include "move_common.hpp"

namespace moe {
namespace big {

constexpr int TILE = 256;
static_assert(TILE == 256, "fused_counters counts 256-row tiles");
constexpr int NTH = 512;
constexpr int STAGE = 32768;     // one operand, one 64-deep K tile
constexpr int LDS = 4 * STAGE;   // two stages of (A, B)
constexpr int LDS_ROWS = 163840; // the row-grouped kernels: also the small-tile ring

typedef __attribute__((address_space(3))) void* lds_vptr;
typedef const __attribute__((address_space(1))) void* gbl_vptr;

// AUX: cache policy of the load (0; or 16 = sc1, coherent at device scope: reads
// data that another XCD wrote through, not a stale line of this XCD's L2)
template <int AUX = 0>
MOE_DEV void dma16(const char* src, char* dst) {
  __builtin_amdgcn_global_load_lds((gbl_vptr)src, (lds_vptr)dst, 16, 0, AUX);
}
constexpr int CPOL_DEVICE = 16;

// The operand loaders below use the buffer-resource form of this load (dma16_buf,
// gemm_common.hpp); dma16 is left for the scale bytes and the zero-row tails.
template <int AUX = 0>
MOE_DEV void dmab(rsrc_t r, uint32_t voff, uint32_t soff, char* dst) {
  dma16_buf<AUX>(r, voff, soff, dst);
}
// the wavefront's index as a scalar (wave-uniform by construction)
MOE_DEV int wave_s() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

MOE_DEV int wave() { return threadIdx.x >> 6; }
MOE_DEV int lane() { return threadIdx.x & 63; }

// Addresses are a wave-uniform base plus a 32-bit per-lane offset (and uniform
// strides), so the loads use the scalar-base addressing form and few registers.

// ------------------------------------------------------------ K-major operand
// Instruction s (0..3) of wavefront w fills stage rows 64 s + 8 w .. +7: lane L
// brings row kmaj_row(s) = 64 s + 8 w + L / 8 into physical chunk L % 8, i.e. its
// logical chunk (L % 8) ^ swizzle(row) (the swizzle of gemm_common.hpp; it depends
// on row % 64 only, so it is the same for the four instructions).
MOE_DEV int kmaj_row(int s) { return 64 * s + 8 * wave() + (lane() >> 3); }
MOE_DEV int kmaj_chunk() {
  const int r = kmaj_row(0);
  return (threadIdx.x & 7) ^ ((r ^ (r >> 3)) & 7);
}
MOE_DEV char* kmaj_dst(char* st, int s) { return st + (8 * s + wave()) * 1024; }

// Rows gathered one by one (tokens through the plan's pull list).  Instructions
// whose 64 rows all lie past the tile's `rows` are not issued: those LDS rows keep
// stale data and feed only output rows that are neither multiplied (blocks_a) nor
// stored.
template <int AUX = 0>
struct DmaKGT {
  rsrc_t r;         // the gathered matrix
  uint32_t off[4];  // byte offset of this lane's row for instruction s, chunk included
  int n;            // instructions issued
  MOE_DEV void set(const bf16_t* b, int rows) {
    r = make_rsrc(b);
    n = (rows + 63) / 64;
  }
  MOE_DEV void row(int s, size_t row_elem_offset) {
    off[s] = (uint32_t)(row_elem_offset * 2) + 16u * kmaj_chunk();
  }
  template <int S0 = 0, int S1 = 4>
  MOE_DEV void issue(int kt, char* st) const {
#pragma unroll
    for (int s = S0; s < S1; ++s)
      if (s < n) dmab<AUX>(r, off[s], (uint32_t)kt * 128u, kmaj_dst(st, s));
  }
};
using DmaKG = DmaKGT<0>;

// Rows at a fixed stride (weights): row r at base + r * ld; rows past `rows` read
// row 0 (only whole 64-row groups can lie past the operand, as rows % 64 == 0).
struct DmaKS {
  rsrc_t r;
  uint32_t off;   // this lane's offset for instruction 0
  uint32_t step;  // 64 rows, bytes
  int valid;      // instructions 0 .. valid-1 read their own rows
  MOE_DEV void set(const bf16_t* b, size_t ld_elems, int rows) {
    r = make_rsrc(b);
    off = (uint32_t)(kmaj_row(0) * ld_elems * 2) + 16u * kmaj_chunk();
    step = (uint32_t)(64 * ld_elems * 2);
    valid = (rows + 63) / 64;
  }
  template <int S0 = 0, int S1 = 4>
  MOE_DEV void issue(int kt, char* st) const {
#pragma unroll
    for (int s = S0; s < S1; ++s)
      dmab(r, off, (uint32_t)kt * 128u + (s < valid ? s * step : 0u), kmaj_dst(st, s));
  }
};

MOE_DEV bf16x8_t frag_k(const char* st, int r0, int ks) {
  return *(const bf16x8_t*)(st + swz(r0 + (lane() & 31), 2 * ks + (lane() >> 5)));
}

// ----------------------------------------------------------- MN-major operand
// Stage: 64 K rows x 256 columns; chunk c of K row k at k * 512 + 16 (c ^ mnswz(k)).
// The swizzle spreads the eight K rows x four chunks that one transposing read
// touches over distinct banks.
MOE_DEV int mnswz(int k) { return mn_swz(k); }  // as for the 128-column tiles
// Instruction s of wavefront w fills K rows 16 s + 2 w and +1: lane L brings K row
// mn_row(s) = 16 s + 2 w + L / 32 into physical chunk L % 32 (the swizzle depends on
// k % 16 only: the same logical chunk for the four instructions).
MOE_DEV int mn_row(int s) { return 16 * s + 2 * wave() + (lane() >> 5); }
MOE_DEV char* mn_dst(char* st, int s) { return st + (8 * s + wave()) * 1024; }

struct DmaMN {
  rsrc_t r;          // element (K row 0, column 0) of this tile
  uint32_t off;      // this lane's offset for instruction 0
  uint32_t sstep;    // 16 K rows, bytes
  uint32_t kstep;    // 64 K rows, bytes
  // ncols valid columns (>= 8); columns past them read chunk 0 (never stored)
  MOE_DEV void set(const bf16_t* b, size_t ld_elems, int ncols) {
    r = make_rsrc(b);
    int c = (lane() & 31) ^ mnswz(mn_row(0));
    if (8 * c >= ncols) c = 0;
    off = (uint32_t)(mn_row(0) * ld_elems * 2) + 16u * c;
    sstep = (uint32_t)(16 * ld_elems * 2);
    kstep = (uint32_t)(64 * ld_elems * 2);
  }
  template <int S0 = 0, int S1 = 4>
  MOE_DEV void issue(int kt, char* st) const {
#pragma unroll
    for (int s = S0; s < S1; ++s) dmab(r, off, (uint32_t)kt * kstep + s * sstep, mn_dst(st, s));
  }
};

// Fragment of columns c0 .. c0 + 31 (c0 a multiple of 32) at K step ks: lane l gets
// column c0 + (l & 31), K values 16 ks + 8 (l >> 5) + 0..7 (the MFMA operand
// layout).  Lane l = 16 g + 4 a + j' addresses K row 16 ks + 8 (g >> 1) + j' (and
// +4 for the second read), columns c0 + 16 (g & 1) + 4 a .. +3.  The swizzle of
// those rows does not depend on ks, and the column chunk splits into the block's
// part (c0 / 8, a multiple of 4) and the lane's (2 (g & 1) + a / 2 < 4), so the
// address is a lane constant plus 16 * ((c0 / 8) ^ (swizzle & 12)) plus immediates.
MOE_DEV int mn_lane_ofs() {
  const int l = lane(), g = l >> 4, a = l & 3, j = (l >> 2) & 3;
  const int k = 8 * (g >> 1) + j;
  const int sw = mnswz(k);
  return k * 512 + (((2 * (g & 1) + (a >> 1)) ^ (sw & 3)) << 4) + (a & 1) * 8;
}
MOE_DEV int mn_blk_ofs(int c0) {
  const int l = lane(), g = l >> 4, j = (l >> 2) & 3;
  const int sw = mnswz(8 * (g >> 1) + j);
  return (((c0 >> 3) ^ (sw & 12)) << 4);
}
// The two reads are issued from inline assembly together with their lgkmcnt(0)
// wait: for the ds_read_b64_tr_b16 builtin the compiler first waits for every
// outstanding direct-to-LDS load (vmcnt(0)), i.e. for the next K tile's loads that
// were just issued, which would serialise the loads with the MFMAs.
MOE_DEV bf16x8_t frag_mn(const char* st, int c0, int ks) {
  const char* p = st + mn_lane_ofs() + mn_blk_ofs(c0) + ks * 16 * 512;
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
  s16x4_t lo, hi;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2\n\t"
      "ds_read_b64_tr_b16 %1, %2 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo), "=&v"(hi)
      : "v"(a)
      : "memory");
  const s16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// ------------------------------------------------------------------ main loop
// A: blocks i = 0..3 at rows 128 wm + 32 i; B: blocks j = 0..1 at columns
// 64 wn + 32 j.  ma / mb: number of leading blocks with any valid row / column
// (wave-uniform); the others are not multiplied.
struct Acc {
  f32x16_t c[4][2];
};

// Operand adaptors: issue(kt, stage) and frag(stage, block, ks, kt).
template <int AUX = 0>
struct OpKGT {  // K-major gathered rows
  DmaKGT<AUX> d;
  template <int S0 = 0, int S1 = 4>
  MOE_DEV void issue(int kt, char* st) const { d.template issue<S0, S1>(kt, st); }
  MOE_DEV bf16x8_t frag(const char* st, int r0, int ks, int) const { return frag_k(st, r0, ks); }
};
using OpKG = OpKGT<0>;
struct OpK {  // K-major strided rows
  DmaKS d;
  template <int S0 = 0, int S1 = 4>
  MOE_DEV void issue(int kt, char* st) const { d.template issue<S0, S1>(kt, st); }
  MOE_DEV bf16x8_t frag(const char* st, int r0, int ks, int) const { return frag_k(st, r0, ks); }
};
// GEMM1 weights: B-tile row 64 s + m (instruction s) is W_g (m < 32) or W_u
// (m >= 32) row 32 s + (m & 31) of this column tile.
struct OpUpW {
  rsrc_t r;       // W_g for wavefronts 0..3 (m < 32), W_u for 4..7
  uint32_t off;   // row (m & 31) + chunk, for instruction 0
  uint32_t step;  // 32 rows, bytes
  MOE_DEV void set(const bf16_t* wg_tile, const bf16_t* wu_tile, int H) {
    const int m = kmaj_row(0);  // 0..63, >= 32 exactly for wavefronts 4..7
    r = make_rsrc(wave_s() >= 4 ? wu_tile : wg_tile);
    off = (uint32_t)((m & 31) * H * 2) + 16u * kmaj_chunk();
    step = (uint32_t)(32 * H * 2);
  }
  template <int S0 = 0, int S1 = 4>
  MOE_DEV void issue(int kt, char* st) const {
#pragma unroll
    for (int s = S0; s < S1; ++s) dmab(r, off, (uint32_t)kt * 128u + s * step, kmaj_dst(st, s));
  }
  MOE_DEV bf16x8_t frag(const char* st, int r0, int ks, int) const { return frag_k(st, r0, ks); }
};
struct OpMN {  // MN-major, full K tiles
  DmaMN d;
  template <int S0 = 0, int S1 = 4>
  MOE_DEV void issue(int kt, char* st) const { d.template issue<S0, S1>(kt, st); }
  MOE_DEV bf16x8_t frag(const char* st, int c0, int ks, int) const { return frag_mn(st, c0, ks); }
};
struct OpMNCat {  // dgrad-up weights: K rows < I from W_g[e], the rest from W_u[e]
  DmaMN g, u;
  int kI;  // K tiles in W_g
  template <int S0 = 0, int S1 = 4>
  MOE_DEV void issue(int kt, char* st) const {
    if (kt < kI) g.template issue<S0, S1>(kt, st);
    else u.template issue<S0, S1>(kt - kI, st);
  }
  MOE_DEV bf16x8_t frag(const char* st, int c0, int ks, int) const { return frag_mn(st, c0, ks); }
};

// K-grouped MN-major operand (the wgrads): K row k is row seg0 + k of a row-major
// matrix, columns c0 .. c0 + 255 (all valid).  K rows at or past the segment's
// `n` rows read a 512-byte zero row in device memory, so the last K tile adds
// exactly zero and never reads another expert's rows.
__device__ __attribute__((aligned(16))) uint4 g_zero_row512[32];

struct OpMNSeg {
  const char* base;  // element (K row 0, column c0): wave-uniform
  rsrc_t r;          // the same base
  size_t ldb;        // row stride, bytes
  uint32_t off;      // this lane's offset for instruction 0 (K row r0, its chunk)
  uint32_t sstep;    // 16 K rows, bytes
  uint32_t col;      // this lane's chunk offset
  int r0, n;         // this lane's K row for instruction 0; rows in the segment
  MOE_DEV void set(const bf16_t* b, size_t ld_elems, int rows) {
    base = (const char*)b;
    r = make_rsrc(b);
    ldb = ld_elems * 2;
    r0 = mn_row(0);
    n = rows;
    col = 16u * (uint32_t)((lane() & 31) ^ mnswz(r0));
    off = (uint32_t)(r0 * ldb) + col;
    sstep = (uint32_t)(16 * ldb);
  }
  template <int S0 = 0, int S1 = 4>
  MOE_DEV void issue(int kt, char* st) const {
    const char* b = base + (size_t)kt * 64 * ldb;
    if (64 * kt + 64 <= n) {
#pragma unroll
      for (int s = S0; s < S1; ++s)
        dmab(r, off, (uint32_t)((size_t)kt * 64 * ldb) + s * sstep, mn_dst(st, s));
    } else {  // the segment's last K tile
#pragma unroll
      for (int s = S0; s < S1; ++s) {
        const char* src = 64 * kt + r0 + 16 * s < n ? b + off + s * sstep
                                                      : (const char*)g_zero_row512 + col;
        dma16(src, mn_dst(st, s));
      }
    }
  }
  MOE_DEV bf16x8_t frag(const char* st, int c0, int ks, int) const { return frag_mn(st, c0, ks); }
};

// Both operands MN-major (the wgrads): the twelve transposing reads of one 16-deep
// step are issued as one block with a single wait, instead of six waits.
MOE_DEV uint32_t lds_u32(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
MOE_DEV bf16x8_t join_tr(const s16x4_t& lo, const s16x4_t& hi) {
  return __builtin_bit_cast(bf16x8_t, (s16x8_t)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5,
                                                                        6, 7));
}
MOE_DEV void load_frags(const OpMNSeg&, const OpMNSeg&, const char* st, int, int ks, int wm, int wn,
                        int, int, bf16x8_t (&a)[4], bf16x8_t (&b)[2]) {
  const uint32_t base = lds_u32(st) + (uint32_t)(mn_lane_ofs() + ks * 16 * 512);
  const uint32_t a0 = base + mn_blk_ofs(128 * wm), a1 = base + mn_blk_ofs(128 * wm + 32);
  const uint32_t a2 = base + mn_blk_ofs(128 * wm + 64), a3 = base + mn_blk_ofs(128 * wm + 96);
  const uint32_t b0 = base + STAGE + mn_blk_ofs(64 * wn), b1 = base + STAGE + mn_blk_ofs(64 * wn + 32);
  s16x4_t r[12];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %12\n\t"
      "ds_read_b64_tr_b16 %1, %12 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %13\n\t"
      "ds_read_b64_tr_b16 %3, %13 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %14\n\t"
      "ds_read_b64_tr_b16 %5, %14 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %15\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:2048\n\t"
      "ds_read_b64_tr_b16 %8, %16\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %10, %17\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b0), "v"(b1)
      : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = join_tr(r[2 * i], r[2 * i + 1]);
#pragma unroll
  for (int j = 0; j < 2; ++j) b[j] = join_tr(r[8 + 2 * j], r[9 + 2 * j]);
}

template <class OA, class OB>
MOE_DEV void load_frags(const OA& A, const OB& B, const char* st, int kt, int ks, int wm, int wn,
                        int ma, int mb, bf16x8_t (&a)[4], bf16x8_t (&b)[2], int boff = STAGE) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < ma) a[i] = A.frag(st, 128 * wm + 32 * i, ks, kt);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (j < mb) b[j] = B.frag(st + boff, 64 * wn + 32 * j, ks, kt);
}

MOE_DEV void mma(Acc& acc, const bf16x8_t (&a)[4], const bf16x8_t (&b)[2], int ma, int mb) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (i < ma && j < mb)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.c[i][j], 0, 0, 0);
}

// LATE_B: the next K tile's B loads are issued after the first step's MFMAs instead
// of together with its A loads (the row-grouped kernels: measured on MI355X at
// T = 4096, Zipf(1.2), dgrad-up 3.12 -> 2.97 ms, GEMM2 1.76 -> 1.67 ms, the step
// 18.64 -> 18.45 ms; with the guard-free full-tile loop GEMM1 gains too, 2.72 ->
// 2.63 ms.  The hot wgrads, 3 % slower with it in this loop, gain with it in the
// interleaved loop below: 1.94 -> 1.90 ms (up), 0.97 -> 0.94 ms (down))
template <bool LATE_B = false, class OA, class OB>
MOE_DEV void main_loop(char* lds, const OA& A, const OB& B, int nk, int ma, int mb, Acc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.0f;
  if (nk <= 0) return;
  const int wm = wave() >> 2, wn = wave() & 3;
  A.issue(0, lds);
  B.issue(0, lds + STAGE);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  bf16x8_t a0[4], b0[2], a1[4], b1[2];
  load_frags(A, B, lds, 0, 0, wm, wn, ma, mb, a0, b0);
  for (int kt = 0; kt < nk; ++kt) {
    const char* cur = lds + (kt & 1) * 2 * STAGE;
    char* nxt = lds + ((kt + 1) & 1) * 2 * STAGE;
    // the last iteration reloads its own K tile into the idle stage (never read)
    const int kn = kt + 1 < nk ? kt + 1 : kt;
    A.issue(kn, nxt);
    if (!LATE_B) B.issue(kn, nxt + STAGE);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(A, B, cur, kt, 1, wm, wn, ma, mb, a1, b1);
    mma(acc, a0, b0, ma, mb);
    __builtin_amdgcn_sched_barrier(0);
    if (LATE_B) {
      B.issue(kn, nxt + STAGE);
      __builtin_amdgcn_sched_barrier(0);
    }
    load_frags(A, B, cur, kt, 2, wm, wn, ma, mb, a0, b0);
    mma(acc, a1, b1, ma, mb);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(A, B, cur, kt, 3, wm, wn, ma, mb, a1, b1);
    mma(acc, a0, b0, ma, mb);
    __builtin_amdgcn_sched_barrier(0);
    // this wavefront's reads of `cur` and its loads into `nxt` are complete; after
    // the barrier every wavefront's are: `nxt` is readable, `cur` reusable
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    load_frags(A, B, nxt, kt + 1, 0, wm, wn, ma, mb, a0, b0);
    mma(acc, a1, b1, ma, mb);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // LDS free for an epilogue
}

// Full tiles whose B operand is MN-major (dgrad-up's weights).  The transposing B
// reads are issued from inline assembly, which must wait for them inside the same
// block, and a block that only reads puts the whole read latency in front of the next
// MFMAs.  Here each 16-deep step issues the next step's A fragments (plain 16-byte
// reads) first, then one block with the next step's four B reads and the current
// step's MFMAs of A blocks 0 and 1, waiting at its end, then the MFMAs of blocks 2 and
// 3.  (Eight accumulators as operands of one block made the compiler run without end.)
// Measured on MI355X: dgrad-up 2.93 / 2.92 -> 2.91 / 2.89 ms at T = 4096 and 0.846 /
// 0.840 -> 0.827 / 0.831 ms on four experts of 4096 rows.  Forcing every fragment
// read of the other loops ahead of its step's MFMAs instead changed nothing for the
// K-major operands and made dgrad-up 2 % slower.
template <class OB> struct is_mn { static constexpr bool value = false; };
template <> struct is_mn<OpMN> { static constexpr bool value = true; };
template <> struct is_mn<OpMNCat> { static constexpr bool value = true; };

template <class OA>
MOE_DEV void step_kmn(const OA& A, const char* st, int kt, int ks, int wm, int wn,
                      const bf16x8_t (&ac)[4], const bf16x8_t (&bc)[2], bf16x8_t (&an)[4],
                      bf16x8_t (&bn)[2], Acc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) an[i] = A.frag(st, 128 * wm + 32 * i, ks, kt);
  const char* bs = st + STAGE + mn_lane_ofs() + ks * 16 * 512;
  const uint32_t p0 = lds_u32(bs + mn_blk_ofs(64 * wn)), p1 = lds_u32(bs + mn_blk_ofs(64 * wn + 32));
  s16x4_t l0, h0, l1, h1;
  asm volatile(
      "s_nop 2\n\t"
      "ds_read_b64_tr_b16 %0, %10\n\t"
      "ds_read_b64_tr_b16 %1, %10 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %11\n\t"
      "ds_read_b64_tr_b16 %3, %11 offset:2048\n\t"
      "v_mfma_f32_32x32x16_bf16 %4, %8, %12, %4\n\t"
      "v_mfma_f32_32x32x16_bf16 %5, %8, %13, %5\n\t"
      "v_mfma_f32_32x32x16_bf16 %6, %9, %12, %6\n\t"
      "v_mfma_f32_32x32x16_bf16 %7, %9, %13, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(l0), "=&v"(h0), "=&v"(l1), "=&v"(h1), "+v"(acc.c[0][0]), "+v"(acc.c[0][1]),
        "+v"(acc.c[1][0]), "+v"(acc.c[1][1])
      : "v"(ac[0]), "v"(ac[1]), "v"(p0), "v"(p1), "v"(bc[0]), "v"(bc[1])
      : "memory");
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 2; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ac[i], bc[j], acc.c[i][j], 0, 0, 0);
  bn[0] = join_tr(l0, h0);
  bn[1] = join_tr(l1, h1);
}

// Both operands MN-major (the hot wgrads): two blocks per step, each with six of the
// next step's twelve transposing reads and four of the current step's MFMAs (measured
// on MI355X against one block of twelve reads and its wait before the MFMAs: hot
// wgrad-up 2.00 -> 1.98 ms, wgrad-down 1.02 -> 1.00 ms at T = 4096).
MOE_DEV void step_mnmn(const char* st, int ks, int wm, int wn, const bf16x8_t (&ac)[4],
                       const bf16x8_t (&bc)[2], bf16x8_t (&an)[4], bf16x8_t (&bn)[2], Acc& acc) {
  const uint32_t base = lds_u32(st) + (uint32_t)(mn_lane_ofs() + ks * 16 * 512);
  const uint32_t pa0 = base + mn_blk_ofs(128 * wm), pa1 = base + mn_blk_ofs(128 * wm + 32);
  const uint32_t pa2 = base + mn_blk_ofs(128 * wm + 64), pa3 = base + mn_blk_ofs(128 * wm + 96);
  const uint32_t pb0 = base + STAGE + mn_blk_ofs(64 * wn);
  const uint32_t pb1 = base + STAGE + mn_blk_ofs(64 * wn + 32);
  s16x4_t r[12];
  asm volatile(
      "s_nop 2\n\t"
      "ds_read_b64_tr_b16 %0, %14\n\t"
      "ds_read_b64_tr_b16 %1, %14 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %15\n\t"
      "ds_read_b64_tr_b16 %3, %15 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %16\n\t"
      "ds_read_b64_tr_b16 %5, %16 offset:2048\n\t"
      "v_mfma_f32_32x32x16_bf16 %6, %10, %12, %6\n\t"
      "v_mfma_f32_32x32x16_bf16 %7, %10, %13, %7\n\t"
      "v_mfma_f32_32x32x16_bf16 %8, %11, %12, %8\n\t"
      "v_mfma_f32_32x32x16_bf16 %9, %11, %13, %9\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "+v"(acc.c[0][0]), "+v"(acc.c[0][1]), "+v"(acc.c[1][0]), "+v"(acc.c[1][1])
      : "v"(ac[0]), "v"(ac[1]), "v"(bc[0]), "v"(bc[1]), "v"(pa0), "v"(pa1), "v"(pa2)
      : "memory");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile(
      "s_nop 2\n\t"
      "ds_read_b64_tr_b16 %0, %14\n\t"
      "ds_read_b64_tr_b16 %1, %14 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %15\n\t"
      "ds_read_b64_tr_b16 %3, %15 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %16\n\t"
      "ds_read_b64_tr_b16 %5, %16 offset:2048\n\t"
      "v_mfma_f32_32x32x16_bf16 %6, %10, %12, %6\n\t"
      "v_mfma_f32_32x32x16_bf16 %7, %10, %13, %7\n\t"
      "v_mfma_f32_32x32x16_bf16 %8, %11, %12, %8\n\t"
      "v_mfma_f32_32x32x16_bf16 %9, %11, %13, %9\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
        "+v"(acc.c[2][0]), "+v"(acc.c[2][1]), "+v"(acc.c[3][0]), "+v"(acc.c[3][1])
      : "v"(ac[2]), "v"(ac[3]), "v"(bc[0]), "v"(bc[1]), "v"(pa3), "v"(pb0), "v"(pb1)
      : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) an[i] = join_tr(r[2 * i], r[2 * i + 1]);
#pragma unroll
  for (int j = 0; j < 2; ++j) bn[j] = join_tr(r[8 + 2 * j], r[9 + 2 * j]);
}

template <class OA, class OB>
MOE_DEV void step_asm(const OA& A, const OB&, const char* st, int kt, int ks, int wm, int wn,
                      const bf16x8_t (&ac)[4], const bf16x8_t (&bc)[2], bf16x8_t (&an)[4],
                      bf16x8_t (&bn)[2], Acc& acc) {
  step_kmn(A, st, kt, ks, wm, wn, ac, bc, an, bn, acc);
}
MOE_DEV void step_asm(const OpMNSeg&, const OpMNSeg&, const char* st, int, int ks, int wm, int wn,
                      const bf16x8_t (&ac)[4], const bf16x8_t (&bc)[2], bf16x8_t (&an)[4],
                      bf16x8_t (&bn)[2], Acc& acc) {
  step_mnmn(st, ks, wm, wn, ac, bc, an, bn, acc);
}

// The two-stage loop of main_loop<LATE_B> for such tiles, with the steps above.
template <bool LATE_B, class OA, class OB>
MOE_DEV void main_loop_kmn(char* lds, const OA& A, const OB& B, int nk, Acc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.0f;
  if (nk <= 0) return;
  const int wm = wave() >> 2, wn = wave() & 3;
  A.issue(0, lds);
  B.issue(0, lds + STAGE);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  bf16x8_t a0[4], b0[2], a1[4], b1[2];
  load_frags(A, B, lds, 0, 0, wm, wn, 4, 2, a0, b0);
  for (int kt = 0; kt < nk; ++kt) {
    const char* cur = lds + (kt & 1) * 2 * STAGE;
    char* nxt = lds + ((kt + 1) & 1) * 2 * STAGE;
    const int kn = kt + 1 < nk ? kt + 1 : kt;  // the last iteration: the idle stage
    A.issue(kn, nxt);
    if (!LATE_B) B.issue(kn, nxt + STAGE);
    __builtin_amdgcn_sched_barrier(0);
    step_asm(A, B, cur, kt, 1, wm, wn, a0, b0, a1, b1, acc);
    __builtin_amdgcn_sched_barrier(0);
    if (LATE_B) {
      B.issue(kn, nxt + STAGE);
      __builtin_amdgcn_sched_barrier(0);
    }
    step_asm(A, B, cur, kt, 2, wm, wn, a1, b1, a0, b0, acc);
    __builtin_amdgcn_sched_barrier(0);
    step_asm(A, B, cur, kt, 3, wm, wn, a0, b0, a1, b1, acc);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    step_asm(A, B, nxt, kt + 1, 0, wm, wn, a1, b1, a0, b0, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  // wait states between the last MFMAs of the assembly blocks and reads of their
  // results by other instructions (not tracked by the compiler across the blocks);
  // every accumulator passes through one of the two blocks, so no read of one can be
  // placed before them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(acc.c[0][0]), "+v"(acc.c[0][1]), "+v"(acc.c[1][0]), "+v"(acc.c[1][1]));
  asm volatile("s_nop 0"
               : "+v"(acc.c[2][0]), "+v"(acc.c[2][1]), "+v"(acc.c[3][0]), "+v"(acc.c[3][1]));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // LDS free for an epilogue
}

// Tiles with at most RA rows (RA = 64 or 128; a small expert's single tile) run K
// through a ring of NS stages instead: a stage holds only the RA rows of A that
// exist (RA * 128 bytes) and the full B part (32 KiB), so RA = 64 fits four stages
// (three in flight, 120 KiB against the 64 KiB of the two-stage loop) and RA = 128
// three.  These tiles are bound by streaming their weights; with more bytes in flight
// a CU streams faster while other CUs run the MFMA-bound tiles of larger experts
// (a CU alone pulls ~40 GB/s, ~20 GB/s when every CU streams).  The A loads of such
// a tile are RA / 64 instructions per lane and the B loads four: the ring's waits
// count (RA / 64 + 4) per stage.
template <int RA>
MOE_DEV void ring_wait_small(int ahead) {
  constexpr int L = RA / 64 + 4;  // loads per stage per lane
  static_assert(2 * L < 16, "vmcnt field");
  if (ahead >= 2) __builtin_amdgcn_s_waitcnt((2 * L) | 0x70);
  else if (ahead == 1) __builtin_amdgcn_s_waitcnt(L | 0x70);
  else __builtin_amdgcn_s_waitcnt(0x70);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");  // no LDS read of the stage moves above the barrier
}

template <int RA, int NS, class OA, class OB>
MOE_DEV void main_loop_small(char* lds, const OA& A, const OB& B, int nk, int ma, int mb,
                             Acc& acc) {
  constexpr int SA = RA * 128, SST = SA + STAGE;
  static_assert(NS * SST <= 163840 && NS >= 2 && NS <= 4, "ring fits the LDS");
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.0f;
  if (nk <= 0) return;
  const int wm = wave() >> 2, wn = wave() & 3;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) {
      A.issue(s, lds + s * SST);
      B.issue(s, lds + s * SST + SA);
    }
  int slot = 0;  // kt % NS
  for (int kt = 0; kt < nk; ++kt) {
    ring_wait_small<RA>(min(NS - 2, nk - 1 - kt));  // stage kt in; kt - 1 no longer read
    if (kt + NS - 1 < nk) {  // into the slot of stage kt - 1
      char* st = lds + (slot == 0 ? NS - 1 : slot - 1) * SST;
      A.issue(kt + NS - 1, st);
      B.issue(kt + NS - 1, st + SA);
    }
    __builtin_amdgcn_sched_barrier(0);
    const char* cur = lds + slot * SST;
    bf16x8_t a0[4], b0[2], a1[4], b1[2];
    load_frags(A, B, cur, kt, 0, wm, wn, ma, mb, a0, b0, SA);
    load_frags(A, B, cur, kt, 1, wm, wn, ma, mb, a1, b1, SA);
    mma(acc, a0, b0, ma, mb);
    load_frags(A, B, cur, kt, 2, wm, wn, ma, mb, a0, b0, SA);
    mma(acc, a1, b1, ma, mb);
    load_frags(A, B, cur, kt, 3, wm, wn, ma, mb, a1, b1, SA);
    mma(acc, a0, b0, ma, mb);
    mma(acc, a1, b1, ma, mb);
    slot = slot == NS - 1 ? 0 : slot + 1;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // LDS free for an epilogue
}

// The K loop of a row-grouped tile: the two-stage loop, or the ring for a tile with
// at most 128 rows.
// A wavefront with all its blocks (ma = 4, mb = 2: every wavefront of a full tile) runs
// a copy of the two-stage loop compiled for them, free of the per-block guards, which
// otherwise split the loop body into a branch around every fragment read and MFMA pair.
// Both copies meet the same barriers, one per K tile.  (The same copies of the small-
// tile rings, for their wavefronts with all blocks, made GEMM2 and dgrad-up slower on
// MI355X: 1.60 -> 1.65 and 2.88 -> 3.00 ms at T = 4096.)
template <class OA, class OB>
MOE_DEV void main_loop_rows(char* lds, const OA& A, const OB& B, int nk, int rows, int ma, int mb,
                            Acc& acc) {
  if (rows <= 64) main_loop_small<64, 4>(lds, A, B, nk, ma, mb, acc);
  else if (rows <= 128) main_loop_small<128, 3>(lds, A, B, nk, ma, mb, acc);
  else if (ma == 4 && mb == 2) {
    if constexpr (is_mn<OB>::value) main_loop_kmn<true>(lds, A, B, nk, acc);
    else main_loop<true>(lds, A, B, nk, 4, 2, acc);
  } else {
    main_loop<true>(lds, A, B, nk, ma, mb, acc);
  }
}

// Output position of register v of block (i, j): row 128 wm + 32 i + 8 (v >> 2) +
// 4 (l >> 5) + (v & 3), column 64 wn + 32 j + (l & 31).
MOE_DEV int out_row(int i, int v) {
  return 128 * (wave() >> 2) + 32 * i + 8 * (v >> 2) + 4 * (lane() >> 5) + (v & 3);
}
MOE_DEV int out_col(int j) { return 64 * (wave() & 3) + 32 * j + (lane() & 31); }
// out_row(i, v) - out_row(0, 0), and out_row(0, 0) hidden from loop-invariant code
// motion: in a persistent kernel the compiler otherwise computes the 64 row indices of
// the epilogue once before the item loop and keeps (or spills) them across the GEMM
MOE_DEV int out_row_rel(int i, int v) { return 32 * i + 8 * (v >> 2) + (v & 3); }
MOE_DEV int out_row_base() {
  int r = out_row(0, 0);
  asm volatile("" : "+v"(r));
  return r;
}

// Leading A blocks of this wavefront with a row below `rows`, B blocks with a
// column below `cols`.
// (read back as wave-uniform values: the block guards of the K loops are then scalar
// branches, and the full case below is recognised as such)
MOE_DEV int blocks_a(int rows) {
  return __builtin_amdgcn_readfirstlane(min(4, max(0, (rows - 128 * (wave() >> 2) + 31) / 32)));
}
MOE_DEV int blocks_b(int cols) {
  return __builtin_amdgcn_readfirstlane(min(2, max(0, (cols - 64 * (wave() & 3) + 31) / 32)));
}

// ------------------------------------------------------------ tile decode
struct Tile {
  int e, row0, row_end;
  int mt;  // index of the row tile in the plan's wide-tile list (dense: the tile)
};

// Rows-grouped launches: a 1-D grid over (256-row tile, column tile) pairs in the
// order of group_rows (groups of 4 row tiles), dealt round-robin to the XCDs.  With
// one workgroup per CU, contiguous runs per XCD (as for the 128-row kernels) left
// the XCDs holding hot experts' full tiles behind those holding small experts'
// weight-bound tiles; dealt round-robin, every XCD gets a share of both, and the
// tiles that share a weight panel run at the same time on neighbouring XCDs
// (dgrad-up 4.10 -> 3.84 ms, GEMM1 + SwiGLU 3.24 -> 3.10 ms measured on MI355X).
//
// GEMM1 + SwiGLU deals blocks of XCD_BLOCK consecutive pairs instead (block j to XCD
// j mod 8, the launch rounded up to whole rounds of 8 blocks): a block covers 4 row
// tiles x 4 column tiles of a group, so the workgroups an XCD runs at once share
// their token rows and weight panels in its L2 (measured on MI355X at T = 4096,
// Zipf(1.2): GEMM1 2.97 -> 2.90 ms over three runs each; the same dealing made
// dgrad-up slower, 3.26 -> 3.29 ms, and left GEMM2 unchanged, so those keep single
// pairs).
constexpr int XCD_BLOCK = 16;
template <bool BLOCKS>
MOE_DEV bool row_tile_at(const GroupInfo& g, int nt_count, int id, Tile& t, int& nt) {
  const int n_row_tiles = g.wtiles ? g.n_wtiles[0] : (g.dense_rows + TILE - 1) / TILE;
  const int total = n_row_tiles * nt_count;
  int L = id;
  if (BLOCKS) {
    const int x = L % N_XCD, q = L / N_XCD;
    L = ((q / XCD_BLOCK) * N_XCD + x) * XCD_BLOCK + q % XCD_BLOCK;
  }
  if (L >= total) return false;
  int mt;
  group_rows(g.wtiles, g.offsets, g.dense_rows, TILE, nt_count, 4, L, mt, nt);
  t.mt = mt;
  if (g.wtiles) {
    t.e = g.wtiles[2 * mt];
    t.row0 = g.wtiles[2 * mt + 1];
    t.row_end = min(t.row0 + TILE, g.offsets[t.e + 1]);
  } else {
    t.e = 0;
    t.row0 = mt * TILE;
    t.row_end = min(t.row0 + TILE, g.dense_rows);
  }
  return true;
}

template <bool BLOCKS>
MOE_DEV bool row_tile(const GroupInfo& g, int nt_count, Tile& t, int& nt) {
  return row_tile_at<BLOCKS>(g, nt_count, blockIdx.x, t, nt);
}

MOE_DEV int row_of_tile(const Tile& t, int r) {  // clamp rows past the tile's end
  return t.row0 + r < t.row_end ? t.row0 + r : t.row0;
}

// ---------------------------------------------------------------- kernels
// GEMM1 + SwiGLU.  Column tile nt covers i in [128 nt, 128 nt + 128): B-tile rows
// 64 wn + rr (rr < 32) are W_g[e] row 128 nt + 32 wn + rr and rows 64 wn + 32 + rr
// the W_u[e] row of the same i, so gate and up of one (row, i) are the same
// register of blocks 0 and 1 of one lane and the SwiGLU is formed in registers.
// Z (fp32) keeps the pre-activations for the backward; h = silu(A) B rounds once.
// COHERENT_H: h is stored through to device scope (for a consumer on another XCD)
template <bool COHERENT_H = false>
MOE_DEV void up_swiglu_tile(char* lds, const GroupInfo& g, const Tile& t, int nt,
                            const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg,
                            const bf16_t* __restrict__ wu, int H, int I, float* __restrict__ Z,
                            bf16_t* __restrict__ hout) {
  const size_t wofs = (size_t)t.e * I * H;
  OpKG A;
  OpUpW B;
  A.d.set(x, t.row_end - t.row0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int r = row_of_tile(t, kmaj_row(s));
    A.d.row(s, (size_t)(g.src_token ? g.src_token[r] : r) * H);
  }
  B.set(wg + wofs + (size_t)128 * nt * H, wu + wofs + (size_t)128 * nt * H, H);
  Acc acc;
  main_loop_rows(lds, A, B, H / 64, t.row_end - t.row0, blocks_a(t.row_end - t.row0), 2, acc);
  const int i = 128 * nt + 32 * (wave() & 3) + (lane() & 31);
  const int rb = t.row0 + out_row_base();
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = rb + out_row_rel(bi, v);
      if (r < t.row_end) {
        const float a = acc.c[bi][0][v], b = acc.c[bi][1][v];
        float* zr = Z + (size_t)r * (2 * I);
        // Z is read back only by the backward: non-temporal (GEMM1 2.91 -> 2.87 ms)
        __builtin_nontemporal_store(a, zr + i);
        __builtin_nontemporal_store(b, zr + I + i);
        const bf16_t hv = f32_to_bf16(silu_f(a) * b);
        if (COHERENT_H)
          __hip_atomic_store((uint16_t*)(hout + (size_t)r * I + i), __builtin_bit_cast(uint16_t, hv),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          hout[(size_t)r * I + i] = hv;
      }
    }
}

__global__ __launch_bounds__(NTH, 1) void k_up_swiglu(GroupInfo g, const bf16_t* __restrict__ x,
                                                      const bf16_t* __restrict__ wg,
                                                      const bf16_t* __restrict__ wu, int H, int I,
                                                      float* __restrict__ Z,
                                                      bf16_t* __restrict__ hout) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_ROWS];
  Tile t;
  int nt;
  if (!row_tile<true>(g, I / 128, t, nt)) return;
  up_swiglu_tile(lds, g, t, nt, x, wg, wu, H, I, Z, hout);
}

// GEMM2: Y[r, n] = sum_i h[r, i] W_d[e][n, i] (grouped and the dense shared expert;
// against the 128 x 128 kernel: 1.86 -> 1.81 ms at the skewed E = 256 workload,
// 0.65 -> 0.55 ms at four experts of 4096 rows)
// AUX: cache policy of the h loads; COHERENT_Y: Y is stored through to device scope
// (for a consumer on another XCD)
template <int AUX = 0, bool COHERENT_Y = false>
MOE_DEV void down_tile(char* lds, const Tile& t, int nt, const bf16_t* __restrict__ h,
                       const bf16_t* __restrict__ wd, int H, int I, bf16_t* __restrict__ Y) {
  const int n0 = nt * TILE;
  OpKGT<AUX> A;
  OpK B;
  A.d.set(h, t.row_end - t.row0);
#pragma unroll
  for (int s = 0; s < 4; ++s) A.d.row(s, (size_t)row_of_tile(t, kmaj_row(s)) * I);
  B.d.set(wd + (size_t)t.e * H * I + (size_t)n0 * I, (size_t)I, H - n0);
  Acc acc;
  main_loop_rows(lds, A, B, I / 64, t.row_end - t.row0, blocks_a(t.row_end - t.row0),
                 blocks_b(H - n0), acc);
  const int rb = t.row0 + out_row_base();
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int n = n0 + out_col(bj);
      if (n < H)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = rb + out_row_rel(bi, v);
          if (r < t.row_end) {
            const bf16_t yv = f32_to_bf16(acc.c[bi][bj][v]);
            if (COHERENT_Y)
              __hip_atomic_store((uint16_t*)(Y + (size_t)r * H + n),
                                 __builtin_bit_cast(uint16_t, yv), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            else
              Y[(size_t)r * H + n] = yv;
          }
        }
    }
}

__global__ __launch_bounds__(NTH, 1) void k_down(GroupInfo g, const bf16_t* __restrict__ h,
                                                 const bf16_t* __restrict__ wd, int H, int I,
                                                 bf16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_ROWS];
  Tile t;
  int nt;
  if (!row_tile<false>(g, (H + TILE - 1) / TILE, t, nt)) return;
  down_tile(lds, t, nt, h, wd, H, I, Y);
}

// ------------------------------------------------ the forward in one launch
// GEMM1 + SwiGLU and GEMM2 of the routed and the shared experts and the combine as
// one persistent kernel, the producer / consumer form of the pages' megakernel on one
// GPU (stamatios.com, "Cursor abre código de megakernel MoE para GPUs NVL72",
// § Granularidade do overlap: units signal each other through local counters;
// § Outras características: one kernel).  The work items, in order, are the routed
// GEMM1 pairs (in the order and XCD dealing of k_up_swiglu), the shared expert's
// GEMM1 pairs, the routed GEMM2 pairs (those of k_down), the shared GEMM2 pairs and
// the combine items (FUSED_CMB_TOKENS tokens each); item q goes to XCD q mod 8 as
// in the separate launches, and the workgroups of one XCD (workgroup b runs on XCD
// b mod 8) take that XCD's items in order from a counter, so that work balances as
// it does when the dispatcher hands out a launch's workgroups.
//   A GEMM1 pair stores h with device-coherent stores (written through to the
// device's coherence point, not left in its XCD's L2), waits for them, and adds one
// to its row tile's counter; a GEMM2 pair waits until that counter has all I / 128
// column tiles and then reads h with device-coherent loads (no stale line of its own
// XCD's L2; measured on MI355X against an acquire / release pair, which invalidates
// and writes back the whole L2: 5.08 -> 4.96 ms before the queues).  A GEMM2 pair
// stores Y the same way and adds one to `done`; a combine item waits until `done`
// holds every GEMM2 pair, then reads Y and the shared rows at device scope.  Each
// XCD's queue hands out all its GEMM1 items before any GEMM2 item and all those
// before any combine item, and GEMM1 items never wait, so every wait ends once the
// workgroups holding the producers run.  A wait gives up after about two seconds
// (err bit 2: possible only if other work keeps CUs from this grid that long); the
// item then reads whatever its input holds.  The arithmetic of every tile and chunk
// is that of the separate kernels, so the outputs are bitwise theirs.
struct FusedFwd {
  GroupInfo g;      // routed rows (wide-tile list)
  GroupInfo gs;     // the shared expert: dense over the T tokens
  const bf16_t* x;
  const bf16_t* wg;
  const bf16_t* wu;
  const bf16_t* wd;
  const bf16_t* sg;  // shared expert weights (NULL: none)
  const bf16_t* su;
  const bf16_t* sd;
  int H, I, Is, T, k;
  float* Z;
  bf16_t* h;
  bf16_t* Y;
  float* Zs;
  bf16_t* hs;
  bf16_t* ys;
  const int32_t* pos;   // [T, k] row of each (token, slot)
  const float* w;       // [T, k] combine weights
  bf16_t* y;            // [T, H] layer output
  int32_t* ready;   // [max_wtiles] routed row-tile counters, zero at launch
  int32_t* readys;  // [n_rts] shared row-tile counters, zero at launch
  int32_t* done;    // [1] GEMM2 pairs finished, zero at launch
  int32_t* next;    // [8] per-XCD item counters, zero at launch
  int32_t* err;
  // item counts of the phases (the virtual grids of the separate kernels), n_rts the
  // shared expert's row tiles
  int n1, n1s, n2, n2s, nc, n_rts;
};

// A GroupInfo of the kernel arguments copied field by field from the constant address
// space (each field a scalar load); the copy constructor does not bind to it.
MOE_DEV GroupInfo group_from_args(const __attribute__((address_space(4))) GroupInfo& s) {
  GroupInfo g;
  g.tiles = s.tiles;
  g.n_tiles = s.n_tiles;
  g.offsets = s.offsets;
  g.src_token = s.src_token;
  g.src_slot = s.src_slot;
  g.active = s.active;
  g.n_active = s.n_active;
  g.counts = s.counts;
  g.wtiles = s.wtiles;
  g.n_wtiles = s.n_wtiles;
  g.max_tiles = s.max_tiles;
  g.max_wtiles = s.max_wtiles;
  g.dense_rows = s.dense_rows;
  g.E = s.E;
  g.hot_rows = s.hot_rows;
  return g;
}
static_assert(sizeof(GroupInfo) == 10 * sizeof(void*) + 5 * sizeof(int) + 4,
              "group_from_args copies every field of GroupInfo");

constexpr int FUSED_SPIN_LIMIT = 1 << 20;  // waits of ~4096 cycles each
constexpr int FUSED_CMB_TOKENS = 4;

// thread 0 waits until *c >= target (bounded: err bit 2 on giving up); then the
// workgroup goes on
MOE_DEV void fused_wait(const int32_t* c, int target, int32_t* err) {
  if (threadIdx.x == 0) {
    int spins = 0;
    while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (++spins > FUSED_SPIN_LIMIT) {
        __hip_atomic_fetch_or(err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(64);
    }
  }
  __syncthreads();
}

// thread 0 claims the workgroup's next item of queue `next` (its index lands in
// `claimed`); then every lane's coherent stores have completed, then one count on c
// for the workgroup.  The claim goes out first so that its round trip overlaps the
// wait for the stores.
MOE_DEV void fused_signal(int32_t* c, int32_t* next, int& claimed) {
  if (threadIdx.x == 0)
    claimed = __hip_atomic_fetch_add(next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The launch's fields are read through a pointer that an empty asm statement hides
// from the compiler at every item, so that each phase loads the few it uses from the
// kernel arguments instead of keeping all of them in scalar registers across the loop
// (with them held, the kernel spilled scalar registers into vector registers).
__global__ __launch_bounds__(NTH, 1) void k_forward_fused(FusedFwd arg) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_ROWS];
  int* s_item = (int*)lds;  // LDS is free between items
  // the launch's only argument, at the start of the kernel-argument segment (taking
  // arg's address would copy it to private memory), read through the constant address
  // space: its fields load as scalars (through a generic pointer they came back in
  // vector registers, and every buffer resource built from them was wrapped in a loop
  // over distinct values)
  typedef const __attribute__((address_space(4))) FusedFwd kfused_t;
  kfused_t* pa = (kfused_t*)__builtin_amdgcn_kernarg_segment_ptr();
  const int x = blockIdx.x % N_XCD;
  int claimed = -1;  // thread 0: the next item, if already claimed
  for (;;) {
    kfused_t* pp = pa;
    asm volatile("" : "+s"(pp));
    kfused_t& p = *pp;
    // next item of this XCD's queue (items x, x + 8, ... in order), claimed here or
    // already at the end of the previous tile
    if (threadIdx.x == 0) {
      if (claimed < 0)
        claimed = __hip_atomic_fetch_add(p.next + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_item = claimed;
      claimed = -1;
    }
    __syncthreads();
    // the same in every lane: scalar, so that the tile's operand bases (buffer
    // resources) are scalar too
    const int q = __builtin_amdgcn_readfirstlane(*s_item * N_XCD + x);
    __syncthreads();  // read by every thread before the tile overwrites the LDS
    const int q1s = p.n1, q2 = q1s + p.n1s, q2s = q2 + p.n2, qc = q2s + p.n2s;
    if (q >= qc + p.nc) break;
    const int nt2 = (p.H + TILE - 1) / TILE;
    Tile t;
    int nt;
    // the tile's coordinates as scalars (they come from loads of the tile list, which
    // the compiler cannot take as uniform here: with them in vector registers every
    // buffer load was wrapped in a loop over distinct resources)
    auto uniform = [](Tile& tt, int& n) {
      tt.e = __builtin_amdgcn_readfirstlane(tt.e);
      tt.mt = __builtin_amdgcn_readfirstlane(tt.mt);
      tt.row0 = __builtin_amdgcn_readfirstlane(tt.row0);
      tt.row_end = __builtin_amdgcn_readfirstlane(tt.row_end);
      n = __builtin_amdgcn_readfirstlane(n);
    };
    // routed and shared items of one GEMM share one inlined tile body (two bodies
    // per GEMM left the routed tiles 5% slower); the operands are picked per item
    if (q < q2) {
      const bool sh = q >= q1s;
      const GroupInfo g = group_from_args(sh ? p.gs : p.g);
      const int I = sh ? p.Is : p.I;
      if (!row_tile_at<true>(g, I / 128, sh ? q - q1s : q, t, nt)) continue;
      uniform(t, nt);
      up_swiglu_tile<true>(lds, g, t, nt, p.x, sh ? p.sg : p.wg, sh ? p.su : p.wu, p.H, I,
                           sh ? p.Zs : p.Z, sh ? p.hs : p.h);
      fused_signal((sh ? p.readys : p.ready) + t.mt, p.next + x, claimed);
    } else if (q < qc) {
      const bool sh = q >= q2s;
      const GroupInfo g = group_from_args(sh ? p.gs : p.g);
      const int I = sh ? p.Is : p.I;
      if (!row_tile_at<false>(g, nt2, sh ? q - q2s : q - q2, t, nt)) continue;
      uniform(t, nt);
      fused_wait((sh ? p.readys : p.ready) + t.mt, I / 128, p.err);
      down_tile<CPOL_DEVICE, true>(lds, t, nt, sh ? p.hs : p.h, sh ? p.sd : p.wd, p.H, I,
                                   sh ? p.ys : p.Y);
      fused_signal(p.done, p.next + x, claimed);
    } else {
      // every routed and shared GEMM2 pair: n_wtiles x nt2 + n_rts x nt2
      fused_wait(p.done, (p.g.n_wtiles[0] + p.n_rts) * nt2, p.err);
      const int rc = p.H / 8, sl = (rc + 63) / 64, t0 = (q - qc) * FUSED_CMB_TOKENS;
      const int ntok = min(FUSED_CMB_TOKENS, p.T - t0);
      const uint4* Y = (const uint4*)p.Y;
      const uint4* ys = (const uint4*)p.ys;
      uint4* y = (uint4*)p.y;
      // one wave per (token, 64 chunks): the token, and so its pos and w, are
      // wave-uniform
      for (int u = wave(); u < ntok * sl; u += NTH / 64) {
        const int tk = t0 + u / sl, c = (u % sl) * 64 + lane();
        if (c < rc)
          combine_chunk<true, true>(Y, p.pos + (size_t)tk * p.k, p.w + (size_t)tk * p.k,
                                    ys ? ys + (size_t)tk * rc : nullptr, y + (size_t)tk * rc,
                                    p.k, rc, c);
      }
    }
  }
}

__global__ void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// dgrad-up: dX[r, n] = sum_{k < 2I} dZ[r, k] Wcat[k, n], Wcat = [W_g[e]; W_u[e]]
__global__ __launch_bounds__(NTH, 1) void k_dgrad_up(GroupInfo g, const bf16_t* __restrict__ dZ,
                                                     const bf16_t* __restrict__ wg,
                                                     const bf16_t* __restrict__ wu, int H, int I,
                                                     bf16_t* __restrict__ dX) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_ROWS];
  Tile t;
  int nt;
  if (!row_tile<false>(g, (H + TILE - 1) / TILE, t, nt)) return;
  const int n0 = nt * TILE, ncols = min(TILE, H - n0);
  const size_t wofs = (size_t)t.e * I * H + n0;
  OpKG A;
  OpMNCat B;
  A.d.set(dZ, t.row_end - t.row0);
#pragma unroll
  for (int s = 0; s < 4; ++s) A.d.row(s, (size_t)row_of_tile(t, kmaj_row(s)) * (2 * I));
  B.g.set(wg + wofs, (size_t)H, ncols);
  B.u.set(wu + wofs, (size_t)H, ncols);
  B.kI = I / 64;
  Acc acc;
  main_loop_rows(lds, A, B, (2 * I) / 64, t.row_end - t.row0, blocks_a(t.row_end - t.row0),
                 blocks_b(ncols), acc);
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int n = n0 + out_col(bj);
      if (n < H)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = t.row0 + out_row(bi, v);
          if (r < t.row_end) dX[(size_t)r * H + n] = f32_to_bf16(acc.c[bi][bj][v]);
        }
    }
}

// ------------------------------------------------------- K-grouped wgrads
// Weight gradients of the experts with many rows, on this core: out[e][m, n] =
// sum over the expert's rows r of A[r, m] B[r, n] (wgrad-up: A = dZ, B = X, M = 2I,
// N = H, rows m < I to dW_g and the rest to dW_u; wgrad-down: A = dYu, B = g h,
// M = H, N = I), K running over the expert's segment of the plan in row order.
// Both operands are K-outer (MN-major) and read as they lie, no transposes.  The
// experts with fewer rows and the zero gradients of the experts without rows stay
// on the 128 x 128 kernel, whose two workgroups per CU overlap those short,
// write-bound items.  (Measured on MI355X: storing the zero gradients from this
// kernel, inside its K loop or from workgroups of their own, overlapped nothing.)
//
// Persistent grid (a multiple of 8 workgroups, one per CU); workgroup b runs on XCD
// b mod 8.  Each expert's PM x PN-tile output is cut into a GM x (8 / GM) grid of
// rectangles, one per XCD, chosen as square as the counts allow (fewest operand
// panels per XCD: each panel an XCD reads comes from the Infinity Cache or HBM), and
// an XCD's workgroups walk its rectangles of all hot experts in id order, M index
// fastest: the workgroups an XCD runs at once share a few panels in its L2.  Every
// output element is produced by one workgroup with a fixed K order.
// XCD x's rectangle of an expert's PM x PN output tiles: the 8 XCDs form a GM x
// (8 / GM) grid over the tiles (XCD x at row x / (8 / GM), column x % (8 / GM)).
MOE_DEV void xcd_rect(int PM, int PN, int GM, int x, int& m_lo, int& n_lo, int& pm, int& pn) {
  const int GN = N_XCD / GM, wm = (PM + GM - 1) / GM, wn = (PN + GN - 1) / GN;
  m_lo = (x / GN) * wm;
  n_lo = (x % GN) * wn;
  pm = max(0, min(wm, PM - m_lo));
  pn = max(0, min(wn, PN - n_lo));
}

struct WgradArgs {
  const int32_t* counts;   // NULL: dense, one "expert" of dense_rows rows
  const int32_t* offsets;
  int E, hot_rows, dense_rows;
  const bf16_t* A;
  const bf16_t* B;
  int lda, ldb;          // row strides (elements)
  bf16_t* out0;          // output rows m < half_rows
  bf16_t* out1;          // output rows m >= half_rows (wgrad-up: dW_u)
  int M, N, half_rows;   // per-expert output
  int PM, PN, GM;        // 256-tiles per expert along M and N; XCD groups along M
};

// wave 0 lists, in id order, the experts with >= hot_rows rows
MOE_DEV int list_hot(const int32_t* counts, int E, int hot_rows, int* hot, int* n) {
  if (wave() == 0) {
    int nh = 0;
    const uint64_t below = (1ull << lane()) - 1ull;
    for (int b = 0; b < E; b += 64) {
      const int e = b + lane();
      const bool h = e < E && counts[e] >= hot_rows;
      const uint64_t mh = __ballot(h);
      if (h) hot[nh + __popcll(mh & below)] = e;
      nh += __popcll(mh);
    }
    if (lane() == 0) n[0] = nh;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(n[0]);
}

__global__ __launch_bounds__(NTH, 1) void k_wgrad_hot(WgradArgs p) {
  __shared__ __attribute__((aligned(16))) char lds[LDS];
  __shared__ int s_hot[MOE_MAX_E], s_n[1];
  const int n_hot = p.counts ? list_hot(p.counts, p.E, p.hot_rows, s_hot, s_n) : 1;
  const int x = blockIdx.x % N_XCD, slot = blockIdx.x / N_XCD, nslot = gridDim.x / N_XCD;
  int m_lo, n_lo, pm, pn;  // this XCD's rectangle: tiles [m_lo, +pm) x [n_lo, +pn)
  xcd_rect(p.PM, p.PN, p.GM, x, m_lo, n_lo, pm, pn);
  const int per = pm * pn;
  const int nq = per * n_hot;  // tiles of this XCD
  const long part0 = (long)p.half_rows * p.N, part1 = (long)(p.M - p.half_rows) * p.N;
  for (int q = slot; q < nq; q += nslot) {
    const int h = q / per, j = q - h * per;
    const int e = p.counts ? __builtin_amdgcn_readfirstlane(s_hot[h]) : 0;
    const int m0 = (m_lo + j % pm) * TILE, n0 = (n_lo + j / pm) * TILE;
    const int seg0 = p.counts ? ld_uniform(p.offsets + e) : 0;
    const int n = p.counts ? ld_uniform(p.offsets + e + 1) - seg0 : p.dense_rows;
    OpMNSeg A, B;
    A.set(p.A + (size_t)seg0 * p.lda + m0, (size_t)p.lda, n);
    B.set(p.B + (size_t)seg0 * p.ldb + n0, (size_t)p.ldb, n);
    Acc acc;
    main_loop_kmn<true>(lds, A, B, (n + 63) / 64, acc);
    bf16_t* base = m0 < p.half_rows
                       ? p.out0 + (size_t)e * part0 + (size_t)m0 * p.N + n0
                       : p.out1 + (size_t)e * part1 + (size_t)(m0 - p.half_rows) * p.N + n0;
    // row stride made opaque per tile: otherwise the 64 row offsets of the stores
    // below are hoisted out of the tile loop and held in registers (spills)
    int ld = p.N;
    asm volatile("" : "+s"(ld));
    bf16_t* lp = base + (size_t)out_row(0, 0) * ld + out_col(0);
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16_t* rp = lp + (size_t)(32 * bi + 8 * g4) * ld;
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            rp[(size_t)r * ld + 32 * bj] = f32_to_bf16(acc.c[bi][bj][4 * g4 + r]);
        __builtin_amdgcn_sched_barrier(0);
      }
  }
}

// ------------------------------------------------------- MXFP8 K-grouped wgrads
// The MXFP8 weight gradients of the experts with many rows, on this core.  Both
// operands are the token-axis-transposed E4M3 rows of the MX path (A: rows of M,
// B: rows of N, each Kp bytes long, one E8M0 scale byte per 32 along the packed
// token axis; expert e owns bytes [kpos[e], kpos[e + 1]) of every row, a multiple of
// 32).  A stage is a 128-byte K piece of 256 rows per operand, in the K-major layout
// of the bf16 kernels (bytes are bytes), and feeds two 64-deep steps of the scaled
// MFMA v_mfma_scale_f32_32x32x64_f8f6f4.  In that instruction lane i + 32 h holds
// row i and takes bytes 0-15 from K block 0 and 16-31 from K block 1 of its step,
// and the scale of (row i, block c) comes from lane i + 32 c: lane (i, h) reads the
// 16-byte chunks 4 ks + h and 4 ks + 2 + h of its row, and uses byte 2 ks + h of its
// row's scale word.  The scale words reach the LDS four pieces at a time (MxScaleLds);
// the bytes of blocks at or past the expert's end are set to 0 (2^-127), so those
// blocks' products (next expert's codes, or the zero tail written after the packed
// axis) vanish.
typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct DmaKB {  // K-major byte rows at a fixed stride
  rsrc_t r;          // row 0, K byte 0 of this expert's range
  uint32_t off;      // this lane's row for instruction 0, chunk included
  uint32_t step;     // 64 rows, bytes
  MOE_DEV void set(const uint8_t* b, size_t ld) {
    r = make_rsrc(b);
    off = (uint32_t)(kmaj_row(0) * ld) + 16u * kmaj_chunk();
    step = (uint32_t)(64 * ld);
  }
  MOE_DEV void issue(int kt, char* st) const {
#pragma unroll
    for (int s = 0; s < 4; ++s) dmab(r, off, (uint32_t)kt * 128u + s * step, kmaj_dst(st, s));
  }
};

// this lane's scale words of one stage: A blocks 0..3, B blocks 0..1
struct MxScales {
  uint32_t a[4], b[2];
};

// Scale bytes of the 256 A and 256 B rows of a wgrad tile, four K pieces (16 bytes
// of each row) at a time, through the LDS: thread t loads, in the stage of part u
// (kt % 4) of the next group, the 4-byte word t % 4 of row u * 128 + t / 4 of the
// 512 (A rows, then B rows), and stores it to that group's LDS buffer after the
// stage's wait.  Each load instruction then covers 16 rows' contiguous bytes, where
// one 4-byte word per fragment row per stage (six loads per lane, each touching 32
// rows' cache lines) cost about a third of the kernel's time.
struct MxScaleLds {
  const uint8_t* as;  // A scale rows (row stride ks bytes)
  const uint8_t* bs;
  uint32_t offa;      // this thread's A row of part 0, its K byte of the range start
  uint32_t offb;
  uint32_t step;      // 128 rows
  int lim;            // largest in-row offset past the range start that keeps a word
                      // inside the row
  long kbytes;        // bytes of the expert's range
  MOE_DEV void set(const uint8_t* a_rows, const uint8_t* b_rows, long ks, long k0, long kb) {
    const int t = threadIdx.x;
    as = a_rows;
    bs = b_rows;
    offa = (uint32_t)((t >> 2) * ks + k0 / 32);
    offb = offa;
    step = (uint32_t)(128 * ks);
    lim = (int)(ks - 4 - k0 / 32);
    kbytes = kb;
  }
  // part u of group G (pieces 4 G .. 4 G + 3)
  MOE_DEV uint32_t load(int G, int u) const {
    const uint32_t o = (u < 2 ? offa : offb) + (u & 1) * step +
                       (uint32_t)min(16 * G + 4 * (int)(threadIdx.x & 3), lim);
    return *(const uint32_t*)((u < 2 ? as : bs) + o);
  }
  MOE_DEV void put(char* sb, int u, uint32_t w) const {
    *(uint32_t*)(sb + 16 * (128 * u + (threadIdx.x >> 2)) + 4 * (threadIdx.x & 3)) = w;
  }
  // this lane's words of piece kt from the group buffer sb, blocks past the range zero
  MOE_DEV void words(const char* sb, int kt, int wm, int wn, MxScales& sc) const {
    const long nb = (kbytes - (long)kt * 128) / 32;  // blocks of this piece inside the range
    const uint32_t keep = nb >= 4 ? 0xffffffffu : (nb <= 0 ? 0u : (1u << (8 * nb)) - 1u);
    const int l = lane() & 31, u = kt & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sc.a[i] = *(const uint32_t*)(sb + 16 * (128 * wm + 32 * i + l) + 4 * u) & keep;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      sc.b[j] = *(const uint32_t*)(sb + 16 * (TILE + 64 * wn + 32 * j + l) + 4 * u) & keep;
  }
};

MOE_DEV i32x8_t frag_mx(const char* st, int r0, int ks) {
  const int r = r0 + (lane() & 31), h = lane() >> 5;
  const uint4 x = *(const uint4*)(st + swz(r, 4 * ks + h));
  const uint4 y = *(const uint4*)(st + swz(r, 4 * ks + 2 + h));
  i32x8_t v;
  v[0] = (int)x.x; v[1] = (int)x.y; v[2] = (int)x.z; v[3] = (int)x.w;
  v[4] = (int)y.x; v[5] = (int)y.y; v[6] = (int)y.z; v[7] = (int)y.w;
  return v;
}

// one stage of scaled MFMAs: A blocks below ma, B blocks below mb (B at st + boff);
// the B fragments of a step first, then the A fragments one block at a time with
// the next block's read in flight during the current block's MFMAs
MOE_DEV void mma_stage_mx_m(const char* st, int boff, const MxScales& sc, int wm, int wn, int ma,
                            int mb, Acc& acc) {
  const int h = lane() >> 5;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int sh = 8 * (2 * ks + h);
    i32x8_t b[2], a[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (j < mb) b[j] = frag_mx(st + boff, 64 * wn + 32 * j, ks);
    if (ma > 0) a[0] = frag_mx(st, 128 * wm, ks);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i + 1 < ma) a[(i + 1) & 1] = frag_mx(st, 128 * wm + 32 * (i + 1), ks);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (i < ma && j < mb)
          acc.c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              a[i & 1], b[j], acc.c[i][j], 0, 0, 0, (int)((sc.a[i] >> sh) & 0xffu), 0,
              (int)((sc.b[j] >> sh) & 0xffu));
    }
  }
}

constexpr int MX_WSBUF = 2 * TILE * 16;  // scale bytes of one group of four pieces

// Two LDS data stages (piece kt + 1 loads while piece kt multiplies) and two scale
// group buffers after them (group G read in pieces 4 G .. 4 G + 3 from buffer G mod 2,
// written during pieces 4 G - 4 .. 4 G - 1; past the last group the words loaded and
// stored are unused, which keeps the loop free of branches: with a branch around
// them the compiler spilled registers).  Every piece ends with the whole workgroup's
// loads and LDS stores done and a barrier.
MOE_DEV void main_loop_mx(char* lds, const DmaKB& A, const DmaKB& B, const MxScaleLds& S, int nk,
                          Acc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.0f;
  if (nk <= 0) return;
  const int wm = wave() >> 2, wn = wave() & 3;
  char* const sb = lds + 4 * STAGE;
  A.issue(0, lds);
  B.issue(0, lds + STAGE);
  uint32_t w0 = S.load(0, 0), w1 = S.load(0, 1), w2 = S.load(0, 2), w3 = S.load(0, 3);
  __builtin_amdgcn_s_waitcnt(0);
  S.put(sb, 0, w0);
  S.put(sb, 1, w1);
  S.put(sb, 2, w2);
  S.put(sb, 3, w3);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const char* cur = lds + (kt & 1) * 2 * STAGE;
    const int kn = kt + 1, gn = (kt >> 2) + 1, u = kt & 3;
    if (kn < nk) {
      char* nxt = lds + (kn & 1) * 2 * STAGE;
      A.issue(kn, nxt);
      B.issue(kn, nxt + STAGE);
    }
    const uint32_t w = S.load(gn, u);  // past the last group: an unused word
    MxScales sc;
    S.words(sb + ((kt >> 2) & 1) * MX_WSBUF, kt, wm, wn, sc);
    __builtin_amdgcn_sched_barrier(0);
    mma_stage_mx_m(cur, STAGE, sc, wm, wn, 4, 2, acc);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    S.put(sb + (gn & 1) * MX_WSBUF, u, w);  // never the buffer being read
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  __syncthreads();  // LDS free for another tile
}

struct MxWgradArgs {
  const int32_t* kpos;  // [E + 1] packed token-axis offsets (bytes)
  int E, hot_bytes;
  const uint8_t* A8;
  const uint8_t* As;
  const uint8_t* B8;
  const uint8_t* Bs;
  long Kp;              // row length of A8, B8 (bytes); scale rows are Kp / 32
  bf16_t* out0;
  bf16_t* out1;
  int M, N, half_rows;
  int PM, PN, GM;
};

// wave 0 lists, in id order, the experts whose packed range has >= hot_bytes bytes
MOE_DEV int list_hot_kpos(const int32_t* kpos, int E, int hot_bytes, int* hot, int* n) {
  if (wave() == 0) {
    int nh = 0;
    const uint64_t below = (1ull << lane()) - 1ull;
    for (int b = 0; b < E; b += 64) {
      const int e = b + lane();
      const bool h = e < E && kpos[e + 1] - kpos[e] >= hot_bytes;
      const uint64_t mh = __ballot(h);
      if (h) hot[nh + __popcll(mh & below)] = e;
      nh += __popcll(mh);
    }
    if (lane() == 0) n[0] = nh;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(n[0]);
}

__global__ __launch_bounds__(NTH, 1) void k_wgrad_hot_mx(MxWgradArgs p) {
  __shared__ __attribute__((aligned(16))) char lds[LDS + 2 * MX_WSBUF];
  __shared__ int s_hot[MOE_MAX_E], s_n[1];
  const int n_hot = list_hot_kpos(p.kpos, p.E, p.hot_bytes, s_hot, s_n);
  const int x = blockIdx.x % N_XCD, slot = blockIdx.x / N_XCD, nslot = gridDim.x / N_XCD;
  int m_lo, n_lo, pm, pn;
  xcd_rect(p.PM, p.PN, p.GM, x, m_lo, n_lo, pm, pn);
  const int per = pm * pn;
  const int nq = per * n_hot;
  const long KS = p.Kp / 32;
  const long part0 = (long)p.half_rows * p.N, part1 = (long)(p.M - p.half_rows) * p.N;
    for (int q = slot; q < nq; q += nslot) {
    const int h = q / per, j = q - h * per;
    const int e = __builtin_amdgcn_readfirstlane(s_hot[h]);
    const int m0 = (m_lo + j % pm) * TILE, n0 = (n_lo + j / pm) * TILE;
    const long k0 = ld_uniform(p.kpos + e), kb = ld_uniform(p.kpos + e + 1) - k0;
    DmaKB A, B;
    A.set(p.A8 + (size_t)m0 * p.Kp + k0, (size_t)p.Kp);
    B.set(p.B8 + (size_t)n0 * p.Kp + k0, (size_t)p.Kp);
    MxScaleLds S;
    S.set(p.As + (size_t)m0 * KS, p.Bs + (size_t)n0 * KS, KS, k0, kb);
    Acc acc;
    main_loop_mx(lds, A, B, S, (int)((kb + 127) / 128), acc);
    bf16_t* base = m0 < p.half_rows
                       ? p.out0 + (size_t)e * part0 + (size_t)m0 * p.N + n0
                       : p.out1 + (size_t)e * part1 + (size_t)(m0 - p.half_rows) * p.N + n0;
    int ld = p.N;  // opaque per tile (see k_wgrad_hot)
    asm volatile("" : "+s"(ld));
    bf16_t* lp = base + (size_t)out_row(0, 0) * ld + out_col(0);
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16_t* rp = lp + (size_t)(32 * bi + 8 * g4) * ld;
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            rp[(size_t)r * ld + 32 * bj] = f32_to_bf16(acc.c[bi][bj][4 * g4 + r]);
        __builtin_amdgcn_sched_barrier(0);
      }
  }
}

// ------------------------------------------------------- MXFP8 row-grouped GEMMs
// GEMM2 and dgrad-up of the MX path on this core.  Every operand is a
// K-major E4M3 byte row with one E8M0 scale byte per 32 (the activations of a
// minibatch's ring slot and the quantised weights, in the orientation whose rows run
// along the GEMM's K).  A stage is a 128-byte K piece of the tile's 256 A and 256 B
// rows in the K-major layout of the bf16 kernels (128 codes: two 64-deep scaled MFMA
// steps).  The scale bytes of four stages (16 per row) reach the LDS with one
// direct-to-LDS load per lane: lane q of the workgroup loads row q of the 512 tile
// rows (A rows, then B rows), one group ahead of its use, into one of two 8 KiB
// buffers; each stage then reads its lane's six scale words from the LDS.  Loading
// the words per stage from global memory instead (six 4-byte loads per lane, each
// instruction touching 32 rows' cache lines) cost about 30 % of these kernels' time.
// The K order of every output element is that of the 128 x 128 MX kernels (64-deep
// steps from K = 0), so the results are the same.  Needs H and I multiples of 512, so
// that scale groups and dgrad-up's W_g / W_u split align.  Measured on MI355X at T =
// 8192 in minibatches of 2048 (H = 7168, I = 2048, E = 256, k = 8, Zipf(1.2)), per
// minibatch launch against the 128 x 128 MX kernels: GEMM2 0.73 -> 0.66 ms, dgrad-up
// 1.34 -> 1.21 ms.  GEMM1 + SwiGLU on this core took 1.58 against 1.54 ms and stays on
// the 128 x 128 kernel; issuing the B loads after the first MFMA step (as the bf16
// kernels do) made all three slower (GEMM2 0.70, dgrad-up 1.32 ms).
constexpr int MX_GROUP = 4;                                  // K stages per scale load
constexpr int MX_SBUF = 2 * TILE * 16;                       // scale bytes of one group
static_assert(4 * STAGE + 2 * MX_SBUF <= LDS_ROWS, "MX stages and scale groups fit");

// A rows row0 .. row0 + rows - 1 of a K-major byte matrix (row stride ld): only the
// instructions whose 64 rows include one of the tile's are issued; rows past the
// tile inside an issued instruction read row 0 of the tile (their outputs are not
// stored).
struct MxDmaA {
  rsrc_t r;
  uint32_t off[4];
  int n;
  MOE_DEV void set(const uint8_t* b, size_t ld, int rows) {
    r = make_rsrc(b);
    n = (rows + 63) / 64;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = kmaj_row(s);
      off[s] = (uint32_t)((r < rows ? r : 0) * ld) + 16u * kmaj_chunk();
    }
  }
  MOE_DEV void issue(int kt, char* st) const {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (s < n) dmab(r, off[s], (uint32_t)kt * 128u, kmaj_dst(st, s));
  }
};

// B: 256 weight rows at a fixed stride, K stages from kI on from a second matrix
// (dgrad-up's W_u^T after W_g^T)
struct MxDmaB {
  rsrc_t r0, r1;
  uint32_t off, step;
  int kI;
  MOE_DEV void set(const uint8_t* b0, const uint8_t* b1, size_t ld, int k_split) {
    r0 = make_rsrc(b0);
    r1 = make_rsrc(b1);
    off = (uint32_t)(kmaj_row(0) * ld) + 16u * kmaj_chunk();
    step = (uint32_t)(64 * ld);
    kI = k_split;
  }
  MOE_DEV void issue(int kt, char* st) const {
    const bool hi = kt >= kI;
    const rsrc_t r = hi ? r1 : r0;
    const uint32_t k0 = (uint32_t)(hi ? kt - kI : kt) * 128u;
#pragma unroll
    for (int s = 0; s < 4; ++s) dmab(r, off, k0 + s * step, kmaj_dst(st, s));
  }
};

// Scale bytes of one group for this lane's tile row q = 64 wave + lane (A rows 0..255,
// then B rows): 16 bytes at src0 + 16 g, or at src1 + 16 g from group g1 on (src1
// pre-offset by -16 g1), into row q of an 8 KiB buffer.
struct MxScaleDma {
  const char* src0;
  const char* src1;
  int g1;
  MOE_DEV void issue(int g, char* sb) const {
    dma16((g >= g1 ? src1 : src0) + 16 * g, sb + wave() * 1024);
  }
};

// this lane's scale words of stage u of the group in sb: A blocks 0..3 of rows
// 128 wm + 32 i + (lane & 31), B blocks 0..1 of rows 64 wn + 32 j + (lane & 31)
MOE_DEV void mx_stage_scales(const char* sb, int u, int wm, int wn, MxScales& sc) {
  const int l = lane() & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) sc.a[i] = *(const uint32_t*)(sb + 16 * (128 * wm + 32 * i + l) + 4 * u);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    sc.b[j] = *(const uint32_t*)(sb + 16 * (TILE + 64 * wn + 32 * j + l) + 4 * u);
}

// Two LDS data stages (stage kt + 1 loads while stage kt multiplies) and two scale
// buffers: group G's scale bytes are issued with the data of stage 4 G, i.e. during
// stage 4 G - 1, into buffer G mod 2, which group G - 2 used.  Every stage ends with
// the whole workgroup's loads in and a barrier, so each buffer is full before it is
// read and no longer read when it is loaded again.
template <class OA, class OB>
MOE_DEV void main_loop_rows_mx_body(char* lds, const OA& A, const OB& B, const MxScaleDma& S,
                                    int nk, int ma, int mb, Acc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.0f;
  if (nk > 0) {
    const int wm = wave() >> 2, wn = wave() & 3;
    char* const sb = lds + 4 * STAGE;
    A.issue(0, lds);
    B.issue(0, lds + STAGE);
    S.issue(0, sb);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const char* cur = lds + (kt & 1) * 2 * STAGE;
      const int kn = kt + 1;
      if (kn < nk) {
        char* nxt = lds + (kn & 1) * 2 * STAGE;
        A.issue(kn, nxt);
        B.issue(kn, nxt + STAGE);
        if (kn % MX_GROUP == 0) S.issue(kn / MX_GROUP, sb + ((kn / MX_GROUP) & 1) * MX_SBUF);
      }
      MxScales sc;
      mx_stage_scales(sb + ((kt / MX_GROUP) & 1) * MX_SBUF, kt % MX_GROUP, wm, wn, sc);
      __builtin_amdgcn_sched_barrier(0);
      mma_stage_mx_m(cur, STAGE, sc, wm, wn, ma, mb, acc);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // LDS free for an epilogue or the next tile
}

// As main_loop_rows: a wavefront with all its blocks runs a copy of the loop free of
// the per-block guards.
template <class OA, class OB>
MOE_DEV void main_loop_rows_mx(char* lds, const OA& A, const OB& B, const MxScaleDma& S, int nk,
                               int ma, int mb, Acc& acc) {
  if (ma == 4 && mb == 2) main_loop_rows_mx_body(lds, A, B, S, nk, 4, 2, acc);
  else main_loop_rows_mx_body(lds, A, B, S, nk, ma, mb, acc);
}

// Scale source of this lane's tile row when it is an A row (q < 256): the tile's row
// q (rows past the tile: its row 0); sc_tile is the scale row of the tile's row 0,
// ks the scale row stride.  Returns NULL for a B row.
MOE_DEV const char* mx_scale_src_a(const uint8_t* sc_tile, size_t ks, int rows) {
  const int q = 64 * wave() + lane();
  if (q >= TILE) return nullptr;
  return (const char*)sc_tile + (size_t)(q < rows ? q : 0) * ks;
}

// GEMM2, MX: Y = Q_I(h) Q_I(W_d)^T in bf16
__global__ __launch_bounds__(NTH, 1) void k_down_mx(GroupInfo g, const uint8_t* __restrict__ hq,
                                                    const uint8_t* __restrict__ hsc,
                                                    const uint8_t* __restrict__ wd8,
                                                    const uint8_t* __restrict__ wds, int H, int I,
                                                    bf16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_ROWS];
  Tile t;
  int nt;
  if (!row_tile<false>(g, H / TILE, t, nt)) return;
  const int rows = t.row_end - t.row0, n0 = nt * TILE, IS = I / 32;
  const size_t wrow = (size_t)t.e * H + n0;
  MxDmaA A;
  A.set(hq + (size_t)t.row0 * I, (size_t)I, rows);
  MxDmaB B;
  B.set(wd8 + wrow * I, wd8 + wrow * I, (size_t)I, 1 << 30);
  MxScaleDma S;
  S.src0 = mx_scale_src_a(hsc + (size_t)t.row0 * IS, (size_t)IS, rows);
  if (!S.src0) S.src0 = (const char*)wds + (wrow + (64 * wave() + lane() - TILE)) * IS;
  S.src1 = S.src0;
  S.g1 = 1 << 30;
  Acc acc;
  main_loop_rows_mx(lds, A, B, S, I / 128, blocks_a(rows), 2, acc);
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int n = n0 + out_col(bj);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = t.row0 + out_row(bi, v);
        if (r < t.row_end) Y[(size_t)r * H + n] = f32_to_bf16(acc.c[bi][bj][v]);
      }
    }
}

// dgrad-up, MX: dX = Q_2I(dZ) [Q_I(W_g); Q_I(W_u)] with the weights stored transposed
// [E, H, I]: B row n takes W_g^T[e][n] for K < I and W_u^T[e][n] after
__global__ __launch_bounds__(NTH, 1) void k_dgrad_up_mx(GroupInfo g, const uint8_t* __restrict__ dZ8,
                                                        const uint8_t* __restrict__ dZs,
                                                        const uint8_t* __restrict__ wgT8,
                                                        const uint8_t* __restrict__ wgTs,
                                                        const uint8_t* __restrict__ wuT8,
                                                        const uint8_t* __restrict__ wuTs, int H,
                                                        int I, bf16_t* __restrict__ dX) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_ROWS];
  Tile t;
  int nt;
  if (!row_tile<false>(g, H / TILE, t, nt)) return;
  const int rows = t.row_end - t.row0, n0 = nt * TILE, IS = I / 32, S2 = (2 * I) / 32;
  const int kI = I / 128;
  const size_t wrow = (size_t)t.e * H + n0;
  MxDmaA A;
  A.set(dZ8 + (size_t)t.row0 * (2 * I), (size_t)(2 * I), rows);
  MxDmaB B;
  B.set(wgT8 + wrow * I, wuT8 + wrow * I, (size_t)I, kI);
  MxScaleDma S;
  S.src0 = mx_scale_src_a(dZs + (size_t)t.row0 * S2, (size_t)S2, rows);
  S.g1 = 1 << 30;
  if (S.src0) {
    S.src1 = S.src0;
  } else {
    const size_t n = wrow + (64 * wave() + lane() - TILE);
    S.src0 = (const char*)wgTs + n * IS;
    S.g1 = kI / MX_GROUP;
    S.src1 = (const char*)wuTs + n * IS - 16 * S.g1;
  }
  Acc acc;
  main_loop_rows_mx(lds, A, B, S, (2 * I) / 128, blocks_a(rows), 2, acc);
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int n = n0 + out_col(bj);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = t.row0 + out_row(bi, v);
        if (r < t.row_end) dX[(size_t)r * H + n] = f32_to_bf16(acc.c[bi][bj][v]);
      }
    }
}

// Zero the 128 bytes after the packed token axis of every row (stages of the last
// expert read up to 96 bytes past its range; those bytes are otherwise never written).
__global__ __launch_bounds__(256) void mx_zero_tail_kernel(uint8_t* __restrict__ q, int rows,
                                                           long Kp,
                                                           const int32_t* __restrict__ kend) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;  // 16-byte piece
  if (i >= (long)rows * 8) return;
  const long row = i / 8, b = kend[0] + 16 * (i % 8);
  if (b + 16 > Kp) return;  // the row ends first (at least 96 bytes follow kpos[E])
  const u32x4_t z = {0u, 0u, 0u, 0u};
  *(u32x4_t*)(q + row * Kp + b) = z;
}

}  // namespace big

// ------------------------------------------------------------------ launchers
static unsigned big_row_tiles(const GroupInfo& g) {
  return g.wtiles ? (unsigned)g.max_wtiles
                  : (unsigned)((g.dense_rows + big::TILE - 1) / big::TILE);
}
// grid of a launch that deals blocks of pairs: whole rounds of 8 blocks
static unsigned big_row_grid(unsigned pairs) {
  const unsigned r = N_XCD * big::XCD_BLOCK;
  return (pairs + r - 1) / r * r;
}

hipError_t launch_big_up_swiglu(const GroupInfo& g, const void* x, const void* wg, const void* wu,
                                int H, int I, void* Z, void* h, hipStream_t s) {
  const unsigned ty = big_row_tiles(g);
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH(g.wtiles ? "gemm_up_swiglu" : "gemm_up_swiglu_shared", s,
                    big::k_up_swiglu<<<big_row_grid(ty * (I / 128)), big::NTH, 0, s>>>(
                        g, (const bf16_t*)x, (const bf16_t*)wg, (const bf16_t*)wu, H, I,
                        (float*)Z, (bf16_t*)h));
}

// The bf16 forward after the plan in one persistent launch (k_forward_fused); the
// counters (fused_counters(g.max_wtiles, T) int32) are zeroed here by a small kernel.
hipError_t launch_big_forward_fused(const FusedForwardArgs& a, hipStream_t s) {
  const GroupInfo& g = a.g;
  if (!g.wtiles || g.max_wtiles == 0) return hipErrorNotSupported;
  if (a.T <= 0) return hipSuccess;
  const int n_rts = a.Is ? (a.T + big::TILE - 1) / big::TILE : 0;
  const int n_cnt = fused_counters(g.max_wtiles, a.T);
  hipError_t e = MOE_LAUNCH(
      "fused_zero", s, big::zero_i32_kernel<<<(n_cnt + 255) / 256, 256, 0, s>>>(a.ready, n_cnt));
  if (e != hipSuccess) return e;
  big::FusedFwd p;
  p.g = g;
  p.gs = a.gs;
  if (a.Is && (a.gs.wtiles || a.gs.dense_rows != a.T)) return hipErrorInvalidValue;
  p.x = (const bf16_t*)a.x;
  p.wg = (const bf16_t*)a.wg;
  p.wu = (const bf16_t*)a.wu;
  p.wd = (const bf16_t*)a.wd;
  p.sg = (const bf16_t*)a.sg;
  p.su = (const bf16_t*)a.su;
  p.sd = (const bf16_t*)a.sd;
  p.H = a.H;
  p.I = a.I;
  p.Is = a.Is;
  p.T = a.T;
  p.k = a.k;
  p.Z = (float*)a.Z;
  p.h = (bf16_t*)a.h;
  p.Y = (bf16_t*)a.Y;
  p.Zs = (float*)a.Zs;
  p.hs = (bf16_t*)a.hs;
  p.ys = a.Is ? (bf16_t*)a.ys : nullptr;
  p.pos = a.pos;
  p.w = a.w;
  p.y = (bf16_t*)a.y;
  p.ready = a.ready;
  p.readys = a.ready + g.max_wtiles;
  p.done = p.readys + n_rts;
  p.next = p.done + 1;
  p.err = a.err;
  const int nt2 = (a.H + big::TILE - 1) / big::TILE;
  p.n1 = (int)big_row_grid((unsigned)g.max_wtiles * (a.I / 128));
  p.n1s = a.Is ? (int)big_row_grid((unsigned)n_rts * (a.Is / 128)) : 0;
  p.n2 = g.max_wtiles * nt2;
  p.n2s = n_rts * nt2;
  p.nc = (a.T + big::FUSED_CMB_TOKENS - 1) / big::FUSED_CMB_TOKENS;
  p.n_rts = n_rts;
  const int cus = device_cus();
  const unsigned grid = (unsigned)(cus >= N_XCD ? cus - cus % N_XCD : N_XCD);
  return MOE_LAUNCH("gemm_forward_fused", s, big::k_forward_fused<<<grid, big::NTH, 0, s>>>(p));
}

hipError_t launch_big_down(const GroupInfo& g, const void* h, const void* wd, int H, int I,
                           void* Y, hipStream_t s) {
  const unsigned ty = big_row_tiles(g);
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH(g.wtiles ? "gemm_down" : "gemm_down_shared", s,
                    big::k_down<<<ty * ((H + big::TILE - 1) / big::TILE), big::NTH, 0, s>>>(
                        g, (const bf16_t*)h, (const bf16_t*)wd, H, I, (bf16_t*)Y));
}

hipError_t launch_big_dgrad_up(const GroupInfo& g, const void* dZ, const void* wg, const void* wu,
                               int H, int I, void* dX, hipStream_t s) {
  const unsigned ty = big_row_tiles(g);
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH(g.wtiles ? "gemm_dgrad_up" : "gemm_dgrad_up_shared", s,
                    big::k_dgrad_up<<<ty * ((H + big::TILE - 1) / big::TILE), big::NTH, 0, s>>>(
                        g, (const bf16_t*)dZ, (const bf16_t*)wg, (const bf16_t*)wu, H, I,
                        (bf16_t*)dX));
}

// MX GEMM2 and dgrad-up on this core: H and I multiples of 512 (scale groups of 512
// bytes of K) and the plan's wide-tile list present; hipErrorNotSupported (nothing
// enqueued) otherwise
static bool big_mx_ok(const GroupInfo& g, int H, int I) {
  return g.wtiles && H % 512 == 0 && I % 512 == 0;
}

hipError_t launch_big_mx_down(const GroupInfo& g, const uint8_t* hq, const uint8_t* hs,
                              const uint8_t* wd8, const uint8_t* wds, int H, int I, void* Y,
                              hipStream_t s) {
  if (!big_mx_ok(g, H, I)) return hipErrorNotSupported;
  const unsigned ty = big_row_tiles(g);
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH("mx_gemm_down", s,
                    big::k_down_mx<<<ty * (H / big::TILE), big::NTH, 0, s>>>(
                        g, hq, hs, wd8, wds, H, I, (bf16_t*)Y));
}

hipError_t launch_big_mx_dgrad_up(const GroupInfo& g, const uint8_t* dZ8, const uint8_t* dZs,
                                  const uint8_t* wgT8, const uint8_t* wgTs, const uint8_t* wuT8,
                                  const uint8_t* wuTs, int H, int I, void* dX, hipStream_t s) {
  if (!big_mx_ok(g, H, I)) return hipErrorNotSupported;
  const unsigned ty = big_row_tiles(g);
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH("mx_gemm_dgrad_up", s,
                    big::k_dgrad_up_mx<<<ty * (H / big::TILE), big::NTH, 0, s>>>(
                        g, dZ8, dZs, wgT8, wgTs, wuT8, wuTs, H, I, (bf16_t*)dX));
}

// GM for xcd_rect: the XCD grid (GM x 8 / GM) whose rectangles need the fewest panels
// (rows + columns of tiles), ties to the more even split
static int xcd_grid_rows(int PM, int PN) {
  int best = 1, cost = 1 << 30;
  for (int gm = 1; gm <= N_XCD; gm *= 2) {
    const int gn = N_XCD / gm, wm = (PM + gm - 1) / gm, wn = (PN + gn - 1) / gn;
    const int c = wm + wn;
    if (c < cost) {
      cost = c;
      best = gm;
    }
  }
  return best;
}

// Wgrads of the experts with >= hot_rows rows (see k_wgrad_hot); in dense mode (the
// shared expert) the one dense operand pair.  Returns hipErrorNotSupported, with
// nothing enqueued, for shapes this core does not tile (the caller then runs the
// 128 x 128 kernel over every expert).
static hipError_t wgrad_hot(const char* name, const GroupInfo& g, const void* A, int lda,
                            const void* B, int ldb, void* out0, void* out1, int M, int N,
                            int half_rows, int hot_rows, hipStream_t s) {
  const bool dense = !g.offsets;
  if ((!dense && !g.counts) || M % big::TILE || N % big::TILE || half_rows % big::TILE ||
      g.E > MOE_MAX_E || hot_rows < 1)
    return hipErrorNotSupported;
  big::WgradArgs p;
  p.counts = dense ? nullptr : g.counts;
  p.offsets = g.offsets;
  p.E = g.E;
  p.hot_rows = hot_rows;
  p.dense_rows = g.dense_rows;
  p.A = (const bf16_t*)A;
  p.B = (const bf16_t*)B;
  p.lda = lda;
  p.ldb = ldb;
  p.out0 = (bf16_t*)out0;
  p.out1 = (bf16_t*)out1;
  p.M = M;
  p.N = N;
  p.half_rows = half_rows;
  const int cus = device_cus();
  const unsigned grid = (unsigned)(cus >= N_XCD ? cus - cus % N_XCD : N_XCD);
  p.PM = M / big::TILE;
  p.PN = N / big::TILE;
  p.GM = xcd_grid_rows(p.PM, p.PN);
  return MOE_LAUNCH(name, s, big::k_wgrad_hot<<<grid, big::NTH, 0, s>>>(p));
}

hipError_t launch_big_wgrad_up_hot(const GroupInfo& g, const void* dZ, const void* X, int H,
                                   int I, void* dwg, void* dwu, int hot_rows, hipStream_t s) {
  return wgrad_hot(g.offsets ? "gemm_wgrad_up_hot" : "gemm_wgrad_up_shared", g, dZ, 2 * I, X, H,
                   dwg, dwu, 2 * I, H, I, hot_rows, s);
}

hipError_t launch_big_wgrad_down_hot(const GroupInfo& g, const void* dYu, const void* gh, int H,
                                     int I, void* dwd, int hot_rows, hipStream_t s) {
  return wgrad_hot(g.offsets ? "gemm_wgrad_down_hot" : "gemm_wgrad_down_shared", g, dYu, H, gh, I,
                   dwd, nullptr, H, I, H, hot_rows, s);
}

// MXFP8 wgrads of the experts whose packed token range has >= hot_bytes bytes
// (k_wgrad_hot_mx), after zeroing the tails of both operands past kpos[E];
// hipErrorNotSupported (nothing enqueued) for shapes the 256-tiles do not cover.
hipError_t launch_mx_wgrad_hot(const char* name, const MbPlans& mp, int E, uint8_t* A8,
                               const uint8_t* As, uint8_t* B8, const uint8_t* Bs, int M, int N,
                               int split, size_t Kp, void* out0, void* out1, int hot_bytes,
                               hipStream_t s) {
  if (M % big::TILE || N % big::TILE || split % big::TILE || E > MOE_MAX_E || hot_bytes < 128 ||
      Kp % 128)
    return hipErrorNotSupported;
  big::MxWgradArgs p;
  p.kpos = mp.kpos;
  p.E = E;
  p.hot_bytes = hot_bytes;
  p.A8 = A8;
  p.As = As;
  p.B8 = B8;
  p.Bs = Bs;
  p.Kp = (long)Kp;
  p.out0 = (bf16_t*)out0;
  p.out1 = (bf16_t*)out1;
  p.M = M;
  p.N = N;
  p.half_rows = split;
  p.PM = M / big::TILE;
  p.PN = N / big::TILE;
  p.GM = xcd_grid_rows(p.PM, p.PN);
  const int cus = device_cus();
  const unsigned grid = (unsigned)(cus >= N_XCD ? cus - cus % N_XCD : N_XCD);
  hipError_t err = MOE_LAUNCH("mx_zero_tail", s,
                              big::mx_zero_tail_kernel<<<(M * 8 + 255) / 256, 256, 0, s>>>(
                                  A8, M, (long)Kp, mp.kpos + E));
  if (err != hipSuccess) return err;
  err = MOE_LAUNCH("mx_zero_tail", s,
                   big::mx_zero_tail_kernel<<<(N * 8 + 255) / 256, 256, 0, s>>>(
                       B8, N, (long)Kp, mp.kpos + E));
  if (err != hipSuccess) return err;
  return MOE_LAUNCH(name, s, big::k_wgrad_hot_mx<<<grid, big::NTH, 0, s>>>(p));
}

}  // namespace moe
