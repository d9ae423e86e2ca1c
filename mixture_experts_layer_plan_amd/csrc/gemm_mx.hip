// MXFP8 grouped expert GEMMs: E4M3 operands with one E8M0 scale per 32 along K,
// on the scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4 (gfx950), fp32 accumulation.
//
// MoK trains in MXFP8 with the format handled inside the kernels (sebask.de,
// "Mixture-of-Kittens: Cursors Open-Source-Ansatz für effizientes MoE-Training auf
// NVL72", § Determinismus und MXFP8-Unterstützung; stamatios.com, "Cursor abre
// código de megakernel MoE para GPUs NVL72", § Outras características).  Every
// operand here is K-major: an E4M3 row of K bytes plus K/32 scale bytes.  The
// operands whose contraction runs over the token axis (the wgrads) are produced
// transposed by the token quantiser, and the weights exist in both orientations,
// so no transposition happens inside these kernels.
//
// Lane layout of the scaled 32x32x64 instruction (established with an in-bounds
// probe): lane i + 32 h holds row i; its bytes 0-15 lie in K block 0 and bytes
// 16-31 in K block 1 of the 64-deep step; the scale of (row i, block c) comes
// from lane i + 32 c.  Here lane (i, h) takes the 16-byte chunks 4 ks + h and
// 4 ks + 2 + h of a 128-byte K tile row (blocks 2 ks and 2 ks + 1), so every
// (lane half, byte) pair names one K index, the same for both operands.
//
// Tiles, LDS layout, swizzle, rasterisation and epilogue staging are those of the
// bf16 GEMMs (gemm_common.hpp) with 128 bytes = 128 fp8 of K per LDS row.  Scale
// words (4 blocks of one row per K tile) go straight from memory into the
// registers of the lanes whose MFMA fragments use them.
#include "gemm_common.hpp"
#include "mx_common.hpp"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
constexpr int MX_BK = 128;  // K bytes per tile row (4 scale blocks)

// One K-major MX operand as seen by one thread: the rows of its loads (rows
// (t >> 3) + 32 s of the tile) as 32-bit byte offsets from wave-uniform bases; the
// same rows' scale bytes sit at offset / 32 from the scale bases (a data row is K
// bytes, its scale row K / 32).  Source 1 replaces source 0 for the rows flagged in
// `sel` (bit s: row s) and for all rows at K >= ksplit (dgrad-up's second weight;
// its bases are then pre-offset by -ksplit so that the same K offset applies).  Rows
// with their bit clear in `ok` load as zeros, and so do the K bytes at or past kend
// (a multiple of 32): their 16-byte chunks are zeroed and their blocks' scale bytes
// set to 0 (2^-127), so no stale scale byte (0xFF is NaN in E8M0) reaches the MFMA.
// klen: bytes of K in a row of source 1 (of source 0 below ksplit), which bounds the
// scale loads.  soff: the scale rows of this lane's two MFMA fragment blocks, for
// the loop that loads their words directly (bits 4 + q of ok flag them valid).
struct MxOp {
  const uint8_t* d[2];   // data bases of source 0 and 1
  const uint8_t* s[2];   // scale bases
  uint32_t off[4];       // data row offsets (bytes)
  uint32_t soff[2];      // fragment scale rows (bytes), direct loads only
  uint32_t sel, ok;
  long ksplit, kend, klen;
};

MOE_DEV void mx_op_clear(MxOp& o) {
  o.d[0] = o.d[1] = nullptr;
  o.s[0] = o.s[1] = nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) o.off[i] = 0;
  o.soff[0] = o.soff[1] = 0;
  o.sel = 0;
  o.ok = 0x3fu;
  o.ksplit = 1L << 62;
  o.kend = 1L << 62;
  o.klen = 0;
}

// Data loads through buffer resources over 2 GiB from each source base: the source of
// row q (sel bit q, the same in every lane, or the second source from ksplit on) is
// a scalar choice, and rows outside the operand (ok) or K bytes at or past kend take
// an offset past the range, which loads zeros (MI355X: buffer loads issue faster than
// 64-bit per-lane addresses; the 256 x 256 core's direct-to-LDS loads went 229 -> 201
// us on a dense product).  Every source's offsets stay below 2 GiB.
constexpr uint32_t MX_RANGE = 0x80000000u;
MOE_DEV void mx_load(const MxOp& o, long koff, uint4 (&r)[4]) {
  const bool hi = koff >= o.ksplit;
  const int ch = (threadIdx.x & 7) * 16;
  const bool kin = koff + ch < o.kend;
  const uint32_t sel = __builtin_amdgcn_readfirstlane(o.sel);
  const rsrc_t r0 = make_rsrc(o.d[0], MX_RANGE), r1 = make_rsrc(o.d[1], MX_RANGE);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t voff = ((o.ok >> q) & 1u) && kin ? o.off[q] + (uint32_t)ch : MX_RANGE;
    r[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                         (hi || ((sel >> q) & 1u)) ? r1 : r0, voff,
                                         (uint32_t)koff, 0));
  }
}

// Scale words through the LDS.  A group is MX_SG K tiles: word j (tile j of the
// group, four blocks) of each of the 256 tile rows (A rows 0..127, B rows 128..255)
// at 4 (256 j + row) of a group buffer.  Thread t loads, in the tile of part p of the
// current group, word t & 7 of row (t >> 3) + 32 (p & 3) of A (p < 4) or B of the
// next group, and stores it after the tile's wait; eight threads then cover a
// row's 32 contiguous scale bytes.  Loading the words of the MFMA fragments' rows
// directly (four loads per lane per tile, each touching 32 rows' cache lines) cost
// about a quarter of these kernels' time.
constexpr int MX_SG = 8;
constexpr int MX_SGB = MX_SG * 256 * 4;
constexpr int MX_LDS = LDS_BYTES + 2 * MX_SGB;

// this thread's word of row s of operand o at K offset kw; 0 for rows outside the
// tile; K offsets past the operand read an unused word inside the row
template <int S>
MOE_DEV uint32_t mx_sword_of(const MxOp& o, long kw) {
  const bool hi = kw >= o.ksplit;
  const long lim = (hi ? o.klen : min(o.ksplit, o.klen)) - MX_BK;
  if (kw > lim) kw = lim;
  // the source as a uniform byte distance from source 0 (selecting between the two
  // 64-bit bases per lane kept both in registers and spilled them)
  const long delta = (long)((uintptr_t)o.s[1] - (uintptr_t)o.s[0]);
  const bool one = hi || ((o.sel >> S) & 1u);
  const uint8_t* p = o.s[0] + (one ? delta : 0L) + (o.off[S] >> 5) + kw / 32;
  return ((o.ok >> S) & 1u) ? *(const uint32_t*)p : 0u;
}

// the word of part p (row p & 3 of A for p < 4, of B after); p is the same for the
// whole workgroup, and the branches keep every register index a constant (a
// runtime index into the row offsets put them in scratch memory)
MOE_DEV uint32_t mx_sword(const MxOp& A, const MxOp& B, int p, long kw) {
  switch (p) {
    case 0: return mx_sword_of<0>(A, kw);
    case 1: return mx_sword_of<1>(A, kw);
    case 2: return mx_sword_of<2>(A, kw);
    case 3: return mx_sword_of<3>(A, kw);
    case 4: return mx_sword_of<0>(B, kw);
    case 5: return mx_sword_of<1>(B, kw);
    case 6: return mx_sword_of<2>(B, kw);
    default: return mx_sword_of<3>(B, kw);
  }
}

MOE_DEV void mx_sput(char* buf, int p, uint32_t w) {
  const int t = threadIdx.x;
  *(uint32_t*)(buf + 4 * (256 * (t & 7) + (t >> 3) + 32 * (p & 3) + (p >= 4 ? 128 : 0))) = w;
}

// the direct form: this lane's words of its fragment rows at K offset koff, blocks
// at or past kend zero (single-source operands)
MOE_DEV void mx_load_words(const MxOp& o, long koff, uint32_t (&sw)[2]) {
  const long nb = (o.kend - koff) / 32;
  const uint32_t keep = nb >= 4 ? 0xffffffffu : (nb <= 0 ? 0u : (1u << (8 * nb)) - 1u);
#pragma unroll
  for (int q = 0; q < 2; ++q)
    sw[q] = ((o.ok >> (4 + q)) & 1u) ? *(const uint32_t*)(o.s[0] + o.soff[q] + koff / 32) & keep
                                     : 0u;
}

MOE_DEV void mx_store(char* t, const uint4 (&r)[4]) {
  const int row = threadIdx.x >> 3, ch = threadIdx.x & 7;
#pragma unroll
  for (int s = 0; s < 4; ++s) *(uint4*)(t + swz(row + 32 * s, ch)) = r[s];
}

MOE_DEV i32x8_t mx_frag(const char* t, int row, int c0, int c1) {
  const uint4 a = *(const uint4*)(t + swz(row, c0));
  const uint4 b = *(const uint4*)(t + swz(row, c1));
  i32x8_t v;
  v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
  v[4] = (int)b.x; v[5] = (int)b.y; v[6] = (int)b.z; v[7] = (int)b.w;
  return v;
}

MOE_DEV void mma_tile_mx(const char* ta, const char* tb, const uint32_t (&sa)[2],
                         const uint32_t (&sb)[2], f32x16_t (&acc)[2][2], int arow,
                         const int (&brow)[2], int lane) {
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int c0 = 4 * ks + h, c1 = 4 * ks + 2 + h, sh = 8 * (2 * ks + h);
    const i32x8_t a0 = mx_frag(ta, arow + r, c0, c1);
    const i32x8_t a1 = mx_frag(ta, arow + 32 + r, c0, c1);
    const i32x8_t b0 = mx_frag(tb, brow[0] + r, c0, c1);
    const i32x8_t b1 = mx_frag(tb, brow[1] + r, c0, c1);
    const int s_a0 = (int)((sa[0] >> sh) & 0xffu), s_a1 = (int)((sa[1] >> sh) & 0xffu);
    const int s_b0 = (int)((sb[0] >> sh) & 0xffu), s_b1 = (int)((sb[1] >> sh) & 0xffu);
    acc[0][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, acc[0][0], 0, 0, 0, s_a0, 0, s_b0);
    acc[0][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b1, acc[0][1], 0, 0, 0, s_a0, 0, s_b1);
    acc[1][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b0, acc[1][0], 0, 0, 0, s_a1, 0, s_b0);
    acc[1][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, acc[1][1], 0, 0, 0, s_a1, 0, s_b1);
  }
}

// K offset (bytes) of K tile kt in a plain operand
struct KLinear {
  MOE_DEV long operator()(int kt) const { return (long)kt * MX_BK; }
};

// Main loop: two LDS stages and one register stage (tile kt + 1 is loaded while
// tile kt is multiplied), and two scale group buffers after the stages (group G,
// tiles 8 G .. 8 G + 7, read from buffer G mod 2 and written during the tiles of
// group G - 1; the words of tiles past the last one are loaded but unused).  `lds`
// holds MX_LDS bytes.  The weight gradients' K loops are short (an expert's tokens,
// mostly one or two tiles), where a group load costs more than it saves: they load
// each tile's words for the fragment rows directly (LDS_SCALES = false; `lds` then
// holds LDS_BYTES).
template <bool LDS_SCALES = true, class KM>
MOE_DEV void gemm_main_mx(char* lds, const MxOp& A, const MxOp& B, const KM& km, int nk,
                          f32x16_t (&acc)[2][2], int arow, const int (&brow)[2], int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  if (nk <= 0) return;
  if constexpr (!LDS_SCALES) {
    uint4 ra[4], rb[4];
    uint32_t sa[2], sb[2], ca[2], cb[2];
    mx_load(A, km(0), ra);
    mx_load(B, km(0), rb);
    mx_load_words(A, km(0), ca);
    mx_load_words(B, km(0), cb);
    mx_store(lds, ra);
    mx_store(lds + TILEB, rb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      char* cur = lds + (kt & 1) * 2 * TILEB;
      char* nxt = lds + ((kt + 1) & 1) * 2 * TILEB;
      const bool more = kt + 1 < nk;
      if (more) {
        mx_load(A, km(kt + 1), ra);
        mx_load(B, km(kt + 1), rb);
        mx_load_words(A, km(kt + 1), sa);
        mx_load_words(B, km(kt + 1), sb);
      }
      mma_tile_mx(cur, cur + TILEB, ca, cb, acc, arow, brow, lane);
      if (more) {
        mx_store(nxt, ra);
        mx_store(nxt + TILEB, rb);
        ca[0] = sa[0]; ca[1] = sa[1]; cb[0] = sb[0]; cb[1] = sb[1];
      }
      __syncthreads();
    }
    return;
  }
  char* const sg = lds + LDS_BYTES;
  const int tj = threadIdx.x & 7, l = lane & 31;
  uint4 ra[4], rb[4];
  mx_load(A, km(0), ra);
  mx_load(B, km(0), rb);
  uint32_t w0[MX_SG];  // group 0; only the words of tiles that exist (short K loops)
#pragma unroll
  for (int p = 0; p < MX_SG; ++p) w0[p] = tj < nk ? mx_sword(A, B, p, km(tj)) : 0u;
  mx_store(lds, ra);
  mx_store(lds + TILEB, rb);
#pragma unroll
  for (int p = 0; p < MX_SG; ++p) mx_sput(sg, p, w0[p]);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = lds + (kt & 1) * 2 * TILEB;
    char* nxt = lds + ((kt + 1) & 1) * 2 * TILEB;
    const bool more = kt + 1 < nk;
    if (more) {
      mx_load(A, km(kt + 1), ra);
      mx_load(B, km(kt + 1), rb);
    }
    const int p = kt & 7, g1 = (kt >> 3) + 1;
    const bool next = MX_SG * g1 < nk;  // a next group exists
    const uint32_t w = next ? mx_sword(A, B, p, km(MX_SG * g1 + tj)) : 0u;
    // this lane's words of tile kt: fragment rows arow + 32 q + l (A), brow[q] + l (B);
    // blocks at or past kend zero
    const char* gb = sg + ((kt >> 3) & 1) * MX_SGB + 4 * 256 * p;
    const long nb = (A.kend - km(kt)) / 32;
    const uint32_t keep = nb >= 4 ? 0xffffffffu : (nb <= 0 ? 0u : (1u << (8 * nb)) - 1u);
    uint32_t ca[2], cb[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      ca[q] = *(const uint32_t*)(gb + 4 * (arow + 32 * q + l)) & keep;
      cb[q] = *(const uint32_t*)(gb + 4 * (128 + brow[q] + l)) & keep;
    }
    mma_tile_mx(cur, cur + TILEB, ca, cb, acc, arow, brow, lane);
    if (more) {
      mx_store(nxt, ra);
      mx_store(nxt + TILEB, rb);
    }
    if (next) mx_sput(sg + (g1 & 1) * MX_SGB, p, w);  // never the buffer being read
    __syncthreads();
  }
}

// Row-quantise 8 consecutive values held by each of 4 neighbouring lanes (one
// 32-block): amax over the 4 lanes, codes to q (8 bytes), the scale from the
// first lane of the group.  Every lane of the wavefront must call this.
MOE_DEV void quant8_group4(const float* v, bool ok, uint8_t* q, uint8_t* sc, bool first) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int X = mx_exp_of_amax(amax);
  if (ok) {
    *(uint2*)q = mx_encode8(v, X);
    if (first) *sc = (uint8_t)(X + 127);
  }
}

// ------------------------------------------------------------------ kernels
// GEMM1 + SwiGLU, MX: A = X8 rows (dispatched, quantised along H), B = W_g / W_u
// quantised along H.  Epilogue: Z = (A | B) fp32, h = silu(A) B quantised along I.
__global__ __launch_bounds__(NTHR, 2) void k_up_swiglu_mx(
    GroupInfo g, const uint8_t* __restrict__ X8, const uint8_t* __restrict__ Xs,
    const uint8_t* __restrict__ wg8, const uint8_t* __restrict__ wgs,
    const uint8_t* __restrict__ wu8, const uint8_t* __restrict__ wus, int H, int I,
    float* __restrict__ Z, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  __shared__ __attribute__((aligned(16))) char lds[MX_LDS];
  RowTile t;
  int nt;
  if (!rows_tile(g, I / 64, t, nt)) return;
  const int i0 = nt * 64, lane = threadIdx.x & 63, HS = H / 32;
  int arow, brow[2];
  wave_coords(arow, brow, true);
  MxOp A, B;
  mx_op_clear(A);
  mx_op_clear(B);
  const size_t we = (size_t)t.e * I + i0;  // first weight row of this column tile
  A.d[0] = X8;
  A.s[0] = Xs;
  B.d[0] = wg8 + we * H;
  B.d[1] = wu8 + we * H;
  B.s[0] = wgs + we * HS;
  B.s[1] = wus + we * HS;
  A.ok = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int rr = (threadIdx.x >> 3) + 32 * s, r = t.row0 + rr;
    const bool ok = r < t.row_end;
    A.ok |= (uint32_t)ok << s;
    A.off[s] = (uint32_t)((ok ? r : t.row0) * H);
    B.off[s] = (uint32_t)((rr & 63) * H);
    B.sel |= (uint32_t)(rr >= 64) << s;
  }
  f32x16_t acc[2][2];
  A.klen = B.klen = H;
  gemm_main_mx(lds, A, B, KLinear(), H / MX_BK, acc, arow, brow, lane);
  float* C = (float*)lds;
  stage_acc(C, acc, arow, brow, lane);
  __syncthreads();
  const int nrows = t.row_end - t.row0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int r = (threadIdx.x >> 3) + 32 * s, c = threadIdx.x & 7;
    const bool ok = r < nrows;
    float a[8], b[8], h[8];
    read8(C, r, 8 * c, a);
    read8(C, r, 64 + 8 * c, b);
#pragma unroll
    for (int q = 0; q < 8; ++q) h[q] = ok ? silu_f(a[q]) * b[q] : 0.0f;
    const size_t row = (size_t)(t.row0 + r);
    if (ok) {
      float* zr = Z + row * (2 * I);
      store8(zr + i0 + 8 * c, a);
      store8(zr + I + i0 + 8 * c, b);
    }
    quant8_group4(h, ok, hq + row * I + i0 + 8 * c, hs + row * (I / 32) + (i0 + 8 * c) / 32,
                  (c & 3) == 0);
  }
}

// GEMM2, MX: Y = Q_I(h) Q_I(W_d)^T, Y in bf16.
__global__ __launch_bounds__(NTHR, 2) void k_down_mx(GroupInfo g, const uint8_t* __restrict__ hq,
                                                     const uint8_t* __restrict__ hs,
                                                     const uint8_t* __restrict__ wd8,
                                                     const uint8_t* __restrict__ wds, int H, int I,
                                                     bf16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) char lds[MX_LDS];
  RowTile t;
  int nt;
  if (!rows_tile(g, H / TN, t, nt)) return;
  const int n0 = nt * TN, lane = threadIdx.x & 63, IS = I / 32;
  int arow, brow[2];
  wave_coords(arow, brow, false);
  MxOp A, B;
  mx_op_clear(A);
  mx_op_clear(B);
  const size_t we = (size_t)t.e * H + n0;
  A.d[0] = hq;
  A.s[0] = hs;
  B.d[0] = wd8 + we * I;
  B.s[0] = wds + we * IS;
  A.ok = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int rr = (threadIdx.x >> 3) + 32 * s, r = t.row0 + rr;
    const bool ok = r < t.row_end;
    A.ok |= (uint32_t)ok << s;
    A.off[s] = (uint32_t)((ok ? r : t.row0) * I);
    B.off[s] = (uint32_t)(rr * I);
  }
  f32x16_t acc[2][2];
  A.klen = B.klen = I;
  gemm_main_mx(lds, A, B, KLinear(), I / MX_BK, acc, arow, brow, lane);
  float* C = (float*)lds;
  stage_acc(C, acc, arow, brow, lane);
  __syncthreads();
  auto out = [&](int r) { return Y + (size_t)(t.row0 + r) * H + n0; };
  epi_store<bf16_t>(C, out, t.row_end - t.row0);
}

// dgrad-down, MX: dh' = Q_H(dYu) Q_H(W_d) with W_d stored transposed [E, I, H];
// epilogue as the bf16 kernel (SwiGLU backward from fp32 Z, router-weight
// gradient partials) writing dZ = (dA | dB) and g h in fp32 for the token
// quantiser, plus dZ quantised along 2I for dgrad-up.
__global__ __launch_bounds__(NTHR, 2) void k_dgrad_down_mx(
    GroupInfo g, const uint8_t* __restrict__ dYu8, const uint8_t* __restrict__ dYus,
    const uint8_t* __restrict__ wdT8, const uint8_t* __restrict__ wdTs,
    const float* __restrict__ Z, const float* __restrict__ topk_w, int H, int I, int k,
    float* __restrict__ dZ, uint8_t* __restrict__ dZ8, uint8_t* __restrict__ dZs,
    float* __restrict__ gh, float* __restrict__ dgp) {
  __shared__ __attribute__((aligned(16))) char lds[MX_LDS];
  RowTile t;
  int nt;
  if (!rows_tile(g, I / TN, t, nt)) return;
  const int i0 = nt * TN, lane = threadIdx.x & 63, HS = H / 32;
  int arow, brow[2];
  wave_coords(arow, brow, false);
  MxOp A, B;
  mx_op_clear(A);
  mx_op_clear(B);
  const size_t we = (size_t)t.e * I + i0;
  A.d[0] = dYu8;
  A.s[0] = dYus;
  B.d[0] = wdT8 + we * H;
  B.s[0] = wdTs + we * HS;
  A.ok = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int rr = (threadIdx.x >> 3) + 32 * s, r = t.row0 + rr;
    const bool ok = r < t.row_end;
    A.ok |= (uint32_t)ok << s;
    A.off[s] = (uint32_t)((ok ? r : t.row0) * H);
    B.off[s] = (uint32_t)(rr * H);
  }
  f32x16_t acc[2][2];
  A.klen = B.klen = H;
  gemm_main_mx(lds, A, B, KLinear(), H / MX_BK, acc, arow, brow, lane);
  float* C = (float*)lds;
  stage_acc(C, acc, arow, brow, lane);
  __syncthreads();
  const int nrows = t.row_end - t.row0, n_parts = I / TN, S2 = (2 * I) / 32;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int r = (threadIdx.x >> 4) + 16 * s, c = threadIdx.x & 15;
    const bool ok = r < nrows;
    const int row = t.row0 + r;
    float part = 0.0f;
    float da[8], db[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) da[q] = db[q] = 0.0f;
    if (ok) {
      const float gate = topk_w[(size_t)g.src_token[row] * k + g.src_slot[row]];
      float d[8], a[8], b[8], gh8[8];
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
      float* dzr = dZ + (size_t)row * (2 * I);
      store8(dzr + i0 + 8 * c, da);
      store8(dzr + I + i0 + 8 * c, db);
      store8(gh + (size_t)row * I + i0 + 8 * c, gh8);
    }
    const size_t qr = (size_t)(ok ? row : 0);
    quant8_group4(da, ok, dZ8 + qr * (2 * I) + i0 + 8 * c, dZs + qr * S2 + (i0 + 8 * c) / 32,
                  (c & 3) == 0);
    quant8_group4(db, ok, dZ8 + qr * (2 * I) + I + i0 + 8 * c,
                  dZs + qr * S2 + (I + i0 + 8 * c) / 32, (c & 3) == 0);
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
    if (ok && c == 0) dgp[(size_t)row * n_parts + nt] = part;
  }
}

// dgrad-up, MX: dX = Q_2I(dZ) [Q_I(W_g); Q_I(W_u)] with the weights stored
// transposed [E, H, I]: B row h takes W_g^T[e][h] for K < I and W_u^T[e][h] after.
__global__ __launch_bounds__(NTHR, 2) void k_dgrad_up_mx(
    GroupInfo g, const uint8_t* __restrict__ dZ8, const uint8_t* __restrict__ dZs,
    const uint8_t* __restrict__ wgT8, const uint8_t* __restrict__ wgTs,
    const uint8_t* __restrict__ wuT8, const uint8_t* __restrict__ wuTs, int H, int I,
    bf16_t* __restrict__ dX) {
  __shared__ __attribute__((aligned(16))) char lds[MX_LDS];
  RowTile t;
  int nt;
  if (!rows_tile(g, H / TN, t, nt)) return;
  const int n0 = nt * TN, lane = threadIdx.x & 63, IS = I / 32;
  int arow, brow[2];
  wave_coords(arow, brow, false);
  MxOp A, B;
  mx_op_clear(A);
  mx_op_clear(B);
  const size_t we = (size_t)t.e * H + n0;
  A.d[0] = dZ8;
  A.s[0] = dZs;
  B.ksplit = I;
  B.d[0] = wgT8 + we * I;
  B.d[1] = wuT8 + we * I - I;
  B.s[0] = wgTs + we * IS;
  B.s[1] = wuTs + we * IS - IS;
  A.ok = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int rr = (threadIdx.x >> 3) + 32 * s, r = t.row0 + rr;
    const bool ok = r < t.row_end;
    A.ok |= (uint32_t)ok << s;
    A.off[s] = (uint32_t)((ok ? r : t.row0) * (2 * I));
    B.off[s] = (uint32_t)(rr * I);
  }
  f32x16_t acc[2][2];
  A.klen = B.klen = 2 * I;
  gemm_main_mx(lds, A, B, KLinear(), (2 * I) / MX_BK, acc, arow, brow, lane);
  float* C = (float*)lds;
  stage_acc(C, acc, arow, brow, lane);
  __syncthreads();
  auto out = [&](int r) { return dX + (size_t)(t.row0 + r) * H + n0; };
  epi_store<bf16_t>(C, out, t.row_end - t.row0);
}

// K tiles of one expert in the tile-padded token axis of all minibatches: tile j
// of expert e in minibatch m sits at K offset (m * max_tiles + first_m[e] + j) * 128.
// K offset (bytes) of K tile kt in an expert's region of the token axis
// Work items per workgroup of the MXFP8 wgrad remainder.  One item per workgroup left
// each item paying a workgroup's launch and set-up (≈ 460 K workgroups for wgrad-up at
// T = 8192): 3.53 -> 3.18 ms (up), 1.86 -> 1.65 ms (down) with four; 8, 16 and a
// persistent grid measured the same as four.
constexpr int MXW_ITEMS = 4;

struct KFrom {
  long k0;
  MOE_DEV long operator()(int kt) const { return k0 + (long)kt * MX_BK; }
};

// wgrad, MX: out[e][m, n] = sum over the expert's columns [kpos[e], kpos[e + 1]) of
// the token axis of Q_t(A)[m, k] Q_t(B)[n, k]; A [M, Kp], B [N, Kp] (Kp: the axis
// length).  The last K tile's bytes past the expert's columns load as zeros.
// Each workgroup takes MXW_ITEMS consecutive (expert, output tile) items; experts
// without rows in any minibatch get zero tiles.  Output rows m < split go to out0[e], the rest to out1[e] (dW_g /
// dW_u); split = M for one.
__global__ __launch_bounds__(NTHR, 2) void k_wgrad_mx(MbPlans mp, int E, bool m_fast,
                                                      const uint8_t* __restrict__ A8,
                                                      const uint8_t* __restrict__ As,
                                                      const uint8_t* __restrict__ B8,
                                                      const uint8_t* __restrict__ Bs, int M, int N,
                                                      int split, long Kp,
                                                      bf16_t* __restrict__ out0,
                                                      bf16_t* __restrict__ out1, int hot_bytes) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int MT = M / TM, NT = N / TN, lane = threadIdx.x & 63;
  const long KS = Kp / 32;
  // one workgroup per (expert, tile) over all E experts, in id order and spread over
  // the XCDs round-robin; the tiles of an expert with no row in any minibatch (an
  // empty run of the token axis) are stored as zeros; the experts whose range has
  // >= hot_bytes bytes belong to the large-tile kernel (a persistent form of this
  // loop spilled 68 registers and measured slower)
  int arow, brow[2];
  wave_coords(arow, brow, false);
#pragma unroll 1
  for (int it = 0; it < MXW_ITEMS; ++it) {
  const int id = blockIdx.x * MXW_ITEMS + it;
  if (id >= E * MT * NT) break;
  const int e = id / (MT * NT), rem = id - e * (MT * NT);
  // the tile index along H runs fastest (M for wgrad-down, N for wgrad-up)
  const int mt = m_fast ? rem % MT : rem / NT, nt = m_fast ? rem / MT : rem % NT;
  const int m0 = mt * TM, n0 = nt * TN;
  bf16_t* base = (m0 < split ? out0 + (size_t)e * split * N + (size_t)m0 * N
                             : out1 + (size_t)e * (M - split) * N + (size_t)(m0 - split) * N) + n0;
  if (ld_uniform(mp.kpos + e + 1) == ld_uniform(mp.kpos + e)) {
    const int mg = m0 < split ? m0 : m0 - split;  // row tile within its output block
    zero_span<bf16_t>((m0 < split ? out0 + (size_t)e * split * N
                                  : out1 + (size_t)e * (M - split) * N) +
                      ((size_t)(mg / TM) * NT + nt) * (TM * TN));
    continue;
  }
  const KFrom km{ld_uniform(mp.kpos + e)};
  const long kend = ld_uniform(mp.kpos + e + 1);
  if (hot_bytes > 0 && kend - km.k0 >= hot_bytes) continue;
  const int nk = (int)((kend - km.k0 + MX_BK - 1) / MX_BK);
  MxOp oa, ob;
  mx_op_clear(oa);
  mx_op_clear(ob);
  oa.kend = ob.kend = kend;
  oa.d[0] = A8 + (size_t)m0 * Kp;
  ob.d[0] = B8 + (size_t)n0 * Kp;
  oa.s[0] = As + (size_t)m0 * KS;
  ob.s[0] = Bs + (size_t)n0 * KS;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int rr = (threadIdx.x >> 3) + 32 * s;
    oa.off[s] = ob.off[s] = (uint32_t)(rr * Kp);
  }
  f32x16_t acc[2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    oa.soff[q] = (uint32_t)((arow + 32 * q + (lane & 31)) * KS);
    ob.soff[q] = (uint32_t)((brow[q] + (lane & 31)) * KS);
  }
  gemm_main_mx<false>(lds, oa, ob, km, nk, acc, arow, brow, lane);
  float* C = (float*)lds;
  // the staging addresses are made opaque per item: otherwise their 64 offsets are
  // computed once before the item loop and held across it (spilled)
  int sr = arow, sb[2] = {brow[0], brow[1]};
  asm volatile("" : "+v"(sr), "+v"(sb[0]), "+v"(sb[1]));
  stage_acc(C, acc, sr, sb, lane);
  __syncthreads();
  auto out = [&](int r) { return base + (size_t)r * N; };
  epi_store<bf16_t, true>(C, out, TM);
  __syncthreads();  // the staged tile is read; the LDS is free for the next item
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_mx_up_swiglu(const GroupInfo& g, const uint8_t* X8, const uint8_t* Xs,
                               const uint8_t* wg8, const uint8_t* wgs, const uint8_t* wu8,
                               const uint8_t* wus, int H, int I, float* Z, uint8_t* hq,
                               uint8_t* hs, hipStream_t s) {
  const unsigned ty = (unsigned)g.max_tiles;
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH("mx_gemm_up_swiglu", s,
                    k_up_swiglu_mx<<<ty * (I / 64), NTHR, 0, s>>>(g, X8, Xs, wg8, wgs, wu8, wus, H,
                                                                  I, Z, hq, hs));
}

hipError_t launch_mx_down(const GroupInfo& g, const uint8_t* hq, const uint8_t* hs,
                          const uint8_t* wd8, const uint8_t* wds, int H, int I, void* Y,
                          hipStream_t s) {
  const hipError_t e = launch_big_mx_down(g, hq, hs, wd8, wds, H, I, Y, s);
  if (e != hipErrorNotSupported) return e;
  const unsigned ty = (unsigned)g.max_tiles;
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH("mx_gemm_down", s,
                    k_down_mx<<<ty * (H / TN), NTHR, 0, s>>>(g, hq, hs, wd8, wds, H, I,
                                                             (bf16_t*)Y));
}

hipError_t launch_mx_dgrad_down(const GroupInfo& g, const uint8_t* dYu8, const uint8_t* dYus,
                                const uint8_t* wdT8, const uint8_t* wdTs, const float* Z,
                                const float* topk_w, int H, int I, int k, void* dZ, uint8_t* dZ8,
                                uint8_t* dZs, void* gh, float* dgp, hipStream_t s) {
  const unsigned ty = (unsigned)g.max_tiles;
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH("mx_gemm_dgrad_down", s,
                    k_dgrad_down_mx<<<ty * (I / TN), NTHR, 0, s>>>(
                        g, dYu8, dYus, wdT8, wdTs, Z, topk_w, H, I, k, (float*)dZ, dZ8, dZs,
                        (float*)gh, dgp));
}

hipError_t launch_mx_dgrad_up(const GroupInfo& g, const uint8_t* dZ8, const uint8_t* dZs,
                              const uint8_t* wgT8, const uint8_t* wgTs, const uint8_t* wuT8,
                              const uint8_t* wuTs, int H, int I, void* dX, hipStream_t s) {
  const hipError_t e = launch_big_mx_dgrad_up(g, dZ8, dZs, wgT8, wgTs, wuT8, wuTs, H, I, dX, s);
  if (e != hipErrorNotSupported) return e;
  const unsigned ty = (unsigned)g.max_tiles;
  if (ty == 0) return hipSuccess;
  return MOE_LAUNCH("mx_gemm_dgrad_up", s,
                    k_dgrad_up_mx<<<ty * (H / TN), NTHR, 0, s>>>(g, dZ8, dZs, wgT8, wgTs, wuT8,
                                                                 wuTs, H, I, (bf16_t*)dX));
}

hipError_t launch_mx_wgrad(const char* name, const MbPlans& mp, int E, const uint8_t* A8,
                           const uint8_t* As, const uint8_t* B8, const uint8_t* Bs, int M, int N,
                           int split, size_t Kp, void* out0, void* out1, int hot_bytes,
                           hipStream_t s) {
  const unsigned grid = (unsigned)(((long)E * (M / TM) * (N / TN) + MXW_ITEMS - 1) / MXW_ITEMS);
  // one output (split == M) is wgrad-down, whose M runs along H
  return MOE_LAUNCH(name, s,
                    k_wgrad_mx<<<grid, NTHR, 0, s>>>(mp, E, split == M, A8, As, B8, Bs, M, N,
                                                     split, (long)Kp, (bf16_t*)out0,
                                                     (bf16_t*)out1, hot_bytes));
}

}  // namespace moe
