// Building blocks of the grouped MFMA GEMMs (bf16/fp32 in gemm.hip, MXFP8 in
// gemm_mx.hip): LDS tile layout and swizzle, operand loaders, the pipelined main
// loop, accumulator staging, tile rasterisation.  See gemm.hip for the design.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int TM = 128, TN = 128, NTHR = 256;
constexpr int ROWB = 128;            // bytes per LDS operand row
constexpr int TILEB = 128 * ROWB;    // one operand tile: 16 KiB
constexpr int LDS_BYTES = 4 * TILEB; // 2 buffers x (A, B) = 64 KiB = the staged C tile

template <typename T> struct Tr;
template <> struct Tr<bf16_t> { static constexpr int BK = 64, VEC = 8; };
template <> struct Tr<float> { static constexpr int BK = 32, VEC = 4; };

// byte offset of 16-byte chunk `chunk` of operand row `row`
MOE_DEV int swz(int row, int chunk) { return row * ROWB + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4); }

// float offset of element (row, col) in the staged 128 x 128 fp32 C tile
MOE_DEV int cidx(int row, int col) { return row * 128 + ((((col >> 3) ^ (row & 15))) << 3) + (col & 7); }

MOE_DEV uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Direct-to-LDS loads through a buffer resource (buffer_load_dwordx4 ... lds: lane L's
// 16 bytes land at the wavefront's LDS base + 16 L): the operand's wave-uniform base
// in scalar registers, a 32-bit per-lane offset and a wave-uniform scalar offset.
// Measured on MI355X against the global_load_lds form with a 64-bit address per lane,
// on the 256 x 256 core's K loop over a dense 4096 x 4096 x 7168 bf16 product: 229 ->
// 201 us (8192 x 4096 x 7168: 467 -> 414 us), with half the address-unit stall
// cycles.  `bytes` is the range from the base: a load at or past it returns zeros
// (default: 4 GiB, i.e. no clamping of the 32-bit offsets).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
MOE_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes = 0xffffffffu) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// AUX: cache policy (0; or 16 = sc1, coherent at device scope)
template <int AUX = 0>
MOE_DEV void dma16_buf(rsrc_t r, uint32_t voff, uint32_t soff, char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff,
                                          soff, 0, AUX);
}

// ------------------------------------------------------------------ loaders
// K-major operand: thread t loads chunk (t & 7) of tile rows (t >> 3) + 32 s; a
// row outside the operand (rp = nullptr) loads as zeros.  (Measured on MI355X:
// this branchy form beats a branch-free load-and-select, whose extra loads of
// padding rows and re-reads of the last K tile cost more than the conservative
// wait the branches cause.)
template <typename T>
struct KLoad {
  static constexpr bool kmajor = true;  // LDS tile is K-major (rows of K)
  const T* rp[4];
  MOE_DEV void set(int s, const T* p, bool valid) { rp[s] = valid ? p : nullptr; }
  MOE_DEV void load(int kt, uint4 (&r)[4]) const {
    const int k = kt * Tr<T>::BK + (threadIdx.x & 7) * Tr<T>::VEC;
#pragma unroll
    for (int s = 0; s < 4; ++s) r[s] = rp[s] ? *(const uint4*)(rp[s] + k) : zero4();
  }
  MOE_DEV void store(char* t, const uint4 (&r)[4]) const {
    const int row = threadIdx.x >> 3, ch = threadIdx.x & 7;
#pragma unroll
    for (int s = 0; s < 4; ++s) *(uint4*)(t + swz(row + 32 * s, ch)) = r[s];
  }
};

// Swizzle of the MN-major bf16 LDS tile (64 K rows x 128 columns, 256 bytes per K
// row): 16-byte chunk c of K row k sits at k * 256 + 16 (c ^ mn_swz(k)).  One
// transposing fragment read touches eight K rows (four consecutive, then four
// more 8 rows down) x four consecutive chunks; the swizzle gives each of the four
// rows a different group of four bank-chunks and the other four rows the
// complementary order, so the read needs the minimum two LDS cycles.
MOE_DEV int mn_swz(int k) { return ((k & 3) << 2) | ((k >> 3) & 1); }

// MN-major operand: element (k, i) of the tile at kr(k)[i]; kr returns nullptr
// for K rows outside the operand (they load as zeros).
// bf16: thread t owns k = 4 (t >> 4) .. +3, i = 8 (t & 15) .. +7, stored as it
//       lies in memory (MN-major LDS tile, read back by transposing LDS reads).
// fp32: thread t owns k = 4 (t >> 5) .. +3, i = 4 (t & 31) .. +3, transposed in
//       registers into the K-major tile (there is no 32-bit transposing read).
template <typename T, class KR>
struct MNLoad {
  static constexpr bool kmajor = sizeof(T) != 2;
  KR kr;
  static constexpr int IB = 128 / Tr<T>::VEC;  // i-blocks per row of 128
  MOE_DEV void load(int kt, uint4 (&r)[4]) const {
    const int kb = threadIdx.x / IB, ib = threadIdx.x % IB;
    const int k0 = kt * Tr<T>::BK + 4 * kb;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const T* p = kr(k0 + kk);
      r[kk] = p ? *(const uint4*)(p + ib * Tr<T>::VEC) : zero4();
    }
  }
  MOE_DEV void store(char* t, const uint4 (&r)[4]) const;
};

MOE_DEV uint32_t u4_word(const uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

template <typename T, class KR>
MOE_DEV void MNLoad<T, KR>::store(char* t, const uint4 (&r)[4]) const {
  const int kb = threadIdx.x / IB, ib = threadIdx.x % IB;
  if constexpr (sizeof(T) == 2) {
    // K rows 4 kb .. +3, chunk ib of each, as stored in memory
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int k = 4 * kb + kk;
      *(uint4*)(t + k * 256 + ((ib ^ mn_swz(k)) << 4)) = r[kk];
    }
  } else {
    // 4 k x 4 i fp32 -> 4 rows (i) of 4 k values (16 bytes)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = ib * 4 + i;
      *(uint4*)(t + swz(row, kb)) =
          make_uint4(u4_word(r[0], i), u4_word(r[1], i), u4_word(r[2], i), u4_word(r[3], i));
    }
  }
}

// MN-major operand over the K rows 0 .. n-1 of a row-major matrix whose row 0 is at
// base (row stride ld elements), columns c0 .. c0 + 127 (base points at column c0):
// the K-grouped operands of the wgrads (an expert's segment of rows).  Addresses are
// the wave-uniform row base of K tile kt plus a 32-bit per-thread offset, and a row
// is valid below one per-thread limit: no per-row pointers or branches on them.
// Same thread-to-element map and LDS layout as MNLoad.
template <typename T>
struct MNSeg {
  static constexpr bool kmajor = sizeof(T) != 2;
  static constexpr int IB = 128 / Tr<T>::VEC;
  const T* base;
  size_t ld;
  int n;         // valid K rows
  uint32_t off;  // element offset of this thread's first row and column group
  int k4;        // this thread's first K row within a tile
  MOE_DEV void set(const T* b, size_t ld_elems, int rows) {
    base = b;
    ld = ld_elems;
    n = rows;
    const int kb = threadIdx.x / IB, ib = threadIdx.x % IB;
    k4 = 4 * kb;
    off = (uint32_t)(k4 * ld_elems + ib * Tr<T>::VEC);
  }
  MOE_DEV void load(int kt, uint4 (&r)[4]) const {
    const T* b = base + (size_t)kt * Tr<T>::BK * ld;
    const int lim = n - kt * Tr<T>::BK - k4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      r[kk] = kk < lim ? *(const uint4*)(b + off + (uint32_t)kk * (uint32_t)ld) : zero4();
  }
  struct NoRows {  // MNLoad's store does not use its row functor
    MOE_DEV const T* operator()(int) const { return nullptr; }
  };
  MOE_DEV void store(char* t, const uint4 (&r)[4]) const { MNLoad<T, NoRows>{}.store(t, r); }
};

// ------------------------------------------------------------- MFMA on a tile
// Fragment of tile rows (K-major) or columns (MN-major) c0 .. c0 + 31 at 16-deep K
// step ks: lane l supplies row/column c0 + (l & 31) and K values 16 ks + 8 (l >> 5)
// + 0..7.  K-major: one 16-byte read.  MN-major: two ds_read_b64_tr_b16 (gfx950:
// within each 16-lane group, lane 4a + b receives element b of the 8-byte rows
// addressed by lanes a, a + 4, a + 8, a + 12), so lane 16 g + 4 a + j addresses K row
// 16 ks + 8 (g >> 1) + j (+4 for the second read) at columns c0 + 16 (g & 1) + 4 a.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

template <bool KMAJOR>
MOE_DEV bf16x8_t frag16(const char* t, int c0, int ks, int lane) {
  if constexpr (KMAJOR) {
    return *(const bf16x8_t*)(t + swz(c0 + (lane & 31), 2 * ks + (lane >> 5)));
  } else {
    const int g = lane >> 4, a = lane & 3, j = (lane >> 2) & 3;
    const int k = 16 * ks + 8 * (g >> 1) + j;  // K row k + 4 has the same swizzle
    const int col = c0 + 16 * (g & 1) + 4 * a;
    const char* p = t + k * 256 + (((col >> 3) ^ mn_swz(k)) << 4) + (col & 7) * 2;
    typedef __attribute__((address_space(3))) s16x4_t* lp;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p + 4 * 256));
    return __builtin_bit_cast(bf16x8_t, (s16x8_t)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4,
                                                                          5, 6, 7));
  }
}

// acc[mb][nb]: wave rows arow + 32 mb, B-tile rows brow[nb]; AK / BK: the A / B
// LDS tile is K-major (else MN-major, bf16 only).
template <typename T, bool AK = true, bool BK = true, int NKS = 4>
MOE_DEV void mma_tile(const char* ta, const char* tb, f32x16_t (&acc)[2][2], int arow,
                      const int (&brow)[2], int lane);

template <>
MOE_DEV void mma_tile<bf16_t, true, true>(const char* ta, const char* tb, f32x16_t (&acc)[2][2],
                                          int arow, const int (&brow)[2], int lane);

// NKS: 16-deep K steps in the tile (4 for the 64-deep register-staged tiles, 2 for
// the 32-deep stages of the DMA-fed wgrads).
template <typename T, bool AK, bool BK, int NKS>
MOE_DEV void mma_tile(const char* ta, const char* tb, f32x16_t (&acc)[2][2], int arow,
                      const int (&brow)[2], int lane) {
  static_assert(sizeof(T) == 2, "MN-major LDS tiles are bf16 only");
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const bf16x8_t a0 = frag16<AK>(ta, arow, ks, lane);
    const bf16x8_t a1 = frag16<AK>(ta, arow + 32, ks, lane);
    const bf16x8_t b0 = frag16<BK>(tb, brow[0], ks, lane);
    const bf16x8_t b1 = frag16<BK>(tb, brow[1], ks, lane);
    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
  }
}

template <>
MOE_DEV void mma_tile<bf16_t, true, true>(const char* ta, const char* tb, f32x16_t (&acc)[2][2],
                                          int arow, const int (&brow)[2], int lane) {
  const int r = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = ks * 2 + hi;
    const bf16x8_t a0 = *(const bf16x8_t*)(ta + swz(arow + r, ch));
    const bf16x8_t a1 = *(const bf16x8_t*)(ta + swz(arow + 32 + r, ch));
    const bf16x8_t b0 = *(const bf16x8_t*)(tb + swz(brow[0] + r, ch));
    const bf16x8_t b1 = *(const bf16x8_t*)(tb + swz(brow[1] + r, ch));
    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
  }
}

template <>
MOE_DEV void mma_tile<float, true, true>(const char* ta, const char* tb, f32x16_t (&acc)[2][2],
                                         int arow, const int (&brow)[2], int lane) {
  const int r = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int ch = ks * 4 + hi * 2;
    float a[2][8], b[2][8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      *(uint4*)&a[0][4 * q] = *(const uint4*)(ta + swz(arow + r, ch + q));
      *(uint4*)&a[1][4 * q] = *(const uint4*)(ta + swz(arow + 32 + r, ch + q));
      *(uint4*)&b[0][4 * q] = *(const uint4*)(tb + swz(brow[0] + r, ch + q));
      *(uint4*)&b[1][4 * q] = *(const uint4*)(tb + swz(brow[1] + r, ch + q));
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0][s], b[0][s], acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0][s], b[1][s], acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1][s], b[0][s], acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1][s], b[1][s], acc[1][1], 0, 0, 0);
    }
  }
}

// ----------------------------------------------------------------- main loop
// Prefetch distance 2: two register sets (r*0, r*1) and two LDS buffers.  While
// the MFMAs consume K tile kt from LDS, tile kt + 1 (loaded one iteration earlier)
// goes from registers into the other LDS buffer and tile kt + 2 is in flight from
// memory, so each global load has a whole iteration to arrive.  The loop is
// unrolled by two so that the register sets stay statically indexed.
// DIST = 1 keeps one register set (fewer registers, for the short-K wgrads):
// tile kt + 1 is loaded while tile kt is multiplied.
template <typename T, int DIST = 2, class LA, class LB>
MOE_DEV void gemm_main(char* lds, const LA& la, const LB& lb, int nk, f32x16_t (&acc)[2][2],
                       int arow, const int (&brow)[2], int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  if (nk <= 0) return;
  if constexpr (DIST == 1) {
    uint4 ra[4], rb[4];
    la.load(0, ra);
    lb.load(0, rb);
    la.store(lds, ra);
    lb.store(lds + TILEB, rb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      char* cur = lds + (kt & 1) * 2 * TILEB;
      char* nxt = lds + ((kt + 1) & 1) * 2 * TILEB;
      const bool more = kt + 1 < nk;
      if (more) {
        la.load(kt + 1, ra);
        lb.load(kt + 1, rb);
      }
      mma_tile<T, LA::kmajor, LB::kmajor>(cur, cur + TILEB, acc, arow, brow, lane);
      if (more) {
        la.store(nxt, ra);
        lb.store(nxt + TILEB, rb);
      }
      __syncthreads();
    }
    return;
  }
  char* buf0 = lds;
  char* buf1 = lds + 2 * TILEB;
  uint4 ra0[4], rb0[4], ra1[4], rb1[4];
  la.load(0, ra0);
  lb.load(0, rb0);
  if (nk > 1) {
    la.load(1, ra1);
    lb.load(1, rb1);
  }
  la.store(buf0, ra0);
  lb.store(buf0 + TILEB, rb0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    if (kt + 2 < nk) {
      la.load(kt + 2, ra0);
      lb.load(kt + 2, rb0);
    }
    mma_tile<T, LA::kmajor, LB::kmajor>(buf0, buf0 + TILEB, acc, arow, brow, lane);
    if (kt + 1 < nk) {
      la.store(buf1, ra1);
      lb.store(buf1 + TILEB, rb1);
    }
    __syncthreads();
    if (kt + 1 >= nk) break;
    if (kt + 3 < nk) {
      la.load(kt + 3, ra1);
      lb.load(kt + 3, rb1);
    }
    mma_tile<T, LA::kmajor, LB::kmajor>(buf1, buf1 + TILEB, acc, arow, brow, lane);
    if (kt + 2 < nk) {
      la.store(buf0, ra0);
      lb.store(buf0 + TILEB, rb0);
    }
    __syncthreads();
  }
}

// Accumulators -> staged C tile.  Output element of acc[mb][nb][v] in lane l:
// row arow + 32 mb + 8 (v >> 2) + 4 (l >> 5) + (v & 3), column brow[nb] + (l & 31).
MOE_DEV void stage_acc(float* C, const f32x16_t (&acc)[2][2], int arow, const int (&brow)[2],
                       int lane) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = arow + 32 * mb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        C[cidx(row, brow[nb] + (lane & 31))] = acc[mb][nb][v];
      }
}

MOE_DEV void read8(const float* C, int row, int col, float* f) {
  const float4 a = *(const float4*)(C + cidx(row, col));
  const float4 b = *(const float4*)(C + cidx(row, col) + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// 8 values -> 8 elements of T at p (16-byte aligned)
MOE_DEV void store8(bf16_t* p, const float* f) { *(uint4*)p = pack8(f); }
MOE_DEV void store8(float* p, const float* f) {
  *(float4*)p = make_float4(f[0], f[1], f[2], f[3]);
  *(float4*)(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}
MOE_DEV void load8(const bf16_t* p, float* f) { unpack8(*(const uint4*)p, f); }
MOE_DEV void load8(const float* p, float* f) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Plain epilogue: the 128 x 128 tile to out_row(r) + n0 for valid rows.  NT: with
// non-temporal stores, for outputs no kernel of the step reads again (the weight
// gradients; measured on MI355X: wgrad-up 2.96 -> 2.84 ms at T = 4096, Zipf(1.2)).
MOE_DEV void store8_nt(bf16_t* p, const float* f) {
  const uint4 v = pack8(f);
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (u32x4_t*)p);
}
MOE_DEV void store8_nt(float* p, const float* f) {
  const u32x4_t a = {__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                     __float_as_uint(f[3])};
  const u32x4_t b = {__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]),
                     __float_as_uint(f[7])};
  __builtin_nontemporal_store(a, (u32x4_t*)p);
  __builtin_nontemporal_store(b, (u32x4_t*)(p + 4));
}
template <typename T, bool NT = false, class RowPtr>
MOE_DEV void epi_store(const float* C, const RowPtr& out_row, int n_valid_rows) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int r = (threadIdx.x >> 4) + 16 * s, c = threadIdx.x & 15;
    if (r < n_valid_rows) {
      float f[8];
      read8(C, r, 8 * c, f);
      if (NT) store8_nt(out_row(r) + 8 * c, f);
      else store8(out_row(r) + 8 * c, f);
    }
  }
}

// --------------------------------------------------------------- tile decode
struct RowTile {
  int e, row0, row_end;
};

constexpr int N_XCD = 8;  // MI355X: workgroup i is dispatched to XCD i mod 8

// Wave-uniform read of plan data that no kernel of this launch writes, through the
// constant address space so that it compiles to a scalar load (lgkmcnt).  A vector
// load here would make its wait vmcnt(0), which also waits for every global store
// of the previous work item of a persistent loop.
MOE_DEV int32_t ld_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// Pair L of a rows-grouped launch -> (row tile mt, column tile nt).  The row tiles
// of one expert (contiguous and in row order in the plan's tile list; the dense
// launch is one "expert") are taken in groups of up to G, and inside a group the
// column tile is outer and the row tile inner.  The workgroups an XCD runs at one
// time (a window of consecutive pairs) then form a G x (window / G) block: each
// weight panel is fetched into that XCD's L2 once per group of row tiles instead
// of once per row tile, and each row tile once per window / G column tiles.
MOE_DEV void group_rows(const int32_t* tiles, const int32_t* offsets, int dense_rows, int tile_m,
                        int nt_count, int G, int L, int& mt, int& nt) {
  const int mt0 = L / nt_count;
  int i, m_e;
  if (tiles) {
    const int e = ld_uniform(tiles + 2 * mt0), row0 = ld_uniform(tiles + 2 * mt0 + 1);
    const int s0 = ld_uniform(offsets + e), s1 = ld_uniform(offsets + e + 1);
    i = (row0 - s0) / tile_m;
    m_e = (s1 - s0 + tile_m - 1) / tile_m;
  } else {
    i = mt0;
    m_e = (dense_rows + tile_m - 1) / tile_m;
  }
  const int gf = mt0 - i % G, gsz = min(G, m_e - (i - i % G));
  const int j = L - gf * nt_count;
  nt = j / gsz;
  mt = gf + (j - nt * gsz);
}

constexpr int ROW_GROUP = 8;  // 64 workgroups per XCD at a time: 8 x 8 blocks

// Rows-grouped launches use a 1-D grid over (row tile, column tile) pairs.  The
// pairs that exist (n_tiles of the plan x nt_count) are renumbered so that the
// workgroups one XCD receives (ids x, x + 8, x + 16, ...) cover a contiguous run
// of pairs, ordered by group_rows: a row tile's activations and an expert's weight
// columns are then fetched into that XCD's L2, not into every XCD's.
// Returns false for workgroups past the last pair.
MOE_DEV bool rows_tile(const GroupInfo& g, int nt_count, RowTile& t, int& nt) {
  const int n_row_tiles = g.tiles ? g.n_tiles[0] : (g.dense_rows + TM - 1) / TM;
  const int total = n_row_tiles * nt_count;
  const int id = blockIdx.x;
  if (id >= total) return false;
  const int per = total / N_XCD, rem = total % N_XCD, x = id % N_XCD, local = id / N_XCD;
  const int L = x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
  int mt;
  group_rows(g.tiles, g.offsets, g.dense_rows, TM, nt_count, ROW_GROUP, L, mt, nt);
  if (g.tiles) {
    t.e = g.tiles[2 * mt];
    t.row0 = g.tiles[2 * mt + 1];
    t.row_end = min(t.row0 + TM, g.offsets[t.e + 1]);
  } else {
    t.e = 0;
    t.row0 = mt * TM;
    t.row_end = min(t.row0 + TM, g.dense_rows);
  }
  return true;
}

MOE_DEV int token_of(const GroupInfo& g, int r) { return g.src_token ? g.src_token[r] : r; }

MOE_DEV void wave_coords(int& arow, int (&brow)[2], bool swiglu) {
  const int w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  arow = wm * 64;
  if (swiglu) {
    brow[0] = wn * 32;        // gate columns i0 + 32 wn ..
    brow[1] = 64 + wn * 32;   // up columns, same i
  } else {
    brow[0] = wn * 64;
    brow[1] = wn * 64 + 32;
  }
}

// K-row pointer of a plain row-major matrix: element (k, i) at base[k * ld + i]
template <typename T>
struct KRowPlain {
  const T* base;
  size_t ld;
  MOE_DEV const T* operator()(int k) const { return base + (size_t)k * ld; }
};

// Weights of dgrad-up as one [2I, H] operand: rows < I from W_g[e], the rest W_u[e]
template <typename T>
struct KRowCat {
  const T* wg;
  const T* wu;
  int I, H;
  MOE_DEV const T* operator()(int k) const {
    return k < I ? wg + (size_t)k * H : wu + (size_t)(k - I) * H;
  }
};

MOE_DEV void k_segment(const GroupInfo& g, int e, int& seg0, int& seg1) {
  if (g.offsets) {
    seg0 = ld_uniform(g.offsets + e);
    seg1 = ld_uniform(g.offsets + e + 1);
  } else {
    seg0 = 0;
    seg1 = g.dense_rows;
  }
}

// Work item w of a K-grouped GEMM over an M_tiles x N_tiles output per expert:
// every expert in id order (the single dense "expert" in dense mode), the tiles of
// an expert with the M index fastest when m_fast, else the N index.  The wgrads
// put the index that runs along H fastest (measured on MI355X: 2.91 against
// 3.19 ms for wgrad-down, 5.67 against 6.13 ms for wgrad-up).  Items of experts
// without rows store zeros (the weight gradients are overwritten), so those writes
// interleave with the multiplying items of the other experts instead of running as
// a separate pass.
struct KTile {
  int e, m0, n0;
};
MOE_DEV KTile k_tile(const GroupInfo& g, int w, int mt_count, int nt_count, bool m_fast) {
  const int per = mt_count * nt_count;
  const int e = w / per, rem = w - e * per;
  KTile t;
  t.e = e;
  if (m_fast) {
    const int nt = rem / mt_count;
    t.m0 = (rem - nt * mt_count) * TM;
    t.n0 = nt * TN;
  } else {
    const int mt = rem / nt_count;
    t.m0 = mt * TM;
    t.n0 = (rem - mt * nt_count) * TN;
  }
  return t;
}

MOE_DEV int k_work_items(const GroupInfo& g, int mt_count, int nt_count) {
  return (g.offsets ? g.E : 1) * mt_count * nt_count;
}

// What a K-grouped wgrad item of expert e does: 0 multiply, 1 store a zero tile,
// 2 nothing (the large-tile kernel owns the expert's output).
MOE_DEV int k_item_kind(const GroupInfo& g, int e) {
  if (!g.counts) return 0;
  const int c = ld_uniform(g.counts + e);
  if (c == 0) return 1;
  return c >= g.hot_rows ? 2 : 0;
}

// For an item w of expert e that is skipped: advance w so that the loop's next
// step (w += gridDim.x) lands on this workgroup's first item of expert e + 1 or later.
MOE_DEV int k_skip_expert(int w, int e, int per) {
  const int nxt = (e + 1) * per;  // > w
  return w + ((nxt - w - 1) / (int)gridDim.x) * (int)gridDim.x;
}

// Zero TM * TN consecutive elements of T at out with 16-byte non-temporal stores.
// An expert without rows gets its whole gradient block zeroed: its tile (mt, nt)
// takes the block's (mt * NT + nt)-th span of TM * TN elements, not the tile's own
// rows, so every workgroup writes one contiguous 32 KiB (bf16) run instead of TM
// rows of TN elements each.
template <typename T>
MOE_DEV void zero_span(T* out) {
  constexpr int CH = TM * TN * (int)sizeof(T) / 16;
  const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < CH / NTHR; ++i)
    __builtin_nontemporal_store(z, (u32x4_t*)out + (int)threadIdx.x + i * NTHR);
}

// Persistent grid: per_cu resident workgroups per compute unit, at most one per item.
inline unsigned persistent_grid(long items, int per_cu = 2) {
  const long g = (long)per_cu * device_cus();
  return (unsigned)(items < g ? (items > 0 ? items : 1) : g);
}

}  // namespace moe
