// MXFP8 conversion on the GPU: E4M3 elements with one E8M0 scale per 32.
//
// The pages name MXFP8 training with the conversion inside the kernels
// (sebask.de, "Mixture-of-Kittens: Cursors Open-Source-Ansatz für effizientes
// MoE-Training auf NVL72", § Determinismus und MXFP8-Unterstützung; stamatios.com,
// "Cursor abre código de megakernel MoE para GPUs NVL72", § Outras
// características) but no rule; the block rule is OCP MX v1.0: scale exponent
// X = floor(log2 amax) - 8 (8 = exponent of E4M3's largest normal, 448), clamped
// to [-127, 127], X = -127 for an all-zero block, scale byte X + 127; elements are
// v / 2^X rounded to nearest even into E4M3 ("FN": no infinities) and saturated at
// +-448; the input's sign bit is kept also when the magnitude rounds to zero.
//
// Kernels here: row quantisation (blocks along the contiguous axis, optionally
// pulling rows through the plan's src_token list: the MX dispatch), column
// quantisation with a transposed output (weights blocked along their outer
// axis), and token quantisation (blocks of 32 rows from each expert segment's
// first row, written transposed for the wgrad GEMMs).
#include "common.hpp"
#include "internal.hpp"
#include "mx_common.hpp"

namespace moe {

// ------------------------------------------------------------------ rows
// One wavefront per row, lane handles 32-element blocks b = lane, lane + 64, ...
// q[r, c] = E4M3(src[g(r), c] / 2^X), s[r, c / 32] = X + 127.
template <typename T>
__global__ __launch_bounds__(256) void quant_rows_kernel(const T* __restrict__ src,
                                                         const int32_t* __restrict__ gather,
                                                         const int32_t* __restrict__ n_rows_dev,
                                                         int n_rows, int cols,
                                                         uint8_t* __restrict__ q,
                                                         uint8_t* __restrict__ sc) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rows = n_rows_dev ? min(n_rows_dev[0], n_rows) : n_rows;
  if (r >= rows) return;
  const T* row = src + (size_t)(gather ? gather[r] : r) * cols;
  const int nb = cols / 32;
  for (int b = lane; b < nb; b += 64) {
    float v[32];
    load32(row + 32 * b, v);
    const int X = mx_scale_exp(v);
    uint4 lo, hi;
    mx_encode32(v, X, lo, hi);
    uint4* qd = (uint4*)(q + (size_t)r * cols + 32 * b);
    qd[0] = lo;
    qd[1] = hi;
    sc[(size_t)r * nb + b] = (uint8_t)(X + 127);
  }
}

// The dispatch form of the same quantisation, walked by source token: row src[t]
// (t < n_tok) is quantised once and its codes and scales go to every destination row
// pos[t, j] >= 0, i.e. q[pos[t, j]] = Q(src[t]), the rows that the pull form
// q[r] = Q(src[src_token[r]]) writes.  One wavefront per token; lane j < k holds
// slot j and the others read it by lane exchange.
template <typename T>
__global__ __launch_bounds__(256) void quant_scatter_rows_kernel(const T* __restrict__ src,
                                                                 const int32_t* __restrict__ pos,
                                                                 int n_tok, int k, int cols,
                                                                 uint8_t* __restrict__ q,
                                                                 uint8_t* __restrict__ sc) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n_tok) return;
  const int my_row = lane < k ? pos[(size_t)t * k + lane] : -1;
  const T* row = src + (size_t)t * cols;
  const int nb = cols / 32;
  for (int b = lane; b < nb; b += 64) {
    float v[32];
    load32(row + 32 * b, v);
    const int X = mx_scale_exp(v);
    uint4 lo, hi;
    mx_encode32(v, X, lo, hi);
    for (int j = 0; j < k; ++j) {
      const int r = __shfl(my_row, j, 64);
      if (r < 0) continue;
      uint4* qd = (uint4*)(q + (size_t)r * cols + 32 * b);
      qd[0] = lo;
      qd[1] = hi;
      sc[(size_t)r * nb + b] = (uint8_t)(X + 127);
    }
  }
}

// ------------------------------------------------------------ columns
// Batched [batch, rows, cols] -> q [batch, cols, rows] with blocks of 32 along
// rows: q[b, c, r] = E4M3(src[b, r, c] / 2^X(b, c, r / 32)).  A workgroup takes a
// 32 x 256 slab (one row block, 256 columns) through LDS.
template <typename T>
__global__ __launch_bounds__(256) void quant_cols_kernel(const T* __restrict__ src, int rows,
                                                         int cols, uint8_t* __restrict__ q,
                                                         uint8_t* __restrict__ sc) {
  __shared__ float tile[32][257];
  const int rb = blockIdx.x, c0 = blockIdx.y * 256, bat = blockIdx.z;
  const T* s = src + (size_t)bat * rows * cols;
  for (int i = threadIdx.x; i < 32 * 256; i += 256) {
    const int rr = i / 256, cc = i % 256;
    tile[rr][cc] = (c0 + cc < cols) ? to_f32(s[(size_t)(32 * rb + rr) * cols + c0 + cc]) : 0.0f;
  }
  __syncthreads();
  const int c = c0 + threadIdx.x;
  if (c >= cols) return;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = tile[i][threadIdx.x];
  const int X = mx_scale_exp(v);
  uint4 lo, hi;
  mx_encode32(v, X, lo, hi);
  uint4* qd = (uint4*)(q + (size_t)bat * cols * rows + (size_t)c * rows + 32 * rb);
  qd[0] = lo;
  qd[1] = hi;
  sc[(size_t)bat * cols * (rows / 32) + (size_t)c * (rows / 32) + rb] = (uint8_t)(X + 127);
}

// ------------------------------------------------------------- tokens
// For plan tile t (expert e, rows row0 .. row_end-1, at most 128) and column c:
// blocks of 32 rows from row0 (a multiple of 32 rows after the segment's first row,
// so the blocks start at the segment's first row); the output is transposed into
// the wgrads' token axis: q[c, kbase + j] for local row j with
// kbase = kpos[e] + kseg[e] + (row0 - offsets[e]) (kseg NULL: 0; rows past row_end inside a block
// are zero), scales s[c, kbase / 32 + j / 32].  Blocks without a row are not
// written: those columns belong to the next segment.  src rows are pulled through
// gather when given.  One workgroup per (tile, 64 columns): 16-byte row loads into
// an LDS tile in the input type, one thread per (column, block) for the scale and
// the codes, which are staged in the same LDS as [column][row] so that 8 lanes store
// each column's 128 codes as one contiguous run.
template <typename T>
__global__ __launch_bounds__(256) void quant_tokens_kernel(
    const T* __restrict__ src, const int32_t* __restrict__ gather, int ld,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ kpos,
    const int32_t* __restrict__ kseg, int cols, size_t kpad_total, uint8_t* __restrict__ q,
    uint8_t* __restrict__ sc) {
  constexpr int VEC = 16 / (int)sizeof(T), VPR = 64 / VEC;  // elements per load, loads per row
  constexpr int TROW = 64 + VEC;  // tile row in elements (padded by one 16-byte piece)
  constexpr int CROW = 128 + 16;  // bytes per staged code column (padded)
  static_assert(64 * CROW <= 128 * TROW * (int)sizeof(T), "codes fit in the tile");
  // the tile in the input type; after every thread has read its 32 values it is
  // reused for the codes
  __shared__ __attribute__((aligned(16))) T tile[128 * TROW];
  uint8_t* codes = (uint8_t*)tile;
  const int t = blockIdx.x, c0 = blockIdx.y * 64;
  if (t >= n_tiles[0]) return;
  const int e = tiles[2 * t], row0 = tiles[2 * t + 1];
  const int nrows = min(row0 + 128, offsets[e + 1]) - row0;
  // every lane issues all its loads before the first LDS store
  constexpr int NL = 128 * VPR / 256;
  uint4 raw[NL];
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    const int i = (int)threadIdx.x + 256 * k, j = i / VPR, v = i - j * VPR;
    raw[k] = make_uint4(0u, 0u, 0u, 0u);
    if (j < nrows) {
      const int r = row0 + j;
      raw[k] = *(const uint4*)(src + (size_t)(gather ? gather[r] : r) * ld + c0 + v * VEC);
    }
  }
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    const int i = (int)threadIdx.x + 256 * k, j = i / VPR, v = i - j * VPR;
    *(uint4*)(tile + j * TROW + v * VEC) = raw[k];
  }
  __syncthreads();
  const int cc = threadIdx.x & 63, blk = threadIdx.x >> 6;
  const bool has = 32 * blk < nrows;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = to_f32(tile[(32 * blk + i) * TROW + cc]);
  __syncthreads();  // the tile is now free for the codes
  const size_t kbase = (size_t)kpos[e] + (kseg ? kseg[e] : 0) + (row0 - offsets[e]);
  if (has) {
    const int X = mx_scale_exp(v);
    uint4 lo, hi;
    mx_encode32(v, X, lo, hi);
    *(uint4*)(codes + cc * CROW + 32 * blk) = lo;
    *(uint4*)(codes + cc * CROW + 32 * blk + 16) = hi;
    sc[(size_t)(c0 + cc) * (kpad_total / 32) + kbase / 32 + blk] = (uint8_t)(X + 127);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int col = i >> 3, ch = i & 7;
    if (16 * ch >= ((nrows + 31) & ~31)) continue;  // 16-byte chunk of a block without rows
    *(uint4*)(q + (size_t)(c0 + col) * kpad_total + kbase + 16 * ch) =
        *(const uint4*)(codes + col * CROW + 16 * ch);
  }
}

// ----------------------------------------------------------- launchers
hipError_t launch_quant_rows(int dt, const void* src, const int32_t* gather,
                             const int32_t* n_rows_dev, int n_rows, int cols, uint8_t* q,
                             uint8_t* sc, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n_rows + 3) / 4);
  if (dt)
    return MOE_LAUNCH("mx_quant_rows", s,
                      quant_rows_kernel<bf16_t><<<grid, 256, 0, s>>>(
                          (const bf16_t*)src, gather, n_rows_dev, n_rows, cols, q, sc));
  return MOE_LAUNCH("mx_quant_rows", s,
                    quant_rows_kernel<float><<<grid, 256, 0, s>>>(
                        (const float*)src, gather, n_rows_dev, n_rows, cols, q, sc));
}

hipError_t launch_quant_scatter_rows(int dt, const void* src, const int32_t* pos, int n_tok, int k,
                                     int cols, uint8_t* q, uint8_t* sc, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n_tok + 3) / 4);
  if (dt)
    return MOE_LAUNCH("mx_quant_rows", s,
                      quant_scatter_rows_kernel<bf16_t><<<grid, 256, 0, s>>>(
                          (const bf16_t*)src, pos, n_tok, k, cols, q, sc));
  return MOE_LAUNCH("mx_quant_rows", s,
                    quant_scatter_rows_kernel<float><<<grid, 256, 0, s>>>(
                        (const float*)src, pos, n_tok, k, cols, q, sc));
}

hipError_t launch_quant_cols(int dt, const void* src, int batch, int rows, int cols, uint8_t* q,
                             uint8_t* sc, hipStream_t s) {
  if (batch == 0 || rows == 0) return hipSuccess;
  const dim3 grid(rows / 32, (cols + 255) / 256, batch);
  if (dt)
    return MOE_LAUNCH("mx_quant_cols", s,
                      quant_cols_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)src, rows,
                                                                     cols, q, sc));
  return MOE_LAUNCH("mx_quant_cols", s,
                    quant_cols_kernel<float><<<grid, 256, 0, s>>>((const float*)src, rows, cols,
                                                                  q, sc));
}

hipError_t launch_quant_tokens(int dt, const void* src, const int32_t* gather, int ld,
                               const int32_t* tiles, const int32_t* n_tiles,
                               const int32_t* offsets, const int32_t* kpos,
                               const int32_t* kseg, int max_tiles, int cols, size_t kpad_total,
                               uint8_t* q, uint8_t* sc, hipStream_t s) {
  if (max_tiles == 0) return hipSuccess;
  const dim3 grid(max_tiles, cols / 64);
  if (dt)
    return MOE_LAUNCH("mx_quant_tokens", s,
                      quant_tokens_kernel<bf16_t><<<grid, 256, 0, s>>>(
                          (const bf16_t*)src, gather, ld, tiles, n_tiles, offsets, kpos, kseg,
                          cols, kpad_total, q, sc));
  return MOE_LAUNCH("mx_quant_tokens", s,
                    quant_tokens_kernel<float><<<grid, 256, 0, s>>>(
                        (const float*)src, gather, ld, tiles, n_tiles, offsets, kpos, kseg, cols,
                        kpad_total, q, sc));
}

}  // namespace moe
