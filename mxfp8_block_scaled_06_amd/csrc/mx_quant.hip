// MXFP8 quantize kernels for gfx950: rowwise 1x32, colwise 32x1 (transposed
// output) and 32x32 square blocks.
//
// Operation: "MXFP8 (Micro-scaling FP8)" page, sections "Definition" (one
// shared power-of-two scale per small block of values) and "Low-precision
// Flash Attention (MXFP8 on FA4)" (scales along each GEMM's K dimension,
// derived by bit manipulation instead of log2/round/clamp; 32x32 blocks with a
// wave-wide max-abs reduction, transpose-invariant).  The 3D colwise weight
// quantization for the backward is the pytorch/ao "3d quant colwise scaling
// kernel" of the PR timeline.
//
// Per block: amax over the |bf16| bit patterns (integer max, exact), E8M0 byte
// = max(exponent field - 8, 0) (0xFF for NaN/Inf), every element multiplied
// by 2^(127 - byte) in fp32 (exact: bf16 has 8 significant bits), clamped to
// +-448 and converted to E4M3 with the hardware RNE convert.  All three are
// HBM-bound streaming passes: 2 bytes read, 1 + 1/32 (or 1/1024) written per
// element.  Both orientations from one read (the weight 4-tuple, and the
// activations of the differentiable step) and the colwise pass on 256-column
// inputs run in quant_dual256_kernel, whose 256 x 256 tiles give every global
// access 256-byte or longer runs; 128 x 128 tile kernels serve the other
// shapes.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mxk {

// ---------------------------------------------------------------------------
// Rowwise: x viewed as [rows, cols] (batch folded into rows), dense outputs.
// One 16-byte chunk (8 values) per lane and load; a DPP quad holds one block.
// Each thread handles kRowU chunks spaced by the block size so every wave-wide
// load instruction reads 1 KiB of contiguous input (two chunks per thread
// measured fastest: more waves in flight, shorter per-wave tails).
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 256;
constexpr int kRowU = 2;

// Scale byte destination.  Row-major: block g (row-major over rows x KB
// blocks) goes to s[g].  GEMM layout (rows_per_batch > 0): [batch][KB/4]
// [rows_per_batch][4], so the 4 blocks of a 128-wide contraction step of 256
// consecutive rows form one contiguous 1 KiB run for the GEMM's loads.
__device__ __forceinline__ uint32_t row_scale_index(uint32_t g, uint32_t kb_per_row, uint32_t rows_per_batch) {
  if (rows_per_batch == 0) return g;
  const uint32_t r = g / kb_per_row, kb = g - r * kb_per_row;
  const uint32_t b = r / rows_per_batch, rr = r - b * rows_per_batch;
  return b * kb_per_row * rows_per_batch + (kb >> 2) * rows_per_batch * 4 + rr * 4 + (kb & 3);
}

__global__ __launch_bounds__(kRowThreads) void quant_rowwise_kernel(const uint16_t* __restrict__ x,
                                                                    int64_t nchunks,
                                                                    uint8_t* __restrict__ q,
                                                                    uint8_t* __restrict__ s,
                                                                    uint32_t kb_per_row,
                                                                    uint32_t rows_per_batch) {
  const int64_t base = (int64_t)blockIdx.x * (kRowThreads * kRowU) + threadIdx.x;
  v4i w[kRowU];
#pragma unroll
  for (int u = 0; u < kRowU; ++u) {
    const int64_t idx = base + (int64_t)u * kRowThreads;
    if (idx < nchunks) {
      w[u] = __builtin_nontemporal_load((const v4i*)(x + idx * 8));
    } else {
      w[u] = (v4i){0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int u = 0; u < kRowU; ++u) {
    const int64_t idx = base + (int64_t)u * kRowThreads;
    // chunks 4k..4k+3 form one block; nchunks is a multiple of 4, so a quad
    // is either fully in range or fully out of range.
    const uint32_t am = quad_max(absmax8(w[u]));
    if (idx < nchunks) {
      const uint32_t byte = e8m0_from_absbits(am);
      v2i codes;
      if (byte == 0xFFu) {
        codes = (v2i){0x7F7F7F7F, 0x7F7F7F7F};
      } else {
        codes = quant8(w[u], inv_scale_from_e8m0(byte));
      }
      *(v2i*)(q + idx * 8) = codes;
      if ((threadIdx.x & 3) == 0) s[row_scale_index((uint32_t)(idx >> 2), kb_per_row, rows_per_batch)] = (uint8_t)byte;
    }
  }
}

// ---------------------------------------------------------------------------
// Rowwise with the token gather fused in: output row r quantizes source row
// rows[r] of x (a negative or out-of-range index gives a zero row, e.g. the
// padding that rounds an expert group up to 32 rows).  Scales go straight to
// the GEMM layout [cols/128][M][4], so the result feeds the grouped GEMM as X
// with no gathered bf16 copy in between.
// ---------------------------------------------------------------------------
// NARROW: nchunks < 2^32, so chunk -> (row, piece) takes a 32-bit division
// (the 64-bit one costs about 5% of the kernel).
template <bool NARROW>
__global__ __launch_bounds__(kRowThreads) void quant_rowwise_gather_kernel(const uint16_t* __restrict__ x,
                                                                           int64_t src_rows,
                                                                           const int32_t* __restrict__ rows,
                                                                           int64_t nchunks, int64_t cols,
                                                                           uint8_t* __restrict__ q,
                                                                           uint8_t* __restrict__ s,
                                                                           uint32_t chunks_per_row,
                                                                           uint32_t out_rows) {
  const int64_t base = (int64_t)blockIdx.x * (kRowThreads * kRowU) + threadIdx.x;
  auto row_of = [&](int64_t idx) -> uint32_t {
    return NARROW ? (uint32_t)idx / chunks_per_row : (uint32_t)(idx / chunks_per_row);
  };
  // the row indices of all kRowU chunks first, then the data: no data load
  // waits behind an index load
  int sr[kRowU];
#pragma unroll
  for (int u = 0; u < kRowU; ++u) {
    const int64_t idx = min(base + (int64_t)u * kRowThreads, nchunks - 1);   // nchunks > 0: the grid is empty otherwise
    sr[u] = rows[row_of(idx)];
  }
  v4i w[kRowU];
#pragma unroll
  for (int u = 0; u < kRowU; ++u) {
    const int64_t idx = base + (int64_t)u * kRowThreads;
    w[u] = (v4i){0, 0, 0, 0};
    if (idx < nchunks && sr[u] >= 0 && sr[u] < src_rows) {
      const uint32_t r = row_of(idx);
      const uint32_t c = (uint32_t)(idx - (int64_t)r * chunks_per_row);
      w[u] = __builtin_nontemporal_load((const v4i*)(x + (int64_t)sr[u] * cols + c * 8));
    }
  }
#pragma unroll
  for (int u = 0; u < kRowU; ++u) {
    const int64_t idx = base + (int64_t)u * kRowThreads;
    const uint32_t am = quad_max(absmax8(w[u]));   // quads never straddle rows (cols % 32 == 0)
    if (idx < nchunks) {
      const uint32_t byte = e8m0_from_absbits(am);
      v2i codes;
      if (byte == 0xFFu) {
        codes = (v2i){0x7F7F7F7F, 0x7F7F7F7F};
      } else {
        codes = quant8(w[u], inv_scale_from_e8m0(byte));
      }
      *(v2i*)(q + idx * 8) = codes;
      if ((threadIdx.x & 3) == 0) s[row_scale_index((uint32_t)(idx >> 2), chunks_per_row / 4, out_rows)] = (uint8_t)byte;
    }
  }
}

// ---------------------------------------------------------------------------
// Colwise: x [batch, rows, cols] -> q_t [batch, cols, ldq], s_t (ldq >= rows,
// ldq % 32 == 0).  Used when cols % 256 != 0 (otherwise quant_dual256_kernel
// without its rowwise half).  Columns [rows, min(ldq, rows rounded up to 128)) of q_t are
// the codes of zero rows (0x00, scale byte 0x00).
// A workgroup stages a 128x128 bf16 tile in LDS (coalesced 256-byte row
// segments); wave w quantizes rows [32w, 32w+32) of the tile: lane l owns
// columns 2l and 2l+1 and reads its 32 dwords conflict-free (one LDS row per
// step).  The codes go back through the same LDS buffer, transposed, so every
// global store instruction writes whole 128-byte lines of q_t (8 lanes per
// output row) instead of 32-byte pieces of 64 different rows.
// ---------------------------------------------------------------------------
constexpr int kColTile = 128;
constexpr int kColPitch = 144;   // bytes per staged output row (128 codes + 16 pad)

static_assert(kColTile * kColPitch + kColTile * 4 <= kColTile * kColTile * 2, "codes and scales fit the input tile");

__global__ __launch_bounds__(256) void quant_colwise_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, uint8_t* __restrict__ q_t,
                                                            int64_t ldq, uint8_t* __restrict__ s_t,
                                                            int64_t lds, int gemm_layout) {
  __shared__ v4i tile[kColTile * (kColTile / 8)];  // [128 rows][16 chunks of 8 bf16], later the codes
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * kColTile;
  const int64_t c0 = (int64_t)blockIdx.x * kColTile;
  const uint16_t* xb = x + b * rows * cols;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int chunk = it * 256 + tid;
    const int rr = chunk >> 4, cc = chunk & 15;
    const int64_t row = r0 + rr, col = c0 + cc * 8;
    v4i w = (v4i){0, 0, 0, 0};
    if (row < rows && col < cols) w = __builtin_nontemporal_load((const v4i*)(xb + row * cols + col));
    tile[rr * 16 + cc] = w;
  }
  __syncthreads();
  const int wv = tid >> 6, lane = tid & 63;
  const uint32_t* t32 = (const uint32_t*)tile;
  uint32_t v[32];
  uint32_t am0 = 0, am1 = 0;
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    v[t] = t32[(32 * wv + t) * 64 + lane];
    am0 = max(am0, v[t] & 0x7FFFu);
    am1 = max(am1, (v[t] >> 16) & 0x7FFFu);
  }
  const uint32_t byte0 = e8m0_from_absbits(am0), byte1 = e8m0_from_absbits(am1);
  const float m0 = inv_scale_from_e8m0(byte0 == 0xFFu ? 127u : byte0);
  const float m1 = inv_scale_from_e8m0(byte1 == 0xFFu ? 127u : byte1);
  v4i out0[2], out1[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int t = h * 16 + d * 4;
      int a = cvt2_e4m3<false>(bf16lo(v[t]) * m0, bf16lo(v[t + 1]) * m0, 0);
      a = cvt2_e4m3<true>(bf16lo(v[t + 2]) * m0, bf16lo(v[t + 3]) * m0, a);
      int c = cvt2_e4m3<false>(bf16hi(v[t]) * m1, bf16hi(v[t + 1]) * m1, 0);
      c = cvt2_e4m3<true>(bf16hi(v[t + 2]) * m1, bf16hi(v[t + 3]) * m1, c);
      out0[h][d] = byte0 == 0xFFu ? 0x7F7F7F7F : a;
      out1[h][d] = byte1 == 0xFFu ? 0x7F7F7F7F : c;
    }
  }
  __syncthreads();   // every wave has its input in registers: the tile becomes the output stage
  uint8_t* o8 = (uint8_t*)tile;
  uint8_t* sc = o8 + kColTile * kColPitch;   // [128 output rows][4 blocks]
  *(v4i*)(o8 + (2 * lane) * kColPitch + 32 * wv) = out0[0];
  *(v4i*)(o8 + (2 * lane) * kColPitch + 32 * wv + 16) = out0[1];
  *(v4i*)(o8 + (2 * lane + 1) * kColPitch + 32 * wv) = out1[0];
  *(v4i*)(o8 + (2 * lane + 1) * kColPitch + 32 * wv + 16) = out1[1];
  sc[(2 * lane) * 4 + wv] = (uint8_t)byte0;
  sc[(2 * lane + 1) * 4 + wv] = (uint8_t)byte1;
  __syncthreads();
  // 128 output rows x 8 pieces of 16 bytes; 8 consecutive lanes fill one line
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = j * 256 + tid;
    const int orow = p >> 3, pc = p & 7;
    const int64_t col = c0 + orow, rr = r0 + 16 * pc;
    // rows past the input read as zeros: with ldq > rows the padding columns
    // of q_t get zero codes (up to the last 128-row tile)
    if (col < cols && rr < ldq) {
      const v4i w = *(const v4i*)(o8 + orow * kColPitch + 16 * pc);
      *(v4i*)(q_t + (b * cols + col) * ldq + rr) = w;
    }
  }
  // scales: thread t < 128 owns output row c0 + t and its (up to) 4 blocks
  if (tid < kColTile) {
    const int64_t col = c0 + tid;
    const int64_t nblk = min((int64_t)4, (ldq - r0) >> 5);    // ldq % 32 == 0
    if (col < cols) {
      const uint32_t w4 = *(const uint32_t*)(sc + tid * 4);
      if (gemm_layout) {
        // [batch][ldq/128][cols][4]: blocks r0/32 .. r0/32+3 of output row `col` (r0 % 128 == 0)
        uint8_t* sp = s_t + b * (ldq / 32) * cols + (r0 >> 7) * cols * 4 + col * 4;
        if (nblk == 4) {
          *(uint32_t*)sp = w4;
        } else {
          for (int k = 0; k < nblk; ++k) sp[k] = (uint8_t)(w4 >> (8 * k));
        }
      } else {
        uint8_t* sp = s_t + (b * cols + col) * lds + (r0 >> 5);
        for (int k = 0; k < nblk; ++k) sp[k] = (uint8_t)(w4 >> (8 * k));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Both orientations in one pass: w [E, N, K] ->
//   q   [E, N, K]   (1x32 blocks along K), s   GEMM layout [E][K/128][N][4]
//   q_t [E, K, ldq] (32x1 blocks along N), s_t GEMM layout [E][ldq/128][K][4]
// (K % 128 == 0, N % 32 == 0, ldq % 128 == 0, ldq >= N; rows [N, ldq) are
// quantized as zero rows, so q_t's padding columns hold zero codes and zero
// scales).  Expert weights use ldq = N; activations (the forward's A, the
// backward's dOut) use ldq = N rounded up to 128, the contraction length of
// the wgrad GEMM.  Used when K % 256 != 0 (otherwise quant_dual256_kernel).
// A workgroup stages a 128 (n) x 128 (k) bf16
// tile in LDS once; the rowwise half quantizes its rows straight to q (four
// threads fill one 128-byte line), the colwise half is the colwise kernel's
// path (column pairs, codes transposed back through LDS for whole-line
// stores).  HBM traffic 4 + 1/16 bytes per element instead of two passes of
// 3 + 1/32.  Operation: the weight 4-tuple of the MoK expert PR review
// (weight_fp8 / weight_scale for the forward, weight_t_fp8 / weight_t_scale
// for the backward).
// ---------------------------------------------------------------------------
constexpr int kDualPitch = 272;   // bytes per staged input row (256 + 16): conflict-free row and column reads

__global__ __launch_bounds__(256) void quant_dual_kernel(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                         int64_t ldq, uint8_t* __restrict__ q,
                                                         uint8_t* __restrict__ s, uint8_t* __restrict__ q_t,
                                                         uint8_t* __restrict__ s_t,
                                                         const int32_t* __restrict__ rows, int64_t n_items,
                                                         uint32_t topk) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kColTile * kDualPitch];
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.z;
  const int64_t n0 = (int64_t)blockIdx.y * kColTile;   // ldq % 128 == 0: rows [N, ldq) read as zeros
  const int64_t k0 = (int64_t)blockIdx.x * kColTile;
  const uint16_t* wb = w + b * N * K;
  // input row of each of the thread's 8 chunks (-1: a zero row).  Gathered
  // rows: row n of the tile is input row rows[n] / topk (negative or out of
  // range: a zero row, the padding of an expert group); the row indices are
  // all loaded before any data.
  int64_t src[8];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int64_t n = n0 + ((it * 256 + tid) >> 4);
    src[it] = n < N ? n : -1;
  }
  if (rows != nullptr && N > 0) {
    int idx[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) idx[it] = rows[min(n0 + ((it * 256 + tid) >> 4), N - 1)];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int64_t item = src[it] >= 0 ? (int64_t)idx[it] : -1;
      src[it] = item >= 0 && item < n_items ? (topk == 1 ? item : (int64_t)((uint32_t)item / topk)) : -1;
    }
  }
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int chunk = it * 256 + tid;
    const int rr = chunk >> 4, cc = chunk & 15;
    v4i v = (v4i){0, 0, 0, 0};
    if (src[it] >= 0) v = __builtin_nontemporal_load((const v4i*)(wb + src[it] * K + k0 + cc * 8));
    *(v4i*)(tile + rr * kDualPitch + cc * 16) = v;
  }
  __syncthreads();

  // ---- rowwise: task = (row, block of 32 along k); threads 4r..4r+3 share a row
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int task = h * 256 + tid;
    const int row = task >> 2, blk = task & 3;
    v4i x[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = *(const v4i*)(tile + row * kDualPitch + blk * 64 + c * 16);
    uint32_t am = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) am = max(am, absmax8(x[c]));
    const uint32_t byte = e8m0_from_absbits(am);
    const float m = inv_scale_from_e8m0(byte == 0xFFu ? 127u : byte);
    v4i o0, o1;
    {
      const v2i c0 = byte == 0xFFu ? (v2i){0x7F7F7F7F, 0x7F7F7F7F} : quant8(x[0], m);
      const v2i c1 = byte == 0xFFu ? (v2i){0x7F7F7F7F, 0x7F7F7F7F} : quant8(x[1], m);
      const v2i c2 = byte == 0xFFu ? (v2i){0x7F7F7F7F, 0x7F7F7F7F} : quant8(x[2], m);
      const v2i c3 = byte == 0xFFu ? (v2i){0x7F7F7F7F, 0x7F7F7F7F} : quant8(x[3], m);
      o0 = (v4i){c0[0], c0[1], c1[0], c1[1]};
      o1 = (v4i){c2[0], c2[1], c3[0], c3[1]};
    }
    if (n0 + row < N) {
      uint8_t* qp = q + (b * N + n0 + row) * K + k0 + blk * 32;
      *(v4i*)qp = o0;
      *(v4i*)(qp + 16) = o1;
      // [E][K/128][N][4]: the tile's 128 columns are one chunk
      s[b * (K / 32) * N + (k0 >> 7) * N * 4 + (n0 + row) * 4 + blk] = (uint8_t)byte;
    }
  }

  // ---- colwise: wave w quantizes rows [32w, 32w+32) of columns 2l, 2l+1
  const int wv = tid >> 6, lane = tid & 63;
  uint32_t v[32];
  uint32_t am0 = 0, am1 = 0;
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    v[t] = *(const uint32_t*)(tile + (32 * wv + t) * kDualPitch + 4 * lane);
    am0 = max(am0, v[t] & 0x7FFFu);
    am1 = max(am1, (v[t] >> 16) & 0x7FFFu);
  }
  const uint32_t byte0 = e8m0_from_absbits(am0), byte1 = e8m0_from_absbits(am1);
  const float m0 = inv_scale_from_e8m0(byte0 == 0xFFu ? 127u : byte0);
  const float m1 = inv_scale_from_e8m0(byte1 == 0xFFu ? 127u : byte1);
  v4i out0[2], out1[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int t = hh * 16 + d * 4;
      int a = cvt2_e4m3<false>(bf16lo(v[t]) * m0, bf16lo(v[t + 1]) * m0, 0);
      a = cvt2_e4m3<true>(bf16lo(v[t + 2]) * m0, bf16lo(v[t + 3]) * m0, a);
      int c = cvt2_e4m3<false>(bf16hi(v[t]) * m1, bf16hi(v[t + 1]) * m1, 0);
      c = cvt2_e4m3<true>(bf16hi(v[t + 2]) * m1, bf16hi(v[t + 3]) * m1, c);
      out0[hh][d] = byte0 == 0xFFu ? 0x7F7F7F7F : a;
      out1[hh][d] = byte1 == 0xFFu ? 0x7F7F7F7F : c;
    }
  }
  __syncthreads();   // both halves are done reading the input: the tile becomes the output stage
  uint8_t* o8 = tile;
  uint8_t* sc = o8 + kColTile * kColPitch;   // [128 output rows][4 blocks]
  *(v4i*)(o8 + (2 * lane) * kColPitch + 32 * wv) = out0[0];
  *(v4i*)(o8 + (2 * lane) * kColPitch + 32 * wv + 16) = out0[1];
  *(v4i*)(o8 + (2 * lane + 1) * kColPitch + 32 * wv) = out1[0];
  *(v4i*)(o8 + (2 * lane + 1) * kColPitch + 32 * wv + 16) = out1[1];
  sc[(2 * lane) * 4 + wv] = (uint8_t)byte0;
  sc[(2 * lane + 1) * 4 + wv] = (uint8_t)byte1;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = j * 256 + tid;
    const int orow = p >> 3, pc = p & 7;
    const v4i x = *(const v4i*)(o8 + orow * kColPitch + 16 * pc);
    *(v4i*)(q_t + (b * K + k0 + orow) * ldq + n0 + 16 * pc) = x;
  }
  if (tid < kColTile) {
    // [E][ldq/128][K][4]: blocks n0/32 .. n0/32 + 3 of output row k0 + tid
    *(uint32_t*)(s_t + b * (ldq / 32) * K + (n0 >> 7) * K * 4 + (k0 + tid) * 4) = *(const uint32_t*)(sc + tid * 4);
  }
}

static_assert(kColTile * kColPitch + kColTile * 4 <= kColTile * kDualPitch, "output stage fits the input tile");

// ---------------------------------------------------------------------------
// Both orientations in one pass, 256 x 256 tiles (K % 256 == 0): the same
// outputs as quant_dual_kernel with every global access twice as long.
// 512 threads; wave w owns rows [n0 + 32w, +32) (one colwise block), lane l
// rows n0 + 32w + 16(l/32) + i (i = 0..15) and the 16-byte piece l%32 of each
// 512-byte row segment (8 columns).  Nothing bf16 goes through LDS:
//  * rowwise: the four lanes of a DPP quad hold one 32-element block of a
//    row; codes go straight to q (a wave stores two 256-byte row runs per
//    instruction);
//  * colwise: a lane's 16 rows and its partner lane l ^ 32's 16 rows are a
//    whole 32-row block of its 8 columns, so the column amax is a packed
//    16-bit max over registers plus one exchange; each column's 16 codes are
//    one 16-byte LDS write into a [256 k][256 n] code tile (16-byte slots
//    swizzled by k / 8 so the writes and the row reads are conflict-free),
//    which the workgroup then stores as 256-byte runs of q_t rows;
//  * both scale sets are staged in LDS and stored as dwords of the GEMM
//    layout (1 KiB runs).
// ---------------------------------------------------------------------------
constexpr int kD2 = 256;                      // tile columns (k)
constexpr int kD2N = 256;                     // tile rows (n)
constexpr int kD2Threads = 2 * kD2N;
constexpr int kD2Slots = kD2N / 16;           // 16-byte slots per code-tile row

__device__ __forceinline__ int d2_slot(int k, int slot) { return slot ^ ((k >> 3) & 15); }

// ROWWISE = false is the colwise quantizer alone (q and s untouched); its
// scales go to the GEMM layout when st_ld == 0, else row-major [batch][K][st_ld]
// (blocks n0/32 .. of row k).  128 VGPRs: two workgroups per CU.
//
// Tile order.  Both passes take a 3D grid, column tiles fastest, except the
// colwise pass when both
//  * ldq % 128 != 0: the transposed rows start off a 128-byte line, so
//    row-tile neighbours write the two halves of shared lines, and
//  * the column-tile count is not a multiple of 8: in that order row-tile
//    neighbours then run on different XCDs, whose L2s write their halves
//    of each shared line separately.
// Then it takes a 1D grid of slots (slot s runs on XCD s % 8) in which each
// XCD walks chunks of kColChunk row tiles of one column tile, row tiles
// fastest, so one L2 merges the halves close together in time: +9% on
// [65600, 5120].  The chunks scatter the row reads, which costs 7-11% where
// there is nothing to merge, hence the two conditions.
constexpr int kColChunk = 4;

__host__ __device__ inline bool col_chunked(int64_t cols, int64_t ldq) {
  return ldq % 128 != 0 && (cols / kD2) % 8 != 0;
}

template <bool ROWWISE>
__global__ __launch_bounds__(kD2Threads) __attribute__((amdgpu_waves_per_eu(4))) void quant_dual256_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, int64_t ldq, uint8_t* __restrict__ q,
    uint8_t* __restrict__ s, uint8_t* __restrict__ q_t, uint8_t* __restrict__ s_t, int64_t st_ld,
    const int32_t* __restrict__ rows, int64_t n_items, uint32_t topk, int64_t batches) {
  __shared__ __attribute__((aligned(16))) uint8_t codes[kD2 * kD2N];      // [256 k][kD2N n] transposed codes
  __shared__ __attribute__((aligned(16))) uint8_t srow[2 * kD2N * 4];     // [k chunk][rows][4 blocks]
  __shared__ __attribute__((aligned(16))) uint8_t scol[kD2N / 128 * kD2 * 4];   // [n chunk][256 cols][4 blocks]
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, pc = lane & 31;
  int64_t b = blockIdx.z, n0 = (int64_t)blockIdx.y * kD2N, k0 = (int64_t)blockIdx.x * kD2;
  if (!ROWWISE && col_chunked(K, ldq)) {
    // 1D grid of slots; 32-bit arithmetic (the launcher bounds the slot count)
    const uint32_t tx = (uint32_t)(K / kD2), ty = (uint32_t)((ldq + kD2N - 1) / kD2N);
    const uint32_t sl = blockIdx.x, si = sl >> 3;
    const uint32_t t = ((si / kColChunk) * 8 + (sl & 7)) * kColChunk + si % kColChunk;
    if (t >= tx * ty * (uint32_t)batches) return;     // padding slot (uniform over the workgroup)
    const uint32_t bt = t / (tx * ty), r = t - bt * tx * ty;
    b = bt;
    n0 = (int64_t)(r % ty) * kD2N;
    k0 = (int64_t)(r / ty) * kD2;
  }
  const uint16_t* wb = w + b * N * K;
  const int r0 = 32 * wv + 16 * half;          // tile row of this lane's i = 0

  // input row of each of the lane's 16 rows (-1: a zero row).  Gathered
  // rows: row n is input row rows[n] / topk (negative or out of range: a zero
  // row, the padding of an expert group).  All 16 row indices are loaded
  // before any data, so no data load waits behind an index load.
  int64_t src[16];
  if (rows != nullptr && N > 0) {
    int idx[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) idx[i] = rows[min(n0 + r0 + i, N - 1)];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t item = n0 + r0 + i < N ? (int64_t)idx[i] : -1;
      src[i] = item >= 0 && item < n_items ? (topk == 1 ? item : (int64_t)((uint32_t)item / topk)) : -1;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) src[i] = rows == nullptr && n0 + r0 + i < N ? n0 + r0 + i : -1;
  }
  v4i v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v4i x = (v4i){0, 0, 0, 0};
    if (src[i] >= 0) x = __builtin_nontemporal_load((const v4i*)(wb + src[i] * K + k0 + 8 * pc));
    v[i] = x;
  }

  // ---- rowwise: block pc / 4 of each row
  const int kb = pc >> 2;
#pragma unroll
  for (int i = 0; i < 16 && ROWWISE; ++i) {
    const int64_t n = n0 + r0 + i;
    const uint32_t byte = e8m0_from_absbits(quad_max(absmax8(v[i])));
    const float m = inv_scale_from_e8m0(byte == 0xFFu ? 127u : byte);
    const v2i c = byte == 0xFFu ? (v2i){0x7F7F7F7F, 0x7F7F7F7F} : quant8(v[i], m);
    if (n < N) *(v2i*)(q + (b * N + n) * K + k0 + 8 * pc) = c;
    if ((pc & 3) == 0) srow[(kb >> 2) * (kD2N * 4) + (r0 + i) * 4 + (kb & 3)] = (uint8_t)byte;
  }

  // ---- colwise: amax of each of the lane's 8 columns over the 32-row block
  us2 cm[4] = {(us2){0, 0}, (us2){0, 0}, (us2){0, 0}, (us2){0, 0}};
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d)
      cm[d] = __builtin_elementwise_max(cm[d], __builtin_bit_cast(us2, (uint32_t)v[i][d] & 0x7FFF7FFFu));
  uint32_t cbyte[8];
  float cmul[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t mine = __builtin_bit_cast(uint32_t, cm[d]);
    const uint32_t other = (uint32_t)__shfl_xor((int)mine, 32);
    const us2 both = __builtin_elementwise_max(cm[d], __builtin_bit_cast(us2, other));
    cbyte[2 * d] = e8m0_from_absbits(both[0]);
    cbyte[2 * d + 1] = e8m0_from_absbits(both[1]);
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) cmul[c] = inv_scale_from_e8m0(cbyte[c] == 0xFFu ? 127u : cbyte[c]);
  // column c (= 2d + hi) of rows r0 .. r0 + 15: 16 codes, one LDS slot
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int d = c >> 1;
    const bool hi = c & 1;
    v4i o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * j;
      const float x0 = hi ? bf16hi((uint32_t)v[i][d]) : bf16lo((uint32_t)v[i][d]);
      const float x1 = hi ? bf16hi((uint32_t)v[i + 1][d]) : bf16lo((uint32_t)v[i + 1][d]);
      const float x2 = hi ? bf16hi((uint32_t)v[i + 2][d]) : bf16lo((uint32_t)v[i + 2][d]);
      const float x3 = hi ? bf16hi((uint32_t)v[i + 3][d]) : bf16lo((uint32_t)v[i + 3][d]);
      int a = cvt2_e4m3<false>(x0 * cmul[c], x1 * cmul[c], 0);
      a = cvt2_e4m3<true>(x2 * cmul[c], x3 * cmul[c], a);
      o[j] = cbyte[c] == 0xFFu ? 0x7F7F7F7F : a;
    }
    const int k = 8 * pc + c;
    *(v4i*)(codes + k * kD2N + 16 * d2_slot(k, 2 * wv + half)) = o;
    if (half == 0) scol[(wv >> 2) * (kD2 * 4) + k * 4 + (wv & 3)] = (uint8_t)cbyte[c];
  }
  __syncthreads();

  // ---- q_t: row k of the code tile is kD2N codes of output row k0 + k
  {
    const int slot = tid % kD2Slots;
    const int64_t n = n0 + 16 * slot;
#pragma unroll
    for (int it = 0; it < kD2 * kD2Slots / kD2Threads; ++it) {
      const int k = tid / kD2Slots + (kD2Threads / kD2Slots) * it;
      const v4i x = *(const v4i*)(codes + k * kD2N + 16 * d2_slot(k, slot));
      if (n < ldq) *(v4i*)(q_t + (b * K + k0 + k) * ldq + n) = x;
    }
  }
  // ---- scales, GEMM layout: s [E][K/128][N][4], s_t [E][ldq/128][K][4]
#pragma unroll
  for (int u = 0; u < 2 * kD2N / kD2Threads && ROWWISE; ++u) {
    const int e = u * kD2Threads + tid;
    const int ch = e / kD2N, r = e % kD2N;
    if (n0 + r < N)
      *(uint32_t*)(s + b * (K / 32) * N + ((k0 >> 7) + ch) * N * 4 + (n0 + r) * 4) =
          *(const uint32_t*)(srow + ch * (kD2N * 4) + r * 4);
  }
  if (st_ld == 0) {
#pragma unroll
    for (int u = 0; u < (kD2N / 128) * kD2 / kD2Threads; ++u) {
      const int e = u * kD2Threads + tid;
      const int ch = e / kD2, r = e % kD2;
      if (n0 + 128 * ch < ldq)
        *(uint32_t*)(s_t + b * (ldq / 32) * K + ((n0 >> 7) + ch) * K * 4 + (k0 + r) * 4) =
            *(const uint32_t*)(scol + ch * (kD2 * 4) + r * 4);
    }
  } else {
    // row-major: thread t owns column k = t / 2 and four of its eight blocks
    const int k = tid >> 1, g = tid & 1;
    const uint32_t w4 = *(const uint32_t*)(scol + g * (kD2 * 4) + k * 4);
    uint8_t* sp = s_t + (b * K + k0 + k) * st_ld + (n0 >> 5) + 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((n0 >> 5) + 4 * g + j < st_ld) sp[j] = (uint8_t)(w4 >> (8 * j));
  }
}

// ---------------------------------------------------------------------------
// 32x32: x viewed as [rows, cols] (batch folded into rows; rows % 32 == 0).
// A workgroup covers 32 rows x 512 columns; wave w covers columns
// [128w, 128w+128) = four 32x32 tiles.  Lane l holds 8 columns (chunk l%16) of
// rows l/16 + 4u, u = 0..7, so every load and store instruction moves whole
// lines (16 lanes per row).  The tile amax is a wave reduction over the 16
// lanes of one tile: DPP quad max (the tile's four chunks), then
// xor-shuffles 16/32 (its four row groups).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_32x32_kernel(const uint16_t* __restrict__ x, int64_t cols,
                                                          uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int64_t r0 = (int64_t)blockIdx.y * 32;
  const int64_t col = (int64_t)blockIdx.x * 512 + wv * 128 + (lane & 15) * 8;
  const bool valid = col < cols;
  v4i w[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t row = r0 + (lane >> 4) + 4 * u;
    w[u] = valid ? __builtin_nontemporal_load((const v4i*)(x + row * cols + col)) : (v4i){0, 0, 0, 0};
  }
  uint32_t am = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) am = max(am, absmax8(w[u]));
  am = quad_max(am);
  am = max(am, (uint32_t)__shfl_xor((int)am, 16));
  am = max(am, (uint32_t)__shfl_xor((int)am, 32));
  if (!valid) return;
  const uint32_t byte = e8m0_from_absbits(am);
  const float m = inv_scale_from_e8m0(byte == 0xFFu ? 127u : byte);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t row = r0 + (lane >> 4) + 4 * u;
    v2i codes = byte == 0xFFu ? (v2i){0x7F7F7F7F, 0x7F7F7F7F} : quant8(w[u], m);
    *(v2i*)(q + row * cols + col) = codes;
  }
  if ((lane & 3) == 0 && (lane >> 4) == 0) s[(r0 >> 5) * (cols >> 5) + (col >> 5)] = (uint8_t)byte;
}

// ---------------------------------------------------------------------------
// Launchers (sizes validated by the caller).
// ---------------------------------------------------------------------------
hipError_t launch_quant_rowwise(const uint16_t* x, int64_t rows_total, int64_t cols, uint8_t* q, uint8_t* s,
                                int64_t gemm_rows_per_batch, hipStream_t st) {
  const int64_t nchunks = rows_total * (cols / 8);
  if (nchunks == 0) return hipSuccess;
  const int64_t per_block = (int64_t)kRowThreads * kRowU;
  const int64_t grid = (nchunks + per_block - 1) / per_block;
  hipLaunchKernelGGL(quant_rowwise_kernel, dim3((unsigned)grid), dim3(kRowThreads), 0, st, x, nchunks, q, s,
                     (uint32_t)(cols / 32), (uint32_t)gemm_rows_per_batch);
  return hipGetLastError();
}

hipError_t launch_quant_dual(const uint16_t* w, int64_t E, int64_t N, int64_t K, int64_t ldq, uint8_t* q,
                             uint8_t* s, uint8_t* q_t, uint8_t* s_t, hipStream_t st, const int32_t* rows,
                             int64_t src_rows, int topk) {
  if (E == 0 || ldq == 0 || K == 0) return hipSuccess;
  if (K % kD2 == 0) {
    dim3 grid((unsigned)(K / kD2), (unsigned)((ldq + kD2N - 1) / kD2N), (unsigned)E);
    hipLaunchKernelGGL(quant_dual256_kernel<true>, grid, dim3(kD2Threads), 0, st, w, N, K, ldq, q, s, q_t, s_t,
                       (int64_t)0, rows, rows ? src_rows * topk : N, (uint32_t)(rows ? topk : 1), (int64_t)E);
    return hipGetLastError();
  }
  dim3 grid((unsigned)(K / kColTile), (unsigned)(ldq / kColTile), (unsigned)E);
  hipLaunchKernelGGL(quant_dual_kernel, grid, dim3(256), 0, st, w, N, K, ldq, q, s, q_t, s_t, rows,
                     rows ? src_rows * topk : N, (uint32_t)(rows ? topk : 1));
  return hipGetLastError();
}

hipError_t launch_quant_rowwise_gather(const uint16_t* x, int64_t src_rows, const int32_t* rows, int64_t M,
                                       int64_t cols, uint8_t* q, uint8_t* s, hipStream_t st) {
  const int64_t nchunks = M * (cols / 8);
  if (nchunks == 0) return hipSuccess;
  const int64_t per_block = (int64_t)kRowThreads * kRowU;
  const int64_t grid = (nchunks + per_block - 1) / per_block;
  if (nchunks <= (int64_t)UINT32_MAX)
    hipLaunchKernelGGL(quant_rowwise_gather_kernel<true>, dim3((unsigned)grid), dim3(kRowThreads), 0, st, x, src_rows,
                       rows, nchunks, cols, q, s, (uint32_t)(cols / 8), (uint32_t)M);
  else
    hipLaunchKernelGGL(quant_rowwise_gather_kernel<false>, dim3((unsigned)grid), dim3(kRowThreads), 0, st, x, src_rows,
                       rows, nchunks, cols, q, s, (uint32_t)(cols / 8), (uint32_t)M);
  return hipGetLastError();
}

hipError_t launch_quant_colwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint8_t* q_t,
                                int64_t ldq, uint8_t* s_t, int64_t lds, int gemm_layout, hipStream_t st) {
  if (batch == 0 || rows == 0 || cols == 0) return hipSuccess;
  if (cols % kD2 == 0 && (gemm_layout ? ldq % 128 == 0 : ldq == rows)) {
    // codes of rows [rows, ldq) are zero codes (ldq rounded up to the tile)
    const int64_t tx = cols / kD2, ty = (ldq + kD2N - 1) / kD2N;
    dim3 grid((unsigned)tx, (unsigned)ty, (unsigned)batch);
    if (col_chunked(cols, ldq)) {
      const int64_t slots = (tx * ty * batch + 8 * kColChunk - 1) / (8 * kColChunk) * (8 * kColChunk);
      if (slots > (int64_t)UINT32_MAX / 2) return hipErrorInvalidValue;
      grid = dim3((unsigned)slots);
    }
    hipLaunchKernelGGL(quant_dual256_kernel<false>, grid, dim3(kD2Threads), 0, st, x, rows, cols, ldq,
                       (uint8_t*)nullptr, (uint8_t*)nullptr, q_t, s_t, gemm_layout ? (int64_t)0 : lds,
                       (const int32_t*)nullptr, rows, 1u, batch);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((cols + kColTile - 1) / kColTile), (unsigned)((rows + kColTile - 1) / kColTile),
            (unsigned)batch);
  hipLaunchKernelGGL(quant_colwise_kernel, grid, dim3(256), 0, st, x, rows, cols, q_t, ldq, s_t, lds, gemm_layout);
  return hipGetLastError();
}

// Row-major scales [batch][rows][kb] -> GEMM layout [batch][kb/4][rows][4]
// (kb % 4 == 0).  One thread per output dword (4 scale bytes).
__global__ __launch_bounds__(256) void scales_to_gemm_kernel(const uint8_t* __restrict__ s, int64_t batch,
                                                             int64_t rows, int64_t kb, uint8_t* __restrict__ out) {
  const int64_t n = batch * rows * (kb / 4);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  // output dword i = (b, c, r): c = chunk of 4 blocks
  const int64_t per_b = rows * (kb / 4);
  const int64_t b = i / per_b, rem = i - b * per_b;
  const int64_t c = rem / rows, r = rem - c * rows;
  const uint8_t* src = s + (b * rows + r) * kb + 4 * c;
  const uint32_t w = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16) | ((uint32_t)src[3] << 24);
  *(uint32_t*)(out + 4 * i) = w;
}

hipError_t launch_scales_to_gemm(const uint8_t* s, int64_t batch, int64_t rows, int64_t kb, uint8_t* out,
                                 hipStream_t st) {
  const int64_t n = batch * rows * (kb / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(scales_to_gemm_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, s, batch, rows, kb,
                     out);
  return hipGetLastError();
}

hipError_t launch_quant_32x32(const uint16_t* x, int64_t rows_total, int64_t cols, uint8_t* q, uint8_t* s,
                              hipStream_t st) {
  if (rows_total == 0 || cols == 0) return hipSuccess;
  dim3 grid((unsigned)((cols + 511) / 512), (unsigned)(rows_total / 32));
  hipLaunchKernelGGL(quant_32x32_kernel, grid, dim3(256), 0, st, x, cols, q, s);
  return hipGetLastError();
}

}  // namespace mxk
