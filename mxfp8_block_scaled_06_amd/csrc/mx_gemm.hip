// Block-scaled grouped GEMM for MoE routed experts on gfx950 (CDNA4).
//
//   C[i, j] = sum_k X[i, k] * Y[j, k] * 2^(sX[i, k/32] + sY[j, k/32] - 254)
//
// Operation: "MXFP8 training for MoEs" article, section "Is MXFP8 Training
// for MoEs Actually Stable?" (scaled grouped GEMM over the routed experts,
// output in the original precision) and "Why Does MXFP8 Speed Up MoE Training
// So Much?" (the backward mirrors the forward).  Mode 0 groups the rows of X
// by expert (forward, dgrad); mode 1 groups the contraction index (wgrad).
//
// Design for gfx950:
//  * V_MFMA_SCALE_F32_32X32X64_F8F6F4 takes the E8M0 scales per lane, so the
//    scales never leave their byte form: no dequantization pass and no
//    per-block fp32 rescaling in the main loop.
//    Operand layout of that MFMA (established by one-hot tests on the
//    hardware): lane l holds row l%32 and two 16-byte K pieces, pieces
//    (l/32) and (l/32)+2 of the instruction's 64-element K window; the scale
//    the lane supplies covers 32-element block l/32 of the window.  The
//    accumulator of lane l holds column l%32 and rows 8(r/4) + 4(l/32) + r%4.
//  * The A operand of the MFMA is Y and the B operand is X, so each lane's
//    accumulators hold four consecutive output columns of one output row:
//    the bf16 epilogue writes 8-byte runs without an LDS round trip.
//  * Workgroup tile 256 x 256 x 128 bytes, 4 waves of 128 x 128 (4x4 MFMA
//    tiles each, 256 fp32 accumulators per lane).  Operand tiles move
//    HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging), double
//    buffered (2 x 68 KiB of the 160 KiB LDS), 16-byte pieces XOR-swizzled
//    by row to spread LDS banks.
//  * Tile scheduler on the device: the group offsets never cross to the host.
//    Mode 0 enumerates (expert, M-tile) pairs from the offsets; tiles are
//    ordered in bands of 8 N-tiles so concurrently running workgroups share
//    operand rows, and the workgroup id is remapped so each XCD (workgroups
//    are dealt round-robin over the 8 XCDs) receives a contiguous slice of the
//    tile order, keeping the shared rows in that XCD's L2.
//  * Ragged groups: rows past a group end are clamped to the last valid row
//    on load and masked on store; K blocks past the end of the range (mode 1
//    group ends, or Kc not a multiple of 128) are zeroed in registers with
//    their scale forced to 1.  Empty wgrad groups store zeros.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mxk {

constexpr int kBM = 256;        // output rows per tile (rows of X)
constexpr int kBN = 256;        // output cols per tile (rows of Y)
constexpr int kBK = 128;        // contraction bytes per stage (4 scale blocks)
constexpr int kThreads = 256;   // 4 waves, 2 x 2 arrangement of 128 x 128
constexpr int kBand = 8;        // N-tiles per band in the tile order
constexpr int kTileBytes = kBM * kBK;             // 32 KiB per operand tile
constexpr int kScaleBytes = kBM * 8;              // 8 scale bytes per row staged
constexpr int kStageBytes = 2 * kTileBytes + 2 * kScaleBytes;
constexpr int kMaxExpertsLds = 1024;

static_assert(kBM == kBN, "operand tiles share the load code");

__device__ __forceinline__ int piece_swz(int row) { return (row >> 1) & 7; }

struct TileDesc {
  int valid;
  int e;
  int64_t i0, i_end;   // rows of X (output rows) covered: [i0, min(i0 + kBM, i_end))
  int64_t j0;
  int64_t k0, k1;      // contraction range [k0, k1)
};

// Wave-0 scan of per-expert M-tile counts (mode 0).  pref[e] = number of
// M-tiles of experts < e; returns the total.  Offsets are clamped to [0, I]
// and made non-decreasing so malformed offsets cannot address out of bounds.
__device__ int scan_mtiles(const int* s_offs, int E, int64_t I, int* pref) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    int tiles = 0;
    if (e < E) {
      int64_t st = e == 0 ? 0 : s_offs[e - 1];
      int64_t en = s_offs[e];
      st = min(max(st, (int64_t)0), I);
      en = min(max(en, st), I);
      tiles = (int)((en - st + kBM - 1) / kBM);
    }
    int incl = tiles;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    if (e < E) pref[e] = carry + incl - tiles;
    carry += __shfl(incl, 63);
  }
  return carry;
}

template <int MODE>
__device__ __forceinline__ TileDesc decode_tile(const GemmArgs& a, int* s_offs, int* s_pref, int* s_misc) {
  TileDesc d;
  d.valid = 0;
  const int tid = threadIdx.x;
  const int64_t ntj = (a.J + kBN - 1) / kBN;
  if (MODE == 0) {
    for (int e = tid; e < a.E; e += kThreads) s_offs[e] = a.offs[e];
    __syncthreads();
    if (tid < 64) {
      const int total_m = scan_mtiles(s_offs, a.E, a.I, s_pref);
      if (tid == 0) s_misc[0] = total_m;
    }
    __syncthreads();
    const int64_t total_m = s_misc[0];
    const int64_t total = total_m * ntj;
    const int64_t t8 = (total + 7) / 8 * 8;
    const int64_t b = blockIdx.x;
    if (b >= t8) return d;
    const int64_t t = (b & 7) * (t8 / 8) + (b >> 3);     // XCD-contiguous slice
    if (t >= total) return d;
    const int64_t band = t / (total_m * kBand);
    const int64_t within = t - band * total_m * kBand;
    const int64_t width = min((int64_t)kBand, ntj - band * kBand);
    const int64_t mt = within / width;
    const int64_t nt = band * kBand + within % width;
    // expert of M-tile mt: last e with pref[e] <= mt (binary search)
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    // experts without tiles share their successor's prefix; the search picks
    // the last expert whose prefix is <= mt, which owns tile mt
    const int e = lo;
    int64_t st = e == 0 ? 0 : s_offs[e - 1];
    int64_t en = s_offs[e];
    st = min(max(st, (int64_t)0), a.I);
    en = min(max(en, st), a.I);
    d.e = e;
    d.i0 = st + (mt - s_pref[e]) * kBM;
    d.i_end = en;
    d.j0 = nt * kBN;
    d.k0 = 0;
    d.k1 = a.Kc;
    d.valid = 1;
  } else {
    const int64_t nti = (a.I + kBM - 1) / kBM;
    const int64_t per_e = nti * ntj;
    const int64_t total = per_e * a.E;
    const int64_t t8 = (total + 7) / 8 * 8;
    const int64_t b = blockIdx.x;
    if (b >= t8) return d;
    const int64_t t = (b & 7) * (t8 / 8) + (b >> 3);
    if (t >= total) return d;
    const int e = (int)(t / per_e);
    const int64_t r = t - e * per_e;
    const int64_t band = r / (nti * kBand);
    const int64_t within = r - band * nti * kBand;
    const int64_t width = min((int64_t)kBand, ntj - band * kBand);
    const int64_t it = within / width;
    const int64_t jt = band * kBand + within % width;
    int64_t st = e == 0 ? 0 : a.offs[e - 1];
    int64_t en = a.offs[e];
    st = min(max(st, (int64_t)0), a.Kc) & ~(int64_t)31;   // group starts are multiples of 32
    en = min(max(en, st), a.Kc) & ~(int64_t)31;
    d.e = e;
    d.i0 = it * kBM;
    d.i_end = a.I;
    d.j0 = jt * kBN;
    d.k0 = st;
    d.k1 = en;
    d.valid = 1;
  }
  return d;
}

// Issue the DMA loads of one stage: operand data (8 x 1 KiB per wave per
// operand) and the 8 scale bytes per row that cover the stage's 4 blocks.
__device__ __forceinline__ void issue_stage(uint8_t* stage, const uint8_t* Xg, const uint8_t* sXg,
                                            const uint8_t* Yg, const uint8_t* sYg, int64_t x_rows_lo,
                                            int64_t x_rows_hi, int64_t y_rows_hi, int64_t ldx, int64_t ldsx,
                                            int64_t ldy, int64_t ldsy, int64_t sx_total, int64_t sy_total,
                                            int64_t kk, int64_t k0, int64_t k1) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // LDS DMA bases must be wave-uniform
  uint8_t* xs = stage;
  uint8_t* ys = stage + kTileBytes;
  uint8_t* sxs = stage + 2 * kTileBytes;
  uint8_t* sys = sxs + kScaleBytes;
  // data: 32 chunks of 1 KiB (8 rows x 128 B) per operand, 8 per wave
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = wv * 8 + u;
    const int row = c * 8 + (lane >> 3);
    const int logical = (lane & 7) ^ piece_swz(row);
    int64_t k = kk + logical * 16;
    if (k >= k1) k = k0;
    int64_t xr = x_rows_lo + row;
    if (xr > x_rows_hi) xr = x_rows_hi;
    int64_t yr = row;  // relative to Yg which already points at row j0
    if (yr > y_rows_hi) yr = y_rows_hi;
    __builtin_amdgcn_global_load_lds((const void*)(Xg + xr * ldx + k), (lds_void*)(xs + c * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(Yg + yr * ldy + k), (lds_void*)(ys + c * 1024), 16, 0, 0);
  }
  // scales: per row the aligned dword pair covering blocks kk/32 .. kk/32+3
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pos = wv * 128 + u * 64 + lane;   // 0..511: row = pos/2, dword = pos%2
    const int row = pos >> 1, dw = pos & 1;
    int64_t xr = x_rows_lo + row;
    if (xr > x_rows_hi) xr = x_rows_hi;
    int64_t yr = row;
    if (yr > y_rows_hi) yr = y_rows_hi;
    const int64_t kb = kk >> 5;
    int64_t px = ((xr * ldsx + kb) & ~(int64_t)3) + 4 * dw;
    if (px + 4 > sx_total) px -= 4;
    int64_t py = ((yr * ldsy + kb) & ~(int64_t)3) + 4 * dw;
    if (py + 4 > sy_total) py -= 4;
    __builtin_amdgcn_global_load_lds((const void*)(sXg + px), (lds_void*)(sxs + (wv * 2 + u) * 256), 4, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(sYg + py), (lds_void*)(sys + (wv * 2 + u) * 256), 4, 0, 0);
  }
}

template <int MODE, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  __shared__ int s_offs[kMaxExpertsLds];
  __shared__ int s_pref[kMaxExpertsLds];
  __shared__ int s_misc[4];

  const TileDesc td = decode_tile<MODE>(a, s_offs, s_pref, s_misc);
  if (!td.valid) return;

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int iw = wv >> 1, jw = wv & 1;   // wave's 128x128 quadrant: rows iw, cols jw
  const int half = lane >> 5, l32 = lane & 31;

  // operand bases
  const uint8_t* Xg = a.X;
  const uint8_t* sXg = a.sX;
  const uint8_t* Yg = a.Y + (MODE == 0 ? (int64_t)td.e * a.y_estride : 0) + td.j0 * a.ldy;
  const uint8_t* sYg = a.sY + (MODE == 0 ? (int64_t)td.e * a.sy_estride : 0);
  const int64_t x_rows_lo = td.i0;
  const int64_t x_rows_hi = (MODE == 0 ? td.i_end : a.I) - 1;   // clamp target (valid row)
  const int64_t y_rows_hi = a.J - 1 - td.j0;                     // relative to j0
  // scale rows are addressed absolutely: shift Y scale rows by j0
  const int64_t sy_row0 = td.j0;
  const int64_t sx_total = a.sx_total;
  const int64_t sy_total = a.sy_total_per_e;

  v16f acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = (v16f){};

  const int64_t klen = td.k1 - td.k0;
  const int nk = (int)((klen + kBK - 1) / kBK);
  // scale-row base: sY rows for this tile start at j0
  const uint8_t* sYt = sYg + sy_row0 * a.ldsy;
  const int64_t sy_total_t = sy_total - sy_row0 * a.ldsy;

  if (nk > 0) {
    issue_stage(smem, Xg, sXg, Yg, sYt, x_rows_lo, x_rows_hi, y_rows_hi, a.ldx, a.ldsx, a.ldy, a.ldsy, sx_total,
                sy_total_t, td.k0, td.k0, td.k1);
  }
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt0();
    __syncthreads();
    const int64_t kk = td.k0 + (int64_t)kt * kBK;
    if (kt + 1 < nk) {
      issue_stage(smem + ((kt + 1) & 1) * kStageBytes, Xg, sXg, Yg, sYt, x_rows_lo, x_rows_hi, y_rows_hi, a.ldx,
                  a.ldsx, a.ldy, a.ldsy, sx_total, sy_total_t, kk + kBK, td.k0, td.k1);
    }
    const uint8_t* st = smem + (kt & 1) * kStageBytes;
    const uint8_t* xs = st;
    const uint8_t* ys = st + kTileBytes;
    const uint8_t* sxs = st + 2 * kTileBytes;
    const uint8_t* sys = sxs + kScaleBytes;
    // number of valid 32-blocks in this stage (1..4)
    const int64_t rem = td.k1 - kk;
    const int nvalid = rem >= kBK ? 4 : (int)(rem >> 5);
    // byte offset of block kk/32 inside each row's staged dword pair
    const int64_t kb = kk >> 5;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8i yf[4], xf[4];
      int ysc[4], xsc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int yrow = jw * 128 + q * 32 + l32;
        const int xrow = iw * 128 + q * 32 + l32;
        // pieces 4s + half and 4s + half + 2 of the row
        const int p0 = 4 * s + half, p1 = p0 + 2;
        const v4i y0 = *(const v4i*)(ys + yrow * kBK + ((p0 ^ piece_swz(yrow)) << 4));
        const v4i y1 = *(const v4i*)(ys + yrow * kBK + ((p1 ^ piece_swz(yrow)) << 4));
        const v4i x0 = *(const v4i*)(xs + xrow * kBK + ((p0 ^ piece_swz(xrow)) << 4));
        const v4i x1 = *(const v4i*)(xs + xrow * kBK + ((p1 ^ piece_swz(xrow)) << 4));
        yf[q] = (v8i){y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
        xf[q] = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        // scale byte of block 2s + half for this row
        int64_t yr = yrow;
        if (yr > y_rows_hi) yr = y_rows_hi;
        int64_t xr = x_rows_lo + xrow;
        if (xr > x_rows_hi) xr = x_rows_hi;
        const int yoff = (int)(((yr)*a.ldsy + kb) & 3) + 2 * s + half;
        const int xoff = (int)((xr * a.ldsx + kb) & 3) + 2 * s + half;
        ysc[q] = sys[yrow * 8 + yoff];
        xsc[q] = sxs[xrow * 8 + xoff];
      }
      if (nvalid < 4) {
        // blocks 2s and 2s+1 of the stage; chunk c of each lane lies in block 2s + c,
        // the lane's scale covers block 2s + half
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            if (2 * s + c >= nvalid) {
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                yf[q][4 * c + v] = 0;
                xf[q][4 * c + v] = 0;
              }
            }
          }
          if (2 * s + half >= nvalid) {
            ysc[q] = 127;
            xsc[q] = 127;
          }
        }
      }
#pragma unroll
      for (int qy = 0; qy < 4; ++qy)
#pragma unroll
        for (int qx = 0; qx < 4; ++qx)
          acc[qy][qx] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(yf[qy], xf[qx], acc[qy][qx], 0, 0, 0,
                                                                        ysc[qy], 0, xsc[qx]);
    }
  }

  // epilogue: lane holds output row i = i0 + iw*128 + qx*32 + l32 and, for
  // register group g, columns j0 + jw*128 + qy*32 + 8g + 4*half + 0..3.
  const int64_t c_off = MODE == 1 ? (int64_t)td.e * a.c_estride : 0;
  const int64_t i_lim = MODE == 0 ? td.i_end : a.I;
#pragma unroll
  for (int qx = 0; qx < 4; ++qx) {
    const int64_t i = td.i0 + iw * 128 + qx * 32 + l32;
    if (i >= i_lim) continue;
#pragma unroll
    for (int qy = 0; qy < 4; ++qy) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t j = td.j0 + jw * 128 + qy * 32 + 8 * g + 4 * half;
        if (j < a.J) {
          const v16f& v = acc[qy][qx];
          if (OUT_F32) {
            float* crow = (float*)a.C + c_off + i * a.ldc;
            *(float4*)(crow + j) = make_float4(v[4 * g + 0], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
          } else {
            uint16_t* crow = (uint16_t*)a.C + c_off + i * a.ldc;
            v2i w;
            w[0] = (int)pack_bf16x2(v[4 * g + 0], v[4 * g + 1]);
            w[1] = (int)pack_bf16x2(v[4 * g + 2], v[4 * g + 3]);
            *(v2i*)(crow + j) = w;
          }
        }
      }
    }
  }
}

size_t gemm_lds_bytes() { return 2 * (size_t)kStageBytes; }

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t st) {
  const int64_t ntj = (a.J + kBN - 1) / kBN;
  int64_t tiles;
  if (a.mode == 0) {
    tiles = ((a.I + kBM - 1) / kBM + a.E) * ntj;   // upper bound of sum_e ceil(m_e / BM)
  } else {
    tiles = (a.I + kBM - 1) / kBM * ntj * a.E;
  }
  const int64_t grid = (tiles + 7) / 8 * 8;
  if (tiles == 0) return hipSuccess;
  const size_t lds = gemm_lds_bytes();
  const void* fn;
  if (a.out_f32) {
    fn = a.mode == 0 ? (const void*)grouped_gemm_kernel<0, true> : (const void*)grouped_gemm_kernel<1, true>;
  } else {
    fn = a.mode == 0 ? (const void*)grouped_gemm_kernel<0, false> : (const void*)grouped_gemm_kernel<1, false>;
  }
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 g3((unsigned)grid), b3(kThreads);
  if (a.mode == 0) {
    if (a.out_f32) hipLaunchKernelGGL((grouped_gemm_kernel<0, true>), g3, b3, lds, st, a);
    else hipLaunchKernelGGL((grouped_gemm_kernel<0, false>), g3, b3, lds, st, a);
  } else {
    if (a.out_f32) hipLaunchKernelGGL((grouped_gemm_kernel<1, true>), g3, b3, lds, st, a);
    else hipLaunchKernelGGL((grouped_gemm_kernel<1, false>), g3, b3, lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace mxk
