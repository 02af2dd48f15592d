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
//    accumulators hold runs of four consecutive output columns of one output
//    row; trading runs with lane l ^ 32 gives 8-column (16-byte) pieces,
//    which the bf16 epilogue stages through the idle LDS so the global
//    stores write whole 512-byte row segments.
//  * Workgroup tile 256 x 256, 8 waves (two per SIMD) of 128 x 64 (4 x 2
//    MFMA tiles each, 128 fp32 accumulators per lane).  Stages of 128 contraction
//    bytes: every row moves as one full 128-byte line, HBM/L2 -> LDS by
//    buffer_load ... lds (no VGPR staging), two stages of 68 KiB in LDS.
//    Buffer descriptors end at the last valid row, so rows past a group end
//    read as zeros without clamping code.  Scales use the GEMM layout
//    [K/128][rows][4] so one stage's scales for 256 rows are one 1 KiB line
//    run per operand.
//  * The operand stream bounds this loop: a stage moves 66 KiB per CU from
//    L2 into LDS through the CU's texture data path, which on gfx950 takes
//    about three quarters as long as the stage's MFMAs and overlaps with
//    them only in part (counters show that path busy ~80% of the kernel's
//    cycles, the LDS ~15%).  A 256 x 256 tile is the largest whose fp32
//    accumulators fit a CU's registers, so the bytes per flop cannot drop;
//    the loop is built to keep the matrix cores fed while the stream runs.
//    Waves 0..3 (one per SIMD: the hardware deals a workgroup's waves
//    round-robin over the SIMDs) issue all of the DMA; waves 4..7 only read
//    LDS and run MFMAs, so while a loading wave waits on a full address
//    queue the other wave of its SIMD keeps the matrix core busy.  Each
//    wave reads the next window's fragments while the current window's
//    MFMAs run: its X sub-tile registers are refilled right after their last
//    MFMA of the window, its Y sub-tiles alternate between two register
//    sets.  One barrier per stage, at the start of its second window: every
//    wave has then finished reading the stage's buffer, which receives the
//    DMA of the stage after next (two loads per MFMA of the loading waves
//    across the window), and the next stage has landed.  Fragment addresses are a
//    per-lane base (row and swizzled piece) per window and operand plus a
//    constant: the 32-row sub-tile rides in the LDS immediate offset, so the
//    loop spends about a dozen vector adds per stage on addressing.
//  * Tile scheduler on the device: the group offsets never cross to the host.
//    Mode 0 enumerates (expert, M-tile) pairs from the offsets; tiles are
//    ordered in bands of 8 N-tiles, expert by expert inside a band with all
//    of an expert's M-tiles together per N-tile, so concurrently running
//    workgroups share operand rows.  Workgroups are dealt round-robin over
//    the 8 XCDs by the hardware; the workgroup id is remapped so that chunks
//    of 16 consecutive tiles of the order land on one XCD (its L2 sees their
//    shared rows) and successive chunks go to successive XCDs, so every XCD
//    gets a slice of every expert however the tokens are routed.
//  * The stage loop is compiled per case and each variant is one straight
//    block: a group's last, partial M-tile runs a loop without the MFMAs and
//    fragment reads of the 32-row X sub-tiles past the group end.
//  * K blocks outside a wgrad group are zeroed in registers with a neutral
//    scale, at a fragment's first use and only in a tile's first and last
//    stage; empty wgrad groups store zeros.
#include "mx_device.h"
#include "mx_kernels.h"

#include <type_traits>

namespace mxk {

constexpr int kBM = 256;        // output rows per tile (rows of X)
constexpr int kBN = 256;        // output cols per tile (rows of Y)
constexpr int kBK = 128;        // contraction bytes per stage (4 scale blocks, 2 MFMA windows)
constexpr int kThreads = 512;   // 8 waves (two per SIMD), 2 x 4 arrangement of 128 x 64 blocks
constexpr int kBand = 8;        // N-tiles per band in the tile order
constexpr int kXcdChunk = 16;   // consecutive tiles of the order dealt to one XCD at a time
constexpr int kTileBytes = kBM * kBK;             // 32 KiB per operand tile
constexpr int kScaleChunk = kBM * 4;              // one [rows][4] scale chunk: 1 KiB
constexpr int kStageBytes = 2 * kTileBytes + 4 * kScaleChunk;
constexpr int kDmaPerStage = 8 + 8 + 1;           // per loading wave (0..3): X data, Y data, one scale chunk
constexpr int kMaxExpertsLds = 1024;
constexpr int kOutPitch = kBN * 2 + 16;          // bytes per staged bf16 output row (+16: spreads banks)
constexpr int kRsrcWord3 = 0x00020000;            // raw buffer, 32-bit elements (gfx9 family)

static_assert(kBM == kBN, "operand tiles share the load code");
static_assert(kBM * kOutPitch <= 2 * kStageBytes, "the bf16 output tile fits the stage buffers");

// 16-byte piece swizzle of a 128-byte LDS row: the 32 lanes that read one
// logical piece of 32 consecutive rows spread over all bank groups.
__device__ __forceinline__ int piece_swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int uni32(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

struct TileDesc {
  int valid;
  int e;
  int64_t i0, i_end;   // rows of X (output rows) covered: [i0, min(i0 + kBM, i_end))
  int64_t j0;
  int64_t k0, k1;      // contraction stages cover [k0, k1), k0 a multiple of kBK
  int64_t k_lo;        // blocks before k_lo are masked (a wgrad group start)
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

// Position in the tile order of workgroup b.  The hardware deals workgroups
// round-robin over the 8 XCDs (b % 8); that XCD's i-th workgroup (i = b / 8)
// takes tile i % kXcdChunk of the XCD's (i / kXcdChunk)-th chunk, and chunks
// of kXcdChunk consecutive tiles go round-robin to the XCDs.  Neighbouring
// tiles of the order (one expert's M-tiles of an N-tile, or one band row)
// share an XCD and its L2, while every XCD gets a slice of every expert: tile
// costs differ (a group's partial last M-tile; in wgrad, the group size), and
// whole experts per XCD left the XCDs unevenly loaded.
__device__ __forceinline__ int64_t tile_of_workgroup(int64_t b) {
  const int64_t i = b >> 3;
  return ((i / kXcdChunk) * 8 + (b & 7)) * kXcdChunk + i % kXcdChunk;
}

// Tile of workgroup b: the XCD-aware order, or (race checks) a seeded
// bijection of it over the grid (mul is coprime with the grid size).
__device__ __forceinline__ int64_t ordered_tile(const GemmArgs& a, int64_t b) {
  const int64_t t = tile_of_workgroup(b);
  return a.order_mul ? (int64_t)(((uint64_t)t * (uint64_t)a.order_mul + (uint64_t)a.order_add) % gridDim.x) : t;
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
    const int64_t t = ordered_tile(a, blockIdx.x);
    if (t >= total) return d;
    // Inside a band of `width` N-tiles, expert e owns positions
    // [pref[e] * width, pref[e+1] * width): its N-tiles in turn, and for each
    // all of its M-tiles, so consecutive tiles (one XCD chunk) share a weight
    // row panel.
    const int64_t band = t / (total_m * kBand);
    const int64_t within = t - band * total_m * kBand;
    const int64_t width = min((int64_t)kBand, ntj - band * kBand);
    const int64_t mw = within / width;
    // expert owning M-tile mw: the last e with pref[e] <= mw (experts without
    // tiles share their successor's prefix and are skipped by this rule)
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= mw) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int64_t cnt = (e + 1 < a.E ? (int64_t)s_pref[e + 1] : total_m) - s_pref[e];
    const int64_t r = within - (int64_t)s_pref[e] * width;
    const int64_t mt = s_pref[e] + r % cnt;
    const int64_t nt = band * kBand + r / cnt;
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
    d.k_lo = 0;
    d.valid = 1;
  } else {
    const int64_t nti = (a.I + kBM - 1) / kBM;
    const int64_t per_e = nti * ntj;
    const int64_t total = per_e * a.E;
    const int64_t t = ordered_tile(a, blockIdx.x);
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
    // whole lines and one scale chunk per stage; an empty group has no stages
    d.k0 = en > st ? (st & ~(int64_t)(kBK - 1)) : st;
    d.k1 = en;
    d.k_lo = st;
    d.valid = 1;
  }
  return d;
}

// Per-tile load state.  Descriptor bases/extents are wave-uniform (SGPRs);
// the per-lane byte offsets of this lane's 16-byte pieces are fixed for the
// whole tile, so a stage's loads cost no vector ALU work.
struct LoadState {
  const uint8_t* xb;      // X row i0
  const uint8_t* yb;      // Y row j0 (expert e in mode 0)
  const uint8_t* sxb;     // X scales, chunk 0, row i0
  const uint8_t* syb;     // Y scales, chunk 0, row j0
  int64_t x_bytes, y_bytes;         // valid data bytes from xb / yb
  int64_t sx_chunk, sy_chunk;       // bytes between scale chunks (rows x 4)
  int64_t sx_rows4, sy_rows4;       // valid scale bytes per chunk from sxb / syb
  int64_t nchunks;                  // scale chunks per row (Kc / 128)
  int voff[2];                      // data piece offsets of loads u = 0, 1 (X and Y share the row stride)
  int ldx16;                        // bytes of 16 rows: load u + 2 is 16 rows below load u (same swizzle)
};

// DMA of one stage (contraction bytes [k0 + 128*stage_no, +128)) into LDS
// buffer `buf`, issued by the loading waves wv = 0..3: per wave 8 + 8 one-KiB
// data loads (rows 64*wv .. +63 of X and Y) and one scale load: stages start
// on a multiple of 128 bytes, so a stage's scales are the single 1 KiB chunk
// q = kk / 128 per operand, loaded by wave 0 (X) and wave 2 (Y); waves 1 and
// 3 issue an empty load into their own slot.  Stages at or past `ns` get
// empty ranges: no data moves, but every loading wave still issues its 17
// loads so the vmcnt bookkeeping is the same for every stage.
struct StageDma {
  __amdgpu_buffer_rsrc_t rx, ry, rs;
  uint8_t* st;
};

__device__ __forceinline__ StageDma make_stage_dma(uint8_t* smem, int buf, const LoadState& L, int64_t k0,
                                                   int stage_no, int ns, int wv) {
  StageDma d;
  d.st = smem + buf * kStageBytes;
  const bool live = stage_no < ns;
  const int64_t kk = k0 + (int64_t)stage_no * kBK;
  d.rx = make_rsrc(L.xb + kk, live ? L.x_bytes - kk : 0);
  d.ry = make_rsrc(L.yb + kk, live ? L.y_bytes - kk : 0);
  const int64_t q = kk / kBK;
  const bool need = live && q < L.nchunks && (wv & 1) == 0;
  const bool is_x = wv < 2;
  const uint8_t* sbase = is_x ? L.sxb + q * L.sx_chunk : L.syb + q * L.sy_chunk;
  d.rs = make_rsrc(sbase, need ? (is_x ? L.sx_rows4 : L.sy_rows4) : 0);
  return d;
}

// Load number `n` (0..16) of a stage's DMA for this wave: even n < 16 move X
// rows, odd n < 16 Y rows, n == 16 the scale chunk.
template <int n>
__device__ __forceinline__ void issue_load(const StageDma& d, const LoadState& L, int wv, int lane) {
  if (n < 16) {
    const int u = n >> 1;
    const int c = wv * 8 + u;   // 1 KiB chunk = 8 rows x 128 B
    const int vo = L.voff[u & 1] + (u >> 1) * L.ldx16;
    if ((n & 1) == 0) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rx, (lds_void*)(d.st + c * 1024), 16, vo, 0, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ry, (lds_void*)(d.st + kTileBytes + c * 1024), 16, vo, 0, 0,
                                               0);
    }
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rs, (lds_void*)(d.st + 2 * kTileBytes + wv * kScaleChunk), 16,
                                             lane * 16, 0, 0, 0);
  }
}

template <int first, int count>
__device__ __forceinline__ void issue_loads(const StageDma& d, const LoadState& L, int wv, int lane) {
  if constexpr (count > 0) {
    issue_load<first>(d, L, wv, lane);
    issue_loads<first + 1, count - 1>(d, L, wv, lane);
  }
}

// One MFMA operand: 32 rows x 64 K of E4M3 (two 16-byte pieces per lane)
// and the lane's E8M0 scale byte.
struct Frag {
  v8i v;
  int s;
};

// Contraction-block mask of one MFMA window (wgrad: blocks of a stage that
// lie outside the expert's group).  keep0/keep1 cover the window's two
// blocks (the fragment's first and second 16-byte piece); `sel` is the byte
// permute that keeps the lane's scale or substitutes the neutral 127.
struct WinMask {
  int keep0, keep1;
  unsigned sel;
};

// Valid stage-relative blocks are [vr & 255, vr >> 8).
__device__ __forceinline__ WinMask make_mask(int vr, int w, int half) {
  const int vlo = vr & 255, vhi = vr >> 8;
  const int b0 = 2 * w, b1 = 2 * w + 1, bh = 2 * w + half;
  WinMask m;
  m.keep0 = (b0 >= vlo && b0 < vhi) ? -1 : 0;
  m.keep1 = (b1 >= vlo && b1 < vhi) ? -1 : 0;
  m.sel = 0x0c0c0c00u | ((bh >= vlo && bh < vhi) ? 0u : 4u);
  return m;
}

// Zero a fragment's masked blocks and neutralise its scale.  The scale goes
// through a byte permute: written as a select, the compiler turns it into a
// divergent branch around the scale load, which splits the main loop into
// blocks and lets MFMAs sink past the stage barrier.
__device__ __forceinline__ void mask_frag(Frag& f, const WinMask& m) {
  f.v &= (v8i){m.keep0, m.keep0, m.keep0, m.keep0, m.keep1, m.keep1, m.keep1, m.keep1};
  f.s = (int)__builtin_amdgcn_perm(127u, (unsigned)f.s, m.sel);
}

// Valid-block range of the stage starting at contraction byte kk, packed as
// lo | hi << 8 (stage-relative blocks 0..4).
__device__ __forceinline__ int stage_valid(int64_t kk, int64_t k_lo, int64_t k1) {
  const int64_t lo = k_lo > kk ? (k_lo - kk) >> 5 : 0;
  const int64_t hi = k1 > kk ? (k1 - kk) >> 5 : 0;
  return (int)min(lo, (int64_t)4) | ((int)min(hi, (int64_t)4) << 8);
}

__device__ __forceinline__ v16f mfma(const Frag& y, const Frag& x, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(y.v, x.v, c, 0, 0, 0, y.s, 0, x.s);
}

// All of this wave's loads have landed (the next stage), then workgroup
// barrier.  One asm statement with a memory clobber: no LDS access moves
// across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
static_assert(kDmaPerStage == 17, "the prologue waits with vmcnt(17)");

#define MX_FENCE() __builtin_amdgcn_sched_barrier(0)

template <int M, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (M < N) {
    f(std::integral_constant<int, M>{});
    static_for<M + 1, N>(f);
  }
}

template <int MODE, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  __shared__ int s_offs[MODE == 0 ? kMaxExpertsLds : 1];
  __shared__ int s_pref[MODE == 0 ? kMaxExpertsLds : 1];
  __shared__ int s_misc[4];

  const TileDesc td0 = decode_tile<MODE>(a, s_offs, s_pref, s_misc);
  if (!td0.valid) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = uni32(tid >> 6);
  const int iw = wv >> 2, jw = wv & 3;   // wave's 128 x 64 block: X rows iw * 128, Y rows jw * 64
  const int half = lane >> 5, l32 = lane & 31;

  // tile description, made wave-uniform (it is identical for every thread)
  const int e = uni32(td0.e);
  const int64_t i0 = uni64(td0.i0), i_end = uni64(td0.i_end), j0 = uni64(td0.j0);
  const int64_t k0 = uni64(td0.k0), k1 = uni64(td0.k1), k_lo = uni64(td0.k_lo);
  const int64_t x_end = MODE == 0 ? i_end : a.I;
  const int64_t rows_x = min((int64_t)kBM, x_end - i0);
  const int64_t rows_y = min((int64_t)kBN, a.J - j0);

  LoadState L;
  L.xb = a.X + i0 * a.ldx;
  L.yb = a.Y + (MODE == 0 ? (int64_t)e * a.y_estride : 0) + j0 * a.ldx;
  L.sx_chunk = a.I * 4;
  L.sy_chunk = a.J * 4;
  L.sxb = a.sX + i0 * 4;
  L.syb = a.sY + (MODE == 0 ? (int64_t)e * a.sy_estride : 0) + j0 * 4;
  L.x_bytes = rows_x * a.ldx;
  L.y_bytes = rows_y * a.ldx;
  L.sx_rows4 = (a.I - i0) * 4;     // rows past a group end hold a neighbour's (finite) scales
  L.sy_rows4 = (a.J - j0) * 4;
  L.nchunks = a.Kc / kBK;
  L.ldx16 = 16 * (int)a.ldx;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = ((wv & 3) * 8 + u) * 8 + (lane >> 3);
    L.voff[u] = row * (int)a.ldx + (((lane & 7) ^ piece_swz(row)) << 4);
  }

  v16f acc[2][4];
#pragma unroll
  for (int y = 0; y < 2; ++y)
#pragma unroll
    for (int x = 0; x < 4; ++x) acc[y][x] = (v16f){};

  const int ns = (int)((k1 - k0 + kBK - 1) / kBK);
  if (ns > 0) {
    // this lane's rows and piece offsets (the swizzle depends only on l32)
    const int sw = piece_swz(l32);
    int pc[2][2];   // [window][chunk] byte offset of the piece inside a row
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
      for (int c = 0; c < 2; ++c) pc[w][c] = ((4 * w + half + 2 * c) ^ sw) << 4;
    const int yrow0 = jw * 64 + l32, xrow0 = iw * 128 + l32;
    // Operands: X sub-tiles qx = 0..3 in FX[0..2] and FX[3 + window] (the last
    // X sub-tile alternates between two registers so its refill never waits
    // for the window's last MFMA), Y sub-tiles qy = 0..1 in FY[window][qy].
    // A window's MFMAs run X sub-tile by X sub-tile, so FX[qx] is refilled for
    // the next window right after its second MFMA.
    Frag FX[5], FY[2][2];
    // Y's fragments sit a wave-uniform distance from X's (same lane row and
    // piece swizzle), so only X's per-lane offsets are held and Y's read
    // goes through a shifted stage base
    int xo[2][2];
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
      for (int c = 0; c < 2; ++c) xo[w][c] = xrow0 * kBK + pc[w][c];
    const int sxo = 2 * kTileBytes + xrow0 * 4 + half;
    const int ydelta = uni32(kTileBytes + (yrow0 - xrow0) * kBK);
    const int sdelta = uni32(2 * kScaleChunk + (yrow0 - xrow0) * 4);
    // sub-tile `sub` of operand X (isx) or Y, window `w`, stage buffer `st`
    auto read = [&](const uint8_t* st, int w, bool isx, int sub, Frag& dst) {
      const uint8_t* sb = st + (isx ? 0 : ydelta);
      const uint8_t* p0 = sb + xo[w][0] + sub * 32 * kBK;
      const uint8_t* p1 = sb + xo[w][1] + sub * 32 * kBK;
      const uint8_t* ps = st + (isx ? 0 : sdelta) + sxo + sub * 32 * 4 + 2 * w;
      const v4i a0 = *(const v4i*)p0;
      const v4i a1 = *(const v4i*)p1;
      dst.s = *ps;
      dst.v = (v8i){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    };

    // One MFMA window: MFMA m = (qx = m / 2, qy = m % 2) from the current
    // registers while the next window's operands are read from `src`
    // (window NW of that stage buffer); with LOADS (a loading wave's second
    // window), DMA loads 2m and 2m + 1 of the stage after next go out with
    // MFMA m, the scale chunk with the first.  NXS = X sub-tiles of this wave
    // that hold rows of the tile (a group's last M-tile may be partial: MFMAs
    // and fragment reads of sub-tiles past its end are not compiled in);
    // MASK = the stage has contraction blocks outside the wgrad group, zeroed
    // where a fragment is first used rather than where it is read (an LDS
    // wait right after each read would stall the MFMAs the read overlaps).
    // Each variant is one straight-line block, so its schedule is the one
    // written here.
    auto window = [&](auto w_c, auto nxs_c, auto mask_c, auto loads_c, const uint8_t* src, const WinMask& mk,
                      const StageDma& pend) __attribute__((always_inline)) {
      constexpr int W = decltype(w_c)::value, NW = W ^ 1;
      constexpr int NXS = decltype(nxs_c)::value;
      constexpr bool MASK = decltype(mask_c)::value;
      constexpr bool LOADS = decltype(loads_c)::value;
      static_for<0, 8>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        constexpr int qx = m >> 1, qy = m & 1;
        constexpr int xi = qx < 3 ? qx : 3 + W;
        if constexpr (qx < NXS) {
          if constexpr (MASK) {
            if (qy == 0) mask_frag(FX[xi], mk);
            if (qx == 0) mask_frag(FY[W][qy], mk);
          }
          acc[qy][qx] = mfma(FY[W][qy], FX[xi], acc[qy][qx]);
        }
        if constexpr (LOADS) {
          issue_load<2 * m>(pend, L, wv, lane);
          issue_load<2 * m + 1>(pend, L, wv, lane);
          if constexpr (m == 0) issue_load<16>(pend, L, wv, lane);
        }
        if constexpr (NXS > 0) {
          if constexpr (m < 2) read(src, NW, false, m, FY[NW][m]);
          if constexpr (m == 0 && NXS > 3) read(src, NW, true, 3, FX[3 + NW]);
          if constexpr (m == 1 || m == 3 || m == 5) {
            if constexpr ((m >> 1) < NXS) read(src, NW, true, m >> 1, FX[m >> 1]);
          }
        }
        MX_FENCE();
      });
    };

    // One stage: window 0 from the registers (reading window 1 of this
    // stage), barrier, window 1 (reading window 0 of the next stage; loading
    // waves issue the DMA of the stage after next into this stage's buffer).
    auto stage = [&](auto nxs_c, auto mask_c, auto dma_c, int kt) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_c)::value;
      const int buf = kt & 1;
      const uint8_t* cs = smem + buf * kStageBytes;
      const uint8_t* nst = smem + (buf ^ 1) * kStageBytes;
      const int64_t kk = k0 + (int64_t)kt * kBK;
      WinMask mk0{}, mk1{};
      if (MASK) {
        const int nvalid = stage_valid(kk, k_lo, k1);
        mk0 = make_mask(nvalid, 0, half);
        mk1 = make_mask(nvalid, 1, half);
      }
      const StageDma none{};
      window(std::integral_constant<int, 0>{}, nxs_c, mask_c, std::false_type{}, cs, mk0, none);
      stage_barrier();   // stage kt+1 landed; every wave is done reading buffer `buf`
      const StageDma pend = make_stage_dma(smem, buf, L, k0, kt + 2, ns, wv);
      window(std::integral_constant<int, 1>{}, nxs_c, mask_c, dma_c, nst, mk1, pend);
    };

    // DMA_C: this is a loading wave (waves 0..3, one per SIMD); waves 4..7
    // issue no DMA and only read LDS and run MFMAs
    auto run = [&](auto nxs_c, auto dma_c) __attribute__((always_inline)) {
      constexpr int NXS = decltype(nxs_c)::value;
      if constexpr (decltype(dma_c)::value) {
        const StageDma d0 = make_stage_dma(smem, 0, L, k0, 0, ns, wv);
        issue_loads<0, 17>(d0, L, wv, lane);
        const StageDma d1 = make_stage_dma(smem, 1, L, k0, 1, ns, wv);
        issue_loads<0, 17>(d1, L, wv, lane);
      }
      asm volatile("s_waitcnt vmcnt(17) lgkmcnt(0)\n\ts_barrier" ::: "memory");   // stage 0 has landed
      if constexpr (NXS > 0) {
        read(smem, 0, false, 0, FY[0][0]);
        read(smem, 0, false, 1, FY[0][1]);
      }
      static_for<0, 4>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        if constexpr (f < NXS) read(smem, 0, true, f, FX[f < 3 ? f : 3]);
      });
      if (MODE == 1) {
        // only a wgrad tile's first and last stage can hold blocks outside
        // its group (stages are whole 128-byte lines of the group's span)
        stage(nxs_c, std::true_type{}, dma_c, 0);
        for (int kt = 1; kt < ns - 1; ++kt) stage(nxs_c, std::false_type{}, dma_c, kt);
        if (ns > 1) stage(nxs_c, std::true_type{}, dma_c, ns - 1);
      } else {
        for (int kt = 0; kt < ns; ++kt) stage(nxs_c, std::false_type{}, dma_c, kt);
      }
    };
    // X sub-tiles of this wave inside the tile (mode 1 tiles are whole in X)
    const int nxs = MODE == 0 ? (int)min(max((rows_x - iw * 128 + 31) >> 5, (int64_t)0), (int64_t)4) : 4;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    auto by_nxs = [&](auto dma_c) __attribute__((always_inline)) {
      if (MODE == 1 || nxs >= 4) run(I4{}, dma_c);
      else if (nxs == 3) run(I3{}, dma_c);
      else if (nxs == 2) run(I2{}, dma_c);
      else if (nxs == 1) run(I1{}, dma_c);
      else run(I0{}, dma_c);
    };
    if (wv < 4) by_nxs(std::true_type{});
    else by_nxs(std::false_type{});
    // drain the empty-range loads still in flight before the workgroup ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // epilogue: lane holds output row i = i0 + iw*128 + qx*32 + l32 and, for
  // register group g, columns j0 + jw*64 + qy*32 + 8g + 4*half + 0..3.
  const int64_t c_off = MODE == 1 ? (int64_t)e * a.c_estride : 0;
  const int64_t i_lim = x_end;
  if (OUT_F32) {
    // destination rows first: a load issued after a store waits for it
    int64_t dsts[4];
#pragma unroll
    for (int qx = 0; qx < 4; ++qx) {
      const int64_t i = i0 + iw * 128 + qx * 32 + l32;
      dsts[qx] = i >= i_lim ? -1 : (a.row_map ? (int64_t)a.row_map[i] : i);
    }
#pragma unroll
    for (int qx = 0; qx < 4; ++qx) {
      const int64_t dst = dsts[qx];
      if (dst < 0 || dst >= a.c_rows) continue;
#pragma unroll
      for (int qy = 0; qy < 2; ++qy) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t j = j0 + jw * 64 + qy * 32 + 8 * g + 4 * half;
          if (j < a.J) {
            const v16f& v = acc[qy][qx];
            float* crow = (float*)a.C + c_off + dst * a.ldc;
            *(float4*)(crow + j) = make_float4(v[4 * g + 0], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
          }
        }
        // one 32x32 tile at a time: keeps the accumulator reads from being
        // hoisted all at once (register pressure)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    // bf16: the tile goes through the (now idle) LDS stage buffers so every
    // store instruction writes two whole 512-byte row segments instead of
    // 16-byte pieces of 32 rows.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");   // nobody reads the stages now
    uint8_t* ot = smem;   // [256 rows][kOutPitch bytes]
#pragma unroll
    for (int qx = 0; qx < 4; ++qx) {
      const int row = iw * 128 + qx * 32 + l32;
#pragma unroll
      for (int qy = 0; qy < 2; ++qy) {
        const v16f& v = acc[qy][qx];
        // register group g holds columns 8g + 4*half + 0..3.  Trading groups
        // with the partner lane l ^ 32 (group 0 of the upper half for group 1
        // of the lower, 2 for 3) leaves each lane 8 consecutive columns,
        // 8*half + 16p + 0..7 for p = 0, 1: two 16-byte LDS writes, which
        // with the 528-byte row pitch hit all banks once per 8 lanes.
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const int g0 = 2 * pr, g1 = 2 * pr + 1;
          const unsigned a0 = pack_bf16x2_rne(v[4 * g0 + 0], v[4 * g0 + 1]);
          const unsigned a1 = pack_bf16x2_rne(v[4 * g0 + 2], v[4 * g0 + 3]);
          const unsigned b0 = pack_bf16x2_rne(v[4 * g1 + 0], v[4 * g1 + 1]);
          const unsigned b1 = pack_bf16x2_rne(v[4 * g1 + 2], v[4 * g1 + 3]);
          // lanes < 32 get (own group g0, partner's g0); lanes >= 32 get
          // (partner's g1, own g1)
          const auto x = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
          const auto y = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
          const v4i w = {(int)x[0], (int)y[0], (int)x[1], (int)y[1]};
          const int col = jw * 64 + qy * 32 + 16 * pr + 8 * half;
          *(v4i*)(ot + row * kOutPitch + col * 2) = w;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    // thread t: 16 bytes (8 columns) of row 16*it + t/32; the J % 8 == 0
    // contract makes an 8-column group wholly valid or wholly past J.
    // Streaming (nontemporal) stores: the output is not read back here and
    // should not evict the operand rows the other workgroups share in L2.
    const int c8 = (tid & 31) * 8;
    const int64_t j = j0 + c8;
    // with a row map (routed tokens) each row goes back to its token's place;
    // the thread's 16 map entries are loaded before any store, since a load
    // issued after a store waits for it (one counter for both)
    int rmv[kBM / 16];
#pragma unroll
    for (int it = 0; it < kBM / 16; ++it) {
      const int64_t i = i0 + it * 16 + (tid >> 5);
      rmv[it] = a.row_map != nullptr && i < i_lim ? a.row_map[i] : -1;
    }
#pragma unroll 4
    for (int it = 0; it < kBM / 16; ++it) {
      const int row = it * 16 + (tid >> 5);
      const int64_t i = i0 + row;
      const v4i w = *(const v4i*)(ot + row * kOutPitch + c8 * 2);
      const int64_t dst = i < i_lim ? (a.row_map ? (int64_t)rmv[it] : i) : -1;
      if (dst >= 0 && dst < a.c_rows && j < a.J)
        __builtin_nontemporal_store(w, (v4i*)((uint16_t*)a.C + c_off + dst * a.ldc + j));
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
  // chunks of kXcdChunk tiles go round-robin to the 8 XCDs (tile_of_workgroup):
  // every XCD gets as many workgroups as the XCD with the most chunks needs
  const int64_t grid = ((tiles + kXcdChunk - 1) / kXcdChunk + 7) / 8 * 8 * kXcdChunk;
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
