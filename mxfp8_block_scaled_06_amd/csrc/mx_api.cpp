// C ABI of the MXFP8 MoE hot path (declared in include/mxmoe.h).
//
// Host-side only: argument validation with a clear error on every
// unsupported setting (the "feat(moe): add MoK MXFP8 expert support" PR
// rejects unsupported configurations with a clear error and raises on a
// mismatched weight/precision contract), workspace carving, and kernel
// launches on the caller's stream.  Nothing here allocates, frees or
// synchronizes.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "mx_kernels.h"
#include "mxmoe.h"

namespace {

thread_local std::string g_last_error;

mx_status fail(mx_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mx_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MX_OK;
  return fail(MX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The rowwise quantizers index scale bytes with 32-bit integers: a launch
// covers fewer than 2^32 blocks of 32 (about 256 GiB of bf16 input).
bool rowwise_blocks_fit(int64_t rows, int64_t cols) { return rows * (cols / 32) < ((int64_t)1 << 32); }
int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Checks shared by the quantizers.
mx_status check_quant(const char* fn, const void* x, int64_t batch, int64_t rows, int64_t cols, const void* q,
                      const void* s, int64_t row_mult, int64_t col_mult) {
  if (batch < 1) return fail(MX_ERR_SHAPE, "%s: batch must be >= 1 (got %lld)", fn, (long long)batch);
  if (rows < 0 || cols < 0) return fail(MX_ERR_SHAPE, "%s: negative size rows=%lld cols=%lld", fn, (long long)rows,
                                        (long long)cols);
  if (rows % row_mult != 0)
    return fail(MX_ERR_SHAPE, "%s: rows=%lld is not a multiple of %lld", fn, (long long)rows, (long long)row_mult);
  if (cols % col_mult != 0)
    return fail(MX_ERR_SHAPE, "%s: cols=%lld is not a multiple of %lld", fn, (long long)cols, (long long)col_mult);
  if (rows == 0 || cols == 0) return MX_OK;
  if (!x || !q || !s) return fail(MX_ERR_NULL, "%s: null pointer (x=%p q=%p s=%p)", fn, x, q, s);
  if (!aligned(x, 16) || !aligned(q, 16))
    return fail(MX_ERR_ALIGN, "%s: x and q must be 16-byte aligned (x=%p q=%p)", fn, x, q);
  return MX_OK;
}

struct WsLayout {
  size_t off[4];
  size_t total;
};

// Workspace regions: [X codes, X scales, Y codes, Y scales], 256-byte aligned.
WsLayout ws_layout(int op, int64_t M, int64_t N, int64_t K, int64_t E) {
  WsLayout L{};
  size_t sz[4];
  if (op == MX_OP_FWD) {
    sz[0] = (size_t)M * K;
    sz[1] = (size_t)M * (K / 32);
    sz[2] = (size_t)E * N * K;
    sz[3] = (size_t)E * N * (K / 32);
  } else if (op == MX_OP_FWD_Q) {
    sz[0] = (size_t)M * K;
    sz[1] = (size_t)M * (K / 32);
    sz[2] = sz[3] = 0;
  } else if (op == MX_OP_DGRAD_Q) {
    sz[0] = (size_t)M * N;
    sz[1] = (size_t)M * (N / 32);
    sz[2] = sz[3] = 0;
  } else if (op == MX_OP_DGRAD) {
    sz[0] = (size_t)M * N;
    sz[1] = (size_t)M * (N / 32);
    sz[2] = (size_t)E * K * N;
    sz[3] = (size_t)E * K * (N / 32);
  } else {
    const int64_t Mp = round_up(M, 128);
    sz[0] = (size_t)N * Mp;
    sz[1] = (size_t)N * (Mp / 32);
    sz[2] = (size_t)K * Mp;
    sz[3] = (size_t)K * (Mp / 32);
  }
  size_t o = 0;
  for (int i = 0; i < 4; ++i) {
    L.off[i] = o;
    o = align_up(o + sz[i], 256);
  }
  L.total = o;
  return L;
}

mx_status check_mm(const char* fn, const void* a, const void* b, const void* offs, const void* out, int64_t M,
                   int64_t N, int64_t K, int64_t E) {
  if (M < 0 || N < 0 || K < 0) return fail(MX_ERR_SHAPE, "%s: negative size M=%lld N=%lld K=%lld", fn,
                                           (long long)M, (long long)N, (long long)K);
  if (E < 1 || E > mxk::kMaxExperts)
    return fail(MX_ERR_SHAPE, "%s: number of experts E=%lld outside [1, %d]", fn, (long long)E, mxk::kMaxExperts);
  if (!a || !b || !offs || !out) return fail(MX_ERR_NULL, "%s: null pointer", fn);
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(out, 16) || !aligned(offs, 4))
    return fail(MX_ERR_ALIGN, "%s: tensors must be 16-byte aligned", fn);
  return MX_OK;
}

}  // namespace

mx_status mxk::set_last_error(mx_status st, const char* text) {
  g_last_error = text;
  return st;
}

extern "C" {

const char* mx_last_error(void) { return g_last_error.c_str(); }

const char* mx_version(void) { return "mxmoe 0.1.0 (gfx950)"; }

mx_status mx_quantize_rowwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s,
                              void* stream) {
  mx_status st = check_quant("mx_quantize_rowwise", x, batch, rows, cols, q, s, 1, 32);
  if (st != MX_OK) return st;
  if (rows == 0 || cols == 0) return MX_OK;
  if (!rowwise_blocks_fit(batch * rows, cols))
    return fail(MX_ERR_SHAPE, "mx_quantize_rowwise: batch*rows*cols/32 must be below 2^32 blocks");
  return hip_status(mxk::launch_quant_rowwise(x, batch * rows, cols, q, s, 0, (hipStream_t)stream),
                    "mx_quantize_rowwise launch");
}

mx_status mx_quantize_colwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint8_t* q_t,
                              uint8_t* s_t, void* stream) {
  mx_status st = check_quant("mx_quantize_colwise", x, batch, rows, cols, q_t, s_t, 32, 8);
  if (st != MX_OK) return st;
  if (rows == 0 || cols == 0) return MX_OK;
  if ((rows + 127) / 128 > 65535 || batch > 65535)
    return fail(MX_ERR_SHAPE, "mx_quantize_colwise: rows or batch too large for one launch");
  return hip_status(
      mxk::launch_quant_colwise(x, batch, rows, cols, q_t, rows, s_t, rows / 32, 0, (hipStream_t)stream),
      "mx_quantize_colwise launch");
}

mx_status mx_quantize_32x32(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s,
                            void* stream) {
  mx_status st = check_quant("mx_quantize_32x32", x, batch, rows, cols, q, s, 32, 32);
  if (st != MX_OK) return st;
  if (rows == 0 || cols == 0) return MX_OK;
  if (batch * rows / 32 > 65535) return fail(MX_ERR_SHAPE, "mx_quantize_32x32: too many row blocks for one launch");
  return hip_status(mxk::launch_quant_32x32(x, batch * rows, cols, q, s, (hipStream_t)stream),
                    "mx_quantize_32x32 launch");
}

}  // extern "C"

namespace {

mx_status grouped_gemm_impl(const char* fn, const uint8_t* X, const uint8_t* sX, const uint8_t* Y,
                            const uint8_t* sY, int scale_layout, const int32_t* offs, int mode, int64_t I, int64_t J,
                            int64_t Kc, int64_t E, void* C, int out_f32, void* stream,
                            const int32_t* row_map = nullptr, int64_t c_rows = -1, uint64_t order_seed = 0) {
  if (scale_layout == MX_SCALES_ROWMAJOR)
    return fail(MX_ERR_LAYOUT,
                "%s: the GEMM reads scales in its blocked layout [K/128][rows][4]; row-major scales "
                "[rows][K/32] (what mx_quantize_rowwise / mx_quantize_colwise write) must be converted with "
                "mx_scales_to_gemm_layout first (mx_quantize_weights and mx_quantize_dual write the GEMM layout)",
                fn);
  if (scale_layout != MX_SCALES_GEMM)
    return fail(MX_ERR_LAYOUT, "%s: unknown scale layout %d (MX_SCALES_GEMM = %d)", fn, scale_layout,
                (int)MX_SCALES_GEMM);
  if (mode != 0 && mode != 1) return fail(MX_ERR_SHAPE, "%s: mode must be 0 or 1 (got %d)", fn, mode);
  if (I < 0 || J < 0 || Kc < 0) return fail(MX_ERR_SHAPE, "%s: negative size", fn);
  if (E < 1 || E > mxk::kMaxExperts)
    return fail(MX_ERR_SHAPE, "%s: number of experts E=%lld outside [1, %d]", fn, (long long)E, mxk::kMaxExperts);
  if (Kc % 128 != 0) return fail(MX_ERR_SHAPE, "%s: Kc=%lld is not a multiple of 128", fn, (long long)Kc);
  if (J % 8 != 0) return fail(MX_ERR_SHAPE, "%s: J=%lld is not a multiple of 8", fn, (long long)J);
  // per-lane offsets inside a 256-row tile are 32-bit (row * Kc), and row
  // indices of X and Y must fit an int
  if (Kc > ((int64_t)1 << 23) || I >= ((int64_t)1 << 31) || J >= ((int64_t)1 << 31))
    return fail(MX_ERR_SHAPE, "%s: too large (I=%lld J=%lld Kc=%lld; Kc <= 2^23)", fn, (long long)I, (long long)J,
                (long long)Kc);
  const bool empty_out = (mode == 0) ? (I == 0 || J == 0) : (I == 0 || J == 0);
  if (empty_out) return MX_OK;
  if (!C || !offs) return fail(MX_ERR_NULL, "%s: null output or offsets", fn);
  if (Kc > 0 && (!X || !sX || !Y || !sY)) return fail(MX_ERR_NULL, "%s: null operand", fn);
  if (!aligned(X, 16) || !aligned(Y, 16) || !aligned(C, 16) || !aligned(sX, 4) || !aligned(sY, 4) ||
      !aligned(offs, 4))
    return fail(MX_ERR_ALIGN, "%s: X, Y, C must be 16-byte and scales/offsets 4-byte aligned", fn);
  mxk::GemmArgs a{};
  a.X = X;
  a.sX = sX;
  a.Y = Y;
  a.sY = sY;
  a.offs = offs;
  a.C = C;
  a.out_f32 = out_f32;
  a.I = I;
  a.J = J;
  a.Kc = Kc;
  a.E = (int)E;
  a.mode = mode;
  a.ldx = Kc;
  a.y_estride = J * Kc;
  a.sy_estride = J * (Kc / 32);
  a.ldc = J;
  a.c_estride = I * J;
  a.row_map = row_map;
  a.c_rows = row_map ? c_rows : I;
  if (order_seed) {
    // large primes: coprime with every grid size the launch can have (< 2^31)
    static const int64_t kPrimes[4] = {2147483647LL, 1000000007LL, 998244353LL, 1000003LL};
    a.order_mul = kPrimes[order_seed % 4];
    a.order_add = (int64_t)((order_seed / 4) % 1000003ULL);
  }
  return hip_status(mxk::launch_grouped_gemm(a, (hipStream_t)stream), fn);
}

mx_status gemm_rows_impl(const char* fn, const uint8_t* X, const uint8_t* sX, const uint8_t* Y, const uint8_t* sY,
                         int scale_layout, const int32_t* offs, int64_t I, int64_t J, int64_t Kc, int64_t E,
                         const int32_t* row_map, void* C, int64_t c_rows, int out_f32, void* stream) {
  if (c_rows < 0 || c_rows >= ((int64_t)1 << 31))
    return fail(MX_ERR_SHAPE, "%s: c_rows=%lld outside [0, 2^31)", fn, (long long)c_rows);
  if (c_rows == 0) return MX_OK;
  if (!row_map) return fail(MX_ERR_NULL, "%s: null row map", fn);
  if (!aligned(row_map, 4)) return fail(MX_ERR_ALIGN, "%s: row_map must be 4-byte aligned", fn);
  return grouped_gemm_impl(fn, X, sX, Y, sY, scale_layout, offs, 0, I, J, Kc, E, C, out_f32, stream, row_map, c_rows);
}

}  // namespace

extern "C" {

mx_status mx_grouped_gemm_mx(const uint8_t* X, const uint8_t* sX, const uint8_t* Y, const uint8_t* sY,
                             int scale_layout, const int32_t* offs, int mode, int64_t I, int64_t J, int64_t Kc,
                             int64_t E, uint16_t* C, void* stream) {
  return grouped_gemm_impl("mx_grouped_gemm_mx", X, sX, Y, sY, scale_layout, offs, mode, I, J, Kc, E, C, 0, stream);
}

mx_status mx_grouped_gemm_mx_f32(const uint8_t* X, const uint8_t* sX, const uint8_t* Y, const uint8_t* sY,
                                 int scale_layout, const int32_t* offs, int mode, int64_t I, int64_t J, int64_t Kc,
                                 int64_t E, float* C, void* stream) {
  return grouped_gemm_impl("mx_grouped_gemm_mx_f32", X, sX, Y, sY, scale_layout, offs, mode, I, J, Kc, E, C, 1,
                           stream);
}


mx_status mx_grouped_gemm_mx_rows(const uint8_t* X, const uint8_t* sX, const uint8_t* Y, const uint8_t* sY,
                                  int scale_layout, const int32_t* offs, int64_t I, int64_t J, int64_t Kc, int64_t E,
                                  const int32_t* row_map, uint16_t* C, int64_t c_rows, void* stream) {
  return gemm_rows_impl("mx_grouped_gemm_mx_rows", X, sX, Y, sY, scale_layout, offs, I, J, Kc, E, row_map, C, c_rows,
                        0, stream);
}

mx_status mx_grouped_gemm_mx_rows_f32(const uint8_t* X, const uint8_t* sX, const uint8_t* Y, const uint8_t* sY,
                                      int scale_layout, const int32_t* offs, int64_t I, int64_t J, int64_t Kc,
                                      int64_t E, const int32_t* row_map, float* C, int64_t c_rows, void* stream) {
  return gemm_rows_impl("mx_grouped_gemm_mx_rows_f32", X, sX, Y, sY, scale_layout, offs, I, J, Kc, E, row_map, C,
                        c_rows, 1, stream);
}

mx_status mx_topk_sum_rows(const float* x, int64_t T, int64_t k, int64_t cols, uint16_t* out, void* stream) {
  const char* fn = "mx_topk_sum_rows";
  if (T < 0 || cols < 0 || k < 1 || k > 1024)
    return fail(MX_ERR_SHAPE, "%s: T=%lld k=%lld cols=%lld (k in [1, 1024])", fn, (long long)T, (long long)k,
                (long long)cols);
  if (cols % 8 != 0) return fail(MX_ERR_SHAPE, "%s: cols=%lld is not a multiple of 8", fn, (long long)cols);
  if (T == 0 || cols == 0) return MX_OK;
  if (T * (cols / 8) >= ((int64_t)1 << 40)) return fail(MX_ERR_SHAPE, "%s: too large", fn);
  if (!x || !out) return fail(MX_ERR_NULL, "%s: null pointer", fn);
  if (!aligned(x, 16) || !aligned(out, 16)) return fail(MX_ERR_ALIGN, "%s: x and out must be 16-byte aligned", fn);
  return hip_status(mxk::launch_topk_sum(x, T, (int)k, cols, out, (hipStream_t)stream), fn);
}

size_t mx_route_workspace_bytes(int64_t n, int64_t E) {
  if (n < 0 || E < 1 || E > mxk::kMaxExperts) return 0;
  return mxk::route_ws_bytes(n, E);
}

mx_status mx_route(const int32_t* expert_idx, int64_t n, int64_t E, int64_t cap, int32_t* offs, int32_t* rows,
                   int32_t* pos, int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "mx_route";
  if (E < 1 || E > mxk::kMaxExperts)
    return fail(MX_ERR_SHAPE, "%s: number of experts E=%lld outside [1, %d]", fn, (long long)E, mxk::kMaxExperts);
  if (n < 0 || n >= ((int64_t)1 << 30)) return fail(MX_ERR_SHAPE, "%s: n=%lld outside [0, 2^30)", fn, (long long)n);
  // every group takes at most 31 padding rows
  if (cap < n + 31 * E || cap >= ((int64_t)1 << 31))
    return fail(MX_ERR_SHAPE, "%s: cap=%lld must be >= n + 31*E = %lld (and < 2^31)", fn, (long long)cap,
                (long long)(n + 31 * E));
  if ((n > 0 && (!expert_idx || !pos)) || !offs || !rows || !status)
    return fail(MX_ERR_NULL, "%s: null pointer", fn);
  if (!aligned(expert_idx, 4) || !aligned(offs, 4) || !aligned(rows, 4) || !aligned(pos, 4) || !aligned(status, 4))
    return fail(MX_ERR_ALIGN, "%s: int32 arrays must be 4-byte aligned", fn);
  const size_t need = mxk::route_ws_bytes(n, E);
  if (!ws || ws_bytes < need)
    return fail(MX_ERR_WORKSPACE, "%s: workspace of %zu bytes at %p, need %zu (mx_route_workspace_bytes)", fn, ws_bytes,
                ws, need);
  if (!aligned(ws, 4)) return fail(MX_ERR_ALIGN, "%s: workspace must be 4-byte aligned", fn);
  return hip_status(mxk::launch_route(expert_idx, n, E, cap, offs, rows, pos, status, (int32_t*)ws, (hipStream_t)stream),
                    fn);
}

mx_status mx_grouped_gemm_mx_ordered(const uint8_t* X, const uint8_t* sX, const uint8_t* Y, const uint8_t* sY,
                                     int scale_layout, const int32_t* offs, int mode, int64_t I, int64_t J, int64_t Kc,
                                     int64_t E, uint16_t* C, uint64_t order_seed, void* stream) {
  return grouped_gemm_impl("mx_grouped_gemm_mx_ordered", X, sX, Y, sY, scale_layout, offs, mode, I, J, Kc, E, C, 0,
                           stream, nullptr, -1, order_seed);
}

mx_status mx_check_offsets(const int32_t* offs, int64_t E, int64_t M, int32_t align, int32_t* status, void* stream) {
  const char* fn = "mx_check_offsets";
  if (E < 1 || E > mxk::kMaxExperts)
    return fail(MX_ERR_SHAPE, "%s: number of experts E=%lld outside [1, %d]", fn, (long long)E, mxk::kMaxExperts);
  if (M < 0 || M > INT32_MAX) return fail(MX_ERR_SHAPE, "%s: M=%lld outside [0, 2^31)", fn, (long long)M);
  if (align < 1) return fail(MX_ERR_SHAPE, "%s: align=%d must be >= 1", fn, (int)align);
  if (!offs || !status) return fail(MX_ERR_NULL, "%s: null pointer", fn);
  if (!aligned(offs, 4) || !aligned(status, 4)) return fail(MX_ERR_ALIGN, "%s: offs and status must be 4-byte aligned", fn);
  return hip_status(mxk::launch_check_offsets(offs, E, M, align, status, (hipStream_t)stream), fn);
}

mx_status mx_scales_to_gemm_layout(const uint8_t* s, int64_t batch, int64_t rows, int64_t kblocks, uint8_t* s_gemm,
                                   void* stream) {
  const char* fn = "mx_scales_to_gemm_layout";
  if (batch < 1 || rows < 0 || kblocks < 0)
    return fail(MX_ERR_SHAPE, "%s: batch=%lld rows=%lld kblocks=%lld", fn, (long long)batch, (long long)rows,
                (long long)kblocks);
  if (kblocks % 4 != 0) return fail(MX_ERR_SHAPE, "%s: kblocks=%lld is not a multiple of 4", fn, (long long)kblocks);
  if (rows == 0 || kblocks == 0) return MX_OK;
  if (!s || !s_gemm) return fail(MX_ERR_NULL, "%s: null pointer", fn);
  if (!aligned(s_gemm, 4)) return fail(MX_ERR_ALIGN, "%s: s_gemm must be 4-byte aligned", fn);
  return hip_status(mxk::launch_scales_to_gemm(s, batch, rows, kblocks, s_gemm, (hipStream_t)stream), fn);
}

size_t mx_grouped_mm_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int64_t E) {
  if (op < MX_OP_FWD || op > MX_OP_DGRAD_Q || M < 0 || N < 0 || K < 0 || E < 1) return 0;
  return ws_layout(op, M, N, K, E).total;
}

mx_status mx_grouped_mm_fwd(const uint16_t* A, const uint16_t* W, const int32_t* offs, int64_t M, int64_t N,
                            int64_t K, int64_t E, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "mx_grouped_mm_fwd";
  mx_status st = check_mm(fn, A, W, offs, out, M, N, K, E);
  if (st != MX_OK) return st;
  if (K % 128 != 0) return fail(MX_ERR_SHAPE, "%s: K=%lld is not a multiple of 128", fn, (long long)K);
  if (N % 8 != 0) return fail(MX_ERR_SHAPE, "%s: N=%lld is not a multiple of 8", fn, (long long)N);
  const WsLayout L = ws_layout(MX_OP_FWD, M, N, K, E);
  if (!ws || ws_bytes < L.total)
    return fail(MX_ERR_WORKSPACE, "%s: workspace of %zu bytes at %p, need %zu", fn, ws_bytes, ws, L.total);
  if (!aligned(ws, 256)) return fail(MX_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  if (M == 0 || N == 0) return MX_OK;
  if ((E * N + M) * (K / 32) >= ((int64_t)1 << 31)) return fail(MX_ERR_SHAPE, "%s: tensors too large", fn);
  uint8_t* w8 = (uint8_t*)ws;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *qA = w8 + L.off[0], *sA = w8 + L.off[1], *qW = w8 + L.off[2], *sW = w8 + L.off[3];
  if ((st = hip_status(mxk::launch_quant_rowwise(A, M, K, qA, sA, M, s), "fwd quantize A")) != MX_OK) return st;
  if ((st = hip_status(mxk::launch_quant_rowwise(W, E * N, K, qW, sW, N, s), "fwd quantize W")) != MX_OK) return st;
  return mx_grouped_gemm_mx(qA, sA, qW, sW, MX_SCALES_GEMM, offs, 0, M, N, K, E, out, stream);
}

mx_status mx_grouped_mm_dgrad(const uint16_t* dOut, const uint16_t* W, const int32_t* offs, int64_t M, int64_t N,
                              int64_t K, int64_t E, uint16_t* dA, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "mx_grouped_mm_dgrad";
  mx_status st = check_mm(fn, dOut, W, offs, dA, M, N, K, E);
  if (st != MX_OK) return st;
  if (N % 128 != 0) return fail(MX_ERR_SHAPE, "%s: N=%lld is not a multiple of 128", fn, (long long)N);
  if (K % 8 != 0) return fail(MX_ERR_SHAPE, "%s: K=%lld is not a multiple of 8", fn, (long long)K);
  const WsLayout L = ws_layout(MX_OP_DGRAD, M, N, K, E);
  if (!ws || ws_bytes < L.total)
    return fail(MX_ERR_WORKSPACE, "%s: workspace of %zu bytes at %p, need %zu", fn, ws_bytes, ws, L.total);
  if (!aligned(ws, 256)) return fail(MX_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  if (M == 0 || K == 0) return MX_OK;
  if ((N + 127) / 128 > 65535 || E > 65535) return fail(MX_ERR_SHAPE, "%s: N too large for one launch", fn);
  if (!rowwise_blocks_fit(M, N)) return fail(MX_ERR_SHAPE, "%s: M*N/32 must be below 2^32 blocks", fn);
  uint8_t* w8 = (uint8_t*)ws;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *qG = w8 + L.off[0], *sG = w8 + L.off[1], *qWt = w8 + L.off[2], *sWt = w8 + L.off[3];
  if ((st = hip_status(mxk::launch_quant_rowwise(dOut, M, N, qG, sG, M, s), "dgrad quantize dOut")) != MX_OK)
    return st;
  // W [E, N, K] quantized in 32-blocks along N, stored transposed [E, K, N]
  if ((st = hip_status(mxk::launch_quant_colwise(W, E, N, K, qWt, N, sWt, N / 32, 1, s), "dgrad quantize W")) != MX_OK)
    return st;
  return mx_grouped_gemm_mx(qG, sG, qWt, sWt, MX_SCALES_GEMM, offs, 0, M, K, N, E, dA, stream);
}

mx_status mx_grouped_mm_wgrad(const uint16_t* dOut, const uint16_t* A, const int32_t* offs, int64_t M, int64_t N,
                              int64_t K, int64_t E, uint16_t* dW, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "mx_grouped_mm_wgrad";
  mx_status st = check_mm(fn, dOut, A, offs, dW, M, N, K, E);
  if (st != MX_OK) return st;
  if (M % 32 != 0) return fail(MX_ERR_SHAPE, "%s: M=%lld is not a multiple of 32", fn, (long long)M);
  if (N % 8 != 0 || K % 8 != 0)
    return fail(MX_ERR_SHAPE, "%s: N=%lld and K=%lld must be multiples of 8", fn, (long long)N, (long long)K);
  const WsLayout L = ws_layout(MX_OP_WGRAD, M, N, K, E);
  if (!ws || ws_bytes < L.total)
    return fail(MX_ERR_WORKSPACE, "%s: workspace of %zu bytes at %p, need %zu", fn, ws_bytes, ws, L.total);
  if (!aligned(ws, 256)) return fail(MX_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  if (N == 0 || K == 0) return MX_OK;
  if ((M + 127) / 128 > 65535) return fail(MX_ERR_SHAPE, "%s: M too large for one launch", fn);
  const int64_t Mp = round_up(M, 128);
  uint8_t* w8 = (uint8_t*)ws;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *qGt = w8 + L.off[0], *sGt = w8 + L.off[1], *qAt = w8 + L.off[2], *sAt = w8 + L.off[3];
  // dOut [M, N] and A [M, K] in 32-blocks along tokens, stored [N, Mp] and [K, Mp]
  if ((st = hip_status(mxk::launch_quant_colwise(dOut, 1, M, N, qGt, Mp, sGt, Mp / 32, 1, s), "wgrad quantize dOut")) !=
      MX_OK)
    return st;
  if ((st = hip_status(mxk::launch_quant_colwise(A, 1, M, K, qAt, Mp, sAt, Mp / 32, 1, s), "wgrad quantize A")) !=
      MX_OK)
    return st;
  return mx_grouped_gemm_mx(qGt, sGt, qAt, sAt, MX_SCALES_GEMM, offs, 1, N, K, Mp, E, dW, stream);
}

mx_status mx_quantize_weights(const uint16_t* w, int64_t E, int64_t N, int64_t K, uint8_t* q, uint8_t* s,
                              uint8_t* q_t, uint8_t* s_t, void* stream) {
  const char* fn = "mx_quantize_weights";
  if (E < 1 || N < 0 || K < 0)
    return fail(MX_ERR_SHAPE, "%s: E=%lld N=%lld K=%lld", fn, (long long)E, (long long)N, (long long)K);
  if (N % 128 != 0 || K % 128 != 0)
    return fail(MX_ERR_SHAPE, "%s: N=%lld and K=%lld must be multiples of 128", fn, (long long)N, (long long)K);
  if (N == 0 || K == 0) return MX_OK;
  if (N / 128 > 65535 || K / 128 > 65535 || E > 65535) return fail(MX_ERR_SHAPE, "%s: too large for one launch", fn);
  if (!w || !q || !s || !q_t || !s_t) return fail(MX_ERR_NULL, "%s: null pointer", fn);
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(q_t, 16) || !aligned(s, 4) || !aligned(s_t, 4))
    return fail(MX_ERR_ALIGN, "%s: w, q, q_t must be 16-byte and s, s_t 4-byte aligned", fn);
  return hip_status(mxk::launch_quant_dual(w, E, N, K, N, q, s, q_t, s_t, (hipStream_t)stream), fn);
}

mx_status mx_quantize_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldq, uint8_t* q, uint8_t* s,
                           uint8_t* q_t, uint8_t* s_t, void* stream) {
  const char* fn = "mx_quantize_dual";
  if (rows < 0 || cols < 0 || ldq < 0)
    return fail(MX_ERR_SHAPE, "%s: rows=%lld cols=%lld ldq=%lld", fn, (long long)rows, (long long)cols, (long long)ldq);
  if (rows % 32 != 0 || cols % 128 != 0)
    return fail(MX_ERR_SHAPE, "%s: rows=%lld must be a multiple of 32 and cols=%lld of 128", fn, (long long)rows,
                (long long)cols);
  if (ldq % 128 != 0 || ldq < rows)
    return fail(MX_ERR_SHAPE, "%s: ldq=%lld must be a multiple of 128 and >= rows=%lld", fn, (long long)ldq,
                (long long)rows);
  if (ldq == 0 || cols == 0) return MX_OK;
  if (ldq / 128 > 65535 || cols / 128 > 65535) return fail(MX_ERR_SHAPE, "%s: too large for one launch", fn);
  if (!x || !q || !s || !q_t || !s_t) return fail(MX_ERR_NULL, "%s: null pointer", fn);
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(q_t, 16) || !aligned(s, 4) || !aligned(s_t, 4))
    return fail(MX_ERR_ALIGN, "%s: x, q, q_t must be 16-byte and s, s_t 4-byte aligned", fn);
  return hip_status(mxk::launch_quant_dual(x, 1, rows, cols, ldq, q, s, q_t, s_t, (hipStream_t)stream), fn);
}

mx_status mx_quantize_dual_gather(const uint16_t* x, int64_t src_rows, const int32_t* rows, int64_t topk, int64_t M,
                                  int64_t cols, int64_t ldq, uint8_t* q, uint8_t* s, uint8_t* q_t, uint8_t* s_t,
                                  void* stream) {
  const char* fn = "mx_quantize_dual_gather";
  if (src_rows < 0 || M < 0 || cols < 0 || ldq < 0)
    return fail(MX_ERR_SHAPE, "%s: src_rows=%lld M=%lld cols=%lld ldq=%lld", fn, (long long)src_rows, (long long)M,
                (long long)cols, (long long)ldq);
  if (topk < 1 || topk > 1024) return fail(MX_ERR_SHAPE, "%s: topk=%lld outside [1, 1024]", fn, (long long)topk);
  if (M % 32 != 0 || cols % 128 != 0)
    return fail(MX_ERR_SHAPE, "%s: M=%lld must be a multiple of 32 and cols=%lld of 128", fn, (long long)M,
                (long long)cols);
  if (ldq % 128 != 0 || ldq < M)
    return fail(MX_ERR_SHAPE, "%s: ldq=%lld must be a multiple of 128 and >= M=%lld", fn, (long long)ldq,
                (long long)M);
  if (src_rows * topk >= ((int64_t)1 << 31))
    return fail(MX_ERR_SHAPE, "%s: src_rows*topk must be below 2^31", fn);
  if (ldq == 0 || cols == 0) return MX_OK;
  if (ldq / 128 > 65535 || cols / 128 > 65535) return fail(MX_ERR_SHAPE, "%s: too large for one launch", fn);
  if ((M > 0 && !rows) || !q || !s || !q_t || !s_t || (src_rows > 0 && !x))
    return fail(MX_ERR_NULL, "%s: null pointer", fn);
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(q_t, 16) || !aligned(s, 4) || !aligned(s_t, 4) ||
      !aligned(rows, 4))
    return fail(MX_ERR_ALIGN, "%s: x, q, q_t must be 16-byte and s, s_t, rows 4-byte aligned", fn);
  return hip_status(mxk::launch_quant_dual(x, 1, M, cols, ldq, q, s, q_t, s_t, (hipStream_t)stream,
                                           M > 0 ? rows : nullptr, src_rows, (int)topk),
                    fn);
}

mx_status mx_grouped_mm_fwd_q(const uint16_t* A, const uint8_t* qW, const uint8_t* sW, const int32_t* offs, int64_t M,
                              int64_t N, int64_t K, int64_t E, uint16_t* out, void* ws, size_t ws_bytes,
                              void* stream) {
  const char* fn = "mx_grouped_mm_fwd_q";
  mx_status st = check_mm(fn, A, qW, offs, out, M, N, K, E);
  if (st != MX_OK) return st;
  if (!sW) return fail(MX_ERR_NULL, "%s: null weight scales", fn);
  if (K % 128 != 0) return fail(MX_ERR_SHAPE, "%s: K=%lld is not a multiple of 128", fn, (long long)K);
  if (N % 8 != 0) return fail(MX_ERR_SHAPE, "%s: N=%lld is not a multiple of 8", fn, (long long)N);
  const WsLayout L = ws_layout(MX_OP_FWD_Q, M, N, K, E);
  if (!ws || ws_bytes < L.total)
    return fail(MX_ERR_WORKSPACE, "%s: workspace of %zu bytes at %p, need %zu", fn, ws_bytes, ws, L.total);
  if (!aligned(ws, 256)) return fail(MX_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  if (M == 0 || N == 0) return MX_OK;
  if (!rowwise_blocks_fit(M, K)) return fail(MX_ERR_SHAPE, "%s: M*K/32 must be below 2^32 blocks", fn);
  uint8_t* w8 = (uint8_t*)ws;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *qA = w8 + L.off[0], *sA = w8 + L.off[1];
  if ((st = hip_status(mxk::launch_quant_rowwise(A, M, K, qA, sA, M, s), "fwd_q quantize A")) != MX_OK) return st;
  return mx_grouped_gemm_mx(qA, sA, qW, sW, MX_SCALES_GEMM, offs, 0, M, N, K, E, out, stream);
}

mx_status mx_grouped_mm_dgrad_q(const uint16_t* dOut, const uint8_t* qWt, const uint8_t* sWt, const int32_t* offs,
                                int64_t M, int64_t N, int64_t K, int64_t E, uint16_t* dA, void* ws, size_t ws_bytes,
                                void* stream) {
  const char* fn = "mx_grouped_mm_dgrad_q";
  mx_status st = check_mm(fn, dOut, qWt, offs, dA, M, N, K, E);
  if (st != MX_OK) return st;
  if (!sWt) return fail(MX_ERR_NULL, "%s: null weight scales", fn);
  if (N % 128 != 0) return fail(MX_ERR_SHAPE, "%s: N=%lld is not a multiple of 128", fn, (long long)N);
  if (K % 8 != 0) return fail(MX_ERR_SHAPE, "%s: K=%lld is not a multiple of 8", fn, (long long)K);
  const WsLayout L = ws_layout(MX_OP_DGRAD_Q, M, N, K, E);
  if (!ws || ws_bytes < L.total)
    return fail(MX_ERR_WORKSPACE, "%s: workspace of %zu bytes at %p, need %zu", fn, ws_bytes, ws, L.total);
  if (!aligned(ws, 256)) return fail(MX_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  if (M == 0 || K == 0) return MX_OK;
  if (!rowwise_blocks_fit(M, N)) return fail(MX_ERR_SHAPE, "%s: M*N/32 must be below 2^32 blocks", fn);
  uint8_t* w8 = (uint8_t*)ws;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *qG = w8 + L.off[0], *sG = w8 + L.off[1];
  if ((st = hip_status(mxk::launch_quant_rowwise(dOut, M, N, qG, sG, M, s), "dgrad_q quantize dOut")) != MX_OK)
    return st;
  return mx_grouped_gemm_mx(qG, sG, qWt, sWt, MX_SCALES_GEMM, offs, 0, M, K, N, E, dA, stream);
}

mx_status mx_quantize_rowwise_gather(const uint16_t* x, int64_t src_rows, const int32_t* rows, int64_t M,
                                     int64_t cols, uint8_t* q, uint8_t* s_gemm, void* stream) {
  const char* fn = "mx_quantize_rowwise_gather";
  if (src_rows < 0 || M < 0 || cols < 0)
    return fail(MX_ERR_SHAPE, "%s: src_rows=%lld M=%lld cols=%lld", fn, (long long)src_rows, (long long)M,
                (long long)cols);
  if (cols % 128 != 0) return fail(MX_ERR_SHAPE, "%s: cols=%lld is not a multiple of 128", fn, (long long)cols);
  if (M == 0 || cols == 0) return MX_OK;
  if (M >= ((int64_t)1 << 31) || !rowwise_blocks_fit(M, cols))
    return fail(MX_ERR_SHAPE, "%s: too large (M < 2^31 rows and M*cols/32 < 2^32 blocks)", fn);
  if (!rows || !q || !s_gemm || (src_rows > 0 && !x)) return fail(MX_ERR_NULL, "%s: null pointer", fn);
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(rows, 4))
    return fail(MX_ERR_ALIGN, "%s: x and q must be 16-byte aligned, rows 4-byte aligned", fn);
  return hip_status(mxk::launch_quant_rowwise_gather(x, src_rows, rows, M, cols, q, s_gemm, (hipStream_t)stream), fn);
}

}  // extern "C"
