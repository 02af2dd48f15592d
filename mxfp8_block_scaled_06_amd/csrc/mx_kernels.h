// Internal interface between the C-ABI host layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mxmoe.h"

namespace mxk {

// Grouped GEMM arguments (see mx_gemm.hip for the operation).
struct GemmArgs {
  const uint8_t* X;
  const uint8_t* sX;
  const uint8_t* Y;
  const uint8_t* sY;
  const int32_t* offs;
  void* C;                    // bf16 (uint16_t) or fp32 output
  int out_f32;                // 1: fp32 output, 0: bf16 (RNE)
  int64_t I, J, Kc;
  int E;
  int mode;
  int64_t ldx;                // bytes per row of X and of Y (== Kc)
  int64_t y_estride;          // mode 0: bytes between experts of Y
  int64_t sy_estride;         // mode 0: bytes between experts of sY
  int64_t ldc;                // elements per row of C
  int64_t c_estride;          // mode 1: elements between experts of C
  const int32_t* row_map;     // mode 0, optional: X row i is stored to C row row_map[i] (skipped if outside [0, c_rows))
  int64_t c_rows;
  int64_t order_mul;          // 0: the library's tile order; else workgroup slot t runs tile (t * mul + add) % grid
  int64_t order_add;
};

// gemm_rows_per_batch == 0: row-major scales [rows_total][cols/32]; > 0:
// GEMM scale layout [rows_total/R][cols/128][R][4] with R = gemm_rows_per_batch.
hipError_t launch_quant_rowwise(const uint16_t* x, int64_t rows_total, int64_t cols, uint8_t* q, uint8_t* s,
                                int64_t gemm_rows_per_batch, hipStream_t st);
// Rowwise of x[rows[r]] for r < M (index < 0 or >= src_rows: a zero row);
// scales in the GEMM layout [cols/128][M][4].
hipError_t launch_quant_rowwise_gather(const uint16_t* x, int64_t src_rows, const int32_t* rows, int64_t M,
                                       int64_t cols, uint8_t* q, uint8_t* s, hipStream_t st);
// gemm_layout == 0: s_t [batch][cols][lds]; 1: GEMM layout [batch][ldq/128][cols][4].
hipError_t launch_quant_colwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint8_t* q_t,
                                int64_t ldq, uint8_t* s_t, int64_t lds, int gemm_layout, hipStream_t st);
// Both orientations of w [E, N, K] (N % 32 == 0, K % 128 == 0, ldq % 128 == 0,
// ldq >= N): q [E, N, K] with s in GEMM layout [E][K/128][N][4]; q_t
// [E, K, ldq] with s_t in GEMM layout [E][ldq/128][K][4], zero past N.
// rows != nullptr: row n of the (batch-1) input is x[rows[n] / topk] (a zero
// row when rows[n] is negative or >= src_rows * topk): the token gather of the
// MoE dispatch.
hipError_t launch_quant_dual(const uint16_t* w, int64_t E, int64_t N, int64_t K, int64_t ldq, uint8_t* q,
                             uint8_t* s, uint8_t* q_t, uint8_t* s_t, hipStream_t st,
                             const int32_t* rows = nullptr, int64_t src_rows = 0, int topk = 1);
hipError_t launch_scales_to_gemm(const uint8_t* s, int64_t batch, int64_t rows, int64_t kb, uint8_t* out,
                                 hipStream_t st);
hipError_t launch_quant_32x32(const uint16_t* x, int64_t rows_total, int64_t cols, uint8_t* q, uint8_t* s,
                              hipStream_t st);
hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t st);
// out[t] = bf16(sum of the k fp32 rows x[t*k .. t*k+k-1]) (see mx_topk_sum_rows).
hipError_t launch_topk_sum(const float* x, int64_t T, int k, int64_t cols, uint16_t* out, hipStream_t st);
// Routing metadata (see mx_route); ws holds route_ws_bytes(n, E) bytes.
size_t route_ws_bytes(int64_t n, int64_t E);
hipError_t launch_route(const int32_t* expert_idx, int64_t n, int64_t E, int64_t cap, int32_t* offs, int32_t* rows,
                        int32_t* pos, int32_t* status, int32_t* ws, hipStream_t st);
// status[0] = validity bitmask of the group offsets (see mx_check_offsets).
hipError_t launch_check_offsets(const int32_t* offs, int64_t E, int64_t M, int align, int32_t* status,
                                hipStream_t st);
size_t gemm_lds_bytes();

constexpr int kMaxExperts = 1024;

// Record `text` as the calling thread's mx_last_error() and return `st`.
mx_status set_last_error(mx_status st, const char* text);

}  // namespace mxk
