// Internal interface between the C-ABI host layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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
  int64_t ldx, ldsx;          // bytes per row of X and of its scales
  int64_t ldy, ldsy;          // bytes per row of Y and of its scales
  int64_t y_estride;          // mode 0: bytes between experts of Y
  int64_t sy_estride;         // mode 0: bytes between experts of sY
  int64_t sx_total;           // bytes of the sX tensor
  int64_t sy_total_per_e;     // bytes of one expert's sY (mode 0) / of sY (mode 1)
  int64_t ldc;                // elements per row of C
  int64_t c_estride;          // mode 1: elements between experts of C
};

hipError_t launch_quant_rowwise(const uint16_t* x, int64_t rows_total, int64_t cols, uint8_t* q, uint8_t* s,
                                hipStream_t st);
hipError_t launch_quant_colwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint8_t* q_t,
                                int64_t ldq, uint8_t* s_t, int64_t lds, hipStream_t st);
hipError_t launch_quant_32x32(const uint16_t* x, int64_t rows_total, int64_t cols, uint8_t* q, uint8_t* s,
                              hipStream_t st);
hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t st);
size_t gemm_lds_bytes();

constexpr int kMaxExperts = 1024;

}  // namespace mxk
