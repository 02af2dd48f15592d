// Routing-side kernels of the grouped GEMMs: validation of the per-expert
// group offsets on the device (the offsets never cross to the host on the
// hot path).
//
// The grouped GEMM of "MXFP8 training for MoEs" (section "Is MXFP8 Training
// for MoEs Actually Stable?") takes each expert's routed tokens as one group;
// the weight gradient sums 32-token blocks, which must not straddle two
// experts, so every group starts on a multiple of 32 there.  Unsupported
// inputs get a clear error ("feat(moe): add MoK MXFP8 expert support" PR,
// summary): this kernel finds them without a host round trip, and the caller
// reads the status word when it chooses to.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mxk {

// One workgroup.  Bits of status[0]: 1 an offset below its predecessor,
// 2 an offset outside [0, M], 4 the last offset is not M, 8 a group start
// that is not a multiple of `align`.
__global__ __launch_bounds__(256) void check_offsets_kernel(const int32_t* __restrict__ offs, int64_t E, int64_t M,
                                                            int align, int32_t* __restrict__ status) {
  __shared__ int flags;
  if (threadIdx.x == 0) flags = 0;
  __syncthreads();
  int f = 0;
  for (int64_t e = threadIdx.x; e < E; e += 256) {
    const int64_t start = e == 0 ? 0 : (int64_t)offs[e - 1];
    const int64_t end = offs[e];
    if (end < start) f |= 1;
    if (end < 0 || end > M) f |= 2;
    if (e == E - 1 && end != M) f |= 4;
    if (align > 1 && (start % align) != 0) f |= 8;
  }
  if (f) atomicOr(&flags, f);
  __syncthreads();
  if (threadIdx.x == 0) status[0] = flags;
}

hipError_t launch_check_offsets(const int32_t* offs, int64_t E, int64_t M, int align, int32_t* status,
                                hipStream_t st) {
  hipLaunchKernelGGL(check_offsets_kernel, dim3(1), dim3(256), 0, st, offs, E, M, align, status);
  return hipGetLastError();
}

}  // namespace mxk
