// Forward grouped GEMM on prequantized expert weights without a caller
// workspace: the MX codes and GEMM-layout scales of the activations live in
// a file-scope device array instead.  For callers that cannot allocate (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  It runs the same kernels as mx_grouped_mm_fwd_q.
//
// The array is a device symbol: in host code its name is only a stand-in, so
// every host use goes through the device address that hipGetSymbolAddress
// returns, looked up once per device (with that device current) and kept.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "mx_kernels.h"
#include "mxmoe.h"

namespace {

constexpr size_t kScratchBytes = (size_t)MX_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

mx_status err(mx_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mx_status err(mx_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return mxk::set_last_error(st, buf);
}

// Device address of `scratch` on the current device (looked up once).
mx_status scratch_ptr(uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return err(MX_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return err(MX_ERR_HIP, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return err(MX_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = (uint8_t*)g_ptr[dev];
  return MX_OK;
}

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

extern "C" {

mx_status mx_grouped_mm_fwd_q_noalloc(const uint16_t* A, const uint8_t* qW, const uint8_t* sW, const int32_t* offs,
                                      int64_t M, int64_t N, int64_t K, int64_t E, uint16_t* out, void* stream) {
  const char* fn = "mx_grouped_mm_fwd_q_noalloc";
  if (M < 0 || N < 0 || K < 0) {
    return err(MX_ERR_SHAPE, "%s: negative size M=%lld N=%lld K=%lld", fn, (long long)M, (long long)N,
               (long long)K);
  }
  const size_t codes = round256((size_t)M * (size_t)K);
  const size_t need = codes + round256((size_t)M * (size_t)(K / 32));
  if (need > kScratchBytes) {
    return err(MX_ERR_WORKSPACE, "%s: M*K = %lld activations need %zu bytes of MX codes and scales, more than the "
               "%zu-byte static scratch; use mx_grouped_mm_fwd_q with a workspace", fn,
               (long long)(M * K), need, kScratchBytes);
  }
  uint8_t* base = nullptr;
  mx_status st = scratch_ptr(&base);
  if (st != MX_OK) return st;
  // mx_grouped_mm_fwd_q checks every other argument and runs the kernels with
  // the scratch as its workspace (quantized A: codes, then GEMM-layout scales)
  return mx_grouped_mm_fwd_q(A, qW, sW, offs, M, N, K, E, out, base, kScratchBytes, stream);
}

}  // extern "C"
