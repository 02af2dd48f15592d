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

namespace mxk {

// ---------------------------------------------------------------------------
// Routing metadata.  Item a (a token, or one token-expert pair of a top-k
// router, flattened token-major) goes to expert expert_idx[a]; each expert's
// items form one group, in their original order, padded with zero rows to a
// multiple of 32 (the weight gradient's 32-token blocks then never straddle
// two experts).  Outputs, all on the device:
//   offs [E]   cumulative padded END offsets (the grouped GEMMs' offsets)
//   rows [cap] grouped row -> item, -1 for padding and rows past the last group
//   pos  [n]   item -> grouped row
// status[0] gets 1 if some expert id lies outside [0, E) (those items are not
// routed: pos = -1).  Three passes over chunks of 1024 items, one workgroup
// per chunk in the first and last:
//   count   per-chunk histogram of expert ids (LDS atomics) -> cnt[chunk][E];
//   scan    one workgroup: each expert's counts become exclusive prefixes over
//           the chunks, the padded group sizes are scanned into the offsets,
//           the padding rows get -1;
//   scatter each item's rank among the earlier items of its expert in its
//           chunk (wave ballots, then a scan of per-wave counts) plus the
//           chunk's prefix and the group start is its grouped row.
// Every position follows from counts and ranks, so the result does not depend
// on thread timing.  The host guarantees cap >= n + 31 * E, the most rows the
// padded groups can take.
// ---------------------------------------------------------------------------
constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;

// Workspace: cnt [nchunks][E] | bad [nchunks] | start [E] (int32).
struct RouteWs {
  int32_t* cnt;
  int32_t* bad;
  int32_t* start;
};

__device__ __forceinline__ RouteWs route_ws(int32_t* ws, int nchunks, int E) {
  RouteWs w;
  w.cnt = ws;
  w.bad = ws + (int64_t)nchunks * E;
  w.start = w.bad + nchunks;
  return w;
}

__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(const int32_t* __restrict__ expert_idx, int n,
                                                                    int E, int32_t* __restrict__ ws) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int bad;
  const int tid = threadIdx.x, c = blockIdx.x;
  const RouteWs w = route_ws(ws, gridDim.x, E);
  for (int e = tid; e < E; e += kRouteThreads) cnt[e] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  const int a = c * kRouteThreads + tid;
  if (a < n) {
    const int e = expert_idx[a];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    else bad = 1;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) w.cnt[(int64_t)c * E + e] = cnt[e];
  if (tid == 0) w.bad[c] = bad;
}

__global__ __launch_bounds__(kRouteThreads) void route_scan_kernel(int nchunks, int E, int cap,
                                                                   int32_t* __restrict__ ws,
                                                                   int32_t* __restrict__ offs,
                                                                   int32_t* __restrict__ rows,
                                                                   int32_t* __restrict__ status) {
  __shared__ int wsum[kRouteWaves];
  __shared__ int bad, total;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const RouteWs w = route_ws(ws, nchunks, E);
  if (tid == 0) bad = 0;
  __syncthreads();
  // expert e = tid: its counts become exclusive prefixes over the chunks
  int cnt = 0;
  if (tid < E) {
    for (int c = 0; c < nchunks; ++c) {
      const int v = w.cnt[(int64_t)c * E + tid];
      w.cnt[(int64_t)c * E + tid] = cnt;
      cnt += v;
    }
  }
  for (int c = tid; c < nchunks; c += kRouteThreads)
    if (w.bad[c]) bad = 1;
  // exclusive scan of the padded counts (E <= 1024: one expert per thread)
  const int pc = tid < E ? (cnt + 31) & ~31 : 0;
  int incl = pc;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int x = 0; x < wv; ++x) before += wsum[x];
  if (tid < E) {
    const int st = before + incl - pc;
    w.start[tid] = st;
    offs[tid] = before + incl;
    for (int r = st + cnt; r < before + incl; ++r) rows[r] = -1;   // this group's padding rows
  }
  if (tid == E - 1) total = before + incl;
  __syncthreads();
  for (int r = total + tid; r < cap; r += kRouteThreads) rows[r] = -1;
  if (tid == 0) status[0] = bad;
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(const int32_t* __restrict__ expert_idx, int n,
                                                                      int E, const int32_t* __restrict__ ws,
                                                                      int32_t* __restrict__ rows,
                                                                      int32_t* __restrict__ pos) {
  __shared__ int base[kMaxExperts];
  __shared__ int wc[kRouteWaves][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, c = blockIdx.x;
  const RouteWs w = route_ws(const_cast<int32_t*>(ws), gridDim.x, E);
  for (int e = tid; e < E; e += kRouteThreads) base[e] = w.start[e] + w.cnt[(int64_t)c * E + e];
  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) wc[i / E][i % E] = 0;
  __syncthreads();
  const int a = c * kRouteThreads + tid;
  const int e = a < n ? expert_idx[a] : -1;
  const bool valid = e >= 0 && e < E;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank = 0;
  uint64_t remaining = __ballot(valid);
  while (remaining) {
    const int leader = __builtin_ctzll(remaining);
    const int le = __shfl(e, leader);
    const uint64_t m = __ballot(valid && e == le);
    if (valid && e == le) {
      rank = __builtin_popcountll(m & lt);
      if (lane == leader) wc[wv][le] = __builtin_popcountll(m);
    }
    remaining &= ~m;
  }
  __syncthreads();
  // per expert: exclusive prefix over the waves of this chunk
  for (int x = tid; x < E; x += kRouteThreads) {
    int acc = 0;
    for (int v = 0; v < kRouteWaves; ++v) {
      const int cv = wc[v][x];
      wc[v][x] = acc;
      acc += cv;
    }
  }
  __syncthreads();
  if (a < n) {
    if (valid) {
      const int p = base[e] + wc[wv][e] + rank;
      pos[a] = p;
      rows[p] = a;
    } else {
      pos[a] = -1;
    }
  }
}

size_t route_ws_bytes(int64_t n, int64_t E) {
  const int64_t nchunks = (n + kRouteThreads - 1) / kRouteThreads;
  return (size_t)(nchunks * E + nchunks + E) * sizeof(int32_t);
}

hipError_t launch_route(const int32_t* expert_idx, int64_t n, int64_t E, int64_t cap, int32_t* offs, int32_t* rows,
                        int32_t* pos, int32_t* status, int32_t* ws, hipStream_t st) {
  const int nchunks = (int)((n + kRouteThreads - 1) / kRouteThreads);
  if (nchunks > 0) {
    hipLaunchKernelGGL(route_count_kernel, dim3(nchunks), dim3(kRouteThreads), 0, st, expert_idx, (int)n, (int)E, ws);
  }
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kRouteThreads), 0, st, nchunks, (int)E, (int)cap, ws, offs, rows,
                     status);
  if (nchunks > 0) {
    hipLaunchKernelGGL(route_scatter_kernel, dim3(nchunks), dim3(kRouteThreads), 0, st, expert_idx, (int)n, (int)E,
                       (const int32_t*)ws, rows, pos);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gradient of the top-k gather: a token's input gradient is the sum of the
// gradients of its k items.  out[t, c] = bf16(sum_{j < k} x[t*k + j, c]) with
// the sum taken in fp32 in slot order and rounded to nearest even once.  One
// thread per 8 columns of one token: k 32-byte loads, one 16-byte store.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void topk_sum_kernel(const float* __restrict__ x, int64_t T, int k, int64_t cols,
                                                       uint16_t* __restrict__ out) {
  const int64_t per_row = cols >> 3;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * per_row) return;
  const int64_t t = idx / per_row, c = (idx - t * per_row) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const v4i& a, const v4i& b) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[u] += __int_as_float(a[u]);
      acc[4 + u] += __int_as_float(b[u]);
    }
  };
  // slots four at a time (then two, then one): their loads go out together,
  // the additions stay in slot order
  int j = 0;
  for (; j + 4 <= k; j += 4) {
    v4i a[4], b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4i* src = (const v4i*)(x + (t * k + j + q) * cols + c);
      a[q] = __builtin_nontemporal_load(src);
      b[q] = __builtin_nontemporal_load(src + 1);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) add(a[q], b[q]);
  }
  if (j + 2 <= k) {
    const v4i* s0 = (const v4i*)(x + (t * k + j) * cols + c);
    const v4i* s1 = (const v4i*)(x + (t * k + j + 1) * cols + c);
    const v4i a0 = __builtin_nontemporal_load(s0), b0 = __builtin_nontemporal_load(s0 + 1);
    const v4i a1 = __builtin_nontemporal_load(s1), b1 = __builtin_nontemporal_load(s1 + 1);
    add(a0, b0);
    add(a1, b1);
    j += 2;
  }
  if (j < k) {
    const v4i* src = (const v4i*)(x + (t * k + j) * cols + c);
    add(__builtin_nontemporal_load(src), __builtin_nontemporal_load(src + 1));
  }
  const v4i o = {(int)pack_bf16x2_rne(acc[0], acc[1]), (int)pack_bf16x2_rne(acc[2], acc[3]),
                 (int)pack_bf16x2_rne(acc[4], acc[5]), (int)pack_bf16x2_rne(acc[6], acc[7])};
  *(v4i*)(out + t * cols + c) = o;
}

hipError_t launch_topk_sum(const float* x, int64_t T, int k, int64_t cols, uint16_t* out, hipStream_t st) {
  const int64_t n = T * (cols / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, T, k, cols, out);
  return hipGetLastError();
}


}  // namespace mxk
