// Device-side helpers shared by the MXFP8 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

// Largest finite E4M3 magnitude.
constexpr float kE4M3Max = 448.0f;

// E8M0 scale byte of a block from the bit pattern of its largest |bf16|.
// The exponent field minus 8 (E4M3's largest exponent) is floor(log2 amax) - 8
// + 127 already biased; subnormal and small amax clamp to 0.  A block holding
// NaN or Inf (|bits| >= 0x7F80) gets 0xFF.  This is the bit-manipulation form
// of clamp(floor(log2 amax) - 8, -127, 127) + 127 for every bf16 amax.
__device__ __forceinline__ uint32_t e8m0_from_absbits(uint32_t amax_bits) {
  if (amax_bits >= 0x7F80u) return 0xFFu;
  int e = (int)(amax_bits >> 7) - 8;
  return (uint32_t)(e > 0 ? e : 0);
}

// 2^(127 - byte) as an fp32 (byte in 0..253): exponent field 254 - byte.
__device__ __forceinline__ float inv_scale_from_e8m0(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

// Two scaled values -> two E4M3 codes in the low (HI=false) or high (HI=true)
// 16 bits of `old`.  The hardware convert rounds to nearest even, keeps
// subnormals and the sign of zero, but does not saturate: values are clamped
// to +-448 first.
template <bool HI>
__device__ __forceinline__ int cvt2_e4m3(float a, float b, int old) {
  a = __builtin_fminf(__builtin_fmaxf(a, -kE4M3Max), kE4M3Max);
  b = __builtin_fminf(__builtin_fmaxf(b, -kE4M3Max), kE4M3Max);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// bf16 pair packed in a dword -> fp32 values (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Quantize 8 bf16 values (4 dwords) of one block with multiplier `m`
// (2^(127-byte)); returns 8 E4M3 codes in two dwords (element order kept).
__device__ __forceinline__ v2i quant8(v4i w, float m) {
  int c0 = cvt2_e4m3<false>(bf16lo(w[0]) * m, bf16hi(w[0]) * m, 0);
  c0 = cvt2_e4m3<true>(bf16lo(w[1]) * m, bf16hi(w[1]) * m, c0);
  int c1 = cvt2_e4m3<false>(bf16lo(w[2]) * m, bf16hi(w[2]) * m, 0);
  c1 = cvt2_e4m3<true>(bf16lo(w[3]) * m, bf16hi(w[3]) * m, c1);
  v2i r;
  r[0] = c0;
  r[1] = c1;
  return r;
}

// Largest |bf16| bit pattern among the 8 values in 4 dwords (as 16-bit max).
__device__ __forceinline__ uint32_t absmax8(v4i w) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t u = (uint32_t)w[i] & 0x7FFF7FFFu;
    uint32_t lo = u & 0xFFFFu, hi = u >> 16;
    m = max(m, max(lo, hi));
  }
  return m;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 pair (low half = lo), round to nearest
// even, with the hardware convert (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  const bf16x2_t h = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

// Max across the 4 lanes of a DPP quad.
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  return v;
}

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace mxk
