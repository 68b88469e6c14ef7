// Device-side helpers shared by the gfx950 kernels of libf8lin.
//
// The arithmetic of tensorwise scaling as this library defines it (the
// pages -- pytorch/torchtitan PR #778 and pytorch/ao issue #1297 -- name
// tensorwise dynamic and delayed scaling but do not write the formulas):
//   scale = fmax / max(amax, 1e-12)       binary32, correctly rounded
//   q     = RNE(clamp(fl32(x * scale), -fmax, fmax))   onto the OCP fp8 grid
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace f8lin {

constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;
constexpr float kEps = 1e-12f;
constexpr int kHistLen = 16;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <int FMT>
__device__ __forceinline__ constexpr float fmt_max() {
  return FMT == 0 ? kE4M3Max : kE5M2Max;
}

// fp32 value of the low / high bf16 of a packed pair (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Largest bf16 magnitude (as 15-bit integers) of a packed pair.  Integer order
// of magnitude bits equals numeric order of |x|, with NaN above Inf, so the
// max of these is the amax's bit pattern and NaN propagates.
__device__ __forceinline__ uint32_t mag_max2(uint32_t m, uint32_t w) {
  return max(m, max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
}

// scale = fmax / max(amax, eps); NaN amax gives a NaN scale.  The division
// is IEEE-correctly rounded (hipcc's default for binary32 division).
__device__ __forceinline__ float scale_from_amax(float amax, float fmax) {
  const float d = (amax != amax) ? amax : (amax > kEps ? amax : kEps);
  return fmax / d;
}

// Saturate to [-fmax, fmax] and keep NaN as NaN (the hardware conversion
// below does not saturate: out-of-range values would become NaN/Inf codes).
__device__ __forceinline__ float saturate(float v, float fmax) {
  const float c = fminf(fmaxf(v, -fmax), fmax);
  return (v != v) ? v : c;
}

// Four saturated fp32 values -> four fp8 codes (byte i = value i), rounded to
// nearest even by v_cvt_pk_{fp8,bf8}_f32 (subnormals kept, sign of zero kept).
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int r = 0;
  if constexpr (FMT == 0) {
    r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, r, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  } else {
    r = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, r, false);
    r = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, r, true);
  }
  return (uint32_t)r;
}

// Two packed bf16 pairs (elements 0,1 in w01 and 2,3 in w23) -> four codes.
template <int FMT>
__device__ __forceinline__ uint32_t quantize4(uint32_t w01, uint32_t w23, float s) {
  constexpr float fm = fmt_max<FMT>();
  return cvt4<FMT>(saturate(bf16_lo(w01) * s, fm), saturate(bf16_hi(w01) * s, fm),
                   saturate(bf16_lo(w23) * s, fm), saturate(bf16_hi(w23) * s, fm));
}

// binary32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

}  // namespace f8lin
