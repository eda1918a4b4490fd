// Shared device helpers of the MoonEP HIP library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moonep.h"

namespace moonep {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (uint64_t(1) << lane_id()) - 1;
}

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even.  Adding 0x7fff plus the
// lowest kept bit to the discarded half rounds up exactly when that half is
// above one half-ulp, or equal to it with an odd kept part; a carry out of
// the significand bumps the exponent (and reaches infinity past the largest
// finite bf16).  NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// bf16 bits of the exact product a*b, rounded once (nearest, ties to even).
// The fp32 product p can only land on a bf16 rounding midpoint when the
// exact product differs from it by the residual e = fma(a, b, -p); then e
// decides the side.  Otherwise rounding p gives the same bf16 as rounding
// the exact product.
__device__ __forceinline__ uint32_t mul_to_bf16(float a, float b) {
  const float p = a * b;
  const uint32_t u = __float_as_uint(p);
  if ((u & 0xffffu) == 0x8000u && (u & 0x7fffffffu) < 0x7f800000u) {
    const float e = fmaf(a, b, -p);
    if (e != 0.f) return ((e > 0.f) == (p > 0.f)) ? (u >> 16) + 1u : (u >> 16);
  }
  return f32_to_bf16(p);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Cross-lane reductions with DPP (no LDS round trip).  row_shr:1,2,4,8 scan
// each row of 16 lanes; row_bcast:15 then row_bcast:31 carry the row totals
// into the later rows.  Every lane of the wave must be active.
#define MOONEP_DPP(old, v, ctrl, rows) __builtin_amdgcn_update_dpp((old), (v), (ctrl), (rows), 0xf, false)

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += MOONEP_DPP(0, v, 0x111, 0xf);
  v += MOONEP_DPP(0, v, 0x112, 0xf);
  v += MOONEP_DPP(0, v, 0x114, 0xf);
  v += MOONEP_DPP(0, v, 0x118, 0xf);
  v += MOONEP_DPP(0, v, 0x142, 0xa);
  v += MOONEP_DPP(0, v, 0x143, 0xc);
  return v;
}

// Value of lane `src` (uniform) in every lane.
__device__ __forceinline__ int wave_bcast(int v, int src) {
  return __builtin_amdgcn_readlane(v, src);
}

__device__ __forceinline__ int wave_sum(int v) {
  return wave_bcast(wave_incl_scan(v), kWave - 1);
}

__device__ __forceinline__ float wave_sum_f(float v) {
#define MOONEP_DPPF(x, ctrl, rows) \
  __int_as_float(MOONEP_DPP(0, __float_as_int(x), (ctrl), (rows)))
  v += MOONEP_DPPF(v, 0x111, 0xf);
  v += MOONEP_DPPF(v, 0x112, 0xf);
  v += MOONEP_DPPF(v, 0x114, 0xf);
  v += MOONEP_DPPF(v, 0x118, 0xf);
  v += MOONEP_DPPF(v, 0x142, 0xa);
  v += MOONEP_DPPF(v, 0x143, 0xc);
#undef MOONEP_DPPF
  return __int_as_float(wave_bcast(__float_as_int(v), kWave - 1));
}

// Lanes without a source (or outside the row mask) see INT_MIN, the identity
// of max, so each step is one max with a DPP operand.
__device__ __forceinline__ int wave_max(int v) {
  constexpr int lo = -2147483647 - 1;
  v = max(v, MOONEP_DPP(lo, v, 0x111, 0xf));
  v = max(v, MOONEP_DPP(lo, v, 0x112, 0xf));
  v = max(v, MOONEP_DPP(lo, v, 0x114, 0xf));
  v = max(v, MOONEP_DPP(lo, v, 0x118, 0xf));
  v = max(v, MOONEP_DPP(lo, v, 0x142, 0xa));
  v = max(v, MOONEP_DPP(lo, v, 0x143, 0xc));
  return wave_bcast(v, kWave - 1);
}


}  // namespace moonep
