// Squared norms of bf16 vectors over their whole exponent range (device code).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

// The quantize kernels sum the squares of a vector's bf16 elements in fp32
// dot2 chains (each square of an 8-bit significand is exact in fp32) and
// combine the chains in fp64.  That is exact up to fp32 rounding of the
// chains only while the squares and the chains stay inside fp32's normal
// range: a total of at least 2^-60 puts any square that underflows more than
// 2^59 below it, and a square or chain past FLT_MAX shows as infinity.
// Vectors outside that range (elements below about 2^-63 or above 2^64)
// redo the sum with every element first scaled by 2^70 (a small total) or
// 2^-70 (an infinite one), exactly, denormal elements included; their
// squares then lie in fp32's normal range wherever they matter.
__device__ __forceinline__ bool sumsq_fast_ok(double ss) { return ss >= 0x1p-60 && ss < __builtin_inf(); }

// The scale 2^70 or 2^-70 of the redone sum, from the first sum.
__device__ __forceinline__ float sumsq_rescale(double ss) { return ss < 0x1p-60 ? 0x1p70f : 0x1p-70f; }

// Sum over the 8 N bf16 elements in w of (x s)^2, in four fp32 chains.
template <int N>
__device__ __forceinline__ float bf16_sumsq_scaled(const uint4 (&w)[N], float s) {
  float c[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const uint32_t ws[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float lo = __uint_as_float(ws[u] << 16) * s;
      const float hi = __uint_as_float(ws[u] & 0xFFFF0000u) * s;
      c[u] = fmaf(lo, lo, c[u]);
      c[u] = fmaf(hi, hi, c[u]);
    }
  }
  return (c[0] + c[1]) + (c[2] + c[3]);
}

}  // namespace tq
