// Cross-lane sums of a wave without an LDS round trip (device code).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

// x + (x of lane l ^ M), M = 1 or 2: quad-permute DPP moves of both halves.
// Both lanes of a pair form the same sum (the addition commutes).
template <int M>
__device__ __forceinline__ double add_quad_xor(double x) {
  static_assert(M == 1 || M == 2, "lane mask");
  constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), ctrl, 0xF, 0xF, false));
  const uint32_t hi =
      static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u >> 32), ctrl, 0xF, 0xF, false));
  return x + __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// x of lane l ^ 32 (the other half of the wave): one permlane32 swap per
// dword.  The swap returns, in each lane, the old value of the other half's
// lane in the operand its own half did not supply.
__device__ __forceinline__ uint32_t other_half(uint32_t v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? sw[0] : sw[1];
}
__device__ __forceinline__ float add_half_swap(float x) {
  return x + __uint_as_float(other_half(__float_as_uint(x)));
}
__device__ __forceinline__ double add_half_swap(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint64_t o = (static_cast<uint64_t>(other_half(static_cast<uint32_t>(u >> 32))) << 32) |
                     other_half(static_cast<uint32_t>(u));
  return x + __builtin_bit_cast(double, o);
}

}  // namespace tq
