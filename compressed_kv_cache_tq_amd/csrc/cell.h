// Cell index of the code tables (device code).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

// Byte offset 8 c of the cell-table entry of y, for -1 - 1/2048 < y <
// 1 + 1/1024 (a rotated unit-vector coordinate, up to rounding): the fp32
// fma rounds 512 y + 512 + 2^23, which lies in [2^23, 2^24) there, once to
// the nearest integer with ties to even, and bits 3..10 of that mantissa are
// c = RNE(512 y + 512) >> 3.  One fma and one AND, where a truncating
// conversion would also need a clamp and a shift; whatever y is, the AND
// keeps the offset below 2048.
__device__ __forceinline__ uint32_t cell_byte_offset(float y) {
  return __float_as_uint(__builtin_fmaf(y, 512.0f, 8389120.0f)) & 0x7F8u;
}

// The cell-table entry of y: {bits of the boundary inside the cell, codes below}.
__device__ __forceinline__ uint2 cell_entry(const uint2* cells, float y) {
  return *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(cells) + cell_byte_offset(y));
}

}  // namespace tq
