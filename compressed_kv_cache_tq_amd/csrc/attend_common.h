// Shared declarations of the decode-attention translation units: the split
// kernel's constants and partial format, and the per-key-width launchers of
// the split kernel (attend_k*.hip), which attend.hip dispatches to.
#pragma once

#include <cmath>

#include "tq_internal.h"

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int ST = 64 * SW;    // threads per split workgroup
constexpr int GMAX = 16;       // query heads per kv head
constexpr int MAX_SINK = 512;  // raw sink tokens per sequence
constexpr int FROW = D + 8;    // fp16 per fragment row in LDS (pad: no bank conflicts)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float QJL_C = 1.2533141373155003f / QJL_M;  // sqrt(pi/2) / m


struct SplitArgs {
  const Tables* ktab;
  const tq_cache* kc;
  const Tables* vtab;
  const tq_cache* vc;
  const tq_attn* a;
  const AttendPlan* plan;
  const float* q;
  const uint16_t* sink_k;
  const uint16_t* sink_v;
  const int32_t* seq_lens;
  float* parts;
  float* out;
  const int32_t* block_table;  // paged cache: [batch][max_pages] pool pages, else NULL
  int max_pages;
  int n_pages;
  hipStream_t st;
  bool norm16;  // K and V norms stored as fp16
};

// Launch the split kernel for keys of widths (bits_lo, bits_hi) = key / 10,
// key % 10 and values of widths vkey / 10, vkey % 10.
hipError_t split_k22(int vkey, bool qjl, const SplitArgs& f);
hipError_t split_k33(int vkey, bool qjl, const SplitArgs& f);
hipError_t split_k44(int vkey, bool qjl, const SplitArgs& f);
hipError_t split_k43(int vkey, bool qjl, const SplitArgs& f);
hipError_t split_k32(int vkey, bool qjl, const SplitArgs& f);
hipError_t split_k88(int vkey, bool qjl, const SplitArgs& f);  // values 2 or 3 bits, no sketch

}  // namespace tq
