// Decode attention read directly from the packed cache: the split kernel
// (templates; attend_k*.hip instantiate them per key width, attend.hip holds
// the combine and the dispatch).
//
// noze.it, "TurboQuant-MLX: quantizzare pesi e KV cache per LLM open-weight su
// Mac", section "Il metodo TurboQuant, in breve": inner products are taken
// against the codebook reconstruction, corrected by the 1-bit residual sketch
// when present.  GitHub issue "Greetings from TurboQuant-MLX & Some Insights
// to Share!": item 1 (the first ~128 tokens stay uncompressed) and item 3
// (value dequantization is skipped when the attention weight is below 1e-6).
//
// One or two launches on one stream:
//  split    one workgroup of 8 waves per (split, kv head, sequence).
//           Prologue: the workgroup rotates the query heads of its group,
//           q~ = Pi_K q (times scale * log2 e), and u = S q~, scales each
//           head by a power of two and splits it into fp16 hi + lo operand
//           fragments in LDS.  Stream: each wave streams 32-token tiles with
//           two tiles in flight in registers: K records -> LUT
//           dequantization -> scores on MFMA for all query heads of the
//           group -> online softmax -> V tiles (coordinate-major sub-blocks)
//           -> P V on MFMA in the rotated domain.  The waves merge in LDS and
//           write one partial (m, l, acc[128]) per query head.  The
//           stream's last split with compressed tokens also writes the
//           partial of the raw sink tokens (slot n_split, acc in the
//           original value domain).  When the plan gives every stream a
//           single split, the workgroup then merges its own partials into
//           the output (no second launch).  A paged cache reads every
//           32-token tile through descriptors over the tile's pool page,
//           looked up in the device block table;
//  combine  (several splits per stream only) one workgroup per (sequence,
//           query head, output slice): log-sum-exp merge of the partials,
//           the slice of one inverse rotation Pi_V^T of the rotated sum,
//           the sink values, and the normalisation.
//
// Codebook LUTs: entry e of width B maps two codes to their two fp16
// centroids.  The centroids depend only on (d, B), so one LUT per width
// serves K and V.  Each entry is replicated 64 times (one copy per lane) so
// every lookup is bank-conflict free; the address (pair << 8) | (lane << 2)
// of a 4-bit byte pair is built by one v_perm.
#pragma once

#include "attend_common.h"

namespace tq {
namespace {


__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(half8, make_uint4(a, b, c, d));
}

// 8B bits starting at stream bit 8B*k of the little-endian words w.
template <int B>
__device__ __forceinline__ uint32_t row_bits(const uint32_t* w, int k) {
  constexpr int NB = 8 * B;
  const int bit = NB * k, wd = bit >> 5, off = bit & 31;
  uint32_t v = w[wd] >> off;
  if (off + NB > 32) v |= w[wd + 1] << (32 - off);
  return NB == 32 ? v : (v & ((1u << NB) - 1u));
}

// LDS layout of the replicated LUTs (bytes): widths 3 and 2 first, then 4
// and 8, so every LUT base (at most 20 KiB) fits the immediate offset of the
// LDS read and the lane-dependent part of the address is one AND-OR.  Widths
// up to 4 map a code pair (one byte of 4-bit codes) to two fp16 centroids,
// each times the width's centroid scale from the tables (divided out of the
// query coordinates and the value accumulator); width 8 maps one code (one
// byte) to one fp16 centroid in the low half (scale 1).
template <int B>
constexpr int lut_entries() { return B == 8 ? 256 : 1 << (2 * B); }
template <int B>
constexpr int lut_size() { return lut_entries<B>() * 256; }
template <int KLO, int KHI, int VLO, int VHI>
struct LutPlan {
  static constexpr bool has(int B) { return KLO == B || KHI == B || VLO == B || VHI == B; }
  static constexpr int off3 = 0;
  static constexpr int off2 = off3 + (has(3) ? lut_size<3>() : 0);
  static constexpr int off4 = off2 + (has(2) ? lut_size<2>() : 0);
  static constexpr int off8 = off4 + (has(4) ? lut_size<4>() : 0);
  static constexpr int bytes = off8 + (has(8) ? lut_size<8>() : 0);
  template <int B>
  static constexpr int off() { return B == 8 ? off8 : B == 4 ? off4 : B == 3 ? off3 : off2; }
};

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint32_t*>(base + off);
}

// 8 codes of width B (row k of the lane's words) -> 8 fp16 centroids.
template <int B>
__device__ __forceinline__ half8 dequant8(const uint32_t* w, int k, const uint8_t* lut, uint32_t lane4) {
  uint32_t a[4];
  if constexpr (B == 8) {
    // one code per byte: codes 8k .. 8k+7 are the bytes of w[2k], w[2k+1]
    uint32_t c[8];
#pragma unroll
    for (int p = 0; p < 8; ++p)
      c[p] = lds_u32(lut, __builtin_amdgcn_perm(w[2 * k + (p >> 2)], lane4, 0x0C0C0000u | ((4u + (p & 3)) << 8)));
    return as_half8(c[0] | (c[1] << 16), c[2] | (c[3] << 16), c[4] | (c[5] << 16), c[6] | (c[7] << 16));
  } else if constexpr (B == 4) {
    const uint32_t v = w[k];
#pragma unroll
    for (int p = 0; p < 4; ++p) a[p] = __builtin_amdgcn_perm(v, lane4, 0x0C0C0000u | ((4u + p) << 8));
  } else {
    // pair p sits at bits [2Bp, 2Bp + 2B) of the row: move it to bit 8
    const uint32_t v = row_bits<B>(w, k);
    constexpr uint32_t M = ((1u << (2 * B)) - 1u) << 8;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int sh = 8 - 2 * B * p;
      const uint32_t t = sh >= 0 ? v << sh : v >> (-sh);
      a[p] = (t & M) | lane4;
    }
  }
  return as_half8(lds_u32(lut, a[0]), lds_u32(lut, a[1]), lds_u32(lut, a[2]), lds_u32(lut, a[3]));
}

// Registers of one 32-token tile for one lane (two tiles in flight per wave);
// KWD = dwords of a lane's 32 key codes (8 for 8-bit keys, else 4).
template <int KWD>
struct TileRegs {
  uint32_t kw[2][KWD];  // K record chunk of token slots mu(0, n), mu(1, n)
  uint32_t vw[8];     // V sub-block (token group j, coordinate group n)
  float4 kn[2];       // K norms of tokens 8j .. 8j+7 (fp16 norms: their bits in kn[0])
  float4 vn[2];       // V norms of tokens 8j .. 8j+7 (fp16 norms: their bits in vn[0])
  uint32_t zw[2];     // QJL sign dword j of token slots mu(0, n), mu(1, n)
  float4 rn[2];       // QJL residual norms of tokens 8j .. 8j+7
};

constexpr int RSRC_WORD3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), RSRC_WORD3);
}

// Buffer descriptors of one (sequence, kv head) stream.  Loads past a
// descriptor's extent return zeros, so the stream loop issues every tile's
// loads unconditionally and runs ahead of the last tile without branches.
struct StreamRsrc {
  __amdgpu_buffer_rsrc_t kc, vc, kn, vn, zs, rn;
};

// Per-lane byte offsets of tile 0 of the stream; tile t0 adds t0 times the
// per-token stride of each array (t0 is a multiple of 32, and a V tile of
// 32 tokens is 32 * VBYTES contiguous bytes).
struct LaneOffsets {
  uint32_t k[2], k2[2], z[2], v, v2, nrm;
  uint32_t tokc;    // compact softmax: the lane's token within its tile (its norms' index)
  uint32_t ksh[2];  // mixed-width keys: bit offset of each part in its two loaded dwords
};

template <int N>
__device__ __forceinline__ void buf_load(uint32_t (&dst)[N], __amdgpu_buffer_rsrc_t r, uint32_t off, int first = 0) {
  static_assert(N == 2 || N == 3 || N == 4 || N == 6 || N == 8, "load width");
  if constexpr (N == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    dst[0] = v[0]; dst[1] = v[1];
  } else if constexpr (N == 3) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
    dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2];
  } else if constexpr (N == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
    uint32_t t[N - 4];
    buf_load<N - 4>(t, r, off + 16);
#pragma unroll
    for (int i = 0; i < N - 4; ++i) dst[4 + i] = t[i];
  }
}

__device__ __forceinline__ float4 buf_load_f4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int KLO, int KHI>
constexpr int key_dwords() { return KLO == 8 ? 8 : 4; }

// Loads of one tile.  CG (the compact softmax of groups of at most 4 query
// heads): each lane loads the norms (and residual norm) of one token only,
// token lo.tokc of the tile, into component x of kn[0], vn[0], rn[0].
template <int KLO, int KHI, int VLO, int VHI, bool QJL, bool NF16, bool CG>
__device__ __forceinline__ void load_tile(TileRegs<key_dwords<KLO, KHI>()>& r, uint32_t t0, const StreamRsrc& rs,
                                          const LaneOffsets& lo) {
  constexpr uint32_t KBYTES = 8 * (KLO + KHI);
  constexpr uint32_t VBYTES = 8 * (VLO + VHI);
  constexpr int KW = KLO > KHI ? KLO : KHI;
  constexpr int VW = 2 * (VLO > VHI ? VLO : VHI);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    if constexpr (KLO != KHI) {
      // two dwords around each width's 16 codes
      uint32_t w[2];
      buf_load<2>(w, rs.kc, lo.k[mb] + t0 * KBYTES);
      r.kw[mb][0] = w[0];
      r.kw[mb][1] = w[1];
      buf_load<2>(w, rs.kc, lo.k2[mb] + t0 * KBYTES);
      r.kw[mb][2] = w[0];
      r.kw[mb][3] = w[1];
    } else {
      uint32_t w[KW];
      buf_load<KW>(w, rs.kc, lo.k[mb] + t0 * KBYTES);
#pragma unroll
      for (int i = 0; i < KW; ++i) r.kw[mb][i] = w[i];
    }
    if constexpr (QJL) r.zw[mb] = __builtin_amdgcn_raw_buffer_load_b32(rs.zs, lo.z[mb] + t0 * (QJL_M / 8), 0, 0);
  }
  if constexpr (VLO != VHI) {
    // four rows of a VLO sub-block and four of a VHI sub-block
    uint32_t w[VLO], w2[VHI];
    buf_load<VLO>(w, rs.vc, lo.v + t0 * VBYTES);
    buf_load<VHI>(w2, rs.vc, lo.v2 + t0 * VBYTES);
#pragma unroll
    for (int i = 0; i < VLO; ++i) r.vw[i] = w[i];
#pragma unroll
    for (int i = 0; i < VHI; ++i) r.vw[4 + i] = w2[i];
  } else {
    uint32_t w[VW];
    buf_load<VW>(w, rs.vc, lo.v + t0 * VBYTES);
#pragma unroll
    for (int i = 0; i < VW; ++i) r.vw[i] = w[i];
  }
  if constexpr (CG) {
    constexpr uint32_t NB = NF16 ? 2 : 4;
    if constexpr (NF16) {
      r.kn[0].x = __uint_as_float(static_cast<uint32_t>(
          __builtin_amdgcn_raw_buffer_load_b16(rs.kn, NB * (lo.tokc + t0), 0, 0)));
      r.vn[0].x = __uint_as_float(static_cast<uint32_t>(
          __builtin_amdgcn_raw_buffer_load_b16(rs.vn, NB * (lo.tokc + t0), 0, 0)));
    } else {
      r.kn[0].x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs.kn, NB * (lo.tokc + t0), 0, 0));
      r.vn[0].x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs.vn, NB * (lo.tokc + t0), 0, 0));
    }
    if constexpr (QJL) r.rn[0].x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs.rn, 4 * (lo.tokc + t0), 0, 0));
    return;
  }
  if constexpr (NF16) {
    // 8 fp16 norms in one 16-byte load, converted where they are used
    r.kn[0] = buf_load_f4(rs.kn, (lo.nrm >> 1) + 2 * t0);
    r.vn[0] = buf_load_f4(rs.vn, (lo.nrm >> 1) + 2 * t0);
  } else {
    r.kn[0] = buf_load_f4(rs.kn, lo.nrm + 4 * t0);
    r.kn[1] = buf_load_f4(rs.kn, lo.nrm + 4 * t0 + 16);
    r.vn[0] = buf_load_f4(rs.vn, lo.nrm + 4 * t0);
    r.vn[1] = buf_load_f4(rs.vn, lo.nrm + 4 * t0 + 16);
  }
  if constexpr (QJL) {
    r.rn[0] = buf_load_f4(rs.rn, lo.nrm + 4 * t0);
    r.rn[1] = buf_load_f4(rs.rn, lo.nrm + 4 * t0 + 16);
  }
}

// Sum over the 32 lanes of each half wave: rotations within 16-lane rows,
// then the row-swap permute.
__device__ __forceinline__ float sum32(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xF, 0xF, false));
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Maximum over lanes l, l^16, l^32, l^48 (the four token groups of a head):
// the row-swap permutes exchange 16- and 32-lane halves without LDS.
__device__ __forceinline__ float max_xor16_32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Maximum and sum over all 64 lanes (row rotations, then the row swaps).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xF, 0xF, false)));
  return max_xor16_32(x);
}
__device__ __forceinline__ float wave_sum(float x) {
  x = sum32(x);
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Row j of the result is row 0 of input j (rows are 16-lane groups): the
// odd rows of the first operand of a 16-row swap trade places with the even
// rows of the second, and the upper half of the first operand of a 32-lane
// swap with the lower half of the second.
__device__ __forceinline__ float gather_rows0(float a0, float a1, float b0, float b1) {
  const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
  const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(b0), __float_as_uint(b1), false, false);
  const auto f = __builtin_amdgcn_permlane32_swap(x[0], z[0], false, false);
  return __uint_as_float(f[0]);
}

__device__ __forceinline__ float f4get(const float4 (&v)[2], int e) {
  const float4 x = v[e >> 2];
  const int k = e & 3;
  return k == 0 ? x.x : k == 1 ? x.y : k == 2 ? x.z : x.w;
}

// norm e (0..7) of a tile's lane: fp32, or fp16 packed two per word of v[0]
template <bool NF16>
__device__ __forceinline__ float norm_get(const float4 (&v)[2], int e) {
  if constexpr (!NF16) return f4get(v, e);
  const float4 x = v[0];
  const int k = e >> 1;
  const uint32_t w = __float_as_uint(k == 0 ? x.x : k == 1 ? x.y : k == 2 ? x.z : x.w);
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> (16 * (e & 1)))));
}

// Partial (m, l, acc) of the raw bf16 sink tokens t < ns of one (sequence,
// kv head) for the G query heads of the group: s = qscale <q, k_t> (log2
// domain), m = max s, l = sum 2^(s - m), acc = sum 2^(s - m) v_t in the
// original value domain.  Head g's partial is written at part + g * stride.
// 512 threads.
__device__ __forceinline__ void sink_partial(uint8_t* smem, const float* __restrict__ qg,
                                             const uint16_t* __restrict__ sk, const uint16_t* __restrict__ sv,
                                             int ns, int G, float qscale, float* __restrict__ part, int64_t stride) {
  float* qs = reinterpret_cast<float*>(smem);  // [GMAX][D]
  float* sc = qs + GMAX * D;                   // [GMAX][MAX_SINK]: scores, then weights
  float* accp = sc + GMAX * MAX_SINK;          // [2][GMAX][D]
  float* mls = accp + 2 * GMAX * D;            // [GMAX][2]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int idx = tid; idx < G * D; idx += ST) qs[idx] = qg[idx] * qscale;
  __syncthreads();
  // scores: thread t takes token t
  if (tid < ns) {
    uint4 row[D / 8];
    const uint4* rp = reinterpret_cast<const uint4*>(sk + static_cast<int64_t>(tid) * D);
#pragma unroll
    for (int k = 0; k < D / 8; ++k) row[k] = rp[k];
    for (int g = 0; g < G; ++g) {
      const float4* qv = reinterpret_cast<const float4*>(qs + g * D);
      float dot = 0.0f;
#pragma unroll
      for (int k = 0; k < D / 8; ++k) {
        const float4 a = qv[2 * k], c = qv[2 * k + 1];
        const uint4 wv = row[k];
        dot = fmaf(__uint_as_float(wv.x << 16), a.x, dot);
        dot = fmaf(__uint_as_float(wv.x & 0xFFFF0000u), a.y, dot);
        dot = fmaf(__uint_as_float(wv.y << 16), a.z, dot);
        dot = fmaf(__uint_as_float(wv.y & 0xFFFF0000u), a.w, dot);
        dot = fmaf(__uint_as_float(wv.z << 16), c.x, dot);
        dot = fmaf(__uint_as_float(wv.z & 0xFFFF0000u), c.y, dot);
        dot = fmaf(__uint_as_float(wv.w << 16), c.z, dot);
        dot = fmaf(__uint_as_float(wv.w & 0xFFFF0000u), c.w, dot);
      }
      sc[g * MAX_SINK + tid] = dot;
    }
  }
  __syncthreads();
  // per head: maximum, weights, their sum (wave w takes heads w, w + 8)
  for (int g = wave; g < G; g += SW) {
    float mx = -INFINITY;
    for (int t = lane; t < ns; t += 64) mx = fmaxf(mx, sc[g * MAX_SINK + t]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float sum = 0.0f;
    for (int t = lane; t < ns; t += 64) {
      const float w = __builtin_amdgcn_exp2f(sc[g * MAX_SINK + t] - mx);
      sc[g * MAX_SINK + t] = w;
      sum += w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) {
      mls[2 * g] = mx;
      mls[2 * g + 1] = sum;
    }
  }
  __syncthreads();
  // weighted values: thread (i, tq) takes coordinate i of tokens tq, tq + 4, ...
  const int i = tid & (D - 1), tq = tid >> 7;
  float acc[GMAX];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) acc[g] = 0.0f;
#pragma unroll 16
  for (int t = tq; t < ns; t += 4) {
    const float v = __uint_as_float(static_cast<uint32_t>(sv[static_cast<int64_t>(t) * D + i]) << 16);
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
      if (g < G) acc[g] = fmaf(sc[g * MAX_SINK + t], v, acc[g]);
  }
  // sum the four token groups
  if (tq >= 2) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
      if (g < G) accp[((tq - 2) * GMAX + g) * D + i] = acc[g];
  }
  __syncthreads();
  if (tq < 2) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
      if (g < G) acc[g] += accp[(tq * GMAX + g) * D + i];
  }
  __syncthreads();
  if (tq == 1) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
      if (g < G) accp[g * D + i] = acc[g];
  }
  __syncthreads();
  if (tq == 0) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
      if (g < G) {
        float* pg = part + g * stride;
        pg[4 + i] = acc[g] + accp[g * D + i];
        if (i == 0) {
          pg[0] = mls[2 * g];
          pg[1] = mls[2 * g + 1];
        }
      }
  }
}

// Index of the r-th longest of the n sequences (ties by index), for n up to
// MAX_RANK; r itself above that.  Every workgroup ranks the lengths anew:
// thread t counts the sequences that sort before t.
constexpr int MAX_RANK = 512;
__device__ __forceinline__ int rank_sequence(const int32_t* __restrict__ seq_lens, int n, int r) {
  if (n <= 1 || n > MAX_RANK) return r;
  __shared__ int lens_s[MAX_RANK];
  __shared__ int order_s[MAX_RANK];
  for (int t = threadIdx.x; t < n; t += ST) lens_s[t] = seq_lens[t];
  __syncthreads();
  for (int t = threadIdx.x; t < n; t += ST) {
    const int lt = lens_s[t];
    int before = 0;
    for (int u = 0; u < n; ++u) {
      const int lu = lens_s[u];
      before += (lu > lt) | ((lu == lt) & (u < t));
    }
    order_s[before] = t;
  }
  __syncthreads();
  return order_s[r];
}

// Merge of one stream's partials, run by the stream's workgroup when it is
// the stream's only split: for each of its G query heads, the log-sum-exp weights of
// the n_split split partials (rotated value domain) and of the sink partial
// (slot n_split, original domain, present when n_slot > n_split), the
// weighted rotated sum (divided by the value codebook's centroid scale), one
// inverse rotation Pi_V^T, the division by l.
// pp: partials of the group's first head; og: its output rows.
__device__ __forceinline__ void merge_stream(uint8_t* smem, const Tables* __restrict__ vtab,
                                             const float* __restrict__ pp, float* __restrict__ og, int G,
                                             int n_split, int n_slot) {
  constexpr int WROW = MAX_SPLIT + 1;
  float* wsm = reinterpret_cast<float*>(smem);  // [GMAX][WROW]: slot maxima, then weights
  float* pr = wsm;                              // [4][GMAX][D]: quarters of the inverse rotation (later)
  float* lsum = wsm + GMAX * WROW;              // [GMAX]
  float* swt = lsum + GMAX;                     // [GMAX]: weight of the sink partial
  float* rs = swt + GMAX;                       // [GMAX][D]: weighted rotated sums
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int o = tid & (D - 1), cq = tid >> 7;
  // this thread's slice of Pi (used last) goes out first
  float pic[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) pic[k] = vtab->pi[(32 * cq + k) * D + o];
  // weights: wave w takes heads w, w + SW
  for (int g = wave; g < G; g += SW) {
    const float* ph = pp + static_cast<int64_t>(g) * n_slot * PART;
    float* wg = wsm + g * WROW;
    float mloc = -INFINITY;
    for (int sl = lane; sl < n_slot; sl += 64) {
      const float m = ph[sl * PART], l = ph[sl * PART + 1];
      const float mv = l > 0.0f ? m : -INFINITY;
      wg[sl] = mv;
      mloc = fmaxf(mloc, mv);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
    float lloc = 0.0f;
    for (int sl = lane; sl < n_slot; sl += 64) {
      const float mv = wg[sl];
      const float f = mv == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv - mloc);
      wg[sl] = f;
      lloc = fmaf(f, ph[sl * PART + 1], lloc);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lloc += __shfl_xor(lloc, off);
    if (lane == 0) lsum[g] = lloc;
  }
  __syncthreads();
  // weighted rotated sums: thread (g, c) per pass
  for (int idx = tid; idx < G * D; idx += ST) {
    const int g = idx >> 7, c = idx & (D - 1);
    const float* ph = pp + static_cast<int64_t>(g) * n_slot * PART + 4 + c;
    const float* wg = wsm + g * WROW;
    float a = 0.0f;
#pragma unroll 8
    for (int sl = 0; sl < n_split; ++sl) a = fmaf(wg[sl], ph[sl * PART], a);
    // (the value lookup tables hold centroids times the codebook's scale)
    rs[idx] = a / vtab->cen16_scale[c < static_cast<int>(vtab->split) ? 0 : 1];
  }
  if (tid < G) swt[tid] = n_slot > n_split ? wsm[tid * WROW + n_split] : 0.0f;
  __syncthreads();
  // inverse rotation: thread (o, cq) takes rotated coordinates [32 cq, 32 cq + 32)
  for (int g = 0; g < G; ++g) {
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) v = fmaf(pic[k], rs[g * D + 32 * cq + k], v);
    pr[(cq * GMAX + g) * D + o] = v;
  }
  __syncthreads();
  const bool has_sink = n_slot > n_split;
  for (int idx = tid; idx < G * D; idx += ST) {
    const int g = idx >> 7, oo = idx & (D - 1);
    float v = ((pr[g * D + oo] + pr[(GMAX + g) * D + oo]) + pr[(2 * GMAX + g) * D + oo]) + pr[(3 * GMAX + g) * D + oo];
    if (has_sink) v = fmaf(swt[g], pp[(static_cast<int64_t>(g) * n_slot + n_split) * PART + 4 + oo], v);
    const float L = lsum[g];
    og[idx] = L > 0.0f ? v / L : 0.0f;
  }
}

// CG: the compact softmax for groups of at most 4 query heads.  The score
// product is taken transposed (query fragments as the A operand), so each
// 32-token M-block leaves the 4 heads of a token in one lane of the first
// 16-lane row; the rows of four blocks (two tiles) are gathered into one
// register set, the softmax then runs on 4 values per lane for 64 tokens
// instead of 16 for 32, and the probabilities reach the P V product through
// a per-wave LDS array.  Each lane loads the norms of its own token only,
// which leaves registers for two pairs of tiles in flight.
template <int KLO, int KHI, int VLO, int VHI, bool QJL, bool PAGED, bool NF16, bool CG>
__global__ __launch_bounds__(ST, 1) void split_kernel(
    const Tables* __restrict__ ktab, const uint8_t* __restrict__ kcodes, const float* __restrict__ knorms,
    const uint8_t* __restrict__ ksigns, const float* __restrict__ krn, int64_t kcap,
    const Tables* __restrict__ vtab, const uint8_t* __restrict__ vcodes, const float* __restrict__ vnorms,
    int64_t vcap, const int32_t* __restrict__ seq_lens, const float* __restrict__ q,
    const uint16_t* __restrict__ sink_k, const uint16_t* __restrict__ sink_v, float* __restrict__ parts,
    float* __restrict__ out, int hq, int hkv, int sink, int n_split, int n_slot,
    int64_t chunk, float v_skip, float qscale, const int32_t* __restrict__ block_table, int max_pages,
    int n_pages, int max_len) {
  using LP = LutPlan<KLO, KHI, VLO, VHI>;
  constexpr int KBYTES = 8 * (KLO + KHI);
  constexpr int VBYTES = 8 * (VLO + VHI);
  // LDS: [LUTs | query prologue] while streaming, then reused by the wave
  // merge.
  constexpr int PRO_OFF = (LP::bytes + 255) / 256 * 256;
  // prologue: qraw [GMAX][D] f32, ppart [4][GMAX][D] f32, qrot [GMAX][D] f32
  // (QJL), fragments [sets][hi, lo][GMAX + 1][FROW] fp16, shx [2][GMAX],
  // umax [GMAX]
  constexpr int NSET = QJL ? 2 : 1;
  constexpr int FRAG_BYTES = NSET * 2 * (GMAX + 1) * FROW * 2;
  constexpr int PRO = (GMAX * D + 4 * GMAX * D + (QJL ? GMAX * D : 0)) * 4 + FRAG_BYTES + 3 * GMAX * 4;
  constexpr int MRG = SW * 16 * (D + 2) * 4;
  constexpr int SMEM = PRO_OFF + PRO > MRG ? PRO_OFF + PRO : MRG;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  static_assert(SMEM >= (GMAX * D + GMAX * MAX_SINK + 2 * GMAX * D + 2 * GMAX) * 4, "LDS of the sink split");
  static_assert(SMEM >= (GMAX * (MAX_SPLIT + 1) + 2 * GMAX + GMAX * D) * 4 && GMAX * (MAX_SPLIT + 1) >= 4 * GMAX * D,
                "LDS of the stream merge");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ uint32_t lutz[4];

  // grid (kv head, sequence rank, split): workgroups are dispatched split by
  // split, so every stream's whole leading splits start before the partial
  // and empty trailing ones of a ragged batch.  Within a split, sequences go
  // longest first (for batches of up to MAX_RANK sequences), so the short
  // ones fill the tail.
  const int kh = blockIdx.x, split = blockIdx.z;
  const int b = rank_sequence(seq_lens, gridDim.y, blockIdx.y);
  const int G = hq / hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
  const int64_t stream = static_cast<int64_t>(b) * hkv + kh;
  // (a length outside [0, max_len] breaks the caller's contract; clamping it
  // keeps every access inside the cache the host validated)
  const int64_t L = min(max(seq_lens[b], 0), max_len);
  // The sink tokens' partial (slot n_split, acc in the original value
  // domain) is computed by the stream's last split that holds compressed
  // tokens (split 0 when there are none), after its own partial, when the
  // whole LDS is free.
  const int64_t comp_all = L > sink ? L - sink : 0;
  const int last_split = comp_all > 0 ? static_cast<int>((comp_all - 1) / chunk) : 0;
  auto sink_part = [&]() {
    if (sink > 0 && split == last_split) {
      __syncthreads();
      sink_partial(smem, q + (static_cast<int64_t>(b) * hq + static_cast<int64_t>(kh) * G) * D,
                   sink_k + stream * sink * D, sink_v + stream * sink * D,
                   static_cast<int>(L < sink ? L : sink), G, qscale,
                   parts + (static_cast<int64_t>(b) * hq + static_cast<int64_t>(kh) * G) * n_slot * PART +
                       static_cast<int64_t>(n_split) * PART,
                   n_slot * PART);
    }
  };
  // A stream with a single split (a large batch) is merged right here, from
  // the partials this workgroup has just written; several splits are merged
  // by the combine kernel.
  auto finish = [&]() {
    if (n_split != 1) return;
    __syncthreads();
    const int64_t h0 = static_cast<int64_t>(b) * hq + static_cast<int64_t>(kh) * G;
    merge_stream(smem, vtab, parts + h0 * n_slot * PART, out + h0 * D, G, n_split, n_slot);
  };
  // ---- prologue: rotate the group's queries.  Thread (pi_i, kq) forms the
  // partial dot of rotated coordinate pi_i over inputs [32 kq, 32 kq + 32).
  float* qraw = reinterpret_cast<float*>(smem + PRO_OFF);  // [GMAX][D]
  float* ppart = qraw + GMAX * D;                            // [4][GMAX][D]
  float* qrot = ppart + 4 * GMAX * D;                        // [GMAX][D] (QJL)
  _Float16* frag = reinterpret_cast<_Float16*>(qrot + (QJL ? GMAX * D : 0));  // [NSET][2][GMAX+1][FROW]
  int* shx = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(frag) + FRAG_BYTES);  // [2][GMAX]
  uint32_t* umax = reinterpret_cast<uint32_t*>(shx + 2 * GMAX);                    // [GMAX] (QJL)
  auto frag_row = [&](int set, int part, int g) { return frag + ((set * 2 + part) * (GMAX + 1) + g) * FROW; };
  const float* qg = q + (static_cast<int64_t>(b) * hq + static_cast<int64_t>(kh) * G) * D;
  const int pi_i = tid & (D - 1), kq = tid >> 7;

  // The prologue's own loads go out first (the centroids before Pi, so that
  // the LUT stores wait for them alone), the sequence length is read only
  // then, and the tile loads follow: the prologue waits only for its small
  // L2-resident operands while the first two tiles stream in from HBM.
  const float4 qv = tid < G * (D / 4) ? reinterpret_cast<const float4*>(qg)[tid] : float4{};
  // replicated pair LUTs: entry e of width B at off_B + e*256 + replica*4;
  // thread t fills 16-byte chunks t, t + ST, ... from centroids (lo, hi)
  auto lut_vals = [&](auto bw, uint16_t(&cl)[lut_entries<decltype(bw)::value>() * 16 / ST + 1],
                      uint16_t(&ch)[lut_entries<decltype(bw)::value>() * 16 / ST + 1]) {
    constexpr int B = decltype(bw)::value;
    if constexpr (LP::has(B) && B == 8) {
      // (8-bit codes: keys only)
#pragma unroll
      for (int r = 0; r * ST < 256 * 16; ++r) {
        cl[r] = ktab->cen16_8[((threadIdx.x + r * ST) >> 4) & 255];
        ch[r] = 0;
      }
    } else if constexpr (LP::has(B)) {
      const uint16_t* cen = (KLO == B) ? ktab->cen16[0] : (KHI == B) ? ktab->cen16[1]
                          : (VLO == B) ? vtab->cen16[0] : vtab->cen16[1];
      constexpr int E = 1 << (2 * B);
      constexpr uint32_t MK = (1u << B) - 1u;
#pragma unroll
      for (int r = 0; r * ST < E * 16; ++r) {
        const int c = threadIdx.x + r * ST;
        const int e = (c >> 4) & (E - 1);
        cl[r] = cen[e & MK];
        ch[r] = cen[e >> B];
      }
    }
  };
  auto lut_store = [&](auto bw, const uint16_t(&cl)[lut_entries<decltype(bw)::value>() * 16 / ST + 1],
                       const uint16_t(&ch)[lut_entries<decltype(bw)::value>() * 16 / ST + 1]) {
    constexpr int B = decltype(bw)::value;
    if constexpr (LP::has(B)) {
      constexpr int E = lut_entries<B>();
#pragma unroll
      for (int r = 0; r * ST < E * 16; ++r) {
        const int c = threadIdx.x + r * ST;
        const uint32_t v = static_cast<uint32_t>(cl[r]) | (static_cast<uint32_t>(ch[r]) << 16);
        if (c < E * 16) reinterpret_cast<uint4*>(smem + LP::template off<B>())[c] = make_uint4(v, v, v, v);
      }
    }
  };
  uint16_t l4l[256 * 16 / ST + 1], l4h[256 * 16 / ST + 1], l3l[64 * 16 / ST + 1], l3h[64 * 16 / ST + 1],
      l2l[16 * 16 / ST + 1], l2h[16 * 16 / ST + 1], l8l[256 * 16 / ST + 1], l8h[256 * 16 / ST + 1];
  lut_vals(std::integral_constant<int, 8>{}, l8l, l8h);
  lut_vals(std::integral_constant<int, 4>{}, l4l, l4h);
  lut_vals(std::integral_constant<int, 3>{}, l3l, l3h);
  lut_vals(std::integral_constant<int, 2>{}, l2l, l2h);
  float w[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) w[k] = ktab->pit[(32 * kq + k) * D + pi_i];

  const int64_t comp = L > sink ? L - sink : 0;
  const int64_t t_begin64 = static_cast<int64_t>(split) * chunk;
  const uint32_t t_begin = static_cast<uint32_t>(t_begin64 < comp ? t_begin64 : comp);
  const uint32_t t_end = static_cast<uint32_t>(t_begin64 + chunk < comp ? t_begin64 + chunk : comp);
  if (t_begin >= t_end) {
    // no compressed token falls in this split (a shorter sequence of a
    // ragged batch): an empty partial, m = -inf, l = 0, acc = 0
    for (int idx = threadIdx.x; idx < G * PART; idx += ST) {
      const int g = idx / PART, c = idx % PART;
      parts[((static_cast<int64_t>(b) * hq + static_cast<int64_t>(kh) * G + g) * n_slot + split) * PART + c] =
          c == 0 ? -INFINITY : 0.0f;
    }
    sink_part();
    finish();
    return;
  }

  // stream descriptors ending at the split's last token (for the value
  // tiles, at the end of its tile): the loads of tiles past a wave's last one
  // read zeros without touching memory, and so do a partial tile's tokens
  // past the end
  StreamRsrc rs;
  const int64_t vend = (static_cast<int64_t>(t_end) + TILE - 1) / TILE * TILE;
  // (paged cache: the stream arguments then address the page pool, and each
  // tile gets descriptors over its own page below)
  rs.kc = rsrc(kcodes + stream * kcap * KBYTES, static_cast<int64_t>(t_end) * KBYTES);
  rs.vc = rsrc(vcodes + stream * vcap * VBYTES, vend * VBYTES);
  // norms: NB bytes each (fp32, or fp16 bits)
  constexpr int NB = NF16 ? 2 : 4;
  const uint8_t* knb = reinterpret_cast<const uint8_t*>(knorms);
  const uint8_t* vnb = reinterpret_cast<const uint8_t*>(vnorms);
  rs.kn = rsrc(knb + stream * kcap * NB, static_cast<int64_t>(t_end) * NB);
  rs.vn = rsrc(vnb + stream * vcap * NB, static_cast<int64_t>(t_end) * NB);
  if constexpr (QJL) {
    rs.zs = rsrc(ksigns + stream * kcap * (QJL_M / 8), static_cast<int64_t>(t_end) * (QJL_M / 8));
    rs.rn = rsrc(krn + stream * kcap, static_cast<int64_t>(t_end) * 4);
  } else {
    rs.zs = rs.rn = rs.kn;
  }
  LaneOffsets lo;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const uint32_t tok = 8 * (n >> 2) + 4 * mb + (n & 3);
    if constexpr (KLO != KHI) {
      // mixed widths: lane j takes codes [16 j, 16 j + 16) of each width
      const uint32_t olo = 2 * KLO * j, ohi = 8 * KLO + 2 * KHI * j;
      lo.k[mb] = tok * KBYTES + (olo & ~3u);
      lo.k2[mb] = tok * KBYTES + (ohi & ~3u);
      lo.ksh[0] = 8 * (olo & 3u);
      lo.ksh[1] = 8 * (ohi & 3u);
    } else {
      lo.k[mb] = tok * KBYTES + (j < 2 ? 4 * KLO * j : 8 * KLO + 4 * KHI * (j - 2));
    }
    lo.z[mb] = tok * (QJL_M / 8) + 4 * j;
  }
  if constexpr (VLO != VHI) {
    // mixed widths: lane n takes rows 4 (n & 1) .. +3 of sub-block n / 2 of
    // each width, i.e. coordinates 4n .. 4n+3 and 64 + 4n .. 64 + 4n+3
    lo.v = j * (64 * (VLO + VHI)) + 8 * VLO * (n >> 1) + 4 * VLO * (n & 1);
    lo.v2 = j * (64 * (VLO + VHI)) + 64 * VLO + 8 * VHI * (n >> 1) + 4 * VHI * (n & 1);
  } else {
    lo.v = j * (64 * (VLO + VHI)) + (n < 8 ? 8 * VLO * n : 64 * VLO + 8 * VHI * (n - 8));
  }
  lo.nrm = 32 * j;
  lo.tokc = 8 * (n >> 2) + 4 * (j & 1) + (n & 3);

  // Tiles of this wave: first + STEP k, k < nt; the first nfull are whole.
  constexpr uint32_t STEP = 32 * SW;
  const uint32_t first = t_begin + 32 * wave;
  const int nt = __builtin_amdgcn_readfirstlane(first < t_end ? static_cast<int>((t_end - first + STEP - 1) / STEP) : 0);
  const int nfull =
      __builtin_amdgcn_readfirstlane(first + 32 <= t_end ? static_cast<int>((t_end - first - 32) / STEP + 1) : 0);

  // Paged cache: compressed token c of the sequence lives at slot c % 64 of
  // pool page block_table[b][c / 64] (pool stream page * hkv + kh).  A wave's
  // tiles are STEP = 256 tokens apart, each inside one page; lane L holds the
  // page of the wave's tile L (pid[0]) and L + 64 (pid[1]), -1 past the table.
  int pid[2] = {-1, -1};
  if constexpr (PAGED) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const uint32_t lp = (first + STEP * static_cast<uint32_t>(lane + 64 * h2)) / TQ_PAGE_TOKENS;
      if (first + STEP * static_cast<uint32_t>(lane + 64 * h2) < t_end && lp < static_cast<uint32_t>(max_pages))
        pid[h2] = block_table[static_cast<int64_t>(b) * max_pages + lp];
    }
  }
  // loads of the wave's tile k (first token t0): on a paged cache through
  // descriptors over the tile's page, bounded by the split's end; a page id
  // outside the pool reads zeros
  using TRg = TileRegs<key_dwords<KLO, KHI>()>;
  auto load_at = [&](TRg& buf, int k, uint32_t t0) __attribute__((always_inline)) {
    if constexpr (!PAGED) {
      load_tile<KLO, KHI, VLO, VHI, QJL, NF16, CG>(buf, t0, rs, lo);
    } else {
      const int pg = __builtin_amdgcn_readlane(k < 64 ? pid[0] : pid[1], k & 63);
      const int64_t base = static_cast<int64_t>(t0 / TQ_PAGE_TOKENS) * TQ_PAGE_TOKENS;
      int64_t nk = static_cast<int64_t>(t_end) - base, nvt = vend - base;
      nk = nk < 0 ? 0 : nk > TQ_PAGE_TOKENS ? TQ_PAGE_TOKENS : nk;
      nvt = nvt < 0 ? 0 : nvt > TQ_PAGE_TOKENS ? TQ_PAGE_TOKENS : nvt;
      const bool ok = pg >= 0 && pg < n_pages;
      if (!ok) nk = nvt = 0;
      const int64_t ps = static_cast<int64_t>(ok ? pg : 0) * hkv + kh;
      StreamRsrc pr;
      pr.kc = rsrc(kcodes + ps * kcap * KBYTES, nk * KBYTES);
      pr.vc = rsrc(vcodes + ps * vcap * VBYTES, nvt * VBYTES);
      pr.kn = rsrc(knb + ps * kcap * NB, nk * NB);
      pr.vn = rsrc(vnb + ps * vcap * NB, nk * NB);
      if constexpr (QJL) {
        pr.zs = rsrc(ksigns + ps * kcap * (QJL_M / 8), nk * (QJL_M / 8));
        pr.rn = rsrc(krn + ps * kcap, nk * 4);
      } else {
        pr.zs = pr.rn = pr.kn;
      }
      load_tile<KLO, KHI, VLO, VHI, QJL, NF16, CG>(buf, t0 % TQ_PAGE_TOKENS, pr, lo);
    }
  };

  TRg bufA, bufB;
  TRg bufC, bufD;  // CG: the second pair of tiles in flight
  load_at(bufA, 0, first);
  load_at(bufB, 1, first + STEP);
  if constexpr (CG) {
    load_at(bufC, 2, first + 2 * STEP);
    load_at(bufD, 3, first + 3 * STEP);
  }

  // Power-of-two scale per head for the fp16 operand: Pi is orthogonal, so
  // |q~_i| <= ||q~|| = ||q|| |qscale|, and sh = 14 - exponent of that bound
  // keeps |q~_i| 2^sh below 2^14.  Head g = tid / 32 sums its squares over
  // its 32 lanes.  (The sketch product u has no such bound; its scale comes
  // from its maximum.)
  {
    const float ss = sum32(fmaf(qv.x, qv.x, fmaf(qv.y, qv.y, fmaf(qv.z, qv.z, qv.w * qv.w))));
    if ((tid & 31) == 0 && tid < G * 32) {
      int ex = 0;
      const float nq = sqrtf(ss) * fabsf(qscale);
      if (nq > 0.0f) frexpf(nq, &ex);
      shx[tid >> 5] = 14 - ex;
    }
  }
  if (tid < G * (D / 4)) reinterpret_cast<float4*>(qraw)[tid] = qv;
  lut_store(std::integral_constant<int, 8>{}, l8l, l8h);
  lut_store(std::integral_constant<int, 4>{}, l4l, l4h);
  lut_store(std::integral_constant<int, 3>{}, l3l, l3h);
  lut_store(std::integral_constant<int, 2>{}, l2l, l2h);
  if (threadIdx.x < 4)
    lutz[threadIdx.x] = ((threadIdx.x & 1) ? 0x3C00u : 0xBC00u) | (((threadIdx.x >> 1) & 1) ? 0x3C000000u : 0xBC000000u);
  // row G of every fragment array is the zero row of the padding heads
  if (tid < NSET * 2 * (FROW / 8))
    reinterpret_cast<uint4*>(frag_row(tid / (2 * (FROW / 8)), (tid / (FROW / 8)) & 1, G))[tid % (FROW / 8)] = uint4{};
  if (QJL && tid < GMAX) umax[tid] = 0u;
  __syncthreads();

  auto partial_dots = [&](const float (&m)[32], const float* src) {
    for (int g = 0; g < G; ++g) {
      const float4* v4 = reinterpret_cast<const float4*>(src + g * D + 32 * kq);
      float a = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float4 x = v4[k];
        a = fmaf(m[4 * k], x.x, a);
        a = fmaf(m[4 * k + 1], x.y, a);
        a = fmaf(m[4 * k + 2], x.z, a);
        a = fmaf(m[4 * k + 3], x.w, a);
      }
      ppart[(kq * GMAX + g) * D + pi_i] = a;
    }
  };
  auto reduce_part = [&](int g, int i) {
    return ((ppart[(0 * GMAX + g) * D + i] + ppart[(1 * GMAX + g) * D + i]) + ppart[(2 * GMAX + g) * D + i]) +
           ppart[(3 * GMAX + g) * D + i];
  };
  // x 2^sh split into fp16 hi + lo, stored as coordinate i of head g
  auto store_split = [&](int set, int g, int i, float x, int sh) {
    const float xs = ldexpf(x, sh);
    const _Float16 h = static_cast<_Float16>(xs);
    frag_row(set, 0, g)[i] = h;
    frag_row(set, 1, g)[i] = static_cast<_Float16>(xs - static_cast<float>(h));
  };
  partial_dots(w, qraw);
  if constexpr (QJL) {
#pragma unroll
    for (int k = 0; k < 32; ++k) w[k] = ktab->sit[(32 * kq + k) * D + pi_i];
  }
  __syncthreads();
  // q~ = scale * log2(e) * Pi q, one coordinate per thread and pass
  constexpr int PER = GMAX * D / ST;
  float uv[QJL ? PER : 1];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int idx = tid + r * ST;
    if (idx < G * D) {
      const int g = idx >> 7, i = idx & (D - 1);
      const float x = reduce_part(g, i) * qscale;
      // the key lookup tables hold centroids times the codebook's scale
      store_split(0, g, i, x / ktab->cen16_scale[i < static_cast<int>(ktab->split) ? 0 : 1], shx[g]);
      if constexpr (QJL) qrot[idx] = x;
    }
  }
  if constexpr (QJL) {
    // u = S q~ and its per-head maximum (the bits of a non-negative float
    // order like the float)
    __syncthreads();
    partial_dots(w, qrot);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int idx = tid + r * ST;
      uv[r] = 0.0f;
      if (idx < G * D) {
        uv[r] = reduce_part(idx >> 7, idx & (D - 1));
        atomicMax(&umax[idx >> 7], __float_as_uint(fabsf(uv[r])));
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int idx = tid + r * ST;
      if (idx < G * D) {
        const int g = idx >> 7;
        int ex = 0;
        const float mx = __uint_as_float(umax[g]);
        if (mx > 0.0f) frexpf(mx, &ex);
        store_split(1, g, idx & (D - 1), uv[r], 14 - ex);
        if ((idx & (D - 1)) == 0) shx[GMAX + g] = 14 - ex;
      }
    }
  }
  __syncthreads();
  // A-operand fragments: lane (n, j) holds coordinates 32 j + 8 ks + e of
  // query head n of the group (row G, zero, for padding heads)
  const bool head_ok = n < G;
  const int frow = head_ok ? n : G;
  // Without the sketch the query fragments live in registers; with it the
  // registers go to the sign and residual-norm tiles, and all four fragment
  // sets are read from LDS per tile instead.
  half8 qh[QJL ? 1 : 4], ql[QJL ? 1 : 4];
  // k-slot (lane j, step ks) of the score MFMA -> first of its 8 rotated
  // coordinates: with mixed key widths steps 0, 1 take the KLO coordinates
  // 16 j .. 16 j + 15 and steps 2, 3 the KHI ones 64 + 16 j .. (the sketch
  // sets are indexed by rows of S: 32 j + 8 ks)
  auto kcoord = [&](int ks) { return KLO != KHI ? (ks < 2 ? 16 * j + 8 * ks : 64 + 16 * j + 8 * (ks - 2)) : 32 * j + 8 * ks; };
  const _Float16* fbase[4] = {frag_row(0, 0, frow), frag_row(0, 1, frow), frag_row(QJL ? 1 : 0, 0, frow) + 32 * j,
                              frag_row(QJL ? 1 : 0, 1, frow) + 32 * j};
  if constexpr (!QJL) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qh[ks] = *reinterpret_cast<const half8*>(fbase[0] + kcoord(ks));
      ql[ks] = *reinterpret_cast<const half8*>(fbase[1] + kcoord(ks));
    }
  }
  auto frag_at = [&](int set, int ks) -> half8 {
    if constexpr (!QJL) return set == 0 ? qh[ks] : ql[ks];
    else return *reinterpret_cast<const half8*>(fbase[set] + (set < 2 ? kcoord(ks) : 8 * ks));
  };
  // column n of P V block nb -> rotated value coordinate (mixed value widths:
  // blocks 0..3 from the VLO sub-blocks, 4..7 from the VHI ones)
  auto vcoord = [&](int nn, int nb) { return VLO != VHI ? (nb < 4 ? 4 * nn + nb : 64 + 4 * nn + nb - 4) : 8 * nn + nb; };
  const float qinv = head_ok ? ldexpf(1.0f, -shx[n]) : 0.0f;
  const float uinv = QJL && head_ok ? ldexpf(QJL_C, -shx[GMAX + n]) : 0.0f;

  const uint8_t* lut_klo = smem + LP::template off<KLO>();
  const uint8_t* lut_khi = smem + LP::template off<KHI>();
  const uint8_t* lut_vlo = smem + LP::template off<VLO>();
  const uint8_t* lut_vhi = smem + LP::template off<VHI>();

  // Online softmax state per query head (replicated over its 4 token lanes).
  // The running maximum is kept lazily: it only moves when a score exceeds it
  // by more than RESCALE_SLACK, so probabilities stay below 2^0.5 and most
  // tiles skip the accumulator rescale.
  constexpr float RESCALE_SLACK = 0.5f;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{};

  // Score products of one tile: sk[mb] the codebook part (hi and lo query
  // parts accumulate into one chain), sz[mb] the sketch sign products.
  // SWAP: the query fragments are the A operand, so lane (n, j) of M-block mb
  // holds heads 4 j + i of the block's token row n (instead of tokens
  // 8 j + 4 mb + i of head n).
  auto score_tile = [&]<bool SWAP>(const TRg& tr, f32x4 (&sk)[2], f32x4 (&sz)[2]) __attribute__((always_inline)) {
    // keeps the LDS fragment reads of the sketch variant inside the loop
    if constexpr (QJL) __asm__ volatile("" ::: "memory");
    auto mm = [&](half8 x, half8 qf, f32x4 c) { return SWAP ? mfma16(qf, x, c) : mfma16(x, qf, c); };
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) sk[mb] = sz[mb] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      half8 a[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if constexpr (KLO == KHI) {
          a[mb] = dequant8<KLO>(tr.kw[mb], ks, lut_klo, lane4);
        } else {
          // k-steps 0, 1: width KLO; 2, 3: width KHI (no divergence)
          uint32_t wk[2];
          const int part = ks >> 1;
          const uint32_t sh = lo.ksh[part];
          const bool aligned = part == 0 ? (2 * KLO) % 4 == 0 : (2 * KHI) % 4 == 0;
          if (aligned) {
            wk[0] = tr.kw[mb][2 * part];
            wk[1] = tr.kw[mb][2 * part + 1];
          } else {
            wk[0] = __builtin_amdgcn_alignbit(tr.kw[mb][2 * part + 1], tr.kw[mb][2 * part], sh);
            wk[1] = tr.kw[mb][2 * part + 1] >> sh;
          }
          a[mb] = part == 0 ? dequant8<KLO>(wk, ks & 1, lut_klo, lane4) : dequant8<KHI>(wk, ks & 1, lut_khi, lane4);
        }
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) sk[mb] = mm(a[mb], frag_at(0, ks), sk[mb]);
      if constexpr (QJL) {
        half8 z[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const uint32_t zv = (tr.zw[mb] >> (8 * ks)) & 0xFFu;
          z[mb] = as_half8(lutz[zv & 3], lutz[(zv >> 2) & 3], lutz[(zv >> 4) & 3], lutz[zv >> 6]);
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sz[mb] = mm(z[mb], frag_at(2, ks), sz[mb]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sk[mb] = mm(a[mb], frag_at(1, ks), sk[mb]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sz[mb] = mm(z[mb], frag_at(3, ks), sz[mb]);
      } else {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sk[mb] = mm(a[mb], frag_at(1, ks), sk[mb]);
      }
    }
  };

  // P V of one tile: pa is this lane's A operand (row n = head n, tokens
  // 8 j .. 8 j + 7), the value sub-blocks through the LUT the B operands.
  auto pv_tile = [&](const TRg& tr, half8 pa) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      half8 bv;
      if constexpr (VLO == VHI) bv = dequant8<VLO>(tr.vw, nb, lut_vlo, lane4);
      else bv = nb < 4 ? dequant8<VLO>(tr.vw, nb, lut_vlo, lane4) : dequant8<VHI>(tr.vw + 4, nb - 4, lut_vhi, lane4);
      acc[nb] = mfma16(pa, bv, acc[nb]);
    }
  };

  auto tile_step = [&]<bool FULL, bool VSKIP>(const TRg& tr, uint32_t t0c) __attribute__((always_inline)) {
    const int nvalid = FULL ? 8 : static_cast<int>(t_end) - static_cast<int>(t0c + 8 * j);
    f32x4 sk[2], sz[2];
    score_tile.template operator()<false>(tr, sk, sz);
    float s[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * mb + i;
        float dot = sk[mb][i] * qinv;
        if constexpr (QJL) dot = fmaf(f4get(tr.rn, e) * sz[mb][i], uinv, dot);
        s[e] = norm_get<NF16>(tr.kn, e) * dot;
        if constexpr (!FULL) s[e] = e < nvalid ? s[e] : -INFINITY;
        tmax = fmaxf(tmax, s[e]);
      }
    tmax = max_xor16_32(tmax);
    // rescale only when some head's maximum grew past the slack
    if (__any(tmax > m_run + RESCALE_SLACK)) {
      const float m_new = tmax > m_run + RESCALE_SLACK ? tmax : m_run;
      const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * j + i);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k][i] *= ai;
      }
    }
    float psum = 0.0f;
    uint32_t pw[4];
    bool any = !VSKIP;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float p0 = __builtin_amdgcn_exp2f(s[e] - m_run), p1 = __builtin_amdgcn_exp2f(s[e + 1] - m_run);
      if constexpr (VSKIP) {
        if (p0 < v_skip) p0 = 0.0f;
        if (p1 < v_skip) p1 = 0.0f;
        any |= (p0 > 0.0f) | (p1 > 0.0f);
      }
      psum += p0 + p1;
      float v0 = norm_get<NF16>(tr.vn, e), v1 = norm_get<NF16>(tr.vn, e + 1);
      if constexpr (!FULL) {
        v0 = e < nvalid ? v0 : 0.0f;
        v1 = e + 1 < nvalid ? v1 : 0.0f;
      }
      const half2v h = {static_cast<_Float16>(p0 * v0), static_cast<_Float16>(p1 * v1)};
      pw[e >> 1] = __builtin_bit_cast(uint32_t, h);
    }
    l_run += psum;
    // skip the value work of a tile whose weights all fell below v_skip
    if (!VSKIP || __any(any && head_ok)) pv_tile(tr, as_half8(pw[0], pw[1], pw[2], pw[3]));
  };

  // ---- compact softmax (CG): the state of head i < 4 of the group sits in
  // component i, the same value in every lane for the maximum (mc); the sums
  // (lc) are per-lane partials, added up after the stream.
  float mc[4], lc[4], qinvc[4], uinvc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mc[i] = -INFINITY;
    lc[i] = 0.0f;
    qinvc[i] = CG && i < G ? ldexpf(1.0f, -shx[i]) : 0.0f;
    uinvc[i] = CG && QJL && i < G ? ldexpf(QJL_C, -shx[GMAX + i]) : 0.0f;
  }
  // per-wave P array: [tile of the pair][head row (16; rows >= G stay zero)][32 tokens + pad]
  constexpr int PWROW = 40;
  _Float16* pwl = reinterpret_cast<_Float16*>(smem + PRO_OFF + GMAX * D * 4) + wave * (2 * 16 * PWROW);
  if constexpr (CG) {
    static_assert(SW * 2 * 16 * PWROW * 2 <= 4 * GMAX * D * 4, "P arrays fit the prologue's partial-dot area");
    // the prologue's partial dots are dead: zero this wave's P array
    uint4* z4 = reinterpret_cast<uint4*>(pwl);
    for (int c = lane; c < 2 * 16 * PWROW * 2 / 16; c += 64) z4[c] = uint4{};
  }
  // Two tiles (A at token t0a, B at t0b) through the compact softmax.  Lane
  // (n, j) takes token lo.tokc of tile A (j < 2) or B (j >= 2), all heads.
  auto pair_step = [&]<bool FULL, bool VSKIP>(const TRg& ta_, uint32_t t0a, const TRg& tb_, uint32_t t0b)
                       __attribute__((always_inline)) {
    f32x4 ska[2], sza[2], skb[2], szb[2];
    score_tile.template operator()<true>(ta_, ska, sza);
    score_tile.template operator()<true>(tb_, skb, szb);
    const bool in_b = j >= 2;
    const uint32_t t0 = in_b ? t0b : t0a;
    const bool valid = FULL || t0 + lo.tokc < t_end;
    auto nval = [&](float a, float bb) {
      const float x = in_b ? bb : a;
      if constexpr (NF16) return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(__float_as_uint(x))));
      else return x;
    };
    const float kn = nval(ta_.kn[0].x, tb_.kn[0].x);
    const float vn = valid ? nval(ta_.vn[0].x, tb_.vn[0].x) : 0.0f;
    const float rn = QJL ? (in_b ? tb_.rn[0].x : ta_.rn[0].x) : 0.0f;
    float sc[4];
    bool up = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float dot = gather_rows0(ska[0][i], ska[1][i], skb[0][i], skb[1][i]) * qinvc[i];
      if constexpr (QJL) dot = fmaf(rn * gather_rows0(sza[0][i], sza[1][i], szb[0][i], szb[1][i]), uinvc[i], dot);
      sc[i] = valid && i < G ? kn * dot : -INFINITY;
      up |= sc[i] > mc[i] + RESCALE_SLACK;
    }
    // rescale only when some head's maximum grew past the slack
    if (__any(up)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mx = wave_max(sc[i]);
        const float mn = mx > mc[i] + RESCALE_SLACK ? mx : mc[i];
        const float al = mc[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mc[i] - mn);
        mc[i] = mn;
        lc[i] *= al;
        // acc row 4 j + i: head i in the first row, padding heads (zero) elsewhere
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k][i] *= al;
      }
    }
    bool any = !VSKIP;
    _Float16* prow = pwl + (in_b ? 16 * PWROW : 0) + lo.tokc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float p = sc[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[i] - mc[i]);
      if constexpr (VSKIP) {
        if (p < v_skip) p = 0.0f;
        any |= p > 0.0f;
      }
      lc[i] += p;
      if (i < G) prow[i * PWROW] = static_cast<_Float16>(p * vn);
    }
    bool any_a = true, any_b = true;
    if constexpr (VSKIP) {
      any_a = __any(any && !in_b);
      any_b = __any(any && in_b);
    }
    // the P array is this wave's own: its writes precede its reads in order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const half8 pa = *reinterpret_cast<const half8*>(pwl + n * PWROW + 8 * j);
    const half8 pb = *reinterpret_cast<const half8*>(pwl + (16 + n) * PWROW + 8 * j);
    if (any_a) pv_tile(ta_, pa);
    if (any_b) pv_tile(tb_, pb);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Two tiles in flight per wave in fixed registers: each buffer is refilled
  // with the tile after next as soon as its tile has been consumed.  The
  // loop body is straight-line, so the outstanding loads at every use are
  // exactly the other buffer's.
  auto stream_tiles = [&]<bool VSKIP>() __attribute__((always_inline)) {
    int k = 0;
    for (; k + 2 <= nfull; k += 2) {
      const uint32_t ta = first + STEP * k;
      tile_step.template operator()<true, VSKIP>(bufA, ta);
      load_at(bufA, k + 2, ta + 2 * STEP);
      tile_step.template operator()<true, VSKIP>(bufB, ta + STEP);
      load_at(bufB, k + 3, ta + 3 * STEP);
    }
    // at most one whole tile and one partial tile remain
    const uint32_t ta = first + STEP * k;
    if (k < nfull) {
      tile_step.template operator()<true, VSKIP>(bufA, ta);
      if (k + 1 < nt) tile_step.template operator()<false, VSKIP>(bufB, ta + STEP);
    } else if (k < nt) {
      tile_step.template operator()<false, VSKIP>(bufA, ta);
    }
  };
  // CG: two pairs of tiles in flight (buffers A, B and C, D), each pair
  // refilled with the pair after next once it has been consumed.
  auto stream_pairs = [&]<bool VSKIP>() __attribute__((always_inline)) {
    int k = 0;
    for (; k + 4 <= nfull; k += 4) {
      const uint32_t ta = first + STEP * k;
      pair_step.template operator()<true, VSKIP>(bufA, ta, bufB, ta + STEP);
      load_at(bufA, k + 4, ta + 4 * STEP);
      load_at(bufB, k + 5, ta + 5 * STEP);
      pair_step.template operator()<true, VSKIP>(bufC, ta + 2 * STEP, bufD, ta + 3 * STEP);
      load_at(bufC, k + 6, ta + 6 * STEP);
      load_at(bufD, k + 7, ta + 7 * STEP);
    }
    // at most three whole tiles and a partial one remain; tokens past the
    // split's end (and tiles past the wave's last) are masked out
    const uint32_t ta = first + STEP * k;
    if (k < nt) pair_step.template operator()<false, VSKIP>(bufA, ta, bufB, ta + STEP);
    if (k + 2 < nt) pair_step.template operator()<false, VSKIP>(bufC, ta + 2 * STEP, bufD, ta + 3 * STEP);
  };
  if constexpr (CG) {
    if (v_skip > 0.0f) stream_pairs.template operator()<true>();
    else stream_pairs.template operator()<false>();
  } else {
    if (v_skip > 0.0f) stream_tiles.template operator()<true>();
    else stream_tiles.template operator()<false>();
  }

  // ---- merge the waves; l: sum over the 4 token lanes of a head (CG: over
  // all lanes, head i from component i).
  if constexpr (CG) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lc[i] = wave_sum(lc[i]);
      if (lane == i) {
        m_run = mc[i];
        l_run = lc[i];
      }
    }
  } else {
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
  }
  __syncthreads();  // LUTs are dead from here on: reuse their space
  float* mrg_m = reinterpret_cast<float*>(smem);           // [SW][16]
  float* mrg_l = mrg_m + SW * 16;                           // [SW][16]
  float* mrg_acc = mrg_l + SW * 16;                         // [SW][16][D]
  if (lane < 16) {
    mrg_m[wave * 16 + lane] = m_run;
    mrg_l[wave * 16 + lane] = l_run;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (4 * j + i < G)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) mrg_acc[(wave * 16 + 4 * j + i) * D + vcoord(n, nb)] = acc[nb][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += ST) {
    const int g = idx / D, c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < SW; ++w) M = fmaxf(M, mrg_m[w * 16 + g]);
    float a = 0.0f, l = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < SW; ++w) {
        const float mw = mrg_m[w * 16 + g];
        const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        a = fmaf(f, mrg_acc[(w * 16 + g) * D + c], a);
        l = fmaf(f, mrg_l[w * 16 + g], l);
      }
    }
    float* part = parts + ((static_cast<int64_t>(b) * hq + static_cast<int64_t>(kh) * G + g) * n_slot + split) * PART;
    part[4 + c] = a;
    if (c == 0) {
      part[0] = M;
      part[1] = l;
    }
  }
  sink_part();
  finish();
}

template <int KLO, int KHI, int VLO, int VHI, bool QJL, bool PAGED, bool NF16, bool CG>
hipError_t launch_split_cg(const SplitArgs& f) {
  const tq_attn& a = *f.a;
  const AttendPlan& plan = *f.plan;
  const tq_cache &kc = *f.kc, &vc = *f.vc;
  const dim3 grid(a.hkv, a.batch, plan.n_split);
  hipLaunchKernelGGL((split_kernel<KLO, KHI, VLO, VHI, QJL, PAGED, NF16, CG>), grid, dim3(ST), 0, f.st, f.ktab, kc.codes,
                     kc.norms, kc.qjl_signs, kc.qjl_rnorms, kc.cap, f.vtab, vc.codes, vc.norms, vc.cap, f.seq_lens,
                     f.q, f.sink_k, f.sink_v, f.parts, f.out, a.hq, a.hkv, a.sink, plan.n_split, plan.n_slot,
                     plan.chunk, a.v_skip, a.scale * LOG2E, f.block_table, PAGED ? f.max_pages : 0,
                     PAGED ? f.n_pages : 0, static_cast<int>(a.max_len));
  return hipGetLastError();
}

// Groups of at most 4 query heads take the compact softmax when every
// stream is a single split (a batch of 256 or more streams): each wave then
// streams its stream's whole length, and the compact step pays for its fixed
// costs.  (With many short splits per stream it measured slower: the
// gqa_decode shape 19.2 -> 21.7 us, long_context 40.7 -> 42.9 us; the
// batched ragged workload 265 -> 253 us.)
template <int KLO, int KHI, int VLO, int VHI, bool QJL, bool PAGED, bool NF16>
hipError_t launch_split_as(const SplitArgs& f) {
  return f.a->hq / f.a->hkv <= 4 && f.plan->n_split == 1
             ? launch_split_cg<KLO, KHI, VLO, VHI, QJL, PAGED, NF16, true>(f)
             : launch_split_cg<KLO, KHI, VLO, VHI, QJL, PAGED, NF16, false>(f);
}

template <int KLO, int KHI, int VLO, int VHI, bool QJL>
hipError_t launch_split(const SplitArgs& f) {
  if (f.norm16)
    return f.block_table ? launch_split_as<KLO, KHI, VLO, VHI, QJL, true, true>(f)
                         : launch_split_as<KLO, KHI, VLO, VHI, QJL, false, true>(f);
  return f.block_table ? launch_split_as<KLO, KHI, VLO, VHI, QJL, true, false>(f)
                       : launch_split_as<KLO, KHI, VLO, VHI, QJL, false, false>(f);
}


template <int KLO, int KHI, int VLO, int VHI>
hipError_t launch_q(bool qjl, const SplitArgs& f) {
  return qjl ? launch_split<KLO, KHI, VLO, VHI, true>(f) : launch_split<KLO, KHI, VLO, VHI, false>(f);
}

template <int KLO, int KHI>
hipError_t dispatch_v(int vkey, bool qjl, const SplitArgs& f) {
  switch (vkey) {
    case 22: return launch_q<KLO, KHI, 2, 2>(qjl, f);
    case 33: return launch_q<KLO, KHI, 3, 3>(qjl, f);
    case 44: return launch_q<KLO, KHI, 4, 4>(qjl, f);
    case 43: return launch_q<KLO, KHI, 4, 3>(qjl, f);
    case 32: return launch_q<KLO, KHI, 3, 2>(qjl, f);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace tq
