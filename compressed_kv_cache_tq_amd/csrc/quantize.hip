// Quantize kernel: norm -> rotation (MFMA) -> Lloyd-Max scalar codes -> bit
// packing [-> QJL sign sketch of the residual].
//
// noze.it, "TurboQuant-MLX: quantizzare pesi e KV cache per LLM open-weight su
// Mac", section "Il metodo TurboQuant, in breve": rotate at random, quantize
// each coordinate with the optimal scalar quantizer for the known
// post-rotation law, optionally keep a 1-bit JL sketch of the residual.
//
// One wave owns a tile of 32 vectors; a workgroup of 8 waves shares the
// rotation fragments in LDS.  The rotation is the dense contraction
// Y = X Pi^T on v_mfma_f32_32x32x16:
//  * bf16 inputs (no QJL stage): x is fed to the bf16 MFMA as stored and Pi
//    is split into three bf16 parts (hi + mid + lo, ~24 bits) accumulated in
//    one fp32 accumulator;
//  * fp32 inputs, and the QJL variant: x is scaled by a power of two per
//    vector and split into fp16 hi (+ lo for fp32), 256*Pi into fp16 hi + lo.
// Either way the rotated coordinate is within ~1e-7 of its float64 value.
//
// Record layout (keys): Pi is the A operand (rows = output coordinates), X^T
// the B operand; the row permutation makes lane (n, h) hold coordinates
// 64h .. 64h+63 of vector n, so its half record is built in registers.
// Tiled layout (values): X is the A operand (rows = tokens), Pi^T the B
// operand; lane (j, h) then holds coordinates 4j .. 4j+3 of tokens 16h ..
// 16h+15, the rows of two 8-token sub-blocks.
//
// Scalar codes are found as bit planes: for each coordinate register the
// wave compares |y| with the positive thresholds (one v_cmp each, a lane
// mask per threshold); because the masks are nested, bit k of the count is
// the xor of the masks j with 2^k | (j+1), done on the scalar unit; the sign
// turns count into code.  Each code bit is appended to the packed word with
// one v_addc (w = 2w + bit), most significant bit first.
#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WAVES = 8;
constexpr int THREADS = 64 * WAVES;
constexpr int FRAGS = 4 * 8 * 64;  // (tile, k-step, lane) fragments of one 128x128 16-bit matrix part

// input modes
constexpr int X_BF16 = 0;      // bf16 x, bf16 MFMA, Pi in 3 bf16 parts
constexpr int X_BF16_F16 = 1;  // bf16 x converted exactly to fp16, Pi in 2 fp16 parts
constexpr int X_F32 = 2;       // fp32 x split into fp16 hi + lo, Pi in 2 fp16 parts

__device__ __forceinline__ half8 as_half8(uint4 v) { return __builtin_bit_cast(half8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x16 mfma(half8 a, half8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// Element k (0..63) of this lane's half vector held as raw 16-byte words.
template <bool F32IN, int N>
__device__ __forceinline__ float elem(const uint4 (&xr)[N], int k) {
  if constexpr (F32IN) return __uint_as_float(word_of(xr[k >> 2], k & 3));
  const uint32_t w = word_of(xr[k >> 3], (k >> 1) & 3);
  return __uint_as_float((k & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// w = 2w + (bit of this lane in mask): appends one code bit.
__device__ __forceinline__ uint32_t append_bit(uint32_t w, uint64_t mask) {
  uint32_t r;
  uint64_t carry_out;
  asm("v_addc_co_u32 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(w), "s"(mask));
  return r;
}

// Output coordinate (record layout) held in accumulator register r of
// M-tile t by lanes of half h is 64h + 16t + r; this is the Pi row that A row
// i of M-tile t must carry.
__device__ __forceinline__ int record_row(int t, int i) {
  return 64 * ((i >> 2) & 1) + 16 * t + 4 * (i >> 3) + (i & 3);
}

// Tiled layout: A row i carries token slot tau(i) so that lanes of half h hold
// tokens 16h + r in register r.
__device__ __forceinline__ int tiled_slot(int i) {
  return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}

template <int B>
struct Width {
  static constexpr int L = 1 << B;
  static constexpr int HALF = L / 2;
  static constexpr int NPOS = HALF - 1;  // positive thresholds
};

template <int B>
__device__ __forceinline__ void load_pos_thresholds(const Tables* tab, int half, float scale, float* tp) {
#pragma unroll
  for (int k = 0; k < Width<B>::NPOS; ++k) tp[k] = tab->bnd[half][Width<B>::HALF + k] * scale;
}

// Bit planes of the code of value v (same scale as the thresholds tp) as lane
// masks: plane[k] = lanes whose code has bit k set.  code = #{t_j < v}; the
// codebook is symmetric with a 0 threshold, v <= 0 counts on the negative side.
template <int B>
__device__ __forceinline__ void code_planes(float v, const float* tp, uint64_t (&plane)[4]) {
  const float a = fabsf(v);
  uint64_t m[Width<B>::NPOS > 0 ? Width<B>::NPOS : 1];
#pragma unroll
  for (int k = 0; k < Width<B>::NPOS; ++k) m[k] = __builtin_amdgcn_ballot_w64(a > tp[k]);
  const uint64_t S = __builtin_amdgcn_ballot_w64(v > 0.0f);
#pragma unroll
  for (int k = 0; k < B - 1; ++k) {
    uint64_t c = 0;
#pragma unroll
    for (int j = 0; j < Width<B>::NPOS; ++j)
      if (((j + 1) & ((1 << k) - 1)) == 0) c ^= m[j];
    plane[k] = ~(c ^ S);  // count bit for v > 0, its complement otherwise
  }
  plane[B - 1] = S;
}

// Scalar code (used by the QJL variant, which also needs the centroid).
template <int B>
__device__ __forceinline__ uint32_t code_of(float v, const float* tp) {
  const float a = fabsf(v);
  uint32_t cnt = 0;
#pragma unroll
  for (int k = 0; k < Width<B>::NPOS; ++k) cnt += a > tp[k] ? 1u : 0u;
  return v > 0.0f ? Width<B>::HALF + cnt : Width<B>::HALF - 1 - cnt;
}

// Record layout: this lane's 64 consecutive coordinates (acc[t][r] is
// coordinate 16t + r of its half) packed LSB first into 2B words, built from
// the top bit down with one append per code bit.
template <int B>
__device__ __forceinline__ void pack_record(const f32x16 (&acc)[4], const float* tp, uint32_t (&w)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = 0;
#pragma unroll
  for (int c = 63; c >= 0; --c) {
    uint64_t pl[4];
    code_planes<B>(acc[c >> 4][c & 15], tp, pl);
#pragma unroll
    for (int k = B - 1; k >= 0; --k) {
      const int wd = (B * c + k) >> 5;
      w[wd] = append_bit(w[wd], pl[k]);
    }
  }
}

template <int B>
__device__ __forceinline__ void pack_record_scalar(const f32x16 (&acc)[4], const float* tp, uint32_t (&w)[8],
                                                   uint32_t (&idx)[64]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = 0;
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    const uint32_t q = code_of<B>(acc[c >> 4][c & 15], tp);
    idx[c] = q;
    const int bit = B * c, wd = bit >> 5, off = bit & 31;
    w[wd] |= q << off;
    if (off + B > 32) w[wd + 1] |= q >> (32 - off);
  }
}

template <int B>
__device__ __forceinline__ void store_record(uint8_t* dst, const uint32_t (&w)[8]) {
  uint2* p = reinterpret_cast<uint2*>(dst);
#pragma unroll
  for (int k = 0; k < B; ++k) p[k] = make_uint2(w[2 * k], w[2 * k + 1]);
}

// Tiled layout: this lane holds coordinates 4j + t (t = 0..3) of token slots
// 16h + r (r = 0..15).  For token group gg (slots 16h + 8gg + s) the chunk
// is rows t = 0..3 x tokens s = 0..7, code bits at (8t + s) B: B words.
template <int B>
__device__ __forceinline__ void pack_tiled(const f32x16 (&acc)[4], const float (&inv)[16], const float* tp, int gg,
                                           uint32_t (&w)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = 0;
#pragma unroll
  for (int t = 3; t >= 0; --t)
#pragma unroll
    for (int s = 7; s >= 0; --s) {
      const int r = 8 * gg + s;
      uint64_t pl[4];
      code_planes<B>(acc[t][r] * inv[r], tp, pl);
#pragma unroll
      for (int k = B - 1; k >= 0; --k) {
        const int wd = ((8 * t + s) * B + k) >> 5;
        w[wd] = append_bit(w[wd], pl[k]);
      }
    }
}

// Mask of the chunk bits that belong to token slots s with (valid >> s) & 1.
template <int B>
__device__ __forceinline__ void slot_mask(uint32_t valid, uint32_t (&m)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) m[k] = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (!((valid >> s) & 1)) continue;
      const uint32_t q = (1u << B) - 1;
      const int bit = (8 * t + s) * B, wd = bit >> 5, off = bit & 31;
      m[wd] |= q << off;
      if (off + B > 32) m[wd + 1] |= q >> (32 - off);
    }
}

template <int B>
__device__ __forceinline__ void store_tiled_chunk(uint8_t* dst, const uint32_t (&w)[4], uint32_t valid) {
  uint32_t* p = reinterpret_cast<uint32_t*>(dst);
  if (valid == 0xFFu) {
#pragma unroll
    for (int k = 0; k < B; ++k) p[k] = w[k];
  } else if (valid) {
    uint32_t m[4];
    slot_mask<B>(valid, m);
#pragma unroll
    for (int k = 0; k < B; ++k) p[k] = (p[k] & ~m[k]) | (w[k] & m[k]);
  }
}

template <int BLO, int BHI, int XM, bool TILED, bool QJL>
__global__ __launch_bounds__(THREADS, 1) void quantize_kernel(
    const Tables* __restrict__ tab, const void* __restrict__ xv, int64_t n_tok, int64_t xss, int64_t xrs,
    int64_t tok0, uint8_t* __restrict__ codes, float* __restrict__ norms, uint8_t* __restrict__ signs,
    float* __restrict__ rnorms, int64_t cap, int64_t stream_code_bytes, int64_t tiles_per_stream, int64_t tile0,
    int64_t total_tiles) {
  constexpr bool F32IN = XM == X_F32;
  constexpr int NPART = XM == X_BF16 ? 3 : 2;
  constexpr int CODE_BYTES = 8 * (BLO + BHI);
  __shared__ uint4 pi_frag[NPART * FRAGS];
  __shared__ uint4 s_frag[QJL ? 2 * FRAGS : 1];
  __shared__ float cen_s[2][16];

  // Stage the rotation (and sketch) fragments in LDS in the order the MFMA
  // loop reads them: fragment (part, t, ks, lane) = 8 consecutive columns
  // 64*(lane/32) + 8*ks of one matrix row.
  for (int c = threadIdx.x; c < NPART * FRAGS; c += THREADS) {
    const int part = c / FRAGS, t = (c >> 9) & 3, ks = (c >> 6) & 7, l = c & 63;
    const int row = TILED ? 4 * (l & 31) + t : record_row(t, l & 31);
    const int col = 64 * (l >> 5) + 8 * ks;
    const uint16_t* src = XM == X_BF16 ? tab->pi_b16[part] : (part ? tab->pi_lo : tab->pi_hi);
    pi_frag[c] = *reinterpret_cast<const uint4*>(src + row * D + col);
    if constexpr (QJL) {
      if (part < 2) {
        const int srow = record_row(t, l & 31);
        const uint16_t* ss = (part ? tab->s_lo : tab->s_hi) + srow * D + col;
        s_frag[c] = *reinterpret_cast<const uint4*>(ss);
      }
    }
  }
  if (threadIdx.x < 32) cen_s[threadIdx.x >> 4][threadIdx.x & 15] = tab->cen[threadIdx.x >> 4][threadIdx.x & 15];
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, h = lane >> 5;

  // Row of x this lane loads for tile w (vector column n for the record
  // layout, token slot tiled_slot(n) for the tiled layout).
  auto locate = [&](int64_t w, int64_t& s, int64_t& T, int64_t& row, int64_t& pos) {
    s = w / tiles_per_stream;
    T = w - s * tiles_per_stream;
    if constexpr (TILED) {
      pos = 32 * (tile0 + T) + tiled_slot(n);
      row = pos - tok0;
    } else {
      row = 32 * T + n;
      pos = tok0 + row;
    }
  };
  // this lane's 64 elements (its half of the vector) as raw words
  constexpr int NW = F32IN ? 16 : 8;
  auto load_x = [&](int64_t w, uint4 (&dst)[NW]) {
    int64_t s, T, row, pos;
    locate(w, s, T, row, pos);
    if (w < total_tiles && row >= 0 && row < n_tok) {
      const uint4* xp = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(xv) +
                                                       (s * xss + row * xrs + 64 * h) * (F32IN ? 4 : 2));
#pragma unroll
      for (int k = 0; k < NW; ++k) dst[k] = xp[k];
    } else {
#pragma unroll
      for (int k = 0; k < NW; ++k) dst[k] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  const int64_t stride = static_cast<int64_t>(gridDim.x) * WAVES;
  uint4 xr[NW];
  load_x(static_cast<int64_t>(blockIdx.x) * WAVES + wave, xr);

  for (int64_t w = static_cast<int64_t>(blockIdx.x) * WAVES + wave; w < total_tiles; w += stride) {
    int64_t s, T, row, pos;
    locate(w, s, T, row, pos);
    const bool valid = row >= 0 && row < n_tok;
    // next tile's input goes out now and lands while this tile is computed
    uint4 xnext[NW];
    load_x(w + stride, xnext);
    // ---- norm.  bf16: exact products summed in eight fp32 chains (dot2),
    // chains combined in fp64; fp32: fp64 accumulation.
    double ss = 0.0;
    if constexpr (F32IN) {
#pragma unroll
      for (int k = 0; k < 64; ++k) {
        const float v = elem<true>(xr, k);
        ss = fma(static_cast<double>(v), static_cast<double>(v), ss);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float c = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 p = __builtin_bit_cast(bf16x2, word_of(xr[k], e));
          c = __builtin_amdgcn_fdot2_f32_bf16(p, p, c, false);
        }
        ss += static_cast<double>(c);
      }
    }
    ss += __shfl_xor(ss, 32);
    const float normf = static_cast<float>(sqrt(ss));
    int ex;
    frexpf(normf, &ex);
    const int sh = 14 - ex;  // fp16 paths: |x * 2^sh| < 2^14

    // ---- rotation on MFMA, one k-step at a time
    f32x16 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if constexpr (XM == X_BF16) {
        const bf16x8 xb = as_bf16x8(xr[ks]);
        // part-major order: consecutive MFMAs go to independent accumulators
#pragma unroll
        for (int part = 0; part < 3; ++part)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const bf16x8 pf = as_bf16x8(pi_frag[((part * 4 + t) * 8 + ks) * 64 + lane]);
            acc[t] = TILED ? mfma(xb, pf, acc[t]) : mfma(pf, xb, acc[t]);
          }
      } else {
        half8 xh, xl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = ldexpf(elem<F32IN>(xr, 8 * ks + e), sh);
          const _Float16 hi = static_cast<_Float16>(v);
          xh[e] = hi;
          if constexpr (F32IN) xl[e] = static_cast<_Float16>(v - static_cast<float>(hi));
        }
        half8 ph[4], pl[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          ph[t] = as_half8(pi_frag[((0 * 4 + t) * 8 + ks) * 64 + lane]);
          pl[t] = as_half8(pi_frag[((1 * 4 + t) * 8 + ks) * 64 + lane]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = TILED ? mfma(xh, ph[t], acc[t]) : mfma(ph[t], xh, acc[t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = TILED ? mfma(xh, pl[t], acc[t]) : mfma(pl[t], xh, acc[t]);
        if constexpr (F32IN) {
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[t] = TILED ? mfma(xl, ph[t], acc[t]) : mfma(ph[t], xl, acc[t]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // scale of acc relative to the rotated unit vector
    const float sc = XM == X_BF16 ? normf : ldexpf(normf, sh + 8);

    if constexpr (!TILED) {
      // ---- record layout: lane (n, h) holds coordinates 64h + 0..63 of vector n
      uint32_t wds[8];
      float tp[7];
      uint8_t* rec = codes + s * stream_code_bytes + pos * CODE_BYTES;
      if constexpr (!QJL) {
        if constexpr (BLO == BHI) {
          load_pos_thresholds<BLO>(tab, 0, sc, tp);
          pack_record<BLO>(acc, tp, wds);
          if (valid) store_record<BLO>(rec + 8 * BLO * h, wds);
        } else if (h == 0) {
          load_pos_thresholds<BLO>(tab, 0, sc, tp);
          pack_record<BLO>(acc, tp, wds);
          if (valid) store_record<BLO>(rec, wds);
        } else {
          load_pos_thresholds<BHI>(tab, 1, sc, tp);
          pack_record<BHI>(acc, tp, wds);
          if (valid) store_record<BHI>(rec + 8 * BLO, wds);
        }
        if (valid && h == 0) norms[s * cap + pos] = normf;
      } else {
        uint32_t idx[64];
        if (h == 0) {
          load_pos_thresholds<BLO>(tab, 0, sc, tp);
          pack_record_scalar<BLO>(acc, tp, wds, idx);
        } else {
          load_pos_thresholds<BHI>(tab, 1, sc, tp);
          pack_record_scalar<BHI>(acc, tp, wds, idx);
        }
        if (valid) {
          if (h == 0) store_record<BLO>(rec, wds);
          else store_record<BHI>(rec + 8 * BLO, wds);
          if (h == 0) norms[s * cap + pos] = normf;
        }
        // residual r = y - c[idx] in the rotated unit-norm domain, scaled by 2^8
        // and split into fp16 hi + lo for the sketch contraction S r.
        const float inv = sc > 0.0f ? 1.0f / sc : 0.0f;
        float rr[64];
        float g2 = 0.0f;
#pragma unroll
        for (int c = 0; c < 64; ++c) {
          const float y = acc[c >> 4][c & 15] * inv;
          rr[c] = y - cen_s[h][idx[c]];
          g2 = fmaf(rr[c], rr[c], g2);
        }
        g2 += __shfl_xor(g2, 32);
        half8 rh[8], rl[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = rr[8 * ks + e] * 256.0f;
            const _Float16 hi = static_cast<_Float16>(v);
            rh[ks][e] = hi;
            rl[ks][e] = static_cast<_Float16>(v - static_cast<float>(hi));
          }
        f32x16 sa[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) sa[t] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          half8 s_h[4], s_l[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            s_h[t] = as_half8(s_frag[((0 * 4 + t) * 8 + ks) * 64 + lane]);
            s_l[t] = as_half8(s_frag[((1 * 4 + t) * 8 + ks) * 64 + lane]);
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) sa[t] = mfma(s_h[t], rh[ks], sa[t]);
#pragma unroll
          for (int t = 0; t < 4; ++t) sa[t] = mfma(s_h[t], rl[ks], sa[t]);
#pragma unroll
          for (int t = 0; t < 4; ++t) sa[t] = mfma(s_l[t], rh[ks], sa[t]);
          __builtin_amdgcn_sched_barrier(0);
        }
        uint32_t sb[2] = {0u, 0u};
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = 16 * t + r;
            sb[j >> 5] |= (sa[t][r] >= 0.0f ? 1u : 0u) << (j & 31);
          }
        if (valid) {
          *reinterpret_cast<uint2*>(signs + (s * cap + pos) * (QJL_M / 8) + 8 * h) = make_uint2(sb[0], sb[1]);
          if (h == 0) rnorms[s * cap + pos] = sqrtf(g2);
        }
      }
    } else {
      // ---- tiled layout: lane (j, h) holds coordinates 4j + t of token slots 16h + r.
      const float inv_own = sc > 0.0f ? 1.0f / sc : 0.0f;
      float inv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) inv[r] = __shfl(inv_own, 8 * (r >> 2) + 4 * h + (r & 3));
      const int j = n;
      const int q = j >> 1;
      constexpr int G = 64 * (BLO + BHI);
      uint8_t* tbase = codes + s * stream_code_bytes + (tile0 + T) * (32 * CODE_BYTES);
      const int64_t p0 = 32 * (tile0 + T);
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int g = 2 * h + gg;
        uint32_t vmask = 0;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int64_t p = p0 + 8 * g + sl;
          vmask |= (p >= tok0 && p < tok0 + n_tok) ? (1u << sl) : 0u;
        }
        uint32_t wds[4];
        float tp[7];
        if constexpr (BLO == BHI) {
          load_pos_thresholds<BLO>(tab, 0, 1.0f, tp);
          pack_tiled<BLO>(acc, inv, tp, gg, wds);
          store_tiled_chunk<BLO>(tbase + g * G + 8 * BLO * q + 4 * BLO * (j & 1), wds, vmask);
        } else if (j < 16) {
          load_pos_thresholds<BLO>(tab, 0, 1.0f, tp);
          pack_tiled<BLO>(acc, inv, tp, gg, wds);
          store_tiled_chunk<BLO>(tbase + g * G + 8 * BLO * q + 4 * BLO * (j & 1), wds, vmask);
        } else {
          load_pos_thresholds<BHI>(tab, 1, 1.0f, tp);
          pack_tiled<BHI>(acc, inv, tp, gg, wds);
          store_tiled_chunk<BHI>(tbase + g * G + 64 * BLO + 8 * BHI * (q - 8) + 4 * BHI * (j & 1), wds, vmask);
        }
      }
      if (valid && h == 0) norms[s * cap + pos] = normf;
    }
#pragma unroll
    for (int k = 0; k < NW; ++k) xr[k] = xnext[k];
  }
}

template <int BLO, int BHI, int XM, bool TILED, bool QJL>
hipError_t launch_one(const Tables* tab, const void* x, int64_t n_streams, int64_t n_tok, int64_t xss, int64_t xrs,
                      int64_t tok0, const tq_cache& c, hipStream_t st) {
  constexpr int CODE_BYTES = 8 * (BLO + BHI);
  int64_t tiles, tile0 = 0;
  if (TILED) {
    tile0 = tok0 / TILE;
    tiles = (tok0 + n_tok + TILE - 1) / TILE - tile0;
  } else {
    tiles = (n_tok + TILE - 1) / TILE;
  }
  const int64_t stream_bytes = c.cap * CODE_BYTES;
  const int64_t total = n_streams * tiles;
  const int64_t blocks = std::min<int64_t>((total + WAVES - 1) / WAVES, 256);
  hipLaunchKernelGGL((quantize_kernel<BLO, BHI, XM, TILED, QJL>), dim3(static_cast<unsigned>(blocks)),
                     dim3(THREADS), 0, st, tab, x, n_tok, xss, xrs, tok0, c.codes, c.norms, c.qjl_signs,
                     c.qjl_rnorms, c.cap, stream_bytes, tiles, tile0, total);
  return hipGetLastError();
}

template <int BLO, int BHI>
hipError_t dispatch_layout(const Spec& sp, const Tables* tab, int dtype, const void* x, int64_t ns, int64_t nt,
                           int64_t xss, int64_t xrs, int64_t tok0, const tq_cache& c, hipStream_t st) {
  const bool f32 = dtype == TQ_F32;
  if (sp.layout == TQ_LAYOUT_TILED) {
    return f32 ? launch_one<BLO, BHI, X_F32, true, false>(tab, x, ns, nt, xss, xrs, tok0, c, st)
               : launch_one<BLO, BHI, X_BF16, true, false>(tab, x, ns, nt, xss, xrs, tok0, c, st);
  }
  if (sp.qjl_m) {
    return f32 ? launch_one<BLO, BHI, X_F32, false, true>(tab, x, ns, nt, xss, xrs, tok0, c, st)
               : launch_one<BLO, BHI, X_BF16_F16, false, true>(tab, x, ns, nt, xss, xrs, tok0, c, st);
  }
  return f32 ? launch_one<BLO, BHI, X_F32, false, false>(tab, x, ns, nt, xss, xrs, tok0, c, st)
             : launch_one<BLO, BHI, X_BF16, false, false>(tab, x, ns, nt, xss, xrs, tok0, c, st);
}

}  // namespace

hipError_t launch_quantize(const Spec& sp, const Tables* tab, int dtype, const void* x, int64_t n_streams,
                           int64_t n_tok, int64_t xss, int64_t xrs, int64_t tok0, const tq_cache& c,
                           hipStream_t st) {
  const int key = sp.bits_lo * 10 + sp.bits_hi;
  switch (key) {
    case 22: return dispatch_layout<2, 2>(sp, tab, dtype, x, n_streams, n_tok, xss, xrs, tok0, c, st);
    case 33: return dispatch_layout<3, 3>(sp, tab, dtype, x, n_streams, n_tok, xss, xrs, tok0, c, st);
    case 44: return dispatch_layout<4, 4>(sp, tab, dtype, x, n_streams, n_tok, xss, xrs, tok0, c, st);
    case 43: return dispatch_layout<4, 3>(sp, tab, dtype, x, n_streams, n_tok, xss, xrs, tok0, c, st);
    case 32: return dispatch_layout<3, 2>(sp, tab, dtype, x, n_streams, n_tok, xss, xrs, tok0, c, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
