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
#include <atomic>
#include <type_traits>
#include <vector>

#include "cell.h"
#include "lanes.h"
#include "norm.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WAVES = 8;
constexpr int THREADS = 64 * WAVES;
constexpr float F16_MAX = 65504.0f;  // fp16 norms saturate here instead of turning into +inf
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
// Code of y (a rotated unit-vector coordinate) from the cell table: the
// cell gives the number of boundaries below it and the one boundary inside.
__device__ __forceinline__ uint32_t cell_code(float y, const uint2* cells) {
  const uint2 e = cell_entry(cells, y);
  return e.y + (y > __uint_as_float(e.x) ? 1u : 0u);
}

// 32 codes code(0..31) packed LSB-first into B dwords (code p at bits
// [B p, B p + B)), built with shift-or chains from the last code down.
template <int B, typename CodeF>
__device__ __forceinline__ void pack_run(CodeF code, uint32_t* w) {
  if constexpr (B == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t x = code(8 * k + 7);
#pragma unroll
      for (int e = 6; e >= 0; --e) x = (x << 4) | code(8 * k + e);
      w[k] = x;
    }
  } else if constexpr (B == 2) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      uint32_t x = code(16 * k + 15);
#pragma unroll
      for (int e = 14; e >= 0; --e) x = (x << 2) | code(16 * k + e);
      w[k] = x;
    }
  } else {
    static_assert(B == 3, "code width");
    // codes 10 and 21 straddle dword boundaries
    const uint32_t c10 = code(10), c21 = code(21);
    uint32_t x = code(9);
#pragma unroll
    for (int e = 8; e >= 0; --e) x = (x << 3) | code(e);
    w[0] = x | (c10 << 30);
    x = c21;
#pragma unroll
    for (int e = 20; e >= 11; --e) x = (x << 3) | code(e);
    w[1] = (x << 1) | (c10 >> 2);
    x = code(31);
#pragma unroll
    for (int e = 30; e >= 22; --e) x = (x << 3) | code(e);
    w[2] = (x << 2) | (c21 >> 1);
  }
}

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

// Sequences of one launch of the general kernel: the launch's tiles are the
// sequences' tiles in order (each sequence's hkv streams, stream-major).
constexpr int GEN_MAX_SEQ = 32;
struct GenSeq {
  int64_t x_off;     // element offset of the sequence's stream 0, row 0
  int64_t tok0;      // cache position of row 0
  int64_t n_tok;     // rows per stream
  int64_t stream0;   // contiguous cache: cache stream of kv head 0 (paged: 0)
  int64_t tiles;     // tiles per stream
  int64_t tile0;     // tiled layout: first tile touched (record: 0)
  int64_t start;     // first launch tile of the sequence
  int64_t page_row;  // paged: the sequence's row of the block table
};
struct GenArgs {
  const Tables* tab;
  const void* x;
  int64_t xss, xrs, cap, stream_code_bytes;
  uint8_t* codes;
  float* norms;
  uint8_t* signs;
  float* rnorms;
  const int32_t* pages;  // paged: the block table (else nullptr)
  int64_t page_ld, n_pages;
  int64_t hkv;
  int64_t total_tiles;
  int32_t n_seq;
  int32_t norm16;
  GenSeq seq[GEN_MAX_SEQ];  // ascending start
};

template <int BLO, int BHI, int XM, bool TILED, bool QJL>
__global__ __launch_bounds__(THREADS, 1) void quantize_kernel(const GenArgs A) {
  const Tables* __restrict__ tab = A.tab;
  const int64_t xss = A.xss, xrs = A.xrs, cap = A.cap, stream_code_bytes = A.stream_code_bytes;
  const int64_t total_tiles = A.total_tiles;
  const int norm16 = A.norm16;
  uint8_t* __restrict__ codes = A.codes;
  float* __restrict__ norms = A.norms;
  uint8_t* __restrict__ signs = A.signs;
  float* __restrict__ rnorms = A.rnorms;
  constexpr bool F32IN = XM == X_F32;
  constexpr int NPART = XM == X_BF16 ? 3 : 2;
  constexpr int CODE_BYTES = 8 * (BLO + BHI);
  __shared__ uint4 pi_frag[NPART * FRAGS];
  __shared__ uint4 s_frag[QJL ? 2 * FRAGS : 1];
  __shared__ float cen_s[2][16];
  __shared__ uint2 cell_s[2][CELL_ENTRIES];

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
  for (int c = threadIdx.x; c < 2 * CELL_ENTRIES; c += THREADS)
    cell_s[c / CELL_ENTRIES][c % CELL_ENTRIES] =
        make_uint2(tab->cell[c / CELL_ENTRIES][c % CELL_ENTRIES][0], tab->cell[c / CELL_ENTRIES][c % CELL_ENTRIES][1]);
  __syncthreads();

  // (wave-uniform: the tile index, its sequence and every address derived
  // from them live in scalar registers, and the sequence search reads the
  // kernel arguments with scalar loads)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, h = lane >> 5;
  // norm i of the launch's streams: fp32, or fp16 rounded to nearest even
  // and saturated at the largest finite binary16 value
  auto put_norm = [&](int64_t i, float v) {
    if (norm16) reinterpret_cast<_Float16*>(norms)[i] = static_cast<_Float16>(fminf(v, F16_MAX));
    else norms[i] = v;
  };

  // Tile w of the launch: its sequence (the last one starting at or before
  // it; wave-uniform), stream s of the sequence, tile T of the stream, and the
  // row of x and the cache position this lane's vector takes (vector column
  // n for the record layout, token slot tiled_slot(n) for the tiled layout).
  struct Loc {
    int64_t x_off, tok0, n_tok, stream0, tile0, page_row;
    int64_t s, T, row, pos;
  };
  auto locate = [&](int64_t w) {
    int sq = 0;
#pragma unroll
    for (int step = GEN_MAX_SEQ / 2; step > 0; step >>= 1)
      if (sq + step < A.n_seq && A.seq[sq + step].start <= w) sq += step;
    const GenSeq& Q = A.seq[sq];
    Loc L;
    L.x_off = Q.x_off;
    L.tok0 = Q.tok0;
    L.n_tok = Q.n_tok;
    L.stream0 = Q.stream0;
    L.tile0 = Q.tile0;
    L.page_row = Q.page_row;
    const int64_t local = w - Q.start;
    L.s = local / Q.tiles;
    L.T = local - L.s * Q.tiles;
    if constexpr (TILED) {
      L.pos = 32 * (L.tile0 + L.T) + tiled_slot(n);
      L.row = L.pos - L.tok0;
    } else {
      L.row = 32 * L.T + n;
      L.pos = L.tok0 + L.row;
    }
    return L;
  };
  // this lane's 64 elements (its half of the vector) as raw words
  constexpr int NW = F32IN ? 16 : 8;
  auto load_x = [&](int64_t w, uint4 (&dst)[NW]) {
    const Loc L = locate(w < total_tiles ? w : total_tiles - 1);
    if (w < total_tiles && L.row >= 0 && L.row < L.n_tok) {
      const uint4* xp = reinterpret_cast<const uint4*>(
          static_cast<const uint8_t*>(A.x) +
          ((L.x_off + L.s * xss + L.row * xrs) + 64 * h) * (F32IN ? 4 : 2));
#pragma unroll
      for (int k = 0; k < NW; ++k) dst[k] = xp[k];
    } else {
#pragma unroll
      for (int k = 0; k < NW; ++k) dst[k] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  const int64_t stride = static_cast<int64_t>(gridDim.x) * WAVES;
  // positive thresholds of each half's codebook (the sketch spec with two
  // widths), read once: scaled per vector in the loop
  float tpos[2][7];
#pragma unroll
  for (int k = 0; k < 7; ++k) {
    tpos[0][k] = k < Width<BLO>::NPOS ? tab->bnd[0][Width<BLO>::HALF + k] : 0.0f;
    tpos[1][k] = k < Width<BHI>::NPOS ? tab->bnd[1][Width<BHI>::HALF + k] : 0.0f;
  }
  uint4 xr[NW];
  load_x(static_cast<int64_t>(blockIdx.x) * WAVES + wave, xr);

  for (int64_t w = static_cast<int64_t>(blockIdx.x) * WAVES + wave; w < total_tiles; w += stride) {
    const Loc L = locate(w);
    const int64_t s = L.s, T = L.T, pos = L.pos, tok0 = L.tok0, n_tok = L.n_tok, tile0 = L.tile0;
    bool valid = L.row >= 0 && L.row < n_tok;
    // destination stream ds and position dp of this lane's vector.  Paged
    // cache: the page of the position (tiled layout: of the tile, which lies
    // inside one page) from the sequence's block-table row; a page outside
    // the pool is not written.
    int64_t ds = L.stream0 + s, dp = pos, dt = tile0 + T;
    bool page_ok = true;
    if (A.pages != nullptr) {
      const int64_t lp = (TILED ? 32 * (tile0 + T) : pos) / TQ_PAGE_TOKENS;
      const int pg = TILED || valid ? A.pages[L.page_row * A.page_ld + lp] : -1;
      page_ok = pg >= 0 && pg < A.n_pages;
      ds = static_cast<int64_t>(page_ok ? pg : 0) * A.hkv + s;
      dp = pos % TQ_PAGE_TOKENS;
      dt = (tile0 + T) % (TQ_PAGE_TOKENS / 32);
      valid = valid && page_ok;
    }
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
    ss = add_half_swap(ss);
    if constexpr (!F32IN) {
      // a sum outside the fp32 chains' exact range (rare): both lanes of
      // such a vector redo theirs on scaled elements
      const bool slow = !sumsq_fast_ok(ss);
      if (__builtin_amdgcn_ballot_w64(slow) != 0) {
        const float s = sumsq_rescale(ss);
        const double s2 = add_half_swap(static_cast<double>(bf16_sumsq_scaled(xr, s)));
        if (slow) ss = s2 / (static_cast<double>(s) * static_cast<double>(s));
      }
    }
    const float normf = static_cast<float>(sqrt(ss));
    int ex;
    frexpf(normf, &ex);
    const int sh = min(14 - ex, 127);  // fp16 paths: |x * 2^sh| < 2^14 (2^sh finite)

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
      uint8_t* rec = codes + ds * stream_code_bytes + dp * CODE_BYTES;
      if constexpr (!QJL) {
        if constexpr (BLO == BHI) {
          // cell-table codes: lane's coordinates 0..31 then 32..63
          const float inv = sc > 0.0f ? 1.0f / sc : 0.0f;
          pack_run<BLO>([&](int p) { return cell_code(acc[p >> 4][p & 15] * inv, cell_s[0]); }, wds);
          pack_run<BLO>([&](int p) { return cell_code(acc[2 + (p >> 4)][p & 15] * inv, cell_s[0]); }, wds + BLO);
          if (valid) store_record<BLO>(rec + 8 * BLO * h, wds);
        } else if (h == 0) {
#pragma unroll
          for (int k = 0; k < Width<BLO>::NPOS; ++k) tp[k] = tpos[0][k] * sc;
          pack_record<BLO>(acc, tp, wds);
          if (valid) store_record<BLO>(rec, wds);
        } else {
#pragma unroll
          for (int k = 0; k < Width<BHI>::NPOS; ++k) tp[k] = tpos[1][k] * sc;
          pack_record<BHI>(acc, tp, wds);
          if (valid) store_record<BHI>(rec + 8 * BLO, wds);
        }
        if (valid && h == 0) put_norm(ds * cap + dp, normf);
      } else {
        uint32_t idx[64];
        if constexpr (BLO == BHI) {
          // one width: cell-table codes for both halves of the vector at once
          const float inv = sc > 0.0f ? 1.0f / sc : 0.0f;
#pragma unroll
          for (int c = 0; c < 64; ++c) idx[c] = cell_code(acc[c >> 4][c & 15] * inv, cell_s[0]);
          pack_run<BLO>([&](int p) { return idx[p]; }, wds);
          pack_run<BLO>([&](int p) { return idx[32 + p]; }, wds + BLO);
          if (valid) store_record<BLO>(rec + 8 * BLO * h, wds);
        } else if (h == 0) {
#pragma unroll
          for (int k = 0; k < Width<BLO>::NPOS; ++k) tp[k] = tpos[0][k] * sc;
          pack_record_scalar<BLO>(acc, tp, wds, idx);
          if (valid) store_record<BLO>(rec, wds);
        } else {
#pragma unroll
          for (int k = 0; k < Width<BHI>::NPOS; ++k) tp[k] = tpos[1][k] * sc;
          pack_record_scalar<BHI>(acc, tp, wds, idx);
          if (valid) store_record<BHI>(rec + 8 * BLO, wds);
        }
        if (valid && h == 0) put_norm(ds * cap + dp, normf);
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
        g2 = add_half_swap(g2);
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
        // sign bits, bit j of word k for sketch row 32 k + j of this half: one
        // funnel shift per row, from the last row down, moves the word up a
        // place and takes the value's IEEE sign bit at the bottom; inverted,
        // a bit is 1 for S r >= 0 (and 0 for a -0.0 sum, where either sign is
        // as good)
        uint32_t sb[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          uint32_t wv = 0u;
#pragma unroll
          for (int j = 31; j >= 0; --j) {
            const int row = 32 * k + j;
            wv = __builtin_amdgcn_alignbit(wv, __float_as_uint(sa[row >> 4][row & 15]), 31);
          }
          sb[k] = ~wv;
        }
        if (valid) {
          *reinterpret_cast<uint2*>(signs + (ds * cap + dp) * (QJL_M / 8) + 8 * h) = make_uint2(sb[0], sb[1]);
          if (h == 0) rnorms[ds * cap + dp] = sqrtf(g2);
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
      uint8_t* tbase = codes + ds * stream_code_bytes + dt * (32 * CODE_BYTES);
      const int64_t p0 = 32 * (tile0 + T);
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int g = 2 * h + gg;
        uint32_t vmask = 0;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int64_t p = p0 + 8 * g + sl;
          vmask |= (page_ok && p >= tok0 && p < tok0 + n_tok) ? (1u << sl) : 0u;
        }
        uint32_t wds[4];
        float tp[7];
        if constexpr (BLO == BHI) {
          // cell-table codes: run position 8 t + s = coordinate 4j + t, token slot s
          pack_run<BLO>([&](int p) { return cell_code(acc[p >> 3][8 * gg + (p & 7)] * inv[8 * gg + (p & 7)],
                                                      cell_s[0]); }, wds);
          store_tiled_chunk<BLO>(tbase + g * G + 8 * BLO * q + 4 * BLO * (j & 1), wds, vmask);
        } else if (j < 16) {
#pragma unroll
          for (int k = 0; k < Width<BLO>::NPOS; ++k) tp[k] = tpos[0][k];
          pack_tiled<BLO>(acc, inv, tp, gg, wds);
          store_tiled_chunk<BLO>(tbase + g * G + 8 * BLO * q + 4 * BLO * (j & 1), wds, vmask);
        } else {
#pragma unroll
          for (int k = 0; k < Width<BHI>::NPOS; ++k) tp[k] = tpos[1][k];
          pack_tiled<BHI>(acc, inv, tp, gg, wds);
          store_tiled_chunk<BHI>(tbase + g * G + 64 * BLO + 8 * BHI * (q - 8) + 4 * BHI * (j & 1), wds, vmask);
        }
      }
      if (valid && h == 0) put_norm(ds * cap + dp, normf);
    }
#pragma unroll
    for (int k = 0; k < NW; ++k) xr[k] = xnext[k];
  }
}

// ---------------------------------------------------------------------------
// Register-resident rotation kernel: every spec without the QJL stage (for
// the tiled layout, the tiles that are written whole).
//
// A workgroup of 2 RQ_PAIRS waves (4) works on RQ_PAIRS 32-vector tiles at a
// time, two workgroups per CU (the register budget allows two waves per
// SIMD; one pair per workgroup and four workgroups measured no faster).  Waves 2p
// and 2p + 1 form pair p and split the 128 rotated coordinates of the pair's
// tile: wave w of the pair owns coordinates [64 w, 64 w + 64) and keeps the
// rows of 256 Pi for them as fp16 hi + lo MFMA fragments in registers for the
// whole launch (the width split of a 3.5-bit spec falls on the same
// boundary).  The pair stages its tile of x through LDS once: norm (partial
// sums in fp32, combined in fp64), a power-of-two scale so |x| 2^sh < 2^14,
// fp16 conversion (hi + lo for fp32 inputs), written straight in MFMA
// operand order; further tiles of x are in flight in registers meanwhile.
// Per tile each wave runs 32 v_mfma_f32_32x32x16_f16 (two 32-coordinate
// blocks x 8 k-steps x hi/lo of Pi; 48 for fp32 inputs) and turns its 64
// coordinates x 32 vectors into codes with the cell table.
//   record layout: A = Pi rows (permuted), B = x^T.  Lane (v, h) holds the
//     32 consecutive coordinates 64 w + 32 h + [0, 32) of vector v: one run
//     of 32 codes, stored as B dwords.
//   tiled layout: A = x (token slots permuted), B = Pi^T.  Lane (c, h) holds
//     coordinate 64 w + 32 t + c of tokens 16 h + [0, 16); the 8 codes of a
//     token group fill one dword, and the 4 lanes of a quad hold the 4
//     coordinates of one half of a sub-block.
// Loads and stores go through per-tile buffer resources whose extent ends at
// the last valid row, and lanes before the first valid row use an offset
// past every extent, so invalid rows read as zero and their stores are
// dropped by the hardware: the loop has no data-dependent branches and the
// prefetched loads stay in flight across iterations.  Tiled-layout tiles
// that are only partly written (the first or last tile of a range that does
// not start or end on a tile boundary) go to a separate launch of the MERGE
// variant, which merges their codes into the stored ones with two returnless
// atomics per word (clear the written tokens' bits, then set them).
// The PAGED variant writes a pool of 64-position pages: tiles start on
// multiples of 32 cache positions in both layouts (so each tile lies in one
// page, and a record-layout range's first and last tiles are written in
// part), and the stores of a tile go to the stream and position of its page,
// read from the block table (a scalar load per tile).
//
// One launch covers up to RQ_MAX_SEQ sequences of a batch (ragged lengths
// and offsets); each sequence's tiles start on a multiple of the tiles per
// pair, so a pair finds its sequence once and all of its tiles lie in it.
constexpr int RQ_PAIRS = 2;  // pairs of waves per workgroup
constexpr int RQ_WAVES = 2 * RQ_PAIRS;
constexpr int RQ_THREADS = 64 * RQ_WAVES;
constexpr int RQ_RESIDENT_PAIRS = 4;  // per CU: two waves per SIMD (the register budget)
constexpr int RSRC_WORD3 = 0x00020000;
constexpr int RQ_MAX_SEQ = 64;
constexpr int RQ_OOB = 0x40000000;  // buffer offset beyond every extent used here

struct RotqSeq {
  int64_t x_off;    // element offset of the sequence's first stream, row 0, in x
  int32_t tok0;     // cache position of row 0
  int32_t n_tok;    // rows (tokens) per stream, > 0
  int32_t stream0;  // cache stream of the sequence's first stream
  int32_t tiles;    // tiles per stream written by this launch
  int32_t start;    // first tile of the sequence in the launch
  int32_t t_lo;     // tile k of a stream is t_lo + k t_step (tiled layout
  int32_t t_step;   //   or paged cache: of the cache positions; else of the rows)
  int32_t page_row; // paged cache: the sequence's row of the block table
};
struct RotqArgs {
  const Tables* tab;
  const void* x;
  uint8_t* codes;
  float* norms;
  int64_t xss, xrs, cap, stream_code_bytes;
  int32_t hkv;  // streams per sequence
  int32_t n_seq;
  const int32_t* pages;     // paged cache: block table [.][page_ld] (device)
  int64_t page_ld;
  int32_t n_pages;
  int32_t norm16;           // norms stored as fp16 (else fp32)
  int64_t n_chunks;         // chunks of K launch tiles
  int32_t n_iter;           // chunks per pair (persistent launch)
  RotqSeq seq[RQ_MAX_SEQ];  // ascending start
};

// token slot v of a tile -> row of the A operand that carries it (inverse of tiled_slot)
__device__ __forceinline__ int tiled_row(int v) { return 8 * ((v >> 2) & 3) + 4 * (v >> 4) + (v & 3); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), RSRC_WORD3);
}

// N codes of run positions p0 .. p0+N-1, table lookups issued together
template <int N, typename YF>
__device__ __forceinline__ void cell_codes(YF yof, int p0, const uint2* cells, uint32_t (&c)[N]) {
  float y[N];
  uint2 e[N];
#pragma unroll
  for (int i = 0; i < N; ++i) y[i] = yof(p0 + i);
#pragma unroll
  for (int i = 0; i < N; ++i) e[i] = cell_entry(cells, y[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) c[i] = e[i].y + (y[i] > __uint_as_float(e[i].x) ? 1u : 0u);
}

// N 8-bit codes of run positions p0 .. p0+N-1 from the 8-bit cell table
// (1024 cells over [-1/2, 1/2]; beyond it the end cells give 0 and 255)
template <int N, typename YF>
__device__ __forceinline__ void cell_codes8(YF yof, int p0, const uint2* cells, uint32_t (&c)[N]) {
  float y[N];
  uint2 e[N];
#pragma unroll
  for (int i = 0; i < N; ++i) y[i] = yof(p0 + i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float f = __builtin_amdgcn_fmed3f(fmaf(y[i], 1024.0f, 512.0f), 0.0f, 1024.0f);
    e[i] = cells[static_cast<uint32_t>(f)];
  }
#pragma unroll
  for (int i = 0; i < N; ++i) c[i] = e[i].y + (y[i] > __uint_as_float(e[i].x) ? 1u : 0u);
}

// 32 codes of y(0..31) packed LSB-first into B dwords
template <int B, typename YF>
__device__ __forceinline__ void code_run(YF yof, const uint2* cells, uint32_t* w) {
  if constexpr (B == 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t c[8];
      cell_codes8<8>(yof, 8 * k, cells, c);
      w[2 * k] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      w[2 * k + 1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    }
  } else if constexpr (B == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t c[8];
      cell_codes<8>(yof, 8 * k, cells, c);
      uint32_t x = c[7];
#pragma unroll
      for (int i = 6; i >= 0; --i) x = (x << 4) | c[i];
      w[k] = x;
    }
  } else if constexpr (B == 2) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      uint32_t c[16];
      cell_codes<16>(yof, 16 * k, cells, c);
      uint32_t x = c[15];
#pragma unroll
      for (int i = 14; i >= 0; --i) x = (x << 2) | c[i];
      w[k] = x;
    }
  } else {
    static_assert(B == 3, "code width");
    uint32_t a[11], b[11], c[10];
    cell_codes<11>(yof, 0, cells, a);    // codes 0..10 (10 straddles)
    cell_codes<11>(yof, 11, cells, b);   // codes 11..21 (21 straddles)
    cell_codes<10>(yof, 22, cells, c);   // codes 22..31
    uint32_t x = a[9];
#pragma unroll
    for (int i = 8; i >= 0; --i) x = (x << 3) | a[i];
    w[0] = x | (a[10] << 30);
    x = b[10];
#pragma unroll
    for (int i = 9; i >= 0; --i) x = (x << 3) | b[i];
    w[1] = (x << 1) | (a[10] >> 2);
    x = c[9];
#pragma unroll
    for (int i = 8; i >= 0; --i) x = (x << 3) | c[i];
    w[2] = (x << 2) | (b[10] >> 1);
  }
}

template <int BLO, int BHI, bool F32IN, bool TILED, int K, bool MERGE, bool PAGED>
__global__ __launch_bounds__(RQ_THREADS, 2) void rotq_kernel(const RotqArgs A) {
  static_assert(!MERGE || TILED, "only the tiled layout merges");
  // 8-bit codes: uniform width, record layout, their own cell table
  constexpr bool B8 = BLO == 8;
  static_assert(!B8 || (BHI == 8 && !TILED), "8-bit codes: uniform width, record layout");
  const Tables* __restrict__ tab = A.tab;
  constexpr int XP = F32IN ? 2 : 1;          // fp16 parts of x
  constexpr int ES = F32IN ? 4 : 2;          // input element bytes
  constexpr int NQW = F32IN ? 8 : 4;         // 16-byte input words per staging thread
  constexpr int CODE_BYTES = 8 * (BLO + BHI);
  __shared__ uint4 xbuf[RQ_PAIRS][2][XP][8 * 64];  // [pair][buffer][part][ks * 64 + lane]
  __shared__ float inv_s[RQ_PAIRS][2][32];         // [pair][buffer][vector]: 1 / (norm 2^(sh+8))
  __shared__ uint2 cell_s[B8 ? 1 : 2][B8 ? CELL8_ENTRIES : CELL_ENTRIES];
  __shared__ uint4 pil1_s[2][8][64];         // low parts of the t = 1 fragments: [w][ks][lane]
  __shared__ int redo_s;                     // a vector needs the robust staging

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform: the pair's tiles, and so the buffer resources, live in SGPRs
  const int pair = __builtin_amdgcn_readfirstlane(tid >> 7), w = __builtin_amdgcn_readfirstlane((tid >> 6) & 1);
  const int pt = tid & 127;
  const int h = lane >> 5, l32 = lane & 31;

  // cell tables: loaded first, stored to LDS once the first tile is staged
  // (a store right here would hold back every later load behind this one)
  constexpr int NCE = B8 ? CELL8_ENTRIES : 2 * CELL_ENTRIES;  // cell entries
  constexpr int CPT = (NCE + RQ_THREADS - 1) / RQ_THREADS;      // per thread
  static_assert(NCE <= CPT * RQ_THREADS && RQ_THREADS <= NCE, "cell table fill");
  const uint2* cell_g = reinterpret_cast<const uint2*>(B8 ? &tab->cell8[0][0] : &tab->cell[0][0][0]);
  uint2 cv[CPT];
  cv[0] = cell_g[tid];
#pragma unroll
  for (int i = 1; i < CPT; ++i) cv[i] = tid + i * RQ_THREADS < NCE ? cell_g[tid + i * RQ_THREADS] : uint2{};

  // ---- rotation fragments of this wave's 64 coordinates, for the whole
  // launch (stored in fragment order: each load is a contiguous 1 KiB).
  // Three quarters stay in registers; the low parts of the second block
  // are shared by both pairs from LDS (read once per k-step), which leaves
  // the registers the loop needs without spilling.
  half8 pih[2][8], pil0[8];
  uint4 pl1[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int f0 = (((w * 2 + 0) * 8 + ks) * 64 + lane) * 8, f1 = (((w * 2 + 1) * 8 + ks) * 64 + lane) * 8;
    pih[0][ks] = as_half8(*reinterpret_cast<const uint4*>(tab->pi_frag[TILED][0] + f0));
    pih[1][ks] = as_half8(*reinterpret_cast<const uint4*>(tab->pi_frag[TILED][0] + f1));
    pil0[ks] = as_half8(*reinterpret_cast<const uint4*>(tab->pi_frag[TILED][1] + f0));
    pl1[ks] = *reinterpret_cast<const uint4*>(tab->pi_frag[TILED][1] + f1);
  }

  // A chunk is K consecutive launch tiles, all in one sequence (each
  // sequence's tiles start on a multiple of K).  With P = RQ_PAIRS pairs per
  // workgroup, PERSIST: pair p of workgroup g takes chunks P g + p +
  // i P gridDim.x for i < A.n_iter, the same count for every pair (a chunk
  // past A.n_chunks is empty: its loads read zeros and its stores are
  // dropped), and its pipeline runs on across chunk boundaries, so the
  // rotation fragments and the pipeline's start are paid once per pair.
  // Otherwise the pair takes chunk P g + p alone.
  constexpr bool PERSIST = K % 6 == 0;  // buffer roles repeat every 3 tiles, LDS buffers every 2
  const int64_t xss = A.xss, xrs = A.xrs, cap = A.cap;
  const int64_t stream_code_bytes = A.stream_code_bytes;
  const int nbytes = A.norm16 ? 2 : 4;  // bytes per stored norm
  // The sequence of a chunk (the last one starting at or before it) and the
  // chunk's place in it; wave-uniform, so it lives in scalar registers.
  struct SeqView {
    const uint8_t* xv;
    uint8_t* codes;
    uint8_t* nrm;
    int64_t n_tok, tok0, tile0, tstep, total_tiles, first;
    uint32_t tps;
    int32_t page_row;
  };
  auto view_of = [&](int64_t chunk) {
    const int64_t first_l = chunk * K;
    int sq = 0;
#pragma unroll
    for (int step = RQ_MAX_SEQ / 2; step > 0; step >>= 1)
      if (sq + step < A.n_seq && A.seq[sq + step].start <= first_l) sq += step;
    const RotqSeq& Q = A.seq[sq];
    SeqView v;
    v.xv = static_cast<const uint8_t*>(A.x) + Q.x_off * ES;
    v.codes = A.codes + static_cast<int64_t>(Q.stream0) * A.stream_code_bytes;
    v.nrm = reinterpret_cast<uint8_t*>(A.norms) + static_cast<int64_t>(Q.stream0) * cap * nbytes;
    v.n_tok = Q.n_tok;
    v.tok0 = Q.tok0;
    v.tile0 = Q.t_lo;
    v.tstep = Q.t_step;
    v.total_tiles = chunk < A.n_chunks ? static_cast<int64_t>(A.hkv) * Q.tiles : 0;
    v.first = first_l - Q.start;  // within the sequence
    v.tps = static_cast<uint32_t>(Q.tiles);
    v.page_row = Q.page_row;
    return v;
  };
  const int64_t chunk0 = static_cast<int64_t>(blockIdx.x) * RQ_PAIRS + pair;
  const int64_t chunk_step = static_cast<int64_t>(gridDim.x) * RQ_PAIRS;
  SeqView cur = view_of(chunk0);

  // Tile tl of the sequence: stream s, tile T of the stream; its rows of x
  // start at r0 and its positions [lo, nv) are written (lo > 0 only for the
  // first tile of a range, in the merge variant and on a paged cache, whose
  // tiles start on multiples of 32 positions, so each lies in one page).
  struct TileAt {
    int64_t s, r0, p0;
    int lo, nv;
  };
  // tile counts fit in 32 bits (checked on the host): branch-free division
  auto tile_at = [&](const SeqView& v, int64_t tl) {
    const uint32_t tps = v.tps;
    const int64_t tile0 = v.tile0, tstep = v.tstep, tok0 = v.tok0, n_tok = v.n_tok;
    TileAt a;
    const uint32_t s32 = static_cast<uint32_t>(tl) / tps;
    a.s = s32;
    const int64_t T = static_cast<uint32_t>(tl) - s32 * tps;
    a.lo = 0;
    if constexpr (MERGE || PAGED) {
      a.p0 = 32 * (tile0 + T * tstep);
      a.r0 = a.p0 - tok0;
      const int64_t lo = -a.r0, hi = n_tok - a.r0;
      a.lo = lo > 0 ? static_cast<int>(lo) : 0;
      a.nv = hi < 32 ? static_cast<int>(hi) : 32;
    } else if constexpr (TILED) {
      a.p0 = 32 * (tile0 + T);
      a.r0 = a.p0 - tok0;
      a.nv = 32;
    } else {
      a.r0 = 32 * T;
      a.p0 = tok0 + a.r0;
      const int64_t left = n_tok - a.r0;
      a.nv = static_cast<int>(left < 32 ? left : 32);
    }
    if (tl >= v.total_tiles) a.lo = a.nv = 0;
    return a;
  };
  // where tile a's positions are stored: stream s (of codes / norms) from
  // position p on; on a paged cache the tile's page from the block table
  // (ok = false: a page outside the pool, nothing is stored)
  struct Dst {
    int64_t s, p;
    bool ok;
  };
  auto dest_at = [&](const SeqView& v, const TileAt& a) {
    Dst d{a.s, a.p0, true};
    if constexpr (PAGED) {
      const int pg = a.nv > a.lo ? A.pages[static_cast<int64_t>(v.page_row) * A.page_ld + a.p0 / TQ_PAGE_TOKENS] : -1;
      d.ok = pg >= 0 && pg < A.n_pages;
      d.s = static_cast<int64_t>(d.ok ? pg : 0) * A.hkv + a.s;
      d.p = a.p0 % TQ_PAGE_TOKENS;
    }
    return d;
  };
  // staging role: vector (token slot) sv of the tile, elements [32 qq, 32 qq + 32)
  const int sv = pt >> 2, qq = pt & 3;
  // rows before lo use an offset past the extent (read as zero)
  auto load_x = [&](const SeqView& v, int64_t tl, uint4 (&dst)[NQW]) {
    const TileAt a = tile_at(v, tl);
    const uint8_t* base = v.xv + (a.s * xss + (a.r0 + a.lo) * xrs) * ES;
    const __amdgpu_buffer_rsrc_t r = rsrc(base, a.nv > a.lo ? ((a.nv - a.lo - 1) * xrs + D) * ES : 0);
    const int off = MERGE || PAGED ? (sv >= a.lo ? static_cast<int>(((sv - a.lo) * xrs + 32 * qq) * ES) : RQ_OOB)
                                   : static_cast<int>((sv * xrs + 32 * qq) * ES);
#pragma unroll
    for (int k = 0; k < NQW; ++k)
      dst[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * k, 0, 0));
  };
  // norm, scale, fp16 conversion into buffer b; the norm goes out here too.
  // Returns whether one of the thread's vectors lies outside the range where
  // the fp32 chains of squares are exact (elements below about 2^-63 or
  // above 2^64); the ROBUST staging (a rare second pass over such a tile)
  // redoes those sums on scaled elements.  The check stays out of the hot
  // path, whose registers and scheduling a branch here would disturb.
  auto stage = [&](auto robust, const SeqView& v, int64_t tl, const uint4 (&xin)[NQW], int b) {
    constexpr bool ROBUST = decltype(robust)::value;
    double ss = 0.0;
    if constexpr (F32IN) {
#pragma unroll
      for (int k = 0; k < NQW; ++k) {
        const float e[4] = {__uint_as_float(xin[k].x), __uint_as_float(xin[k].y), __uint_as_float(xin[k].z),
                            __uint_as_float(xin[k].w)};
#pragma unroll
        for (int u = 0; u < 4; ++u) ss = fma(static_cast<double>(e[u]), static_cast<double>(e[u]), ss);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NQW; ++k) {
        float c = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x2 pr = __builtin_bit_cast(bf16x2, word_of(xin[k], u));
          c = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, c, false);
        }
        ss += static_cast<double>(c);
      }
    }
    ss = add_quad_xor<1>(ss);
    ss = add_quad_xor<2>(ss);
    // (fp32 inputs: squares in fp64, exact over the whole range; rows the
    // tile does not write, such as the zero rows past a partial tile's end,
    // do not count)
    const TileAt a = tile_at(v, tl);
    const bool slow = !F32IN && !sumsq_fast_ok(ss) && sv >= a.lo && sv < a.nv;
    if constexpr (ROBUST && !F32IN) {
      const float s = sumsq_rescale(ss);
      double s2 = static_cast<double>(bf16_sumsq_scaled(xin, s));
      s2 = add_quad_xor<1>(s2);
      s2 = add_quad_xor<2>(s2);
      if (slow) ss = s2 / (static_cast<double>(s) * static_cast<double>(s));
    }
    const float normf = static_cast<float>(sqrt(ss));
    int ex = 0;
    frexpf(normf, &ex);
    // (2^sh stays finite for the smallest norms, where |x| 2^127 < 2^14)
    const int sh = min(14 - ex, 127);
    const float up = ldexpf(1.0f, sh);
    const int arow = TILED ? tiled_row(sv) : sv;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k8 = 4 * qq + c;  // 8-element chunk of the vector
      const int fi = (k8 >> 1) * 64 + arow + 32 * (k8 & 1);
      if constexpr (F32IN) {
        const uint4 a0 = xin[2 * c], a1 = xin[2 * c + 1];
        const uint32_t ww[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        half8 hi, lo;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float e = __uint_as_float(ww[u]) * up;
          hi[u] = static_cast<_Float16>(e);
          lo[u] = static_cast<_Float16>(e - static_cast<float>(hi[u]));
        }
        xbuf[pair][b][0][fi] = __builtin_bit_cast(uint4, hi);
        xbuf[pair][b][XP - 1][fi] = __builtin_bit_cast(uint4, lo);
      } else {
        uint32_t ow[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t wd = word_of(xin[c], u);
          // bf16 x 2^sh is exact in fp16 over its normal range
          const auto hv = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(wd << 16) * up,
                                                     __uint_as_float(wd & 0xFFFF0000u) * up);
          ow[u] = __builtin_bit_cast(uint32_t, hv);
        }
        xbuf[pair][b][0][fi] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
      }
    }
    // the four threads of a vector write the same values
    inv_s[pair][b][sv] = normf > 0.0f ? 1.0f / ldexpf(normf, sh + 8) : 0.0f;
    const Dst d = dest_at(v, a);
    const __amdgpu_buffer_rsrc_t rn =
        rsrc(v.nrm + (d.s * cap + d.p) * nbytes, d.ok ? static_cast<int64_t>(a.nv) * nbytes : 0);
    const int noff = !(MERGE || PAGED) || sv >= a.lo ? nbytes * sv : RQ_OOB;
    if (A.norm16)
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<_Float16>(fminf(normf, F16_MAX))),
                                            rn, noff, 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(normf), rn, noff, 0, 0);
    return slow;
  };
  // ---- pipeline, straight-line over each chunk's K tiles: three register
  // buffers with fixed roles (tile k+1 is staged from X[(k+1) % 3] while
  // tiles k+2, k+3 are still loading; the buffer is then refilled with tile
  // k+4), so the waits on in-flight loads are exact.  PERSIST: tiles k+1 and
  // k+4 past the chunk's end are the first tiles of the pair's next chunk.
  //
  // The loop runs once with the fast staging and collects whether any of
  // its vectors lay outside the fast norm's range; if one did anywhere in
  // the workgroup (never, for data of any ordinary scale), the workgroup
  // runs it again with the robust staging, which rewrites every output of
  // its tiles.  The hot loop itself then has no extra branch.
  if (tid == 0) redo_s = 0;
  auto pass = [&, pl1, cv](auto robust) __attribute__((always_inline)) -> bool {
  constexpr bool R = decltype(robust)::value;
  uint64_t need = 0;
  cur = view_of(chunk0);
  uint4 X[3][NQW];
  load_x(cur, cur.first, X[0]);
  if (PERSIST || K > 1) load_x(cur, cur.first + 1, X[1]);
  if (PERSIST || K > 2) load_x(cur, cur.first + 2, X[2]);
  // (the fragment loads are older than the tile loads: this waits for them only)
  if (!R && pair == 0) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) pil1_s[w][ks][lane] = pl1[ks];
  }
  need |= __builtin_amdgcn_ballot_w64(stage(robust, cur, cur.first, X[0], 0));
  if (PERSIST || K > 3) load_x(cur, cur.first + 3, X[0]);
  if constexpr (!R) {
    reinterpret_cast<uint2*>(cell_s)[tid] = cv[0];
#pragma unroll
    for (int i = 1; i < CPT; ++i)
      if (tid + i * RQ_THREADS < NCE) reinterpret_cast<uint2*>(cell_s)[tid + i * RQ_THREADS] = cv[i];
  }
  __syncthreads();
  const int n_iter = PERSIST ? A.n_iter : 1;
  for (int it = 0; it < n_iter; ++it) {
  const SeqView nxt = PERSIST ? view_of(chunk0 + (it + 1) * chunk_step) : cur;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t tl = cur.first + k;
    const int b = k & 1;
    f32x16 acc[2];
    acc[0] = acc[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const half8 xh = as_half8(xbuf[pair][b][0][ks * 64 + lane]);
      const half8 pil[2] = {pil0[ks], as_half8(pil1_s[w][ks][lane])};
      if constexpr (TILED) {
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[t] = mfma(xh, pih[t][ks], acc[t]);
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[t] = mfma(xh, pil[t], acc[t]);
        if constexpr (F32IN) {
          const half8 xl = as_half8(xbuf[pair][b][XP - 1][ks * 64 + lane]);
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[t] = mfma(xl, pih[t][ks], acc[t]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[t] = mfma(pih[t][ks], xh, acc[t]);
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[t] = mfma(pil[t], xh, acc[t]);
        if constexpr (F32IN) {
          const half8 xl = as_half8(xbuf[pair][b][XP - 1][ks * 64 + lane]);
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[t] = mfma(pih[t][ks], xl, acc[t]);
        }
      }
    }
    // stage the next tile into the other buffer while the products finish,
    // and refill its registers: they are free before the codes are made
    if (k + 1 < K) {
      need |= __builtin_amdgcn_ballot_w64(stage(robust, cur, tl + 1, X[(k + 1) % 3], b ^ 1));
      if (k + 4 < K) load_x(cur, tl + 4, X[(k + 1) % 3]);
      else if (PERSIST) load_x(nxt, nxt.first + (k + 4 - K), X[(k + 1) % 3]);
    } else if (PERSIST) {
      need |= __builtin_amdgcn_ballot_w64(stage(robust, nxt, nxt.first, X[(k + 1) % 3], b ^ 1));
      load_x(nxt, nxt.first + 3, X[(k + 1) % 3]);
    }
    const TileAt a = tile_at(cur, tl);
    const Dst to = dest_at(cur, a);
    uint8_t* sbase = cur.codes + to.s * stream_code_bytes;
    if constexpr (!TILED) {
      const float inv = inv_s[pair][b][l32];
      const __amdgpu_buffer_rsrc_t rc =
          rsrc(sbase + to.p * CODE_BYTES, to.ok ? static_cast<int64_t>(a.nv) * CODE_BYTES : 0);
      uint32_t wd[B8 ? 8 : 4];
      auto yv = [&](int p) { return acc[p >> 4][p & 15] * inv; };
      auto put = [&](auto bw, int off) {
        constexpr int BW = decltype(bw)::value;
        // (slots before lo: past the extent, dropped)
        const int o = !PAGED || l32 >= a.lo ? l32 * CODE_BYTES + off : RQ_OOB;
        using V4 = decltype(__builtin_amdgcn_raw_buffer_load_b128(rc, 0, 0, 0));
        if constexpr (BW == 8) {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(V4, make_uint4(wd[0], wd[1], wd[2], wd[3])), rc, o,
                                                 0, 0);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(V4, make_uint4(wd[4], wd[5], wd[6], wd[7])), rc,
                                                 o + 16, 0, 0);
        } else if constexpr (BW == 4) {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(V4, make_uint4(wd[0], wd[1], wd[2], wd[3])), rc, o,
                                                 0, 0);
        } else if constexpr (BW == 2) {
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b64(rc, 0, 0, 0)),
                                                                   make_uint2(wd[0], wd[1])), rc, o, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(wd[0], rc, o, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(wd[1], rc, o + 4, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(wd[2], rc, o + 8, 0, 0);
        }
      };
      if (BLO == BHI || w == 0) {
        code_run<BLO>(yv, cell_s[0], wd);
        put(std::integral_constant<int, BLO>{}, w == 0 ? 4 * BLO * h : 8 * BLO + 4 * BLO * h);
      } else {
        code_run<BHI>(yv, cell_s[B8 ? 0 : 1], wd);
        put(std::integral_constant<int, BHI>{}, 8 * BLO + 4 * BHI * h);
      }
    } else {
      const float* invb = inv_s[pair][b] + 16 * h;
      constexpr int G = 64 * (BLO + BHI);
      const __amdgpu_buffer_rsrc_t rc =
          rsrc(sbase + to.p * CODE_BYTES, to.ok && a.nv > a.lo ? static_cast<int64_t>(32) * CODE_BYTES : 0);
      const int qa = l32 & 3;
      auto emit = [&](auto bw, const uint2* cells) {
        constexpr int BW = decltype(bw)::value;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int cabs = 64 * w + 32 * t + l32;
          const int q = cabs >> 3, rh = (cabs >> 2) & 1;
          const int qoff = q < 8 ? 8 * BLO * q : 64 * BLO + 8 * BHI * (q - 8);
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            const float4 i0 = *reinterpret_cast<const float4*>(invb + 8 * gg);
            const float4 i1 = *reinterpret_cast<const float4*>(invb + 8 * gg + 4);
            const float iv[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
            uint32_t c[8];
            cell_codes<8>([&](int p) { return acc[t][8 * gg + p] * iv[p]; }, 0, cells, c);
            uint32_t d = c[7];
#pragma unroll
            for (int sl = 6; sl >= 0; --sl) d = (d << BW) | c[sl];
            // dword qa of the 32-code chunk of the quad (coordinates 4m .. 4m+3)
            const uint32_t nx =
                static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(d), 0x39, 0xF, 0xF, false));
            uint32_t out;
            if constexpr (BW == 4) out = d;
            else if constexpr (BW == 2) out = d | (nx << 16);
            else out = (d >> (8 * qa)) | (nx << (24 - 8 * qa));
            const int dw = BW == 2 ? (qa >> 1) : qa;
            const bool owner = BW == 4 || (BW == 2 ? (qa & 1) == 0 : qa < 3);
            const int o = (2 * h + gg) * G + qoff + 4 * BW * rh + 4 * dw;
            if constexpr (!MERGE) {
              // non-owners store past the tile's extent (dropped)
              __builtin_amdgcn_raw_buffer_store_b32(out, rc, owner ? o : 32 * CODE_BYTES, 0, 0);
            } else {
              // bits of the tokens [lo, nv) of group g: in each coordinate's
              // 8 BW-bit field, token s holds bits [s BW, s BW + BW)
              const int g8 = 8 * (2 * h + gg);
              const int sl = min(max(a.lo - g8, 0), 8), sh = min(max(a.nv - g8, 0), 8);
              const uint64_t fm = sh > sl ? ((uint64_t{1} << (BW * (sh - sl))) - 1) << (BW * sl) : 0;
              const int dbit = 32 * (BW * rh + dw);  // first bit of the word in its sub-block
              uint32_t m = 0;
#pragma unroll
              for (int f = 0; f < 3; ++f) {
                const int fs = 8 * BW * (dbit / (8 * BW) + f) - dbit;  // field start, relative to the word
                if (fs < 32) m |= fs >= 0 ? static_cast<uint32_t>(fm << fs) : static_cast<uint32_t>(fm >> -fs);
              }
              // clear, then set, with returnless atomics: same lane and word,
              // so they apply in order; m != 0 only for a word of a real tile
              if (owner && m != 0 && to.ok) {
                uint32_t* wp = reinterpret_cast<uint32_t*>(sbase + to.p * CODE_BYTES + o);
                __hip_atomic_fetch_and(wp, ~m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_fetch_or(wp, out & m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              }
            }
          }
        }
      };
      if (BLO == BHI || w == 0) emit(std::integral_constant<int, BLO>{}, cell_s[0]);
      else emit(std::integral_constant<int, BHI>{}, cell_s[1]);
    }
    if (PERSIST || k + 1 < K) __syncthreads();
  }
  cur = nxt;
  }
  return need != 0;
  };
  if (pass(std::false_type{})) redo_s = 1;
  __syncthreads();
  if (redo_s != 0) pass(std::true_type{});
}

// The general kernel over a ragged batch: one launch per GEN_MAX_SEQ
// sequences, each launch's workgroups walking all of its tiles (so every
// workgroup stages the rotation and sketch fragments once per launch).
template <int BLO, int BHI, int XM, bool TILED, bool QJL>
hipError_t launch_general(const Tables* tab, const void* x, const QSeq* seqs, int64_t n_seq, int64_t hkv,
                          int64_t xss, int64_t xrs, const tq_cache& c, const PageMap& pm, int norm16,
                          hipStream_t st) {
  constexpr int CODE_BYTES = 8 * (BLO + BHI);
  GenArgs a{};
  a.tab = tab;
  a.x = x;
  a.xss = xss;
  a.xrs = xrs;
  a.cap = c.cap;
  a.stream_code_bytes = c.cap * CODE_BYTES;
  a.codes = c.codes;
  a.norms = c.norms;
  a.signs = c.qjl_signs;
  a.rnorms = c.qjl_rnorms;
  a.pages = pm.table;
  a.page_ld = pm.ld;
  a.n_pages = pm.n_pages;
  a.hkv = hkv;
  a.norm16 = norm16;
  auto flush = [&]() -> hipError_t {
    if (a.n_seq == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((a.total_tiles + WAVES - 1) / WAVES, 256);
    hipLaunchKernelGGL((quantize_kernel<BLO, BHI, XM, TILED, QJL>), dim3(static_cast<unsigned>(blocks)),
                       dim3(THREADS), 0, st, a);
    a.n_seq = 0;
    a.total_tiles = 0;
    return hipGetLastError();
  };
  for (int64_t i = 0; i < n_seq; ++i) {
    const QSeq& q = seqs[i];
    if (q.n_tok <= 0) continue;
    GenSeq g{};
    g.x_off = q.x_off;
    g.tok0 = q.tok0;
    g.n_tok = q.n_tok;
    g.stream0 = pm.table ? 0 : q.stream0;
    g.page_row = q.page_row;
    if (TILED) {
      g.tile0 = q.tok0 / TILE;
      g.tiles = (q.tok0 + q.n_tok + TILE - 1) / TILE - g.tile0;
    } else {
      g.tile0 = 0;
      g.tiles = (q.n_tok + TILE - 1) / TILE;
    }
    g.start = a.total_tiles;
    a.seq[a.n_seq++] = g;
    a.total_tiles += hkv * g.tiles;
    if (a.n_seq == GEN_MAX_SEQ) {
      const hipError_t e = flush();
      if (e != hipSuccess) return e;
    }
  }
  return flush();
}

// Compute units of the current device (cached per device).
int cu_count_cached() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// tiles [t_lo, t_lo + t_step, ...) (tiles of them) of every stream of a sequence
struct RotqPart {
  QSeq q;
  int64_t t_lo, t_step, tiles;
};

template <int BLO, int BHI, bool F32IN, bool TILED, bool MERGE, bool PAGED>
hipError_t launch_rotq_list(const Tables* tab, const void* x, const std::vector<RotqPart>& list, int64_t hkv,
                            int64_t xss, int64_t xrs, const tq_cache& c, const PageMap& pm, int norm16,
                            hipStream_t st) {
  constexpr int CODE_BYTES = 8 * (BLO + BHI);
  const int64_t n = static_cast<int64_t>(list.size());
  for (int64_t b0 = 0; b0 < n; b0 += RQ_MAX_SEQ) {
    const int nb = static_cast<int>(std::min<int64_t>(RQ_MAX_SEQ, n - b0));
    int64_t raw = 0;
    for (int i = 0; i < nb; ++i) raw += hkv * list[b0 + i].tiles;
    // A persistent launch (chunks of 6 tiles, each pair looping over its
    // chunks) once every resident pair gets at least 8 chunks; else one chunk
    // per pair: 8 tiles once that still fills every CU twice over, or 2.
    const int64_t pairs = RQ_RESIDENT_PAIRS * static_cast<int64_t>(cu_count_cached());
    const int K = MERGE ? 2 : raw >= 6 * 8 * pairs ? 6 : raw >= 8 * 1024 ? 8 : 2;

    RotqArgs a{};
    a.tab = tab;
    a.x = x;
    a.codes = c.codes;
    a.norms = c.norms;
    a.xss = xss;
    a.xrs = xrs;
    a.cap = c.cap;
    a.stream_code_bytes = c.cap * CODE_BYTES;
    a.hkv = static_cast<int32_t>(hkv);
    a.n_seq = nb;
    a.pages = pm.table;
    a.page_ld = pm.ld;
    a.n_pages = static_cast<int32_t>(pm.n_pages);
    a.norm16 = norm16;
    int64_t total = 0;  // each sequence's tiles start on a multiple of K
    for (int i = 0; i < nb; ++i) {
      const RotqPart& p = list[b0 + i];
      a.seq[i] = RotqSeq{p.q.x_off,
                         static_cast<int32_t>(p.q.tok0),
                         static_cast<int32_t>(p.q.n_tok),
                         static_cast<int32_t>(p.q.stream0),
                         static_cast<int32_t>(p.tiles),
                         static_cast<int32_t>(total),
                         static_cast<int32_t>(p.t_lo),
                         static_cast<int32_t>(p.t_step),
                         static_cast<int32_t>(p.q.page_row)};
      total += (hkv * p.tiles + K - 1) / K * K;
    }
    a.n_chunks = total / K;
    unsigned blocks = static_cast<unsigned>((a.n_chunks + RQ_PAIRS - 1) / RQ_PAIRS);
    a.n_iter = 1;
    if (K == 6) {
      // the resident workgroups only (two waves per SIMD, the register
      // budget of the kernel), each pair looping over its chunks
      const int64_t resident = RQ_RESIDENT_PAIRS / RQ_PAIRS * static_cast<int64_t>(cu_count_cached());
      if (blocks > resident) blocks = static_cast<unsigned>(resident);
      a.n_iter = static_cast<int32_t>((a.n_chunks + RQ_PAIRS * blocks - 1) / (RQ_PAIRS * blocks));
    }
    if constexpr (MERGE) {
      hipLaunchKernelGGL((rotq_kernel<BLO, BHI, F32IN, TILED, 2, true, PAGED>), dim3(blocks), dim3(RQ_THREADS), 0,
                         st, a);
    } else {
      if (K == 6)
        hipLaunchKernelGGL((rotq_kernel<BLO, BHI, F32IN, TILED, 6, false, PAGED>), dim3(blocks), dim3(RQ_THREADS),
                           0, st, a);
      else if (K == 8)
        hipLaunchKernelGGL((rotq_kernel<BLO, BHI, F32IN, TILED, 8, false, PAGED>), dim3(blocks), dim3(RQ_THREADS),
                           0, st, a);
      else
        hipLaunchKernelGGL((rotq_kernel<BLO, BHI, F32IN, TILED, 2, false, PAGED>), dim3(blocks), dim3(RQ_THREADS),
                           0, st, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BLO, int BHI, bool F32IN, bool TILED>
hipError_t launch_rotq(const Tables* tab, const void* x, const QSeq* seqs, int64_t n_seq, int64_t hkv, int64_t xss,
                       int64_t xrs, const tq_cache& c, const PageMap& pm, int norm16, hipStream_t st) {
  constexpr int64_t ES = F32IN ? 4 : 2;
  constexpr int XM = F32IN ? X_F32 : X_BF16;
  const bool paged = pm.table != nullptr;
  // whole tiles in one list; tiled-layout tiles written only in part in another
  std::vector<RotqPart> whole, part;
  int64_t all = 0, streams = paged ? pm.n_pages * hkv : 0;
  for (int64_t i = 0; i < n_seq; ++i) {
    const QSeq& q = seqs[i];
    const int64_t end = q.tok0 + q.n_tok;
    if constexpr (!TILED) {
      // paged: tiles on multiples of 32 positions (each in one page), the
      // first and last written in part
      if (paged)
        whole.push_back(RotqPart{q, q.tok0 / TILE, 1, (end + TILE - 1) / TILE - q.tok0 / TILE});
      else
        whole.push_back(RotqPart{q, 0, 1, (q.n_tok + TILE - 1) / TILE});
    } else {
      const int64_t f = q.tok0 / TILE, e = (end + TILE - 1) / TILE;     // tiles touched
      const int64_t wf = (q.tok0 + TILE - 1) / TILE, we = end / TILE;  // tiles written whole
      if (we > wf) whole.push_back(RotqPart{q, wf, 1, we - wf});
      const bool head = q.tok0 % TILE != 0, tail = end % TILE != 0;
      if (f == e - 1) {
        if (head || tail) part.push_back(RotqPart{q, f, 1, 1});
      } else if (head && tail) {
        part.push_back(RotqPart{q, f, e - 1 - f, 2});
      } else if (head || tail) {
        part.push_back(RotqPart{q, head ? f : e - 1, 1, 1});
      }
    }
    all += hkv * ((q.n_tok + TILE - 1) / TILE + 2) + 16;
    if (!paged) streams = std::max(streams, q.stream0 + hkv);
  }
  // 32-bit tile, position and stream arithmetic, and buffer offsets below RQ_OOB
  if (all + 16 * 1024 >= (int64_t{1} << 31) || 32 * xrs * ES >= RQ_OOB || c.cap >= (int64_t{1} << 31) - 64 ||
      streams >= (int64_t{1} << 31)) {
    // (8-bit codes have no general-kernel path)
    if constexpr (BLO == 8) return hipErrorNotSupported;
    else return launch_general<BLO, BHI, XM, TILED, false>(tab, x, seqs, n_seq, hkv, xss, xrs, c, pm, norm16, st);
  }
  auto run = [&](auto pg) {
    constexpr bool P = decltype(pg)::value;
    hipError_t e = launch_rotq_list<BLO, BHI, F32IN, TILED, false, P>(tab, x, whole, hkv, xss, xrs, c, pm, norm16, st);
    if constexpr (TILED) {
      if (e == hipSuccess && !part.empty())
        e = launch_rotq_list<BLO, BHI, F32IN, TILED, true, P>(tab, x, part, hkv, xss, xrs, c, pm, norm16, st);
    }
    return e;
  };
  return paged ? run(std::true_type{}) : run(std::false_type{});
}

template <int BLO, int BHI>
hipError_t dispatch_layout(const Spec& sp, const Tables* tab, int dtype, const void* x, const QSeq* seqs,
                           int64_t n_seq, int64_t hkv, int64_t xss, int64_t xrs, const tq_cache& c,
                           const PageMap& pm, hipStream_t st) {
  const bool f32 = dtype == TQ_F32;
  if (sp.qjl_m) {
    const int nf = sp.norm16;
    return f32 ? launch_general<BLO, BHI, X_F32, false, true>(tab, x, seqs, n_seq, hkv, xss, xrs, c, pm, nf, st)
               : launch_general<BLO, BHI, X_BF16_F16, false, true>(tab, x, seqs, n_seq, hkv, xss, xrs, c, pm, nf, st);
  }
  if (sp.layout == TQ_LAYOUT_TILED) {
    return f32 ? launch_rotq<BLO, BHI, true, true>(tab, x, seqs, n_seq, hkv, xss, xrs, c, pm, sp.norm16, st)
               : launch_rotq<BLO, BHI, false, true>(tab, x, seqs, n_seq, hkv, xss, xrs, c, pm, sp.norm16, st);
  }
  return f32 ? launch_rotq<BLO, BHI, true, false>(tab, x, seqs, n_seq, hkv, xss, xrs, c, pm, sp.norm16, st)
             : launch_rotq<BLO, BHI, false, false>(tab, x, seqs, n_seq, hkv, xss, xrs, c, pm, sp.norm16, st);
}

}  // namespace


hipError_t launch_quantize(const Spec& sp, const Tables* tab, int dtype, const void* x, const QSeq* seqs,
                           int64_t n_seq, int64_t hkv, int64_t xss, int64_t xrs, const tq_cache& c,
                           const PageMap& pm, hipStream_t st) {
  // the Hadamard rotation by butterflies where that kernel applies (and its
  // 32-bit buffer offsets hold); otherwise the same matrix on the MFMA path
  if (sp.rotation == TQ_ROT_HADAMARD_FWHT && fwht_supported(sp, dtype, pm.table != nullptr) &&
      64 * xrs < (int64_t{1} << 30) && c.cap < (int64_t{1} << 24))
    return launch_quantize_fwht(sp, tab, x, seqs, n_seq, hkv, xss, xrs, c, st);
  const int key = sp.bits_lo * 10 + sp.bits_hi;
  switch (key) {
    case 22: return dispatch_layout<2, 2>(sp, tab, dtype, x, seqs, n_seq, hkv, xss, xrs, c, pm, st);
    case 33: return dispatch_layout<3, 3>(sp, tab, dtype, x, seqs, n_seq, hkv, xss, xrs, c, pm, st);
    case 44: return dispatch_layout<4, 4>(sp, tab, dtype, x, seqs, n_seq, hkv, xss, xrs, c, pm, st);
    case 43: return dispatch_layout<4, 3>(sp, tab, dtype, x, seqs, n_seq, hkv, xss, xrs, c, pm, st);
    case 32: return dispatch_layout<3, 2>(sp, tab, dtype, x, seqs, n_seq, hkv, xss, xrs, c, pm, st);
    case 88:  // 8-bit keys: record layout, no sketch (checked on the host)
      return dtype == TQ_F32
                 ? launch_rotq<8, 8, true, false>(tab, x, seqs, n_seq, hkv, xss, xrs, c, pm, sp.norm16, st)
                 : launch_rotq<8, 8, false, false>(tab, x, seqs, n_seq, hkv, xss, xrs, c, pm, sp.norm16, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
