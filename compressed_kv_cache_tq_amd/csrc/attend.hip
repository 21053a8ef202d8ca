// Decode attention read directly from the packed cache.
//
// noze.it, "TurboQuant-MLX: quantizzare pesi e KV cache per LLM open-weight su
// Mac", section "Il metodo TurboQuant, in breve": inner products are taken
// against the codebook reconstruction, corrected by the 1-bit residual sketch
// when present.  GitHub issue "Greetings from TurboQuant-MLX & Some Insights
// to Share!": item 1 (the first ~128 tokens stay uncompressed) and item 3
// (value dequantization is skipped when the attention weight is below 1e-6).
//
// Two launches on one stream:
//  split    one workgroup of 8 waves per (split, kv head, sequence).
//           Prologue: the workgroup rotates the query heads of its group,
//           q~ = Pi_K q (times scale * log2 e), and u = S q~, scales each
//           head by a power of two and splits it into fp16 hi + lo, straight
//           into the register layout of the score MFMA's A operand.  Stream:
//           each wave streams 32-token tiles with one tile prefetched into
//           registers: K records -> LUT dequantization -> scores on MFMA for
//           all query heads of the group -> online softmax -> V tiles
//           (coordinate-major sub-blocks) -> P V on MFMA in the rotated
//           domain.  The waves merge in LDS and write one partial
//           (m, l, acc[128]) per query head;
//  combine  one workgroup per (sequence, query head, output slice):
//           log-sum-exp merge of the partials and the raw bf16 sink tokens,
//           the slice of one inverse rotation Pi_V^T, normalisation.
//
// Codebook LUTs: entry e of width B maps two codes to their two fp16
// centroids.  The centroids depend only on (d, B), so one LUT per width
// serves K and V.  Each entry is replicated 64 times (one copy per lane) so
// every lookup is bank-conflict free; the address (pair << 8) | (lane << 2)
// of a 4-bit byte pair is built by one v_perm.
#include <cmath>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int SW = 8;          // waves per split workgroup
constexpr int ST = 64 * SW;    // threads per split workgroup
constexpr int PART = 132;      // floats per partial: m, l, 2 pad, acc[128]
constexpr int GMAX = 16;       // query heads per kv head
constexpr int MAX_SINK = 512;  // raw sink tokens per sequence
constexpr int MAX_SPLIT = 512; // splits per (sequence, kv head)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float QJL_C = 1.2533141373155003f / QJL_M;  // sqrt(pi/2) / m

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

// LDS layout of the replicated pair LUTs (bytes): width 4 first, then 3, 2.
template <int B>
constexpr int lut_size() { return (1 << (2 * B)) * 256; }
template <int KLO, int KHI, int VLO, int VHI>
struct LutPlan {
  static constexpr bool has(int B) { return KLO == B || KHI == B || VLO == B || VHI == B; }
  static constexpr int off4 = 0;
  static constexpr int off3 = has(4) ? lut_size<4>() : 0;
  static constexpr int off2 = off3 + (has(3) ? lut_size<3>() : 0);
  static constexpr int bytes = off2 + (has(2) ? lut_size<2>() : 0);
  template <int B>
  static constexpr int off() { return B == 4 ? off4 : B == 3 ? off3 : off2; }
};

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint32_t*>(base + off);
}

// 8 codes of width B (row k of the lane's words) -> 8 fp16 centroids.
template <int B>
__device__ __forceinline__ half8 dequant8(const uint32_t* w, int k, const uint8_t* lut, uint32_t lane4) {
  uint32_t a[4];
  if constexpr (B == 4) {
    const uint32_t v = w[k];
#pragma unroll
    for (int p = 0; p < 4; ++p) a[p] = __builtin_amdgcn_perm(v, lane4, 0x0C0C0000u | ((4u + p) << 8));
  } else {
    const uint32_t v = row_bits<B>(w, k);
    constexpr uint32_t M = (1u << (2 * B)) - 1u;
#pragma unroll
    for (int p = 0; p < 4; ++p) a[p] = (((v >> (2 * B * p)) & M) << 8) | lane4;
  }
  return as_half8(lds_u32(lut, a[0]), lds_u32(lut, a[1]), lds_u32(lut, a[2]), lds_u32(lut, a[3]));
}

// Registers of one 32-token tile for one lane (prefetched one tile ahead).
struct TileRegs {
  uint32_t kw[2][4];  // K record chunk of token slots mu(0, n), mu(1, n)
  uint32_t vw[8];     // V sub-block (token group j, coordinate group n)
  float4 kn[2];       // K norms of tokens 8j .. 8j+7
  float4 vn[2];       // V norms of tokens 8j .. 8j+7
  uint32_t zw[2];     // QJL sign dword j of token slots mu(0, n), mu(1, n)
  float4 rn[2];       // QJL residual norms of tokens 8j .. 8j+7
};

// Offsets are 32-bit and relative to the stream's base pointers.
template <int KLO, int KHI, int VLO, int VHI, bool QJL>
__device__ __forceinline__ void load_tile(TileRegs& r, uint32_t t0, int n, int j, const uint8_t* kbase,
                                          const uint8_t* vbase, const float* knb, const float* vnb,
                                          const uint32_t* zb, const float* rnb) {
  constexpr uint32_t KBYTES = 8 * (KLO + KHI);
  constexpr uint32_t VBYTES = 8 * (VLO + VHI);
  constexpr uint32_t VG = 64 * (VLO + VHI);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const uint32_t tok = t0 + 8 * (n >> 2) + 4 * mb + (n & 3);
    if (j < 2) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(kbase + (tok * KBYTES + 4 * KLO * j));
#pragma unroll
      for (int w = 0; w < KLO; ++w) r.kw[mb][w] = p[w];
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(kbase + (tok * KBYTES + 8 * KLO + 4 * KHI * (j - 2)));
#pragma unroll
      for (int w = 0; w < KHI; ++w) r.kw[mb][w] = p[w];
    }
    if constexpr (QJL) r.zw[mb] = zb[tok * (QJL_M / 32) + j];
  }
  const uint32_t tile = (t0 / TILE) * (TILE * VBYTES) + j * VG;
  if (n < 8) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(vbase + (tile + 8 * VLO * n));
#pragma unroll
    for (int w = 0; w < 2 * VLO; ++w) r.vw[w] = p[w];
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(vbase + (tile + 64 * VLO + 8 * VHI * (n - 8)));
#pragma unroll
    for (int w = 0; w < 2 * VHI; ++w) r.vw[w] = p[w];
  }
  const uint32_t tb = t0 + 8 * j;
  r.kn[0] = *reinterpret_cast<const float4*>(knb + tb);
  r.kn[1] = *reinterpret_cast<const float4*>(knb + tb + 4);
  r.vn[0] = *reinterpret_cast<const float4*>(vnb + tb);
  r.vn[1] = *reinterpret_cast<const float4*>(vnb + tb + 4);
  if constexpr (QJL) {
    r.rn[0] = *reinterpret_cast<const float4*>(rnb + tb);
    r.rn[1] = *reinterpret_cast<const float4*>(rnb + tb + 4);
  }
}

__device__ __forceinline__ float f4get(const float4 (&v)[2], int e) {
  const float4 x = v[e >> 2];
  const int k = e & 3;
  return k == 0 ? x.x : k == 1 ? x.y : k == 2 ? x.z : x.w;
}

// Split kernel: one workgroup of 8 waves per (split, kv head, sequence).
template <int KLO, int KHI, int VLO, int VHI, bool QJL>
__global__ __launch_bounds__(ST, 1) void split_kernel(
    const Tables* __restrict__ ktab, const uint8_t* __restrict__ kcodes, const float* __restrict__ knorms,
    const uint8_t* __restrict__ ksigns, const float* __restrict__ krn, int64_t kcap,
    const Tables* __restrict__ vtab, const uint8_t* __restrict__ vcodes, const float* __restrict__ vnorms,
    int64_t vcap, const int32_t* __restrict__ seq_lens, const float* __restrict__ q, float* __restrict__ parts,
    int hq, int hkv, int sink, int n_split, int64_t chunk, float v_skip, float qscale) {
  using LP = LutPlan<KLO, KHI, VLO, VHI>;
  constexpr int KBYTES = 8 * (KLO + KHI);
  constexpr int VBYTES = 8 * (VLO + VHI);
  // LDS: [LUTs | query prologue] while streaming, then reused by the wave
  // merge.
  constexpr int PRO_OFF = (LP::bytes + 255) / 256 * 256;
  constexpr int PRO = (GMAX * D + 4 * GMAX * D + GMAX * D + (QJL ? GMAX * D : 0) + 2 * GMAX) * 4;
  constexpr int MRG = SW * 16 * (D + 2) * 4;
  constexpr int SMEM = PRO_OFF + PRO > MRG ? PRO_OFF + PRO : MRG;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ uint32_t lutz[4];

  const int split = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int G = hq / hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
  const int64_t stream = static_cast<int64_t>(b) * hkv + kh;
  const int64_t L = seq_lens[b];
  const int64_t comp = L > sink ? L - sink : 0;
  const int64_t t_begin64 = static_cast<int64_t>(split) * chunk;
  const uint32_t t_begin = static_cast<uint32_t>(t_begin64 < comp ? t_begin64 : comp);
  const uint32_t t_end = static_cast<uint32_t>(t_begin64 + chunk < comp ? t_begin64 + chunk : comp);

  const uint8_t* kbase = kcodes + stream * kcap * KBYTES;
  const uint8_t* vbase = vcodes + stream * vcap * VBYTES;
  const float* knb = knorms + stream * kcap;
  const float* vnb = vnorms + stream * vcap;
  const uint32_t* zb = QJL ? reinterpret_cast<const uint32_t*>(ksigns) + stream * kcap * (QJL_M / 32) : nullptr;
  const float* rnb = QJL ? krn + stream * kcap : nullptr;

  // First tile's loads go out before anything else.
  TileRegs cur;
  uint32_t t0 = t_begin + 32 * wave;
  if (t0 < t_end) load_tile<KLO, KHI, VLO, VHI, QJL>(cur, t0, n, j, kbase, vbase, knb, vnb, zb, rnb);

  // ---- prologue: rotate the group's queries.  Thread (pi_i, kq) forms the
  // partial dot of rotated coordinate pi_i over inputs [32 kq, 32 kq + 32).
  float* qraw = reinterpret_cast<float*>(smem + PRO_OFF);  // [GMAX][D]
  float* ppart = qraw + GMAX * D;                            // [4][GMAX][D]
  float* qrot = ppart + 4 * GMAX * D;                        // [GMAX][D]
  float* urot = qrot + GMAX * D;                             // [GMAX][D] (QJL)
  int* shx = reinterpret_cast<int*>(urot + (QJL ? GMAX * D : 0));  // [2][GMAX]
  const float* qg = q + (static_cast<int64_t>(b) * hq + static_cast<int64_t>(kh) * G) * D;
  if (tid < G * (D / 4)) reinterpret_cast<float4*>(qraw)[tid] = reinterpret_cast<const float4*>(qg)[tid];
  const int pi_i = tid & (D - 1), kq = tid >> 7;
  float w[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) w[k] = ktab->pit[(32 * kq + k) * D + pi_i];

  // replicated pair LUTs: entry e of width B at off_B + e*256 + replica*4
  auto build_lut = [&](auto bw) {
    constexpr int B = decltype(bw)::value;
    if constexpr (LP::has(B)) {
      const uint16_t* cen = (KLO == B) ? ktab->cen16[0] : (KHI == B) ? ktab->cen16[1]
                          : (VLO == B) ? vtab->cen16[0] : vtab->cen16[1];
      constexpr int E = 1 << (2 * B);
      constexpr uint32_t MK = (1u << B) - 1u;
      for (int c = threadIdx.x; c < E * 16; c += ST) {
        const int e = c >> 4;
        const uint32_t v = static_cast<uint32_t>(cen[e & MK]) | (static_cast<uint32_t>(cen[e >> B]) << 16);
        reinterpret_cast<uint4*>(smem + LP::template off<B>())[c] = make_uint4(v, v, v, v);
      }
    }
  };
  build_lut(std::integral_constant<int, 4>{});
  build_lut(std::integral_constant<int, 3>{});
  build_lut(std::integral_constant<int, 2>{});
  if (threadIdx.x < 4)
    lutz[threadIdx.x] = ((threadIdx.x & 1) ? 0x3C00u : 0xBC00u) | (((threadIdx.x >> 1) & 1) ? 0x3C000000u : 0xBC000000u);
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
  auto reduce_parts = [&](float* dst, float scale) {
    for (int idx = tid; idx < G * D; idx += ST) {
      const int g = idx >> 7, i = idx & (D - 1);
      dst[idx] = (ppart[(0 * GMAX + g) * D + i] + ppart[(1 * GMAX + g) * D + i] + ppart[(2 * GMAX + g) * D + i] +
                  ppart[(3 * GMAX + g) * D + i]) * scale;
    }
  };
  partial_dots(w, qraw);
  // Power-of-two scale per head for the fp16 operand: Pi is orthogonal, so
  // |q~_i| <= ||q~|| = ||q|| |qscale|, and sh = 14 - exponent of that bound
  // keeps |q~_i| 2^sh below 2^14.  (The sketch product u has no such bound;
  // its scale comes from its maximum.)
  for (int g = wave; g < G; g += SW) {
    const float a0 = qraw[g * D + lane], a1 = qraw[g * D + lane + 64];
    float ss = fmaf(a0, a0, a1 * a1);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if (lane == 0) {
      int ex = 0;
      const float nq = sqrtf(ss) * fabsf(qscale);
      if (nq > 0.0f) frexpf(nq, &ex);
      shx[g] = 14 - ex;
    }
  }
  __syncthreads();
  // A-operand fragments: lane (n, j) holds coordinates 32 j + 8 ks + e of
  // query head n of the group, as fp16 hi and lo parts
  const bool head_ok = n < G;
  half8 qh[4], ql[4], uh[QJL ? 4 : 1], ul[QJL ? 4 : 1];
  auto split_hl = [&](const float (&xs)[8], int sh, half8& hi, half8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = ldexpf(xs[e], sh);
      const _Float16 h = static_cast<_Float16>(x);
      hi[e] = head_ok ? h : static_cast<_Float16>(0.0f);
      lo[e] = head_ok ? static_cast<_Float16>(x - static_cast<float>(h)) : static_cast<_Float16>(0.0f);
    }
  };
  auto fragments = [&](const float* v, int sh, half8 (&hi)[4], half8 (&lo)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float4* src = reinterpret_cast<const float4*>(v + n * D + 32 * j + 8 * ks);
      const float4 x0 = src[0], x1 = src[1];
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      split_hl(xs, sh, hi[ks], lo[ks]);
    }
  };
  const int nn = head_ok ? n : 0;
  const int shq = head_ok ? shx[n] : 0;
  const float qinv = head_ok ? ldexpf(1.0f, -shq) : 0.0f;
  float uinv = 0.0f;
  if constexpr (!QJL) {
    // straight from the four partial dots (same summation order as q~)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float xs[8];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        float4 t[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          t[k] = *reinterpret_cast<const float4*>(ppart + (k * GMAX + nn) * D + 32 * j + 8 * ks + 4 * h2);
        xs[4 * h2 + 0] = (t[0].x + t[1].x + t[2].x + t[3].x) * qscale;
        xs[4 * h2 + 1] = (t[0].y + t[1].y + t[2].y + t[3].y) * qscale;
        xs[4 * h2 + 2] = (t[0].z + t[1].z + t[2].z + t[3].z) * qscale;
        xs[4 * h2 + 3] = (t[0].w + t[1].w + t[2].w + t[3].w) * qscale;
      }
      split_hl(xs, shq, qh[ks], ql[ks]);
    }
  } else {
    reduce_parts(qrot, qscale);
#pragma unroll
    for (int k = 0; k < 32; ++k) w[k] = ktab->sit[(32 * kq + k) * D + pi_i];
    __syncthreads();
    partial_dots(w, qrot);
    __syncthreads();
    reduce_parts(urot, 1.0f);
    __syncthreads();
    for (int g = wave; g < G; g += SW) {
      const float* v = urot + g * D;
      float mx = fmaxf(fabsf(v[lane]), fabsf(v[lane + 64]));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      int ex = 0;
      if (mx > 0.0f) frexpf(mx, &ex);
      if (lane == 0) shx[GMAX + g] = 14 - ex;
    }
    __syncthreads();
    fragments(qrot, shq, qh, ql);
    const int shu = head_ok ? shx[GMAX + n] : 0;
    fragments(urot, shu, uh, ul);
    uinv = head_ok ? ldexpf(QJL_C, -shu) : 0.0f;
  }

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
  const bool vskip_on = v_skip > 0.0f;

  auto tile_step = [&]<bool FULL, bool VSKIP>(const TileRegs& tr, uint32_t t0c) {
    const int nvalid = FULL ? 8 : static_cast<int>(t_end) - static_cast<int>(t0c + 8 * j);
    // two accumulator chains per M-block: hi and lo query parts accumulate
    // into one; the QJL sign products into another
    f32x4 sk[2], sz[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) sk[mb] = sz[mb] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      half8 a[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if constexpr (KLO == KHI) a[mb] = dequant8<KLO>(tr.kw[mb], ks, lut_klo, lane4);
        else a[mb] = j < 2 ? dequant8<KLO>(tr.kw[mb], ks, lut_klo, lane4) : dequant8<KHI>(tr.kw[mb], ks, lut_khi, lane4);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) sk[mb] = mfma16(a[mb], qh[ks], sk[mb]);
      if constexpr (QJL) {
        half8 z[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const uint32_t zv = (tr.zw[mb] >> (8 * ks)) & 0xFFu;
          z[mb] = as_half8(lutz[zv & 3], lutz[(zv >> 2) & 3], lutz[(zv >> 4) & 3], lutz[zv >> 6]);
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sz[mb] = mfma16(z[mb], uh[ks], sz[mb]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sk[mb] = mfma16(a[mb], ql[ks], sk[mb]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sz[mb] = mfma16(z[mb], ul[ks], sz[mb]);
      } else {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sk[mb] = mfma16(a[mb], ql[ks], sk[mb]);
      }
    }
    float s[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * mb + i;
        float dot = sk[mb][i] * qinv;
        if constexpr (QJL) dot = fmaf(f4get(tr.rn, e) * sz[mb][i], uinv, dot);
        s[e] = f4get(tr.kn, e) * dot;
        if constexpr (!FULL) s[e] = e < nvalid ? s[e] : -INFINITY;
        tmax = fmaxf(tmax, s[e]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
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
      float v0 = f4get(tr.vn, e), v1 = f4get(tr.vn, e + 1);
      if constexpr (!FULL) {
        v0 = e < nvalid ? v0 : 0.0f;
        v1 = e + 1 < nvalid ? v1 : 0.0f;
      }
      const _Float16 h0 = static_cast<_Float16>(p0 * v0), h1 = static_cast<_Float16>(p1 * v1);
      pw[e >> 1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
                   (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
    }
    l_run += psum;
    // skip the value work of a tile whose weights all fell below v_skip
    if (!VSKIP || __any(any && head_ok)) {
      const half8 pa = as_half8(pw[0], pw[1], pw[2], pw[3]);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        half8 bv;
        if constexpr (VLO == VHI) bv = dequant8<VLO>(tr.vw, nb, lut_vlo, lane4);
        else bv = n < 8 ? dequant8<VLO>(tr.vw, nb, lut_vlo, lane4) : dequant8<VHI>(tr.vw, nb, lut_vhi, lane4);
        acc[nb] = mfma16(pa, bv, acc[nb]);
      }
    }
  };

  // Tiles in flight per wave: two (the buffers swap roles each tile); the
  // three-deep variant is kept for register-light instances.
  constexpr uint32_t STEP = 32 * SW;
  constexpr int DEPTH = 2;
  auto run = [&](TileRegs& compute, TileRegs& refill, uint32_t ahead) -> bool {
    if (t0 >= t_end) return false;
    if (t0 + ahead < t_end) load_tile<KLO, KHI, VLO, VHI, QJL>(refill, t0 + ahead, n, j, kbase, vbase, knb, vnb, zb, rnb);
    if (vskip_on) {
      if (t0 + 32 <= t_end) tile_step.template operator()<true, true>(compute, t0);
      else tile_step.template operator()<false, true>(compute, t0);
    } else {
      if (t0 + 32 <= t_end) tile_step.template operator()<true, false>(compute, t0);
      else tile_step.template operator()<false, false>(compute, t0);
    }
    t0 += STEP;
    return true;
  };
  if constexpr (DEPTH == 3) {
    TileRegs b1, b2;
    if (t0 + STEP < t_end) load_tile<KLO, KHI, VLO, VHI, QJL>(b1, t0 + STEP, n, j, kbase, vbase, knb, vnb, zb, rnb);
    while (run(cur, b2, 2 * STEP) && run(b1, cur, 2 * STEP) && run(b2, b1, 2 * STEP)) {
    }
  } else {
    TileRegs b1;
    while (run(cur, b1, STEP) && run(b1, cur, STEP)) {
    }
  }

  // ---- merge the waves; l: sum over the 4 token lanes of a head.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
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
      for (int nb = 0; nb < 8; ++nb) mrg_acc[(wave * 16 + 4 * j + i) * D + 8 * n + nb] = acc[nb][i];
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
    float* part = parts + ((static_cast<int64_t>(b) * hq + static_cast<int64_t>(kh) * G + g) * n_split + split) * PART;
    part[4 + c] = a;
    if (c == 0) {
      part[0] = M;
      part[1] = l;
    }
  }

}

// ---------------------------------------------------------------------------
// combine: one workgroup of 256 threads per (sequence, query head, output
// slice of 128 / NQ coordinates): log-sum-exp merge of the split partials
// and the raw bf16 sink tokens, and the slice of the inverse rotation
// Pi_V^T.  Many small workgroups keep the loads spread over many CUs, and
// every global load is issued before the first barrier.
constexpr int CT = 256;

template <int NQ>
__global__ __launch_bounds__(CT) void combine_kernel(const Tables* __restrict__ vtab, const float* __restrict__ q,
                                                     const uint16_t* __restrict__ sink_k,
                                                     const uint16_t* __restrict__ sink_v,
                                                     const int32_t* __restrict__ seq_lens,
                                                     const float* __restrict__ parts, float* __restrict__ out,
                                                     int hq, int hkv, int sink, int n_split, float qscale) {
  constexpr int OW = D / NQ;         // output coordinates of this workgroup
  constexpr int CQ = CT / OW;        // rotated-coordinate chunks
  constexpr int CK = D / CQ;         // rotated coordinates per chunk
  __shared__ float wsp[MAX_SPLIT];   // split maxima, then weights
  __shared__ float lsp[MAX_SPLIT];   // split sums
  __shared__ float ssc[MAX_SINK];    // sink scores, then weights
  __shared__ float qv[D];
  __shared__ float rs[2][D];         // rotated-domain sums (two split halves)
  __shared__ float ob[CQ][OW];
  __shared__ float red[8];
  const int bh = blockIdx.x / NQ, qo = blockIdx.x % NQ;
  const int b = bh / hq, h = bh % hq, kh = h / (hq / hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* pp = parts + static_cast<int64_t>(bh) * n_split * PART;
  const int64_t L = seq_lens[b];
  const int ns = static_cast<int>(L < sink ? L : sink);
  const int64_t stream = static_cast<int64_t>(b) * hkv + kh;
  const uint16_t* sk = sink_k + stream * static_cast<int64_t>(sink) * D;
  const uint16_t* sv = sink_v + stream * static_cast<int64_t>(sink) * D;
  // thread roles: (c, hs) for the rotated sums, (i, cq) for the rotation
  const int c = tid & (D - 1), hs = tid >> 7;
  const int oi = tid % OW, cq = tid / OW, gi = qo * OW + oi;

  // ---- loads
  constexpr int PA = 16;
  float pa[PA];
#pragma unroll
  for (int u = 0; u < PA; ++u) {
    const int sp = hs + 2 * u;
    pa[u] = sp < n_split ? pp[static_cast<int64_t>(sp) * PART + 4 + c] : 0.0f;
  }
  float pic[CK];
#pragma unroll
  for (int k = 0; k < CK; ++k) pic[k] = vtab->pi[(CK * cq + k) * D + gi];
  constexpr int SVN = 16;
  float svv[SVN];
#pragma unroll
  for (int u = 0; u < SVN; ++u) {
    const int t = cq + CQ * u;
    svv[u] = t < ns ? __uint_as_float(static_cast<uint32_t>(sv[static_cast<int64_t>(t) * D + gi]) << 16) : 0.0f;
  }
  const bool has_row = tid < ns;
  uint4 krow[D / 8];
  if (has_row) {
    const uint4* row = reinterpret_cast<const uint4*>(sk + static_cast<int64_t>(tid) * D);
#pragma unroll
    for (int k = 0; k < D / 8; ++k) krow[k] = row[k];
  }
  float mloc = -INFINITY;
  for (int sp = tid; sp < n_split; sp += CT) {
    const float m = pp[static_cast<int64_t>(sp) * PART], l = pp[static_cast<int64_t>(sp) * PART + 1];
    const float mv = l > 0.0f ? m : -INFINITY;
    wsp[sp] = mv;
    lsp[sp] = l;
    mloc = fmaxf(mloc, mv);
  }
  if (ns > 0 && tid < D) qv[tid] = q[static_cast<int64_t>(bh) * D + tid] * qscale;
  __syncthreads();

  // ---- sink scores, maximum
  auto row_dot = [&](const uint4 (&rw)[D / 8]) {
    float dot = 0.0f;
#pragma unroll
    for (int k = 0; k < D / 8; ++k) {
      const uint4 wv = rw[k];
      dot = fmaf(__uint_as_float(wv.x << 16), qv[8 * k], dot);
      dot = fmaf(__uint_as_float(wv.x & 0xFFFF0000u), qv[8 * k + 1], dot);
      dot = fmaf(__uint_as_float(wv.y << 16), qv[8 * k + 2], dot);
      dot = fmaf(__uint_as_float(wv.y & 0xFFFF0000u), qv[8 * k + 3], dot);
      dot = fmaf(__uint_as_float(wv.z << 16), qv[8 * k + 4], dot);
      dot = fmaf(__uint_as_float(wv.z & 0xFFFF0000u), qv[8 * k + 5], dot);
      dot = fmaf(__uint_as_float(wv.w << 16), qv[8 * k + 6], dot);
      dot = fmaf(__uint_as_float(wv.w & 0xFFFF0000u), qv[8 * k + 7], dot);
    }
    return dot;
  };
  if (has_row) {
    const float d0 = row_dot(krow);
    ssc[tid] = d0;
    mloc = fmaxf(mloc, d0);
  }
  for (int t = tid + CT; t < ns; t += CT) {
    uint4 rw[D / 8];
    const uint4* row = reinterpret_cast<const uint4*>(sk + static_cast<int64_t>(t) * D);
#pragma unroll
    for (int k = 0; k < D / 8; ++k) rw[k] = row[k];
    const float d1 = row_dot(rw);
    ssc[t] = d1;
    mloc = fmaxf(mloc, d1);
  }
  for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
  if (lane == 0) red[wave] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // ---- weights and normaliser
  float lloc = 0.0f;
  for (int sp = tid; sp < n_split; sp += CT) {
    const float mv = wsp[sp];
    const float f = mv == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
    wsp[sp] = f;
    lloc = fmaf(f, lsp[sp], lloc);
  }
  for (int t = tid; t < ns; t += CT) {
    const float wt = __builtin_amdgcn_exp2f(ssc[t] - M);
    ssc[t] = wt;
    lloc += wt;
  }
  for (int o = 32; o > 0; o >>= 1) lloc += __shfl_xor(lloc, o);
  __syncthreads();
  if (lane == 0) red[4 + wave] = lloc;
  // ---- rotated-domain sums: thread (c, hs) takes splits hs, hs + 2, ...
  float a = 0.0f;
#pragma unroll
  for (int u = 0; u < PA; ++u)
    if (hs + 2 * u < n_split) a = fmaf(wsp[hs + 2 * u], pa[u], a);
#pragma unroll 8
  for (int sp = hs + 2 * PA; sp < n_split; sp += 2) a = fmaf(wsp[sp], pp[static_cast<int64_t>(sp) * PART + 4 + c], a);
  rs[hs][c] = a;
  __syncthreads();
  const float Ls = red[4] + red[5] + red[6] + red[7];
  // ---- slice of the inverse rotation (+ raw sink values): thread (oi, cq)
  float o = 0.0f;
#pragma unroll
  for (int k = 0; k < CK; ++k) o = fmaf(pic[k], rs[0][CK * cq + k] + rs[1][CK * cq + k], o);
#pragma unroll
  for (int u = 0; u < SVN; ++u)
    if (cq + CQ * u < ns) o = fmaf(ssc[cq + CQ * u], svv[u], o);
  for (int t = cq + CQ * SVN; t < ns; t += CQ)
    o = fmaf(ssc[t], __uint_as_float(static_cast<uint32_t>(sv[static_cast<int64_t>(t) * D + gi]) << 16), o);
  ob[cq][oi] = o;
  __syncthreads();
  if (tid < OW) {
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < CQ; ++k) v += ob[k][tid];
    out[static_cast<int64_t>(bh) * D + qo * OW + tid] = Ls > 0.0f ? v / Ls : 0.0f;
  }
}

template <int KLO, int KHI, int VLO, int VHI, bool QJL>
hipError_t launch_split(const Tables* ktab, const tq_cache& kc, const Tables* vtab, const tq_cache& vc,
                        const tq_attn& a, const AttendPlan& plan, const float* q, const int32_t* seq_lens,
                        float* parts, hipStream_t st) {
  hipLaunchKernelGGL((split_kernel<KLO, KHI, VLO, VHI, QJL>), dim3(plan.n_split, a.hkv, a.batch), dim3(ST), 0, st,
                     ktab, kc.codes, kc.norms, kc.qjl_signs, kc.qjl_rnorms, kc.cap, vtab, vc.codes, vc.norms, vc.cap,
                     seq_lens, q, parts, a.hq, a.hkv, a.sink, plan.n_split, plan.chunk, a.v_skip, a.scale * LOG2E);
  return hipGetLastError();
}

struct SplitArgs {
  const Tables* ktab;
  const tq_cache* kc;
  const Tables* vtab;
  const tq_cache* vc;
  const tq_attn* a;
  const AttendPlan* plan;
  const float* q;
  const int32_t* seq_lens;
  float* parts;
  hipStream_t st;
};

template <int KLO, int KHI, int VLO, int VHI>
hipError_t launch_q(bool qjl, const SplitArgs& f) {
  return qjl ? launch_split<KLO, KHI, VLO, VHI, true>(f.ktab, *f.kc, f.vtab, *f.vc, *f.a, *f.plan, f.q, f.seq_lens,
                                                      f.parts, f.st)
             : launch_split<KLO, KHI, VLO, VHI, false>(f.ktab, *f.kc, f.vtab, *f.vc, *f.a, *f.plan, f.q, f.seq_lens,
                                                       f.parts, f.st);
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

AttendPlan plan_attend(const tq_attn& a) {
  AttendPlan p{};
  const int64_t streams = static_cast<int64_t>(a.batch) * a.hkv;
  const int64_t comp = a.max_len > a.sink ? a.max_len - a.sink : 0;
  const int64_t tiles = (comp + TILE - 1) / TILE;
  // about one 8-wave workgroup per CU, no split longer than 8192 tokens
  // (ragged batches balance better with shorter splits), at most MAX_SPLIT
  int64_t ns = streams > 0 ? (256 + streams - 1) / streams : 1;
  const int64_t by_len = (comp + 8191) / 8192;
  if (ns < by_len) ns = by_len;
  const int64_t cap_ns = (tiles + SW - 1) / SW;  // at least one tile per wave
  if (ns > cap_ns) ns = cap_ns;
  if (ns > MAX_SPLIT) ns = MAX_SPLIT;
  if (ns < 1) ns = 1;
  int64_t chunk_tiles = (tiles + ns - 1) / ns;
  if (chunk_tiles < 1) chunk_tiles = 1;
  ns = (tiles + chunk_tiles - 1) / chunk_tiles;
  if (ns < 1) ns = 1;
  p.n_split = static_cast<int>(ns);
  p.chunk = chunk_tiles * TILE;
  const int64_t heads = static_cast<int64_t>(a.batch) * a.hq;
  p.ws_bytes = static_cast<size_t>(heads) * static_cast<int64_t>(p.n_split) * PART * sizeof(float);
  return p;
}

hipError_t launch_attend(const Spec& ks, const Tables* ktab, const tq_cache& kc, const Spec& vs, const Tables* vtab,
                         const tq_cache& vc, const tq_attn& a, const AttendPlan& plan, const float* q,
                         const uint16_t* sink_k, const uint16_t* sink_v, const int32_t* seq_lens, float* out,
                         void* workspace, hipStream_t st) {
  float* parts = static_cast<float*>(workspace);
  const SplitArgs f{ktab, &kc, vtab, &vc, &a, &plan, q, seq_lens, parts, st};
  const int vkey = vs.bits_lo * 10 + vs.bits_hi;
  const bool qjl = ks.qjl_m != 0;
  hipError_t e;
  switch (ks.bits_lo * 10 + ks.bits_hi) {
    case 22: e = dispatch_v<2, 2>(vkey, qjl, f); break;
    case 33: e = dispatch_v<3, 3>(vkey, qjl, f); break;
    case 44: e = dispatch_v<4, 4>(vkey, qjl, f); break;
    case 43: e = dispatch_v<4, 3>(vkey, qjl, f); break;
    case 32: e = dispatch_v<3, 2>(vkey, qjl, f); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  // four output slices per head while the heads alone would leave most CUs idle
  const int64_t heads = static_cast<int64_t>(a.batch) * a.hq;
  if (heads < 256)
    hipLaunchKernelGGL(combine_kernel<4>, dim3(static_cast<unsigned>(heads * 4)), dim3(CT), 0, st, vtab, q, sink_k,
                       sink_v, seq_lens, parts, out, a.hq, a.hkv, a.sink, plan.n_split, a.scale * LOG2E);
  else
    hipLaunchKernelGGL(combine_kernel<1>, dim3(static_cast<unsigned>(heads)), dim3(CT), 0, st, vtab, q, sink_k,
                       sink_v, seq_lens, parts, out, a.hq, a.hkv, a.sink, plan.n_split, a.scale * LOG2E);
  return hipGetLastError();
}

}  // namespace tq
