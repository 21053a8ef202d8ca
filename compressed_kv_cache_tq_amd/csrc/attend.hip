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
//  split   one workgroup (4 waves) per (split, kv head, sequence).  It first
//          rotates the group's queries, q~ = Pi_K q (times scale*log2 e), and
//          u = S q~, with a power-of-two scale so they split into fp16 hi +
//          lo.  Each wave then streams 32-token tiles, prefetching the next
//          tile into registers: K records -> LUT dequantization in registers
//          -> scores on MFMA for all query heads of the group -> online
//          softmax -> V tiles (coordinate-major sub-blocks) -> P V on MFMA in
//          the rotated domain.  The 4 waves merge in LDS and write one
//          partial (m, l, acc[128]) per query head;
//  combine per query head: log-sum-exp merge of the splits and the raw bf16
//          sink tokens, one inverse rotation Pi_V^T, normalisation.
#include <cmath>

#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int PART = 132;  // floats per partial: m, l, 2 pad, acc[128]
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

// 8 codes of width B -> 8 fp16 centroids, two per LUT entry (pair of codes).
template <int B>
__device__ __forceinline__ half8 dequant8(const uint32_t* w, int k, const uint32_t* lut) {
  const uint32_t v = row_bits<B>(w, k);
  constexpr uint32_t M = (1u << (2 * B)) - 1u;
  return as_half8(lut[v & M], lut[(v >> (2 * B)) & M], lut[(v >> (4 * B)) & M], lut[(v >> (6 * B)) & M]);
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

template <int KLO, int KHI, int VLO, int VHI, bool QJL>
__device__ __forceinline__ void load_tile(TileRegs& r, int64_t t0, int n, int j, const uint8_t* kbase,
                                          const uint8_t* vbase, const float* knb, const float* vnb,
                                          const uint32_t* zb, const float* rnb) {
  constexpr int KBYTES = 8 * (KLO + KHI);
  constexpr int VBYTES = 8 * (VLO + VHI);
  constexpr int VG = 64 * (VLO + VHI);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int64_t tok = t0 + 8 * (n >> 2) + 4 * mb + (n & 3);
    const uint8_t* rec = kbase + tok * KBYTES;
    if (j < 2) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(rec + 4 * KLO * j);
#pragma unroll
      for (int w = 0; w < KLO; ++w) r.kw[mb][w] = p[w];
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(rec + 8 * KLO + 4 * KHI * (j - 2));
#pragma unroll
      for (int w = 0; w < KHI; ++w) r.kw[mb][w] = p[w];
    }
    if constexpr (QJL) r.zw[mb] = zb[tok * (QJL_M / 32) + j];
  }
  const uint8_t* tile = vbase + (t0 / TILE) * (TILE * VBYTES) + j * VG;
  if (n < 8) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(tile + 8 * VLO * n);
#pragma unroll
    for (int w = 0; w < 2 * VLO; ++w) r.vw[w] = p[w];
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(tile + 64 * VLO + 8 * VHI * (n - 8));
#pragma unroll
    for (int w = 0; w < 2 * VHI; ++w) r.vw[w] = p[w];
  }
  const int64_t tb = t0 + 8 * j;
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

// Split kernel: one workgroup per (split, kv head, sequence).
template <int KLO, int KHI, int VLO, int VHI, bool QJL>
__global__ __launch_bounds__(THREADS, 2) void split_kernel(
    const Tables* __restrict__ ktab, const uint8_t* __restrict__ kcodes, const float* __restrict__ knorms,
    const uint8_t* __restrict__ ksigns, const float* __restrict__ krn, int64_t kcap,
    const Tables* __restrict__ vtab, const uint8_t* __restrict__ vcodes, const float* __restrict__ vnorms,
    int64_t vcap, const int32_t* __restrict__ seq_lens, const float* __restrict__ q, float* __restrict__ parts,
    int hq, int hkv, int sink, int n_split, int64_t chunk, float qscale, float v_skip) {
  constexpr int KBYTES = 8 * (KLO + KHI);
  constexpr int VBYTES = 8 * (VLO + VHI);
  __shared__ uint32_t lutk[2][256];
  __shared__ uint32_t lutv[2][256];
  __shared__ uint32_t lutz[4];
  __shared__ float qraw[16][D];
  __shared__ float qrot[16][D];
  __shared__ float urot[QJL ? 16 : 1][D];
  __shared__ float qexp[16][2];
  __shared__ float mrg_m[WAVES][16];
  __shared__ float mrg_l[WAVES][16];
  __shared__ float mrg_acc[WAVES][16][D];

  const int split = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int G = hq / hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int64_t stream = static_cast<int64_t>(b) * hkv + kh;
  const int64_t L = seq_lens[b];
  const int64_t comp = L > sink ? L - sink : 0;
  const int64_t t_begin = static_cast<int64_t>(split) * chunk;
  const int64_t t_end = t_begin + chunk < comp ? t_begin + chunk : comp;

  const uint8_t* kbase = kcodes + stream * kcap * KBYTES;
  const uint8_t* vbase = vcodes + stream * vcap * VBYTES;
  const float* knb = knorms + stream * kcap;
  const float* vnb = vnorms + stream * vcap;
  const uint32_t* zb = QJL ? reinterpret_cast<const uint32_t*>(ksigns) + stream * kcap * (QJL_M / 32) : nullptr;
  const float* rnb = QJL ? krn + stream * kcap : nullptr;

  // First tile's loads go out before the query preparation below.
  TileRegs cur;
  int64_t t0 = t_begin + 32 * wave;
  if (t0 < t_end) load_tile<KLO, KHI, VLO, VHI, QJL>(cur, t0, n, j, kbase, vbase, knb, vnb, zb, rnb);

  // LUTs: entry e of width B = centroid(e & mask) | centroid(e >> B) << 16 (fp16 bits)
  for (int e = threadIdx.x; e < 256; e += THREADS) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int bk = hh ? KHI : KLO, bv = hh ? VHI : VLO;
      const int mk = (1 << bk) - 1, mv = (1 << bv) - 1;
      lutk[hh][e] = e < (1 << (2 * bk))
                        ? static_cast<uint32_t>(ktab->cen16[hh][e & mk]) | (static_cast<uint32_t>(ktab->cen16[hh][e >> bk]) << 16)
                        : 0u;
      lutv[hh][e] = e < (1 << (2 * bv))
                        ? static_cast<uint32_t>(vtab->cen16[hh][e & mv]) | (static_cast<uint32_t>(vtab->cen16[hh][e >> bv]) << 16)
                        : 0u;
    }
    if (e < 4) lutz[e] = ((e & 1) ? 0x3C00u : 0xBC00u) | (((e >> 1) & 1) ? 0x3C000000u : 0xBC000000u);
  }
  // ---- query preparation: qrot = Pi_K q * scale * log2(e); urot = S qrot.
  const float* qg = q + (static_cast<int64_t>(b) * hq + static_cast<int64_t>(kh) * G) * D;
  for (int idx = threadIdx.x; idx < G * D; idx += THREADS) qraw[idx / D][idx % D] = qg[idx];
  __syncthreads();
  // thread (i, hf): output coordinate i, inputs [64 hf, 64 hf + 64), all heads.
  // The thread's 64 matrix entries are loaded at once (one round trip), then
  // reused for every head.
  {
    const int i = threadIdx.x & (D - 1), hf = threadIdx.x >> 7;
    float w[64];
#pragma unroll
    for (int k = 0; k < 64; ++k) w[k] = ktab->pit[(64 * hf + k) * D + i];
    for (int g = 0; g < G; ++g) {
      const float4* qv4 = reinterpret_cast<const float4*>(&qraw[g][64 * hf]);
      float a = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float4 x = qv4[k];
        a = fmaf(w[4 * k], x.x, a);
        a = fmaf(w[4 * k + 1], x.y, a);
        a = fmaf(w[4 * k + 2], x.z, a);
        a = fmaf(w[4 * k + 3], x.w, a);
      }
      if (hf) qrot[g][i] = a;
      __syncthreads();
      if (!hf) qrot[g][i] = (qrot[g][i] + a) * qscale;
      __syncthreads();
    }
    if constexpr (QJL) {
#pragma unroll
      for (int k = 0; k < 64; ++k) w[k] = ktab->sit[(64 * hf + k) * D + i];
      for (int g = 0; g < G; ++g) {
        const float4* qv4 = reinterpret_cast<const float4*>(&qrot[g][64 * hf]);
        float a = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float4 x = qv4[k];
          a = fmaf(w[4 * k], x.x, a);
          a = fmaf(w[4 * k + 1], x.y, a);
          a = fmaf(w[4 * k + 2], x.z, a);
          a = fmaf(w[4 * k + 3], x.w, a);
        }
        if (hf) urot[g][i] = a;
        __syncthreads();
        if (!hf) urot[g][i] += a;
        __syncthreads();
      }
    }
  }
  // power-of-two scale per head so |value| * 2^sh < 2^14: fp16 hi + lo keeps ~22 bits
  for (int g = wave; g < G; g += WAVES) {
#pragma unroll
    for (int which = 0; which < (QJL ? 2 : 1); ++which) {
      const float* v = which ? urot[QJL ? g : 0] : qrot[g];
      float m = fmaxf(fabsf(v[lane]), fabsf(v[lane + 64]));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      int ex = 0;
      if (m > 0.0f) frexpf(m, &ex);
      if (lane == 0) qexp[g][which] = static_cast<float>(14 - ex);
    }
  }
  __syncthreads();

  // query fragments (B operand of the score MFMA): column n = query head n
  const bool head_ok = n < G;
  half8 qh[4], ql[4], uh[QJL ? 4 : 1], ul[QJL ? 4 : 1];
  float qinv = 0.0f, uinv = 0.0f;
  {
    const int g = head_ok ? n : 0;
    const int sq = static_cast<int>(qexp[g][0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = head_ok ? ldexpf(qrot[g][32 * j + 8 * ks + e], sq) : 0.0f;
        const _Float16 hv = static_cast<_Float16>(v);
        qh[ks][e] = hv;
        ql[ks][e] = static_cast<_Float16>(v - static_cast<float>(hv));
      }
    qinv = head_ok ? ldexpf(1.0f, -sq) : 0.0f;
    if constexpr (QJL) {
      const int su = static_cast<int>(qexp[g][1]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = head_ok ? ldexpf(urot[g][32 * j + 8 * ks + e], su) : 0.0f;
          const _Float16 hv = static_cast<_Float16>(v);
          uh[ks][e] = hv;
          ul[ks][e] = static_cast<_Float16>(v - static_cast<float>(hv));
        }
      uinv = head_ok ? ldexpf(QJL_C, -su) : 0.0f;
    }
  }

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{};

  for (; t0 < t_end; t0 += 32 * WAVES) {
    TileRegs nxt;
    const int64_t t1 = t0 + 32 * WAVES;
    if (t1 < t_end) load_tile<KLO, KHI, VLO, VHI, QJL>(nxt, t1, n, j, kbase, vbase, knb, vnb, zb, rnb);
    const int64_t tb = t0 + 8 * j;

    // ---- scores on MFMA: A = dequantized K (16 tokens x 32 coords), B = q~
    f32x4 sk[2], sz[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sk[mb] = f32x4{};
      sz[mb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        half8 a;
        if constexpr (KLO == KHI) a = dequant8<KLO>(cur.kw[mb], ks, lutk[0]);
        else a = j < 2 ? dequant8<KLO>(cur.kw[mb], ks, lutk[0]) : dequant8<KHI>(cur.kw[mb], ks, lutk[1]);
        sk[mb] = mfma16(a, qh[ks], sk[mb]);
        sk[mb] = mfma16(a, ql[ks], sk[mb]);
        if constexpr (QJL) {
          const uint32_t zv = (cur.zw[mb] >> (8 * ks)) & 0xFFu;
          const half8 z = as_half8(lutz[zv & 3], lutz[(zv >> 2) & 3], lutz[(zv >> 4) & 3], lutz[zv >> 6]);
          sz[mb] = mfma16(z, uh[ks], sz[mb]);
          sz[mb] = mfma16(z, ul[ks], sz[mb]);
        }
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
        if constexpr (QJL) dot = fmaf(f4get(cur.rn, e) * sz[mb][i], uinv, dot);
        s[e] = tb + e < t_end ? f4get(cur.kn, e) * dot : -INFINITY;
        tmax = fmaxf(tmax, s[e]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = m_run == -INFINITY ? 0.0f : exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.0f;
    uint32_t pw[4];
    bool any = false;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float p0 = exp2f(s[e] - m_new), p1 = exp2f(s[e + 1] - m_new);
      if (p0 < v_skip) p0 = 0.0f;
      if (p1 < v_skip) p1 = 0.0f;
      psum += p0 + p1;
      any |= (p0 > 0.0f) | (p1 > 0.0f);
      const float v0 = tb + e < t_end ? f4get(cur.vn, e) : 0.0f;
      const float v1 = tb + e + 1 < t_end ? f4get(cur.vn, e + 1) : 0.0f;
      const _Float16 h0 = static_cast<_Float16>(p0 * v0), h1 = static_cast<_Float16>(p1 * v1);
      pw[e >> 1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
                   (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
    }
    l_run = l_run * alpha + psum;
    // rescale the accumulator rows (query heads 4j + i) only when a maximum moved
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * j + i);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k][i] *= ai;
      }
    }
    // skip the value work of a tile whose weights all fell below v_skip
    if (__any(any && head_ok)) {
      const half8 pa = as_half8(pw[0], pw[1], pw[2], pw[3]);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        half8 bv;
        if constexpr (VLO == VHI) bv = dequant8<VLO>(cur.vw, nb, lutv[0]);
        else bv = n < 8 ? dequant8<VLO>(cur.vw, nb, lutv[0]) : dequant8<VHI>(cur.vw, nb, lutv[1]);
        acc[nb] = mfma16(pa, bv, acc[nb]);
      }
    }
    cur = nxt;
  }

  // ---- merge the 4 waves; l: sum over the 4 token lanes of a head.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (lane < 16) {
    mrg_m[wave][lane] = m_run;
    mrg_l[wave][lane] = l_run;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) mrg_acc[wave][4 * j + i][8 * n + nb] = acc[nb][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += THREADS) {
    const int g = idx / D, c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, mrg_m[w][g]);
    float a = 0.0f, l = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float f = mrg_m[w][g] == -INFINITY ? 0.0f : exp2f(mrg_m[w][g] - M);
        a = fmaf(f, mrg_acc[w][g][c], a);
        l = fmaf(f, mrg_l[w][g], l);
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
// combine: one block of 512 threads per (b, query head): log-sum-exp merge of
// the split partials and the raw sink tokens, one inverse rotation.  Thread
// (i, hf) handles coordinate i and a quarter hf of every reduction, so each
// thread has few, independent loads in flight.
constexpr int CT = 512;

__global__ __launch_bounds__(CT) void combine_kernel(const Tables* __restrict__ vtab, const float* __restrict__ q,
                                                     const uint16_t* __restrict__ sink_k,
                                                     const uint16_t* __restrict__ sink_v,
                                                     const int32_t* __restrict__ seq_lens,
                                                     const float* __restrict__ parts, float* __restrict__ out,
                                                     int hq, int hkv, int sink, int n_split, float qscale) {
  extern __shared__ float sm[];
  float* fs = sm;                 // [n_split] split maxima, then weights
  float* ls = fs + n_split;       // [n_split] split sums
  float* ssc = ls + n_split;      // [sink] sink scores, then weights
  __shared__ float qv[D];
  __shared__ float orot[4][D];
  __shared__ float obuf[4][D];
  __shared__ float red[16];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = bh / hq, h = bh % hq, kh = h / (hq / hkv);
  const int64_t L = seq_lens[b];
  const int ns = static_cast<int>(L < sink ? L : sink);
  const float* pp = parts + static_cast<int64_t>(bh) * n_split * PART;
  if (tid < D) qv[tid] = q[static_cast<int64_t>(bh) * D + tid] * qscale;
  float mloc = -INFINITY;
  for (int sp = tid; sp < n_split; sp += CT) {
    const float m = pp[sp * PART], l = pp[sp * PART + 1];
    fs[sp] = m;
    ls[sp] = l;
    if (l > 0.0f) mloc = fmaxf(mloc, m);
  }
  __syncthreads();
  const uint16_t* sk = sink_k + (static_cast<int64_t>(b) * hkv + kh) * sink * D;
  const uint16_t* sv = sink_v + (static_cast<int64_t>(b) * hkv + kh) * sink * D;
  for (int t = tid; t < ns; t += CT) {
    const uint4* row = reinterpret_cast<const uint4*>(sk + static_cast<int64_t>(t) * D);
    float dot = 0.0f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const uint4 w = row[c];
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dot = fmaf(__uint_as_float(u[k] << 16), qv[8 * c + 2 * k], dot);
        dot = fmaf(__uint_as_float(u[k] & 0xFFFF0000u), qv[8 * c + 2 * k + 1], dot);
      }
    }
    ssc[t] = dot;
    mloc = fmaxf(mloc, dot);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
  if (lane == 0) red[wave] = mloc;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < CT / 64; ++w) M = fmaxf(M, red[w]);
  float lloc = 0.0f;
  for (int sp = tid; sp < n_split; sp += CT) {
    const float f = (ls[sp] > 0.0f && M != -INFINITY) ? exp2f(fs[sp] - M) : 0.0f;
    fs[sp] = f;
    lloc = fmaf(f, ls[sp], lloc);
  }
  for (int t = tid; t < ns; t += CT) {
    const float w = exp2f(ssc[t] - M);
    ssc[t] = w;
    lloc += w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lloc += __shfl_xor(lloc, o);
  __syncthreads();
  if (lane == 0) red[8 + wave] = lloc;
  const int i = tid & (D - 1), hf = tid >> 7;
  float a = 0.0f;
#pragma unroll 4
  for (int sp = hf; sp < n_split; sp += 4) a = fmaf(fs[sp], pp[sp * PART + 4 + i], a);
  orot[hf][i] = a;
  __syncthreads();
  float Lsum = 0.0f;
#pragma unroll
  for (int w = 0; w < CT / 64; ++w) Lsum += red[8 + w];
  // one inverse rotation: out_i = sum_c Pi[c][i] orot[c] (+ raw sink values)
  float o = 0.0f;
#pragma unroll
  for (int cc = 32 * hf; cc < 32 * hf + 32; ++cc)
    o = fmaf(vtab->pi[cc * D + i], orot[0][cc] + orot[1][cc] + orot[2][cc] + orot[3][cc], o);
  for (int t = hf; t < ns; t += 4)
    o = fmaf(ssc[t], __uint_as_float(static_cast<uint32_t>(sv[static_cast<int64_t>(t) * D + i]) << 16), o);
  obuf[hf][i] = o;
  __syncthreads();
  if (tid < D) {
    const float v = obuf[0][tid] + obuf[1][tid] + obuf[2][tid] + obuf[3][tid];
    out[static_cast<int64_t>(bh) * D + tid] = Lsum > 0.0f ? v / Lsum : 0.0f;
  }
}

template <int KLO, int KHI, int VLO, int VHI, bool QJL>
hipError_t launch_split(const Tables* ktab, const tq_cache& kc, const Tables* vtab, const tq_cache& vc,
                        const tq_attn& a, const AttendPlan& plan, const int32_t* seq_lens, const float* q,
                        float* parts, hipStream_t st) {
  hipLaunchKernelGGL((split_kernel<KLO, KHI, VLO, VHI, QJL>), dim3(plan.n_split, a.hkv, a.batch), dim3(THREADS), 0,
                     st, ktab, kc.codes, kc.norms, kc.qjl_signs, kc.qjl_rnorms, kc.cap, vtab, vc.codes, vc.norms,
                     vc.cap, seq_lens, q, parts, a.hq, a.hkv, a.sink, plan.n_split, plan.chunk, a.scale * LOG2E,
                     a.v_skip);
  return hipGetLastError();
}

template <int KLO, int KHI>
hipError_t dispatch_v(int vkey, bool qjl, const Tables* ktab, const tq_cache& kc, const Tables* vtab,
                      const tq_cache& vc, const tq_attn& a, const AttendPlan& plan, const int32_t* sl,
                      const float* q, float* parts, hipStream_t st) {
#define TQ_V(VL, VH)                                                                                  \
  case VL * 10 + VH:                                                                                  \
    return qjl ? launch_split<KLO, KHI, VL, VH, true>(ktab, kc, vtab, vc, a, plan, sl, q, parts, st)  \
               : launch_split<KLO, KHI, VL, VH, false>(ktab, kc, vtab, vc, a, plan, sl, q, parts, st);
  switch (vkey) {
    TQ_V(2, 2)
    TQ_V(3, 3)
    TQ_V(4, 4)
    TQ_V(4, 3)
    TQ_V(3, 2)
    default: return hipErrorInvalidValue;
  }
#undef TQ_V
}

}  // namespace

AttendPlan plan_attend(const tq_attn& a) {
  AttendPlan p{};
  const int64_t streams = static_cast<int64_t>(a.batch) * a.hkv;
  const int64_t comp = a.max_len > a.sink ? a.max_len - a.sink : 0;
  const int64_t tiles = (comp + TILE - 1) / TILE;
  int64_t ns = streams > 0 ? (512 + streams - 1) / streams : 1;
  if (comp >= 16384 && ns < 4) ns = 4;
  const int64_t cap_ns = (tiles + WAVES - 1) / WAVES;  // at least one tile per wave
  if (ns > cap_ns) ns = cap_ns;
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
  const int64_t heads = static_cast<int64_t>(a.batch) * a.hq;
  float* parts = static_cast<float*>(workspace);
  const int vkey = vs.bits_lo * 10 + vs.bits_hi;
  const bool qjl = ks.qjl_m != 0;
  hipError_t e;
  switch (ks.bits_lo * 10 + ks.bits_hi) {
    case 22: e = dispatch_v<2, 2>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, q, parts, st); break;
    case 33: e = dispatch_v<3, 3>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, q, parts, st); break;
    case 44: e = dispatch_v<4, 4>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, q, parts, st); break;
    case 43: e = dispatch_v<4, 3>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, q, parts, st); break;
    case 32: e = dispatch_v<3, 2>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, q, parts, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const size_t smem = (2 * static_cast<size_t>(plan.n_split) + static_cast<size_t>(a.sink)) * sizeof(float);
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>(heads)), dim3(CT), smem, st, vtab, q, sink_k, sink_v,
                     seq_lens, parts, out, a.hq, a.hkv, a.sink, plan.n_split, a.scale * LOG2E);
  return hipGetLastError();
}

}  // namespace tq
