// Decode attention read directly from the packed cache.
//
// noze.it, "TurboQuant-MLX: quantizzare pesi e KV cache per LLM open-weight su
// Mac", section "Il metodo TurboQuant, in breve": inner products are taken
// against the codebook reconstruction, corrected by the 1-bit residual sketch
// when present.  GitHub issue "Greetings from TurboQuant-MLX & Some Insights
// to Share!": item 1 (the first ~128 tokens stay uncompressed) and item 3
// (value dequantization is skipped when the attention weight is below 1e-6).
//
// Three launches on one stream:
//  prep    q~ = Pi_K q (times scale*log2 e) and u = S q~, per query head,
//          stored with a power-of-two scale so they split into fp16 hi + lo;
//  split   one workgroup (4 waves) per (split, kv head, sequence); each wave
//          streams 32-token tiles: K records -> LUT dequantization in
//          registers -> scores on MFMA for all query heads of the group ->
//          online softmax -> V tiles (token-major sub-blocks) -> P V on MFMA
//          in the rotated domain; the 4 waves merge in LDS and write one
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

// ---------------------------------------------------------------------------
// prep: one block of 128 threads per (b, query head).
__global__ __launch_bounds__(128) void prep_kernel(const Tables* __restrict__ ktab, const float* __restrict__ q,
                                                   float* __restrict__ qs, float* __restrict__ qexp,
                                                   float scale, int qjl) {
  __shared__ float qv[D];
  __shared__ float qr[D];
  __shared__ float red[4];
  const int bh = blockIdx.x, i = threadIdx.x;
  qv[i] = q[static_cast<int64_t>(bh) * D + i];
  __syncthreads();
  float acc = 0.0f;
  for (int j = 0; j < D; ++j) acc = fmaf(ktab->pi[i * D + j], qv[j], acc);
  acc *= scale * LOG2E;
  qr[i] = acc;
  // power-of-two scale so that max |value| lands in [2^13, 2^14)
  auto pow2_scale = [&](float v, int slot) {
    float m = fabsf(v);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((i & 63) == 0) red[i >> 6] = m;
    __syncthreads();
    const float mx = fmaxf(red[0], red[1]);
    __syncthreads();
    int ex = 0;
    if (mx > 0.0f) frexpf(mx, &ex);
    const int sh = 14 - ex;
    if (i == 0) qexp[static_cast<int64_t>(bh) * 4 + slot] = ldexpf(1.0f, -sh);
    return sh;
  };
  const int sq = pow2_scale(acc, 0);
  qs[static_cast<int64_t>(bh) * 2 * D + i] = ldexpf(acc, sq);
  if (qjl) {
    __syncthreads();
    float u = 0.0f;
    for (int j = 0; j < D; ++j) u = fmaf(ktab->s[i * D + j], qr[j], u);
    const int su = pow2_scale(u, 1);
    qs[static_cast<int64_t>(bh) * 2 * D + D + i] = ldexpf(u, su);
  }
}

// Load this lane's q~ (or u) fragment for k-steps 0..3: head n (0 if n >= G),
// coordinates 32j + 8ks + e, split into fp16 hi + lo.
__device__ __forceinline__ void load_qfrag(const float* qsrc, bool ok, int j, half8 (&hi)[4], half8 (&lo)[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = ok ? qsrc[32 * j + 8 * ks + e] : 0.0f;
      const _Float16 h = static_cast<_Float16>(v);
      hi[ks][e] = h;
      lo[ks][e] = static_cast<_Float16>(v - static_cast<float>(h));
    }
}

template <int KLO, int KHI, int VLO, int VHI, bool QJL>
__global__ __launch_bounds__(THREADS) void split_kernel(
    const Tables* __restrict__ ktab, const uint8_t* __restrict__ kcodes, const float* __restrict__ knorms,
    const uint8_t* __restrict__ ksigns, const float* __restrict__ krn, int64_t kcap,
    const Tables* __restrict__ vtab, const uint8_t* __restrict__ vcodes, const float* __restrict__ vnorms,
    int64_t vcap, const int32_t* __restrict__ seq_lens, const float* __restrict__ qs,
    const float* __restrict__ qexp, float* __restrict__ parts, int hq, int hkv, int sink, int n_split,
    int64_t chunk, float v_skip) {
  constexpr int KBYTES = 8 * (KLO + KHI);
  constexpr int VBYTES = 8 * (VLO + VHI);
  constexpr int VG = 64 * (VLO + VHI);  // bytes of one 8-token group of a V tile
  __shared__ uint32_t lutk[2][256];
  __shared__ uint32_t lutv[2][256];
  __shared__ uint32_t lutz[4];
  __shared__ float mrg_m[WAVES][16];
  __shared__ float mrg_l[WAVES][16];
  __shared__ float mrg_acc[WAVES][16][D];

  const int split = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int G = hq / hkv;
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
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int64_t stream = static_cast<int64_t>(b) * hkv + kh;
  const int64_t L = seq_lens[b];
  const int64_t comp = L > sink ? L - sink : 0;
  const int64_t t_begin = static_cast<int64_t>(split) * chunk;
  const int64_t t_end = t_begin + chunk < comp ? t_begin + chunk : comp;

  // query fragments (B operand of the score MFMA): column n = query head
  const int64_t qh_idx = static_cast<int64_t>(b) * hq + static_cast<int64_t>(kh) * G + n;
  const bool head_ok = n < G;
  half8 qh[4], ql[4], uh[QJL ? 4 : 1], ul[QJL ? 4 : 1];
  const float* qsrc = qs + (head_ok ? qh_idx : 0) * 2 * D;
  load_qfrag(qsrc, head_ok, j, qh, ql);
  float qinv = head_ok ? qexp[qh_idx * 4 + 0] : 0.0f;
  float uinv = 0.0f;
  if constexpr (QJL) {
    load_qfrag(qsrc + D, head_ok, j, uh, ul);
    uinv = head_ok ? qexp[qh_idx * 4 + 1] * (1.2533141373155003f / QJL_M) : 0.0f;  // sqrt(pi/2)/m
  }

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{};

  const uint8_t* kbase = kcodes + stream * kcap * KBYTES;
  const uint8_t* vbase = vcodes + stream * vcap * VBYTES;
  const float* knb = knorms + stream * kcap;
  const float* vnb = vnorms + stream * vcap;

  for (int64_t t0 = t_begin + 32 * wave; t0 < t_end; t0 += 32 * WAVES) {
    // ---- K: lane (rho = n, j) loads chunk j of the record of token slot
    // mu(mb, rho) = 8(rho/4) + 4mb + rho%4 for M-blocks mb = 0, 1.
    uint32_t kw[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int slot = 8 * (n >> 2) + 4 * mb + (n & 3);
      const int64_t tok = t0 + slot;
      const uint8_t* rec = kbase + (tok < t_end ? tok : t0) * KBYTES;
      if (j < 2) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(rec + 4 * KLO * j);
#pragma unroll
        for (int w = 0; w < KLO; ++w) kw[mb][w] = p[w];
      } else {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(rec + 8 * KLO + 4 * KHI * (j - 2));
#pragma unroll
        for (int w = 0; w < KHI; ++w) kw[mb][w] = p[w];
      }
    }
    uint32_t zw[2];
    if constexpr (QJL) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int slot = 8 * (n >> 2) + 4 * mb + (n & 3);
        const int64_t tok = t0 + slot;
        zw[mb] = reinterpret_cast<const uint32_t*>(ksigns + ((stream * kcap) + (tok < t_end ? tok : t0)) * (QJL_M / 8))[j];
      }
    }
    // ---- V: lane (n, j) loads sub-block (g = j, q = n) of the tile.
    uint32_t vw[8];
    {
      const uint8_t* tile = vbase + (t0 / TILE) * (TILE * VBYTES) + j * VG;
      if (n < 8) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(tile + 8 * VLO * n);
#pragma unroll
        for (int w = 0; w < 2 * VLO; ++w) vw[w] = p[w];
      } else {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(tile + 64 * VLO + 8 * VHI * (n - 8));
#pragma unroll
        for (int w = 0; w < 2 * VHI; ++w) vw[w] = p[w];
      }
    }
    // norms of tokens 8j + e (score layout: lane (head n, j) holds tokens 8j + 4mb + i)
    float kn[8], vn[8], rn[8];
    const int64_t tb = t0 + 8 * j;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = tb + e < t_end;
      kn[e] = ok ? knb[tb + e] : 0.0f;
      vn[e] = ok ? vnb[tb + e] : 0.0f;
      if constexpr (QJL) rn[e] = ok ? krn[stream * kcap + tb + e] : 0.0f;
    }

    // ---- scores on MFMA: A = dequantized K (16 tokens x 32 coords), B = q~
    f32x4 sk[2], sz[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sk[mb] = f32x4{};
      sz[mb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        half8 a;
        if constexpr (KLO == KHI) a = dequant8<KLO>(kw[mb], ks, lutk[0]);
        else a = j < 2 ? dequant8<KLO>(kw[mb], ks, lutk[0]) : dequant8<KHI>(kw[mb], ks, lutk[1]);
        sk[mb] = mfma16(a, qh[ks], sk[mb]);
        sk[mb] = mfma16(a, ql[ks], sk[mb]);
        if constexpr (QJL) {
          const uint32_t zb = (zw[mb] >> (8 * ks)) & 0xFFu;
          const half8 z = as_half8(lutz[zb & 3], lutz[(zb >> 2) & 3], lutz[(zb >> 4) & 3], lutz[zb >> 6]);
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
        if constexpr (QJL) dot = fmaf(rn[e] * sz[mb][i], uinv, dot);
        s[e] = tb + e < t_end ? kn[e] * dot : -INFINITY;
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
      const _Float16 h0 = static_cast<_Float16>(p0 * vn[e]), h1 = static_cast<_Float16>(p1 * vn[e + 1]);
      pw[e >> 1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
                   (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
    }
    l_run = l_run * alpha + psum;
    // rescale the accumulator rows (query heads 4j + i) by their alpha
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, 4 * j + i);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k][i] *= ai;
    }
    // skip the value work of a tile whose weights all fell below v_skip
    if (__any(any && head_ok)) {
      const half8 pa = as_half8(pw[0], pw[1], pw[2], pw[3]);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        half8 bv;
        if constexpr (VLO == VHI) bv = dequant8<VLO>(vw, nb, lutv[0]);
        else bv = n < 8 ? dequant8<VLO>(vw, nb, lutv[0]) : dequant8<VHI>(vw, nb, lutv[1]);
        acc[nb] = mfma16(pa, bv, acc[nb]);
      }
    }
  }

  // ---- merge the 4 waves.  l: sum over the 4 token lanes of a head.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (lane < 16) {
    mrg_m[wave][lane] = m_run;
    mrg_l[wave][lane] = l_run;
  }
  // acc[nb][i]: query head 4j + i, coordinate 8n + nb
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
// combine: one block of 128 threads per (b, query head).
__global__ __launch_bounds__(128) void combine_kernel(const Tables* __restrict__ vtab, const float* __restrict__ q,
                                                      const uint16_t* __restrict__ sink_k,
                                                      const uint16_t* __restrict__ sink_v,
                                                      const int32_t* __restrict__ seq_lens,
                                                      const float* __restrict__ parts, float* __restrict__ out,
                                                      int hq, int hkv, int sink, int n_split, float scale) {
  extern __shared__ float sm[];
  float* orot = sm;            // [D]
  float* qv = sm + D;          // [D]
  float* ssc = sm + 2 * D;     // [sink] sink scores, then weights
  __shared__ float red[2];
  const int bh = blockIdx.x, i = threadIdx.x;
  const int b = bh / hq, h = bh % hq, kh = h / (hq / hkv);
  const int64_t L = seq_lens[b];
  const int ns = static_cast<int>(L < sink ? L : sink);
  const float* pp = parts + static_cast<int64_t>(bh) * n_split * PART;
  qv[i] = q[static_cast<int64_t>(bh) * D + i] * (scale * LOG2E);
  // global maximum over splits and sink scores
  float M = -INFINITY;
  for (int sp = 0; sp < n_split; ++sp)
    if (pp[sp * PART + 1] > 0.0f) M = fmaxf(M, pp[sp * PART]);
  __syncthreads();
  const uint16_t* sk = sink_k + (static_cast<int64_t>(b) * hkv + kh) * sink * D;
  const uint16_t* sv = sink_v + (static_cast<int64_t>(b) * hkv + kh) * sink * D;
  float smax = -INFINITY;
  for (int t = i; t < ns; t += 128) {
    float dot = 0.0f;
    for (int c = 0; c < D; ++c) dot = fmaf(__uint_as_float(static_cast<uint32_t>(sk[t * D + c]) << 16), qv[c], dot);
    ssc[t] = dot;
    smax = fmaxf(smax, dot);
  }
  for (int o = 32; o > 0; o >>= 1) smax = fmaxf(smax, __shfl_xor(smax, o));
  if ((i & 63) == 0) red[i >> 6] = smax;
  __syncthreads();
  M = fmaxf(M, fmaxf(red[0], red[1]));
  // merged rotated accumulator and total weight
  float a = 0.0f, l = 0.0f;
  if (M != -INFINITY) {
    for (int sp = 0; sp < n_split; ++sp) {
      const float lp = pp[sp * PART + 1];
      if (lp > 0.0f) {
        const float f = exp2f(pp[sp * PART] - M);
        a = fmaf(f, pp[sp * PART + 4 + i], a);
        l = fmaf(f, lp, l);
      }
    }
  }
  orot[i] = a;
  __syncthreads();
  for (int t = i; t < ns; t += 128) ssc[t] = exp2f(ssc[t] - M);
  __syncthreads();
  for (int t = 0; t < ns; ++t) l += ssc[t];
  // one inverse rotation: out_i = sum_c Pi[c][i] orot[c]
  float o = 0.0f;
  for (int c = 0; c < D; ++c) o = fmaf(vtab->pi[c * D + i], orot[c], o);
  for (int t = 0; t < ns; ++t) o = fmaf(ssc[t], __uint_as_float(static_cast<uint32_t>(sv[t * D + i]) << 16), o);
  out[static_cast<int64_t>(bh) * D + i] = l > 0.0f ? o / l : 0.0f;
}

template <int KLO, int KHI, int VLO, int VHI, bool QJL>
hipError_t launch_split(const Tables* ktab, const tq_cache& kc, const Tables* vtab, const tq_cache& vc,
                        const tq_attn& a, const AttendPlan& plan, const int32_t* seq_lens, const float* qs,
                        const float* qexp, float* parts, hipStream_t st) {
  hipLaunchKernelGGL((split_kernel<KLO, KHI, VLO, VHI, QJL>), dim3(plan.n_split, a.hkv, a.batch), dim3(THREADS), 0,
                     st, ktab, kc.codes, kc.norms, kc.qjl_signs, kc.qjl_rnorms, kc.cap, vtab, vc.codes, vc.norms,
                     vc.cap, seq_lens, qs, qexp, parts, a.hq, a.hkv, a.sink, plan.n_split, plan.chunk, a.v_skip);
  return hipGetLastError();
}

template <int KLO, int KHI>
hipError_t dispatch_v(int vkey, bool qjl, const Tables* ktab, const tq_cache& kc, const Tables* vtab,
                      const tq_cache& vc, const tq_attn& a, const AttendPlan& plan, const int32_t* sl,
                      const float* qs, const float* qe, float* parts, hipStream_t st) {
#define TQ_V(VL, VH)                                                                                        \
  case VL * 10 + VH:                                                                                        \
    return qjl ? launch_split<KLO, KHI, VL, VH, true>(ktab, kc, vtab, vc, a, plan, sl, qs, qe, parts, st)  \
               : launch_split<KLO, KHI, VL, VH, false>(ktab, kc, vtab, vc, a, plan, sl, qs, qe, parts, st);
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
  p.ws_bytes = static_cast<size_t>(heads) * (2 * D + 4 + static_cast<int64_t>(p.n_split) * PART) * sizeof(float);
  return p;
}

hipError_t launch_attend(const Spec& ks, const Tables* ktab, const tq_cache& kc, const Spec& vs, const Tables* vtab,
                         const tq_cache& vc, const tq_attn& a, const AttendPlan& plan, const float* q,
                         const uint16_t* sink_k, const uint16_t* sink_v, const int32_t* seq_lens, float* out,
                         void* workspace, hipStream_t st) {
  const int64_t heads = static_cast<int64_t>(a.batch) * a.hq;
  float* qs = static_cast<float*>(workspace);
  float* qexp = qs + heads * 2 * D;
  float* parts = qexp + heads * 4;
  hipLaunchKernelGGL(prep_kernel, dim3(static_cast<unsigned>(heads)), dim3(128), 0, st, ktab, q, qs, qexp, a.scale,
                     ks.qjl_m ? 1 : 0);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int vkey = vs.bits_lo * 10 + vs.bits_hi;
  const bool qjl = ks.qjl_m != 0;
  hipError_t e;
  switch (ks.bits_lo * 10 + ks.bits_hi) {
    case 22: e = dispatch_v<2, 2>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, qs, qexp, parts, st); break;
    case 33: e = dispatch_v<3, 3>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, qs, qexp, parts, st); break;
    case 44: e = dispatch_v<4, 4>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, qs, qexp, parts, st); break;
    case 43: e = dispatch_v<4, 3>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, qs, qexp, parts, st); break;
    case 32: e = dispatch_v<3, 2>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, qs, qexp, parts, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const size_t smem = (2 * D + static_cast<size_t>(a.sink)) * sizeof(float);
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>(heads)), dim3(128), smem, st, vtab, q, sink_k, sink_v,
                     seq_lens, parts, out, a.hq, a.hkv, a.sink, plan.n_split, a.scale);
  return hipGetLastError();
}

}  // namespace tq
