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
//  prep    one workgroup per (sequence, query head): q~ = Pi_K q (times
//          scale*log2 e) and u = S q~, scaled by a power of two and split
//          into fp16 hi + lo, written in exactly the register layout the
//          split kernel's MFMA reads;
//  split   one workgroup (8 waves) per (split, kv head, sequence).  Each wave
//          streams 32-token tiles with two tiles prefetched into registers:
//          K records -> LUT dequantization -> scores on MFMA for all query
//          heads of the group -> online softmax -> V tiles (coordinate-major
//          sub-blocks) -> P V on MFMA in the rotated domain.  The waves merge
//          in LDS and write one partial (m, l, acc[128]) per query head;
//  combine per query head: log-sum-exp merge of the splits and the raw bf16
//          sink tokens, one inverse rotation Pi_V^T, normalisation.
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
constexpr float LOG2E = 1.4426950408889634f;
constexpr float QJL_C = 1.2533141373155003f / QJL_M;  // sqrt(pi/2) / m
// prep output per kv stream: q fragments [4 ks][hi, lo][64 lanes] uint4,
// u fragments likewise, then qinv[16], uinv[16]
constexpr int PREP_FRAG = 4 * 2 * 64 * 16;
constexpr int PREP_BYTES = 2 * PREP_FRAG + 128;

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

// ---------------------------------------------------------------------------
// prep: one block of 256 threads per (sequence, query head).  Thread (i, hf)
// produces rotated coordinate i from inputs [64 hf, 64 hf + 64); every load
// it needs (its slice of the transposed rotation and sketch, the query) is
// issued before any arithmetic.
__global__ __launch_bounds__(256) void prep_kernel(const Tables* __restrict__ ktab, const float* __restrict__ q,
                                                   uint8_t* __restrict__ prep, int hq, int hkv, float qscale,
                                                   int qjl) {
  __shared__ float qraw[D];
  __shared__ float part[2][D];
  __shared__ float qrot[D];
  __shared__ float urot[D];
  __shared__ int shx[2];
  const int bh = blockIdx.x, b = bh / hq, h = bh % hq, G = hq / hkv, kh = h / G, n = h % G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = tid & (D - 1), hf = tid >> 7;
  float w[64], ws[64];
#pragma unroll
  for (int k = 0; k < 64; ++k) w[k] = ktab->pit[(64 * hf + k) * D + i];
  if (qjl) {
#pragma unroll
    for (int k = 0; k < 64; ++k) ws[k] = ktab->sit[(64 * hf + k) * D + i];
  }
  if (tid < D) qraw[tid] = q[static_cast<int64_t>(bh) * D + tid];
  __syncthreads();
  auto dot64 = [&](const float (&m)[64], const float* src) {
    const float4* v4 = reinterpret_cast<const float4*>(src + 64 * hf);
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float4 x = v4[k];
      a = fmaf(m[4 * k], x.x, a);
      a = fmaf(m[4 * k + 1], x.y, a);
      a = fmaf(m[4 * k + 2], x.z, a);
      a = fmaf(m[4 * k + 3], x.w, a);
    }
    return a;
  };
  part[hf][i] = dot64(w, qraw);
  __syncthreads();
  if (tid < D) qrot[tid] = (part[0][tid] + part[1][tid]) * qscale;
  __syncthreads();
  if (qjl) {
    part[hf][i] = dot64(ws, qrot);
    __syncthreads();
    if (tid < D) urot[tid] = part[0][tid] + part[1][tid];
    __syncthreads();
  }
  // power-of-two scale so that |value| * 2^sh < 2^14 (wave 0: q~, wave 1: u)
  if (wave < (qjl ? 2 : 1)) {
    const float* v = wave ? urot : qrot;
    float m = fmaxf(fabsf(v[lane]), fabsf(v[lane + 64]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    int ex = 0;
    if (m > 0.0f) frexpf(m, &ex);
    if (lane == 0) shx[wave] = 14 - ex;
  }
  __syncthreads();
  // fragments of lanes l with l & 15 == n: (ks, hilo, j) -> lane l = 16 j + n,
  // coordinates 32 j + 8 ks + e
  uint8_t* dst = prep + (static_cast<int64_t>(b) * hkv + kh) * PREP_BYTES;
  if (tid < (qjl ? 64 : 32)) {
    const int which = tid >> 5, c = tid & 31, ks = c >> 3, hl = (c >> 2) & 1, j = c & 3;
    const float* v = which ? urot : qrot;
    const int sh = shx[which];
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      _Float16 hv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float x = ldexpf(v[32 * j + 8 * ks + e + u], sh);
        const _Float16 hi = static_cast<_Float16>(x);
        hv[u] = hl ? static_cast<_Float16>(x - static_cast<float>(hi)) : hi;
      }
      wv[e >> 1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hv[0])) |
                   (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hv[1])) << 16);
    }
    reinterpret_cast<uint4*>(dst + which * PREP_FRAG)[(ks * 2 + hl) * 64 + 16 * j + n] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
  if (tid == 64) {
    float* inv = reinterpret_cast<float*>(dst + 2 * PREP_FRAG);
    inv[n] = ldexpf(1.0f, -shx[0]);
    inv[16 + n] = qjl ? ldexpf(QJL_C, -shx[1]) : 0.0f;
  }
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
    int64_t vcap, const int32_t* __restrict__ seq_lens, const uint8_t* __restrict__ prep,
    float* __restrict__ parts, int hq, int hkv, int sink, int n_split, int64_t chunk, float v_skip) {
  using LP = LutPlan<KLO, KHI, VLO, VHI>;
  constexpr int KBYTES = 8 * (KLO + KHI);
  constexpr int VBYTES = 8 * (VLO + VHI);
  constexpr int MRG = SW * 16 * (D + 2) * 4;
  constexpr int SMEM = LP::bytes > MRG ? LP::bytes : MRG;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ uint32_t lutz[4];

  const int split = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
  const int G = hq / hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

  // First tile's loads go out before the LUT build.
  TileRegs cur;
  uint32_t t0 = t_begin + 32 * wave;
  if (t0 < t_end) load_tile<KLO, KHI, VLO, VHI, QJL>(cur, t0, n, j, kbase, vbase, knb, vnb, zb, rnb);

  // query fragments from the prep kernel
  const uint8_t* pq = prep + stream * PREP_BYTES;
  half8 qh[4], ql[4], uh[QJL ? 4 : 1], ul[QJL ? 4 : 1];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qh[ks] = __builtin_bit_cast(half8, reinterpret_cast<const uint4*>(pq)[(ks * 2 + 0) * 64 + lane]);
    ql[ks] = __builtin_bit_cast(half8, reinterpret_cast<const uint4*>(pq)[(ks * 2 + 1) * 64 + lane]);
    if constexpr (QJL) {
      uh[ks] = __builtin_bit_cast(half8, reinterpret_cast<const uint4*>(pq + PREP_FRAG)[(ks * 2 + 0) * 64 + lane]);
      ul[ks] = __builtin_bit_cast(half8, reinterpret_cast<const uint4*>(pq + PREP_FRAG)[(ks * 2 + 1) * 64 + lane]);
    }
  }
  const bool head_ok = n < G;
  if (!head_ok) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qh[ks] = ql[ks] = half8{};
      if constexpr (QJL) uh[ks] = ul[ks] = half8{};
    }
  }
  const float qinv = head_ok ? reinterpret_cast<const float*>(pq + 2 * PREP_FRAG)[n] : 0.0f;
  const float uinv = (QJL && head_ok) ? reinterpret_cast<const float*>(pq + 2 * PREP_FRAG)[16 + n] : 0.0f;

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
  const uint8_t* lut_klo = smem + LP::template off<KLO>();
  const uint8_t* lut_khi = smem + LP::template off<KHI>();
  const uint8_t* lut_vlo = smem + LP::template off<VLO>();
  const uint8_t* lut_vhi = smem + LP::template off<VHI>();

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{};

  auto tile_step = [&]<bool FULL>(const TileRegs& tr, uint32_t t0c) {
    const int nvalid = FULL ? 8 : static_cast<int>(t_end) - static_cast<int>(t0c + 8 * j);
    // four independent accumulator chains (M-block x hi/lo) keep the matrix
    // pipe busy; hi and lo partial dots are added afterwards
    f32x4 sk[2], sl[2], sz[2], szl[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) sk[mb] = sl[mb] = sz[mb] = szl[mb] = f32x4{};
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
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) sl[mb] = mfma16(a[mb], ql[ks], sl[mb]);
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
        for (int mb = 0; mb < 2; ++mb) szl[mb] = mfma16(z[mb], ul[ks], szl[mb]);
      }
    }
    float s[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * mb + i;
        float dot = (sk[mb][i] + sl[mb][i]) * qinv;
        if constexpr (QJL) dot = fmaf(f4get(tr.rn, e) * (sz[mb][i] + szl[mb][i]), uinv, dot);
        s[e] = f4get(tr.kn, e) * dot;
        if constexpr (!FULL) s[e] = e < nvalid ? s[e] : -INFINITY;
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
      float v0 = f4get(tr.vn, e), v1 = f4get(tr.vn, e + 1);
      if constexpr (!FULL) {
        v0 = e < nvalid ? v0 : 0.0f;
        v1 = e + 1 < nvalid ? v1 : 0.0f;
      }
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
        if constexpr (VLO == VHI) bv = dequant8<VLO>(tr.vw, nb, lut_vlo, lane4);
        else bv = n < 8 ? dequant8<VLO>(tr.vw, nb, lut_vlo, lane4) : dequant8<VHI>(tr.vw, nb, lut_vhi, lane4);
        acc[nb] = mfma16(pa, bv, acc[nb]);
      }
    }
  };

  // Tiles in flight per wave: three where the registers allow it (the
  // buffers rotate through fixed roles), else two.
  constexpr uint32_t STEP = 32 * SW;
  constexpr int DEPTH = (!QJL && KLO == KHI && VLO == VHI) ? 3 : 2;
  auto run = [&](TileRegs& compute, TileRegs& refill, uint32_t ahead) -> bool {
    if (t0 >= t_end) return false;
    if (t0 + ahead < t_end) load_tile<KLO, KHI, VLO, VHI, QJL>(refill, t0 + ahead, n, j, kbase, vbase, knb, vnb, zb, rnb);
    if (t0 + 32 <= t_end) tile_step.template operator()<true>(compute, t0);
    else tile_step.template operator()<false>(compute, t0);
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
        const float f = mw == -INFINITY ? 0.0f : exp2f(mw - M);
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
// combine: one block of 512 threads per (b, query head): log-sum-exp merge of
// the split partials and the raw sink tokens, one inverse rotation.  Thread
// (i, hf) handles coordinate i and a quarter hf of every reduction; its
// loads of the rotation column and of the first partials go out first.
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
  const int i = tid & (D - 1), hf = tid >> 7;
  const int64_t L = seq_lens[b];
  const int ns = static_cast<int>(L < sink ? L : sink);
  const float* pp = parts + static_cast<int64_t>(bh) * n_split * PART;
  // independent loads first: rotation column slice and the first partials
  float pic[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) pic[k] = vtab->pi[(32 * hf + k) * D + i];
  constexpr int PF = 8;
  float pa[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    const int sp = hf + 4 * k;
    pa[k] = sp < n_split ? pp[sp * PART + 4 + i] : 0.0f;
  }
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
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < PF; ++k) a = fmaf(hf + 4 * k < n_split ? fs[hf + 4 * k] : 0.0f, pa[k], a);
  for (int sp = hf + 4 * PF; sp < n_split; sp += 4) a = fmaf(fs[sp], pp[sp * PART + 4 + i], a);
  orot[hf][i] = a;
  __syncthreads();
  float Lsum = 0.0f;
#pragma unroll
  for (int w = 0; w < CT / 64; ++w) Lsum += red[8 + w];
  // one inverse rotation: out_i = sum_c Pi[c][i] orot[c] (+ raw sink values)
  float o = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int cc = 32 * hf + k;
    o = fmaf(pic[k], orot[0][cc] + orot[1][cc] + orot[2][cc] + orot[3][cc], o);
  }
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
                        const tq_attn& a, const AttendPlan& plan, const int32_t* seq_lens, const uint8_t* prep,
                        float* parts, hipStream_t st) {
  hipLaunchKernelGGL((split_kernel<KLO, KHI, VLO, VHI, QJL>), dim3(plan.n_split, a.hkv, a.batch), dim3(ST), 0, st,
                     ktab, kc.codes, kc.norms, kc.qjl_signs, kc.qjl_rnorms, kc.cap, vtab, vc.codes, vc.norms, vc.cap,
                     seq_lens, prep, parts, a.hq, a.hkv, a.sink, plan.n_split, plan.chunk, a.v_skip);
  return hipGetLastError();
}

template <int KLO, int KHI>
hipError_t dispatch_v(int vkey, bool qjl, const Tables* ktab, const tq_cache& kc, const Tables* vtab,
                      const tq_cache& vc, const tq_attn& a, const AttendPlan& plan, const int32_t* sl,
                      const uint8_t* prep, float* parts, hipStream_t st) {
#define TQ_V(VL, VH)                                                                                     \
  case VL * 10 + VH:                                                                                     \
    return qjl ? launch_split<KLO, KHI, VL, VH, true>(ktab, kc, vtab, vc, a, plan, sl, prep, parts, st)  \
               : launch_split<KLO, KHI, VL, VH, false>(ktab, kc, vtab, vc, a, plan, sl, prep, parts, st);
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
  // about one 8-wave workgroup per CU, and no split longer than 8192 tokens
  // (ragged batches balance better with shorter splits)
  int64_t ns = streams > 0 ? (256 + streams - 1) / streams : 1;
  const int64_t by_len = (comp + 8191) / 8192;
  if (ns < by_len) ns = by_len;
  const int64_t cap_ns = (tiles + SW - 1) / SW;  // at least one tile per wave
  if (ns > cap_ns) ns = cap_ns;
  if (ns < 1) ns = 1;
  int64_t chunk_tiles = (tiles + ns - 1) / ns;
  if (chunk_tiles < 1) chunk_tiles = 1;
  ns = (tiles + chunk_tiles - 1) / chunk_tiles;
  if (ns < 1) ns = 1;
  p.n_split = static_cast<int>(ns);
  p.chunk = chunk_tiles * TILE;
  const int64_t heads = static_cast<int64_t>(a.batch) * a.hq;
  p.ws_bytes = static_cast<size_t>(streams) * PREP_BYTES +
               static_cast<size_t>(heads) * static_cast<int64_t>(p.n_split) * PART * sizeof(float);
  return p;
}

hipError_t launch_attend(const Spec& ks, const Tables* ktab, const tq_cache& kc, const Spec& vs, const Tables* vtab,
                         const tq_cache& vc, const tq_attn& a, const AttendPlan& plan, const float* q,
                         const uint16_t* sink_k, const uint16_t* sink_v, const int32_t* seq_lens, float* out,
                         void* workspace, hipStream_t st) {
  const int64_t heads = static_cast<int64_t>(a.batch) * a.hq;
  const int64_t streams = static_cast<int64_t>(a.batch) * a.hkv;
  uint8_t* prep = static_cast<uint8_t*>(workspace);
  float* parts = reinterpret_cast<float*>(prep + streams * PREP_BYTES);
  hipLaunchKernelGGL(prep_kernel, dim3(static_cast<unsigned>(heads)), dim3(256), 0, st, ktab, q, prep, a.hq, a.hkv,
                     a.scale * LOG2E, ks.qjl_m ? 1 : 0);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int vkey = vs.bits_lo * 10 + vs.bits_hi;
  const bool qjl = ks.qjl_m != 0;
  hipError_t e;
  switch (ks.bits_lo * 10 + ks.bits_hi) {
    case 22: e = dispatch_v<2, 2>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, prep, parts, st); break;
    case 33: e = dispatch_v<3, 3>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, prep, parts, st); break;
    case 44: e = dispatch_v<4, 4>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, prep, parts, st); break;
    case 43: e = dispatch_v<4, 3>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, prep, parts, st); break;
    case 32: e = dispatch_v<3, 2>(vkey, qjl, ktab, kc, vtab, vc, a, plan, seq_lens, prep, parts, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const size_t smem = (2 * static_cast<size_t>(plan.n_split) + static_cast<size_t>(a.sink)) * sizeof(float);
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>(heads)), dim3(CT), smem, st, vtab, q, sink_k, sink_v,
                     seq_lens, parts, out, a.hq, a.hkv, a.sink, plan.n_split, a.scale * LOG2E);
  return hipGetLastError();
}

}  // namespace tq
