// Inner-product search over packed key vectors: estimates of <q_i, x_t> for a
// batch of queries against every vector of a record-layout cache.
//
// noze.it, "TurboQuant-MLX: quantizzare pesi e KV cache per LLM open-weight su
// Mac", section "Il metodo TurboQuant, in breve": similarity search (in place
// of product quantization) is the method's second application, and the
// 1-bit sketch of the residual is what makes the inner-product estimate
// unbiased.  The estimate for query q and stored vector x (norm n, codes idx,
// sketch bits z, residual norm gamma) is
//   n (<Pi q, c[idx]> + sqrt(pi/2)/m gamma <S Pi q, z>),
// the second term only when the spec carries the sketch.
//
// Two launches on one stream:
//  prep    one workgroup per query: q~ = Pi q (and u = S q~), each scaled by
//          a power of two and split into fp16 hi + lo rows in the workspace;
//  scores  8 waves per workgroup, each streaming 32-token tiles of one
//          stream: the record chunk of a token -> LUT dequantization (the
//          decode's) -> MFMA against the query rows of every 16-query block
//          -> norm (and sketch term) -> fp32 scores.
#include "attend_split.h"

namespace tq {
namespace {

constexpr int IW = 8;             // waves per scores workgroup
constexpr int IT = 64 * IW;
constexpr int ITILES = 8;         // tiles per wave
constexpr int IQMAX = TQ_IP_MAX_QUERIES;
constexpr int QROW = D + 8;       // fp16 per query row in LDS (pad: no bank conflicts)

// Query rows written by the prep kernel (device workspace).
struct IpWork {
  _Float16 q[IQMAX][2][D];  // hi, lo of q~ 2^sh_q
  _Float16 u[IQMAX][2][D];  // hi, lo of u 2^sh_u
  float qinv[IQMAX];        // 2^-sh_q
  float uinv[IQMAX];        // sqrt(pi/2)/m 2^-sh_u
};

// Block-wide sum and maximum over the 128 threads of a prep workgroup.
__device__ __forceinline__ float block_sum128(float x, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return red[0] + red[1];
}
__device__ __forceinline__ float block_max128(float x, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return fmaxf(red[0], red[1]);
}

// x 2^(14 - exponent of bound) split into fp16 hi + lo; returns the scale's inverse
__device__ __forceinline__ float split_row(float x, float bound, _Float16* hi, _Float16* lo, int i) {
  int ex = 0;
  if (bound > 0.0f) frexpf(bound, &ex);
  const int sh = 14 - ex;
  const float xs = ldexpf(x, sh);
  const _Float16 h = static_cast<_Float16>(xs);
  hi[i] = h;
  lo[i] = static_cast<_Float16>(xs - static_cast<float>(h));
  return ldexpf(1.0f, -sh);
}

__global__ __launch_bounds__(D) void ipq_prep_kernel(const Tables* __restrict__ tab, const float* __restrict__ q,
                                                    IpWork* __restrict__ w, int qjl) {
  __shared__ float qs[D], qt[D], red[2];
  const int qi = blockIdx.x, i = threadIdx.x;
  const float qv = q[static_cast<int64_t>(qi) * D + i];
  qs[i] = qv;
  // Pi is orthogonal: |q~_i| <= ||q~|| = ||q||
  const float nq = sqrtf(block_sum128(qv * qv, red));
  float a = 0.0f;
#pragma unroll 8
  for (int k = 0; k < D; ++k) a = fmaf(tab->pit[k * D + i], qs[k], a);
  // (the lookup tables hold centroids times the codebook's scale, s >= 1:
  // the bound nq still holds for the divided coordinate)
  const float qinv =
      split_row(a / tab->cen16_scale[i < static_cast<int>(tab->split) ? 0 : 1], nq, w->q[qi][0], w->q[qi][1], i);
  if (i == 0) w->qinv[qi] = qinv;
  if (qjl) {
    qt[i] = a;
    __syncthreads();
    float u = 0.0f;
#pragma unroll 8
    for (int k = 0; k < D; ++k) u = fmaf(tab->sit[k * QJL_M + i], qt[k], u);
    const float umax = block_max128(fabsf(u), red);
    const float uinv = split_row(u, umax, w->u[qi][0], w->u[qi][1], i);
    if (i == 0) w->uinv[qi] = uinv * QJL_C;
  }
}

template <int KLO, int KHI, bool QJL>
__global__ __launch_bounds__(IT, 1) void ip_kernel(const Tables* __restrict__ ktab, const uint8_t* __restrict__ kcodes,
                                                   const float* __restrict__ knorms,
                                                   const uint8_t* __restrict__ ksigns,
                                                   const float* __restrict__ krn, int64_t cap, int64_t n_tok,
                                                   const IpWork* __restrict__ wk, int nq, float* __restrict__ scores,
                                                   int64_t ld) {
  constexpr int KBYTES = 8 * (KLO + KHI);
  constexpr int KW = KLO > KHI ? KLO : KHI;
  constexpr int LUT_LO = 0;
  constexpr int LUT_HI = KLO == KHI ? 0 : lut_size<KLO>();
  constexpr int LUT_BYTES = LUT_HI + (KLO == KHI ? lut_size<KLO>() : lut_size<KHI>());
  constexpr int NSET = QJL ? 2 : 1;
  constexpr int QBYTES = NSET * 2 * IQMAX * QROW * 2;
  static_assert(LUT_BYTES + QBYTES + 2 * IQMAX * 4 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LUT_BYTES + QBYTES];
  __shared__ float qinv_s[IQMAX], uinv_s[IQMAX];
  __shared__ uint32_t lutz[4];
  _Float16* qrows = reinterpret_cast<_Float16*>(smem + LUT_BYTES);  // [set][part][IQMAX][QROW]
  auto qrow = [&](int set, int part, int qi) { return qrows + ((set * 2 + part) * IQMAX + qi) * QROW; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
  const int64_t s = blockIdx.y;
  const int nqb = (nq + 15) / 16;

  // ---- the first tiles' loads go out before the LDS set-up
  // token slot of A-operand row n in M-block mb (output rows 4 j + i of
  // block mb are then tokens 8 j + 4 mb + i); lane j takes the coordinates
  // 32 j .. 32 j + 31 (uniform width) or 16 j .. + 15 of each width
  uint32_t ko[2], ko2[2], zo[2], ksh[2] = {0u, 0u};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const uint32_t tok = 8 * (n >> 2) + 4 * mb + (n & 3);
    if constexpr (KLO != KHI) {
      const uint32_t olo = 2 * KLO * j, ohi = 8 * KLO + 2 * KHI * j;
      ko[mb] = tok * KBYTES + (olo & ~3u);
      ko2[mb] = tok * KBYTES + (ohi & ~3u);
      ksh[0] = 8 * (olo & 3u);
      ksh[1] = 8 * (ohi & 3u);
    } else {
      ko[mb] = tok * KBYTES + 4 * KLO * j;
      ko2[mb] = 0;
    }
    zo[mb] = tok * (QJL_M / 8) + 4 * j;
  }
  const __amdgpu_buffer_rsrc_t rkc = rsrc(kcodes + s * cap * KBYTES, n_tok * KBYTES);
  const __amdgpu_buffer_rsrc_t rkn = rsrc(knorms + s * cap, n_tok * 4);
  const __amdgpu_buffer_rsrc_t rzs = QJL ? rsrc(ksigns + s * cap * (QJL_M / 8), n_tok * (QJL_M / 8)) : rkn;
  const __amdgpu_buffer_rsrc_t rrn = QJL ? rsrc(krn + s * cap, n_tok * 4) : rkn;
  struct Tile {
    uint32_t kw[2][4];
    uint32_t zw[2];
    float4 kn[2], rn[2];
  };
  auto load = [&](Tile& t, uint32_t t0) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if constexpr (KLO != KHI) {
        uint32_t w[2];
        buf_load<2>(w, rkc, ko[mb] + t0 * KBYTES);
        t.kw[mb][0] = w[0];
        t.kw[mb][1] = w[1];
        buf_load<2>(w, rkc, ko2[mb] + t0 * KBYTES);
        t.kw[mb][2] = w[0];
        t.kw[mb][3] = w[1];
      } else {
        uint32_t w[KW];
        buf_load<KW>(w, rkc, ko[mb] + t0 * KBYTES);
#pragma unroll
        for (int i = 0; i < KW; ++i) t.kw[mb][i] = w[i];
      }
      if constexpr (QJL) t.zw[mb] = __builtin_amdgcn_raw_buffer_load_b32(rzs, zo[mb] + t0 * (QJL_M / 8), 0, 0);
    }
    t.kn[0] = buf_load_f4(rkn, 32 * j + 4 * t0);
    t.kn[1] = buf_load_f4(rkn, 32 * j + 4 * t0 + 16);
    if constexpr (QJL) {
      t.rn[0] = buf_load_f4(rrn, 32 * j + 4 * t0);
      t.rn[1] = buf_load_f4(rrn, 32 * j + 4 * t0 + 16);
    }
  };
  constexpr uint32_t STEP = 32 * IW;
  const uint32_t first = static_cast<uint32_t>(blockIdx.x) * (STEP * ITILES) + 32 * wave;
  Tile buf[2];
  load(buf[0], first);
  load(buf[1], first + STEP);

  // ---- LUTs of the key widths (pair entries, replicated per lane)
  auto lut_fill = [&](auto bw, int off) {
    constexpr int B = decltype(bw)::value;
    constexpr int E = 1 << (2 * B);
    constexpr uint32_t MK = (1u << B) - 1u;
    const uint16_t* cen = KLO == B ? ktab->cen16[0] : ktab->cen16[1];
    for (int c = tid; c < E * 16; c += IT) {
      const int e = c >> 4;
      const uint32_t v = static_cast<uint32_t>(cen[e & MK]) | (static_cast<uint32_t>(cen[e >> B]) << 16);
      reinterpret_cast<uint4*>(smem + off)[c] = make_uint4(v, v, v, v);
    }
  };
  lut_fill(std::integral_constant<int, KLO>{}, LUT_LO);
  if constexpr (KLO != KHI) lut_fill(std::integral_constant<int, KHI>{}, LUT_HI);
  // query rows (zero rows for the padding queries of the last block)
  for (int c = tid; c < NSET * 2 * 16 * nqb * (D / 8); c += IT) {
    const int k8 = c % (D / 8), row = c / (D / 8);
    const int qi = row % (16 * nqb), part = (row / (16 * nqb)) & 1, set = row / (32 * nqb);
    uint4 v{};
    if (qi < nq) v = *reinterpret_cast<const uint4*>((set ? wk->u[qi][part] : wk->q[qi][part]) + 8 * k8);
    *reinterpret_cast<uint4*>(qrow(set, part, qi) + 8 * k8) = v;
  }
  if (tid < IQMAX) {
    qinv_s[tid] = tid < nq ? wk->qinv[tid] : 0.0f;
    uinv_s[tid] = QJL && tid < nq ? wk->uinv[tid] : 0.0f;
  }
  if (tid < 4)
    lutz[tid] = ((tid & 1) ? 0x3C00u : 0xBC00u) | (((tid >> 1) & 1) ? 0x3C000000u : 0xBC000000u);
  __syncthreads();

  // k-slot (lane j, step ks) -> first of its 8 coordinates (sketch rows:
  // 32 j + 8 ks in both cases)
  auto kcoord = [&](int ks) { return KLO != KHI ? (ks < 2 ? 16 * j + 8 * ks : 64 + 16 * j + 8 * (ks - 2)) : 32 * j + 8 * ks; };
  const uint8_t* lut_lo = smem + LUT_LO;
  const uint8_t* lut_hi = smem + LUT_HI;

  auto tile = [&](const Tile& t, uint32_t t0) __attribute__((always_inline)) {
    half8 a[2][4], z[2][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if constexpr (KLO == KHI) {
          a[mb][ks] = dequant8<KLO>(t.kw[mb], ks, lut_lo, lane4);
        } else {
          const int part = ks >> 1;
          const uint32_t sh = ksh[part];
          const bool aligned = part == 0 ? (2 * KLO) % 4 == 0 : (2 * KHI) % 4 == 0;
          uint32_t wk2[2];
          if (aligned) {
            wk2[0] = t.kw[mb][2 * part];
            wk2[1] = t.kw[mb][2 * part + 1];
          } else {
            wk2[0] = __builtin_amdgcn_alignbit(t.kw[mb][2 * part + 1], t.kw[mb][2 * part], sh);
            wk2[1] = t.kw[mb][2 * part + 1] >> sh;
          }
          a[mb][ks] = part == 0 ? dequant8<KLO>(wk2, ks & 1, lut_lo, lane4) : dequant8<KHI>(wk2, ks & 1, lut_hi, lane4);
        }
        if constexpr (QJL) {
          const uint32_t zv = (t.zw[mb] >> (8 * ks)) & 0xFFu;
          z[mb][ks] = as_half8(lutz[zv & 3], lutz[(zv >> 2) & 3], lutz[(zv >> 4) & 3], lutz[zv >> 6]);
        }
      }
    const int64_t row0 = s * n_tok + t0 + 8 * j;  // lane's first token (8 consecutive)
    for (int qb = 0; qb < nqb; ++qb) {
      const int qi = 16 * qb + n;
      f32x4 sk[2], sz[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) sk[mb] = sz[mb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const half8 qh = *reinterpret_cast<const half8*>(qrow(0, 0, qi) + kcoord(ks));
        const half8 ql = *reinterpret_cast<const half8*>(qrow(0, 1, qi) + kcoord(ks));
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sk[mb] = mfma16(a[mb][ks], qh, sk[mb]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sk[mb] = mfma16(a[mb][ks], ql, sk[mb]);
        if constexpr (QJL) {
          const half8 uh = *reinterpret_cast<const half8*>(qrow(1, 0, qi) + 32 * j + 8 * ks);
          const half8 ul = *reinterpret_cast<const half8*>(qrow(1, 1, qi) + 32 * j + 8 * ks);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) sz[mb] = mfma16(z[mb][ks], uh, sz[mb]);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) sz[mb] = mfma16(z[mb][ks], ul, sz[mb]);
        }
      }
      if (qi >= nq) continue;
      const float qinv = qinv_s[qi], uinv = uinv_s[qi];
      float v[8];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float dot = sk[mb][i] * qinv;
          if constexpr (QJL) dot = fmaf(f4get(t.rn, 4 * mb + i) * sz[mb][i], uinv, dot);
          v[4 * mb + i] = f4get(t.kn, 4 * mb + i) * dot;
        }
      float* out = scores + static_cast<int64_t>(qi) * ld + row0;
      const int64_t left = n_tok - (static_cast<int64_t>(t0) + 8 * j);
      // the scores are written once and not read back here: streaming stores
      if (left >= 8 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(out));
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(out) + 1);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < left) __builtin_nontemporal_store(v[e], out + e);
      }
    }
  };
#pragma unroll
  for (int r = 0; r < ITILES; ++r) {
    const uint32_t t0 = first + r * STEP;
    tile(buf[r & 1], t0);
    if (r + 2 < ITILES) load(buf[r & 1], t0 + 2 * STEP);
  }
}

template <int KLO, int KHI>
hipError_t launch_ip(bool qjl, const Tables* tab, const tq_cache& c, int64_t n_streams, int64_t n_tok,
                     const IpWork* w, int nq, float* scores, int64_t ld, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((n_tok + 32 * IW * ITILES - 1) / (32 * IW * ITILES)),
                  static_cast<unsigned>(n_streams));
  if (qjl)
    hipLaunchKernelGGL((ip_kernel<KLO, KHI, true>), grid, dim3(IT), 0, st, tab, c.codes, c.norms, c.qjl_signs,
                       c.qjl_rnorms, c.cap, n_tok, w, nq, scores, ld);
  else
    hipLaunchKernelGGL((ip_kernel<KLO, KHI, false>), grid, dim3(IT), 0, st, tab, c.codes, c.norms, c.qjl_signs,
                       c.qjl_rnorms, c.cap, n_tok, w, nq, scores, ld);
  return hipGetLastError();
}

}  // namespace

static_assert(sizeof(IpWork) == IP_WORK_BYTES, "search workspace layout");

hipError_t launch_ip_scores(const Spec& sp, const Tables* tab, const tq_cache& c, int64_t n_streams, int64_t n_tok,
                            const float* q, int nq, float* scores, int64_t ld, void* workspace, hipStream_t st) {
  IpWork* w = static_cast<IpWork*>(workspace);
  const bool qjl = sp.qjl_m != 0;
  hipLaunchKernelGGL(ipq_prep_kernel, dim3(static_cast<unsigned>(nq)), dim3(D), 0, st, tab, q, w, qjl ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (sp.bits_lo * 10 + sp.bits_hi) {
    case 22: return launch_ip<2, 2>(qjl, tab, c, n_streams, n_tok, w, nq, scores, ld, st);
    case 33: return launch_ip<3, 3>(qjl, tab, c, n_streams, n_tok, w, nq, scores, ld, st);
    case 44: return launch_ip<4, 4>(qjl, tab, c, n_streams, n_tok, w, nq, scores, ld, st);
    case 43: return launch_ip<4, 3>(qjl, tab, c, n_streams, n_tok, w, nq, scores, ld, st);
    case 32: return launch_ip<3, 2>(qjl, tab, c, n_streams, n_tok, w, nq, scores, ld, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
