// Quantize with the randomized Hadamard rotation applied by butterflies.
//
// noze.it, "TurboQuant-MLX: quantizzare pesi e KV cache per LLM open-weight su
// Mac", section "Cosa aggiunge turboquant-mlx": one port realises the random
// rotation with a Hadamard transform, the fast and cheap way.  With
// Pi = H diag(sigma) / sqrt(d) (Sylvester H), y = Pi x / ||x|| is the fast
// Walsh-Hadamard transform of the sign-flipped vector: log2(128) = 7 stages
// of add/subtract butterflies, 7 * 64 pairs per vector, instead of the
// 128 x 128 product on the matrix cores.  The codes are those of the dense
// path (same Pi); the rotated coordinates differ only by rounding (fp32
// butterflies on exact bf16 inputs: each y_i within about 1e-8 of its
// float64 value, against about 2e-7 for the split-fp16 MFMA product).
//
// One wave owns a 32-vector tile: lane (v, h) holds coordinates 64 h .. 64 h
// + 63 of vector v.  Six butterfly stages run inside the lane's 64
// registers; the last pairs coordinate i with i + 64 across the two halves
// of the wave (a 32-lane swap).  Codes come from the cell table as in the
// dense kernel, packed LSB first into the record's half of lane h.  Keys in
// the record layout, bf16 input, uniform 2-, 3- or 4-bit codes, no sketch,
// contiguous caches; one launch covers up to 64 sequences of a ragged batch.
#include "cell.h"
#include "lanes.h"
#include "norm.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int FW_WAVES = 4;
constexpr int FW_THREADS = 64 * FW_WAVES;
constexpr int FW_MAX_SEQ = 64;
constexpr int FW_RSRC_WORD3 = 0x00020000;
constexpr float FW_F16_MAX = 65504.0f;
constexpr float INV_SQRT_D = 0.08838834764831845f;  // 1 / sqrt(128)

typedef __bf16 fw_bf16x2 __attribute__((ext_vector_type(2)));

struct FwSeq {
  int64_t x_off;    // element offset of the sequence's stream 0, row 0
  int32_t tok0;     // cache position of row 0
  int32_t n_tok;    // rows per stream, > 0
  int32_t stream0;  // cache stream of the sequence's stream 0
  int32_t tiles;    // tiles per stream
  int32_t start;    // first tile of the sequence in the launch
};
struct FwArgs {
  const Tables* tab;
  const void* x;
  uint8_t* codes;
  float* norms;
  int64_t xss, xrs, cap, stream_code_bytes;
  int32_t hkv;
  int32_t n_seq;
  int32_t norm16;
  int64_t total;  // tiles of the launch
  FwSeq seq[FW_MAX_SEQ];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t fw_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), FW_RSRC_WORD3);
}

__device__ __forceinline__ uint32_t fw_word(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

template <int B>
__global__ __launch_bounds__(FW_THREADS) void fwht_kernel(const FwArgs A) {
  constexpr int CODE_BYTES = 16 * B;
  __shared__ uint2 cell_s[CELL_ENTRIES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v = lane & 31, h = lane >> 5;
  const Tables* __restrict__ tab = A.tab;
  for (int c = tid; c < CELL_ENTRIES; c += FW_THREADS) cell_s[c] = make_uint2(tab->cell[0][c][0], tab->cell[0][c][1]);
  // sign flips of the lane's 64 coordinates, as xor masks of its 32 bf16
  // words: row 0 of Pi = H diag(sigma) / sqrt(d) is sigma / sqrt(d)
  uint32_t flip[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int c0 = 64 * h + 2 * k;
    flip[k] = (tab->pi[c0] < 0.0f ? 0x8000u : 0u) | (tab->pi[c0 + 1] < 0.0f ? 0x80000000u : 0u);
  }
  __syncthreads();

  const int64_t waves = static_cast<int64_t>(gridDim.x) * FW_WAVES;
  // tile tl of the launch -> sequence, stream, tile within the stream (wave-uniform)
  struct At {
    int64_t x0, rows, dst_stream, pos0;
  };
  auto locate = [&](int64_t tl) {
    int sq = 0;
#pragma unroll
    for (int step = FW_MAX_SEQ / 2; step > 0; step >>= 1)
      if (sq + step < A.n_seq && A.seq[sq + step].start <= tl) sq += step;
    const FwSeq& Q = A.seq[sq];
    const int64_t t = tl - Q.start;
    const int64_t s = t / Q.tiles, T = t - s * Q.tiles;
    At a;
    a.x0 = Q.x_off + s * A.xss + 32 * T * A.xrs;
    const int64_t left = static_cast<int64_t>(Q.n_tok) - 32 * T;
    a.rows = tl < A.total ? (left < 32 ? left : 32) : 0;
    a.dst_stream = Q.stream0 + s;
    a.pos0 = Q.tok0 + 32 * T;
    return a;
  };
  auto load = [&](const At& a, uint4 (&dst)[8]) {
    const uint8_t* base = static_cast<const uint8_t*>(A.x) + a.x0 * 2;
    const __amdgpu_buffer_rsrc_t r = fw_rsrc(base, a.rows > 0 ? ((a.rows - 1) * A.xrs + D) * 2 : 0);
    const int off = static_cast<int>((v * A.xrs + 64 * h) * 2);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      dst[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * k, 0, 0));
  };

  int64_t tl = static_cast<int64_t>(blockIdx.x) * FW_WAVES + wave;
  At cur = locate(tl);
  uint4 xr[8];
  load(cur, xr);
  for (; tl < A.total; tl += waves) {
    const At nxt = locate(tl + waves);
    uint4 xn[8];
    load(nxt, xn);
    // ---- norm: exact bf16 squares summed in fp32 chains, combined in fp64
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float c = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const fw_bf16x2 p = __builtin_bit_cast(fw_bf16x2, fw_word(xr[k], e));
        c = __builtin_amdgcn_fdot2_f32_bf16(p, p, c, false);
      }
      ss += static_cast<double>(c);
    }
    ss = add_half_swap(ss);
    // a sum outside the fp32 chains' exact range (rare): both lanes of such
    // a vector redo theirs on scaled elements
    const bool slow = !sumsq_fast_ok(ss);
    const bool any_slow = __builtin_amdgcn_ballot_w64(slow) != 0;
    if (any_slow) {
      const float s = sumsq_rescale(ss);
      const double s2 = add_half_swap(static_cast<double>(bf16_sumsq_scaled(xr, s)));
      if (slow) ss = s2 / (static_cast<double>(s) * static_cast<double>(s));
    }
    const float normf = static_cast<float>(sqrt(ss));
    // ---- sign flips, then the transform on the lane's 64 coordinates
    float y[64];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const uint32_t w = fw_word(xr[k >> 2], k & 3) ^ flip[k];
      y[2 * k] = __uint_as_float(w << 16);
      y[2 * k + 1] = __uint_as_float(w & 0xFFFF0000u);
    }
    // Such vectors are scaled by a power of two to a norm in [1/2, 1) (exact in
    // fp32, denormal inputs included), so that neither the butterfly sums
    // nor 1 / norm leave fp32's range; the transform is linear.
    float nrm_eff = normf;
    if (any_slow) {
      int ex = 0;
      frexpf(normf, &ex);
      const int e = min(-ex, 126);  // (a norm below 2^-126 ends in [2^-7, 1))
      const float f = slow ? ldexpf(1.0f, e) : 1.0f;
#pragma unroll
      for (int i = 0; i < 64; ++i) y[i] *= f;
      nrm_eff = slow ? ldexpf(normf, e) : normf;
    }
#pragma unroll
    for (int len = 1; len < 64; len <<= 1)
#pragma unroll
      for (int i = 0; i < 64; ++i)
        if ((i & len) == 0) {
          const float a = y[i], b = y[i + len];
          y[i] = a + b;
          y[i + len] = a - b;
        }
    // last stage: coordinate i (lower lane, a) with i + 64 (upper lane, b):
    // the lower lane keeps a + b, the upper one a - b
    const float sgn = h ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const uint32_t u = __float_as_uint(y[i]);
      const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      const float other = __uint_as_float(h ? sw[0] : sw[1]);
      y[i] = fmaf(y[i], sgn, other);
    }
    // ---- codes from the cell table: y / (sqrt(d) ||x||) is the rotated unit vector
    const float inv = nrm_eff > 0.0f ? INV_SQRT_D / nrm_eff : 0.0f;
    uint32_t wd[2 * B];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t c[32];
#pragma unroll
      for (int p = 0; p < 32; ++p) {
        const float yy = y[32 * half + p] * inv;
        const uint2 e = cell_entry(cell_s, yy);
        c[p] = e.y + (yy > __uint_as_float(e.x) ? 1u : 0u);
      }
      // 32 codes LSB first into B dwords
#pragma unroll
      for (int k = 0; k < B; ++k) {
        uint32_t acc = 0;
#pragma unroll
        for (int p = 0; p < 32; ++p) {
          const int bit = B * p;
          if (bit >= 32 * k + 32 || bit + B <= 32 * k) continue;
          const int sh = bit - 32 * k;
          acc |= sh >= 0 ? c[p] << sh : c[p] >> (-sh);
        }
        wd[B * half + k] = acc;
      }
    }
    // ---- stores: the lane's half record and (lane h == 0) the norm
    const int64_t rows = cur.rows;
    uint8_t* rec = A.codes + cur.dst_stream * A.stream_code_bytes + cur.pos0 * CODE_BYTES;
    const __amdgpu_buffer_rsrc_t rc = fw_rsrc(rec, rows * CODE_BYTES);
    const int o = v * CODE_BYTES + 8 * B * h;
#pragma unroll
    for (int k = 0; k < 2 * B; ++k) __builtin_amdgcn_raw_buffer_store_b32(wd[k], rc, o + 4 * k, 0, 0);
    const int nb = A.norm16 ? 2 : 4;
    uint8_t* nrm = reinterpret_cast<uint8_t*>(A.norms) + (cur.dst_stream * A.cap + cur.pos0) * nb;
    const __amdgpu_buffer_rsrc_t rn = fw_rsrc(nrm, rows * nb);
    const int noff = h == 0 ? nb * v : 0x40000000;  // upper lanes: past the extent, dropped
    if (A.norm16)
      __builtin_amdgcn_raw_buffer_store_b16(
          __builtin_bit_cast(uint16_t, static_cast<_Float16>(fminf(normf, FW_F16_MAX))), rn, noff, 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(normf), rn, noff, 0, 0);
    cur = nxt;
#pragma unroll
    for (int k = 0; k < 8; ++k) xr[k] = xn[k];
  }
}

template <int B>
hipError_t launch_fwht_b(const FwArgs& a, hipStream_t st) {
  const int64_t blocks64 = (a.total + FW_WAVES - 1) / FW_WAVES;
  const unsigned blocks = static_cast<unsigned>(blocks64 < 4096 ? blocks64 : 4096);
  hipLaunchKernelGGL(fwht_kernel<B>, dim3(blocks), dim3(FW_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace

bool fwht_supported(const Spec& sp, int dtype, bool paged) {
  return dtype == TQ_BF16 && !paged && sp.layout == TQ_LAYOUT_RECORD && sp.qjl_m == 0 && sp.bits_lo == sp.bits_hi &&
         sp.bits_lo >= 2 && sp.bits_lo <= 4;
}

hipError_t launch_quantize_fwht(const Spec& sp, const Tables* tab, const void* x, const QSeq* seqs, int64_t n_seq,
                                int64_t hkv, int64_t xss, int64_t xrs, const tq_cache& c, hipStream_t st) {
  const int64_t code_bytes = 16 * sp.bits_lo;
  for (int64_t b0 = 0; b0 < n_seq; b0 += FW_MAX_SEQ) {
    FwArgs a{};
    a.tab = tab;
    a.x = x;
    a.codes = c.codes;
    a.norms = c.norms;
    a.xss = xss;
    a.xrs = xrs;
    a.cap = c.cap;
    a.stream_code_bytes = c.cap * code_bytes;
    a.hkv = static_cast<int32_t>(hkv);
    a.norm16 = sp.norm16;
    const int nb = static_cast<int>(n_seq - b0 < FW_MAX_SEQ ? n_seq - b0 : FW_MAX_SEQ);
    a.n_seq = nb;
    int64_t total = 0;
    for (int i = 0; i < nb; ++i) {
      const QSeq& q = seqs[b0 + i];
      const int64_t tiles = (q.n_tok + TILE - 1) / TILE;
      a.seq[i] = FwSeq{q.x_off, static_cast<int32_t>(q.tok0), static_cast<int32_t>(q.n_tok),
                       static_cast<int32_t>(q.stream0), static_cast<int32_t>(tiles), static_cast<int32_t>(total)};
      total += hkv * tiles;
    }
    a.total = total;
    hipError_t e = hipErrorInvalidValue;
    switch (sp.bits_lo) {
      case 2: e = launch_fwht_b<2>(a, st); break;
      case 3: e = launch_fwht_b<3>(a, st); break;
      case 4: e = launch_fwht_b<4>(a, st); break;
      default: break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
