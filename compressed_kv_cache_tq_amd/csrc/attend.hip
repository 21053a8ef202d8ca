// Decode attention read directly from the packed cache: the combine kernel,
// the split plan and the launch (the split kernel, which merges a stream's
// partials itself when the stream has one split, is in attend_split.h).
//
// noze.it, "TurboQuant-MLX: quantizzare pesi e KV cache per LLM open-weight su
// Mac", section "Il metodo TurboQuant, in breve": inner products in the
// rotated domain, one inverse rotation per query head.
#include "attend_common.h"

namespace tq {
namespace {

// ---------------------------------------------------------------------------
// combine: one workgroup of 256 threads per (sequence, query head, output
// slice of 128 / NQ coordinates): log-sum-exp merge of the split partials
// (rotated value domain) and of the sink partial (original domain, slot
// n_split when present), and the slice of the inverse rotation Pi_V^T.
// Many small workgroups keep the loads spread over many CUs, and every
// global load is issued before the first barrier.
constexpr int CT = 256;

template <int NQ>
__global__ __launch_bounds__(CT) void combine_kernel(const Tables* __restrict__ vtab, const float* __restrict__ parts,
                                                     float* __restrict__ out, int n_split, int n_slot) {
  constexpr int OW = D / NQ;         // output coordinates of this workgroup
  constexpr int CQ = CT / OW;        // rotated-coordinate chunks
  constexpr int CK = D / CQ;         // rotated coordinates per chunk
  __shared__ float wsp[MAX_SPLIT + 1];  // slot maxima, then weights
  __shared__ float lsp[MAX_SPLIT + 1];  // slot sums
  __shared__ float rs[2][D];            // rotated-domain sums (two split halves)
  __shared__ float ob[CQ][OW];
  __shared__ float red[8];
  const int bh = blockIdx.x / NQ, qo = blockIdx.x % NQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* pp = parts + static_cast<int64_t>(bh) * n_slot * PART;
  // thread roles: (c, hs) for the rotated sums, (oi, cq) for the rotation
  const int c = tid & (D - 1), hs = tid >> 7;
  const int oi = tid % OW, cq = tid / OW, gi = qo * OW + oi;
  const bool has_sink = n_slot > n_split;

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
  const float sacc = has_sink && cq == 0 ? pp[static_cast<int64_t>(n_split) * PART + 4 + gi] : 0.0f;
  float mloc = -INFINITY;
  for (int sp = tid; sp < n_slot; sp += CT) {
    const float m = pp[static_cast<int64_t>(sp) * PART], l = pp[static_cast<int64_t>(sp) * PART + 1];
    const float mv = l > 0.0f ? m : -INFINITY;
    wsp[sp] = mv;
    lsp[sp] = l;
    mloc = fmaxf(mloc, mv);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
  if (lane == 0) red[wave] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // ---- weights and normaliser
  float lloc = 0.0f;
  for (int sp = tid; sp < n_slot; sp += CT) {
    const float mv = wsp[sp];
    const float f = mv == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
    wsp[sp] = f;
    lloc = fmaf(f, lsp[sp], lloc);
  }
#pragma unroll
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
  // (the value lookup tables hold centroids times the codebook's scale)
  rs[hs][c] = a / vtab->cen16_scale[c < static_cast<int>(vtab->split) ? 0 : 1];
  __syncthreads();
  const float Ls = red[4] + red[5] + red[6] + red[7];
  // ---- slice of the inverse rotation (+ the sink values): thread (oi, cq)
  float o = 0.0f;
#pragma unroll
  for (int k = 0; k < CK; ++k) o = fmaf(pic[k], rs[0][CK * cq + k] + rs[1][CK * cq + k], o);
  if (has_sink && cq == 0) o = fmaf(wsp[n_split], sacc, o);
  ob[cq][oi] = o;
  __syncthreads();
  if (tid < OW) {
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < CQ; ++k) v += ob[k][tid];
    out[static_cast<int64_t>(bh) * D + qo * OW + tid] = Ls > 0.0f ? v / Ls : 0.0f;
  }
}

}  // namespace

hipError_t launch_attend(const Spec& ks, const Tables* ktab, const tq_cache& kc, const Spec& vs, const Tables* vtab,
                         const tq_cache& vc, const tq_attn& a, const AttendPlan& plan, const float* q,
                         const uint16_t* sink_k, const uint16_t* sink_v, const int32_t* seq_lens, float* out,
                         void* workspace, hipStream_t st, const int32_t* block_table, int max_pages, int n_pages) {
  float* parts = static_cast<float*>(workspace);
  const SplitArgs f{ktab, &kc, vtab, &vc, &a, &plan, q, sink_k, sink_v, seq_lens, parts, out,
                    block_table, max_pages, n_pages, st, ks.norm16 != 0};
  const int vkey = vs.bits_lo * 10 + vs.bits_hi;
  const bool qjl = ks.qjl_m != 0;
  hipError_t e;
  switch (ks.bits_lo * 10 + ks.bits_hi) {
    case 22: e = split_k22(vkey, qjl, f); break;
    case 33: e = split_k33(vkey, qjl, f); break;
    case 44: e = split_k44(vkey, qjl, f); break;
    case 43: e = split_k43(vkey, qjl, f); break;
    case 32: e = split_k32(vkey, qjl, f); break;
    case 88: e = split_k88(vkey, qjl, f); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  // with one split per stream the split kernel has merged its own partials
  if (plan.n_split == 1) return hipSuccess;
  // four output slices per head while the heads alone would leave most CUs idle
  const int64_t heads = static_cast<int64_t>(a.batch) * a.hq;
  if (heads < 256)
    hipLaunchKernelGGL(combine_kernel<4>, dim3(static_cast<unsigned>(heads * 4)), dim3(CT), 0, st, vtab, parts, out,
                       plan.n_split, plan.n_slot);
  else
    hipLaunchKernelGGL(combine_kernel<1>, dim3(static_cast<unsigned>(heads)), dim3(CT), 0, st, vtab, parts, out,
                       plan.n_split, plan.n_slot);
  return hipGetLastError();
}

}  // namespace tq
