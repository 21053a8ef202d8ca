// Internal declarations shared by the host half (host.cpp) and the HIP
// kernels (quantize.hip, attend.hip) of libtq.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "tq.h"

namespace tq {

constexpr int D = TQ_DIM;
constexpr int TILE = TQ_TILE_TOKENS;
constexpr int QJL_M = TQ_QJL_M;
constexpr uint32_t TABLES_MAGIC = 0x31515454u;  // "TTQ1"
constexpr int CELLS = 128;        // cells of the code table over [-1, 1] (each 1/64 wide)
constexpr int CELL_ENTRIES = 132; // CELLS + 1, padded
constexpr int CELLS8 = 1024;        // cells of the 8-bit code table over [-1/2, 1/2]
constexpr int CELL8_ENTRIES = 1028; // CELLS8 + 1, padded

// Device tables of one tq_spec, built on the host by tq_tables_build.
//
// Half index 0 is the codebook of rotated coordinates [0, split), 1 of
// [split, d) (both the same codebook for a uniform width).  Boundaries are
// ascending and padded with +inf; centroids ascending, padded with 0.
//
// The rotation is stored row-major (y = pi x) in fp32 and, for the MFMA
// contraction, as an fp16 pair pi_hi + pi_lo = 256 * pi (hi = fp16 of
// 256*pi, lo = fp16 of the remainder), which keeps about 22 significant bits.
// The sketch S (qjl_m x d, row-major) is stored the same way without the 256
// factor.  pit / sit are the transposes in fp32 (coalesced matrix-vector
// products with one output per thread).  pi_b16 splits pi itself into three
// bf16 parts (hi, mid, lo) for the bf16 MFMA path.  All arrays start on
// 256-byte boundaries.
struct alignas(256) Tables {
  uint32_t magic;
  uint32_t version;
  uint32_t bits[2];
  uint32_t split;
  uint32_t qjl_m;
  uint32_t layout;
  uint32_t pad0;
  float bnd[2][16];
  float cen[2][16];
  // fp16 centroids for the lookup tables of the decode and the search:
  // cen16[h][j] = fp16(cen[h][j] * cen16_scale[h]), with the scale s in [1, 2)
  // that minimises the largest relative rounding error of the codebook (a
  // function of the width alone, 1 for 8-bit codes).  The kernels divide s
  // out in fp32 on the other operand.
  uint16_t cen16[2][16];
  float cen16_scale[2];
  uint8_t pad1[512 - 32 - 128 - 128 - 64 - 8];
  float pi[D * D];
  uint16_t pi_hi[D * D];
  uint16_t pi_lo[D * D];
  float s[D * D];
  uint16_t s_hi[D * D];
  uint16_t s_lo[D * D];
  float pit[D * D];
  float sit[D * D];
  uint16_t pi_b16[3][D * D];  // bf16 split of pi: hi + mid + lo keeps ~24 bits
  // Cell table of each half's codebook: y in [-1, 1] falls in cell
  // c = RNE(512 y + 512) >> 3 in [0, 128] (cell.h), the interval
  // [(8c - 1/2) / 512 - 1, (8c + 15/2) / 512 - 1).  Entry c = {bits of the one
  // boundary in the cell or of +inf, number of boundaries below the cell}, so
  // the code of y is code_low + (y > boundary).
  uint32_t cell[2][CELL_ENTRIES][2];
  // pi_hi / pi_lo again, in the register order of the rotation kernel's MFMA
  // fragments so that every fragment load is one contiguous 1 KiB read:
  // [layout (record, tiled)][hi, lo][w][t][ks][lane][8], the 8 values of
  // row frag_row(layout, w, t, lane), columns 16 ks + 8 (lane / 32) + e.
  uint16_t pi_frag[2][2][D * D];
  // The 8-bit codebook (keys: uniform width, record layout, no sketch; the
  // arrays above then hold nothing): boundaries padded with +inf, centroids
  // in fp32 and fp16, and its cell table over [-1/2, 1/2] (every boundary
  // lies inside): y falls in cell clamp(floor(1024 (y + 1/2)), 0, 1024),
  // entries as in `cell`.
  float bnd8[256];
  float cen8[256];
  uint16_t cen16_8[256];
  uint32_t cell8[CELL8_ENTRIES][2];
};

// Row of 256 Pi held by lane `lane` (of wave w of a pair, M-block t) in the
// rotation kernel's fragments.  Record layout: Pi is the A operand, rows
// permuted so that a lane's 32 accumulator values are 32 consecutive rotated
// coordinates; tiled layout: Pi^T is the B operand, row 64 w + 32 t + lane.
inline int frag_row(int tiled, int w, int t, int lane) {
  const int l32 = lane & 31;
  if (tiled) return 64 * w + 32 * t + l32;
  return 64 * w + 32 * ((l32 >> 2) & 1) + 16 * t + 4 * (l32 >> 3) + (l32 & 3);
}

constexpr float PI_SCALE = 256.0f;

// Validated, normalised view of a tq_spec.
struct Spec {
  int bits_lo;
  int bits_hi;   // == bits_lo for a uniform width
  int qjl_m;
  int layout;
  int code_bytes;  // per token
  int norm16;      // norms stored as fp16 (else fp32)
  int rotation;    // tq_rotation
};

// One sequence of a quantize call: hkv streams whose rows start at element
// x_off of x (stream h at x_off + h * x_stream_stride); their n_tok (> 0)
// vectors fill positions [tok0, tok0 + n_tok) of cache streams stream0 + h.
struct QSeq {
  int64_t x_off;
  int64_t tok0;
  int64_t n_tok;
  int64_t stream0;   // contiguous cache: stream of kv head 0; paged: 0
  int64_t page_row;  // paged: the sequence's row of the block table
};

// A paged cache: position c of a sequence lives at position c % 64 of pool
// page table[page_row * ld + c / 64] (streams page * hkv + h); table ==
// nullptr for a contiguous cache.  Pages outside [0, n_pages) are not written.
struct PageMap {
  const int32_t* table = nullptr;  // device
  int64_t ld = 0;
  int64_t n_pages = 0;
};

// The butterfly quantize (fwht.hip): keys in the record layout, bf16, uniform
// 2-4 bit codes, no sketch, contiguous cache.
bool fwht_supported(const Spec& sp, int dtype, bool paged);
hipError_t launch_quantize_fwht(const Spec& sp, const Tables* tab, const void* x, const QSeq* seqs, int64_t n_seq,
                                int64_t hkv, int64_t xss, int64_t xrs, const tq_cache& c, hipStream_t st);

hipError_t launch_quantize(const Spec& sp, const Tables* tab, int dtype, const void* x, const QSeq* seqs,
                           int64_t n_seq, int64_t hkv, int64_t x_stream_stride, int64_t x_row_stride,
                           const tq_cache& cache, const PageMap& pages, hipStream_t stream);

// Inner-product scores of nq <= TQ_IP_MAX_QUERIES queries against a
// record-layout cache (search.hip).
size_t ip_workspace_bytes();
hipError_t launch_ip_scores(const Spec& sp, const Tables* tab, const tq_cache& c, int64_t n_streams, int64_t n_tok,
                            const float* q, int nq, float* scores, int64_t ld, void* workspace, hipStream_t st);

// Decode split plan (plan.cpp): every workgroup of the split kernel has SW
// waves; a partial is PART floats (m, l, 2 pad, acc[128]); at most
// MAX_SPLIT splits per (sequence, kv head).
constexpr int SW = 8;
constexpr int PART = 132;
constexpr int MAX_SPLIT = 512;

// Bytes of the search workspace: fp16 hi + lo rows of the rotated query and
// of u = S q~ per query, and two fp32 scales per query.
constexpr size_t IP_WORK_BYTES = 2 * 2 * TQ_IP_MAX_QUERIES * D * 2 + 2 * TQ_IP_MAX_QUERIES * 4;

struct AttendPlan {
  int n_split;       // splits of the compressed token range per (b, kv head)
  int n_slot;        // partials per query head: n_split, plus one for the sink tokens
  int64_t chunk;     // tokens per split (multiple of TILE)
  size_t ws_bytes;   // workspace needed
};

AttendPlan plan_attend(const tq_attn& a);

hipError_t launch_attend(const Spec& ks, const Tables* ktab, const tq_cache& kc,
                         const Spec& vs, const Tables* vtab, const tq_cache& vc,
                         const tq_attn& a, const AttendPlan& plan, const float* q,
                         const uint16_t* sink_k, const uint16_t* sink_v,
                         const int32_t* seq_lens, float* out, void* workspace,
                         hipStream_t stream, const int32_t* block_table = nullptr, int max_pages = 0,
                         int n_pages = 0);

// Sets the thread's tq_last_error text and returns st.
tq_status set_error(tq_status st, const char* msg);

// Validation and launch shared by the decode entry points (host.cpp):
// block_table == NULL for a contiguous cache.
tq_status attend_checked(const tq_spec* ks, const void* ktables, const tq_cache* kc, const tq_spec* vs,
                         const void* vtables, const tq_cache* vc, const tq_attn* attn, const float* q,
                         const uint16_t* sink_k, const uint16_t* sink_v, const int32_t* seq_lens,
                         const int32_t* block_table, int32_t max_pages, int64_t n_pages, float* out,
                         void* workspace, size_t ws_bytes, void* stream, const char* what);

}  // namespace tq
