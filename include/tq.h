/*
 * tq.h - TurboQuant packed KV cache for AMD MI355X (gfx950): C ABI of libtq.so.
 *
 * The method (noze.it, "TurboQuant-MLX: quantizzare pesi e KV cache per LLM
 * open-weight su Mac", section "Il metodo TurboQuant, in breve"): every key or
 * value head vector keeps its norm, is rotated by a seeded random orthogonal
 * matrix, and each rotated coordinate is quantized on its own with a b-bit
 * Lloyd-Max codebook built for the post-rotation coordinate law (section
 * "Cosa aggiunge turboquant-mlx").  An optional second stage stores a 1-bit
 * quantized Johnson-Lindenstrauss sketch of the residual plus the residual
 * norm, which makes the inner-product estimate unbiased.  It is online and
 * data-oblivious: no calibration input exists in this interface.
 *
 * Decode attention reads the packed cache directly: the query is rotated
 * once, scores come from codebook lookups (plus the sketch correction), the
 * values are accumulated in the rotated domain and one inverse rotation is
 * applied per query head.  The first `sink` tokens of every sequence may be
 * kept raw in bf16 (GitHub issue "Greetings from TurboQuant-MLX & Some
 * Insights to Share!", item 1), and value tokens whose attention weight is
 * below a threshold may be dropped (same issue, item 3).
 *
 * Conventions for every entry point
 *  - Ownership: the caller owns every host and device buffer, including the
 *    device copy of the tables and the attention workspace.  The library
 *    allocates no device memory at run time; its one device array is the
 *    static scratch of tq_attend_decode_noalloc, part of the loaded code
 *    object.  Host state: a thread-local error string and process-wide
 *    caches of derived constants (compute units and that scratch's address
 *    per device, the codebook centroid scales), none of it caller data.
 *  - Errors: arguments are validated on the host before any launch.  A
 *    failed check returns a negative tq_status, launches nothing and sets
 *    tq_last_error().  A failed launch returns TQ_E_HIP with the HIP error
 *    text.
 *  - Data: kernels never fail on data.  Non-finite inputs give unspecified
 *    codes and outputs, and so does a vector whose norm exceeds FLT_MAX.
 *    Every other input vector, denormal elements included, is quantized to
 *    the same rule (stored norm within 1 ulp, codes exact but for ties
 *    within rounding of a boundary), except on the bf16 fallback for row
 *    strides beyond 32-bit offsets, where norms below about 2^-100 may lose
 *    accuracy.
 *  - Streams: `stream` is a hipStream_t (NULL = default stream).  Every
 *    device call is asynchronous on that stream; the library never
 *    synchronizes.  A device call issues kernel launches only (no memset,
 *    copy or allocation), so it can be captured in a HIP graph and replayed
 *    (with the same arguments, pointing at the same buffers).
 *  - Device pointers must be 16-byte aligned unless stated otherwise.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_FORMAT_VERSION 2   /* bit layouts described at tq_cache below; 2: 8-bit keys */
#define TQ_DIM 128            /* head dimension d supported by the kernels */
#define TQ_TILE_TOKENS 32     /* tokens per tile of the tiled layout */
#define TQ_IP_MAX_QUERIES 64  /* queries per tq_ip_scores call */
#define TQ_PAGE_TOKENS 64     /* positions per page of a paged cache */
#define TQ_QJL_M 128          /* rows m of the QJL sketch when enabled */

typedef enum {
  TQ_OK = 0,
  TQ_E_ARG = -1,          /* invalid argument (shape, pointer, alignment, range) */
  TQ_E_UNSUPPORTED = -2,  /* valid request outside what the kernels implement */
  TQ_E_WORKSPACE = -3,    /* workspace smaller than tq_attend_workspace_bytes */
  TQ_E_HIP = -4           /* a HIP launch failed; see tq_last_error() */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

typedef enum {
  TQ_LAYOUT_RECORD = 0,   /* one packed record per token (keys) */
  TQ_LAYOUT_TILED = 1     /* 32-token tiles, coordinate-major sub-blocks (values) */
} tq_layout;

/* Quantizer of one tensor (the keys or the values of a cache).
 * Rotated coordinates [0, split) use bits_lo bits, [split, d) use bits_hi
 * (noze.it page, section "Il metodo TurboQuant, in breve": 3.5 and 2.5 bits
 * per channel; 3.5 bits = split 64 with 4 and 3 bits).  split == d means a
 * uniform width and bits_hi is then ignored.  8-bit codes (the K8 keys of
 * the K8/V3 default that section "Cosa aggiunge turboquant-mlx" of the same
 * page names) need split == d, the record layout and no sketch; quantize
 * and decode take them for keys (decode: with values of 2 or 3 bits,
 * uniform), tq_ip_scores does not.  An 8-bit quantize needs 32 rows of x to
 * span less than 2^30 bytes (else TQ_E_UNSUPPORTED). */
/* How the rotation Pi is drawn from rot_seed. */
typedef enum {
  TQ_ROT_HAAR = 0,          /* Haar-distributed orthogonal matrix (tq_rotation_build) */
  TQ_ROT_HADAMARD = 1,      /* randomized Hadamard matrix (tq_hadamard_rotation_build) */
  TQ_ROT_HADAMARD_FWHT = 2  /* the same matrix, applied in the quantize by the O(d log d)
                               butterfly transform where that kernel applies (bf16 keys in
                               the record layout, uniform 2-4 bit codes, no sketch,
                               contiguous cache), by the dense product elsewhere; the
                               tables and the decode are those of TQ_ROT_HADAMARD, and
                               so are the codes except where a rotated coordinate lies
                               within rounding of a boundary.  On gfx950 the butterfly
                               kernel is slower than the dense product (it loads the
                               vector ALUs that the codes already use); it is kept as
                               the transform the pages' port applies */
} tq_rotation;

typedef struct {
  int32_t d;          /* must be TQ_DIM */
  int32_t bits_lo;    /* 2, 3, 4 or 8 (see above) */
  int32_t bits_hi;    /* 2, 3 or 4 (ignored when split == d) */
  int32_t split;      /* 64 or 128 */
  int32_t qjl_m;      /* 0 (no sketch) or TQ_QJL_M; only with TQ_LAYOUT_RECORD */
  int32_t layout;     /* tq_layout */
  uint64_t rot_seed;  /* seed of the rotation (SplitMix64 stream) */
  uint64_t qjl_seed;  /* seed of the sketch matrix S */
  int32_t rotation;   /* tq_rotation */
  int32_t norm_f16;   /* 0: fp32 norms; 1: fp16 norms (see tq_cache) */
} tq_spec;

/* One tensor of a packed cache, for n_streams = batch * kv_heads streams of
 * `cap` token positions each (stream s = b * kv_heads + h).
 *
 * codes   RECORD: stream s, position p at byte (s*cap + p) * tq_code_bytes(spec).
 *         The record is a little-endian LSB-first bit stream: coordinate i's
 *         index occupies stream bits [o_i, o_i + b_i), o_i = sum_{k<i} b_k,
 *         stream bit j = bit (j mod 8) of byte j/8.
 *         TILED: stream s at byte s * tq_cache_code_bytes(spec, cap); tile
 *         T = p / 32 at T * 32 * tq_code_bytes(spec) within the stream.  A
 *         tile has 4 token groups (tokens 8g..8g+7) x 16 coordinate groups
 *         (coordinates 8q..8q+7); sub-block (g, q) holds 8 coordinates x 8
 *         tokens in 8*b_q bytes at g*G + sum_{q'<q} 8*b_q' (G = sum_q 8*b_q),
 *         and (coordinate 8q+r, token 8g+s) occupies its bits
 *         [(8r+s)*b_q, (8r+s)*b_q + b_q).  cap must be a multiple of 32.
 * norms   fp32 [n_streams][cap]: Euclidean norm of the stored input vector;
 *         with spec->norm_f16 the IEEE binary16 bits of that fp32 norm
 *         rounded to nearest even and saturated at 65504, the largest finite
 *         binary16 value (a larger norm is stored as 65504, and the decode
 *         then scales that vector down), uint16 [n_streams][cap]; the pointer
 *         is passed as the same float*.  The K and V specs of one decode must
 *         agree on norm_f16.
 * qjl_signs  [n_streams][cap][qjl_m/8] bytes, bit j set iff (S r)_j >= 0
 *         (r = rotated unit vector minus its centroids); NULL if qjl_m == 0.
 * qjl_rnorms fp32 [n_streams][cap]: ||r||; NULL if qjl_m == 0.
 * Codes/norms are 4-byte aligned at least; codes must be 16-byte aligned. */
typedef struct {
  uint8_t* codes;
  float* norms;
  uint8_t* qjl_signs;
  float* qjl_rnorms;
  int64_t cap;
} tq_cache;

/* Decode-attention problem.  Query head h reads KV head h / (hq / hkv). */
typedef struct {
  int32_t batch;    /* B */
  int32_t hq;       /* query heads per sequence */
  int32_t hkv;      /* KV heads per sequence; hq % hkv == 0, hq/hkv <= 16 */
  int32_t sink;     /* leading tokens kept raw bf16 (0 = none) */
  float scale;      /* softmax scale, normally 1/sqrt(d) */
  float v_skip;     /* drop value tokens with weight below this (0 = off) */
  int64_t max_len;  /* host-side upper bound of seq_lens (sizes the split grid) */
} tq_attn;

/* Version of the bit layouts produced and read by this library. */
int32_t tq_format_version(void);

/* Thread-local text describing the last non-OK status of this thread. */
const char* tq_last_error(void);

/* Host only.  Lloyd-Max codebook for one coordinate of a uniformly random
 * unit vector in R^d, whose density is proportional to (1-x^2)^((d-3)/2)
 * (noze.it page, sections "Il metodo TurboQuant, in breve" and "Cosa
 * aggiunge turboquant-mlx").  Writes 2^bits centroids ascending and 2^bits-1
 * boundaries (midpoints of consecutive centroids).  3 <= d <= 65536,
 * 1 <= bits <= 8.  Deterministic. */
tq_status tq_codebook_build(int32_t d, int32_t bits, double* centroids, double* boundaries);

/* Host only.  The seeded rotation Pi (d x d, row-major, y = Pi x) that
 * every vector goes through before its coordinates are quantized (noze.it
 * page, section "Il metodo TurboQuant, in breve": the vector is first rotated
 * at random, which gives its coordinates a known law).  The page does not say
 * how the rotation is drawn; this is the Haar-distributed reading: the Q
 * factor of a SplitMix64/Box-Muller Gaussian matrix, with column signs chosen
 * so that R has a positive diagonal.  Writes d*d doubles to the caller's
 * host buffer `pi`.  1 <= d <= 1024, else TQ_E_ARG. */
tq_status tq_rotation_build(int32_t d, uint64_t seed, double* pi);

/* Host only.  The seeded randomized Hadamard rotation (noze.it page, section
 * "Cosa aggiunge turboquant-mlx": a Hadamard transform as the fast way to
 * realise the random rotation): Pi = H_d diag(sigma) / sqrt(d), with H_d the
 * Sylvester Hadamard matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]],
 * so entry (i, k) is (-1)^popcount(i & k)) and sigma_k = -1 if bit 63 of the
 * k-th SplitMix64 output of `seed` is set, else +1.  d a power of two,
 * 1 <= d <= 1024; row-major, y = Pi x. */
tq_status tq_hadamard_rotation_build(int32_t d, uint64_t seed, double* pi);

/* Host only.  The sketch matrix S (m x d, row-major) of the second stage
 * (noze.it page, section "Il metodo TurboQuant, in breve": a 1-bit quantized
 * Johnson-Lindenstrauss transform of the residual, which removes the bias of
 * the inner-product estimate): i.i.d. N(0,1) entries from the same generator
 * seeded with `seed`, not orthogonalised.  Writes m*d doubles to the
 * caller's host buffer `s`.  1 <= m, d <= 1024, else TQ_E_ARG. */
tq_status tq_sketch_build(int32_t m, int32_t d, uint64_t seed, double* s);

/* Size in bytes of the device tables of one tq_spec (same for every spec). */
size_t tq_tables_bytes(void);

/* Host only.  Fills `host_buf` (tq_tables_bytes() bytes, 16-byte aligned)
 * with everything the kernels need for `spec`: codebooks, rotation and
 * sketch in fp32 and as fp16 high/low splits.  The caller copies it to
 * device memory once and passes that copy as `tables` below. */
tq_status tq_tables_build(const tq_spec* spec, void* host_buf, size_t bytes);

/* Bytes of one token's packed codes: d * (average bits) / 8. */
size_t tq_code_bytes(const tq_spec* spec);

/* Bytes of the code array of one stream holding `cap` positions. */
size_t tq_cache_code_bytes(const tq_spec* spec, int64_t cap);

/* Quantize n_tok vectors of each of n_streams streams into cache positions
 * [tok0, tok0 + n_tok) (noze.it page, section "Il metodo TurboQuant, in
 * breve": norm, random rotation, per-coordinate Lloyd-Max quantization, and
 * the optional 1-bit sketch of the residual).
 *   tables  device copy of tq_tables_build(spec)
 *   dtype   TQ_F32 or TQ_BF16 elements of x
 *   x       device; vector (s, i) starts at element s*x_stream_stride +
 *           i*x_row_stride and holds d contiguous elements; 16-byte aligned
 *           rows
 *   cache   device arrays (tq_cache); positions outside the written range,
 *           including the other tokens of partially written tiles, keep
 *           their previous contents.
 * Requires tok0 >= 0, tok0 + n_tok <= cache->cap.  n_streams or n_tok may be
 * 0 (nothing is launched). */
tq_status tq_quantize_kv(const tq_spec* spec, const void* tables, int32_t dtype, const void* x,
                         int64_t n_streams, int64_t n_tok, int64_t x_stream_stride,
                         int64_t x_row_stride, int64_t tok0, const tq_cache* cache,
                         void* stream);

/* The same quantization for a ragged batch in one call (one launch for up to
 * 64 sequences with a spec without the QJL stage; a spec with the QJL stage
 * launches once per sequence).  Sequence b (0 <= b < batch) appends n_tok[b]
 * vectors to each of its hkv streams, at positions [tok0[b], tok0[b] +
 * n_tok[b]) of cache streams b*hkv .. b*hkv + hkv - 1 (the stream order
 * tq_attend_decode reads).
 *   x       device; vector i of stream h of sequence b starts at element
 *           x_off[b] + h*x_stream_stride + i*x_row_stride (a padded
 *           [batch][hkv][len][d] tensor and a packed [tokens][hkv][d] one
 *           are both of this form); every offset a multiple of 16 bytes
 *   x_off, tok0, n_tok  HOST int64 arrays [batch], read during the call
 * Requires hkv > 0 and, for every b, tok0[b] >= 0, x_off[b] >= 0 and
 * tok0[b] + n_tok[b] <= cache->cap; sequences with n_tok[b] == 0 are
 * skipped.  Tables, dtype, alignment and the keeping of positions outside
 * the written ranges are as for tq_quantize_kv. */
tq_status tq_quantize_kv_ragged(const tq_spec* spec, const void* tables, int32_t dtype, const void* x,
                                int32_t batch, int32_t hkv, const int64_t* x_off, const int64_t* tok0,
                                const int64_t* n_tok, int64_t x_stream_stride, int64_t x_row_stride,
                                const tq_cache* cache, void* stream);

/* Workspace bytes tq_attend_decode needs for this problem. */
size_t tq_attend_workspace_bytes(const tq_attn* attn);

/* One decode step of attention read directly from the packed cache
 * (noze.it page, section "Il metodo TurboQuant, in breve": inner products are
 * taken against the codebook reconstruction in the rotated domain, plus the
 * sketch's correction of the residual; GitHub issue "Greetings from
 * TurboQuant-MLX & Some Insights to Share!", items 1 and 3: raw sink tokens
 * and skipped values of negligible weight).
 *   ks/ktables/kc  keys: TQ_LAYOUT_RECORD, optional QJL sketch
 *   vs/vtables/vc  values: TQ_LAYOUT_TILED, no QJL
 *   q        device fp32 [batch][hq][d]; batch <= 65535, hq / hkv <= 16
 *   sink_k/sink_v  device bf16 [batch][hkv][sink][d] (NULL iff sink == 0);
 *            sink <= 512
 *   kc->cap and vc->cap must be multiples of 32 and at most 2^24 (one
 *            stream's arrays are addressed with 32-bit offsets).
 *   seq_lens device int32 [batch]: tokens of each sequence including the
 *            sink; compressed token t >= sink lives at cache position t-sink.
 *            Each value must lie in [0, sink + min(kc->cap, vc->cap)] and
 *            not exceed max_len (the kernels clamp a value outside [0,
 *            max_len] into it, so no access leaves the validated cache, but
 *            the output is then unspecified).  A sequence of length 0 gives
 *            zeros.
 *   out      device fp32 [batch][hq][d]
 *   workspace device, >= tq_attend_workspace_bytes(attn) bytes, 16-byte
 *            aligned; no state is kept in it between calls.  Calls that
 *            share a workspace must not run concurrently.
 * Value norms must stay below 2^15 (the weighted values pass through fp16
 * on the way into the matrix cores).
 * scores: s_t = scale * n_t * (<Pi q, c[idx_t]> + sqrt(pi/2)/m * gamma_t *
 * <S Pi q, z_t>) for compressed tokens, scale * <q, k_t> for sink tokens;
 * out = Pi_V^T sum_t w_t n^V_t c_V[idx^V_t] + sum_sink w_t v_t with w the
 * softmax over all tokens.  With v_skip > 0 a compressed token's value is
 * dropped (not renormalised) when exp(s_t - m) < v_skip for the running
 * maximum m of its split, which implies its final weight is below v_skip. */
tq_status tq_attend_decode(const tq_spec* ks, const void* ktables, const tq_cache* kc,
                           const tq_spec* vs, const void* vtables, const tq_cache* vc,
                           const tq_attn* attn, const float* q, const uint16_t* sink_k,
                           const uint16_t* sink_v, const int32_t* seq_lens, float* out,
                           void* workspace, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): the decode step
 * of tq_attend_decode, same arguments and result, without the workspace.  The
 * split partials go to a static device array of TQ_NOALLOC_SCRATCH_BYTES that
 * every GPU the library runs on holds until the process ends; the call itself
 * allocates nothing.  A problem whose tq_attend_workspace_bytes exceeds that
 * size is refused with TQ_E_UNSUPPORTED before any launch.  All calls on one
 * GPU share its array: calls that overlap on one GPU (other streams or
 * threads) race and must be serialised by the caller. */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
tq_status tq_attend_decode_noalloc(const tq_spec* ks, const void* ktables, const tq_cache* kc,
                                   const tq_spec* vs, const void* vtables, const tq_cache* vc,
                                   const tq_attn* attn, const float* q, const uint16_t* sink_k,
                                   const uint16_t* sink_v, const int32_t* seq_lens, float* out, void* stream);

/* Paged cache (a pool of pages shared by all sequences).  A pool of n_pages
 * pages is a tq_cache with cap = TQ_PAGE_TOKENS and n_pages * hkv streams:
 * page p holds TQ_PAGE_TOKENS positions of every kv head h, as stream
 * p * hkv + h.  Compressed token c (= token t - sink) of sequence b lives at
 * position c % TQ_PAGE_TOKENS of page block_table[b * max_pages + c /
 * TQ_PAGE_TOKENS].  The pages of one sequence must be distinct.
 *
 * Quantize into a paged cache: sequence b appends n_tok[b] vectors at
 * compressed positions [pos0[b], pos0[b] + n_tok[b]) (host int64 arrays;
 * pos0[b] + n_tok[b] <= max_pages * TQ_PAGE_TOKENS, else TQ_E_ARG); rows of
 * x as for tq_quantize_kv_ragged.  block_table is DEVICE int32 [batch]
 * [max_pages], 4-byte aligned, read by the kernels; a token whose page lies
 * outside [0, n_pages) (n_pages <= 2^30) is not written, the others are.
 * Only the pages of the written range are read.  The same codes, norms and
 * sketch as tq_quantize_kv_ragged land at the mapped positions.  One launch
 * per 64 sequences (a spec with the sketch: one per sequence). */
tq_status tq_quantize_kv_paged(const tq_spec* spec, const void* tables, int32_t dtype, const void* x,
                               int32_t batch, int32_t hkv, const int64_t* x_off, const int64_t* pos0,
                               const int64_t* n_tok, int64_t x_stream_stride, int64_t x_row_stride,
                               const int32_t* block_table, int32_t max_pages, int64_t n_pages,
                               const tq_cache* pool, void* stream);

/* One decode step over paged K and V pools (same arguments and result as
 * tq_attend_decode, the caches replaced by the pools).  block_table: DEVICE
 * int32 [batch][max_pages]; max_pages * TQ_PAGE_TOKENS >= max_len - sink.
 * A page id outside [0, n_pages) reads as zero codes and norms (no access).
 * kpool->cap and vpool->cap must equal TQ_PAGE_TOKENS. */
tq_status tq_attend_decode_paged(const tq_spec* ks, const void* ktables, const tq_cache* kpool,
                                 const tq_spec* vs, const void* vtables, const tq_cache* vpool,
                                 const tq_attn* attn, const float* q, const uint16_t* sink_k,
                                 const uint16_t* sink_v, const int32_t* seq_lens, const int32_t* block_table,
                                 int32_t max_pages, int64_t n_pages, float* out, void* workspace,
                                 size_t ws_bytes, void* stream);

/* Workspace bytes of tq_ip_scores (the same for every call). */
size_t tq_ip_workspace_bytes(void);

/* Inner-product search over packed vectors (noze.it page, section "Il metodo
 * TurboQuant, in breve": similarity search is the method's second
 * application, and the 1-bit sketch makes the inner-product estimate
 * unbiased).  For queries i < nq, streams s < n_streams and positions
 * t < n_tok of `db`:
 *   scores[i*ld + s*n_tok + t] = n_st (<Pi q_i, c[idx_st]>
 *                                      + sqrt(pi/2)/m gamma_st <S Pi q_i, z_st>),
 * the estimate of <q_i, x_st>; the second term only when spec->qjl_m != 0.
 *   spec/tables/db  TQ_LAYOUT_RECORD vectors as written by tq_quantize_kv;
 *            n_tok <= db->cap, n_tok <= 2^24, n_streams <= 65535
 *   q        device fp32 [nq][d], 1 <= nq <= TQ_IP_MAX_QUERIES
 *   scores   device fp32, 4-byte aligned; ld >= n_streams * n_tok
 *   workspace device, >= tq_ip_workspace_bytes(), 16-byte aligned; calls
 *            that share it must not run concurrently.
 * Two launches on `stream` (the query rotation, then the scores). */
tq_status tq_ip_scores(const tq_spec* spec, const void* tables, const tq_cache* db, int64_t n_streams,
                       int64_t n_tok, const float* q, int32_t nq, float* scores, int64_t ld, void* workspace,
                       size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
