/*
 * tq.h -- C ABI of the TurboQuant hot path on AMD MI355X (gfx950).
 *
 * The library compresses key/value vectors with the two-stage scheme the pages
 * describe and runs decode attention and inner-product search directly on the
 * compressed bytes:
 *   stage 1 ("PolarQuant"): random rotation (sign flip, then Walsh-Hadamard), one
 *     stored fp16 norm, and a precomputed per-coordinate Lloyd-Max codebook with
 *     (b-1) bits -- 163.com explainer (m.163.com/dy/article/KOV7P8JI0556C3J2),
 *     section "第一步：PolarQuant"; Walsh-Hadamard with a random sign flip -- zhidx
 *     turboquant_plus article (course.zhidx.com), section "01 turboquant_plus：介绍与详解";
 *   stage 2 ("QJL"): a 1-bit sign sketch of the residual under a Gaussian
 *     Johnson-Lindenstrauss matrix, giving an unbiased inner-product estimator --
 *     163.com explainer, section "第二步：QJL".
 *
 * Conventions shared by every entry point
 *   - Every function returns int: TQ_OK (0) or a negative TQ_ERR_* code.  Nothing
 *     throws, nothing prints.  tq_strerror() names a code.
 *   - Argument errors are detected on the host before anything is launched; then no
 *     output is touched.
 *   - Device entry points are asynchronous on `stream` (a hipStream_t, NULL = the
 *     null stream).  They never allocate, free or synchronize.  A device-side fault
 *     surfaces at the caller's next synchronization; a failed launch returns
 *     TQ_ERR_HIP.
 *   - The caller owns every buffer.  Pointers marked "device" must be device memory
 *     that stays valid until the stream work that reads it has finished.  Pointers
 *     marked "host" are read during the call only.
 *   - Device pointers must be 16-byte aligned (TQ_ERR_ALIGN otherwise).
 *
 * Packed vector format (tq_format)
 *   d in {128, 256}; coordinates j < split use bits_lo codebook bits, the others
 *   bits_hi (split a multiple of 32; split == d means a single width).  For each block
 *   of 32 coordinates, in order: bits_B code bit-planes (plane p holds bit p of every
 *   code), then one word of QJL sign bits.  Bit i of a word belongs to coordinate
 *   (or projection) 32*block + i; words are little-endian uint32; the words of one
 *   vector are contiguous and vectors are contiguous (tq_record_bytes() bytes each).
 *   Norms live in a separate uint16 array [n][2]: fp16 ||x|| then fp16 ||r||.
 *   With qjl == 0 the sign word of every block is absent (MSE-only record; ||r|| is
 *   still stored).
 *   Supported widths: d = 128: (bits_lo, bits_hi) in {(1,1), (2,2), (3,3), (3,2),
 *   (2,1)}; d = 256: (2,2), (3,3).  The "block-32" layout follows the zhidx article
 *   (section "01 turboquant_plus：介绍与详解").
 *
 * Rotation (tq_tables)
 *   y = H (D x) / sqrt(d): D = diag(signs), H the natural-order Sylvester Hadamard
 *   matrix.  S is the d x d Gaussian JL matrix (row-major fp32, device memory);
 *   sign bit i of a vector is 1 when (S r)_i >= 0, r its rotated-domain residual.
 *   signs and the codebooks are host memory, copied into each launch.
 */
#ifndef TQ_H
#define TQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_OK            0
#define TQ_ERR_ARG      -1  /* null pointer, bad enum, negative size            */
#define TQ_ERR_SHAPE    -2  /* unsupported d / bits / split, hq % hkv, d_in > d */
#define TQ_ERR_ALIGN    -3  /* device pointer not 16-byte aligned               */
#define TQ_ERR_HIP      -4  /* a HIP runtime call or kernel launch failed       */
#define TQ_ERR_NOCONV   -5  /* codebook iteration did not converge              */
#define TQ_ERR_WORKSPACE -6 /* workspace smaller than the *_workspace_bytes size */

#define TQ_F32  0
#define TQ_BF16 1
#define TQ_F16  2

typedef void* tq_stream_t;  /* hipStream_t */

typedef struct tq_format {
  int32_t d;        /* 128 or 256 */
  int32_t bits_lo;  /* codebook bits (b - 1) for coordinates j < split */
  int32_t bits_hi;  /* codebook bits for coordinates j >= split          */
  int32_t split;    /* multiple of 32, 0 < split <= d                    */
  int32_t qjl;      /* 1: one QJL sign word per block; 0: MSE-only ("PolarQuant
                       alone", no residual sketch: juejin post, section "第二步：QJL"
                       names QJL as the bias fix on top of the MSE stage)        */
  int32_t layout;   /* 0: per-vector records (above).  1: token-sliced (d = 128, QJL
                       formats): the same bits grouped by 32 consecutive vectors; within
                       a group, for each coordinate j in order, the words of j (its code
                       bit-planes, then its sign bit), bit t of a word belonging to vector
                       32 * group + t.  A group is 32 * tq_record_bytes() bytes.  Only
                       tq_quantize_kv writes it (n a multiple of 32) and only
                       tq_attend_decode reads it (for the values, keys in layout 0);
                       every other entry point returns TQ_ERR_SHAPE for layout 1.     */
} tq_format;

typedef struct tq_tables {
  const float* centroids_lo;  /* host, 2^bits_lo ascending fp32 (tq_build_codebook) */
  const float* bounds_lo;     /* host, 2^bits_lo - 1 ascending fp32                  */
  const float* centroids_hi;  /* host, 2^bits_hi (may equal the lo pointers)         */
  const float* bounds_hi;     /* host, 2^bits_hi - 1                                 */
  const int8_t* signs;        /* host, d entries, each +1 or -1                      */
  const float* S;             /* device, d x d row-major fp32                        */
} tq_tables;

/* Lloyd-Max codebook for one coordinate of a uniformly random unit vector in R^d
 * (density proportional to (1 - t^2)^((d-3)/2) on [-1, 1]) with 2^bits levels: the
 * fixed table that is computed once and looked up online (163.com explainer,
 * section "第一步：PolarQuant").  Host only, synchronous, deterministic.
 *   d        : power of two, 8 <= d <= 4096
 *   bits     : 1..4
 *   centroids: out, host, 2^bits fp32, ascending, exactly mirror-symmetric
 *   bounds   : out, host, 2^bits - 1 fp32 midpoints of adjacent centroids
 *   mse      : out, host, nullable: expected squared error per coordinate
 * Errors: TQ_ERR_ARG, TQ_ERR_SHAPE, TQ_ERR_NOCONV. */
int tq_build_codebook(int32_t d, int32_t bits, float* centroids, float* bounds, double* mse);

/* Seeded draws of the rotation: the +-1 diagonal D of y = H (D x) / sqrt(d) and the d x d
 * Gaussian JL matrix S (163.com explainer, sections "第一步：PolarQuant" (random rotation)
 * and "第二步：QJL" (JL transform of the residual)).  The pages name no generator; this one
 * is counter-based, so (d, seed) names the same tables on every machine:
 *   x_k  = output k of SplitMix64 started at state `seed`;  u(x) = (x >> 11) * 2^-53;
 *   signs[i] = +1 if the top bit of x_i is 0, else -1 (i = 0 .. d-1);
 *   then, for the entries of S in row-major order two at a time, the next two draws give
 *   u1 = 1 - u(x_a), u2 = u(x_b), and in fp64 (Box-Muller) r = sqrt(-2 ln u1),
 *   a = 2 pi u2; S[2k] = fp32(r cos a), S[2k+1] = fp32(r sin a), rounded to nearest even.
 * Host only, synchronous, deterministic.  The caller copies S to device memory for
 * tq_tables.S.
 *   d     : power of two, 8 <= d <= 4096
 *   signs : out, host, d int8 entries (+1 / -1)
 *   S     : out, host, d * d fp32, row-major
 * Errors: TQ_ERR_SHAPE (d), TQ_ERR_ARG (null pointer). */
int tq_make_rotation(int32_t d, uint64_t seed, int8_t* signs, float* S);

/* Bytes of one packed vector's code words (norms excluded); < 0 on a bad format. */
int64_t tq_record_bytes(const tq_format* fmt);

/* TQ_OK when the kernels support `fmt`, else TQ_ERR_ARG / TQ_ERR_SHAPE. */
int tq_check_format(const tq_format* fmt);

/* Quantize n vectors (rotation, norm, codebook encode, residual, QJL signs, pack).
 * Each vector is compressed independently with no calibration input (163.com
 * explainer, sections "TurboQuant 怎么做的" and "四个工程属性").
 *   x        : device, n rows of d_in elements (dtype x_dtype: TQ_F32 / TQ_BF16 /
 *              TQ_F16), row stride ld_x elements; coordinates d_in..d-1 are zero
 *   codes    : device out, n * tq_record_bytes(fmt) bytes
 *   norms    : device out, n * 2 uint16 (fp16 ||x||, fp16 ||r||)
 *   counters : device, nullable, 4 int64 the call ADDS to (caller zeroes):
 *              [0] coordinates within 1e-6 of a codebook boundary,
 *              [1] projections with |S r/||r|| |_i < 1e-6 (after fp64 recheck),
 *              [2] projections rechecked in fp64 (|.| < 1e-5 in fp32),
 *              [3] vectors whose norm overflowed fp16 (stored as +inf)
 * n == 0 is a no-op.  Errors: TQ_ERR_ARG, TQ_ERR_SHAPE, TQ_ERR_ALIGN, TQ_ERR_HIP. */
int tq_quantize_kv(const tq_format* fmt, const tq_tables* tab, const void* x, int32_t x_dtype,
                   int64_t n, int32_t d_in, int64_t ld_x, void* codes, uint16_t* norms,
                   int64_t* counters, tq_stream_t stream);

/* Workspace bytes tq_attend_decode needs for this shape. */
int64_t tq_attend_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv, int64_t capacity,
                                  int32_t d);

/* One decode step of attention straight from the packed cache: logits by the
 * unbiased estimator n16 <q_rot, c[idx]> + gamma r16 <S q_rot, 2 sigma - 1>, times
 * `scale`; softmax; value rows dequantized and accumulated in the rotated domain
 * and rotated back once per head (163.com explainer, sections "第二步：QJL" and
 * "速度").  Grouped-query layout: query head h reads KV head h / (hq / hkv).
 *   fk, tk / fv, tv : formats and tables of the key and value caches (asymmetric
 *              K/V widths allowed: zhidx article, section "01 turboquant_plus：介绍与详解")
 *   q        : device [batch][hq][d], dtype q_dtype (TQ_F32 / TQ_BF16 / TQ_F16)
 *   codes_k  : device [batch][hkv][capacity] records of tq_record_bytes(fk) bytes
 *   norms_k  : device [batch][hkv][capacity][2] uint16
 *   codes_v, norms_v : the same for values with fv
 *   seq_lens : device int32 [batch], each in [0, capacity]; tokens t < seq_len attend
 *   scale    : logit scale, normally 1/sqrt(d)
 *   tau      : Sparse-V gate (zhidx article, section "01 turboquant_plus：介绍与详解"):
 *              0 disables it; otherwise a value row's contribution to head h is
 *              dropped when its running softmax weight estimate is < tau.  The
 *              estimate bounds the final weight from above, so only rows whose
 *              final weight is < tau are dropped; the softmax denominator keeps
 *              every row.  A row dropped by all heads of its group is not read.
 *   out      : device out fp32 [batch][hq][d]
 *   logits   : device out, nullable, fp32 [batch][hq][capacity] (scaled logits for
 *              t < seq_len; other entries untouched)
 *   skipped  : device, nullable, int64 the call ADDS the number of value rows it
 *              did not read to
 *   workspace: device, >= tq_attend_workspace_bytes(...) bytes, no initial contents
 *              (split partials); calls that share a workspace must not overlap in time
 * Errors: TQ_ERR_ARG, TQ_ERR_SHAPE (d != 128, hq % hkv, unsupported widths),
 * TQ_ERR_ALIGN, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
int tq_attend_decode(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                     const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch,
                     int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                     const void* codes_v, const uint16_t* norms_v, int64_t capacity,
                     const int32_t* seq_lens, float scale, float tau, float* out,
                     float* logits, int64_t* skipped, void* workspace,
                     int64_t workspace_bytes, tq_stream_t stream);

/* tq_attend_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments
 * without a workspace, the same kernels and results.  The split partials go to a device
 * array of 8 MiB inside the library, one per GPU, held until the process ends; the call
 * allocates nothing.  Every call on a GPU shares that GPU's array, so calls that overlap in
 * time on one GPU (other streams, other threads) race and must be ordered by the caller.
 * Errors: as tq_attend_decode; TQ_ERR_WORKSPACE when tq_attend_workspace_bytes for the
 * shape exceeds 8 MiB; TQ_ERR_HIP when the array's device address cannot be obtained. */
int tq_attend_decode_noalloc(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                             const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch,
                             int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                             const void* codes_v, const uint16_t* norms_v, int64_t capacity,
                             const int32_t* seq_lens, float scale, float tau, float* out,
                             float* logits, int64_t* skipped, tq_stream_t stream);

/* Decode over a cache kept in segments of different formats, as temporal decay leaves
 * it (zhidx article, section "01 turboquant_plus：介绍与详解": older tokens drop to a
 * narrower format, e.g. re-encoded in place by tq_requantize, while new ones are
 * written at full width).  Each query attends to the concatenation of its tokens in
 * segment 0, then segment 1, ...: one softmax over all of them.
 *   segs     : host array of n_seg (1..8) segments; segment s holds its own key and value
 *              formats and tables and its packed records [batch][hkv][capacity] with
 *              norms, and seq_lens (device int32 [batch], each in [0, capacity]).
 *              Key formats and tables may differ between segments.  Value tables must
 *              share one rotation (the same S device array and equal sign diagonals),
 *              since every segment's value sums are mapped back once; their codebook
 *              widths may differ.
 *   q, q_dtype, batch, hq, hkv, scale, tau, out, skipped : as tq_attend_decode
 *   workspace: device, >= tq_attend_segments_workspace_bytes(...) bytes
 * Errors: as tq_attend_decode; TQ_ERR_ARG for n_seg outside 1..8, a null segment
 * array or value tables of different rotations. */
typedef struct {
  const tq_format* fk;
  const tq_tables* tk;
  const tq_format* fv;
  const tq_tables* tv;
  const void* codes_k;
  const uint16_t* norms_k;
  const void* codes_v;
  const uint16_t* norms_v;
  int64_t capacity;
  const int32_t* seq_lens;
} tq_cache_segment;

/* Workspace bytes tq_attend_decode_segments needs; capacities: host array [n_seg]. */
int64_t tq_attend_segments_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv,
                                           int32_t n_seg, const int64_t* capacities, int32_t d);

int tq_attend_decode_segments(const tq_cache_segment* segs, int32_t n_seg, const void* q,
                              int32_t q_dtype, int32_t batch, int32_t hq, int32_t hkv,
                              float scale, float tau, float* out, int64_t* skipped,
                              void* workspace, int64_t workspace_bytes, tq_stream_t stream);

/* Paged cache.  A cache of fixed-size pages, as serving engines keep it: codes
 * [num_pages][hkv][page_size] records and norms [num_pages][hkv][page_size][2] uint16;
 * a sequence's token t lives in page block_table[b][t / page_size] at offset
 * t % page_size.  page_size is a power of two in [64, 2^20].
 *
 * Append (quantize-on-write): quantize the keys or values of n_tokens new tokens and
 * write each one's records into its slot.
 *   x            : device, n_tokens * hkv rows of d_in elements ([token][kv head] order),
 *                  dtype x_dtype, row stride ld_x elements
 *   slot_mapping : device int64 [n_tokens]: page * page_size + offset of each token; a
 *                  negative slot, or one >= num_pages * page_size, is not written.  Two
 *                  tokens must not share a slot.
 *   codes_cache, norms_cache : device, the paged cache (only the slots written change)
 *   counters     : as for tq_quantize_kv
 * Errors: as tq_quantize_kv, and TQ_ERR_ARG for a bad page_size / num_pages / hkv. */
int tq_quantize_kv_paged(const tq_format* fmt, const tq_tables* tab, const void* x,
                         int32_t x_dtype, int64_t n_tokens, int32_t hkv, int32_t d_in,
                         int64_t ld_x, const int64_t* slot_mapping, int32_t page_size,
                         int64_t num_pages, void* codes_cache, uint16_t* norms_cache,
                         int64_t* counters, tq_stream_t stream);

/* tq_attend_decode over paged caches.  block_table: device int32 [batch][max_blocks]
 * page ids; the logical capacity is max_blocks * page_size (seq_lens are clamped to it,
 * logits are laid out [batch][hq][capacity], and the workspace is
 * tq_attend_workspace_bytes(batch, hq, hkv, max_blocks * page_size, 128)).  A page id
 * outside [0, num_pages) makes its tokens absent (they take no part in the softmax).
 * Errors: as tq_attend_decode, and TQ_ERR_ARG for a bad page_size / num_pages /
 * max_blocks or a null block_table. */
int tq_attend_decode_paged(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                           const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch,
                           int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                           const void* codes_v, const uint16_t* norms_v, int32_t page_size,
                           int64_t num_pages, const int32_t* block_table, int32_t max_blocks,
                           const int32_t* seq_lens, float scale, float tau, float* out,
                           float* logits, int64_t* skipped, void* workspace,
                           int64_t workspace_bytes, tq_stream_t stream);

/* Workspace bytes tq_prefill_paged needs for a chunk of n_new tokens starting at `start`. */
int64_t tq_prefill_workspace_bytes(int32_t n_new, int32_t hq, int32_t hkv, int64_t start);

/* One prefill chunk of one sequence on a paged cache: the chunk's new keys and values are
 * quantized and written at positions start .. start + n_new - 1 of the sequence (the
 * step before decode: quantize-on-write), then each new query attends with the decode
 * estimator, softmax and value sum to the cached tokens at or before its own position --
 * causal attention over the compressed cache.  The attention runs on MFMA with fp16
 * operands (the query rows q_rot and gamma S q_rot, the dequantized n16 c[idx] and
 * +-r16, the softmax weights) and fp32 accumulation.  Any d = 128 formats; the keys must
 * carry QJL.
 *   q            : device [n_new][hq][128], dtype q_dtype
 *   k_new, v_new : device [n_new][hkv] rows of 128 elements, dtype kv_dtype, row stride
 *                  ld_kv elements
 *   start        : position of the chunk's first token (the tokens before it are cached)
 *   block_table  : device int32 [max_blocks], the sequence's pages; positions up to
 *                  start + n_new - 1 must have a page
 *   out          : device out fp32 [n_new][hq][128]
 *   counters     : as for tq_quantize_kv (both tensors add to it), nullable
 *   workspace    : device, 256-byte aligned, >= tq_prefill_workspace_bytes(n_new, hq, hkv,
 *                  start)
 * Errors: as tq_quantize_kv_paged and tq_attend_decode_paged; TQ_ERR_SHAPE when
 * start + n_new exceeds max_blocks * page_size.  Nothing is written when the arguments
 * are rejected. */
int tq_prefill_paged(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                     const tq_tables* tv, const void* q, int32_t q_dtype, int32_t n_new,
                     int32_t hq, int32_t hkv, const void* k_new, const void* v_new,
                     int32_t kv_dtype, int64_t ld_kv, int64_t start, void* codes_k,
                     uint16_t* norms_k, void* codes_v, uint16_t* norms_v, int32_t page_size,
                     int64_t num_pages, const int32_t* block_table, int32_t max_blocks, float scale,
                     float* out, int64_t* counters, void* workspace, int64_t workspace_bytes,
                     tq_stream_t stream);

/* Workspace bytes tq_ip_search needs. */
int64_t tq_search_workspace_bytes(int64_t n_q, int32_t k, int64_t n_db, int32_t d);

/* Exhaustive top-k inner-product search over a packed database: score_i =
 * n16_i <q_rot, c[idx_i]> + gamma r16_i <S q_rot, 2 sigma_i - 1>, the same estimator
 * (163.com explainer, section "向量搜索").  Larger scores first; equal scores go to
 * the lower id.
 *   codes_db, norms_db : device, n_db packed vectors of format fmt
 *   queries  : device fp32 [n_q][d_in], d_in <= d (zero-padded to d)
 *   k        : 1..64, k <= n_db
 *   out_ids  : device out int64 [n_q][k]
 *   out_scores: device out fp32 [n_q][k]
 *   workspace: device, >= tq_search_workspace_bytes(n_q, k, n_db, fmt->d)
 * Errors: TQ_ERR_ARG, TQ_ERR_SHAPE, TQ_ERR_ALIGN, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
int tq_ip_search(const tq_format* fmt, const tq_tables* tab, const void* codes_db,
                 const uint16_t* norms_db, int64_t n_db, const float* queries, int32_t d_in,
                 int64_t n_q, int32_t k, int64_t* out_ids, float* out_scores,
                 void* workspace, int64_t workspace_bytes, tq_stream_t stream);

/* Workspace bytes tq_requantize uses to re-encode n vectors in one pass (n * 580 for
 * d = 128: per vector one fp32 row of the reconstruction, a copy of its record and of its
 * norms).  A smaller workspace is allowed: the call then works in chunks of
 * workspace_bytes / 580 vectors. */
int64_t tq_requantize_workspace_bytes(int64_t n, int32_t d);

/* Temporal decay (zhidx article, section "01 turboquant_plus：介绍与详解": older tokens
 * drop to lower precision): re-encode n stored vectors at another format.  Each record's
 * reconstruction in the rotated domain, y~ = n16 c[idx] + gamma r16 S_in^T (2 sigma - 1)
 * (the sign term only when f_in has QJL), is encoded again by the steps of
 * tq_quantize_kv that follow the rotation: norm ||y~||, codes of f_out, residual and
 * (with f_out QJL) its signs under t_out->S.  Both formats share the rotation, so the
 * tables must hold the same sign flips (t_in->S and t_out->S may differ).
 *   f_in, t_in   : format and tables of the stored records, d = 128
 *   codes_in     : device, n records of tq_record_bytes(f_in) bytes
 *   norms_in     : device, n * 2 uint16
 *   f_out, t_out : the new format and tables, d = 128
 *   codes_out    : device out, n * tq_record_bytes(f_out) bytes; may equal codes_in
 *                  (in place) when tq_record_bytes(f_out) <= tq_record_bytes(f_in)
 *   norms_out    : device out, n * 2 uint16; may equal norms_in
 *                  Any other overlap between inputs and outputs is an error.
 *   counters     : as for tq_quantize_kv, nullable
 *   workspace    : device, >= 580 bytes (see tq_requantize_workspace_bytes); no
 *                  initial contents; calls that share it must not overlap in time
 * The stored norm, codes and signs are those of the exact (fp64) reconstruction outside
 * the windows the quantize path has: decisions the fp32 reconstruction leaves within
 * reach of a boundary are recomputed in fp64 from the stored record.
 * n == 0 is a no-op.  Errors: TQ_ERR_ARG (null pointers, different sign flips, bad
 * overlap), TQ_ERR_SHAPE (d != 128), TQ_ERR_ALIGN, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
int tq_requantize(const tq_format* f_in, const tq_tables* t_in, const void* codes_in,
                  const uint16_t* norms_in, int64_t n, const tq_format* f_out,
                  const tq_tables* t_out, void* codes_out, uint16_t* norms_out,
                  int64_t* counters, void* workspace, int64_t workspace_bytes,
                  tq_stream_t stream);

/* Static string naming a status code. */
const char* tq_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
