// Internal launch entry points behind the C ABI (not exported in tq.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

// Compute units of the current device; <= 0 on failure.
int tq_num_cus();

// Paged destination of a quantize launch: vector v = token * page_heads + head is written
// to row (page * page_heads + head) * 2^page_log2 + offset of the cache.
struct tq_paged_dst {
  const int64_t* slots;   // device, one slot per token; or null and:
  int64_t num_pages;
  int32_t page_heads, page_log2;
  const int32_t* block_table;  // the sequence's page list, token i at position pos0 + i
  int64_t pos0;
  int32_t max_blocks;
};

int tq_launch_quantize(const tq_format* f, const tq_tables* t, const void* x, int32_t x_dtype,
                       int64_t n, int32_t d_in, int64_t ld_x, void* codes, uint16_t* norms,
                       int64_t* counters, hipStream_t stream, const tq_paged_dst* paged = nullptr);

// Rewrite n (a multiple of 32) freshly quantized records in place as token-sliced groups.
int tq_launch_tiles(const tq_format* f, void* codes, int64_t n, hipStream_t stream);

struct tq_decode_plan {
  int32_t n_split;        // token splits per (batch, kv head)
  int32_t waves;          // waves per scan workgroup
  int32_t parts;          // partial results per (batch, q head) = n_split
  int64_t tokens_per_split;
  int64_t units;          // (batch, kv head, chunk) units = scan grid height
  int64_t ws_part_off;    // byte offset of the split partials inside the workspace
  int64_t ws_bytes;
};

// Key/value format pairs the decode kernels are instantiated for.
bool tq_decode_formats_supported(const tq_format* fk, const tq_format* fv);

tq_decode_plan tq_plan_decode(int32_t batch, int32_t hq, int32_t hkv, int64_t capacity, int32_t d);

// Paged source of a decode launch (see DecodeParams).
struct tq_paged_src {
  const int32_t* block_table;  // device [batch][bt_stride]
  int64_t num_pages;
  int32_t max_blocks, page_log2;
  int32_t bt_stride;           // 0: all queries share row 0
  int64_t causal_start;        // >= 0: query b sees tokens <= causal_start + b
};

int tq_launch_decode(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                     const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch,
                     int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                     const void* codes_v, const uint16_t* norms_v, int64_t capacity,
                     const int32_t* seq_lens, float scale, float tau, float* out, float* logits,
                     int64_t* skipped, void* workspace, const tq_decode_plan& plan,
                     hipStream_t stream, const tq_paged_src* paged = nullptr,
                     int32_t split_base = 0, int32_t split_total = 0, bool combine = true);

// Decode with token-sliced values (keys per-vector): the fp8 x fp4 MFMA scan + combine.
bool tq_decode_mx_supported(const tq_format* fk, const tq_format* fv);
tq_decode_plan tq_plan_decode_mx(int32_t batch, int32_t hq, int32_t hkv, int64_t capacity);
int tq_launch_decode_mx(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                        const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch,
                        int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                        const void* codes_v, const uint16_t* norms_v, int64_t capacity,
                        const int32_t* seq_lens, float scale, float tau, float* out,
                        float* logits, int64_t* skipped, void* workspace,
                        const tq_decode_plan& plan, hipStream_t stream);

// Two decode segments in one fused scan launch + one combine, when their format pairs have
// a fused instance; TQ_ERR_SHAPE (nothing launched) otherwise.  Arguments checked by the caller.
int tq_launch_decode_pair(const tq_cache_segment* segs, const void* q, int32_t q_dtype,
                          int32_t batch, int32_t hq, int32_t hkv, float scale, float tau,
                          float* out, int64_t* skipped, void* workspace, hipStream_t stream);

struct tq_search_plan {
  int32_t n_chunks;       // database chunks scanned independently
  int64_t chunk_len;
  int64_t ws_q_off, ws_cand_off, ws_bytes;
};

tq_search_plan tq_plan_search(int64_t n_q, int32_t k, int64_t n_db, int32_t d);

int tq_launch_search(const tq_format* f, const tq_tables* t, const void* codes_db,
                     const uint16_t* norms_db, int64_t n_db, const float* queries, int32_t d_in,
                     int64_t n_q, int32_t k, int64_t* out_ids, float* out_scores,
                     void* workspace, const tq_search_plan& plan, hipStream_t stream);

// Workspace bytes per vector of a tq_requantize chunk (d = 128): fp32 row, record copy of
// at most 16 words, norms.
constexpr int64_t tq_requant_vector_bytes() { return 128 * 4 + 64 + 4; }

int tq_launch_requant(const tq_format* fi, const tq_tables* ti, const void* codes_in,
                      const uint16_t* norms_in, int64_t n, const tq_format* fo,
                      const tq_tables* to, void* codes_out, uint16_t* norms_out,
                      int64_t* counters, void* workspace, int64_t workspace_bytes,
                      hipStream_t stream);

struct tq_prefill_plan {
  int32_t n_split;         // key splits
  int64_t keys_per_split;  // multiple of 64
  int64_t row_blocks;      // 64-row blocks per KV head
  int64_t ws_q_off, ws_part_off, ws_bytes;
};

tq_prefill_plan tq_plan_prefill(int32_t n_new, int32_t hq, int32_t hkv, int64_t start);

int tq_launch_prefill(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                      const tq_tables* tv, const void* q, int32_t q_dtype, int32_t n_new,
                      int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                      const void* codes_v, const uint16_t* norms_v, int32_t page_log2,
                      int64_t num_pages, const int32_t* block_table, int32_t max_blocks,
                      int64_t start, float scale, float* out, void* workspace,
                      const tq_prefill_plan& pl, hipStream_t stream);

// Walsh coefficients alpha_S = 2^-B sum_idx c[idx] prod_{k in S} (2 b_k(idx) - 1) for the odd
// subsets S in the order the scan reads the planes: {0}, {1}, {2}, {0,1,2}.
inline void tq_walsh_coeffs(int bits, const float* c, float* alpha) {
  const int L = 1 << bits;
  const int subsets[4] = {1, 2, 4, 7};
  for (int k = 0; k < 4; ++k) alpha[k] = 0.0f;
  const int nw = bits == 3 ? 4 : bits;
  for (int k = 0; k < nw; ++k) {
    double s = 0.0;
    for (int idx = 0; idx < L; ++idx) {
      double prod = 1.0;
      for (int bit = 0; bit < bits; ++bit)
        if ((subsets[k] >> bit) & 1) prod *= ((idx >> bit) & 1) ? 1.0 : -1.0;
      s += (double)c[idx] * prod;
    }
    alpha[k] = (float)(s / L);
  }
}
