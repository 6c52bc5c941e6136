// C ABI: argument validation and dispatch.  Every check runs on the host before any
// launch; nothing here allocates, frees or synchronizes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <mutex>

#include "tq.h"
#include "tq_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_widths(int d, int lo, int hi) {
  if (d == 128)
    return (lo == hi && lo >= 1 && lo <= 3) || (lo == 3 && hi == 2) || (lo == 2 && hi == 1);
  if (d == 256) return lo == hi && (lo == 2 || lo == 3);
  return false;
}

// The kernels use the positive half of a codebook and mirror it, so tables must be
// exactly symmetric, ascending, and the middle boundary must be 0.
int check_codebook(int bits, const float* c, const float* b) {
  if (!c || !b) return TQ_ERR_ARG;
  const int L = 1 << bits;
  for (int m = 0; m < L; ++m) {
    if (!std::isfinite(c[m]) || c[m] != -c[L - 1 - m]) return TQ_ERR_ARG;
    if (m + 1 < L && !(c[m] < c[m + 1])) return TQ_ERR_ARG;
  }
  for (int m = 0; m + 1 < L; ++m) {
    if (b[m] != -b[L - 2 - m]) return TQ_ERR_ARG;
    if (!(c[m] <= b[m] && b[m] <= c[m + 1])) return TQ_ERR_ARG;
  }
  return TQ_OK;
}

int check_tables(const tq_format* f, const tq_tables* t) {
  if (!t || !t->signs || !t->S) return TQ_ERR_ARG;
  if (!aligned(t->S, 16)) return TQ_ERR_ALIGN;
  for (int j = 0; j < f->d; ++j)
    if (t->signs[j] != 1 && t->signs[j] != -1) return TQ_ERR_ARG;
  int rc = check_codebook(f->bits_lo, t->centroids_lo, t->bounds_lo);
  if (rc) return rc;
  return check_codebook(f->bits_hi, t->centroids_hi, t->bounds_hi);
}

bool dtype_ok(int dt) { return dt == TQ_F32 || dt == TQ_BF16 || dt == TQ_F16; }

// log2 of a page size that is a power of two in [64, 2^20], else -1
int page_log2(int32_t page_size) {
  if (page_size < 64 || page_size > (1 << 20) || (page_size & (page_size - 1))) return -1;
  int lg = 0;
  while ((1 << lg) < page_size) ++lg;
  return lg;
}

int quantize_checked(const tq_format* f, const tq_tables* t, const void* x, int32_t x_dtype,
                     int64_t n, int32_t d_in, int64_t ld_x, void* codes, uint16_t* norms,
                     int64_t* counters, tq_stream_t stream, const tq_paged_dst* paged,
                     bool launch = true);
int decode_checked(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                   const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch, int32_t hq,
                   int32_t hkv, const void* codes_k, const uint16_t* norms_k, const void* codes_v,
                   const uint16_t* norms_v, int64_t capacity, const int32_t* seq_lens, float scale,
                   float tau, float* out, float* logits, int64_t* skipped, void* workspace,
                   int64_t workspace_bytes, tq_stream_t stream, const tq_paged_src* paged,
                   bool launch = true);
uintptr_t dtype_size(int dt) { return dt == TQ_F32 ? 4 : 2; }

// Split-partial array of tq_attend_decode_noalloc: one copy per GPU, held until the process
// ends.  Host code never uses the name `scratch` as an address (on the host it is only a
// stand-in for the device symbol): its device address is asked of the runtime once per
// device, with that device current, and kept.
constexpr int64_t kNoAllocScratchBytes = int64_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

void* noalloc_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

int tq_num_cus() {
  // asked of the runtime on every call (it keeps the device properties), so the library
  // holds no mutable state of its own here
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return n;
}

extern "C" {

int tq_check_format(const tq_format* f) {
  if (!f) return TQ_ERR_ARG;
  if (f->d != 128 && f->d != 256) return TQ_ERR_SHAPE;
  if (f->split <= 0 || f->split > f->d || (f->split % 32)) return TQ_ERR_SHAPE;
  const int hi = (f->split == f->d) ? f->bits_lo : f->bits_hi;
  if (f->split == f->d && f->bits_hi != f->bits_lo) return TQ_ERR_SHAPE;
  if (!supported_widths(f->d, f->bits_lo, hi)) return TQ_ERR_SHAPE;
  if (f->qjl != 0 && f->qjl != 1) return TQ_ERR_ARG;
  if (f->layout != 0 && f->layout != 1) return TQ_ERR_ARG;
  if (f->layout == 1 && (f->d != 128 || !f->qjl)) return TQ_ERR_SHAPE;
  return TQ_OK;
}

int64_t tq_record_bytes(const tq_format* f) {
  if (tq_check_format(f) != TQ_OK) return -1;
  const int lo_blocks = f->split / 32, hi_blocks = (f->d - f->split) / 32;
  return 4 * ((int64_t)lo_blocks * (f->bits_lo + f->qjl) + (int64_t)hi_blocks * (f->bits_hi + f->qjl));
}

int tq_quantize_kv(const tq_format* f, const tq_tables* t, const void* x, int32_t x_dtype,
                   int64_t n, int32_t d_in, int64_t ld_x, void* codes, uint16_t* norms,
                   int64_t* counters, tq_stream_t stream) {
  return quantize_checked(f, t, x, x_dtype, n, d_in, ld_x, codes, norms, counters, stream, nullptr);
}

int tq_quantize_kv_paged(const tq_format* f, const tq_tables* t, const void* x, int32_t x_dtype,
                         int64_t n_tokens, int32_t hkv, int32_t d_in, int64_t ld_x,
                         const int64_t* slot_mapping, int32_t page_size, int64_t num_pages,
                         void* codes_cache, uint16_t* norms_cache, int64_t* counters,
                         tq_stream_t stream) {
  const int lg = page_log2(page_size);
  if (lg < 0 || num_pages < 1 || hkv < 1 || n_tokens < 0) return TQ_ERR_ARG;
  if (n_tokens > 0 && !slot_mapping) return TQ_ERR_ARG;
  if (slot_mapping && !aligned(slot_mapping, 8)) return TQ_ERR_ALIGN;
  const tq_paged_dst dst{slot_mapping, num_pages, hkv, lg, nullptr, 0, 0};
  return quantize_checked(f, t, x, x_dtype, n_tokens * hkv, d_in, ld_x, codes_cache, norms_cache,
                          counters, stream, &dst);
}

}  // extern "C"

namespace {
int quantize_checked(const tq_format* f, const tq_tables* t, const void* x, int32_t x_dtype,
                     int64_t n, int32_t d_in, int64_t ld_x, void* codes, uint16_t* norms,
                     int64_t* counters, tq_stream_t stream, const tq_paged_dst* paged,
                     bool launch) {
  int rc = tq_check_format(f);
  if (rc) return rc;
  if (n < 0 || !dtype_ok(x_dtype)) return TQ_ERR_ARG;
  if (d_in <= 0 || d_in > f->d || ld_x < d_in) return TQ_ERR_SHAPE;
  if (f->layout == 1 && (paged || n % 32)) return TQ_ERR_SHAPE;
  rc = check_tables(f, t);
  if (rc) return rc;
  if (n == 0) return TQ_OK;
  if (!x || !codes || !norms) return TQ_ERR_ARG;
  if (!aligned(x, dtype_size(x_dtype)) || !aligned(codes, 16) || !aligned(norms, 4) ||
      (counters && !aligned(counters, 8)))
    return TQ_ERR_ALIGN;
  if (!launch) return TQ_OK;
  rc = tq_launch_quantize(f, t, x, x_dtype, n, d_in, ld_x, codes, norms, counters,
                          reinterpret_cast<hipStream_t>(stream), paged);
  if (rc || f->layout != 1) return rc;
  return tq_launch_tiles(f, codes, n, reinterpret_cast<hipStream_t>(stream));
}
}  // namespace

extern "C" {

int64_t tq_attend_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv, int64_t capacity,
                                  int32_t d) {
  if (batch <= 0 || hq <= 0 || hkv <= 0 || capacity < 0 || d != 128 || hq % hkv) return -1;
  return tq_plan_decode(batch, hq, hkv, capacity, d).ws_bytes;
}

int tq_attend_decode(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                     const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch,
                     int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                     const void* codes_v, const uint16_t* norms_v, int64_t capacity,
                     const int32_t* seq_lens, float scale, float tau, float* out,
                     float* logits, int64_t* skipped, void* workspace,
                     int64_t workspace_bytes, tq_stream_t stream) {
  return decode_checked(fk, tk, fv, tv, q, q_dtype, batch, hq, hkv, codes_k, norms_k, codes_v,
                        norms_v, capacity, seq_lens, scale, tau, out, logits, skipped, workspace,
                        workspace_bytes, stream, nullptr);
}

int tq_attend_decode_noalloc(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                             const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch,
                             int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                             const void* codes_v, const uint16_t* norms_v, int64_t capacity,
                             const int32_t* seq_lens, float scale, float tau, float* out,
                             float* logits, int64_t* skipped, tq_stream_t stream) {
  int rc = tq_check_format(fk);
  if (rc) return rc;
  if ((rc = tq_check_format(fv))) return rc;
  if (batch <= 0 || hq <= 0 || hkv <= 0 || capacity < 0 || hq % hkv) return TQ_ERR_ARG;
  // the split partials must fit the library's own device array
  const tq_decode_plan plan = fv->layout == 1 ? tq_plan_decode_mx(batch, hq, hkv, capacity)
                                              : tq_plan_decode(batch, hq, hkv, capacity, fk->d);
  if (plan.ws_bytes > kNoAllocScratchBytes) return TQ_ERR_WORKSPACE;
  void* ws = noalloc_scratch();
  if (!ws) return TQ_ERR_HIP;
  return decode_checked(fk, tk, fv, tv, q, q_dtype, batch, hq, hkv, codes_k, norms_k, codes_v,
                        norms_v, capacity, seq_lens, scale, tau, out, logits, skipped, ws,
                        kNoAllocScratchBytes, stream, nullptr);
}

int64_t tq_attend_segments_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv,
                                           int32_t n_seg, const int64_t* capacities, int32_t d) {
  if (batch <= 0 || hq <= 0 || hkv <= 0 || d != 128 || hq % hkv) return -1;
  if (n_seg < 1 || n_seg > 8 || !capacities) return -1;
  // the segments' split partials side by side: each plan's partial array, summed
  int64_t bytes = 0;
  for (int s = 0; s < n_seg; ++s) {
    if (capacities[s] < 0) return -1;
    bytes += tq_plan_decode(batch, hq, hkv, capacities[s], d).ws_bytes;
  }
  return bytes;
}

int tq_attend_decode_segments(const tq_cache_segment* segs, int32_t n_seg, const void* q,
                              int32_t q_dtype, int32_t batch, int32_t hq, int32_t hkv,
                              float scale, float tau, float* out, int64_t* skipped,
                              void* workspace, int64_t workspace_bytes, tq_stream_t stream) {
  if (!segs || n_seg < 1 || n_seg > 8) return TQ_ERR_ARG;
  int64_t caps[8];
  for (int s = 0; s < n_seg; ++s) {
    const tq_cache_segment& g = segs[s];
    if (!g.fk || !g.tk || !g.fv || !g.tv) return TQ_ERR_ARG;
    if (g.fk->layout != 0 || g.fv->layout != 0) return TQ_ERR_SHAPE;
    // every argument check of a plain decode, except the workspace size
    const int rc = decode_checked(g.fk, g.tk, g.fv, g.tv, q, q_dtype, batch, hq, hkv, g.codes_k,
                                  g.norms_k, g.codes_v, g.norms_v, g.capacity, g.seq_lens, scale,
                                  tau, out, nullptr, skipped, workspace, INT64_MAX, stream,
                                  nullptr, false);
    if (rc) return rc;
    // the value sums of all segments are mapped back with one rotation
    if (g.tv->S != segs[0].tv->S) return TQ_ERR_ARG;
    for (int j = 0; j < g.fv->d; ++j)
      if ((g.tv->signs[j] < 0) != (segs[0].tv->signs[j] < 0)) return TQ_ERR_ARG;
    caps[s] = g.capacity;
  }
  const int64_t need = tq_attend_segments_workspace_bytes(batch, hq, hkv, n_seg, caps, 128);
  if (need < 0) return TQ_ERR_ARG;
  if (workspace_bytes < need) return TQ_ERR_WORKSPACE;
  if (n_seg == 2) {  // a fused instance runs both segments in one scan launch
    const int rc = tq_launch_decode_pair(segs, q, q_dtype, batch, hq, hkv, scale, tau, out, skipped,
                                         workspace, reinterpret_cast<hipStream_t>(stream));
    if (rc != TQ_ERR_SHAPE) return rc;
  }
  int32_t total = 0, base[8];
  tq_decode_plan plans[8];
  for (int s = 0; s < n_seg; ++s) {
    plans[s] = tq_plan_decode(batch, hq, hkv, caps[s], 128);
    base[s] = total;
    total += plans[s].n_split;
  }
  for (int s = 0; s < n_seg; ++s) {
    const tq_cache_segment& g = segs[s];
    const int rc = tq_launch_decode(g.fk, g.tk, g.fv, g.tv, q, q_dtype, batch, hq, hkv, g.codes_k,
                                    g.norms_k, g.codes_v, g.norms_v, g.capacity, g.seq_lens,
                                    scale, tau, out, nullptr, skipped, workspace, plans[s],
                                    reinterpret_cast<hipStream_t>(stream), nullptr, base[s],
                                    total, s == n_seg - 1);
    if (rc) return rc;
  }
  return TQ_OK;
}

int tq_attend_decode_paged(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                           const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch,
                           int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                           const void* codes_v, const uint16_t* norms_v, int32_t page_size,
                           int64_t num_pages, const int32_t* block_table, int32_t max_blocks,
                           const int32_t* seq_lens, float scale, float tau, float* out,
                           float* logits, int64_t* skipped, void* workspace,
                           int64_t workspace_bytes, tq_stream_t stream) {
  const int lg = page_log2(page_size);
  if (lg < 0 || num_pages < 1 || max_blocks < 1 || !block_table) return TQ_ERR_ARG;
  if (!aligned(block_table, 4)) return TQ_ERR_ALIGN;
  if ((fk && fk->layout) || (fv && fv->layout)) return TQ_ERR_SHAPE;
  const tq_paged_src src{block_table, num_pages, max_blocks, lg, max_blocks, -1};
  return decode_checked(fk, tk, fv, tv, q, q_dtype, batch, hq, hkv, codes_k, norms_k, codes_v,
                        norms_v, (int64_t)max_blocks << lg, seq_lens, scale, tau, out, logits,
                        skipped, workspace, workspace_bytes, stream, &src);
}

}  // extern "C"

namespace {
int decode_checked(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                   const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch, int32_t hq,
                   int32_t hkv, const void* codes_k, const uint16_t* norms_k, const void* codes_v,
                   const uint16_t* norms_v, int64_t capacity, const int32_t* seq_lens, float scale,
                   float tau, float* out, float* logits, int64_t* skipped, void* workspace,
                   int64_t workspace_bytes, tq_stream_t stream, const tq_paged_src* paged,
                   bool launch) {
  int rc = tq_check_format(fk);
  if (rc) return rc;
  if ((rc = tq_check_format(fv))) return rc;
  const bool sliced = fv->layout == 1;
  if (fk->layout != 0) return TQ_ERR_SHAPE;
  if (fk->d != 128 || fv->d != 128) return TQ_ERR_SHAPE;
  if (sliced ? !tq_decode_mx_supported(fk, fv) : !tq_decode_formats_supported(fk, fv))
    return TQ_ERR_SHAPE;
  if (batch <= 0 || hq <= 0 || hkv <= 0 || capacity < 0) return TQ_ERR_ARG;
  if (sliced && (paged || capacity % 32 || (hq % hkv == 0 && (hq / hkv) % 4))) return TQ_ERR_SHAPE;
  if (hq % hkv) return TQ_ERR_SHAPE;
  const int g = hq / hkv;
  if (g != 1 && g != 2 && g % 4) return TQ_ERR_SHAPE;
  if (!dtype_ok(q_dtype) || !std::isfinite(scale) || !(tau >= 0.0f) || !(tau <= 1.0f)) return TQ_ERR_ARG;
  if ((rc = check_tables(fk, tk)) || (rc = check_tables(fv, tv))) return rc;
  const bool need_lens = !paged || paged->causal_start < 0;
  if (!q || !out || (need_lens && !seq_lens) || !workspace) return TQ_ERR_ARG;
  if (capacity > 0 && (!codes_k || !norms_k || !codes_v || !norms_v)) return TQ_ERR_ARG;
  if (!aligned(q, dtype_size(q_dtype)) || !aligned(codes_k, 16) || !aligned(codes_v, 16) ||
      !aligned(norms_k, 4) || !aligned(norms_v, 4) || (seq_lens && !aligned(seq_lens, 4)) || !aligned(out, 16) ||
      (logits && !aligned(logits, 4)) || (skipped && !aligned(skipped, 8)) || !aligned(workspace, 16))
    return TQ_ERR_ALIGN;
  const tq_decode_plan plan = sliced ? tq_plan_decode_mx(batch, hq, hkv, capacity)
                                    : tq_plan_decode(batch, hq, hkv, capacity, fk->d);
  if (workspace_bytes < plan.ws_bytes) return TQ_ERR_WORKSPACE;
  if (!launch) return TQ_OK;
  if (sliced)
    return tq_launch_decode_mx(fk, tk, fv, tv, q, q_dtype, batch, hq, hkv, codes_k, norms_k,
                               codes_v, norms_v, capacity, seq_lens, scale, tau, out, logits,
                               skipped, workspace, plan, reinterpret_cast<hipStream_t>(stream));
  return tq_launch_decode(fk, tk, fv, tv, q, q_dtype, batch, hq, hkv, codes_k, norms_k, codes_v,
                          norms_v, capacity, seq_lens, scale, tau, out, logits, skipped, workspace,
                          plan, reinterpret_cast<hipStream_t>(stream), paged);
}
}  // namespace

extern "C" {

int64_t tq_search_workspace_bytes(int64_t n_q, int32_t k, int64_t n_db, int32_t d) {
  if (n_q < 0 || k < 1 || k > 64 || n_db < k || (d != 128 && d != 256)) return -1;
  return tq_plan_search(n_q, k, n_db, d).ws_bytes;
}

int tq_ip_search(const tq_format* f, const tq_tables* t, const void* codes_db,
                 const uint16_t* norms_db, int64_t n_db, const float* queries, int32_t d_in,
                 int64_t n_q, int32_t k, int64_t* out_ids, float* out_scores, void* workspace,
                 int64_t workspace_bytes, tq_stream_t stream) {
  int rc = tq_check_format(f);
  if (rc) return rc;
  if (!f->qjl || f->layout) return TQ_ERR_SHAPE;  // the score is the estimator with the QJL term
  if (n_q < 0 || n_db < 0 || k < 1 || k > 64 || k > n_db) return TQ_ERR_ARG;
  if (d_in <= 0 || d_in > f->d) return TQ_ERR_SHAPE;
  if ((rc = check_tables(f, t))) return rc;
  if (n_q == 0) return TQ_OK;
  if (!codes_db || !norms_db || !queries || !out_ids || !out_scores || !workspace) return TQ_ERR_ARG;
  if (!aligned(codes_db, 16) || !aligned(norms_db, 4) || !aligned(queries, 4) ||
      !aligned(out_ids, 8) || !aligned(out_scores, 4) || !aligned(workspace, 16))
    return TQ_ERR_ALIGN;
  const tq_search_plan plan = tq_plan_search(n_q, k, n_db, f->d);
  if (workspace_bytes < plan.ws_bytes) return TQ_ERR_WORKSPACE;
  return tq_launch_search(f, t, codes_db, norms_db, n_db, queries, d_in, n_q, k, out_ids,
                          out_scores, workspace, plan, reinterpret_cast<hipStream_t>(stream));
}

int64_t tq_prefill_workspace_bytes(int32_t n_new, int32_t hq, int32_t hkv, int64_t start) {
  if (n_new < 1 || hq < 1 || hkv < 1 || hq % hkv || start < 0) return -1;
  return tq_plan_prefill(n_new, hq, hkv, start).ws_bytes;
}

int tq_prefill_paged(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                     const tq_tables* tv, const void* q, int32_t q_dtype, int32_t n_new,
                     int32_t hq, int32_t hkv, const void* k_new, const void* v_new,
                     int32_t kv_dtype, int64_t ld_kv, int64_t start, void* codes_k,
                     uint16_t* norms_k, void* codes_v, uint16_t* norms_v, int32_t page_size,
                     int64_t num_pages, const int32_t* block_table, int32_t max_blocks, float scale,
                     float* out, int64_t* counters, void* workspace, int64_t workspace_bytes,
                     tq_stream_t stream) {
  const int lg = page_log2(page_size);
  if (lg < 0 || num_pages < 1 || max_blocks < 1 || !block_table || n_new < 0 || hkv < 1 ||
      hq < 1 || start < 0)
    return TQ_ERR_ARG;
  if (!aligned(block_table, 4)) return TQ_ERR_ALIGN;
  if (hq % hkv) return TQ_ERR_SHAPE;
  const int64_t capacity = (int64_t)max_blocks << lg;
  if (start + n_new > capacity) return TQ_ERR_SHAPE;
  int rc = tq_check_format(fk);
  if (rc) return rc;
  if ((rc = tq_check_format(fv))) return rc;
  if (fk->d != 128 || fv->d != 128 || !fk->qjl || fk->layout || fv->layout) return TQ_ERR_SHAPE;
  if (n_new == 0) return TQ_OK;
  if (!dtype_ok(q_dtype) || !std::isfinite(scale)) return TQ_ERR_ARG;
  if (!q || !out || !workspace) return TQ_ERR_ARG;
  if (!aligned(q, dtype_size(q_dtype)) || !aligned(out, 16) || !aligned(workspace, 256))
    return TQ_ERR_ALIGN;
  const tq_prefill_plan plan = tq_plan_prefill(n_new, hq, hkv, start);
  if (workspace_bytes < plan.ws_bytes) return TQ_ERR_WORKSPACE;
  const tq_paged_dst dst{nullptr, num_pages, hkv, lg, block_table, start, max_blocks};
  const int64_t nv = (int64_t)n_new * hkv;
  // every part is validated before anything is written or launched
  for (int pass = 0; pass < 2; ++pass) {
    const bool go = pass == 1;
    if ((rc = quantize_checked(fk, tk, k_new, kv_dtype, nv, 128, ld_kv, codes_k, norms_k, counters,
                               stream, &dst, go)))
      return rc;
    if ((rc = quantize_checked(fv, tv, v_new, kv_dtype, nv, 128, ld_kv, codes_v, norms_v, counters,
                               stream, &dst, go)))
      return rc;
  }
  return tq_launch_prefill(fk, tk, fv, tv, q, q_dtype, n_new, hq, hkv, codes_k, norms_k, codes_v,
                           norms_v, lg, num_pages, block_table, max_blocks, start, scale, out,
                           workspace, plan, reinterpret_cast<hipStream_t>(stream));
}

int64_t tq_requantize_workspace_bytes(int64_t n, int32_t d) {
  if (n < 0 || d != 128) return -1;
  return (n > 0 ? n : 1) * tq_requant_vector_bytes();
}

int tq_requantize(const tq_format* f_in, const tq_tables* t_in, const void* codes_in,
                  const uint16_t* norms_in, int64_t n, const tq_format* f_out,
                  const tq_tables* t_out, void* codes_out, uint16_t* norms_out,
                  int64_t* counters, void* workspace, int64_t workspace_bytes,
                  tq_stream_t stream) {
  int rc = tq_check_format(f_in);
  if (rc) return rc;
  if ((rc = tq_check_format(f_out))) return rc;
  if (f_in->d != 128 || f_out->d != 128 || f_in->layout || f_out->layout) return TQ_ERR_SHAPE;
  if (n < 0) return TQ_ERR_ARG;
  if ((rc = check_tables(f_in, t_in)) || (rc = check_tables(f_out, t_out))) return rc;
  for (int j = 0; j < f_in->d; ++j)
    if (t_in->signs[j] != t_out->signs[j]) return TQ_ERR_ARG;  // one shared rotation
  if (n == 0) return TQ_OK;
  if (!codes_in || !norms_in || !codes_out || !norms_out || !workspace) return TQ_ERR_ARG;
  if (!aligned(codes_in, 16) || !aligned(codes_out, 16) || !aligned(norms_in, 4) ||
      !aligned(norms_out, 4) || !aligned(workspace, 16) || (counters && !aligned(counters, 8)))
    return TQ_ERR_ALIGN;
  if (workspace_bytes < tq_requant_vector_bytes()) return TQ_ERR_WORKSPACE;
  const int64_t rbi = tq_record_bytes(f_in), rbo = tq_record_bytes(f_out);
  auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
  };
  if (codes_out == codes_in ? rbo > rbi : overlap(codes_in, n * rbi, codes_out, n * rbo))
    return TQ_ERR_ARG;
  if (norms_out != norms_in && overlap(norms_in, n * 4, norms_out, n * 4)) return TQ_ERR_ARG;
  const int64_t ws = workspace_bytes;
  if (overlap(workspace, ws, codes_in, n * rbi) || overlap(workspace, ws, codes_out, n * rbo) ||
      overlap(workspace, ws, norms_in, n * 4) || overlap(workspace, ws, norms_out, n * 4))
    return TQ_ERR_ARG;
  return tq_launch_requant(f_in, t_in, codes_in, norms_in, n, f_out, t_out, codes_out, norms_out,
                           counters, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
}

const char* tq_strerror(int code) {
  switch (code) {
    case TQ_OK: return "ok";
    case TQ_ERR_ARG: return "invalid argument";
    case TQ_ERR_SHAPE: return "unsupported shape or format";
    case TQ_ERR_ALIGN: return "misaligned device pointer";
    case TQ_ERR_HIP: return "HIP runtime error";
    case TQ_ERR_NOCONV: return "codebook iteration did not converge";
    case TQ_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status code";
  }
}

}  // extern "C"
