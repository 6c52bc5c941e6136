// Host side of decode attention: the split-combine kernel, the launch plan, the Walsh
// coefficients of the key codebooks and the dispatch over the supported format pairs.  The
// scan kernel is in tq_decode_kernel.h.
#include "tq_decode_kernel.h"

namespace tqk {

// ----------------------------------------------------------------------------- combine
// One workgroup per (batch, query head).  Every load of the first splits is issued before
// the first use, at most 34 per thread so that one round trip to memory brings them all:
// the 16 x 4 S_v entries of this thread's part of S^T Q (16-byte loads), each split's (m, l)
// (thread i loads split i) and the first 32 splits' partial sums, one (A | Q) float pair per
// thread and split parity.  The splits' weights 2^(m_i - M) go through LDS in chunks of 256
// splits, so any number of partials fits (segmented caches add theirs up); every sum runs in
// a fixed order (the denominator in split order, the same for every thread).
constexpr int kCombPairs = 16;    // partial-sum pairs in flight per thread (one parity)
constexpr int kCombSplits = 256;  // split weights per LDS chunk

__global__ __launch_bounds__(256) void decode_combine(DecodeParams p) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const int bh = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  __shared__ float red[4];
  __shared__ float scl[kCombSplits];
  __shared__ float lw[kCombSplits];
  __shared__ f32x2 accp[2][kD];      // per split parity: sums of the (A | Q) float pairs
  __shared__ float vec[2 * kD];      // merged A | Q
  __shared__ float part_s[8][kD];    // S^T Q over row groups of 16
  const float* parts = p.ws_part + (int64_t)bh * p.n_split * kPartFloats;
  const int np = p.n_split;
  // S^T Q: thread (column group j4, row group rq) holds S_v[16 rq + i][4 j4 .. 4 j4 + 3]
  const int j4 = tid & 31, rq = tid >> 5;
  f32x4 sv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    sv[i] = *reinterpret_cast<const f32x4*>(p.S_v + (int64_t)(16 * rq + i) * kD + 4 * j4);
  // merge: thread (float pair c2 of A | Q, split parity hs) sums splits hs, hs + 2, ...
  const int c2 = tid & 127, hs = tid >> 7;
  float m0 = -INFINITY, l0 = 0.0f;
  if (tid < np) {
    m0 = parts[(int64_t)tid * kPartFloats];
    l0 = parts[(int64_t)tid * kPartFloats + 1];
  }
  f32x2 pv[kCombPairs];
#pragma unroll
  for (int k = 0; k < kCombPairs; ++k) {
    const int sp = hs + 2 * k;
    pv[k] = sp < np ? *reinterpret_cast<const f32x2*>(parts + (int64_t)sp * kPartFloats + 2 + 2 * c2)
                    : (f32x2){0.0f, 0.0f};
  }
  // the largest split maximum
  float M = m0;
  for (int i = tid + kCombSplits; i < np; i += 256) M = fmaxf(M, parts[(int64_t)i * kPartFloats]);
  M = wave_max_fast(M);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  f32x2 acc = {0.0f, 0.0f};
  float lsum = 0.0f;
  for (int c0 = 0; c0 < np; c0 += kCombSplits) {
    const int nc = np - c0 < kCombSplits ? np - c0 : kCombSplits;
    if (tid < nc) {
      float m = m0, l = l0;
      if (c0 > 0) {
        m = parts[(int64_t)(c0 + tid) * kPartFloats];
        l = parts[(int64_t)(c0 + tid) * kPartFloats + 1];
      }
      const float sw = (m == -INFINITY || M == -INFINITY) ? 0.0f : exp2f(m - M);
      scl[tid] = sw;
      lw[tid] = sw * l;
    }
    __syncthreads();
    for (int c = 0; c < nc; c += 2 * kCombPairs) {
      if (c0 + c > 0) {
#pragma unroll
        for (int k = 0; k < kCombPairs; ++k) {
          const int sp = c + hs + 2 * k;
          pv[k] = sp < nc ? *reinterpret_cast<const f32x2*>(parts + (int64_t)(c0 + sp) * kPartFloats + 2 + 2 * c2)
                          : (f32x2){0.0f, 0.0f};
        }
      }
#pragma unroll
      for (int k = 0; k < kCombPairs; ++k) {
        const int sp = c + hs + 2 * k;
        if (sp < nc) {
          acc[0] = fmaf(pv[k][0], scl[sp], acc[0]);
          acc[1] = fmaf(pv[k][1], scl[sp], acc[1]);
        }
      }
    }
    // the denominator, in split order (every thread reads the same LDS values)
    for (int k = 0; k < nc; ++k) lsum += lw[k];
    __syncthreads();
  }
  accp[hs][c2] = acc;
  __syncthreads();
  if (tid < kD) {
    const f32x2 t = accp[0][tid] + accp[1][tid];
    vec[2 * tid] = t[0];
    vec[2 * tid + 1] = t[1];
  }
  __syncthreads();
  {  // S^T Q over this thread's 16 rows and 4 columns
    f32x4 ps = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float qv = vec[kD + 16 * rq + i];
      ps[0] = fmaf(sv[i][0], qv, ps[0]);
      ps[1] = fmaf(sv[i][1], qv, ps[1]);
      ps[2] = fmaf(sv[i][2], qv, ps[2]);
      ps[3] = fmaf(sv[i][3], qv, ps[3]);
    }
    *reinterpret_cast<f32x4*>(&part_s[rq][4 * j4]) = ps;
  }
  __syncthreads();
  if (tid < 64) {
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int jj = lane + 64 * e;
      float st = 0.0f;
#pragma unroll
      for (int r = 0; r < 8; ++r) st += part_s[r][jj];
      v[e] = vec[jj] + st;
    }
    fwht128(v, lane);
    const float inv = (lsum > 0.0f) ? 1.0f / (lsum * sqrtf((float)kD)) : 0.0f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int jj = lane + 64 * e;
      float o = v[e] * inv;
      const uint32_t sw = (lane & 32) ? uniform_u32(p.sign_v[2 * e + 1]) : uniform_u32(p.sign_v[2 * e]);
      if ((sw >> (jj & 31)) & 1u) o = -o;
      p.out[(int64_t)bh * kD + jj] = o;
    }
  }
}

}  // namespace tqk

// ---------------------------------------------------------------------------------------
namespace {
// (lo bits, hi bits, split in blocks) of a format; one width is reported with split 4
void shape_of(const tq_format* f, int& lo, int& hi, int& sb) {
  lo = f->bits_lo;
  hi = f->split == f->d ? f->bits_lo : f->bits_hi;
  sb = lo == hi ? 4 : f->split / 32;
}
}  // namespace

bool tq_decode_formats_supported(const tq_format* fk, const tq_format* fv) {
  if (!fk->qjl) return false;  // the logit estimator needs the keys' QJL term
  int kl, kh, ks, vl, vh, vs;
  shape_of(fk, kl, kh, ks);
  shape_of(fv, vl, vh, vs);
#define TQ_DECODE_MATCH(a, b, c, d, e, f) \
  if (kl == a && kh == b && ks == c && vl == d && vh == e && vs == f) return true;
  TQ_DECODE_PAIRS(TQ_DECODE_MATCH)
#undef TQ_DECODE_MATCH
  return false;
}

// The split merge and rotation back, for callers that produce split partials in the scan's
// format (the prefill kernel).
int tqk::launch_decode_combine(const DecodeParams& p, int rows, hipStream_t stream) {
  hipLaunchKernelGGL(decode_combine, dim3(rows), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

tq_decode_plan tq_plan_decode(int32_t batch, int32_t hq, int32_t hkv, int64_t capacity, int32_t d) {
  using namespace tqk;
  (void)d;
  tq_decode_plan p{};
  const int group = hq / hkv;
  const int gc = group >= 4 ? 4 : group;
  const int64_t units = (int64_t)batch * hkv * (group / gc);
  // about one workgroup per compute unit of a 256-CU MI355X, at least one tile per wave
  const int64_t per_wg = (int64_t)kTile * kWaves;
  int64_t max_split = (capacity + per_wg - 1) / per_wg;
  if (max_split < 1) max_split = 1;
  int64_t n_split = (256 + units - 1) / units;
  if (n_split > max_split) n_split = max_split;
  if (n_split > 1024) n_split = 1024;
  if (n_split < 1) n_split = 1;
  int64_t tps = (capacity + n_split - 1) / n_split;
  tps = ((tps + kTile - 1) / kTile) * kTile;
  if (tps < kTile) tps = kTile;
  p.n_split = (int32_t)n_split;
  p.waves = kWaves;
  p.parts = (int32_t)n_split;
  p.tokens_per_split = tps;
  p.units = units;
  p.ws_part_off = 0;
  p.ws_bytes = (int64_t)batch * hq * p.parts * kPartFloats * 4;
  return p;
}

namespace {
// Scan / combine parameters of one cache (segment): formats, tables, records, query, output
// and the split plan (tokens per split, total partial count, this cache's first partial).
tqk::DecodeParams make_decode_params(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                                     const tq_tables* tv, const void* q, int32_t q_dtype,
                                     int32_t batch, int32_t hq, int32_t hkv, const void* codes_k,
                                     const uint16_t* norms_k, const void* codes_v,
                                     const uint16_t* norms_v, int64_t capacity,
                                     const int32_t* seq_lens, float scale, float tau, float* out,
                                     float* logits, int64_t* skipped, void* workspace,
                                     const tq_decode_plan& plan, const tq_paged_src* paged,
                                     int32_t split_base, int32_t split_total) {
  using namespace tqk;
  DecodeParams p{};
  p.causal_start = -1;
  if (paged) {
    p.block_table = paged->block_table;
    p.num_pages = paged->num_pages;
    p.max_blocks = paged->max_blocks;
    p.page_log2 = paged->page_log2;
    p.bt_stride = paged->bt_stride;
    p.causal_start = paged->causal_start;
  }
  p.q = q;
  p.codes_k = reinterpret_cast<const uint32_t*>(codes_k);
  p.norms_k = reinterpret_cast<const uint32_t*>(norms_k);
  p.codes_v = reinterpret_cast<const uint32_t*>(codes_v);
  p.norms_v = reinterpret_cast<const uint32_t*>(norms_v);
  p.seq_lens = seq_lens;
  p.S_k = tk->S;
  p.S_v = tv->S;
  p.out = out;
  p.logits = logits;
  p.skipped = reinterpret_cast<unsigned long long*>(skipped);
  p.ws_part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + plan.ws_part_off);
  p.capacity = capacity;
  p.tokens_per_split = plan.tokens_per_split;
  p.batch = batch;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.q_dtype = q_dtype;
  p.n_split = split_total > 0 ? split_total : plan.n_split;
  p.split_base = split_base;
  p.ksplitb = fk->split / 32;
  p.scale = scale;
  p.tau = tau;
  p.gamma = (float)(std::sqrt(M_PI / 2.0) / fk->d);
  for (int i = 0; i < 4; ++i) p.sign_k[i] = p.sign_v[i] = 0;
  for (int j = 0; j < 128; ++j) {
    if (tk->signs[j] < 0) p.sign_k[j >> 5] |= 1u << (j & 31);
    if (tv->signs[j] < 0) p.sign_v[j >> 5] |= 1u << (j & 31);
  }
  tq_walsh_coeffs(fk->bits_lo, tk->centroids_lo, p.alpha_k[0]);
  tq_walsh_coeffs(fk->bits_hi, tk->centroids_hi, p.alpha_k[1]);
  for (int i = 0; i < 8; ++i) {
    p.cent_v[0][i] = i < (1 << fv->bits_lo) ? tv->centroids_lo[i] : 0.0f;
    p.cent_v[1][i] = i < (1 << fv->bits_hi) ? tv->centroids_hi[i] : 0.0f;
  }
  return p;
}
}  // namespace

int tq_launch_decode(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                     const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch,
                     int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                     const void* codes_v, const uint16_t* norms_v, int64_t capacity,
                     const int32_t* seq_lens, float scale, float tau, float* out, float* logits,
                     int64_t* skipped, void* workspace, const tq_decode_plan& plan,
                     hipStream_t stream, const tq_paged_src* paged, int32_t split_base,
                     int32_t split_total, bool combine) {
  using namespace tqk;
  DecodeParams p = make_decode_params(fk, tk, fv, tv, q, q_dtype, batch, hq, hkv, codes_k, norms_k,
                                      codes_v, norms_v, capacity, seq_lens, scale, tau, out,
                                      logits, skipped, workspace, plan, paged, split_base,
                                      split_total);
  const int gc = p.group >= 4 ? 4 : p.group;
  const int nchunk = p.group / gc;
  const unsigned units = (unsigned)(batch * hkv * nchunk);
  const dim3 grid((unsigned)plan.n_split, units);
  int kl, kh, ks, vl, vh, vs;
  shape_of(fk, kl, kh, ks);
  shape_of(fv, vl, vh, vs);
  const bool vq = fv->qjl != 0;
  int rc = TQ_ERR_SHAPE;
#define TQ_DECODE_LAUNCH(a, b, c, d, e, f)                                      \
  if (kl == a && kh == b && ks == c && vl == d && vh == e && vs == f)          \
    rc = launch_pair<a, b, c, d, e, f>(p, vq, gc, grid, stream);                \
  else
  TQ_DECODE_PAIRS(TQ_DECODE_LAUNCH) {}
#undef TQ_DECODE_LAUNCH
  if (rc != TQ_OK || !combine) return rc;
  hipLaunchKernelGGL(decode_combine, dim3(batch * hq), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

// Two segments whose format pairs have a fused instance (TQ_DECAY_PAIRS) in one scan launch:
// the plan of the concatenated length split between the segments in proportion to their
// capacities, then one combine.  Returns TQ_ERR_SHAPE, before launching anything, when the
// combination, the group size or an empty segment rules the fused path out.
int tq_launch_decode_pair(const tq_cache_segment* segs, const void* q, int32_t q_dtype,
                          int32_t batch, int32_t hq, int32_t hkv, float scale, float tau,
                          float* out, int64_t* skipped, void* workspace, hipStream_t stream) {
  using namespace tqk;
  const tq_cache_segment& s0 = segs[0];
  const tq_cache_segment& s1 = segs[1];
  if ((hq / hkv) % 4 || !s0.fv->qjl || !s1.fv->qjl || s0.capacity <= 0 || s1.capacity <= 0)
    return TQ_ERR_SHAPE;
  int sh[2][6];
  for (int i = 0; i < 2; ++i) {
    shape_of(segs[i].fk, sh[i][0], sh[i][1], sh[i][2]);
    shape_of(segs[i].fv, sh[i][3], sh[i][4], sh[i][5]);
  }
  const int64_t cap = s0.capacity + s1.capacity;
  const int32_t total = tq_plan_decode(batch, hq, hkv, cap, 128).n_split;
  if (total < 2) return TQ_ERR_SHAPE;
  int32_t n0 = (int32_t)((total * s0.capacity + cap / 2) / cap);
  if (n0 < 1) n0 = 1;
  if (n0 > total - 1) n0 = total - 1;
  const int32_t n1 = total - n0;
  tq_decode_plan pl[2];
  for (int i = 0; i < 2; ++i) {
    const int64_t c = segs[i].capacity, n = i == 0 ? n0 : n1;
    pl[i] = tq_plan_decode(batch, hq, hkv, c, 128);
    int64_t tps = (c + n - 1) / n;
    tps = (tps + kTile - 1) / kTile * kTile;
    pl[i].n_split = (int32_t)n;
    pl[i].tokens_per_split = tps < kTile ? kTile : tps;
  }
  const DecodeParams p0 = make_decode_params(s0.fk, s0.tk, s0.fv, s0.tv, q, q_dtype, batch, hq, hkv,
                                             s0.codes_k, s0.norms_k, s0.codes_v, s0.norms_v,
                                             s0.capacity, s0.seq_lens, scale, tau, out, nullptr,
                                             skipped, workspace, pl[0], nullptr, 0, total);
  const DecodeParams p1 = make_decode_params(s1.fk, s1.tk, s1.fv, s1.tv, q, q_dtype, batch, hq, hkv,
                                             s1.codes_k, s1.norms_k, s1.codes_v, s1.norms_v,
                                             s1.capacity, s1.seq_lens, scale, tau, out, nullptr,
                                             skipped, workspace, pl[1], nullptr, n0, total);
  const dim3 grid((unsigned)total, (unsigned)(batch * hkv * (hq / hkv / 4)));
  int rc = TQ_ERR_SHAPE;
#define TQ_DECAY_LAUNCH(a0, a1, a2, a3, a4, a5, b0, b1, b2, b3, b4, b5)                      \
  if (sh[0][0] == a0 && sh[0][1] == a1 && sh[0][2] == a2 && sh[0][3] == a3 &&              \
      sh[0][4] == a4 && sh[0][5] == a5 && sh[1][0] == b0 && sh[1][1] == b1 &&              \
      sh[1][2] == b2 && sh[1][3] == b3 && sh[1][4] == b4 && sh[1][5] == b5)                \
    rc = launch_scan_pair<a0, a1, a2, a3, a4, a5, b0, b1, b2, b3, b4, b5>(p0, p1, n0, grid, stream); \
  else
  TQ_DECAY_PAIRS(TQ_DECAY_LAUNCH) {}
#undef TQ_DECAY_LAUNCH
  if (rc != TQ_OK) return rc;
  hipLaunchKernelGGL(decode_combine, dim3(batch * hq), dim3(256), 0, stream, p1);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
