// Compressed inner-product top-k search (163.com explainer,
// m.163.com/dy/article/KOV7P8JI0556C3J2, section "向量搜索"): every database vector is
// scored with the same unbiased estimator as decode attention,
//   score_i = n16_i <q_rot, c[idx_i]> + gamma r16_i <S q_rot, 2 sigma_i - 1>,
// and the k largest are returned (equal scores: lower id first).
//
//   prologue: per query one workgroup: zero-pad to d, q_rot = H D q / sqrt(d), S q_rot,
//             the query's slice of the nibble subset-sum tables of its query group, and the
//             constants of <w, 2b - 1> = 2 <w, b> - sum(w).
//   scan:     grid (query group of QG queries, database split).  The workgroup expands the
//             nibble tables into byte-indexed tables in LDS (one float per query) and
//             streams its database range, lane = database vector, 16 table reads per
//             32-coordinate sign word (Walsh planes of the codebook, then the QJL word).
//             Each wave keeps, per query, a sorted top-k list in registers (lane i holds
//             the i-th best); a ballot finds the tile's candidates above the k-th score
//             and each is inserted with one lane shift.  The waves' lists are merged in LDS.
//             All workgroups walk the database in the same order, so the ones running at
//             the same time on an XCD read the same records through its L2.
//   merge:    per query, the lists of the database splits are merged (skipped when there is
//             one split: the scan then writes the final result).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSWaves = 4;
constexpr int kSTile = 64;

template <int D>
struct SCfg {
  static constexpr int NB = D / 32;
  static constexpr int G = D / 8;                 // byte groups
  static constexpr int QG = (D == 256) ? 2 : 4;   // queries per workgroup (128 KB of tables)
  static constexpr int NIB = 2 * G * 2 * 16;      // nibble floats per query
  static constexpr int NIB_STRIDE = ((NIB + 2) * QG + 3) / 4 * 4;
  static constexpr int kTable = 2 * G * 256 * QG;
};

struct SearchParams {
  const uint32_t* codes;
  const uint32_t* norms;
  const float* queries;
  const float* S;
  int64_t* out_ids;
  float* out_scores;
  float* ws_q;       // [n_q][2][D]
  float* ws_nib;     // [n_groups][NIB_STRIDE]
  float* ws_cand_s;  // [n_q][n_split][k]
  int64_t* ws_cand_i;
  int64_t n_db, n_q, chunk_len;
  int32_t d_in, k, n_split, bits, words;
  float gamma;
  uint32_t sign_mask[8];
  float alpha[4];    // Walsh coefficients of the codebook
};

// ----------------------------------------------------------------------------- prologue
template <int D>
__global__ __launch_bounds__(256) void search_prologue(SearchParams p) {
  using C = SCfg<D>;
  const int64_t qi = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int64_t grp = qi / C::QG;
  const int slot = (int)(qi % C::QG);
  __shared__ float wv[2][D];
  __shared__ float red[2][8];
  constexpr int NE = D / 64;
  if (wave == 0) {
    float v[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int j = lane + 64 * e;
      float x = (j < p.d_in) ? p.queries[qi * p.d_in + j] : 0.0f;
      uint32_t sw = uniform_u32(p.sign_mask[2 * e]);
      if (lane & 32) sw = uniform_u32(p.sign_mask[2 * e + 1]);
      if ((sw >> (j & 31)) & 1u) x = -x;
      v[e] = x;
    }
#pragma unroll
    for (int hh = 1; hh < NE; hh <<= 1)
#pragma unroll
      for (int e = 0; e < NE; ++e)
        if (!(e & hh)) {
          const float a = v[e], b = v[e + hh];
          v[e] = a + b;
          v[e + hh] = a - b;
        }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const float t = __shfl_xor(v[e], m, 64);
        v[e] = (lane & m) ? t - v[e] : v[e] + t;
      }
    const float isd = 1.0f / sqrtf((float)D);
#pragma unroll
    for (int e = 0; e < NE; ++e) wv[0][lane + 64 * e] = v[e] * isd;
  }
  __syncthreads();
  for (int r = tid; r < D; r += 256) {
    const f32x4* row = reinterpret_cast<const f32x4*>(p.S + (int64_t)r * D);
    float s = 0.0f;
#pragma unroll 8
    for (int k = 0; k < D / 4; ++k) {
      const f32x4 a = row[k];
      s = fmaf(a[0], wv[0][4 * k], s);
      s = fmaf(a[1], wv[0][4 * k + 1], s);
      s = fmaf(a[2], wv[0][4 * k + 2], s);
      s = fmaf(a[3], wv[0][4 * k + 3], s);
    }
    wv[1][r] = s;
  }
  __syncthreads();
  float* dq = p.ws_q + qi * 2 * D;
  for (int j = tid; j < 2 * D; j += 256) dq[j] = wv[j / D][j % D];
  float* nib = p.ws_nib + grp * C::NIB_STRIDE;
  for (int i = tid; i < C::NIB; i += 256) {
    const int n = i % 16, half = (i / 16) % 2, g = (i / 32) % C::G, vv = i / (32 * C::G);
    float sum = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if ((n >> k) & 1) sum += wv[vv][8 * g + 4 * half + k];
    nib[i * C::QG + slot] = sum;
  }
  // constants: (sum_k alpha_k) sum(q_rot), sum(S q_rot); fixed-order reduction
  float aq = 0.0f, as = 0.0f;
  for (int j = tid; j < D; j += 256) {
    aq += wv[0][j];
    as += wv[1][j];
  }
  aq = wave_sum_fast(aq);
  as = wave_sum_fast(as);
  if (lane == 0) {
    red[0][wave] = aq;
    red[1][wave] = as;
  }
  __syncthreads();
  if (tid == 0) {
    float asum = 0.0f;
    for (int k = 0; k < 4; ++k) asum += p.alpha[k];
    nib[C::NIB * C::QG + slot] = asum * (((red[0][0] + red[0][1]) + red[0][2]) + red[0][3]);
    nib[C::NIB * C::QG + C::QG + slot] = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
  }
}

// a before b in the result order: larger score, then lower id
__device__ __forceinline__ bool better(float sa, int64_t ia, float sb, int64_t ib) {
  return sa > sb || (sa == sb && ia < ib);
}

// Insert (s, id) into the wave's sorted list (lane i < k holds the i-th best) if it beats
// the current k-th entry.  Wave-uniform arguments.
__device__ __forceinline__ void list_insert(float& ls, int64_t& li, float s, int64_t id, int k) {
  const int lane = lane_id();
  const bool mine_better = lane < k && better(ls, li, s, id);
  const int pos = __popcll(__ballot(mine_better));  // number of entries that stay ahead
  if (pos >= k) return;
  // lanes > pos take the entry of lane - 1; lane pos takes the candidate
  const float ps = __shfl_up(ls, 1, 64);
  const int64_t pi = __shfl_up(li, 1, 64);
  if (lane > pos && lane < k) {
    ls = ps;
    li = pi;
  } else if (lane == pos) {
    ls = s;
    li = id;
  }
}

template <int D, int B>
__global__ __launch_bounds__(64 * kSWaves) void search_scan(SearchParams p) {
  using C = SCfg<D>;
  constexpr int QG = C::QG, NB = C::NB, W = NB * (B + 1);
  extern __shared__ __attribute__((aligned(16))) float lds[];
  float* Tq = lds;                          // [G][256][QG]
  float* Ts = lds + C::G * 256 * QG;        // [G][256][QG]
  float* stage = lds + C::kTable;           // nibble staging, later the waves' lists
  __shared__ float cst[2][QG];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int64_t grp = blockIdx.x;
  const int split = blockIdx.y;
  const int64_t q0 = grp * QG;
  const int64_t db_begin = (int64_t)split * p.chunk_len;
  int64_t db_end = db_begin + p.chunk_len;
  if (db_end > p.n_db) db_end = p.n_db;

  // ---- tables
  {
    const float* src = p.ws_nib + grp * C::NIB_STRIDE;
    for (int i = threadIdx.x; i < C::NIB * QG / 4; i += blockDim.x)
      reinterpret_cast<f32x4*>(stage)[i] = reinterpret_cast<const f32x4*>(src)[i];
    if (threadIdx.x < 2 * QG) (&cst[0][0])[threadIdx.x] = src[C::NIB * QG + threadIdx.x];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * C::G * 16; i += blockDim.x) {
    const int lo = i % 16, g = (i / 16) % C::G, vv = i / (16 * C::G);
    const float* nl = stage + (((vv * C::G + g) * 2 + 0) * 16 + lo) * QG;
    const float* nh = stage + (((vv * C::G + g) * 2 + 1) * 16) * QG;
    float a[QG];
#pragma unroll
    for (int h = 0; h < QG; ++h) a[h] = nl[h];
    float* dst = (vv == 0 ? Tq : Ts) + (g * 256 + lo) * QG;
#pragma unroll 4
    for (int hi = 0; hi < 16; ++hi)
#pragma unroll
      for (int h = 0; h < QG; ++h) dst[hi * 16 * QG + h] = a[h] + nh[hi * QG + h];
  }
  __syncthreads();

  float cq[QG], cs[QG];
#pragma unroll
  for (int h = 0; h < QG; ++h) {
    cq[h] = cst[0][h];
    cs[h] = cst[1][h];
  }
  float al[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) al[k] = 2.0f * p.alpha[k];
  const int k = p.k;

  float ls[QG];
  int64_t li[QG];
#pragma unroll
  for (int h = 0; h < QG; ++h) {
    ls[h] = -INFINITY;
    li[h] = INT64_MAX;
  }

  uint32_t rw[W], nr = 0;
  int64_t t0 = db_begin + (int64_t)wave * kSTile;
  auto fetch = [&](int64_t tt0) {
    const int64_t t = tt0 + lane;
    if (t < db_end) {
#pragma unroll
      for (int i = 0; i < W / 4; ++i) {
        const u32x4 v = reinterpret_cast<const u32x4*>(p.codes + t * W)[i];
        rw[4 * i] = v[0]; rw[4 * i + 1] = v[1]; rw[4 * i + 2] = v[2]; rw[4 * i + 3] = v[3];
      }
      nr = p.norms[t];
    }
  };
  fetch(t0);
  for (; t0 < db_end; t0 += (int64_t)kSWaves * kSTile) {
    const int64_t t = t0 + lane;
    const bool valid = t < db_end;
    uint32_t w[W];
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = rw[i];
    const uint32_t nn = nr;
    fetch(t0 + (int64_t)kSWaves * kSTile);
    float mse[QG], qjl[QG];
#pragma unroll
    for (int h = 0; h < QG; ++h) mse[h] = qjl[h] = 0.0f;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const uint32_t* wb = w + blk * (B + 1);
#pragma unroll
      for (int pl = 0; pl < (B == 3 ? 4 : B); ++pl) {
        const uint32_t word = (pl < B) ? wb[pl] : (wb[0] ^ wb[1] ^ wb[2]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float* e = Tq + ((4 * blk + i) * 256 + ((word >> (8 * i)) & 0xFFu)) * QG;
#pragma unroll
          for (int h = 0; h < QG; ++h) mse[h] = fmaf(al[pl], e[h], mse[h]);
        }
      }
      const uint32_t sw = wb[B];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* e = Ts + ((4 * blk + i) * 256 + ((sw >> (8 * i)) & 0xFFu)) * QG;
#pragma unroll
        for (int h = 0; h < QG; ++h) qjl[h] += e[h];
      }
    }
    const float n16 = f16_bits_to_f32(nn), r16 = f16_bits_to_f32(nn >> 16);
#pragma unroll
    for (int h = 0; h < QG; ++h) {
      if (q0 + h >= p.n_q) continue;
      const float sc = valid ? n16 * (mse[h] - cq[h]) + p.gamma * r16 * (2.0f * qjl[h] - cs[h]) : -INFINITY;
      // k-th entry of the list, then the tile's candidates that beat it
      const float ks = __shfl(ls[h], k - 1, 64);
      const int64_t ki = __shfl(li[h], k - 1, 64);
      uint64_t cand = __ballot(valid && better(sc, t, ks, ki));
      while (cand) {
        const int L = __builtin_ctzll(cand);
        cand &= cand - 1;
        const float s = __shfl(sc, L, 64);
        list_insert(ls[h], li[h], s, t0 + L, k);
      }
    }
  }
  // ---- merge the waves' lists per query (fixed order), write candidates / result
  __syncthreads();
  float* lst_s = stage;                                           // [waves][QG][64]
  int64_t* lst_i = reinterpret_cast<int64_t*>(stage + kSWaves * QG * 64);
#pragma unroll
  for (int h = 0; h < QG; ++h) {
    lst_s[(wave * QG + h) * 64 + lane] = ls[h];
    lst_i[(wave * QG + h) * 64 + lane] = li[h];
  }
  __syncthreads();
  if (wave < QG && q0 + wave < p.n_q) {
    const int h = wave;
    float ms = -INFINITY;
    int64_t mi = INT64_MAX;
    for (int w2 = 0; w2 < kSWaves; ++w2)
      for (int i = 0; i < k; ++i) {
        const float s = lst_s[(w2 * QG + h) * 64 + i];
        const int64_t id = lst_i[(w2 * QG + h) * 64 + i];
        if (better(s, id, __shfl(ms, k - 1, 64), __shfl(mi, k - 1, 64))) list_insert(ms, mi, s, id, k);
      }
    const int64_t qi = q0 + h;
    if (lane < k) {
      if (p.n_split == 1) {
        p.out_scores[qi * k + lane] = ms;
        p.out_ids[qi * k + lane] = mi;
      } else {
        p.ws_cand_s[(qi * p.n_split + split) * k + lane] = ms;
        p.ws_cand_i[(qi * p.n_split + split) * k + lane] = mi;
      }
    }
  }
}

// ----------------------------------------------------------------------------- merge
__global__ __launch_bounds__(64) void search_merge(SearchParams p) {
  const int64_t qi = blockIdx.x;
  const int lane = lane_id(), k = p.k;
  float ms = -INFINITY;
  int64_t mi = INT64_MAX;
  for (int s = 0; s < p.n_split; ++s)
    for (int i = 0; i < k; ++i) {
      const float sc = p.ws_cand_s[(qi * p.n_split + s) * k + i];
      const int64_t id = p.ws_cand_i[(qi * p.n_split + s) * k + i];
      if (better(sc, id, __shfl(ms, k - 1, 64), __shfl(mi, k - 1, 64))) list_insert(ms, mi, sc, id, k);
    }
  if (lane < k) {
    p.out_scores[qi * k + lane] = ms;
    p.out_ids[qi * k + lane] = mi;
  }
}

template <int D, int B>
static int launch_search(const SearchParams& p, int64_t n_groups, hipStream_t stream) {
  using C = SCfg<D>;
  const int nstage = (kSWaves * C::QG * 64 * 3 > C::NIB * C::QG) ? kSWaves * C::QG * 64 * 3 : C::NIB * C::QG;
  const size_t lds = sizeof(float) * (size_t)(C::kTable + nstage);
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute((const void*)search_scan<D, B>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
      return TQ_ERR_HIP;
    attr = true;
  }
  hipLaunchKernelGGL(search_prologue<D>, dim3((unsigned)p.n_q), dim3(256), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
  hipLaunchKernelGGL((search_scan<D, B>), dim3((unsigned)n_groups, (unsigned)p.n_split),
                     dim3(64 * kSWaves), lds, stream, p);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
  if (p.n_split > 1) {
    hipLaunchKernelGGL(search_merge, dim3((unsigned)p.n_q), dim3(64), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
  }
  return TQ_OK;
}

static void walsh_s(int bits, const float* c, float* alpha) {
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

}  // namespace tqk

// ---------------------------------------------------------------------------------------
tq_search_plan tq_plan_search(int64_t n_q, int32_t k, int64_t n_db, int32_t d) {
  using namespace tqk;
  tq_search_plan p{};
  const int qg = d == 256 ? SCfg<256>::QG : SCfg<128>::QG;
  const int nib_stride = d == 256 ? SCfg<256>::NIB_STRIDE : SCfg<128>::NIB_STRIDE;
  const int64_t groups = (n_q + qg - 1) / qg;
  // split the database when there are too few query groups to fill a 256-CU MI355X
  int64_t n_split = groups >= 256 ? 1 : (256 + groups - 1) / (groups > 0 ? groups : 1);
  const int64_t max_split = (n_db + 16383) / 16384;
  if (n_split > max_split) n_split = max_split;
  if (n_split < 1) n_split = 1;
  const int64_t chunk = (n_db + n_split - 1) / n_split;
  p.n_chunks = (int32_t)n_split;
  p.chunk_len = (chunk + kSTile - 1) / kSTile * kSTile;
  p.ws_q_off = 0;
  const int64_t q_bytes = (n_q > 0 ? n_q : 1) * 2 * d * 4;
  const int64_t nib_off = (q_bytes + 255) / 256 * 256;
  const int64_t nib_bytes = (groups > 0 ? groups : 1) * nib_stride * 4;
  p.ws_cand_off = nib_off + (nib_bytes + 255) / 256 * 256;
  const int64_t cand = (n_split > 1) ? (n_q > 0 ? n_q : 1) * n_split * k * 12 : 0;
  p.ws_bytes = p.ws_cand_off + cand + 256;
  return p;
}

int tq_launch_search(const tq_format* f, const tq_tables* t, const void* codes_db,
                     const uint16_t* norms_db, int64_t n_db, const float* queries, int32_t d_in,
                     int64_t n_q, int32_t k, int64_t* out_ids, float* out_scores, void* workspace,
                     const tq_search_plan& plan, hipStream_t stream) {
  using namespace tqk;
  if (f->bits_lo != f->bits_hi || f->split != f->d || !f->qjl) return TQ_ERR_SHAPE;
  SearchParams p{};
  p.codes = reinterpret_cast<const uint32_t*>(codes_db);
  p.norms = reinterpret_cast<const uint32_t*>(norms_db);
  p.queries = queries;
  p.S = t->S;
  p.out_ids = out_ids;
  p.out_scores = out_scores;
  char* ws = reinterpret_cast<char*>(workspace);
  const int64_t q_bytes = (n_q > 0 ? n_q : 1) * 2 * f->d * 4;
  const int64_t nib_off = (q_bytes + 255) / 256 * 256;
  p.ws_q = reinterpret_cast<float*>(ws);
  p.ws_nib = reinterpret_cast<float*>(ws + nib_off);
  const int64_t nsk = n_q * plan.n_chunks * k;
  p.ws_cand_i = reinterpret_cast<int64_t*>(ws + plan.ws_cand_off);
  p.ws_cand_s = reinterpret_cast<float*>(ws + plan.ws_cand_off + nsk * 8);
  p.n_db = n_db;
  p.n_q = n_q;
  p.chunk_len = plan.chunk_len;
  p.d_in = d_in;
  p.k = k;
  p.n_split = plan.n_chunks;
  p.bits = f->bits_lo;
  p.words = (int)(tq_record_bytes(f) / 4);
  p.gamma = (float)(std::sqrt(M_PI / 2.0) / f->d);
  for (int j = 0; j < 8; ++j) p.sign_mask[j] = 0;
  for (int j = 0; j < f->d; ++j)
    if (t->signs[j] < 0) p.sign_mask[j >> 5] |= 1u << (j & 31);
  walsh_s(f->bits_lo, t->centroids_lo, p.alpha);
  const int qg = f->d == 256 ? SCfg<256>::QG : SCfg<128>::QG;
  const int64_t groups = (n_q + qg - 1) / qg;
  if (f->d == 256) {
    if (f->bits_lo == 3) return launch_search<256, 3>(p, groups, stream);
    if (f->bits_lo == 2) return launch_search<256, 2>(p, groups, stream);
  } else {
    if (f->bits_lo == 3) return launch_search<128, 3>(p, groups, stream);
    if (f->bits_lo == 2) return launch_search<128, 2>(p, groups, stream);
    if (f->bits_lo == 1) return launch_search<128, 1>(p, groups, stream);
  }
  return TQ_ERR_SHAPE;
}
