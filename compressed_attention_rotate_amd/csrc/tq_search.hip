// Compressed inner-product top-k search (163.com explainer,
// m.163.com/dy/article/KOV7P8JI0556C3J2, section "向量搜索"): every database vector is
// scored with the same unbiased estimator as decode attention,
//   score_i = n16_i <q_rot, c[idx_i]> + gamma r16_i <S q_rot, 2 sigma_i - 1>,
// and the k largest are returned (equal scores: lower id first).
//
// For a batch of queries the scores are a (vectors x coordinates) x (coordinates x queries)
// product, so the scan runs on v_mfma_f32_16x16x32_f16 straight from the packed records:
//   prologue: per query eight workgroups: zero-pad to d, q_rot = H D q / sqrt(d), and one
//             eighth of the rows of S q_rot each (fp32, to the workspace).
//   scan:     grid (block of 32 queries, database split), 4 waves.  Wave w owns the record
//             blocks of coordinates [w d/4, (w + 1) d/4) of every 64-vector tile, for all 32
//             queries: lane (j, r) loads block b of vector 16 m + r and expands byte j of its
//             planes into the A operand, centroid pairs (fp16 hi and lo of 2^6 c) from one
//             read of a table indexed by the code bits of two coordinates and +-1 pairs
//             from the sign word; the B operands are q_rot and S q_rot of the queries, each
//             scaled by a power of two and split into fp16 hi + lo.  Five products per 32
//             coordinates (c hi q hi, c lo q hi, c hi q lo, sign (S q) hi, sign (S q) lo)
//             with fp32 accumulation give the two dot products to ~2^-22.  Each wave turns
//             its sums into partial scores (n16 and gamma r16 applied in fp32) in LDS; after
//             one barrier wave w adds the four partials of queries 8w .. 8w + 7 (lane =
//             vector, fixed order) and keeps their top-k lists in registers (lane i holds the
//             i-th best; a ballot finds the tile's candidates above the k-th score and each
//             is inserted with one lane shift).  The partial scores are double-buffered: one
//             barrier per tile.  Concurrent workgroups walk the same database range, so the
//             records come through the L2.
//   merge:    per query, the lists of the database splits are merged (skipped when there is
//             one split: the scan then writes the final result); each wave sorts its first
//             64 candidates whole and screens the rest against its k-th entry.
// At most 20 queries take a scan of their own on the block-scaled fp6 x fp4 matrix cores
// (search_mxq below), which scores each block of four from one pass over the records.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_mx.h"

namespace tqk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

constexpr int kSWaves = 4;    // waves per scan workgroup (one per coordinate quarter)
constexpr int kSTile = 64;    // database vectors per tile
constexpr int kSQ = 32;       // queries per scan workgroup
constexpr int kSQW = kSQ / kSWaves;  // queries whose lists one wave keeps
constexpr uint32_t kSPatMask = 0x1998u;
constexpr float kSCent = 64.0f;  // centroids in the operand table are 2^6 c

// Entries of the centroid-pair table of a B-bit codebook: four coordinates with code-bit
// nibbles b0, b1, b2 give f = b0 << 1 | b1 << 5 | b2 << 9; (f & 0x1998) is 8 times the
// sparse pattern P = p0 | p1 << 4 | p2 << 8 of coordinates (2, 3) and ((f << 2) & 0x1998)
// that of coordinates (0, 1).  Entry P: fp16 (hi(c'[lo]), hi(c'[hi])), (lo(c'[lo]), lo(c'[hi])).
__host__ __device__ constexpr int s_pat_entries(int B) { return B == 3 ? 0x334 : (B == 2 ? 0x34 : 4); }

struct SearchParams {
  const uint32_t* codes;
  const uint32_t* norms;
  const float* queries;
  const float* S;
  int64_t* out_ids;
  float* out_scores;
  float* ws_q;       // [n_q][2][D]: q_rot, S q_rot
  float* ws_cand_s;  // [n_q][n_split][k]
  int64_t* ws_cand_i;
  int64_t n_db, n_q, chunk_len;
  int32_t d_in, k, n_split;
  float gamma;
  uint32_t sign_mask[8];
  float cent[8];     // codebook, ascending
  float alpha[4];    // Walsh coefficients of the codebook (few-query scan: plane weights)
};

// ----------------------------------------------------------------------------- prologue
// the query prologue's S q_rot rows are split over this many workgroups per query
constexpr int kPrologueSlices = 8;

template <int D>
__global__ __launch_bounds__(256) void search_prologue(SearchParams p) {
  const int64_t qi = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  __shared__ float wv[2][D];
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
  // S q_rot, rows [blockIdx.y kRows, +kRows) of it: kP consecutive threads share a row and
  // each sums every kP-th 16-byte column group, so one load instruction reads whole rows
  // and every load of a thread is in flight at once; the kP lanes then reduce by butterfly
  constexpr int kRows = D / kPrologueSlices, kP = 256 / kRows, kC = D / (4 * kP);
  static_assert(kRows * kP == 256 && kP <= 64 && kC >= 1, "prologue split");
  const int r = (int)blockIdx.y * kRows + tid / kP, part = tid % kP;
  const f32x4* row = reinterpret_cast<const f32x4*>(p.S + (int64_t)r * D);
  f32x4 a[kC];
#pragma unroll
  for (int c = 0; c < kC; ++c) a[c] = row[part + kP * c];
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int col = 4 * (part + kP * c);
    s = fmaf(a[c][0], wv[0][col], s);
    s = fmaf(a[c][1], wv[0][col + 1], s);
    s = fmaf(a[c][2], wv[0][col + 2], s);
    s = fmaf(a[c][3], wv[0][col + 3], s);
  }
#pragma unroll
  for (int m = 1; m < kP; m <<= 1) s += __shfl_xor(s, m, 64);
  float* dq = p.ws_q + qi * 2 * D;
  if (part == 0) dq[D + r] = s;
  if (blockIdx.y == 0)
    for (int j = tid; j < D; j += 256) dq[j] = wv[0][j];
}

// a before b in the result order: larger score, then lower id
__device__ __forceinline__ bool better(float sa, int64_t ia, float sb, int64_t ib) {
  return sa > sb || (sa == sb && ia < ib);
}

// Value of lane L (wave-uniform) in every lane, through the scalar unit.
__device__ __forceinline__ float lane_f(float x, int L) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), L));
}
__device__ __forceinline__ int64_t lane_i64(int64_t x, int L) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, L);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), L);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Insert (s, id) into the wave's sorted list (lane i < k holds the i-th best) if it beats
// the current k-th entry.  Wave-uniform arguments.
__device__ __forceinline__ void list_insert(float& ls, int64_t& li, float s, int64_t id, int k) {
  const int lane = lane_id();
  const bool mine_better = lane < k && better(ls, li, s, id);
  const int pos = __popcll(__ballot(mine_better));  // number of entries that stay ahead
  if (pos >= k) return;
  // lanes > pos take the entry of lane - 1 (a DPP shift of the whole wave by one lane);
  // lane pos takes the candidate
  const float ps = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ls), 0x138, 0xF, 0xF, false));
  const uint32_t plo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)li, 0x138, 0xF, 0xF, false);
  const uint32_t phi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)((uint64_t)li >> 32), 0x138, 0xF, 0xF, false);
  const int64_t pi = (int64_t)(((uint64_t)phi << 32) | plo);
  if (lane > pos && lane < k) {
    ls = ps;
    li = pi;
  } else if (lane == pos) {
    ls = s;
    li = id;
  }
}

// Sorts the wave's 64 (score, id) pairs into result order, lane 0 first: a bitonic network
// of lane-xor exchanges (ids travel as two 32-bit halves).
__device__ __forceinline__ void wave_sort(float& s, int64_t& id) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const float os = __shfl_xor(s, stride, 64);
      const uint32_t olo = (uint32_t)__shfl_xor((int)(uint32_t)id, stride, 64);
      const uint32_t ohi = (uint32_t)__shfl_xor((int)(uint32_t)((uint64_t)id >> 32), stride, 64);
      const int64_t oi = (int64_t)(((uint64_t)ohi << 32) | olo);
      // the lower lane of a pair keeps the better entry in blocks sorted first-to-last
      const bool keep_better = ((lane & stride) == 0) == ((lane & size) == 0);
      if (keep_better ? better(os, oi, s, id) : better(s, id, os, oi)) {
        s = os;
        id = oi;
      }
    }
  }
}

template <int D, int B>
__global__ __launch_bounds__(64 * kSWaves) void search_scan(SearchParams p) {
  constexpr int NB = D / 32, W = NB * (B + 1);
  constexpr int KS = NB / kSWaves;      // record blocks per wave
  constexpr int kPat = s_pat_entries(B);
  // one LDS block carved by hand so that the centroid-pair table sits at address 0 (its
  // masked pattern is then the whole address):
  //   cpt  [kPat][2] u32     centroid pairs (hi, lo)
  //   spt  [16][2] u32       nibble -> 4 fp16 +-1 (set bit +1)
  //   part [2][waves][32][68] partial scores, rows padded by 4 floats so a wave's 16-row
  //                          writes hit distinct banks
  //   nrm  [2][64][2]        n16, 2^6 gamma r16 of the tile's vectors
  //   qscl [32]              per-query scales
  constexpr int oSpt = (2 * kPat + 3) / 4 * 4, oPart = oSpt + 32;
  constexpr int kPartN = 2 * kSWaves * kSQ * (kSTile + 4);
  constexpr int oNrm = oPart + kPartN, oQs = oNrm + 2 * kSTile * 2, kSmem = oQs + kSQ;
  __shared__ __attribute__((aligned(16))) uint32_t smem[kSmem];
  uint32_t* cpt = smem;
  uint32_t (*spt)[2] = reinterpret_cast<uint32_t (*)[2]>(smem + oSpt);
  float (*part)[kSWaves][kSQ][kSTile + 4] = reinterpret_cast<float (*)[kSWaves][kSQ][kSTile + 4]>(smem + oPart);
  float (*nrm)[kSTile][2] = reinterpret_cast<float (*)[kSTile][2]>(smem + oNrm);
  float* qscl = reinterpret_cast<float*>(smem + oQs);
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int64_t q0 = (int64_t)blockIdx.x * kSQ;
  const int split = blockIdx.y;
  const int64_t db_begin = (int64_t)split * p.chunk_len;
  int64_t db_end = db_begin + p.chunk_len;
  if (db_end > p.n_db) db_end = p.n_db;

  // ---- centroid-pair table
  for (int P = tid; P < kPat; P += 64 * kSWaves) {
    const int mask = (1 << B) - 1;
    const int p0 = P & 15, p1 = (P >> 4) & 15, p2 = (P >> 8) & 15;
    const int ilo = ((p0 & 1) | ((p1 & 1) << 1) | ((p2 & 1) << 2)) & mask;
    const int ihi = (((p0 >> 1) & 1) | (((p1 >> 1) & 1) << 1) | (((p2 >> 1) & 1) << 2)) & mask;
    const float c0 = p.cent[ilo] * kSCent, c1 = p.cent[ihi] * kSCent;
    const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    const _Float16 l0 = (_Float16)(c0 - (float)h0), l1 = (_Float16)(c1 - (float)h1);
    cpt[2 * P] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    cpt[2 * P + 1] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
  }
  if (tid < 32) {
    const int n = tid >> 1, d = tid & 1;
    const uint32_t lo = ((n >> (2 * d)) & 1) ? 0x3C00u : 0xBC00u;
    const uint32_t hi = ((n >> (2 * d + 1)) & 1) ? 0x3C00u : 0xBC00u;
    spt[n][d] = lo | (hi << 16);
  }
  // ---- per-query power-of-two scale putting the largest of |q_rot|, |S q_rot| in [128, 256)
  // (one scale for both, so the two terms of a score share it)
#pragma unroll
  for (int h = 0; h < kSQW; ++h) {
    const int q = kSQW * wave + h;
    const int64_t qi = q0 + q;
    float m = 0.0f;
    if (qi < p.n_q) {
#pragma unroll
      for (int e = 0; e < 2 * D / 64; ++e) m = fmaxf(m, fabsf(p.ws_q[qi * 2 * D + lane + 64 * e]));
    }
    m = wave_max_fast(m);
    if (lane == 0) qscl[q] = m > 0.0f ? exp2f(7.0f - floorf(log2f(m))) : 1.0f;
  }
  __syncthreads();

  // lane roles: A operand / loads, lane (kj, kr): byte kj of the record blocks of vector
  // 16 m + kr; B operand, lane (kj, n): coordinates 32 b + 8 kj + e of query 16 nb + n;
  // result, lane (kq, n): vectors 16 m + 4 kq + i of query 16 nb + n
  const int kj = lane >> 4, kr = lane & 15;
  const int blk0 = KS * wave;
  u32x4 bqh[2][KS], bql[2][KS], bsh[2][KS], bsl[2][KS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int q = 16 * nb + kr;
    const int64_t qi = q0 + q;
    const bool qv = qi < p.n_q;
    const float fq = qscl[q], fs = fq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = 32 * (blk0 + ks) + 8 * kj;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        float x0 = 0.0f, x1 = 0.0f, y0 = 0.0f, y1 = 0.0f;
        if (qv) {
          x0 = p.ws_q[(qi * 2) * D + c0 + 2 * d] * fq;
          x1 = p.ws_q[(qi * 2) * D + c0 + 2 * d + 1] * fq;
          y0 = p.ws_q[(qi * 2 + 1) * D + c0 + 2 * d] * fs;
          y1 = p.ws_q[(qi * 2 + 1) * D + c0 + 2 * d + 1] * fs;
        }
        const _Float16 a0 = (_Float16)x0, a1 = (_Float16)x1, b0 = (_Float16)y0, b1 = (_Float16)y1;
        const _Float16 a0l = (_Float16)(x0 - (float)a0), a1l = (_Float16)(x1 - (float)a1);
        const _Float16 b0l = (_Float16)(y0 - (float)b0), b1l = (_Float16)(y1 - (float)b1);
        auto pk = [](_Float16 u, _Float16 v) {
          return (uint32_t)__builtin_bit_cast(uint16_t, u) | ((uint32_t)__builtin_bit_cast(uint16_t, v) << 16);
        };
        bqh[nb][ks][d] = pk(a0, a1);
        bql[nb][ks][d] = pk(a0l, a1l);
        bsh[nb][ks][d] = pk(b0, b1);
        bsl[nb][ks][d] = pk(b0l, b1l);
      }
    }
  }

  // ---- register prefetch of one tile's record blocks of this wave (A layout); wave 0 also
  // fetches the norms of the tile after it (lane = vector), staged in LDS one tile ahead
  uint32_t rw[4][KS][B + 1], nr = 0;
  auto fetch = [&](int64_t tt0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int64_t v = tt0 + 16 * m + kr;
      if (v < db_end) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint32_t* rec = p.codes + v * W + (blk0 + ks) * (B + 1);
          if constexpr (B == 3) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(rec);
            rw[m][ks][0] = x[0]; rw[m][ks][1] = x[1]; rw[m][ks][2] = x[2]; rw[m][ks][3] = x[3];
          } else {
#pragma unroll
            for (int i = 0; i <= B; ++i) rw[m][ks][i] = rec[i];
          }
        }
      }
    }
    if (wave == 0) nr = tt0 + kSTile + lane < db_end ? p.norms[tt0 + kSTile + lane] : 0u;
  };
  // partial score = n16 * (c-term sum) + 2^6 gamma r16 * (sign-term sum); the query's
  // 1 / (2^6 scale) multiplies the total
  const float g64 = p.gamma * kSCent;
  auto put_norm = [&](int bsel, uint32_t x) {
    nrm[bsel][lane][0] = f16_bits_to_f32(x & 0xFFFFu);
    nrm[bsel][lane][1] = g64 * f16_bits_to_f32(x >> 16);
  };
  const char* cpb = reinterpret_cast<const char*>(cpt);
  const int k = p.k;
  float qf[kSQW];  // 1 / (2^6 scale) of the wave's list queries
#pragma unroll
  for (int h = 0; h < kSQW; ++h) qf[h] = 1.0f / (kSCent * qscl[kSQW * wave + h]);
  float ls[kSQW];
  int64_t li[kSQW];
#pragma unroll
  for (int h = 0; h < kSQW; ++h) {
    ls[h] = -INFINITY;
    li[h] = INT64_MAX;
  }

  if (wave == 0) put_norm(0, db_begin + lane < db_end ? p.norms[db_begin + lane] : 0u);
  fetch(db_begin);
  __syncthreads();
  int buf = 0;
  for (int64_t t0 = db_begin; t0 < db_end; t0 += kSTile, buf ^= 1) {
    // ---------------- this wave's coordinates of the tile on MFMA, one 16-vector block at a
    // time, then its partial scores into LDS
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f32x4 ac[2], as[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) ac[nb] = as[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t p0 = rw[m][ks][0];
        const uint32_t p1 = B >= 2 ? rw[m][ks][1] : 0u;
        const uint32_t p2 = B >= 3 ? rw[m][ks][2] : 0u;
        const uint32_t sg = rw[m][ks][B];
        u32x4 ah, al, so;
        {  // F: the pattern field of the byte's low nibble in bits 0..15, high nibble in 16..31
          // (nibble bits of plane k at 1 + 4k ..), from the three plane bytes by multiplies
          const uint32_t F = ((__builtin_amdgcn_ubfe(p0, 8 * kj, 8) * 0x2002u) & 0x001E001Eu) |
                             ((__builtin_amdgcn_ubfe(p1, 8 * kj, 8) * 0x20020u) & 0x01E001E0u) |
                             ((__builtin_amdgcn_ubfe(p2, 8 * kj, 8) * 0x200200u) & 0x1E001E00u);
          const u32x2 e0 = *reinterpret_cast<const u32x2*>(cpb + ((F << 2) & kSPatMask));
          const u32x2 e1 = *reinterpret_cast<const u32x2*>(cpb + (F & kSPatMask));
          const u32x2 e2 = *reinterpret_cast<const u32x2*>(cpb + ((F >> 14) & kSPatMask));
          const u32x2 e3 = *reinterpret_cast<const u32x2*>(cpb + ((F >> 16) & kSPatMask));
          ah[0] = e0[0]; al[0] = e0[1];
          ah[1] = e1[0]; al[1] = e1[1];
          ah[2] = e2[0]; al[2] = e2[1];
          ah[3] = e3[0]; al[3] = e3[1];
        }
        {  // sign pairs from the nibble table: bit 2d -> half 0, bit 2d + 1 -> half 1
          const u32x2 s0 = *reinterpret_cast<const u32x2*>(&spt[__builtin_amdgcn_ubfe(sg, 8 * kj, 4)][0]);
          const u32x2 s1 = *reinterpret_cast<const u32x2*>(&spt[__builtin_amdgcn_ubfe(sg, 8 * kj + 4, 4)][0]);
          so[0] = s0[0]; so[1] = s0[1]; so[2] = s1[0]; so[3] = s1[1];
        }
        const h16x8 Ah = __builtin_bit_cast(h16x8, ah), Al = __builtin_bit_cast(h16x8, al);
        const h16x8 Ao = __builtin_bit_cast(h16x8, so);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          ac[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, __builtin_bit_cast(h16x8, bqh[nb][ks]), ac[nb], 0, 0, 0);
          ac[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, __builtin_bit_cast(h16x8, bqh[nb][ks]), ac[nb], 0, 0, 0);
          ac[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, __builtin_bit_cast(h16x8, bql[nb][ks]), ac[nb], 0, 0, 0);
          as[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, __builtin_bit_cast(h16x8, bsh[nb][ks]), as[nb], 0, 0, 0);
          as[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, __builtin_bit_cast(h16x8, bsl[nb][ks]), as[nb], 0, 0, 0);
        }
      }
      const f32x4 na = *reinterpret_cast<const f32x4*>(&nrm[buf][16 * m + 4 * kj][0]);
      const f32x4 nb4 = *reinterpret_cast<const f32x4*>(&nrm[buf][16 * m + 4 * kj + 2][0]);
      const float nn[4] = {na[0], na[2], nb4[0], nb4[2]}, rr[4] = {na[1], na[3], nb4[1], nb4[3]};
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        f32x4 ps;
#pragma unroll
        for (int i = 0; i < 4; ++i) ps[i] = fmaf(nn[i], ac[nb][i], rr[i] * as[nb][i]);
        *reinterpret_cast<f32x4*>(&part[buf][wave][16 * nb + kr][16 * m + 4 * kj]) = ps;
      }
    }
    if (wave == 0) put_norm(buf ^ 1, nr);  // the next tile's norms, fetched a tile ago
    fetch(t0 + kSTile);
    __syncthreads();
    // ---------------- scores and top-k lists of queries kSQW * wave + h (lane = vector)
    const int64_t v = t0 + lane;
    const bool valid = v < db_end;
#pragma unroll
    for (int h = 0; h < kSQW; ++h) {
      const int q = kSQW * wave + h;
      if (q0 + q >= p.n_q) continue;
      float sc = part[buf][0][q][lane];
#pragma unroll
      for (int w2 = 1; w2 < kSWaves; ++w2) sc += part[buf][w2][q][lane];
      sc = valid ? sc * qf[h] : -INFINITY;
      const float kth = lane_f(ls[h], k - 1);
      uint64_t cand = __ballot(sc >= kth);  // a superset of the candidates (-inf never enters)
      if (cand == 0) continue;
      const int64_t kid = lane_i64(li[h], k - 1);
      cand = __ballot(valid && better(sc, v, kth, kid));
      while (cand) {
        const int L = __builtin_ctzll(cand);
        cand &= cand - 1;
        const float s = lane_f(sc, L);
        list_insert(ls[h], li[h], s, t0 + L, k);
      }
    }
  }
  // ---- results (each query's list is complete in its owner wave)
#pragma unroll
  for (int h = 0; h < kSQW; ++h) {
    const int64_t qi = q0 + kSQW * wave + h;
    if (qi >= p.n_q || lane >= k) continue;
    if (p.n_split == 1) {
      p.out_scores[qi * k + lane] = ls[h];
      p.out_ids[qi * k + lane] = li[h];
    } else {
      p.ws_cand_s[(qi * p.n_split + split) * k + lane] = ls[h];
      p.ws_cand_i[(qi * p.n_split + split) * k + lane] = li[h];
    }
  }
}

// ----------------------------------------------------------------------------- merge
// One workgroup per query, of up to kMWaves waves (about 512 candidates per wave).  Wave w
// screens a contiguous share of the query's n_split * k split candidates, 64 at a time (one
// per lane): a ballot against its list's current k-th entry, then the survivors are
// inserted in lane order.  Wave 0 then inserts the other waves' lists.  (score, id) is a
// total order, so the result does not depend on the order of the inserts.
constexpr int kMWaves = 16;
__host__ __device__ inline int merge_waves(int64_t candidates) {
  const int64_t w = (candidates + 511) / 512;
  return w < 1 ? 1 : (w > kMWaves ? kMWaves : (int)w);
}
__global__ __launch_bounds__(64 * kMWaves) void search_merge(SearchParams p) {
  const int64_t qi = blockIdx.x;
  const int lane = lane_id(), wave = threadIdx.x >> 6, k = p.k;
  const int nw = (int)(blockDim.x >> 6);
  __shared__ float xs[kMWaves][64];
  __shared__ int64_t xi[kMWaves][64];
  const int64_t total = (int64_t)p.n_split * k;
  const int64_t per = (total + nw - 1) / nw;
  const int64_t c0 = wave * per;
  const int64_t c1 = c0 + per < total ? c0 + per : total;
  const float* cs = p.ws_cand_s + qi * total;
  const int64_t* ci = p.ws_cand_i + qi * total;
  float ms = -INFINITY;
  int64_t mi = INT64_MAX;
  constexpr int kR = 8;  // batches of 64 whose loads are issued together
  for (int64_t c = c0; c < c1; c += 64 * kR) {
    float scr[kR];
    int64_t idr[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const bool ok = c + 64 * r + lane < c1;
      scr[r] = ok ? cs[c + 64 * r + lane] : -INFINITY;
      idr[r] = ok ? ci[c + 64 * r + lane] : INT64_MAX;
    }
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      float sc = scr[r];
      int64_t id = idr[r];
      if (r == 0 && c == c0) {  // the list is empty: the first batch, sorted, gives it
        wave_sort(sc, id);
        ms = lane < k ? sc : -INFINITY;
        mi = lane < k ? id : INT64_MAX;
        continue;
      }
      uint64_t cand = __ballot(id != INT64_MAX && better(sc, id, lane_f(ms, k - 1), lane_i64(mi, k - 1)));
      while (cand) {
        const int L = __builtin_ctzll(cand);
        cand &= cand - 1;
        list_insert(ms, mi, lane_f(sc, L), lane_i64(id, L), k);
      }
    }
  }
  xs[wave][lane] = ms;
  xi[wave][lane] = mi;
  __syncthreads();
  if (wave != 0) return;
  for (int w = 1; w < nw; ++w) {
    const float sc = xs[w][lane];
    const int64_t id = xi[w][lane];
    uint64_t cand = __ballot(lane < k && better(sc, id, lane_f(ms, k - 1), lane_i64(mi, k - 1)));
    while (cand) {
      const int L = __builtin_ctzll(cand);
      cand &= cand - 1;
      list_insert(ms, mi, lane_f(sc, L), lane_i64(id, L), k);
    }
  }
  if (lane < k) {
    p.out_scores[qi * k + lane] = ms;
    p.out_ids[qi * k + lane] = mi;
  }
}

// With at most kFewQ queries (five blocks of four) the scan below, which reads the database
// once per block of four, beats the batched scan, which expands it once per 32 queries.
constexpr int kFewQ = 20;

// A float as an int whose signed order is the float order (for an LDS maximum), and back.
__device__ __forceinline__ int ord_of(float f) {
  const int b = __float_as_int(f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float float_of_ord(int o) {
  return __int_as_float(o ^ ((o >> 31) & 0x7FFFFFFF));
}

// ----------------------------------------------------------------------------- few queries
// on the block-scaled matrix cores.  Up to four queries are scored together by
// v_mfma_scale_f32_16x16x128_f8f6f4 straight from the records (the operand encodings are
// described in tq_mx.h): the symmetric codebook is an odd function of the code bits, so
// c[idx] = sum_k alpha_k s_k over the odd Walsh monomials s_k of the bit-planes (for 3 bits:
// s0, s1, s2 and s0 s1 s2, the XOR plane), and the estimator of query q and vector x is
//   n16 sum_k <alpha_k q_rot, s_k> + gamma r16 <S q_rot, sigma>,
// a sum of products of real query weights with +-1 planes.  A: the weights, 16 rows = 4
// queries x 4 base-16 digits, eight digits in two products (x truncated to 32 bits), per
// plane and 128-coordinate K block; B: one plane word of 16 database vectors per 32-row
// block, lane (g, n) holding block 4 kb + g of vector n.  Lane (h, n) of a result holds
// query h's sum for vector n.  Each wave walks 32-vector tiles of the workgroup's database
// range (the next tile's records in flight) and keeps one top-k list per query (lane i the
// i-th best); the workgroup's lists of each query (one per wave) are merged at the end.
// Grid: (database split, block of four queries).
constexpr int kMqWaves = 8;   // two per SIMD
constexpr int kMqTile = 32;   // vectors per wave tile: two 16-vector products

template <int D, int B>
__global__ __launch_bounds__(64 * kMqWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void search_mxq(SearchParams p) {
  using tqx::i32x4;
  using tqx::i32x8;
  constexpr int NKB = D / 128;              // K blocks of 128 coordinates
  constexpr int NP = (B == 3) ? 4 : B;      // Walsh planes of the codebook
  constexpr int WB = B + 1;                 // words per 32-coordinate block (planes, signs)
  constexpr int W = (D / 32) * WB;          // words per record
  constexpr int NU = (NP + 1) * NKB;        // A operand units: (plane or signs, K block)
  constexpr int NG = kMqTile / 16;          // products per tile and K block
  __shared__ float s_q[4 * 2 * D];          // per query: q_rot, then S q_rot (zero: no query)
  __shared__ uint32_t s_ak[NU][2][6][64];   // A operands, digits 0-3 and 4-7
  __shared__ int s_ke[NU][64];              // block exponent of each A lane
  __shared__ float s_c[4][2];               // per query: constants of the two terms
  __shared__ int s_thr[4];                  // per query: the best k-th score of any wave's list
  __shared__ float xs[kMqWaves][4][64];
  __shared__ int64_t xi[kMqWaves][4][64];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int64_t split = blockIdx.x;
  const int64_t q0 = (int64_t)blockIdx.y * 4;   // this workgroup's block of four queries
  const int nq = (int)(p.n_q - q0 < 4 ? p.n_q - q0 : 4);
  const int k = p.k;
  const int64_t db_begin = split * p.chunk_len;
  const int64_t db_end = db_begin + p.chunk_len < p.n_db ? db_begin + p.chunk_len : p.n_db;
  const int g = lane >> 4, n = lane & 15, hh = lane >> 4;

  // ---- records of a tile: lane (g, n) holds block 4 kb + g of vector t0 + 16 j + n
  uint32_t cw[NG][NKB][WB], cn[NG];
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int64_t v = t0 + 16 * j + n;
      if (v < db_end) {
        const uint32_t* rec = p.codes + v * W;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const uint32_t* bw = rec + (4 * kb + g) * WB;
          if constexpr (WB == 4) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(bw);
            cw[j][kb][0] = x[0]; cw[j][kb][1] = x[1]; cw[j][kb][2] = x[2]; cw[j][kb][3] = x[3];
          } else if constexpr (WB == 2) {
            const u32x2 x = *reinterpret_cast<const u32x2*>(bw);
            cw[j][kb][0] = x[0]; cw[j][kb][1] = x[1];
          } else {
#pragma unroll
            for (int i = 0; i < WB; ++i) cw[j][kb][i] = bw[i];
          }
        }
        cn[j] = p.norms[v];
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < WB; ++i) cw[j][kb][i] = 0u;
        cn[j] = 0u;
      }
    }
  };
  int64_t t0 = db_begin + (int64_t)wave * kMqTile;
  if (t0 < db_end) fetch(t0);

  // ---- the queries' q_rot and S q_rot (from the prologue kernel), zero rows past n_q
  for (int i = tid; i < 4 * 2 * D; i += 64 * kMqWaves)
    s_q[i] = i < nq * 2 * D ? p.ws_q[q0 * 2 * D + i] : 0.0f;
  if (tid < 4) s_thr[tid] = ord_of(-INFINITY);
  __syncthreads();
  if (wave < 4) {  // per query (wave): the constants left by the D < 3 nibble positions
    const float* qr = s_q + wave * 2 * D;
    const float asum = p.alpha[0] + p.alpha[1] + p.alpha[2] + p.alpha[3];
    float cc = 0.f, cs = 0.f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
      const int j = lane + 64 * e;
      if ((j & 3) != 3) {
        cc = fmaf(asum, qr[j], cc);
        cs += qr[D + j];
      }
    }
    cc = wave_sum_fast(cc);
    cs = wave_sum_fast(cs);
    if (lane == 0) {
      s_c[wave][0] = cc;
      s_c[wave][1] = cs;
    }
  }
  {  // A operands: unit u = kb (NP + 1) + plane, spread over the waves.  A lane (g, m) holds
     // row m = (query m / 4, digit m % 4) for K = 32 g + p, coordinate
     // 128 kb + 32 g + 4 (p % 8) + p / 8, weight f_{p / 8} alpha_k q_rot (planes) or
     // f_{p / 8} (S q_rot) (signs); x = |a| 2^-e truncated to 32 bits, digits 0-3 and 4-7.
    const int m = lane & 15, hq = m >> 2, l = m & 3;
    for (int u = wave; u < NU; u += kMqWaves) {
      const int kb = u / (NP + 1), kk = u % (NP + 1);
      const float alpha = kk < NP ? p.alpha[kk] : 1.0f;
      const float* src = s_q + hq * 2 * D + (kk < NP ? 0 : D) + 128 * kb + 32 * g;
      float av[32];
      float amax = 0.f;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        const int Dn = q >> 3;
        const float f = Dn == 0 ? 4.0f : Dn == 1 ? 2.0f : Dn == 2 ? 1.0f : -2.0f;
        av[q] = f * (alpha * src[4 * (q & 7) + Dn]);
        amax = fmaxf(amax, fabsf(av[q]));
      }
      const int e = tqx::block_exp(amax);
      uint32_t rr[32];
#pragma unroll
      for (int q = 0; q < 32; ++q)
        rr[q] = e == tqx::kZeroExp ? 0u : (uint32_t)ldexpf(fabsf(av[q]), 32 - e);
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        const int sh = (part == 0 ? 28 : 12) - 4 * l;
        tqx::u32x16 hd16;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          hd16[i] = ((rr[2 * i] >> sh) & 15u) | (((rr[2 * i + 1] >> sh) & 15u) << 16) |
                    ((__float_as_uint(av[2 * i]) >> 16) & 0x8000u) |
                    (__float_as_uint(av[2 * i + 1]) & 0x80000000u);
        const i32x8 a = tqx::fp6_row_f16(hd16);
#pragma unroll
        for (int r = 0; r < 6; ++r) s_ak[u][part][r][lane] = (uint32_t)a[r];
      }
      s_ke[u][lane] = e;
    }
  }
  __syncthreads();
  i32x8 akh[NU], akl[NU];
  int ksh[NU], ksl[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      akh[u][r] = r < 6 ? (int)s_ak[u][0][r][lane] : 0;
      akl[u][r] = r < 6 ? (int)s_ak[u][1][r][lane] : 0;
    }
    const int e = s_ke[u][lane];
    ksh[u] = tqx::digit_scale(e, lane & 3);
    ksl[u] = tqx::digit_scale(e, 4 + (lane & 3));
  }
  const f32x4 c0_c = {-s_c[hh][0], 0.f, 0.f, 0.f}, c0_s = {-s_c[hh][1], 0.f, 0.f, 0.f};
  const uint32_t ones = __builtin_amdgcn_readfirstlane(0x11111111);

  float ls[4];        // per query: the list (lane i the i-th best)
  int64_t li[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    ls[h] = -INFINITY;
    li[h] = INT64_MAX;
  }
  for (; t0 < db_end; t0 += (int64_t)kMqWaves * kMqTile) {
    uint32_t w[NG][NKB][WB], wn[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      wn[j] = cn[j];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < WB; ++i) w[j][kb][i] = cw[j][kb][i];
    }
    const int64_t tn = t0 + (int64_t)kMqWaves * kMqTile;
    if (tn < db_end) fetch(tn);
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      f32x4 ac = c0_c, as = c0_s;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int u0 = kb * (NP + 1);
        const i32x4 b0 = tqx::fp4_of(w[j][kb][0], ones);
        ac = tqx::mma(akh[u0], b0, ac, ksh[u0]);
        ac = tqx::mma(akl[u0], b0, ac, ksl[u0]);
        if constexpr (NP >= 2) {
          const i32x4 b1 = tqx::fp4_of(w[j][kb][1], ones);
          ac = tqx::mma(akh[u0 + 1], b1, ac, ksh[u0 + 1]);
          ac = tqx::mma(akl[u0 + 1], b1, ac, ksl[u0 + 1]);
          if constexpr (NP == 4) {
            const i32x4 b2 = tqx::fp4_of(w[j][kb][2], ones), b3 = tqx::fp4_xor3(b0, b1, b2);
            ac = tqx::mma(akh[u0 + 2], b2, ac, ksh[u0 + 2]);
            ac = tqx::mma(akl[u0 + 2], b2, ac, ksl[u0 + 2]);
            ac = tqx::mma(akh[u0 + 3], b3, ac, ksh[u0 + 3]);
            ac = tqx::mma(akl[u0 + 3], b3, ac, ksl[u0 + 3]);
          }
        }
        const i32x4 bs = tqx::fp4_of(w[j][kb][B], ones);
        as = tqx::mma(akh[u0 + NP], bs, as, ksh[u0 + NP]);
        as = tqx::mma(akl[u0 + NP], bs, as, ksl[u0 + NP]);
      }
      // lane (hh, n): query hh's score of vector t0 + 16 j + n
      const float dc = (ac[0] + ac[1]) + (ac[2] + ac[3]);
      const float ds = (as[0] + as[1]) + (as[2] + as[3]);
      const float n16 = f16_bits_to_f32(wn[j] & 0xFFFFu), r16 = f16_bits_to_f32(wn[j] >> 16);
      const float sc = fmaf(n16, dc, p.gamma * r16 * ds);
      const int64_t vb = t0 + 16 * j;
      const bool valid = vb + n < db_end;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (h >= nq) break;
        // a score below another wave's k-th score cannot reach the workgroup's top k (that
        // list already holds k better entries); the shared bound only grows, so an older
        // value read here is still a valid one
        const float thr = float_of_ord(s_thr[h]);
        const float kth = lane_f(ls[h], k - 1);
        const int64_t kid = lane_i64(li[h], k - 1);
        uint64_t cand = __ballot(hh == h && valid && sc >= thr && better(sc, vb + n, kth, kid));
        if (cand) {
          while (cand) {
            const int L = __builtin_ctzll(cand);
            cand &= cand - 1;
            list_insert(ls[h], li[h], lane_f(sc, L), vb + (L & 15), k);
          }
          const float kth2 = lane_f(ls[h], k - 1);
          if (lane == 0 && kth2 > -INFINITY) atomicMax(&s_thr[h], ord_of(kth2));
        }
      }
    }
  }
  // ---- the waves' lists of each query into one (wave h merges query h)
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    xs[wave][h][lane] = ls[h];
    xi[wave][h][lane] = li[h];
  }
  __syncthreads();
  if (wave >= nq) return;
  const int h = wave;
  float ms = xs[0][h][lane];
  int64_t mi = xi[0][h][lane];
#pragma unroll
  for (int w2 = 1; w2 < kMqWaves; ++w2) {
    const float s2 = xs[w2][h][lane];
    const int64_t i2 = xi[w2][h][lane];
    uint64_t cand = __ballot(lane < k && better(s2, i2, lane_f(ms, k - 1), lane_i64(mi, k - 1)));
    while (cand) {
      const int L = __builtin_ctzll(cand);
      cand &= cand - 1;
      list_insert(ms, mi, lane_f(s2, L), lane_i64(i2, L), k);
    }
  }
  if (lane < k) {
    if (p.n_split == 1) {
      p.out_scores[(q0 + h) * k + lane] = ms;
      p.out_ids[(q0 + h) * k + lane] = mi;
    } else {
      p.ws_cand_s[((q0 + h) * p.n_split + split) * k + lane] = ms;
      p.ws_cand_i[((q0 + h) * p.n_split + split) * k + lane] = mi;
    }
  }
}

template <int D, int B>
static int launch_search(const SearchParams& p, int64_t n_blocks, hipStream_t stream) {
  hipLaunchKernelGGL(search_prologue<D>, dim3((unsigned)p.n_q, kPrologueSlices), dim3(256), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
  if (p.n_q <= kFewQ)
    hipLaunchKernelGGL((search_mxq<D, B>), dim3((unsigned)p.n_split, (unsigned)((p.n_q + 3) / 4)),
                       dim3(64 * kMqWaves), 0, stream, p);
  else
    hipLaunchKernelGGL((search_scan<D, B>), dim3((unsigned)n_blocks, (unsigned)p.n_split),
                       dim3(64 * kSWaves), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
  if (p.n_split > 1) {
    const int nw = merge_waves((int64_t)p.n_split * p.k);
    hipLaunchKernelGGL(search_merge, dim3((unsigned)p.n_q), dim3(64 * nw), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
  }
  return TQ_OK;
}

}  // namespace tqk

// ---------------------------------------------------------------------------------------
tq_search_plan tq_plan_search(int64_t n_q, int32_t k, int64_t n_db, int32_t d) {
  using namespace tqk;
  tq_search_plan p{};
  const int64_t blocks = (n_q + kSQ - 1) / kSQ;
  // split the database so that the grid has several rounds of two workgroups per CU of a
  // 256-CU MI355X (a short last round costs less), with at least 16 tiles per split
  const int64_t nb = blocks > 0 ? blocks : 1;
  int64_t n_split = (2048 + nb - 1) / nb;
  {
    // every workgroup scans an equal share, so the grid runs in rounds of 512 (two per CU);
    // among n_split .. 2 n_split take the first count whose last round is at most 1/32 idle,
    // else the least idle one (313 query blocks: 8 splits leave 2% of the last round idle, 7
    // splits 14%)
    const int64_t base = n_split;
    int64_t best_c = base;
    double best = 2.0;
    for (int64_t c = base; c <= 2 * base; ++c) {
      const int64_t wg = nb * c, rounds = (wg + 511) / 512;
      const double idle = (double)(rounds * 512 - wg) / (double)(rounds * 512);
      if (idle < best) {
        best = idle;
        best_c = c;
      }
      if (idle <= 1.0 / 32.0) break;
    }
    n_split = best_c;
  }
  // few queries (one workgroup of 8 waves per split and block of four queries): one
  // workgroup per CU and block, two waves per SIMD
  if (n_q <= kFewQ) n_split = 256;
  const int64_t max_split = (n_db + 16 * kSTile - 1) / (16 * kSTile);
  if (n_split > max_split) n_split = max_split;
  if (n_split > 4096) n_split = 4096;
  if (n_split < 1) n_split = 1;
  const int64_t chunk = (n_db + n_split - 1) / n_split;
  p.n_chunks = (int32_t)n_split;
  p.chunk_len = (chunk + kSTile - 1) / kSTile * kSTile;
  p.ws_q_off = 0;
  const int64_t q_bytes = (n_q > 0 ? n_q : 1) * 2 * d * 4;
  p.ws_cand_off = (q_bytes + 255) / 256 * 256;
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
  p.ws_q = reinterpret_cast<float*>(ws + plan.ws_q_off);
  const int64_t nsk = n_q * plan.n_chunks * k;
  p.ws_cand_i = reinterpret_cast<int64_t*>(ws + plan.ws_cand_off);
  p.ws_cand_s = reinterpret_cast<float*>(ws + plan.ws_cand_off + nsk * 8);
  p.n_db = n_db;
  p.n_q = n_q;
  p.chunk_len = plan.chunk_len;
  p.d_in = d_in;
  p.k = k;
  p.n_split = plan.n_chunks;
  p.gamma = (float)(std::sqrt(M_PI / 2.0) / f->d);
  for (int j = 0; j < 8; ++j) p.sign_mask[j] = 0;
  for (int j = 0; j < f->d; ++j)
    if (t->signs[j] < 0) p.sign_mask[j >> 5] |= 1u << (j & 31);
  for (int i = 0; i < 8; ++i) p.cent[i] = i < (1 << f->bits_lo) ? t->centroids_lo[i] : 0.0f;
  tq_walsh_coeffs(f->bits_lo, t->centroids_lo, p.alpha);
  const int64_t n_blocks = (n_q + kSQ - 1) / kSQ;
  if (f->d == 256) {
    if (f->bits_lo == 3) return launch_search<256, 3>(p, n_blocks, stream);
    if (f->bits_lo == 2) return launch_search<256, 2>(p, n_blocks, stream);
  } else {
    if (f->bits_lo == 3) return launch_search<128, 3>(p, n_blocks, stream);
    if (f->bits_lo == 2) return launch_search<128, 2>(p, n_blocks, stream);
    if (f->bits_lo == 1) return launch_search<128, 1>(p, n_blocks, stream);
  }
  return TQ_ERR_SHAPE;
}
