// Decode attention straight from the packed cache (163.com explainer,
// m.163.com/dy/article/KOV7P8JI0556C3J2, sections "第二步：QJL" and "速度"):
//   logit_t = scale * ( n16_t <q_rot, c[idx_t]> + gamma r16_t <S q_rot, 2 sigma_t - 1> ),
//   q_rot = H D q / sqrt(d), gamma = sqrt(pi/2) / d;
//   softmax over t < seq_len; out = Pi^T ( sum_t p_t (n16 c[idx] + gamma r16 S^T sigma) ).
// Because <q, Pi^T v> = <Pi q, v> and <q_rot, S^T s> = <S q_rot, s>, the cache is never
// rotated back per token: values are accumulated in the rotated domain and each head's
// result is mapped back once (S^T, then D H / sqrt(d)).
//
// Two launches:
//   scan:     grid (split, batch * KV head * chunk of GC query heads), about one
//             workgroup of 8 waves per CU.  The workgroup first derives its own query
//             tables (while its first cache tile is in flight): q_rot of the GC
//             heads (FWHT over the wave), S q_rot (S rows from L2), and in LDS
//               Tq[g][m] = sum of q_rot over the set bits of byte m of coordinate group g
//               Ts[g][n] = 2 * sum of S q_rot over the set bits of nibble n,
//             one float per head.  A sign dot product <w, 2b - 1> over 128 coordinates is
//             then 16 byte (or 32 nibble) table reads: the codebook term through the Walsh
//             expansion of the symmetric codebook, c[idx] = sum_S alpha_S prod_{k in S}
//             (2 b_k - 1) over odd subsets S of the code bit-planes (the planes, and for
//             3 bits their XOR), the QJL term directly.
//             Keys: lane = token, key records and norms of the wave's next 64-token tile
//             prefetched into registers; value records are read after the softmax step.  Online softmax per head with wavefront reductions; the Sparse-V
//             gate (zhidx turboquant_plus article, section "01 turboquant_plus：介绍与详解")
//             drops a value row for a head when its running weight estimate is below tau,
//             and skips reading rows dropped by every head.
//             Values: the weighted sums A = sum_t u_t c[idx_t] (u = w n16) and
//             Q = sum_t u'_t (2 sigma_t - 1) (u' = w gamma r16) are products of a
//             (coordinates x tokens) matrix with a (tokens x heads) matrix, so they run on
//             v_mfma_f32_16x16x32_f16 per 32-token group: lane (q, r) expands coordinates
//             8r .. 8r + 7 of tokens 8q .. 8q + 7 (one byte of each code plane) into fp16
//             operands, the centroid pair of two coordinates from one read of a table
//             indexed by their code bits, the sign pair directly from the bits.  Centroids
//             (scaled by 2^6) and weights are split into fp16 hi + lo halves and the weight
//             columns carry both halves (heads x {hi, lo}), so the fp32 accumulation sees
//             the full product to ~2^-22; sign operands (+-1) are exact.  Groups with no
//             kept token are skipped.
//             The waves' partial (m, l, acc) are merged in LDS: one partial per workgroup.
//             MSE-only values (no sign words) drop the QJL term of the value sum.
//   combine:  per (batch, query head) one workgroup merges the splits in a fixed order and
//             maps back: out = D H (A + S^T Q) / (sqrt(d) l).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

constexpr int kD = 128;
constexpr int kNB = kD / 32;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;
constexpr int kPartFloats = 2 + 2 * kD;  // m (log2 domain), l, A[d], Q[d]
constexpr float kLog2e = 1.4426950408889634f;

__host__ __device__ constexpr int round4(int x) { return (x + 3) / 4 * 4; }

// Record layout of a format with SPLITB blocks of BLO bits then blocks of BHI bits; each
// block holds its code planes and, when Q is 1, one QJL sign word.
template <int BLO, int BHI, int SPLITB, int Q = 1>
struct Rec {
  static constexpr int W = SPLITB * (BLO + Q) + (kNB - SPLITB) * (BHI + Q);  // words
  static constexpr int VEC = (W % 4 == 0) ? 4 : ((W % 2 == 0) ? 2 : 1);      // load width
  static constexpr int bits(int blk) { return blk < SPLITB ? BLO : BHI; }
  __host__ __device__ static constexpr int off(int blk) {
    return blk < SPLITB ? blk * (BLO + Q) : SPLITB * (BLO + Q) + (blk - SPLITB) * (BHI + Q);
  }
};

template <int W, int VEC>
__device__ __forceinline__ void load_record(const uint32_t* rec, uint32_t (&w)[W]) {
  if constexpr (VEC == 4) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const u32x4 v = reinterpret_cast<const u32x4*>(rec)[i];
      w[4 * i] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
    }
  } else if constexpr (VEC == 2) {
#pragma unroll
    for (int i = 0; i < W / 2; ++i) {
      const u32x2 v = reinterpret_cast<const u32x2*>(rec)[i];
      w[2 * i] = v[0]; w[2 * i + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = rec[i];
  }
}

// Value centroid-pair tables (one per codebook width): the entry for the 6-bit index
// x = a0 | b0 << 1 | a1 << 2 | b1 << 3 | a2 << 4 | b2 << 5, where a_k and b_k are the
// plane-k code bits of two coordinates, is 8 bytes: fp16 (hi(c'[a]), hi(c'[b])) then
// (lo(c'[a]), lo(c'[b])), with c' = 2^6 c, lo = c' - hi and a, b the two codes.
constexpr int kPairEntries = 64;
constexpr float kCentScale = 64.0f;   // value centroids in the operand tables are 2^6 c
constexpr float kQjlScale = 16.0f;    // QJL value weights in the operands are 2^4 u'

struct DecodeParams {
  const void* q;
  const uint32_t* codes_k;
  const uint32_t* norms_k;
  const uint32_t* codes_v;
  const uint32_t* norms_v;
  const int32_t* seq_lens;
  const float* S_k;
  const float* S_v;
  float* out;
  float* logits;
  unsigned long long* skipped;
  float* ws_part;   // [batch*hq][n_split][kPartFloats]
  int64_t capacity;
  int64_t tokens_per_split;
  int32_t batch, hq, hkv, group, q_dtype, n_split;
  float scale, tau, gamma;
  uint32_t sign_k[4], sign_v[4];
  float alpha_k[2][4];  // Walsh coefficients of the key codebooks (lo, hi parts)
  float cent_v[2][8];   // value codebooks (lo, hi)
  int32_t ksplitb;
  // Paged cache (block_table == nullptr: contiguous [batch][hkv][capacity] rows).  Token t
  // of batch b, KV head h is row (page * hkv + h) * 2^page_log2 + t % 2^page_log2 with
  // page = block_table[b * max_blocks + t / 2^page_log2]; a page id outside
  // [0, num_pages) makes its tokens count as absent.
  const int32_t* block_table;
  int64_t num_pages;
  int32_t max_blocks, page_log2;
  int32_t bt_stride;      // block-table row stride (0: every query reads one table)
  int64_t causal_start;   // >= 0: query b sees tokens t <= causal_start + b (prefill chunk)
  int32_t split_base;     // index of this launch's first split among the n_split partials
};

// LDS layout of one scan workgroup (floats).
template <int GC, int VW, int BVLO, int BVHI, int VSPLIT>
struct ScanLds {
  static constexpr int kTq = 16 * 256 * GC;   // [16 byte groups][256][GC]
  static constexpr int kTs = 32 * 16 * GC;    // [32 nibble groups][16][GC]
  // pair tables at byte 0 and 512: an entry's address is its index times 8, OR the base
  static constexpr int kCpLo = 2 * kPairEntries;
  static constexpr int kCpHi = VSPLIT < kNB ? 2 * kPairEntries : 0;
  static constexpr int kRS = round4(VW);                 // value record row stride (words)
  // per wave: 64 value records, then fp16 weight rows [17][kWS]: 0..7 codebook-term
  // columns (u hi for the GC heads, then u lo), 8..15 QJL-term columns, 16 zero; rows
  // padded so the 8 rows one read touches fall in distinct banks
  static constexpr int kWRows = 17;
  static constexpr int kWS = kTile + 8;
  static constexpr int kArea = kTile * kRS + kWRows * kWS / 2;
  // small tables first so their reads use the instruction's immediate offset
  static constexpr int oCpLo = 0, oCpHi = oCpLo + kCpLo, oTs = oCpHi + kCpHi;
  static constexpr int oCc = oTs + kTs;                   // [2][GC] per-head constants
  static constexpr int oTq = oCc + round4(2 * GC), oArea = oTq + kTq;
  static constexpr int kTotal = oArea + kWaves * kArea;
  static constexpr int kMerge = round4(2 * GC) + 2 * kD * GC;  // per wave
  static constexpr int oWM = oTq;  // the waves' partials after the scan (aliases Tq)
  static_assert(kWaves * kMerge <= kTq, "merge area must fit in the byte tables");
  static_assert(2 * GC * kD + 16 * 2 * 16 * GC + 16 <= kWaves * kArea, "setup scratch must fit");
};

// Value of lane (lane ^ 32): v_permlane32_swap exchanges the two half-waves.
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((lane_id() & 32) ? r[0] : r[1]);
}

template <int M>
__device__ __forceinline__ float hbfly(float x, int lane) {  // lower lane a + b, upper a - b
  const float t = (M == 32) ? other_half(x) : xchg<(M < 32 ? M : 1)>(x);
  return (lane & M) ? t - x : x + t;
}

// Unnormalized natural-order Walsh-Hadamard transform of 128 values held by one wave as
// v[0] = x[lane], v[1] = x[lane + 64].
__device__ __forceinline__ void fwht128(float (&v)[2], int lane) {
  {
    const float a = v[0], c = v[1];
    v[0] = a + c;
    v[1] = a - c;
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    float x = v[e];
    x = hbfly<1>(x, lane);
    x = hbfly<2>(x, lane);
    x = hbfly<4>(x, lane);
    x = hbfly<8>(x, lane);
    x = hbfly<16>(x, lane);
    x = hbfly<32>(x, lane);
    v[e] = x;
  }
}

// LDS floats one scan workgroup of a format pair needs.
template <int BVLO, int BVHI, int VSPLIT, bool VQ, int GC>
constexpr int scan_lds_floats() {
  return ScanLds<GC, Rec<BVLO, BVHI, VSPLIT, VQ ? 1 : 0>::W, BVLO, BVHI, VSPLIT>::kTotal;
}

// The scan of split `split` of one (batch, KV head, head chunk) unit (blockIdx.y); lds is
// the workgroup's LDS array of at least scan_lds_floats<...>() floats.
// VQ: the value records carry QJL sign words (else MSE-only values: no residual term).
template <int BKLO, int BKHI, int KSPLIT, int BVLO, int BVHI, int VSPLIT, bool VQ, int GC>
__device__ __forceinline__ void scan_body(const DecodeParams& p, float* lds, int split) {
  using KR = Rec<BKLO, BKHI, KSPLIT>;
  using VR = Rec<BVLO, BVHI, VSPLIT, VQ ? 1 : 0>;
  constexpr int KW = KR::W, VW = VR::W;
  using L = ScanLds<GC, VW, BVLO, BVHI, VSPLIT>;
  constexpr int kRS = L::kRS;
  float* Tq = lds + L::oTq;
  float* Ts = lds + L::oTs;
  float* cpLo = lds + L::oCpLo;
  float* cpHi = lds + L::oCpHi;
  float* cconst = lds + L::oCc;  // [2][GC]: codebook-term and QJL-term constants per head

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const int nchunk = p.group / GC;
  const int unit = blockIdx.y;
  const int chunk = unit % nchunk;
  const int bk = unit / nchunk;  // b * hkv + kv head
  const int b = bk / p.hkv;
  const int h0 = (bk % p.hkv) * p.group + chunk * GC;
  int64_t seq = p.causal_start >= 0 ? p.causal_start + b + 1 : (int64_t)p.seq_lens[b];
  if (seq > p.capacity) seq = p.capacity;
  const int64_t t_begin = (int64_t)split * p.tokens_per_split;
  int64_t t_end = t_begin + p.tokens_per_split;
  if (t_end > seq) t_end = seq;
  const int64_t kv_base = (int64_t)bk * p.capacity;
  const bool gated = p.tau > 0.0f;

  // cache row of token tt0 (a multiple of the 64-token tile, so a tile never straddles a
  // page); -1 for a page id out of range
  auto tile_row = [&](int64_t tt0) -> int64_t {
    if (!p.block_table) return kv_base + tt0;
    const int32_t pg = p.block_table[(int64_t)b * p.bt_stride + (tt0 >> p.page_log2)];
    if (pg < 0 || (int64_t)pg >= p.num_pages) return -1;
    return (((int64_t)pg * p.hkv + (bk % p.hkv)) << p.page_log2) + (tt0 & ((1ll << p.page_log2) - 1));
  };
  // ---- register prefetch of one tile: key record and both norms.  The value record is
  // read later, once the tile's weights are known (fewer live registers while the keys
  // are scored, and no read of a row that no head keeps)
  uint32_t kw[KW], knr = 0, vnr = 0;
  int64_t prow = -1;  // cache row of the prefetched tile's first token
  // the cache row of the tile after the prefetched one is looked up a tile ahead, so a
  // block-table read never sits right before the record loads that depend on it
  constexpr int64_t kStride = (int64_t)kWaves * kTile;
  int64_t row_ahead = -1;
  auto fetch = [&](int64_t tt0) {
    const int64_t t = tt0 + lane;
    prow = tt0 < t_end ? row_ahead : -1;
    row_ahead = tt0 + kStride < t_end ? tile_row(tt0 + kStride) : -1;
    if (prow >= 0 && t < t_end) {
      const int64_t row = prow + lane;
      load_record<KW, KR::VEC>(p.codes_k + row * KW, kw);
      knr = p.norms_k[row];
      vnr = p.norms_v[row];
    }
  };
  int64_t t0 = t_begin + (int64_t)wave * kTile;
  if (t0 < t_end) row_ahead = tile_row(t0);

  // ---- query tables
  float* qs = lds + L::oArea;             // [2][GC][kD]: q_rot, S q_rot (setup scratch)
  float* nibq = qs + 2 * GC * kD;         // [16 groups][2 halves][16][GC]
  const int srow = tid >> 2, sq4 = tid & 3;
  f32x4 sr[8];  // S_k[srow][32 sq4 .. 32 sq4 + 31]
  {
    const f32x4* src = reinterpret_cast<const f32x4*>(p.S_k + (int64_t)srow * kD + 32 * sq4);
#pragma unroll
    for (int c = 0; c < 8; ++c) sr[c] = src[c];
  }

  float* cents = qs + 2 * GC * kD + 16 * 2 * 16 * GC;  // [2][8] value codebooks
  if (tid == 0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      cents[k] = p.cent_v[0][k];
      cents[8 + k] = p.cent_v[1][k];
    }
  }
  if (wave < GC) {  // q_rot of head h0 + wave
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = lane + 64 * e;
      float x = load_elem(p.q, ((int64_t)b * p.hq + h0 + wave) * kD + j, p.q_dtype);
      const uint32_t sw = (lane & 32) ? uniform_u32(p.sign_k[2 * e + 1]) : uniform_u32(p.sign_k[2 * e]);
      if ((sw >> (j & 31)) & 1u) x = -x;
      v[e] = x;
    }
    fwht128(v, lane);
    const float isd = 1.0f / sqrtf((float)kD);
    qs[wave * kD + lane] = v[0] * isd;
    qs[wave * kD + lane + 64] = v[1] * isd;
  }
  // the first tile is requested only now: waits on the S and q loads above must not also
  // wait for it (vector-memory counters complete in issue order)
  fetch(t0);
  __syncthreads();
  {  // S q_rot: thread (row srow, quarter sq4) sums 32 columns, then the 4 quarter lanes
    float acc[GC];
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      float s = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f32x4 qv = *reinterpret_cast<const f32x4*>(qs + h * kD + 32 * sq4 + 4 * c);
        s = fmaf(sr[c][0], qv[0], s);
        s = fmaf(sr[c][1], qv[1], s);
        s = fmaf(sr[c][2], qv[2], s);
        s = fmaf(sr[c][3], qv[3], s);
      }
      s += xchg<1>(s);
      s += xchg<2>(s);
      acc[h] = s;
    }
    if (sq4 == 0) {
#pragma unroll
      for (int h = 0; h < GC; ++h) qs[(GC + h) * kD + srow] = acc[h];
    }
  }
  __syncthreads();
  if (wave < GC) {  // constants: codebook term (sum_k alpha_k) sum_j q_j per block; sum S q
    const int h = wave;
    float asum[2] = {0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      asum[0] += p.alpha_k[0][k];
      asum[1] += p.alpha_k[1][k];
    }
    const int blk0 = lane >> 5, blk1 = 2 + (lane >> 5);  // blocks of j = lane, lane + 64
    const float v = (blk0 < p.ksplitb ? asum[0] : asum[1]) * qs[h * kD + lane] +
                    (blk1 < p.ksplitb ? asum[0] : asum[1]) * qs[h * kD + lane + 64];
    const float cq = wave_sum_fast(v);
    const float ws = wave_sum_fast(qs[(GC + h) * kD + lane] + qs[(GC + h) * kD + lane + 64]);
    if (lane == 0) {
      cconst[h] = cq;
      cconst[GC + h] = ws;
    }
  }
  static_assert((16 * 2 * 16 * GC) % kThreads == 0 && (16 * 256) % kThreads == 0, "setup split");
  float nibsum_q[16 * 2 * 16 * GC / kThreads], nibsum_s[32 * 16 * GC / kThreads];
#pragma unroll
  for (int r = 0; r < 16 * 2 * 16 * GC / kThreads; ++r) {  // nibble sums of q_rot
    // (all reads of an entry before its write: the write may alias later reads for the
    // compiler, which would otherwise serialize every round trip)
    const int i = tid + r * kThreads;
    const int h = i % GC, n = (i / GC) % 16, half = (i / (16 * GC)) % 2, g = i / (32 * GC);
    const f32x4 x = *reinterpret_cast<const f32x4*>(qs + h * kD + 8 * g + 4 * half);
    nibsum_q[r] = ((n & 1) ? x[0] : 0.0f) + ((n & 2) ? x[1] : 0.0f) + ((n & 4) ? x[2] : 0.0f) +
                  ((n & 8) ? x[3] : 0.0f);
  }
#pragma unroll
  for (int r = 0; r < 32 * 16 * GC / kThreads; ++r) {  // Ts: 2 * nibble sums of S q_rot
    const int i = tid + r * kThreads;
    const int h = i % GC, n = (i / GC) % 16, g = i / (16 * GC);
    const f32x4 x = *reinterpret_cast<const f32x4*>(qs + (GC + h) * kD + 4 * g);
    nibsum_s[r] = 2.0f * (((n & 1) ? x[0] : 0.0f) + ((n & 2) ? x[1] : 0.0f) +
                          ((n & 4) ? x[2] : 0.0f) + ((n & 8) ? x[3] : 0.0f));
  }
#pragma unroll
  for (int r = 0; r < 16 * 2 * 16 * GC / kThreads; ++r) nibq[tid + r * kThreads] = nibsum_q[r];
#pragma unroll
  for (int r = 0; r < 32 * 16 * GC / kThreads; ++r) Ts[tid + r * kThreads] = nibsum_s[r];
  constexpr int kPat = kPairEntries * (VSPLIT < kNB ? 2 : 1);
  if (tid < kPat) {
    const bool hi = tid >= kPairEntries;
    const int x = tid & (kPairEntries - 1);
    const int mask = (1 << (hi ? BVHI : BVLO)) - 1;
    const int ia = ((x & 1) | ((x >> 1) & 2) | ((x >> 2) & 4)) & mask;         // bits 0, 2, 4
    const int ib = (((x >> 1) & 1) | ((x >> 2) & 2) | ((x >> 3) & 4)) & mask;  // bits 1, 3, 5
    uint32_t* dst = reinterpret_cast<uint32_t*>(hi ? cpHi : cpLo);
    const float c0 = cents[(hi ? 8 : 0) + ia] * kCentScale, c1 = cents[(hi ? 8 : 0) + ib] * kCentScale;
    const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
    const _Float16 l0 = (_Float16)(c0 - (float)h0), l1 = (_Float16)(c1 - (float)h1);
    dst[2 * x] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    dst[2 * x + 1] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
  }
  __syncthreads();
  float tq_v[16 * 256 / kThreads][GC];
#pragma unroll
  for (int r = 0; r < 16 * 256 / kThreads; ++r) {  // byte tables from nibble sums
    const int i = tid + r * kThreads;
    const int g = i >> 8, m = i & 255;
    float lo[GC], hi[GC];
    table_read<GC>(nibq + ((g * 2 + 0) * 16) * GC, m & 15, lo);
    table_read<GC>(nibq + ((g * 2 + 1) * 16) * GC, m >> 4, hi);
#pragma unroll
    for (int h = 0; h < GC; ++h) tq_v[r][h] = lo[h] + hi[h];
  }
#pragma unroll
  for (int r = 0; r < 16 * 256 / kThreads; ++r) {
    const int i = tid + r * kThreads;
    if constexpr (GC == 4) {
      *reinterpret_cast<f32x4*>(Tq + i * 4) = f32x4{tq_v[r][0], tq_v[r][1], tq_v[r][2], tq_v[r][3]};
    } else {
#pragma unroll
      for (int h = 0; h < GC; ++h) Tq[i * GC + h] = tq_v[r][h];
    }
  }
  __syncthreads();

  float cq[GC], wsum[GC];
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    cq[h] = cconst[h];
    wsum[h] = cconst[GC + h];
  }
  float alo[4], ahi[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    alo[k] = 2.0f * p.alpha_k[0][k];
    ahi[k] = 2.0f * p.alpha_k[1][k];
  }

  // ---- per-wave area: 64 value records + the weight rows.  Row bases are kept opaque to
  // the compiler so that row and field offsets fold into the LDS instructions' 16-bit
  // immediate instead of being re-added per access.
  int area_off = L::oArea + wave * L::kArea;
  asm volatile("" : "+v"(area_off));
  float* area = lds + area_off;
  _Float16* wts = reinterpret_cast<_Float16*>(area + kTile * kRS);
  for (int i = lane; i < L::kWRows * L::kWS / 2; i += 64) area[kTile * kRS + i] = 0.0f;
  // value lane mapping: lane (vq, vr) owns tokens 4 j + vq (j = 0..7) of each 32-token
  // group and reads block vr >> 2 of their records.  The weight rows hold token
  // 32 g + 4 j + q at position 32 g + 8 q + j, so a lane's 8 weights are contiguous, and
  // the 4 record rows one read touches are adjacent.
  // Codebook term: A rows are coordinate pairs and k = (token, coordinate of the pair,
  // fp16 hi or lo part), so two centroid-pair table entries (hi pair, lo pair) read back
  // to back are an operand as read.  Product i (one per code byte) gives row vr the pair
  // 32 (vr >> 2) + 8 i + 2 (vr & 3) + {0, 1}, and 8-token slab s gives lane group vq
  // tokens j = 2 s, 2 s + 1; output column vr = (c, head, hi/lo) with c = vr & 1 the
  // coordinate of the pair it sums, head (vr >> 1) & 3, lo weights if vr >= 8.
  // QJL term: A rows are coordinates 8 vr .. 8 vr + 7 (byte vr & 3 of the sign word, one
  // product per coordinate), k = the lane group's 8 tokens; column vr = weight column vr.
  const int vq = lane >> 4, vr = lane & 15;
  const int vblk = vr >> 2, vsh = 8 * (vr & 3);
  const bool vlo = vblk < VSPLIT;
  const int vnb = vlo ? BVLO : BVHI;
  const int voff = VR::off(vblk);
  const uint32_t cpoff = (uint32_t)((vlo ? L::oCpLo : L::oCpHi) * 4);
  const uint32_t pm0 = 0x03030303u << (2 * (vr & 3));              // plane-0 bits of the pairs
  const uint32_t pm1 = __builtin_amdgcn_alignbit(pm0, pm0, 30);    // rotated left by 2
  const uint32_t prs = 2 * (vr & 3) + 29;  // rotate right by 8 i + prs: pair field at bits 3-8
  const int vh = (vr >> 1) & 3;
  const int wrow_m = vh < GC ? (vr >> 3) * GC + vh : 16, wrow_s = vr < 8 ? 8 + vr : 16;
  const uint32_t psel0 = (vr & 1) ? 0x01000C0Cu : 0x0C0C0100u;  // weight in the half of
  const uint32_t psel1 = (vr & 1) ? 0x03020C0Cu : 0x0C0C0302u;  // this column's coordinate
  // the lane's record rows (float index; the token's row offset folds into the reads)
  int vrow = area_off + vq * kRS + voff;
  asm volatile("" : "+v"(vrow));

  float m_run[GC], l_run[GC];
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
  }
  // accm[i][j]: coordinate 32 vq + 8 i + 2 j + (vr & 1), column vr;
  // accq[e][j]: coordinate 8 (4 vq + j) + e, weight column vr
  f32x4 accm[4], accq[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) accq[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) accm[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  unsigned long long n_skipped = 0;
  const float kscale = p.scale * kLog2e;

  for (; t0 < t_end; t0 += (int64_t)kWaves * kTile) {
    const int64_t t = t0 + lane;
    const int64_t row0 = prow;
    const bool valid = t < t_end && row0 >= 0;
    uint32_t w[KW], vrec[VW];
#pragma unroll
    for (int i = 0; i < KW; ++i) w[i] = kw[i];
    // norms of absent tokens are zeroed so a stale value never meets a zero weight
    const uint32_t kn = valid ? knr : 0u, vn = valid ? vnr : 0u;
    fetch(t0 + kStride);
    // ---------------- keys: lane = token
    float mse[GC], qjl[GC];
#pragma unroll
    for (int h = 0; h < GC; ++h) mse[h] = qjl[h] = 0.0f;
#pragma unroll
    for (int blk = 0; blk < kNB; ++blk) {
      const uint32_t* wb = w + KR::off(blk);
      const int nb = blk < KSPLIT ? BKLO : BKHI;
      const float* al = blk < KSPLIT ? alo : ahi;
      lut_byte<GC>(Tq, 4 * blk, wb[0], al[0], mse);
      if (nb >= 2) lut_byte<GC>(Tq, 4 * blk, wb[1], al[1], mse);
      if (nb >= 3) {
        lut_byte<GC>(Tq, 4 * blk, wb[2], al[2], mse);
        lut_byte<GC>(Tq, 4 * blk, wb[0] ^ wb[1] ^ wb[2], al[3], mse);
      }
      lut_nib<GC>(Ts, 8 * blk, wb[nb], qjl);
    }
    const float n16 = f16_bits_to_f32(kn), r16 = f16_bits_to_f32(kn >> 16);
    float est[GC], lg[GC];
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      est[h] = n16 * (mse[h] - cq[h]) + p.gamma * r16 * (qjl[h] - wsum[h]);
      lg[h] = valid ? est[h] * kscale : -INFINITY;  // log2 domain
    }
    if (p.logits && valid) {
#pragma unroll
      for (int h = 0; h < GC; ++h)
        p.logits[((int64_t)b * p.hq + h0 + h) * p.capacity + t] = est[h] * p.scale;
    }
    // ---------------- online softmax (per head, wavefront reductions)
    const float vn16 = f16_bits_to_f32(vn), vr16 = f16_bits_to_f32(vn >> 16);
    // The running maximum moves only when some lane's logit exceeds it (a wave-uniform
    // test), so most tiles of a long split skip the max reduction and the rescale.
    // Ungated, l_run is a per-lane partial sum, reduced once after the scan; gated, the
    // test against tau needs the wave's running sum every tile.
    bool any_keep = false, grow = false;
    float u[GC], u2[GC], corr[GC];
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      corr[h] = 1.0f;
      if (__ballot(lg[h] > m_run[h]) != 0u) {
        const float mn = fmaxf(m_run[h], wave_max_fast(lg[h]));
        corr[h] = (m_run[h] == -INFINITY) ? 0.0f : exp2f(m_run[h] - mn);
        m_run[h] = mn;
        grow = true;
      }
      // hardware exp2: weights below 2^-126 of the running maximum flush to zero
      float wgt = valid ? __builtin_amdgcn_exp2f(lg[h] - m_run[h]) : 0.0f;
      if (gated) {
        l_run[h] = l_run[h] * corr[h] + wave_sum_fast(wgt);
        wgt = wgt < p.tau * l_run[h] ? 0.0f : wgt;
      } else {
        l_run[h] = l_run[h] * corr[h] + wgt;
      }
      any_keep |= wgt > 0.0f;
      u[h] = wgt * vn16;
      u2[h] = wgt * (p.gamma * kQjlScale) * vr16;
    }
    if (grow) {  // rescale the accumulators to the new running maxima
      float cm = corr[0], cs = corr[0];
#pragma unroll
      for (int h = 1; h < GC; ++h) {
        cm = (vh & (GC - 1)) == h ? corr[h] : cm;
        cs = (vr & (GC - 1)) == h ? corr[h] : cs;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) accm[i] *= cm;
      if constexpr (VQ) {
#pragma unroll
        for (int e = 0; e < 8; ++e) accq[e] *= cs;
      }
    }
    const uint64_t keep = __ballot(any_keep);
    n_skipped += (unsigned long long)__popcll(__ballot(valid) & ~keep);
    // this token's weight columns (fp16 hi, lo) and value record (read only for a token
    // some head keeps); a row not written keeps codes from an earlier tile (or LDS bits
    // never written, which still decode to finite table entries), met by zero weights
    {
      constexpr int kWS = L::kWS;
      _Float16* wl = wts + ((lane & 32) | ((lane & 3) << 3) | ((lane >> 2) & 7));
#pragma unroll
      for (int h = 0; h < GC; ++h) {
        const _Float16 uh = (_Float16)u[h];
        wl[h * kWS] = uh;
        wl[(GC + h) * kWS] = (_Float16)(u[h] - (float)uh);
        if constexpr (VQ) {
          const _Float16 sh = (_Float16)u2[h];
          wl[(8 + h) * kWS] = sh;
          wl[(8 + GC + h) * kWS] = (_Float16)(u2[h] - (float)sh);
        }
      }
      if (any_keep) {
        load_record<VW, VR::VEC>(p.codes_v + (row0 + lane) * VW, vrec);
        int own = area_off + lane * kRS;
        asm volatile("" : "+v"(own));
        uint32_t* rv = reinterpret_cast<uint32_t*>(lds + own);
#pragma unroll
        for (int i = 0; i < VW; ++i) rv[i] = vrec[i];
      }
    }
    // ---------------- values on MFMA, per 32-token group
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if ((uint32_t)(keep >> (32 * g)) == 0u) continue;  // no kept token in the group
      const int wb = 32 * g + 8 * vq;
      h16x8 bs{};
      if constexpr (VQ) bs = *reinterpret_cast<const h16x8*>(wts + wrow_s * L::kWS + wb);
      // codebook-term B operand of slab s: token j = 2 s, 2 s + 1's weight of column vr in
      // the half of this column's coordinate (0 in the other), once for the entry's hi
      // dword and once for its lo dword
      u32x4 bm[4];
      {
        const u32x4 w = *reinterpret_cast<const u32x4*>(wts + wrow_m * L::kWS + wb);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const uint32_t d0 = __builtin_amdgcn_perm(w[s2], w[s2], psel0);
          const uint32_t d1 = __builtin_amdgcn_perm(w[s2], w[s2], psel1);
          bm[s2] = u32x4{d0, d0, d1, d1};
        }
      }
      // per token: the code bits of the lane's 4 coordinate pairs, plane k rotated left
      // by 2 k, so the 6-bit table index of pair i sits at bits 8 i + 2 (vr & 3) .. + 5
      uint32_t pf[8], sb[8];
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const uint32_t* rw = reinterpret_cast<const uint32_t*>(lds + vrow + (32 * g + 4 * tt) * kRS);
        uint32_t p0, p1 = 0, p2 = 0, sg = 0;
        if constexpr (VQ && BVLO == 3 && BVHI == 3) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(rw);
          p0 = x[0]; p1 = x[1]; p2 = x[2]; sg = x[3];
        } else {
          p0 = rw[0];
          if constexpr (BVLO >= 2 || BVHI >= 2) p1 = vnb >= 2 ? rw[1] : 0u;
          if constexpr (BVLO == 3 || BVHI == 3) p2 = vnb == 3 ? rw[2] : 0u;
          if constexpr (VQ) sg = rw[vnb];
        }
        uint32_t t = 0;
        if constexpr (BVLO >= 2 || BVHI >= 2) {
          const uint32_t r1 = __builtin_amdgcn_alignbit(p1, p1, 30);
          t = r1;
          if constexpr (BVLO == 3 || BVHI == 3) {
            const uint32_t r2 = __builtin_amdgcn_alignbit(p2, p2, 28);
            t = r2 ^ ((r1 ^ r2) & pm1);
          }
        }
        pf[tt] = t ^ ((p0 ^ t) & pm0);
        sb[tt] = VQ ? __builtin_amdgcn_ubfe(sg, vsh, 8) : 0u;
      }
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t x0 = pf[2 * s2], x1 = pf[2 * s2 + 1];
          const uint32_t a0 = (__builtin_amdgcn_alignbit(x0, x0, prs + 8 * i) & 0x1F8u) | cpoff;
          const uint32_t a1 = (__builtin_amdgcn_alignbit(x1, x1, prs + 8 * i) & 0x1F8u) | cpoff;
          const u32x2 e0 = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(lds) + a0);
          const u32x2 e1 = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(lds) + a1);
          const u32x4 a = u32x4{e0[0], e0[1], e1[0], e1[1]};
          accm[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h16x8, a), __builtin_bit_cast(h16x8, bm[s2]), accm[i], 0, 0, 0);
        }
      }
      if constexpr (VQ) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          u32x4 so;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t x = sb[2 * j] | (sb[2 * j + 1] << 16);
            so[j] = ((x << (15 - e)) & 0x80008000u) ^ 0xBC00BC00u;  // bit 1 -> +1, 0 -> -1
          }
          accq[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h16x8, so), bs, accq[e], 0, 0, 0);
        }
      }
    }
  }
  // ---------------- workgroup epilogue: the lo-weight columns are folded into the hi
  // ones, then the waves' partials are merged in LDS (aliases Tq) and stored at device scope
  if (!gated) {
#pragma unroll
    for (int h = 0; h < GC; ++h) l_run[h] = wave_sum_fast(l_run[h]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) accm[i][j] += xchg<8>(accm[i][j]);
  if constexpr (VQ) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) accq[e][j] += xchg<GC>(accq[e][j]);
  }
  __syncthreads();
  float* mine = lds + L::oWM + wave * L::kMerge;  // [2*GC] m, l | [GC][2][kD]
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      mine[h] = m_run[h];
      mine[GC + h] = l_run[h];
    }
  }
  if (vr < 8 && vh < GC) {
    float* a = mine + round4(2 * GC) + vh * 2 * kD + 32 * vq + (vr & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) a[8 * i + 2 * j] = accm[i][j] * (1.0f / kCentScale);
  }
  if (vr < GC) {
    float* a = mine + round4(2 * GC) + vr * 2 * kD + kD;
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) a[8 * (4 * vq + j) + e] = VQ ? accq[e][j] * (1.0f / kQjlScale) : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < (GC * 2 * kD + kThreads - 1) / kThreads; ++r) {
    const int i = tid + r * kThreads;
    if (i >= GC * 2 * kD) break;
    const int h = i / (2 * kD), k = i % (2 * kD);
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) M = fmaxf(M, lds[L::oWM + w2 * L::kMerge + h]);
    float acc = 0.0f, lsum = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) {
        const float* o = lds + L::oWM + w2 * L::kMerge;
        if (o[h] == -INFINITY) continue;
        const float sc = exp2f(o[h] - M);
        acc = fmaf(o[round4(2 * GC) + h * 2 * kD + k], sc, acc);
        lsum = fmaf(o[GC + h], sc, lsum);
      }
    }
    float* part = p.ws_part + (((int64_t)b * p.hq + h0 + h) * p.n_split + p.split_base + split) * kPartFloats;
    part[2 + k] = acc;
    if (k == 0) {
      part[0] = M;
      part[1] = lsum;
    }
  }
  if (p.skipped) {
    const unsigned long long tot = n_skipped;  // wave-uniform
    if (lane == 0 && tot) atomicAdd(p.skipped, tot);
  }
}

template <int BKLO, int BKHI, int KSPLIT, int BVLO, int BVHI, int VSPLIT, bool VQ, int GC>
__global__ __launch_bounds__(kThreads) void decode_scan(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float lds[scan_lds_floats<BVLO, BVHI, VSPLIT, VQ, GC>()];
  scan_body<BKLO, BKHI, KSPLIT, BVLO, BVHI, VSPLIT, VQ, GC>(p, lds, blockIdx.x);
}

// Two cache segments of different format pairs in one launch (decode over a decayed cache):
// workgroups x < n0 scan segment 0 (format pair A, params p0), the others segment 1 (pair
// B, params p1, split x - n0); p1.split_base = n0 puts both segments' partials side by side
// for one combine.
template <int A0, int A1, int A2, int A3, int A4, int A5, int B0, int B1, int B2, int B3, int B4,
          int B5, int GC>
__global__ __launch_bounds__(kThreads) void decode_scan_pair(DecodeParams p0, DecodeParams p1, int n0) {
  constexpr int kA = scan_lds_floats<A3, A4, A5, true, GC>();
  constexpr int kB = scan_lds_floats<B3, B4, B5, true, GC>();
  __shared__ __attribute__((aligned(16))) float lds[kA > kB ? kA : kB];
  if ((int)blockIdx.x < n0)
    scan_body<A0, A1, A2, A3, A4, A5, true, GC>(p0, lds, blockIdx.x);
  else
    scan_body<B0, B1, B2, B3, B4, B5, true, GC>(p1, lds, blockIdx.x - n0);
}

template <int BKLO, int BKHI, int KS, int BVLO, int BVHI, int VS, bool VQ, int GC>
static int launch_scan(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_scan<BKLO, BKHI, KS, BVLO, BVHI, VS, VQ, GC>), grid, dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

// Launches the scan of one (key format, value format) pair, split given in blocks of 32
// (4 = one width); instantiated in the tq_decode_*.hip translation units.
template <int BKLO, int BKHI, int KS, int BVLO, int BVHI, int VS>
int launch_pair(const DecodeParams& p, bool vq, int gc, dim3 grid, hipStream_t s) {
  if (gc == 4) return vq ? launch_scan<BKLO, BKHI, KS, BVLO, BVHI, VS, true, 4>(p, grid, s)
                         : launch_scan<BKLO, BKHI, KS, BVLO, BVHI, VS, false, 4>(p, grid, s);
  if (gc == 2) return vq ? launch_scan<BKLO, BKHI, KS, BVLO, BVHI, VS, true, 2>(p, grid, s)
                         : launch_scan<BKLO, BKHI, KS, BVLO, BVHI, VS, false, 2>(p, grid, s);
  return vq ? launch_scan<BKLO, BKHI, KS, BVLO, BVHI, VS, true, 1>(p, grid, s)
            : launch_scan<BKLO, BKHI, KS, BVLO, BVHI, VS, false, 1>(p, grid, s);
}

// Supported (key format, value format) pairs as (key bits below / above the split, key split
// in blocks, value bits below / above, value split).  Values may be stored with or without
// QJL sign words; keys carry them.
#define TQ_DECODE_PAIRS(X) \
  X(3, 3, 4, 3, 3, 4) /* K / V: b4 / b4 */ \
  X(3, 3, 4, 2, 2, 4) /* K / V: b4 / b3 */ \
  X(2, 2, 4, 2, 2, 4) /* K / V: b3 / b3 */ \
  X(1, 1, 4, 1, 1, 4) /* K / V: b2 / b2 */ \
  X(2, 2, 4, 1, 1, 4) /* K / V: b3 / b2 */ \
  X(3, 2, 1, 3, 2, 1) /* K / V: 3+2 bits split at 32 (3.25 bit) */ \
  X(3, 2, 2, 3, 2, 2) /* K / V: 3+2 bits split at 64 (3.5 bit) */ \
  X(2, 1, 1, 2, 1, 1) /* K / V: 2+1 bits split at 32 (2.25 bit) */ \
  X(2, 1, 2, 2, 1, 2) /* K / V: 2+1 bits split at 64 (2.5 bit) */ \
  X(2, 1, 3, 2, 1, 3) /* K / V: 2+1 bits split at 96 (2.75 bit) */ \
  X(3, 3, 4, 2, 1, 2) /* K / V: b4 / b2.5 */ \
  X(3, 2, 2, 2, 1, 2) /* K / V: b3.5 / b2.5 */ \
  X(3, 2, 2, 2, 2, 4) /* K / V: b3.5 / b3 */ \
  /* end */

// decode_combine over `rows` (batch * hq) partial sets (defined with the kernel in
// tq_decode.hip).
int launch_decode_combine(const DecodeParams& p, int rows, hipStream_t stream);

#define TQ_DECODE_EXTERN(a, b, c, d, e, f) \
  extern template int launch_pair<a, b, c, d, e, f>(const DecodeParams&, bool, int, dim3, hipStream_t);
TQ_DECODE_PAIRS(TQ_DECODE_EXTERN)
#undef TQ_DECODE_EXTERN

// Format-pair combinations (old segment, new segment) that decode over a decayed cache in
// one launch (values with QJL, query-head groups of a multiple of 4): b3 / b3 tokens
// before b4 / b4 ones, and 2.5-bit before 3.5-bit.
#define TQ_DECAY_PAIRS(X) \
  X(2, 2, 4, 2, 2, 4, 3, 3, 4, 3, 3, 4) \
  X(2, 1, 2, 2, 1, 2, 3, 2, 2, 3, 2, 2)

// Launch of the fused two-segment scan for combination A -> B (tq_decode_decay.hip).
template <int A0, int A1, int A2, int A3, int A4, int A5, int B0, int B1, int B2, int B3, int B4,
          int B5>
int launch_scan_pair(const DecodeParams& p0, const DecodeParams& p1, int n0, dim3 grid,
                     hipStream_t s);

}  // namespace tqk
