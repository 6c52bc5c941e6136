// Decode attention straight from the packed cache (163.com explainer,
// m.163.com/dy/article/KOV7P8JI0556C3J2, sections "第二步：QJL" and "速度"):
//   logit_t = scale * ( n16_t <q_rot, c[idx_t]> + gamma r16_t <S q_rot, 2 sigma_t - 1> ),
//   q_rot = H D q / sqrt(d), gamma = sqrt(pi/2) / d;
//   softmax over t < seq_len; out = Pi^T ( sum_t p_t (n16 c[idx] + gamma r16 S^T sigma) ).
// Because <q, Pi^T v> = <Pi q, v> and <q_rot, S^T s> = <S q_rot, s>, the cache is never
// rotated back per token: values are accumulated in the rotated domain and each head's
// result is mapped back once (S^T, then D H / sqrt(d)).
//
// Three launches:
//   prologue: per (batch, KV head, chunk of GC query heads) one workgroup: q_rot and
//             S q_rot of the GC heads, and their nibble subset-sum tables (sums of w over
//             the set bits of a 4-bit index, for every 4-coordinate group).
//   scan:     grid (split, batch * KV head * chunk), about one workgroup per CU.  The
//             workgroup expands the nibble tables into byte-indexed tables in LDS,
//             T[g][m] = sum of w_{8g+i} over the set bits i of m (one float per head), so
//             a sign dot product <w, 2b - 1> over 128 coordinates is 16 table reads: the
//             QJL term directly, and the codebook term through the Walsh expansion of the
//             symmetric codebook, c[idx] = sum_S alpha_S prod_{k in S} (2 b_k - 1) over odd
//             subsets S of the code bit-planes (the planes, and for 3 bits their XOR).
//             Keys: lane = token; records of the next 64-token tile are prefetched into
//             registers.  Online softmax per head with wavefront reductions; the Sparse-V
//             gate (zhidx turboquant_plus article, section "01 turboquant_plus：介绍与详解")
//             drops a value row for a head when its running weight estimate is below tau,
//             and skips reading rows dropped by every head.  Values: lane = coordinate
//             pair, fp32 accumulation of w n16 c[idx] and w gamma r16 sigma per head.  The
//             waves' partial (m, l, acc) are merged in LDS: one partial per workgroup.
//   combine:  per (batch, query head) one workgroup merges the splits in a fixed order and
//             maps back: out = D H (A + S^T Q) / (sqrt(d) l).
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

constexpr int kD = 128;
constexpr int kNB = kD / 32;
constexpr int kScanWaves = 4;
constexpr int kTile = 64;
constexpr int kPartFloats = 2 + 2 * kD;  // m (log2 domain), l, A[d], Q[d]
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kNibFloats = 2 * 16 * 2 * 16;  // per head: [vec][group][half][nibble]
// per-unit stride of the nibble tables + 2 constants per head, kept a multiple of 16 bytes
__host__ __device__ constexpr int nib_stride(int gc) { return ((kNibFloats + 2) * gc + 3) / 4 * 4; }

template <int B>
struct Walsh {  // number of odd plane subsets of a B-bit code: the Walsh planes used
  static constexpr int N = (B == 3) ? 4 : B;
};

// Record layout of a format with SPLITB blocks of BLO bits then blocks of BHI bits.
template <int BLO, int BHI, int SPLITB>
struct Rec {
  static constexpr int W = SPLITB * (BLO + 1) + (kNB - SPLITB) * (BHI + 1);  // words
  static constexpr int VEC = (W % 4 == 0) ? 4 : ((W % 2 == 0) ? 2 : 1);      // load width
  static constexpr int bits(int blk) { return blk < SPLITB ? BLO : BHI; }
  static constexpr int off(int blk) {
    return blk < SPLITB ? blk * (BLO + 1) : SPLITB * (BLO + 1) + (blk - SPLITB) * (BHI + 1);
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
  float* ws_qrot;   // [batch*hq][2][d]: q_rot, S_k q_rot
  float* ws_nib;    // [units][kNibFloats][GC] + [units][2][GC] constants
  float* ws_part;   // [batch*hq][n_split][kPartFloats]
  int64_t capacity;
  int64_t tokens_per_split;
  int32_t batch, hq, hkv, group, gc, q_dtype, n_split;
  float scale, tau, gamma;
  uint32_t sign_k[4], sign_v[4];
  float alpha_k[2][4];  // Walsh coefficients of the key codebooks (lo, hi parts)
  float cent_v[2][8];   // value codebooks (lo, hi)
  int32_t ksplitb;
};

// ----------------------------------------------------------------------------- prologue
// One workgroup of 128 threads per (batch, query head): q_rot = H D q / sqrt(d),
// S q_rot, this head's slice of the nibble subset-sum tables of its chunk, and the two
// constants of <w, 2b - 1> = 2 <w, b> - sum(w).
template <int GC>
__global__ __launch_bounds__(128) void decode_prologue(DecodeParams p) {
  const int bh = blockIdx.x;               // b * hq + h
  const int b = bh / p.hq, h = bh % p.hq;
  const int bk = b * p.hkv + h / p.group;  // kv unit
  const int hin = h % p.group;
  const int unit = bk * (p.group / GC) + hin / GC;
  const int hh = hin % GC;                 // head slot inside the chunk
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  __shared__ float wv[2][kD];
  __shared__ float red[4];
  if (wave == 0) {
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = lane + 64 * e;
      float x = load_elem(p.q, (int64_t)bh * kD + j, p.q_dtype);
      if ((p.sign_k[j >> 5] >> (j & 31)) & 1u) x = -x;
      v[e] = x;
    }
    {
      const float a = v[0], c = v[1];
      v[0] = a + c;
      v[1] = a - c;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float t = __shfl_xor(v[e], m, 64);
        v[e] = (lane & m) ? t - v[e] : v[e] + t;
      }
    const float isd = 1.0f / sqrtf((float)kD);
    wv[0][lane] = v[0] * isd;
    wv[0][lane + 64] = v[1] * isd;
  }
  __syncthreads();
  // S q_rot: thread t computes row t (16-byte reads of the row)
  {
    const f32x4* row = reinterpret_cast<const f32x4*>(p.S_k + (int64_t)tid * kD);
    float s = 0.0f;
#pragma unroll 8
    for (int k = 0; k < kD / 4; ++k) {
      const f32x4 a = row[k];
      s = fmaf(a[0], wv[0][4 * k], s);
      s = fmaf(a[1], wv[0][4 * k + 1], s);
      s = fmaf(a[2], wv[0][4 * k + 2], s);
      s = fmaf(a[3], wv[0][4 * k + 3], s);
    }
    wv[1][tid] = s;
    float* dst = p.ws_qrot + (int64_t)bh * 2 * kD;
    dst[tid] = wv[0][tid];
    dst[kD + tid] = s;
  }
  __syncthreads();
  // nibble subset sums [vec][group][half][nibble][GC], this head's slot
  float* nib = p.ws_nib + (int64_t)unit * nib_stride(GC);
  for (int i = tid; i < kNibFloats; i += 128) {
    const int n = i % 16, half = (i / 16) % 2, g = (i / 32) % 16, vv = i / 512;
    float sum = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if ((n >> k) & 1) sum += wv[vv][8 * g + 4 * half + k];
    nib[i * GC + hh] = sum;
  }
  // constants: codebook term sum_blk (sum_k alpha_k) W_blk, QJL term sum(S q_rot)
  {
    const int blk = tid >> 5;  // 4 blocks of 32 coordinates over the 128 threads
    const float wb = half_sum(wv[0][tid]);
    const bool lo = blk < p.ksplitb;
    float asum = 0.0f;
    for (int k = 0; k < 4; ++k) asum += p.alpha_k[lo ? 0 : 1][k];
    const float ss = half_sum(wv[1][tid]);
    __shared__ float sred[4];
    if ((tid & 31) == 0) {
      red[blk] = asum * wb;
      sred[blk] = ss;
    }
    __syncthreads();
    if (tid == 0) {
      nib[kNibFloats * GC + hh] = ((red[0] + red[1]) + red[2]) + red[3];
      nib[kNibFloats * GC + GC + hh] = ((sred[0] + sred[1]) + sred[2]) + sred[3];
    }
  }
}

// ----------------------------------------------------------------------------- scan
template <int GC, int VW>
struct ScanLds {
  static constexpr int kTable = 2 * 16 * 256 * GC;     // [vec][16 groups][256][GC]
  static constexpr int kWave = (kTile + 1) * 2 * GC + (kTile + 1) * VW + 4;  // weights + V staging
  static constexpr int kPartW = 2 * GC + 2 * kD * GC;  // merged partial of one wave
  static constexpr int kArea = (kWave > kPartW ? kWave : kPartW);
  static constexpr int kTotal = kTable + kScanWaves * kArea;
  static_assert(kScanWaves * kArea >= kNibFloats * GC, "nibble tables alias the wave areas");
};

template <int GC>
__device__ __forceinline__ void table_read(const float* T, int idx, float (&out)[GC]) {
  if constexpr (GC == 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(T + 4 * idx);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  } else if constexpr (GC == 2) {
    const f32x2 v = *reinterpret_cast<const f32x2*>(T + 2 * idx);
    out[0] = v[0]; out[1] = v[1];
  } else {
    out[0] = T[idx];
  }
}

// Add alpha times the byte-table reads of one 32-bit sign word (groups g0 .. g0+3).
template <int GC>
__device__ __forceinline__ void lut_word(const float* T, int g0, uint32_t w, float alpha,
                                         float (&acc)[GC]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float t[GC];
    table_read<GC>(T, (g0 + i) * 256 + ((w >> (8 * i)) & 0xFFu), t);
#pragma unroll
    for (int h = 0; h < GC; ++h) acc[h] = fmaf(alpha, t[h], acc[h]);
  }
}

template <int B, int GC>
__device__ __forceinline__ void key_block(const float* Tq, int blk, const uint32_t* w,
                                          const float* alpha, float (&acc)[GC]) {
  lut_word<GC>(Tq, 4 * blk, w[0], alpha[0], acc);
  if constexpr (B >= 2) lut_word<GC>(Tq, 4 * blk, w[1], alpha[1], acc);
  if constexpr (B >= 3) {
    lut_word<GC>(Tq, 4 * blk, w[2], alpha[2], acc);
    lut_word<GC>(Tq, 4 * blk, w[0] ^ w[1] ^ w[2], alpha[3], acc);
  }
}

template <int BKLO, int BKHI, int KSPLIT, int BVLO, int BVHI, int VSPLIT, int GC>
__global__ __launch_bounds__(64 * kScanWaves) void decode_scan(DecodeParams p) {
  using KR = Rec<BKLO, BKHI, KSPLIT>;
  using VR = Rec<BVLO, BVHI, VSPLIT>;
  constexpr int KW = KR::W, VW = VR::W;
  using L = ScanLds<GC, VW>;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  float* Tq = lds;                         // [16][256][GC]
  float* Ts = lds + 16 * 256 * GC;         // [16][256][GC]
  float* nib = lds + L::kTable;            // aliases the wave areas during setup
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  float* area = lds + L::kTable + wave * L::kArea;
  float* wts = area;                                                        // [65][2*GC]
  uint32_t* vst = reinterpret_cast<uint32_t*>(area + (kTile + 1) * 2 * GC);  // [65][VW] + 4
  __shared__ float centv[16];
  __shared__ __attribute__((aligned(16))) float cpair_s[2][128];  // [part][6-bit pair index][2]
  __shared__ f32x2 spair[4];
  __shared__ float cconst[2][GC];

  const int nchunk = p.group / GC;
  const int unit = blockIdx.y;
  const int chunk = unit % nchunk;
  const int bk = unit / nchunk;  // b * hkv + kv head
  const int b = bk / p.hkv;
  const int h0 = (bk % p.hkv) * p.group + chunk * GC;
  const int64_t seq = p.seq_lens[b];
  const int64_t t_begin = (int64_t)blockIdx.x * p.tokens_per_split;
  int64_t t_end = t_begin + p.tokens_per_split;
  if (t_end > seq) t_end = seq;

  // ---- tables: nibble sums -> LDS -> byte tables
  {
    const float* src = p.ws_nib + (int64_t)unit * nib_stride(GC);
    for (int i = threadIdx.x; i < kNibFloats * GC / 4; i += blockDim.x)
      reinterpret_cast<f32x4*>(nib)[i] = reinterpret_cast<const f32x4*>(src)[i];
    if (threadIdx.x < 2 * GC) (&cconst[0][0])[threadIdx.x] = src[kNibFloats * GC + threadIdx.x];
    if (threadIdx.x < 16) centv[threadIdx.x] = (&p.cent_v[0][0])[threadIdx.x];
    if (threadIdx.x < 128) {
      // pair index f = (plane-0 bits, plane-1 bits, plane-2 bits) of two coordinates
      const int part = threadIdx.x >> 6, f = threadIdx.x & 63;
      const int nb = part == 0 ? BVLO : BVHI;
      const int mask = (1 << nb) - 1;
      const int i0 = ((f & 1) | (((f >> 2) & 1) << 1) | (((f >> 4) & 1) << 2)) & mask;
      const int i1 = (((f >> 1) & 1) | (((f >> 3) & 1) << 1) | (((f >> 5) & 1) << 2)) & mask;
      cpair_s[part][2 * f] = p.cent_v[part][i0];
      cpair_s[part][2 * f + 1] = p.cent_v[part][i1];
    }
    if (threadIdx.x < 4) {
      const f32x2 v = {(threadIdx.x & 1) ? 1.0f : -1.0f, (threadIdx.x & 2) ? 1.0f : -1.0f};
      spair[threadIdx.x] = v;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * 16 * 16; i += blockDim.x) {
    // thread: (vec, group, low nibble); loops over the high nibble
    const int lo = i % 16, g = (i / 16) % 16, vv = i / 256;
    float a[GC];
    const float* nl = nib + (((vv * 16 + g) * 2 + 0) * 16 + lo) * GC;
#pragma unroll
    for (int h = 0; h < GC; ++h) a[h] = nl[h];
    float* dst = (vv == 0 ? Tq : Ts) + (g * 256 + lo) * GC;
    const float* nh = nib + (((vv * 16 + g) * 2 + 1) * 16) * GC;
#pragma unroll 4
    for (int hi = 0; hi < 16; ++hi) {
      float hv[GC];
      table_read<GC>(nh, hi, hv);
      if constexpr (GC == 4) {
        f32x4 o = {a[0] + hv[0], a[1] + hv[1], a[2] + hv[2], a[3] + hv[3]};
        *reinterpret_cast<f32x4*>(dst + hi * 16 * GC) = o;
      } else {
#pragma unroll
        for (int h = 0; h < GC; ++h) dst[hi * 16 * GC + h] = a[h] + hv[h];
      }
    }
  }
  __syncthreads();

  float cq[GC], ws[GC];
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    cq[h] = cconst[0][h];
    ws[h] = cconst[1][h];
  }
  float alo[4], ahi[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    alo[k] = 2.0f * p.alpha_k[0][k];
    ahi[k] = 2.0f * p.alpha_k[1][k];
  }

  // value lane mapping: lane -> coordinates j0 = 32 (lane / 16) + 2 (lane % 16), j0 + 1
  const int vblk = lane >> 4, vbit = 2 * (lane & 15);
  const bool vlo = vblk < VSPLIT;
  const int vnb = vlo ? BVLO : BVHI;
  const int voff = vlo ? vblk * (BVLO + 1) : VSPLIT * (BVLO + 1) + (vblk - VSPLIT) * (BVHI + 1);
  const float* cpair = cpair_s[vlo ? 0 : 1];
  // the zero row used to pad the 4-token value steps
  for (int i = lane; i < 2 * GC; i += 64) wts[kTile * 2 * GC + i] = 0.0f;
  for (int i = lane; i < VW + 4; i += 64) vst[kTile * VW + i] = 0u;

  float m_run[GC], l_run[GC], am[GC][2], aq[GC][2];
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
    am[h][0] = am[h][1] = aq[h][0] = aq[h][1] = 0.0f;
  }
  unsigned long long n_skipped = 0;
  const int64_t kv_base = (int64_t)bk * p.capacity;
  const float kscale = p.scale * kLog2e;

  // register prefetch of one tile: key record, value record, both norms
  uint32_t kw[KW], vwr[VW], knr = 0, vnr = 0;
  int64_t t0 = t_begin + (int64_t)wave * kTile;
  // with the Sparse-V gate on, value records are read only for rows that survive it
  const bool gated = p.tau > 0.0f;
  auto fetch = [&](int64_t tt0) {
    const int64_t t = tt0 + lane;
    if (tt0 < t_end && t < t_end) {
      load_record<KW, KR::VEC>(p.codes_k + (kv_base + t) * KW, kw);
      if (!gated) load_record<VW, VR::VEC>(p.codes_v + (kv_base + t) * VW, vwr);
      knr = p.norms_k[kv_base + t];
      vnr = p.norms_v[kv_base + t];
    }
  };
  fetch(t0);

  for (; t0 < t_end; t0 += (int64_t)kScanWaves * kTile) {
    const int64_t t = t0 + lane;
    const bool valid = t < t_end;
    uint32_t w[KW], vrec[VW];
#pragma unroll
    for (int i = 0; i < KW; ++i) w[i] = kw[i];
#pragma unroll
    for (int i = 0; i < VW; ++i) vrec[i] = vwr[i];
    const uint32_t kn = knr, vn = vnr;
    fetch(t0 + (int64_t)kScanWaves * kTile);
    // ---------------- keys: lane = token
    float mse[GC], qjl[GC];
#pragma unroll
    for (int h = 0; h < GC; ++h) mse[h] = qjl[h] = 0.0f;
#pragma unroll
    for (int blk = 0; blk < kNB; ++blk) {
      if (blk < KSPLIT) {
        key_block<BKLO, GC>(Tq, blk, w + KR::off(blk), alo, mse);
        lut_word<GC>(Ts, 4 * blk, w[KR::off(blk) + BKLO], 2.0f, qjl);
      } else {
        key_block<BKHI, GC>(Tq, blk, w + KR::off(blk), ahi, mse);
        lut_word<GC>(Ts, 4 * blk, w[KR::off(blk) + BKHI], 2.0f, qjl);
      }
    }
    const float n16 = f16_bits_to_f32(kn), r16 = f16_bits_to_f32(kn >> 16);
    float lg[GC];
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      const float est = n16 * (mse[h] - cq[h]) + p.gamma * r16 * (qjl[h] - ws[h]);
      lg[h] = valid ? est * kscale : -INFINITY;  // log2 domain
      if (p.logits && valid)
        p.logits[((int64_t)b * p.hq + h0 + h) * p.capacity + t] = est * p.scale;
    }
    // ---------------- online softmax (per head, wavefront reductions)
    const float vn16 = f16_bits_to_f32(vn), vr16 = f16_bits_to_f32(vn >> 16);
    bool any_keep = false;
    float* wrow = wts + lane * 2 * GC;
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      const float mt = wave_max_fast(lg[h]);
      const float mn = fmaxf(m_run[h], mt);
      const float corr = (m_run[h] == -INFINITY) ? 0.0f : exp2f(m_run[h] - mn);
      float wgt = valid ? exp2f(lg[h] - mn) : 0.0f;
      l_run[h] = l_run[h] * corr + wave_sum_fast(wgt);
      m_run[h] = mn;
      if (p.tau > 0.0f && wgt < p.tau * l_run[h]) wgt = 0.0f;
      any_keep |= wgt > 0.0f;
      am[h][0] *= corr;
      am[h][1] *= corr;
      aq[h][0] *= corr;
      aq[h][1] *= corr;
      wrow[h] = wgt * vn16;
      wrow[GC + h] = wgt * p.gamma * vr16;
    }
    uint64_t keep = __ballot(any_keep);
    n_skipped += (unsigned long long)__popcll(__ballot(valid) & ~keep);
    // value rows of kept tokens to LDS
    if (any_keep) {
      if (gated) load_record<VW, VR::VEC>(p.codes_v + (kv_base + t) * VW, vrec);
#pragma unroll
      for (int i = 0; i < VW; ++i) vst[lane * VW + i] = vrec[i];
    }
    // ---------------- values: lane = coordinate pair, loop over kept tokens, 4 at a time
    // (missing slots point at the all-zero row kTile)
    while (keep) {
      int tl[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        tl[u] = keep ? __builtin_ctzll(keep) : kTile;
        keep &= keep - 1;
      }
      float c0[4], c1[4], s0[4], s1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t* vw = vst + tl[u] * VW + voff;
        const uint32_t w0 = vw[0], w1 = vw[1], w2 = vw[2], w3 = vw[3];
        const uint32_t p2 = (vnb == 3) ? w2 : 0u;
        const uint32_t sg = (vnb == 3) ? w3 : ((vnb == 2) ? w2 : w1);
        const uint32_t p1 = (vnb >= 2) ? w1 : 0u;
        const uint32_t f = ((w0 >> vbit) & 3u) | (((p1 >> vbit) & 3u) << 2) | (((p2 >> vbit) & 3u) << 4);
        const f32x2 cc = *reinterpret_cast<const f32x2*>(cpair + 2 * f);
        const f32x2 ss = spair[(sg >> vbit) & 3u];
        c0[u] = cc[0]; c1[u] = cc[1]; s0[u] = ss[0]; s1[u] = ss[1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* wr = wts + tl[u] * 2 * GC;
        float uu[GC], uq[GC];
        table_read<GC>(wr, 0, uu);
        table_read<GC>(wr + GC, 0, uq);
#pragma unroll
        for (int h = 0; h < GC; ++h) {
          am[h][0] = fmaf(uu[h], c0[u], am[h][0]);
          am[h][1] = fmaf(uu[h], c1[u], am[h][1]);
          aq[h][0] = fmaf(uq[h], s0[u], aq[h][0]);
          aq[h][1] = fmaf(uq[h], s1[u], aq[h][1]);
        }
      }
    }
  }
  // ---------------- merge the waves' partials in LDS, one partial per workgroup
  __syncthreads();
  float* mine = lds + L::kTable + wave * L::kArea;  // [2*GC] m, l then [GC][2][kD]
  const int j0 = 32 * vblk + vbit;
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      mine[h] = m_run[h];
      mine[GC + h] = l_run[h];
    }
  }
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    float* a = mine + 2 * GC + h * 2 * kD;
    a[j0] = am[h][0];
    a[j0 + 1] = am[h][1];
    a[kD + j0] = aq[h][0];
    a[kD + j0 + 1] = aq[h][1];
  }
  __syncthreads();
  // thread t: head h = t / 64 (when GC >= ...), coordinates handled in a loop
  for (int i = threadIdx.x; i < GC * 2 * kD; i += blockDim.x) {
    const int h = i / (2 * kD), k = i % (2 * kD);
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < kScanWaves; ++w2) M = fmaxf(M, lds[L::kTable + w2 * L::kArea + h]);
    float acc = 0.0f, lsum = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w2 = 0; w2 < kScanWaves; ++w2) {
        const float* o = lds + L::kTable + w2 * L::kArea;
        if (o[h] == -INFINITY) continue;
        const float sc = exp2f(o[h] - M);
        acc = fmaf(o[2 * GC + h * 2 * kD + k], sc, acc);
        lsum = fmaf(o[GC + h], sc, lsum);
      }
    }
    float* part = p.ws_part + (((int64_t)b * p.hq + h0 + h) * p.n_split + blockIdx.x) * kPartFloats;
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

// ----------------------------------------------------------------------------- combine
__global__ __launch_bounds__(256) void decode_combine(DecodeParams p) {
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ float scl[1024];
  __shared__ float red[256];
  __shared__ float vec[2][kD];
  __shared__ float Lsh;
  const float* parts = p.ws_part + (int64_t)bh * p.n_split * kPartFloats;
  const int np = p.n_split;
  // global max over splits
  float M = -INFINITY;
  for (int i = tid; i < np; i += 256) M = fmaxf(M, parts[(int64_t)i * kPartFloats]);
  red[tid] = M;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
    __syncthreads();
  }
  M = red[0];
  __syncthreads();
  for (int i = tid; i < np; i += 256) {
    const float m = parts[(int64_t)i * kPartFloats];
    scl[i] = (m == -INFINITY || M == -INFINITY) ? 0.0f : exp2f(m - M);
  }
  __syncthreads();
  // thread t: component t / 128 (A or Q), coordinate t % 128; fixed order over splits
  {
    const int k = tid;  // 0 .. 255 = [A | Q]
    float acc = 0.0f;
    for (int i = 0; i < np; ++i) acc = fmaf(parts[(int64_t)i * kPartFloats + 2 + k], scl[i], acc);
    vec[k >> 7][k & 127] = acc;
    if (tid == 0) {
      float L = 0.0f;
      for (int i = 0; i < np; ++i) L = fmaf(parts[(int64_t)i * kPartFloats + 1], scl[i], L);
      Lsh = L;
    }
  }
  __syncthreads();
  // S^T Q: thread (j, half) sums half of the 128 rows
  {
    const int j = tid & 127, half = tid >> 7;
    float s = 0.0f;
#pragma unroll 8
    for (int i = 64 * half; i < 64 * half + 64; ++i) s = fmaf(p.S_v[(int64_t)i * kD + j], vec[1][i], s);
    red[tid] = s;
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = lane + 64 * e;
      v[e] = vec[0][j] + red[j] + red[128 + j];
    }
    {
      const float x = v[0], y = v[1];
      v[0] = x + y;
      v[1] = x - y;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float t = __shfl_xor(v[e], m, 64);
        v[e] = (lane & m) ? t - v[e] : v[e] + t;
      }
    const float L = Lsh;
    const float inv = (L > 0.0f) ? 1.0f / (L * sqrtf((float)kD)) : 0.0f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = lane + 64 * e;
      float o = v[e] * inv;
      if ((p.sign_v[j >> 5] >> (j & 31)) & 1u) o = -o;
      p.out[(int64_t)bh * kD + j] = o;
    }
  }
}

template <int BKLO, int BKHI, int KS, int BVLO, int BVHI, int VS, int GC>
static int launch_scan(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  const size_t lds = sizeof(float) * (size_t)ScanLds<GC, Rec<BVLO, BVHI, VS>::W>::kTotal;
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute((const void*)decode_scan<BKLO, BKHI, KS, BVLO, BVHI, VS, GC>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return TQ_ERR_HIP;
    attr = true;
  }
  hipLaunchKernelGGL((decode_scan<BKLO, BKHI, KS, BVLO, BVHI, VS, GC>), grid, dim3(64 * kScanWaves),
                     lds, stream, p);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

// Supported (key format, value format) pairs; split given in blocks of 32.
template <int GC>
static int dispatch_scan(const tq_format* fk, const tq_format* fv, const DecodeParams& p, dim3 grid,
                         hipStream_t s) {
  const int kl = fk->bits_lo, kh = fk->split == fk->d ? fk->bits_lo : fk->bits_hi;
  const int vl = fv->bits_lo, vh = fv->split == fv->d ? fv->bits_lo : fv->bits_hi;
  const int ks = fk->split / 32, vs = fv->split / 32;
  const bool ku = kl == kh, vu = vl == vh;
  if (ku && vu) {
    if (kl == 3 && vl == 3) return launch_scan<3, 3, 4, 3, 3, 4, GC>(p, grid, s);
    if (kl == 3 && vl == 2) return launch_scan<3, 3, 4, 2, 2, 4, GC>(p, grid, s);
    if (kl == 2 && vl == 2) return launch_scan<2, 2, 4, 2, 2, 4, GC>(p, grid, s);
    if (kl == 1 && vl == 1) return launch_scan<1, 1, 4, 1, 1, 4, GC>(p, grid, s);
  }
  if (kl == 3 && kh == 2 && ks == 2 && vl == 3 && vh == 2 && vs == 2)
    return launch_scan<3, 2, 2, 3, 2, 2, GC>(p, grid, s);
  return TQ_ERR_SHAPE;
}

// Walsh coefficients alpha_S = 2^-B sum_idx c[idx] prod_{k in S} (2 b_k(idx) - 1) for the odd
// subsets S in the order used by key_block: {0}, {1}, {2}, {0,1,2}.
static void walsh(int bits, const float* c, float* alpha) {
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
bool tq_decode_formats_supported(const tq_format* fk, const tq_format* fv) {
  const int kl = fk->bits_lo, kh = fk->split == fk->d ? fk->bits_lo : fk->bits_hi;
  const int vl = fv->bits_lo, vh = fv->split == fv->d ? fv->bits_lo : fv->bits_hi;
  if (kl == kh && vl == vh)
    return (kl == 3 && (vl == 3 || vl == 2)) || (kl == 2 && vl == 2) || (kl == 1 && vl == 1);
  return kl == 3 && kh == 2 && fk->split == 64 && vl == 3 && vh == 2 && fv->split == 64;
}

tq_decode_plan tq_plan_decode(int32_t batch, int32_t hq, int32_t hkv, int64_t capacity, int32_t d) {
  using namespace tqk;
  tq_decode_plan p{};
  const int group = hq / hkv;
  const int gc = group >= 4 ? 4 : group;
  const int64_t units = (int64_t)batch * hkv * (group / gc);
  // about one workgroup per compute unit of a 256-CU MI355X, at least one tile per wave
  const int64_t per_wg = (int64_t)kTile * kScanWaves;
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
  p.waves = kScanWaves;
  p.parts = (int32_t)n_split;
  p.tokens_per_split = tps;
  p.ws_qrot_off = 0;
  const int64_t qrot_bytes = (int64_t)batch * hq * 2 * d * 4;
  p.ws_nib_off = (qrot_bytes + 255) / 256 * 256;
  const int64_t nib_bytes = units * nib_stride(gc) * 4;
  p.ws_part_off = p.ws_nib_off + (nib_bytes + 255) / 256 * 256;
  p.ws_bytes = p.ws_part_off + (int64_t)batch * hq * p.parts * kPartFloats * 4;
  return p;
}

int tq_launch_decode(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                     const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch,
                     int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                     const void* codes_v, const uint16_t* norms_v, int64_t capacity,
                     const int32_t* seq_lens, float scale, float tau, float* out, float* logits,
                     int64_t* skipped, void* workspace, const tq_decode_plan& plan,
                     hipStream_t stream) {
  using namespace tqk;
  DecodeParams p{};
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
  char* ws = reinterpret_cast<char*>(workspace);
  p.ws_qrot = reinterpret_cast<float*>(ws + plan.ws_qrot_off);
  p.ws_nib = reinterpret_cast<float*>(ws + plan.ws_nib_off);
  p.ws_part = reinterpret_cast<float*>(ws + plan.ws_part_off);
  p.capacity = capacity;
  p.tokens_per_split = plan.tokens_per_split;
  p.batch = batch;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.gc = p.group >= 4 ? 4 : p.group;
  p.q_dtype = q_dtype;
  p.n_split = plan.n_split;
  p.ksplitb = fk->split / 32;
  p.scale = scale;
  p.tau = tau;
  p.gamma = (float)(std::sqrt(M_PI / 2.0) / fk->d);
  for (int i = 0; i < 4; ++i) p.sign_k[i] = p.sign_v[i] = 0;
  for (int j = 0; j < 128; ++j) {
    if (tk->signs[j] < 0) p.sign_k[j >> 5] |= 1u << (j & 31);
    if (tv->signs[j] < 0) p.sign_v[j >> 5] |= 1u << (j & 31);
  }
  walsh(fk->bits_lo, tk->centroids_lo, p.alpha_k[0]);
  walsh(fk->bits_hi, tk->centroids_hi, p.alpha_k[1]);
  for (int i = 0; i < 8; ++i) {
    p.cent_v[0][i] = i < (1 << fv->bits_lo) ? tv->centroids_lo[i] : 0.0f;
    p.cent_v[1][i] = i < (1 << fv->bits_hi) ? tv->centroids_hi[i] : 0.0f;
  }
  const int gc = p.gc;
  const int nchunk = p.group / gc;
  const unsigned units = (unsigned)(batch * hkv * nchunk);
  if (gc == 4) hipLaunchKernelGGL(decode_prologue<4>, dim3(batch * hq), dim3(128), 0, stream, p);
  else if (gc == 2) hipLaunchKernelGGL(decode_prologue<2>, dim3(batch * hq), dim3(128), 0, stream, p);
  else hipLaunchKernelGGL(decode_prologue<1>, dim3(batch * hq), dim3(128), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
  const dim3 grid((unsigned)plan.n_split, units);
  int rc;
  if (gc == 4) rc = dispatch_scan<4>(fk, fv, p, grid, stream);
  else if (gc == 2) rc = dispatch_scan<2>(fk, fv, p, grid, stream);
  else rc = dispatch_scan<1>(fk, fv, p, grid, stream);
  if (rc != TQ_OK) return rc;
  hipLaunchKernelGGL(decode_combine, dim3(batch * hq), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
