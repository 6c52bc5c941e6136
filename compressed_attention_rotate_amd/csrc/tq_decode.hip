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
//   prologue: per (batch, q head) one wave -> q_rot, S q_rot into the workspace.
//   scan:     grid (split, batch * kv-head * head-chunk).  The workgroup builds, in LDS,
//             byte-indexed subset-sum tables of q_rot and S q_rot for the GC query heads
//             that share the KV head (T[g][m] = sum of w_{8g+i} over the set bits i of m,
//             one float per head).  A sign dot product <w, 2b - 1> over 128 coordinates
//             is then 16 table reads: the QJL term directly, and the codebook term
//             through the Walsh expansion of the symmetric codebook,
//             c[idx] = sum_S alpha_S prod_{k in S} (2 b_k - 1) over odd subsets S of the
//             code bit-planes (the planes, and for 3 bits their XOR).  Keys: lane = token.
//             Online softmax per head with wavefront reductions; the Sparse-V gate (zhidx
//             turboquant_plus article, section "01 turboquant_plus：介绍与详解") drops a
//             value row for a head when its running weight estimate is below tau, and
//             skips reading rows dropped by every head.  Values: lane = coordinate pair,
//             fp32 accumulation of w n16 c[idx] and w gamma r16 sigma per head.
//   combine:  per (batch, q head) merge the partial (m, l, acc) of all waves in a fixed
//             order, then out = D H (A + S^T Q) / (sqrt(d) l).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kNB = kD / 32;
constexpr int kScanWaves = 4;
constexpr int kTile = 64;
constexpr int kPartFloats = 2 + 2 * kD;  // m (log2 domain), l, A[d], Q[d]
constexpr float kLog2e = 1.4426950408889634f;

template <int B>
struct Walsh {  // number of odd plane subsets of a B-bit code: the Walsh planes used
  static constexpr int N = (B == 3) ? 4 : B;
};

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
  float* ws_part;   // [batch*hq][parts][kPartFloats]
  int64_t capacity;
  int64_t tokens_per_split;
  int32_t batch, hq, hkv, group, q_dtype, parts;
  int32_t kwords, vwords, ksplitb, vsplitb;
  float scale, tau, gamma;
  uint32_t sign_k[4], sign_v[4];
  float alpha_k[2][4];  // Walsh coefficients of the key codebooks (lo, hi parts)
  float cent_v[2][8];   // value codebooks (lo, hi)
};

// ----------------------------------------------------------------------------- prologue
__global__ __launch_bounds__(64) void decode_prologue(DecodeParams p) {
  const int bh = blockIdx.x;
  const int lane = lane_id();
  __shared__ float qr[kD];
  float v[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int j = lane + 64 * e;
    float x = load_elem(p.q, (int64_t)bh * kD + j, p.q_dtype);
    if ((p.sign_k[j >> 5] >> (j & 31)) & 1u) x = -x;
    v[e] = x;
  }
  {
    const float a = v[0], b = v[1];
    v[0] = a + b;
    v[1] = a - b;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float t = __shfl_xor(v[e], m, 64);
      v[e] = (lane & m) ? t - v[e] : v[e] + t;
    }
  const float isd = 1.0f / sqrtf((float)kD);
  v[0] *= isd;
  v[1] *= isd;
  qr[lane] = v[0];
  qr[lane + 64] = v[1];
  __syncthreads();
  float* dst = p.ws_qrot + (int64_t)bh * 2 * kD;
  dst[lane] = v[0];
  dst[lane + 64] = v[1];
  // S q_rot: lane computes rows lane and lane + 64
  float s0 = 0.0f, s1 = 0.0f;
  const float* r0 = p.S_k + (int64_t)lane * kD;
  const float* r1 = p.S_k + (int64_t)(lane + 64) * kD;
#pragma unroll 8
  for (int k = 0; k < kD; ++k) {
    s0 = fmaf(r0[k], qr[k], s0);
    s1 = fmaf(r1[k], qr[k], s1);
  }
  dst[kD + lane] = s0;
  dst[kD + lane + 64] = s1;
}

// ----------------------------------------------------------------------------- scan
template <int GC>
struct ScanLds {
  // subset-sum tables: [2 (q_rot, S q_rot)][16 groups][256][GC]
  static constexpr int kTable = 2 * 16 * 256 * GC;
  static constexpr int kNib = 2 * 16 * 2 * 16 * GC;    // nibble tables (setup only)
  static constexpr int kWave = kTile * 2 * GC + kTile * 16;  // weights + V staging (<=16 words)
  static constexpr int kTotal = kTable + kScanWaves * kWave;
  static_assert(kScanWaves * kWave >= kNib, "nibble tables alias the per-wave areas");
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

// Add the byte-table reads of one 32-bit sign word (4 groups starting at g0) times alpha.
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

// Codebook term of one key block: Walsh planes of the B code planes.
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

template <int BKLO, int BKHI, int BVLO, int BVHI, int GC>
__global__ __launch_bounds__(64 * kScanWaves) void decode_scan(DecodeParams p) {
  using L = ScanLds<GC>;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  float* Tq = lds;                         // [16][256][GC]
  float* Ts = lds + 16 * 256 * GC;         // [16][256][GC]
  float* nib = lds + L::kTable;            // [2][16][2][16][GC], aliases the wave areas
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  float* wts = lds + L::kTable + wave * L::kWave;  // [64][2*GC]
  uint32_t* vst = reinterpret_cast<uint32_t*>(wts + kTile * 2 * GC);  // [64][16]
  __shared__ float wvec[2][GC][kD];
  __shared__ float corr_q[GC], sum_s[GC];
  __shared__ float centv[16];

  const int nchunk = p.group / GC;
  const int unit = blockIdx.y;
  const int chunk = unit % nchunk;
  const int bk = unit / nchunk;  // b * hkv + kv head
  const int b = bk / p.hkv;
  const int h0 = (bk % p.hkv) * p.group + chunk * GC;  // first q head of this chunk
  const int64_t seq = p.seq_lens[b];
  const int64_t t_begin = (int64_t)blockIdx.x * p.tokens_per_split;
  int64_t t_end = t_begin + p.tokens_per_split;
  if (t_end > seq) t_end = seq;

  // ---- tables (every workgroup, also empty ones: their partials must be written)
  for (int i = threadIdx.x; i < 2 * GC * kD; i += blockDim.x) {
    const int v = i / (GC * kD), h = (i / kD) % GC, j = i % kD;
    wvec[v][h][j] = p.ws_qrot[((int64_t)b * p.hq + h0 + h) * 2 * kD + v * kD + j];
  }
  if (threadIdx.x < 16) centv[threadIdx.x] = (&p.cent_v[0][0])[threadIdx.x];
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * 16 * 2 * 16 * GC; i += blockDim.x) {
    const int h = i % GC, n = (i / GC) % 16, half = (i / (GC * 16)) % 2;
    const int g = (i / (GC * 32)) % 16, v = i / (GC * 32 * 16);
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if ((n >> k) & 1) s += wvec[v][h][8 * g + 4 * half + k];
    nib[i] = s;
  }
  if (wave == 0) {
    // constant parts of the sign dot products: <w, 2b - 1> = 2 <w, b> - sum(w)
    for (int h = 0; h < GC; ++h) {
      float cq = 0.0f;
#pragma unroll
      for (int blk = 0; blk < kNB; ++blk) {
        const float wb = half_sum(wvec[0][h][32 * blk + (lane & 31)]);
        const bool lo = blk < p.ksplitb;
        const int nw = lo ? Walsh<BKLO>::N : Walsh<BKHI>::N;
        float asum = 0.0f;
        for (int k = 0; k < nw; ++k) asum += p.alpha_k[lo ? 0 : 1][k];
        cq += asum * wb;
      }
      const float ss = wave_sum(wvec[1][h][lane] + wvec[1][h][lane + 64]);
      if (lane == 0) {
        corr_q[h] = cq;
        sum_s[h] = ss;
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * 16 * 256; i += blockDim.x) {
    const int v = i / (16 * 256), g = (i / 256) % 16, m = i % 256;
    const float* nl = nib + (((v * 16 + g) * 2 + 0) * 16 + (m & 15)) * GC;
    const float* nh = nib + (((v * 16 + g) * 2 + 1) * 16 + (m >> 4)) * GC;
    float* dst = (v == 0 ? Tq : Ts) + (g * 256 + m) * GC;
#pragma unroll
    for (int h = 0; h < GC; ++h) dst[h] = nl[h] + nh[h];
  }
  __syncthreads();

  float cq[GC], ws[GC];
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    cq[h] = corr_q[h];
    ws[h] = sum_s[h];
  }
  float alo[4], ahi[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    alo[k] = 2.0f * p.alpha_k[0][k];
    ahi[k] = 2.0f * p.alpha_k[1][k];
  }

  // value lane mapping: lane -> coordinates j0 = 32 (lane / 16) + 2 (lane % 16), j0 + 1
  const int vblk = lane >> 4, vbit = 2 * (lane & 15);
  const bool vlo = vblk < p.vsplitb;
  const int vnb = vlo ? BVLO : BVHI;
  const int voff = vlo ? vblk * (BVLO + 1) : p.vsplitb * (BVLO + 1) + (vblk - p.vsplitb) * (BVHI + 1);
  const float* cv = centv + (vlo ? 0 : 8);

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

  for (int64_t t0 = t_begin + (int64_t)wave * kTile; t0 < t_end; t0 += (int64_t)kScanWaves * kTile) {
    const int64_t t = t0 + lane;
    const bool valid = t < t_end;
    // ---------------- keys: lane = token
    float mse[GC], qjl[GC];
#pragma unroll
    for (int h = 0; h < GC; ++h) mse[h] = qjl[h] = 0.0f;
    uint32_t kn = 0;
    if (valid) {
      const uint32_t* rec = p.codes_k + (kv_base + t) * p.kwords;
      kn = p.norms_k[kv_base + t];
#pragma unroll
      for (int blk = 0; blk < kNB; ++blk) {
        if (blk < p.ksplitb) {
          const uint32_t* wb = rec + blk * (BKLO + 1);
          uint32_t w[BKLO + 1];
#pragma unroll
          for (int i = 0; i <= BKLO; ++i) w[i] = wb[i];
          key_block<BKLO, GC>(Tq, blk, w, alo, mse);
          lut_word<GC>(Ts, 4 * blk, w[BKLO], 2.0f, qjl);
        } else {
          const uint32_t* wb = rec + p.ksplitb * (BKLO + 1) + (blk - p.ksplitb) * (BKHI + 1);
          uint32_t w[BKHI + 1];
#pragma unroll
          for (int i = 0; i <= BKHI; ++i) w[i] = wb[i];
          key_block<BKHI, GC>(Tq, blk, w, ahi, mse);
          lut_word<GC>(Ts, 4 * blk, w[BKHI], 2.0f, qjl);
        }
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
    uint32_t vn = valid ? p.norms_v[kv_base + t] : 0u;
    const float vn16 = f16_bits_to_f32(vn), vr16 = f16_bits_to_f32(vn >> 16);
    bool any_keep = false;
    float* wrow = wts + lane * 2 * GC;
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      const float mt = wave_max(lg[h]);
      const float mn = fmaxf(m_run[h], mt);
      const float corr = (m_run[h] == -INFINITY) ? 0.0f : exp2f(m_run[h] - mn);
      float wgt = valid ? exp2f(lg[h] - mn) : 0.0f;
      l_run[h] = l_run[h] * corr + wave_sum(wgt);
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
    if (any_keep) {
      const uint32_t* rec = p.codes_v + (kv_base + t) * p.vwords;
      for (int i = 0; i < p.vwords; ++i) vst[lane * 16 + i] = rec[i];
    }
    // ---------------- values: lane = coordinate pair, loop over kept tokens
    while (keep) {
      const int tl = __builtin_ctzll(keep);
      keep &= keep - 1;
      const uint32_t* vw = vst + tl * 16 + voff;
      uint32_t f[3] = {0u, 0u, 0u};
      for (int q = 0; q < 3; ++q)
        if (q < vnb) f[q] = (vw[q] >> vbit) & 3u;
      const uint32_t fs = (vw[vnb] >> vbit) & 3u;
      const int i0 = (int)((f[0] & 1u) | ((f[1] & 1u) << 1) | ((f[2] & 1u) << 2));
      const int i1 = (int)(((f[0] >> 1) & 1u) | (((f[1] >> 1) & 1u) << 1) | (((f[2] >> 1) & 1u) << 2));
      const float c0 = cv[i0], c1 = cv[i1];
      const float s0 = (fs & 1u) ? 1.0f : -1.0f, s1 = (fs & 2u) ? 1.0f : -1.0f;
      const float* wr = wts + tl * 2 * GC;
#pragma unroll
      for (int h = 0; h < GC; ++h) {
        const float u = wr[h], uq = wr[GC + h];
        am[h][0] = fmaf(u, c0, am[h][0]);
        am[h][1] = fmaf(u, c1, am[h][1]);
        aq[h][0] = fmaf(uq, s0, aq[h][0]);
        aq[h][1] = fmaf(uq, s1, aq[h][1]);
      }
    }
  }
  // ---------------- partial results of this wave
  const int pidx = blockIdx.x * kScanWaves + wave;
  const int j0 = 32 * vblk + vbit;
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    float* part = p.ws_part + (((int64_t)b * p.hq + h0 + h) * p.parts + pidx) * kPartFloats;
    if (lane == 0) {
      part[0] = m_run[h];
      part[1] = l_run[h];
    }
    part[2 + j0] = am[h][0];
    part[2 + j0 + 1] = am[h][1];
    part[2 + kD + j0] = aq[h][0];
    part[2 + kD + j0 + 1] = aq[h][1];
  }
  if (p.skipped && lane == 0 && n_skipped) atomicAdd(p.skipped, n_skipped);
}

// ----------------------------------------------------------------------------- combine
__global__ __launch_bounds__(64) void decode_combine(DecodeParams p) {
  const int bh = blockIdx.x;
  const int lane = lane_id();
  __shared__ float qv[kD];
  const float* parts = p.ws_part + (int64_t)bh * p.parts * kPartFloats;
  float M = -INFINITY;
  for (int i = 0; i < p.parts; ++i) M = fmaxf(M, parts[(int64_t)i * kPartFloats]);
  float Lsum = 0.0f, a[2] = {0.0f, 0.0f}, qq[2] = {0.0f, 0.0f};
  if (M != -INFINITY) {
    for (int i = 0; i < p.parts; ++i) {
      const float* pt = parts + (int64_t)i * kPartFloats;
      if (pt[0] == -INFINITY) continue;
      const float sc = exp2f(pt[0] - M);
      Lsum = fmaf(pt[1], sc, Lsum);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        a[e] = fmaf(pt[2 + lane + 64 * e], sc, a[e]);
        qq[e] = fmaf(pt[2 + kD + lane + 64 * e], sc, qq[e]);
      }
    }
  }
  qv[lane] = qq[0];
  qv[lane + 64] = qq[1];
  __syncthreads();
  // rotated-domain value: A + S^T Q
  float v[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int j = lane + 64 * e;
    float s = a[e];
    for (int i = 0; i < kD; ++i) s = fmaf(p.S_v[(int64_t)i * kD + j], qv[i], s);
    v[e] = s;
  }
  // back to the original basis: D H v / sqrt(d)
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
  const float inv = (Lsum > 0.0f) ? 1.0f / (Lsum * sqrtf((float)kD)) : 0.0f;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int j = lane + 64 * e;
    float o = v[e] * inv;
    if ((p.sign_v[j >> 5] >> (j & 31)) & 1u) o = -o;
    p.out[(int64_t)bh * kD + j] = o;
  }
}

template <int BKLO, int BKHI, int BVLO, int BVHI, int GC>
static int launch_scan(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  const size_t lds = sizeof(float) * (size_t)ScanLds<GC>::kTotal;
  static bool attr = false;
  if (!attr) {
    if (hipFuncSetAttribute((const void*)decode_scan<BKLO, BKHI, BVLO, BVHI, GC>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return TQ_ERR_HIP;
    attr = true;
  }
  hipLaunchKernelGGL((decode_scan<BKLO, BKHI, BVLO, BVHI, GC>), grid, dim3(64 * kScanWaves), lds,
                     stream, p);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

template <int GC>
static int dispatch_scan(int kl, int kh, int vl, int vh, const DecodeParams& p, dim3 grid,
                         hipStream_t s) {
  if (kl == 3 && kh == 3 && vl == 3 && vh == 3) return launch_scan<3, 3, 3, 3, GC>(p, grid, s);
  if (kl == 3 && kh == 2 && vl == 3 && vh == 2) return launch_scan<3, 2, 3, 2, GC>(p, grid, s);
  if (kl == 3 && kh == 3 && vl == 2 && vh == 2) return launch_scan<3, 3, 2, 2, GC>(p, grid, s);
  if (kl == 2 && kh == 2 && vl == 2 && vh == 2) return launch_scan<2, 2, 2, 2, GC>(p, grid, s);
  if (kl == 1 && kh == 1 && vl == 1 && vh == 1) return launch_scan<1, 1, 1, 1, GC>(p, grid, s);
  if (kl == 2 && kh == 1 && vl == 2 && vh == 1) return launch_scan<2, 1, 2, 1, GC>(p, grid, s);
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
tq_decode_plan tq_plan_decode(int32_t batch, int32_t hq, int32_t hkv, int64_t capacity, int32_t d) {
  using namespace tqk;
  tq_decode_plan p{};
  const int group = hq / hkv;
  const int gc = group >= 4 ? 4 : group;
  const int64_t units = (int64_t)batch * hkv * (group / gc);
  // aim at about two workgroups per compute unit of a 256-CU MI355X, at least one tile
  // per wave per split
  const int64_t per_wave = (int64_t)kTile * kScanWaves;
  int64_t max_split = (capacity + per_wave - 1) / per_wave;
  if (max_split < 1) max_split = 1;
  int64_t n_split = (512 + units - 1) / units;
  if (n_split > max_split) n_split = max_split;
  if (n_split < 1) n_split = 1;
  int64_t tps = (capacity + n_split - 1) / n_split;
  tps = ((tps + kTile - 1) / kTile) * kTile;
  if (tps < kTile) tps = kTile;
  p.n_split = (int32_t)n_split;
  p.waves = kScanWaves;
  p.parts = (int32_t)(n_split * kScanWaves);
  p.tokens_per_split = tps;
  p.ws_qrot_off = 0;
  const int64_t qrot_bytes = (int64_t)batch * hq * 2 * d * 4;
  p.ws_part_off = (qrot_bytes + 255) / 256 * 256;
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
  p.ws_qrot = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + plan.ws_qrot_off);
  p.ws_part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + plan.ws_part_off);
  p.capacity = capacity;
  p.tokens_per_split = plan.tokens_per_split;
  p.batch = batch;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.q_dtype = q_dtype;
  p.parts = plan.parts;
  p.kwords = (int)(tq_record_bytes(fk) / 4);
  p.vwords = (int)(tq_record_bytes(fv) / 4);
  p.ksplitb = fk->split / 32;
  p.vsplitb = fv->split / 32;
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
  const int gc = p.group >= 4 ? 4 : p.group;
  const int nchunk = p.group / gc;
  hipLaunchKernelGGL(decode_prologue, dim3(batch * hq), dim3(64), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
  const dim3 grid((unsigned)plan.n_split, (unsigned)(batch * hkv * nchunk));
  int rc;
  const int kl = fk->bits_lo, kh = fk->split == fk->d ? fk->bits_lo : fk->bits_hi;
  const int vl = fv->bits_lo, vh = fv->split == fv->d ? fv->bits_lo : fv->bits_hi;
  if (gc == 4) rc = dispatch_scan<4>(kl, kh, vl, vh, p, grid, stream);
  else if (gc == 2) rc = dispatch_scan<2>(kl, kh, vl, vh, p, grid, stream);
  else rc = dispatch_scan<1>(kl, kh, vl, vh, p, grid, stream);
  if (rc != TQ_OK) return rc;
  hipLaunchKernelGGL(decode_combine, dim3(batch * hq), dim3(64), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
