// Prefill attention on MFMA: a chunk of new queries attends causally to a paged compressed
// cache (the chunk's own keys and values are already written to it).
//
// The decode estimator of each logit,
//   n16_t <q_rot, c[idx_t]> + gamma r16_t <S q_rot, 2 sigma_t - 1>
// (163.com explainer, sections "第二步：QJL" and "速度"), is a 256-wide dot product between a
// query row [q_rot | gamma S q_rot] and a key row [n16 c[idx] | r16 (2 sigma - 1)]; the value
// sum splits the same way into A = sum_t p_t n16_t c[idx_t] and Q = gamma sum_t p_t r16_t
// (2 sigma_t - 1), rotated back once per row as in decode (out = D H (A + S^T Q) / (sqrt(d) l)).
// With many query rows per key these are dense contractions, so they run on
// v_mfma_f32_16x16x32_f16 (logits and values; the 16x16x16 form takes as many cycles for
// half the work on this part), fp32 accumulation:
//   prefill_q:     per row, q_rot (FWHT) and gamma S q_rot as fp16 operand rows;
//   prefill_scan:  grid (64-row block, KV head, key split); per 64-key tile the workgroup
//                  dequantizes the keys into LDS as [key][coord] fp16 rows (n16 c, +-r16)
//                  and the values transposed, [coord][key] (n16 c, +-r16), then each wave
//                  computes the logits of its 16 rows transposed (keys x rows, so the
//                  accumulator is directly the B operand of the value product), applies the
//                  causal mask and an online softmax, and accumulates A^T and Q^T;
//   decode_combine merges the key splits and rotates back.
// Precision: every operand is exact in fp16 or split into fp16 hi + lo.  The per-key norms
// are kept out of the operands (the logit is n16 * acc_c + r16 * acc_s, the value weights are
// p n16 and p r16), so the key-side operands are codebook values (hi + lo from a table) and
// +-1 (exact); q_rot, gamma S q_rot and the weights are split hi + lo.  Three products per
// split pair (hi hi, hi lo, lo hi) give ~2^-22 relative accuracy with fp32 accumulation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "tq_decode_kernel.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

constexpr int kPfRows = 64;             // query rows per workgroup (4 waves x 16)
constexpr int kPfKeys = 64;             // keys per tile
constexpr int kPfThreads = 256;
constexpr int kKcStride = kD + 8;       // halves per [key][coord] row (padded)
constexpr int kVtStride = kPfKeys + 8;  // halves per [coord][key] row (padded)

struct PrefillQParams {
  const void* q;        // [n_new][hq][128]
  const float* S;       // key JL matrix [projection][coord]
  _Float16* qop;        // [rows][512]: q_rot hi | lo | gamma S q_rot hi | lo, rows (kv head,
                        // query, head in group)
  int64_t rows;
  int32_t q_dtype, n_new, hq, group;
  uint32_t sign[4];     // key sign flips
  float gamma;
};

// 16 rows per workgroup, one wave per row at a time; S stays in LDS.
__global__ __launch_bounds__(256) void prefill_q(PrefillQParams p) {
  __shared__ float Sl[kD * (kD + 1)];   // padded rows: lane j reads row j conflict-free
  __shared__ float qr[4][kD];
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  for (int e = tid; e < kD * kD; e += 256) Sl[(e / kD) * (kD + 1) + (e % kD)] = p.S[e];
  __syncthreads();
  const float isd = 1.0f / sqrtf((float)kD);
  for (int k = wave; k < 16; k += 4) {
    const int64_t R = (int64_t)blockIdx.x * 16 + k;
    if (R >= p.rows) break;
    // R = (kv head * n_new + query) * group + g
    const int64_t qg = R / p.group;
    const int g = (int)(R - qg * p.group);
    const int64_t kvh = qg / p.n_new, qi = qg - kvh * p.n_new;
    const int64_t head = kvh * p.group + g;
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = lane + 64 * e;
      float x = load_elem(p.q, (qi * p.hq + head) * kD + j, p.q_dtype);
      const uint32_t sw = (lane & 32) ? uniform_u32(p.sign[2 * e + 1]) : uniform_u32(p.sign[2 * e]);
      if ((sw >> (j & 31)) & 1u) x = -x;
      v[e] = x;
    }
    fwht128(v, lane);
    v[0] *= isd;
    v[1] *= isd;
    qr[wave][lane] = v[0];
    qr[wave][lane + 64] = v[1];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the row is visible to the wave
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = lane + 64 * e;
      float s = 0.0f;
#pragma unroll 8
      for (int i = 0; i < kD; ++i) s = fmaf(Sl[j * (kD + 1) + i], qr[wave][i], s);
      const float gs = p.gamma * s;
      const _Float16 qh = (_Float16)v[e], sh = (_Float16)gs;
      p.qop[R * 512 + j] = qh;
      p.qop[R * 512 + kD + j] = (_Float16)(v[e] - (float)qh);
      p.qop[R * 512 + 2 * kD + j] = sh;
      p.qop[R * 512 + 3 * kD + j] = (_Float16)(gs - (float)sh);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of qr done before the next row
  }
}

struct PrefillParams {
  const _Float16* qop;
  const uint32_t* codes_k;
  const uint32_t* norms_k;
  const uint32_t* codes_v;
  const uint32_t* norms_v;
  const int32_t* block_table;
  float* ws_part;               // [n_new * hq][n_split][kPartFloats]
  int64_t num_pages;
  int64_t start;                // position of the chunk's first token
  int64_t keys_per_split;       // multiple of 64
  int32_t page_log2, max_blocks;
  int32_t n_new, hq, hkv, group, n_split;
  float scale_log2;             // scale * log2(e)
  float gamma;
  int32_t kw, ksb, kblo, kbhi;  // key record: words, split blocks, widths
  int32_t vw, vsb, vblo, vbhi, vq;
  float cent_k[16], cent_v[16]; // lo table, hi table
};

// Centroid-pair table of a B-bit codebook, indexed by the sparse code-bit pattern of two
// coordinates: four coordinates with code-bit nibbles b0, b1, b2 give f = b0 << 1 |
// b1 << 5 | b2 << 9, and (f & 0x1998) is 8 times the pattern P = p0 | p1 << 4 | p2 << 8 of
// coordinates (2, 3), ((f << 2) & 0x1998) that of coordinates (0, 1).  Entry P holds the
// fp16 (hi(c'[lo]), hi(c'[hi])), (lo(c'[lo]), lo(c'[hi])) of c' = 2^6 c.
constexpr int kPfPat = 0x334;          // entries of the 3-bit table (and room for 1 or 2 bits)
constexpr uint32_t kPfPatMask = 0x1998u;
constexpr float kPfCent = 64.0f;

// Pattern fields of one code byte (bits sh .. sh + 7 of the planes): the low nibble's field in
// bits 0..15, the high nibble's in 16..31 (three byte x constant products place the plane
// nibbles 4 bits apart).
__device__ __forceinline__ uint32_t pattern_fields(uint32_t p0, uint32_t p1, uint32_t p2, int sh) {
  return ((__builtin_amdgcn_ubfe(p0, sh, 8) * 0x2002u) & 0x001E001Eu) |
         ((__builtin_amdgcn_ubfe(p1, sh, 8) * 0x20020u) & 0x01E001E0u) |
         ((__builtin_amdgcn_ubfe(p2, sh, 8) * 0x200200u) & 0x1E001E00u);
}

// The four centroid pairs (coordinates 0-1, 2-3, 4-5, 6-7 of the byte) from table cp.
__device__ __forceinline__ void pattern_pairs(const char* cp, uint32_t F, u32x2 (&e)[4]) {
  e[0] = *reinterpret_cast<const u32x2*>(cp + ((F << 2) & kPfPatMask));
  e[1] = *reinterpret_cast<const u32x2*>(cp + (F & kPfPatMask));
  e[2] = *reinterpret_cast<const u32x2*>(cp + ((F >> 14) & kPfPatMask));
  e[3] = *reinterpret_cast<const u32x2*>(cp + ((F >> 16) & kPfPatMask));
}

__global__ __launch_bounds__(kPfThreads) void prefill_scan(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) _Float16 Kh[kPfKeys * kKcStride];
  __shared__ __attribute__((aligned(16))) _Float16 Kl[kPfKeys * kKcStride];
  __shared__ __attribute__((aligned(16))) _Float16 Ks[kPfKeys * kKcStride];
  __shared__ __attribute__((aligned(16))) _Float16 Vh[kD * kVtStride];
  __shared__ __attribute__((aligned(16))) _Float16 Vl[kD * kVtStride];
  __shared__ __attribute__((aligned(16))) _Float16 Vs[kD * kVtStride];
  // n16 / 2^6, r16 of the tile's keys and n16, r16 of its values (zero for absent tokens)
  __shared__ float knorm[2][kPfKeys], vnorm[2][kPfKeys];
  __shared__ __attribute__((aligned(16))) uint32_t cpt[4][2 * kPfPat];  // key lo, key hi, value lo, value hi
  __shared__ __attribute__((aligned(16))) uint32_t spt[16][2];          // nibble -> 4 fp16 +-1
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  {  // centroid-pair tables (every pattern slot written; unused widths stay finite) and signs
    const int nbits[4] = {p.kblo, p.kbhi, p.vblo, p.vbhi};
    for (int i = tid; i < 4 * kPfPat; i += kPfThreads) {
      const int tb = i / kPfPat, P = i % kPfPat;
      const int mask = (1 << nbits[tb]) - 1;
      const int p0 = P & 15, p1 = (P >> 4) & 15, p2 = (P >> 8) & 15;
      const int ilo = ((p0 & 1) | ((p1 & 1) << 1) | ((p2 & 1) << 2)) & mask;
      const int ihi = (((p0 >> 1) & 1) | (((p1 >> 1) & 1) << 1) | (((p2 >> 1) & 1) << 2)) & mask;
      const float* ct = tb < 2 ? p.cent_k + 8 * tb : p.cent_v + 8 * (tb - 2);
      const float c0 = ct[ilo] * kPfCent, c1 = ct[ihi] * kPfCent;
      const _Float16 h0 = (_Float16)c0, h1 = (_Float16)c1;
      const _Float16 l0 = (_Float16)(c0 - (float)h0), l1 = (_Float16)(c1 - (float)h1);
      cpt[tb][2 * P] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      cpt[tb][2 * P + 1] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }
    if (tid < 32) {
      const int n = tid >> 1, d = tid & 1;
      const uint32_t lo = ((n >> (2 * d)) & 1) ? 0x3C00u : 0xBC00u;
      const uint32_t hi = ((n >> (2 * d + 1)) & 1) ? 0x3C00u : 0xBC00u;
      spt[n][d] = lo | (hi << 16);
    }
    if (!p.vq)  // MSE-only values: the sign operands stay zero
      for (int i = tid; i < kD * kVtStride / 2; i += kPfThreads) reinterpret_cast<uint32_t*>(Vs)[i] = 0u;
  }
  const int64_t rows_kvh = (int64_t)p.n_new * p.group;
  const int kvh = blockIdx.y, split = blockIdx.z;
  const int64_t rb0 = (int64_t)blockIdx.x * kPfRows;
  // this lane's row (one of the wave's 16); lanes l, l^16, l^32, l^48 share it
  const int64_t rloc = rb0 + wave * 16 + (lane & 15);
  const bool row_ok = rloc < rows_kvh;
  const int64_t qi = row_ok ? rloc / p.group : 0;
  const int64_t limit = p.start + qi;            // the row sees keys t <= limit
  const int64_t R = (int64_t)kvh * rows_kvh + (row_ok ? rloc : 0);
  // query operands (B of the logit product): coords 32 ks + 8 (lane >> 4) .. + 7, hi and lo
  h16x8 qh[4], ql[4], sh[4], sl[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const _Float16* src = p.qop + R * 512 + 32 * ks + 8 * (lane >> 4);
    qh[ks] = row_ok ? *reinterpret_cast<const h16x8*>(src) : h16x8{};
    ql[ks] = row_ok ? *reinterpret_cast<const h16x8*>(src + kD) : h16x8{};
    sh[ks] = row_ok ? *reinterpret_cast<const h16x8*>(src + 2 * kD) : h16x8{};
    sl[ks] = row_ok ? *reinterpret_cast<const h16x8*>(src + 3 * kD) : h16x8{};
  }
  const int64_t total = p.start + p.n_new;
  const int64_t last_row = (rb0 + kPfRows < rows_kvh ? rb0 + kPfRows : rows_kvh) - 1;
  int64_t t_lo = (int64_t)split * p.keys_per_split;
  int64_t t_hi = t_lo + p.keys_per_split;
  if (t_hi > total) t_hi = total;
  if (t_hi > p.start + last_row / p.group + 1) t_hi = p.start + last_row / p.group + 1;

  f32x4 om[8], oq[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    om[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    oq[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  float m_run = -INFINITY, l_run = 0.0f;
  // ---- register prefetch of one tile's records.  Keys: thread (key = lane, block = wave);
  // values: thread (keys 2 kp, 2 kp + 1 with kp = lane & 31, block = wave, bytes 2 bh,
  // 2 bh + 1 with bh = lane >> 5); wave 0 also takes the norms (lane = token).
  const int b = wave, kp = lane & 31, bh = lane >> 5;
  const bool klo = b < p.ksb, vlo = b < p.vsb;
  const int knb = klo ? p.kblo : p.kbhi, vnb = vlo ? p.vblo : p.vbhi;
  const int koff = klo ? b * (p.kblo + 1) : p.ksb * (p.kblo + 1) + (b - p.ksb) * (p.kbhi + 1);
  const int voff = vlo ? b * (p.vblo + p.vq) : p.vsb * (p.vblo + p.vq) + (b - p.vsb) * (p.vbhi + p.vq);
  const char* kcp = reinterpret_cast<const char*>(cpt[klo ? 0 : 1]);
  const char* vcp = reinterpret_cast<const char*>(cpt[vlo ? 2 : 3]);
  uint32_t kwr[4] = {0u, 0u, 0u, 0u}, vwr[2][4] = {}, nkr = 0, nvr = 0;
  auto block_words = [](const uint32_t* rec, int nb, int qj, uint32_t (&w)[4]) {
    w[0] = rec[0];
    w[1] = nb >= 2 ? rec[1] : 0u;
    w[2] = nb >= 3 ? rec[2] : 0u;
    w[3] = qj ? rec[nb] : 0u;
  };
  auto fetch = [&](int64_t tt0) {
    if (tt0 >= t_hi) return;
    const int32_t pg = p.block_table[tt0 >> p.page_log2];
    const bool pok = pg >= 0 && (int64_t)pg < p.num_pages;
    const int64_t base = (((int64_t)(pok ? pg : 0) * p.hkv + kvh) << p.page_log2) + (tt0 & ((1ll << p.page_log2) - 1));
    const bool kok = pok && tt0 + lane < total;
    if (kok) block_words(p.codes_k + (base + lane) * p.kw + koff, knb, 1, kwr);
    else kwr[0] = kwr[1] = kwr[2] = kwr[3] = 0u;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (pok && tt0 + 2 * kp + u < total) block_words(p.codes_v + (base + 2 * kp + u) * p.vw + voff, vnb, p.vq, vwr[u]);
      else vwr[u][0] = vwr[u][1] = vwr[u][2] = vwr[u][3] = 0u;
    }
    if (wave == 0) {
      nkr = kok ? p.norms_k[base + lane] : 0u;
      nvr = kok ? p.norms_v[base + lane] : 0u;
    }
  };
  fetch(t_lo);
  for (int64_t t0 = t_lo; t0 < t_hi; t0 += kPfKeys) {
    __syncthreads();  // the previous tile is consumed
    {  // dequantize into LDS: key rows [key][coord] and value columns [coord][key]
      if (wave == 0) {
        knorm[0][lane] = f16_bits_to_f32(nkr & 0xFFFFu) * (1.0f / kPfCent);
        knorm[1][lane] = f16_bits_to_f32(nkr >> 16);
        vnorm[0][lane] = f16_bits_to_f32(nvr & 0xFFFFu);
        vnorm[1][lane] = f16_bits_to_f32(nvr >> 16);
      }
      const int ko = lane * kKcStride + 32 * b;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 e[4];
        pattern_pairs(kcp, pattern_fields(kwr[0], kwr[1], kwr[2], 8 * q), e);
        *reinterpret_cast<u32x4*>(Kh + ko + 8 * q) = u32x4{e[0][0], e[1][0], e[2][0], e[3][0]};
        *reinterpret_cast<u32x4*>(Kl + ko + 8 * q) = u32x4{e[0][1], e[1][1], e[2][1], e[3][1]};
        const u32x2 s0 = *reinterpret_cast<const u32x2*>(&spt[__builtin_amdgcn_ubfe(kwr[3], 8 * q, 4)][0]);
        const u32x2 s1 = *reinterpret_cast<const u32x2*>(&spt[__builtin_amdgcn_ubfe(kwr[3], 8 * q + 4, 4)][0]);
        *reinterpret_cast<u32x4*>(Ks + ko + 8 * q) = u32x4{s0[0], s0[1], s1[0], s1[1]};
      }
      uint32_t* vh = reinterpret_cast<uint32_t*>(Vh);
      uint32_t* vl = reinterpret_cast<uint32_t*>(Vl);
      uint32_t* vs = reinterpret_cast<uint32_t*>(Vs);
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q = 2 * bh + qq;
        u32x2 ea[4], eb[4];
        pattern_pairs(vcp, pattern_fields(vwr[0][0], vwr[0][1], vwr[0][2], 8 * q), ea);
        pattern_pairs(vcp, pattern_fields(vwr[1][0], vwr[1][1], vwr[1][2], 8 * q), eb);
        const uint32_t sx = __builtin_amdgcn_ubfe(vwr[0][3], 8 * q, 8) | (__builtin_amdgcn_ubfe(vwr[1][3], 8 * q, 8) << 16);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int c = 32 * b + 8 * q + 2 * d;  // coordinates c, c + 1; keys 2 kp, 2 kp + 1
          const int o0 = (c * kVtStride) / 2 + kp, o1 = ((c + 1) * kVtStride) / 2 + kp;
          vh[o0] = __builtin_amdgcn_perm(eb[d][0], ea[d][0], 0x05040100u);
          vh[o1] = __builtin_amdgcn_perm(eb[d][0], ea[d][0], 0x07060302u);
          vl[o0] = __builtin_amdgcn_perm(eb[d][1], ea[d][1], 0x05040100u);
          vl[o1] = __builtin_amdgcn_perm(eb[d][1], ea[d][1], 0x07060302u);
          if (p.vq) {
            vs[o0] = ((sx << (15 - 2 * d)) & 0x80008000u) ^ 0xBC00BC00u;
            vs[o1] = ((sx << (14 - 2 * d)) & 0x80008000u) ^ 0xBC00BC00u;
          }
        }
      }
    }
    fetch(t0 + kPfKeys);
    __syncthreads();
    // ---- logits, transposed: lg[kb][r] = key kb*16 + 4 (lane >> 4) + r, row lane & 15
    float lg[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 ac = {0.0f, 0.0f, 0.0f, 0.0f}, as = {0.0f, 0.0f, 0.0f, 0.0f};
      const int ko = (kb * 16 + (lane & 15)) * kKcStride + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const h16x8 kh = *reinterpret_cast<const h16x8*>(Kh + ko + 32 * ks);
        const h16x8 kl = *reinterpret_cast<const h16x8*>(Kl + ko + 32 * ks);
        const h16x8 kss = *reinterpret_cast<const h16x8*>(Ks + ko + 32 * ks);
        ac = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, qh[ks], ac, 0, 0, 0);
        ac = __builtin_amdgcn_mfma_f32_16x16x32_f16(kl, qh[ks], ac, 0, 0, 0);
        ac = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, ql[ks], ac, 0, 0, 0);
        as = __builtin_amdgcn_mfma_f32_16x16x32_f16(kss, sh[ks], as, 0, 0, 0);
        as = __builtin_amdgcn_mfma_f32_16x16x32_f16(kss, sl[ks], as, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = kb * 16 + 4 * (lane >> 4) + r;
        const int64_t key = t0 + kk;
        const bool vis = row_ok && key <= limit && key < t_hi;
        const float est = fmaf(knorm[0][kk], ac[r], knorm[1][kk] * as[r]);
        lg[kb][r] = vis ? est * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, lg[kb][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, other_half(mx));
    const float m_new = fmaxf(m_run, mx);
    const float corr = (m_new == -INFINITY) ? 1.0f : exp2f(m_run - m_new);
    float psum = 0.0f;
    // value weights p n16 and p r16 of each key, split hi + lo (B operands of the value sum)
    h16x4 pch[4], pcl[4], psh[4], psl[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = kb * 16 + 4 * (lane >> 4) + r;
        // hardware exp2: weights below 2^-126 of the running maximum flush to zero
        const float pv = (lg[kb][r] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(lg[kb][r] - m_new);
        psum += pv;
        const float wc = pv * vnorm[0][kk], wq = pv * vnorm[1][kk];
        const _Float16 wch = (_Float16)wc, wqh = (_Float16)wq;
        pch[kb][r] = wch;
        pcl[kb][r] = (_Float16)(wc - (float)wch);
        psh[kb][r] = wqh;
        psl[kb][r] = (_Float16)(wq - (float)wqh);
      }
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += other_half(psum);
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      om[cb] *= corr;
      oq[cb] *= corr;
    }
    // ---- values: om[cb][r] = A^T[coord cb*16 + 4 (lane >> 4) + r][row lane & 15], 32 keys
    // per product: K slots 8 g .. 8 g + 3 of lane group g are keys 32 j + 4 g + 0..3 and slots
    // 8 g + 4 .. 8 g + 7 keys 32 j + 16 + 4 g + 0..3, so the B operand is this lane's weights
    // of key blocks 2 j and 2 j + 1 as they are
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const h16x8 bch = __builtin_shufflevector(pch[2 * j], pch[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
      const h16x8 bcl = __builtin_shufflevector(pcl[2 * j], pcl[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
      const h16x8 bsh = __builtin_shufflevector(psh[2 * j], psh[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
      const h16x8 bsl = __builtin_shufflevector(psl[2 * j], psl[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const int off = (cb * 16 + (lane & 15)) * kVtStride + 32 * j + 4 * (lane >> 4);
        const h16x8 vh = __builtin_shufflevector(*reinterpret_cast<const h16x4*>(Vh + off),
                                                 *reinterpret_cast<const h16x4*>(Vh + off + 16),
                                                 0, 1, 2, 3, 4, 5, 6, 7);
        const h16x8 vl = __builtin_shufflevector(*reinterpret_cast<const h16x4*>(Vl + off),
                                                 *reinterpret_cast<const h16x4*>(Vl + off + 16),
                                                 0, 1, 2, 3, 4, 5, 6, 7);
        const h16x8 vs = __builtin_shufflevector(*reinterpret_cast<const h16x4*>(Vs + off),
                                                 *reinterpret_cast<const h16x4*>(Vs + off + 16),
                                                 0, 1, 2, 3, 4, 5, 6, 7);
        om[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, bch, om[cb], 0, 0, 0);
        om[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl, bch, om[cb], 0, 0, 0);
        om[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, bcl, om[cb], 0, 0, 0);
        oq[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vs, bsh, oq[cb], 0, 0, 0);
        oq[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vs, bsl, oq[cb], 0, 0, 0);
      }
    }
  }
  // ---- this split's partial of each row, in the decode scan's format
  if (row_ok) {
    const int64_t head = (int64_t)kvh * p.group + (rloc - qi * p.group);
    float* part = p.ws_part + ((qi * p.hq + head) * p.n_split + split) * kPartFloats;
    if ((lane >> 4) == 0) {
      part[0] = m_run;
      part[1] = l_run;
    }
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int coord = cb * 16 + 4 * (lane >> 4) + r;
        part[2 + coord] = om[cb][r] * (1.0f / kPfCent);
        part[2 + kD + coord] = p.gamma * oq[cb][r];
      }
  }
}

}  // namespace tqk

// ---------------------------------------------------------------------------------------
tq_prefill_plan tq_plan_prefill(int32_t n_new, int32_t hq, int32_t hkv, int64_t start) {
  using namespace tqk;
  tq_prefill_plan pl{};
  const int group = hq / hkv;
  const int64_t rows_kvh = (int64_t)n_new * group;
  const int64_t blocks = (rows_kvh + kPfRows - 1) / kPfRows;
  const int64_t keys = start + n_new;
  const int64_t tiles = (keys + kPfKeys - 1) / kPfKeys;
  int64_t n_split = (512 + blocks * hkv - 1) / (blocks * hkv);   // about two workgroups per CU
  if (n_split > tiles) n_split = tiles;
  if (n_split > 256) n_split = 256;
  if (n_split < 1) n_split = 1;
  const int64_t tps = ((tiles + n_split - 1) / n_split) * kPfKeys;
  pl.n_split = (int32_t)n_split;
  pl.keys_per_split = tps;
  pl.row_blocks = blocks;
  pl.ws_q_off = 0;
  pl.ws_part_off = ((int64_t)hkv * rows_kvh * 512 * 2 + 255) / 256 * 256;
  pl.ws_bytes = pl.ws_part_off + (int64_t)n_new * hq * n_split * kPartFloats * 4;
  return pl;
}

int tq_launch_prefill(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                      const tq_tables* tv, const void* q, int32_t q_dtype, int32_t n_new,
                      int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                      const void* codes_v, const uint16_t* norms_v, int32_t page_log2,
                      int64_t num_pages, const int32_t* block_table, int32_t max_blocks,
                      int64_t start, float scale, float* out, void* workspace,
                      const tq_prefill_plan& pl, hipStream_t stream) {
  using namespace tqk;
  const int group = hq / hkv;
  const int64_t rows = (int64_t)hkv * n_new * group;
  char* ws = reinterpret_cast<char*>(workspace);
  _Float16* qop = reinterpret_cast<_Float16*>(ws + pl.ws_q_off);
  const float gamma = (float)(std::sqrt(M_PI / 2.0) / kD);
  PrefillQParams qp{};
  qp.q = q;
  qp.S = tk->S;
  qp.qop = qop;
  qp.rows = rows;
  qp.q_dtype = q_dtype;
  qp.n_new = n_new;
  qp.hq = hq;
  qp.group = group;
  qp.gamma = gamma;
  for (int i = 0; i < 4; ++i) qp.sign[i] = 0;
  for (int j = 0; j < kD; ++j)
    if (tk->signs[j] < 0) qp.sign[j >> 5] |= 1u << (j & 31);
  hipLaunchKernelGGL(prefill_q, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, qp);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;

  PrefillParams p{};
  p.qop = qop;
  p.codes_k = reinterpret_cast<const uint32_t*>(codes_k);
  p.norms_k = reinterpret_cast<const uint32_t*>(norms_k);
  p.codes_v = reinterpret_cast<const uint32_t*>(codes_v);
  p.norms_v = reinterpret_cast<const uint32_t*>(norms_v);
  p.block_table = block_table;
  p.ws_part = reinterpret_cast<float*>(ws + pl.ws_part_off);
  p.num_pages = num_pages;
  p.start = start;
  p.keys_per_split = pl.keys_per_split;
  p.page_log2 = page_log2;
  p.max_blocks = max_blocks;
  p.n_new = n_new;
  p.hq = hq;
  p.hkv = hkv;
  p.group = group;
  p.n_split = pl.n_split;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.gamma = gamma;
  p.kw = (int)(tq_record_bytes(fk) / 4);
  p.ksb = fk->split / 32;
  p.kblo = fk->bits_lo;
  p.kbhi = fk->split == fk->d ? fk->bits_lo : fk->bits_hi;
  p.vw = (int)(tq_record_bytes(fv) / 4);
  p.vsb = fv->split / 32;
  p.vblo = fv->bits_lo;
  p.vbhi = fv->split == fv->d ? fv->bits_lo : fv->bits_hi;
  p.vq = fv->qjl;
  for (int i = 0; i < 8; ++i) {
    p.cent_k[i] = i < (1 << p.kblo) ? tk->centroids_lo[i] : 0.0f;
    p.cent_k[8 + i] = i < (1 << p.kbhi) ? tk->centroids_hi[i] : 0.0f;
    p.cent_v[i] = i < (1 << p.vblo) ? tv->centroids_lo[i] : 0.0f;
    p.cent_v[8 + i] = i < (1 << p.vbhi) ? tv->centroids_hi[i] : 0.0f;
  }
  const dim3 grid((unsigned)pl.row_blocks, (unsigned)hkv, (unsigned)pl.n_split);
  hipLaunchKernelGGL(prefill_scan, grid, dim3(kPfThreads), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;

  DecodeParams cp{};
  cp.S_v = tv->S;
  cp.out = out;
  cp.ws_part = p.ws_part;
  cp.n_split = pl.n_split;
  for (int i = 0; i < 4; ++i) cp.sign_v[i] = 0;
  for (int j = 0; j < kD; ++j)
    if (tv->signs[j] < 0) cp.sign_v[j >> 5] |= 1u << (j & 31);
  return launch_decode_combine(cp, n_new * hq, stream);
}
