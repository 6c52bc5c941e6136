// Quantize kernel: rotation -> norm -> per-coordinate Lloyd-Max encode -> residual ->
// QJL sign sketch -> block-32 packing.  One wave owns a tile of 16 vectors at a time.
//
// What is computed (163.com explainer, m.163.com/dy/article/KOV7P8JI0556C3J2):
//   section "第一步：PolarQuant": rotate, keep one norm, encode every rotated coordinate of
//     the unit direction with the stored scalar codebook (b - 1 bits);
//   section "第二步：QJL": project the residual with a Gaussian JL matrix, keep the signs.
// The rotation is a random sign flip followed by a Walsh-Hadamard transform (zhidx
// turboquant_plus article, section "01 turboquant_plus：介绍与详解"), done here as an
// in-register / cross-lane FWHT.
//
// Per tile:
//   staging:  the 16 input rows arrive in LDS through coalesced 16-byte loads; the next
//             tile's rows are fetched into registers while this tile is on the MFMA pipe.
//   phase 1 (VALU): two vectors per pass, one per 32-lane half, two passes interleaved.
//             Lane c holds coordinates 32*s + c (s = 0 .. D/32-1), so FWHT stages on
//             coordinate bits >= 5 are in-lane and bits 0..4 are DPP / ds_swizzle
//             butterflies, and one ballot per compare yields a code bit-plane word of both
//             vectors.  ||x|| is accumulated in fp64 (so the fp16 norm is correctly
//             rounded); rotation, codes and residual run in fp32.
//   phase 2 (MFMA): U = R^ S^T with v_mfma_f32_16x16x4f32 (the d x d projection is the
//             one dense contraction of the path); each 16x16 accumulator block gives sign
//             bits by ballot.  Entries with |u| < 1e-5 (fp32 error is ~1e-7) are recomputed
//             in fp64 from x, so every stored sign is the sign of the exact projection.
// With 8 waves per workgroup (2 per SIMD) one wave's VALU phase overlaps another's MFMA.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kGuard = 1e-5f;   // fp32 projections below this are rechecked in fp64
constexpr float kWindow = 1e-6f;  // ambiguity window reported through the counters

template <int D>
struct QCfg {
  static constexpr int NB = D / 32;                  // 32-coordinate blocks
  static constexpr int TV = 16;                      // vectors per wave tile
  static constexpr int NW = (D == 128) ? 8 : 4;      // waves per workgroup
  static constexpr bool kResidentS = (D == 128);     // S stays in LDS (else 32-row slices)
  static constexpr int kSRows = kResidentS ? D : 32;
  static constexpr int kWaveF = TV * D + TV * 32 + TV;  // rhat/input, record staging, norms
  static constexpr int MAXC = TV * D * 4 / 16 / 64;     // 16-byte input chunks per lane
  static constexpr int PG = 2;                          // passes interleaved in phase 1
};

// LDS word offset of element (row, col) of a [rows][D] fp32 tile; 16-byte units are XOR-
// swizzled by (row & 15) so 16 lanes reading the same column chunk of 16 rows (MFMA
// operand reads) hit distinct banks.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  return row * D + ((((col >> 2) ^ (row & 15))) << 2) + (col & 3);
}

template <int B>
struct Thermo {
  static constexpr int H = 1 << (B - 1);  // positive centroids
};

// Code plane words from the thermometer ballots T[1..H-1] and the sign ballot P:
// idx = P ? H + k : H - 1 - k, k = #{j : t_j < |z|}.  Bit q of k is the XOR of T_j over
// the multiples j of 2^q; plane q (< B-1) is that bit, complemented when z <= 0; plane
// B-1 is P.
template <int B>
__device__ __forceinline__ void planes_from_ballots(const uint64_t (&T)[(1 << (B - 1)) > 1 ? (1 << (B - 1)) : 2],
                                                    uint64_t P, uint64_t (&out)[B]) {
  constexpr int H = Thermo<B>::H;
#pragma unroll
  for (int q = 0; q + 1 < B; ++q) {
    uint64_t k = 0;
#pragma unroll
    for (int j = (1 << q); j < H; j += (1 << q)) k ^= T[j];
    out[q] = ~(k ^ P);
  }
  out[B - 1] = P;
}

struct QParams {
  const void* x;
  const float* S;
  uint32_t* codes;
  uint32_t* norms;
  unsigned long long* counters;
  int64_t n;
  int64_t ld_x;          // elements
  int32_t d_in;
  int32_t x_dtype;
  int32_t esize;         // bytes per input element
  int32_t staged;        // rows are 16-byte aligned with a 16-byte multiple of valid bytes
  int32_t cpr;           // 16-byte chunks per row (staged path)
  int32_t split_blocks;  // blocks using the lo table
  int32_t words;         // words per vector
  uint32_t sign_mask[8]; // bit j set: coordinate j is multiplied by -1
  float cpos_lo[8], tpos_lo[8], cpos_hi[8], tpos_hi[8];  // positive halves; tpos[0] unused
  float cent_lo[16], cent_hi[16];
};

// Encode one slot (block) of the two vectors of a pass: returns the signed centroid of
// this lane's coordinate and deposits the B code-plane words of both vectors into `myword`
// (lane L of half h receives word L of that half's vector).
template <int B>
__device__ __forceinline__ float encode_slot(float z, const float* cpos_lds, const float* tpos,
                                             int off, uint32_t& myword, int& amb, bool count) {
  constexpr int H = Thermo<B>::H;
  const bool pos = z > 0.0f;
  // a' = |z|, nudged to the next float up when z <= 0 so that one strict compare
  // t_j < a' realises idx = #{m : t_m < z} for both signs (ties go to the lower cell)
  const float az = fabsf(z);
  const float a = as_f(as_u(az) + (pos ? 0u : 1u));
  uint64_t T[H > 1 ? H : 2];
  int k = 0;
#pragma unroll
  for (int j = 1; j < H; ++j) {
    const bool cj = tpos[j] < a;
    T[j] = __ballot(cj);
    k += cj ? 1 : 0;
  }
  const float cv = cpos_lds[k];
  const uint64_t P = __ballot(pos);
  uint64_t planes[B];
  planes_from_ballots<B>(T, P, planes);
#pragma unroll
  for (int q = 0; q < B; ++q) myword = deposit(myword, planes[q], off + q);
  if (count) {
    float dmin = az;
#pragma unroll
    for (int j = 1; j < H; ++j) dmin = fminf(dmin, fabsf(az - tpos[j]));
    amb += dmin < kWindow ? 1 : 0;
  }
  return pos ? cv : -cv;
}

// fp64 recomputation of projection n of local vector m (rare path, whole wave).
template <int D>
__device__ void guard_fix(const QParams& p, int64_t v, int m, int n, const float* S_rows,
                          int s_row0, uint32_t* stage, const uint32_t* stage_norms,
                          const float* cent_lds, const int* word_off, const int* blk_bits,
                          unsigned long long& cnt_zero) {
  constexpr int NE = D / 64;
  const int lane = lane_id();
  double xd[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int j = lane + 64 * e;
    float xv = (j < p.d_in) ? load_elem(p.x, v * p.ld_x + j, p.x_dtype) : 0.0f;
    if ((p.sign_mask[j >> 5] >> (j & 31)) & 1u) xv = -xv;
    xd[e] = (double)xv;
  }
#pragma unroll
  for (int h = 1; h < NE; h <<= 1)
#pragma unroll
    for (int e = 0; e < NE; ++e)
      if (!(e & h)) {
        double a = xd[e], b = xd[e + h];
        xd[e] = a + b;
        xd[e + h] = a - b;
      }
#pragma unroll
  for (int mm = 1; mm < 64; mm <<= 1)
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      double t = shfl_xor_d(xd[e], mm);
      xd[e] = (lane & mm) ? t - xd[e] : xd[e] + t;
    }
  const double isd = 1.0 / sqrt((double)D);
  const double n16 = (double)f16_bits_to_f32(stage_norms[m] & 0xFFFFu);
  double dot = 0.0, rr = 0.0;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int j = lane + 64 * e;
    const int blk = j >> 5, bit = j & 31;
    int idx = 0;
    for (int q = 0; q < blk_bits[blk]; ++q) idx |= ((stage[m * 32 + word_off[blk] + q] >> bit) & 1u) << q;
    const float c = cent_lds[(blk < p.split_blocks ? 0 : 16) + idx];
    const double r = xd[e] * isd - n16 * (double)c;
    dot += (double)S_rows[swz<D>(n - s_row0, j)] * r;
    rr += r * r;
  }
  dot = wave_sum_d(dot);
  rr = wave_sum_d(rr);
  if (lane == 0) {
    uint32_t* w = &stage[m * 32 + word_off[n >> 5] + blk_bits[n >> 5]];
    const uint32_t bitmask = 1u << (n & 31);
    *w = (dot >= 0.0) ? (*w | bitmask) : (*w & ~bitmask);
  }
  if (rr == 0.0 || fabs(dot) < (double)kWindow * sqrt(rr)) cnt_zero += 1;
}

// Input chunk plan of one lane (fixed for every tile): global byte offset inside the tile
// and LDS byte offset of each 16-byte chunk it moves; -1 = no chunk.
template <int D>
struct ChunkPlan {
  int64_t goff[QCfg<D>::MAXC];
  int loff[QCfg<D>::MAXC];
  int row[QCfg<D>::MAXC];
};

template <int D>
__device__ __forceinline__ void fetch_tile(const QParams& p, const ChunkPlan<D>& cp, int64_t v0,
                                           u32x4 (&buf)[QCfg<D>::MAXC]) {
  const char* base = reinterpret_cast<const char*>(p.x) + v0 * p.ld_x * p.esize;
#pragma unroll
  for (int i = 0; i < QCfg<D>::MAXC; ++i) {
    if (cp.loff[i] >= 0 && v0 + cp.row[i] < p.n)
      buf[i] = *reinterpret_cast<const u32x4*>(base + cp.goff[i]);
  }
}

template <int D>
__device__ __forceinline__ void stash_tile(const ChunkPlan<D>& cp, const u32x4 (&buf)[QCfg<D>::MAXC],
                                           float* tile) {
#pragma unroll
  for (int i = 0; i < QCfg<D>::MAXC; ++i)
    if (cp.loff[i] >= 0) *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(tile) + cp.loff[i]) = buf[i];
}

template <int D, int BLO, int BHI>
__global__ __launch_bounds__(64 * QCfg<D>::NW) void quantize_kernel(QParams p) {
  using C = QCfg<D>;
  constexpr int NB = C::NB;
  constexpr int NW = C::NW;
  constexpr int TV = C::TV;
  constexpr int PG = C::PG;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  float* S_l = lds;                                   // [kSRows][D] swizzled
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  float* wl = lds + C::kSRows * D + wave * C::kWaveF;
  float* rhat = wl;                                               // [TV][D]: input, then rhat
  uint32_t* stage = reinterpret_cast<uint32_t*>(wl + TV * D);     // [TV][32] record words
  uint32_t* snorm = stage + TV * 32;                              // [TV]
  __shared__ float cent_lds[32];
  __shared__ float cpos_lds[16];  // positive centroids: lo table, then hi table
  __shared__ int word_off_s[8], blk_bits_s[8];

  if (threadIdx.x < 16) {
    cent_lds[threadIdx.x] = p.cent_lo[threadIdx.x];
    cent_lds[16 + threadIdx.x] = p.cent_hi[threadIdx.x];
    cpos_lds[threadIdx.x] = threadIdx.x < 8 ? p.cpos_lo[threadIdx.x] : p.cpos_hi[threadIdx.x - 8];
  }
  if (threadIdx.x == 0) {
    int off = 0;
    for (int b = 0; b < NB; ++b) {
      const int bb = b < p.split_blocks ? BLO : BHI;
      word_off_s[b] = off;
      blk_bits_s[b] = bb;
      off += bb + 1;
    }
  }
  if constexpr (C::kResidentS) {
    for (int i = threadIdx.x; i < D * D / 4; i += blockDim.x) {
      const int row = (4 * i) / D, col = (4 * i) % D;
      const f32x4 v = reinterpret_cast<const f32x4*>(p.S)[i];
      *reinterpret_cast<f32x4*>(&S_l[swz<D>(row, col)]) = v;
    }
  }
  __syncthreads();

  const int h = lane >> 5, c = lane & 31;
  float dsg[NB];
#pragma unroll
  for (int s = 0; s < NB; ++s) dsg[s] = ((p.sign_mask[s] >> c) & 1u) ? -1.0f : 1.0f;
  const float bs1 = (c & 1) ? -1.0f : 1.0f, bs2 = (c & 2) ? -1.0f : 1.0f;
  const float bs4 = (c & 4) ? -1.0f : 1.0f, bs8 = (c & 8) ? -1.0f : 1.0f;
  const float bs16 = (c & 16) ? -1.0f : 1.0f;
  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  const float sqrt_d = sqrtf((float)D);
  float tpl[8], tph[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    tpl[k] = p.tpos_lo[k];
    tph[k] = p.tpos_hi[k];
  }
  const bool count = p.counters != nullptr;

  // per-lane input chunk plan (the same for every tile)
  ChunkPlan<D> cp;
#pragma unroll
  for (int i = 0; i < C::MAXC; ++i) {
    const int ci = lane + 64 * i;
    const int row = p.staged ? ci / p.cpr : 0;
    const int cc = p.staged ? ci % p.cpr : 0;
    const bool ok = p.staged && row < TV;
    cp.row[i] = row;
    cp.goff[i] = (int64_t)row * p.ld_x * p.esize + 16 * cc;
    cp.loff[i] = ok ? row * D * 4 + 16 * cc : -1;
  }

  unsigned long long cnt_amb = 0, cnt_zero = 0, cnt_guard = 0, cnt_ovf = 0;
  const int64_t ntiles = (p.n + TV - 1) / TV;
  const int64_t ngroups = (ntiles + NW - 1) / NW;
  u32x4 pre[C::MAXC];

  int64_t g = blockIdx.x;
  if (p.staged && g < ngroups && g * NW + wave < ntiles) fetch_tile<D>(p, cp, (g * NW + wave) * TV, pre);

  for (; g < ngroups; g += gridDim.x) {
    const int64_t tile = g * NW + wave;
    const int64_t v0 = tile * TV;
    const bool active = tile < ntiles;
    if (active) {
      if (p.staged) stash_tile<D>(cp, pre, rhat);
      // ---------------- phase 1: rotation, norm, codes, residual (PG passes at once)
      for (int pp0 = 0; pp0 < TV / 2; pp0 += PG) {
        float xv[PG][NB];
        double ss[PG];
        bool valid[PG];
        int vloc[PG];
#pragma unroll
        for (int gg = 0; gg < PG; ++gg) {
          vloc[gg] = 2 * (pp0 + gg) + h;
          const int64_t v = v0 + vloc[gg];
          valid[gg] = v < p.n;
          ss[gg] = 0.0;
#pragma unroll
          for (int s = 0; s < NB; ++s) {
            const int j = 32 * s + c;
            float x = 0.0f;
            if (valid[gg] && j < p.d_in) {
              if (p.staged) {
                const char* rowp = reinterpret_cast<const char*>(rhat) + vloc[gg] * D * 4;
                if (p.x_dtype == 0) x = *reinterpret_cast<const float*>(rowp + 4 * j);
                else {
                  const uint32_t hb = *reinterpret_cast<const uint16_t*>(rowp + 2 * j);
                  x = (p.x_dtype == 1) ? __uint_as_float(hb << 16) : f16_bits_to_f32(hb);
                }
              } else {
                x = load_elem(p.x, v * p.ld_x + j, p.x_dtype);
              }
            }
            ss[gg] = fma((double)x, (double)x, ss[gg]);
            xv[gg][s] = x * dsg[s];
          }
        }
#pragma unroll
        for (int gg = 0; gg < PG; ++gg) {
          ss[gg] = half_sum_d(ss[gg]);
#pragma unroll
          for (int hh = 1; hh < NB; hh <<= 1)
#pragma unroll
            for (int s = 0; s < NB; ++s)
              if (!(s & hh)) {
                const float a = xv[gg][s], b = xv[gg][s + hh];
                xv[gg][s] = a + b;
                xv[gg][s + hh] = a - b;
              }
        }
#pragma unroll
        for (int s = 0; s < NB; ++s)
#pragma unroll
          for (int gg = 0; gg < PG; ++gg) xv[gg][s] = butterfly<1>(xv[gg][s], bs1);
#pragma unroll
        for (int s = 0; s < NB; ++s)
#pragma unroll
          for (int gg = 0; gg < PG; ++gg) xv[gg][s] = butterfly<2>(xv[gg][s], bs2);
#pragma unroll
        for (int s = 0; s < NB; ++s)
#pragma unroll
          for (int gg = 0; gg < PG; ++gg) xv[gg][s] = butterfly<4>(xv[gg][s], bs4);
#pragma unroll
        for (int s = 0; s < NB; ++s)
#pragma unroll
          for (int gg = 0; gg < PG; ++gg) xv[gg][s] = butterfly<8>(xv[gg][s], bs8);
#pragma unroll
        for (int s = 0; s < NB; ++s)
#pragma unroll
          for (int gg = 0; gg < PG; ++gg) xv[gg][s] = butterfly<16>(xv[gg][s], bs16);

        float r[PG][NB];
        float rsq[PG];
        uint32_t n16[PG];
#pragma unroll
        for (int gg = 0; gg < PG; ++gg) {
          const double nrm = sqrt(ss[gg]);
          n16[gg] = f64_to_f16_bits(nrm);
          const float n16f = f16_bits_to_f32(n16[gg]);
          const float nf = (float)nrm;
          const float zinv = nf > 0.0f ? __builtin_amdgcn_rcpf(nf * sqrt_d) : 0.0f;
          uint32_t myword = 0;
          int amb = 0;
          rsq[gg] = 0.0f;
#pragma unroll
          for (int s = 0; s < NB; ++s) {
            const float z = xv[gg][s] * zinv;
            const int off = s < p.split_blocks ? s * (BLO + 1)
                                               : p.split_blocks * (BLO + 1) + (s - p.split_blocks) * (BHI + 1);
            const float cv = (s < p.split_blocks)
                                 ? encode_slot<BLO>(z, cpos_lds, tpl, off, myword, amb, count)
                                 : encode_slot<BHI>(z, cpos_lds + 8, tph, off, myword, amb, count);
            r[gg][s] = fmaf(xv[gg][s], inv_sqrt_d, -n16f * cv);
            rsq[gg] = fmaf(r[gg][s], r[gg][s], rsq[gg]);
          }
          if (c < p.words) stage[vloc[gg] * 32 + c] = myword;
          if (count) cnt_amb += valid[gg] ? (unsigned long long)amb : 0ull;
        }
#pragma unroll
        for (int gg = 0; gg < PG; ++gg) {
          const float rs = half_sum(rsq[gg]);
          const float rn = sqrtf(rs);
          const uint32_t r16 = f32_to_f16_bits(rn);
          const float rinv = rn > 0.0f ? 1.0f / rn : 0.0f;
#pragma unroll
          for (int s = 0; s < NB; ++s) rhat[swz<D>(vloc[gg], 32 * s + c)] = r[gg][s] * rinv;
          if (c == 0) snorm[vloc[gg]] = n16[gg] | (r16 << 16);
          if (count && c == 0 && valid[gg] && n16[gg] == 0x7C00u) cnt_ovf += 1;  // lanes 0, 32
        }
      }
      // next tile's input is fetched while this one is on the MFMA pipe
      const int64_t gn = g + gridDim.x;
      if (p.staged && gn < ngroups && gn * NW + wave < ntiles) fetch_tile<D>(p, cp, (gn * NW + wave) * TV, pre);
    }
    // ---------------- phase 2: JL projection on MFMA, sign words (one block per step)
    for (int blk = 0; blk < NB; ++blk) {
      if constexpr (!C::kResidentS) {
        __syncthreads();
        for (int i = threadIdx.x; i < 32 * D / 4; i += blockDim.x) {
          const int row = (4 * i) / D, col = (4 * i) % D;
          const f32x4 v = reinterpret_cast<const f32x4*>(p.S + (int64_t)blk * 32 * D)[i];
          *reinterpret_cast<f32x4*>(&S_l[swz<D>(row, col)]) = v;
        }
        __syncthreads();
      }
      if (!active) continue;
      const int s_row0 = C::kResidentS ? 0 : blk * 32;
      const int arow = lane & 15, kg = (lane >> 4) * (D / 4);
      f32x4 acc0 = {}, acc1 = {};
      const int brow0 = blk * 32 + arow - s_row0;
#pragma unroll 4
      for (int kc = 0; kc < D / 16; ++kc) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(&rhat[swz<D>(arow, kg + 4 * kc)]);
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(&S_l[swz<D>(brow0, kg + 4 * kc)]);
        const f32x4 c4 = *reinterpret_cast<const f32x4*>(&S_l[swz<D>(brow0 + 16, kg + 4 * kc)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[i], b4[i], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[i], c4[i], acc1, 0, 0, 0);
        }
      }
      // acc_t[r] of lane l: u[vector 4(l/16) + r][32 blk + 16 t + l%16]
      uint64_t sg0[4], sg1[4];
      bool any_guard = false;
      uint64_t gm0[4], gm1[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        sg0[rr] = __ballot(acc0[rr] >= 0.0f);
        sg1[rr] = __ballot(acc1[rr] >= 0.0f);
        gm0[rr] = __ballot(fabsf(acc0[rr]) < kGuard);
        gm1[rr] = __ballot(fabsf(acc1[rr]) < kGuard);
        any_guard |= (gm0[rr] | gm1[rr]) != 0;
      }
      // lane v (< 16) assembles the sign word of vector v for this block
      uint32_t sword = 0;
      const int vq = lane & 3, vsh = 16 * ((lane >> 2) & 3);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint32_t w = (uint32_t)((sg0[rr] >> vsh) & 0xFFFFu) |
                           ((uint32_t)((sg1[rr] >> vsh) & 0xFFFFu) << 16);
        sword = (vq == rr) ? w : sword;
      }
      const int sw_off = word_off_s[blk] + blk_bits_s[blk];
      if (lane < TV) stage[lane * 32 + sw_off] = sword;
      if (any_guard) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            uint64_t gm = t ? gm1[rr] : gm0[rr];
            while (gm) {
              const int L = __builtin_ctzll(gm);
              gm &= gm - 1;
              const int m = 4 * (L >> 4) + rr;
              const int64_t v = v0 + m;
              if (v >= p.n) continue;
              cnt_guard += (lane == 0);
              guard_fix<D>(p, v, m, blk * 32 + 16 * t + (L & 15), S_l, s_row0, stage, snorm,
                           cent_lds, word_off_s, blk_bits_s, cnt_zero);
            }
          }
      }
    }
    if (!active) continue;
    // ---------------- store the tile: records (contiguous) and norms
    const int nvalid = (int)((p.n - v0) < TV ? (p.n - v0) : TV);
    uint32_t* dst = p.codes + v0 * p.words;
    for (int i = lane; i < nvalid * p.words; i += 64) dst[i] = stage[(i / p.words) * 32 + (i % p.words)];
    if (lane < nvalid) p.norms[v0 + lane] = snorm[lane];
  }
  if (count) {
    unsigned long long tot = cnt_amb, ovf = cnt_ovf;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      tot += __shfl_xor(tot, m, 64);
      ovf += __shfl_xor(ovf, m, 64);
    }
    if (lane == 0) {
      if (tot) atomicAdd(&p.counters[0], tot);
      if (cnt_zero) atomicAdd(&p.counters[1], cnt_zero);
      if (cnt_guard) atomicAdd(&p.counters[2], cnt_guard);
      if (ovf) atomicAdd(&p.counters[3], ovf);
    }
  }
}

template <int D, int BLO, int BHI>
static int launch_quantize(const QParams& p, hipStream_t stream, int num_cu) {
  using C = QCfg<D>;
  const size_t lds = sizeof(float) * (size_t)(C::kSRows * D + C::NW * C::kWaveF);
  static bool attr_set = false;  // per template instance
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)quantize_kernel<D, BLO, BHI>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return TQ_ERR_HIP;
    attr_set = true;
  }
  const int64_t ntiles = (p.n + C::TV - 1) / C::TV;
  const int64_t ngroups = (ntiles + C::NW - 1) / C::NW;
  const int64_t grid = ngroups < (int64_t)num_cu ? ngroups : (int64_t)num_cu;
  hipLaunchKernelGGL((quantize_kernel<D, BLO, BHI>), dim3((unsigned)grid), dim3(64 * C::NW), lds,
                     stream, p);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

}  // namespace tqk

// ---------------------------------------------------------------------------------------
int tq_launch_quantize(const tq_format* f, const tq_tables* t, const void* x, int32_t x_dtype,
                       int64_t n, int32_t d_in, int64_t ld_x, void* codes, uint16_t* norms,
                       int64_t* counters, hipStream_t stream) {
  using namespace tqk;
  QParams p{};
  p.x = x;
  p.S = t->S;
  p.codes = reinterpret_cast<uint32_t*>(codes);
  p.norms = reinterpret_cast<uint32_t*>(norms);
  p.counters = reinterpret_cast<unsigned long long*>(counters);
  p.n = n;
  p.ld_x = ld_x;
  p.d_in = d_in;
  p.x_dtype = x_dtype;
  p.esize = x_dtype == TQ_F32 ? 4 : 2;
  const int64_t row_bytes = (int64_t)d_in * p.esize;
  p.staged = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && ((ld_x * p.esize) % 16 == 0) &&
             (row_bytes % 16 == 0);
  p.cpr = p.staged ? (int32_t)(row_bytes / 16) : 1;
  p.split_blocks = f->split / 32;
  p.words = (int)(tq_record_bytes(f) / 4);
  for (int j = 0; j < 8; ++j) p.sign_mask[j] = 0;
  for (int j = 0; j < f->d; ++j)
    if (t->signs[j] < 0) p.sign_mask[j >> 5] |= 1u << (j & 31);
  auto fill = [](int bits, const float* cent, const float* bnd, float* cpos, float* tpos, float* full) {
    const int H = 1 << (bits - 1);
    for (int k = 0; k < 8; ++k) cpos[k] = tpos[k] = 0.0f;
    for (int k = 0; k < H; ++k) cpos[k] = cent[H + k];
    for (int k = 1; k < H; ++k) tpos[k] = bnd[H + k - 1];
    for (int k = 0; k < 16; ++k) full[k] = k < (1 << bits) ? cent[k] : 0.0f;
  };
  fill(f->bits_lo, t->centroids_lo, t->bounds_lo, p.cpos_lo, p.tpos_lo, p.cent_lo);
  fill(f->bits_hi, t->centroids_hi, t->bounds_hi, p.cpos_hi, p.tpos_hi, p.cent_hi);
  const int ncu = tq_num_cus();
  if (ncu <= 0) return TQ_ERR_HIP;
  const int lo = f->bits_lo, hi = f->bits_hi;
  if (f->d == 128) {
    if (lo == 1 && hi == 1) return launch_quantize<128, 1, 1>(p, stream, ncu);
    if (lo == 2 && hi == 2) return launch_quantize<128, 2, 2>(p, stream, ncu);
    if (lo == 3 && hi == 3) return launch_quantize<128, 3, 3>(p, stream, ncu);
    if (lo == 3 && hi == 2) return launch_quantize<128, 3, 2>(p, stream, ncu);
    if (lo == 2 && hi == 1) return launch_quantize<128, 2, 1>(p, stream, ncu);
  } else if (f->d == 256) {
    if (lo == 2 && hi == 2) return launch_quantize<256, 2, 2>(p, stream, ncu);
    if (lo == 3 && hi == 3) return launch_quantize<256, 3, 3>(p, stream, ncu);
  }
  return TQ_ERR_SHAPE;
}
