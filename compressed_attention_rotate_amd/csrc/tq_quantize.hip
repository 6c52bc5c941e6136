// Quantize kernel: rotation -> norm -> per-coordinate Lloyd-Max encode -> residual ->
// QJL sign sketch -> block-32 packing.  One wave owns a tile of 32 vectors.
//
// What is computed (163.com explainer, m.163.com/dy/article/KOV7P8JI0556C3J2):
//   section "第一步：PolarQuant": rotate, keep one norm, encode every rotated coordinate of
//     the unit direction with the stored scalar codebook (b - 1 bits);
//   section "第二步：QJL": project the residual with a Gaussian JL matrix, keep the signs.
// The rotation is a random sign flip followed by a Walsh-Hadamard transform (zhidx
// turboquant_plus article, section "01 turboquant_plus：介绍与详解"), done here as an
// in-register / cross-lane FWHT.
//
// Phase 1 (VALU), two vectors per pass, one per 32-lane half: lane c holds coordinates
//   32*s + c (s = 0 .. D/32-1), so the FWHT stages on coordinate bits 5.. are in-lane and
//   bits 0..4 are DPP / ds_swizzle butterflies, and a ballot over one compare yields a
//   code bit-plane word of both vectors at once.  ||x|| is accumulated in fp64 (so the
//   fp16 norm is correctly rounded); the rotation, codes and residual run in fp32.
// Phase 2 (MFMA): U = R^ . S^T for the 32-vector tile with v_mfma_f32_32x32x2f32; the
//   32 x 32 output block of N-tile nt holds, per accumulator register, the sign words of
//   two vectors for block nt, extracted with one ballot.  Entries with |u| < 1e-5 (fp32
//   accumulation error is ~1e-7) are recomputed in fp64 from x so the stored sign is the
//   sign of the exact projection.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kGuard = 1e-5f;   // fp32 projections below this are rechecked in fp64
constexpr float kWindow = 1e-6f;  // ambiguity window reported through the counters

// LDS word offset of element (row, col) of a [rows][D] fp32 tile, 16-byte units XOR-
// swizzled by (row & 7) so that 32 lanes reading one column chunk of 32 rows hit
// distinct banks.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  return row * D + ((((col >> 2) ^ (row & 7))) << 2) + (col & 3);
}

template <int D>
struct QCfg {
  static constexpr int NB = D / 32;           // blocks (= slots per lane)
  static constexpr int NW = (D == 128) ? 4 : 2;  // waves per workgroup
  static constexpr bool kResidentS = (D == 128);
  static constexpr int kSRows = kResidentS ? D : 32;
};

// Per-wave LDS footprint (floats / words).
template <int D>
__host__ __device__ constexpr int wave_lds_words() {
  return 32 * D /*rhat tile*/ + 32 * 32 /*record staging (<= 32 words per vector)*/ + 32 /*norms*/;
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
  int64_t ld_x;
  int32_t d_in;
  int32_t x_dtype;
  int32_t split_blocks;  // blocks using the lo table
  int32_t words;         // words per vector
  uint32_t sign_mask[8]; // bit j set: coordinate j is multiplied by -1
  float cpos_lo[8], tpos_lo[8], cpos_hi[8], tpos_hi[8];  // positive halves; tpos[0] unused
  float cent_lo[16], cent_hi[16];
};

// Encode one slot (block) of the two vectors of this pass: returns the (signed) centroid
// of this lane's coordinate and deposits the B code-plane words of both vectors into
// `myword` (lane L of half h receives word L of that half's vector).
template <int B>
__device__ __forceinline__ float encode_slot(float z, const float* cpos_lds, const float* tpos,
                                             int off, uint32_t& myword, int& amb) {
  constexpr int H = Thermo<B>::H;
  const bool pos = z > 0.0f;
  // a' = |z|, nudged to the next float up when z <= 0 so that one strict compare
  // t_j < a' realises idx = #{m : t_m < z} for both signs (ties go to the lower cell)
  const float a = as_f(as_u(fabsf(z)) + (pos ? 0u : 1u));
  uint64_t T[H > 1 ? H : 2];
  int k = 0;
  float dmin = fabsf(z);
#pragma unroll
  for (int j = 1; j < H; ++j) {
    const bool cj = tpos[j] < a;
    T[j] = __ballot(cj);
    k += cj ? 1 : 0;
    dmin = fminf(dmin, fabsf(fabsf(z) - tpos[j]));
  }
  const float cv = cpos_lds[k];
  const uint64_t P = __ballot(pos);
  uint64_t planes[B];
  planes_from_ballots<B>(T, P, planes);
#pragma unroll
  for (int q = 0; q < B; ++q) {
    myword = deposit(myword, planes[q], off + q);
  }
  amb += dmin < kWindow ? 1 : 0;
  return pos ? cv : -cv;
}

// fp64 recomputation of projection n of local vector m (rare path, whole wave).
template <int D>
__device__ void guard_fix(const QParams& p, int64_t v, int m, int n, const float* S_rows,
                          int s_row0, uint32_t* stage, const uint32_t* stage_norms,
                          const float* cent_lds, int* word_off, int* blk_bits,
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
  // in-lane stages (coordinate bits 6, 7), then lane bits 0..5
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

template <int D, int BLO, int BHI>
__global__ __launch_bounds__(64 * QCfg<D>::NW) __attribute__((amdgpu_waves_per_eu(1, 2))) void quantize_kernel(QParams p) {
  using C = QCfg<D>;
  constexpr int NB = C::NB;
  constexpr int NW = C::NW;
  extern __shared__ float lds[];
  float* S_l = lds;                                   // [kSRows][D] swizzled
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  float* wl = lds + C::kSRows * D + wave * wave_lds_words<D>();
  float* rhat = wl;                                               // [32][D] swizzled
  uint32_t* stage = reinterpret_cast<uint32_t*>(wl + 32 * D);     // [32][32]
  uint32_t* snorm = stage + 32 * 32;                              // [32]
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
  // per-lane sign of the random diagonal for each slot, and butterfly signs per lane bit
  float dsg[NB];
#pragma unroll
  for (int s = 0; s < NB; ++s) dsg[s] = ((p.sign_mask[s] >> c) & 1u) ? -1.0f : 1.0f;
  const float bs1 = (c & 1) ? -1.0f : 1.0f, bs2 = (c & 2) ? -1.0f : 1.0f;
  const float bs4 = (c & 4) ? -1.0f : 1.0f, bs8 = (c & 8) ? -1.0f : 1.0f;
  const float bs16 = (c & 16) ? -1.0f : 1.0f;
  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  const double sqrt_d = sqrt((double)D);
  float tpl[8], tph[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    tpl[k] = p.tpos_lo[k];
    tph[k] = p.tpos_hi[k];
  }

  unsigned long long cnt_amb = 0, cnt_zero = 0, cnt_guard = 0, cnt_ovf = 0;
  const int64_t ntiles = (p.n + 31) / 32;
  const int64_t ngroups = (ntiles + NW - 1) / NW;

  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const int64_t tile = g * NW + wave;
    const int64_t v0 = tile * 32;
    const bool active = tile < ntiles;
    if (active) {
      // ---------------- phase 1: rotation, norm, codes, residual (2 vectors per pass)
      for (int pp = 0; pp < 16; ++pp) {
        const int vloc = 2 * pp + h;
        const int64_t v = v0 + vloc;
        const bool valid = v < p.n;
        float xv[NB];
        double ss = 0.0;
#pragma unroll
        for (int s = 0; s < NB; ++s) {
          const int j = 32 * s + c;
          xv[s] = (valid && j < p.d_in) ? load_elem(p.x, v * p.ld_x + j, p.x_dtype) : 0.0f;
          ss = fma((double)xv[s], (double)xv[s], ss);
          xv[s] *= dsg[s];
        }
        ss = half_sum_d(ss);
#pragma unroll
        for (int hh = 1; hh < NB; hh <<= 1)
#pragma unroll
          for (int s = 0; s < NB; ++s)
            if (!(s & hh)) {
              const float a = xv[s], b = xv[s + hh];
              xv[s] = a + b;
              xv[s + hh] = a - b;
            }
#pragma unroll
        for (int s = 0; s < NB; ++s) {
          float y = xv[s];
          y = butterfly<1>(y, bs1);
          y = butterfly<2>(y, bs2);
          y = butterfly<4>(y, bs4);
          y = butterfly<8>(y, bs8);
          y = butterfly<16>(y, bs16);
          xv[s] = y;  // unnormalized H D x
        }
        const double nrm = sqrt(ss);
        const uint32_t n16 = f64_to_f16_bits(nrm);
        const float n16f = f16_bits_to_f32(n16);
        const float zinv = nrm > 0.0 ? (float)(1.0 / (nrm * sqrt_d)) : 0.0f;
        uint32_t myword = 0;  // lane L (< words) of half h collects word L of vector vloc
        float rsq = 0.0f;
        float r[NB];
        int amb = 0;
#pragma unroll
        for (int s = 0; s < NB; ++s) {
          const float z = xv[s] * zinv;
          const int off = s < p.split_blocks ? s * (BLO + 1)
                                             : p.split_blocks * (BLO + 1) + (s - p.split_blocks) * (BHI + 1);
          const float cv = (s < p.split_blocks) ? encode_slot<BLO>(z, cpos_lds, tpl, off, myword, amb)
                                                : encode_slot<BHI>(z, cpos_lds + 8, tph, off, myword, amb);
          r[s] = fmaf(xv[s], inv_sqrt_d, -n16f * cv);
          rsq = fmaf(r[s], r[s], rsq);
        }
        rsq = half_sum(rsq);
        const float rn = sqrtf(rsq);
        const uint32_t r16 = f32_to_f16_bits(rn);
        const float rinv = rn > 0.0f ? 1.0f / rn : 0.0f;
#pragma unroll
        for (int s = 0; s < NB; ++s) rhat[swz<D>(vloc, 32 * s + c)] = r[s] * rinv;
        if (c < p.words) stage[vloc * 32 + c] = myword;
        if (c == 0) snorm[vloc] = n16 | (r16 << 16);
        if (p.counters) {
          cnt_amb += valid ? (unsigned long long)amb : 0ull;
          if (c == 0 && valid && n16 == 0x7C00u) cnt_ovf += 1;  // lanes 0 and 32
        }
      }
    }
    // ---------------- phase 2: JL projection on MFMA, sign words
    for (int nt = 0; nt < NB; ++nt) {
      if constexpr (!C::kResidentS) {
        __syncthreads();
        for (int i = threadIdx.x; i < 32 * D / 4; i += blockDim.x) {
          const int row = (4 * i) / D, col = (4 * i) % D;
          const f32x4 v = reinterpret_cast<const f32x4*>(p.S + (int64_t)nt * 32 * D)[i];
          *reinterpret_cast<f32x4*>(&S_l[swz<D>(row, col)]) = v;
        }
        __syncthreads();
      }
      if (!active) continue;
      const int s_row0 = C::kResidentS ? 0 : nt * 32;
      const int arow = lane & 31, kh = (lane >> 5) * (D / 2);
      const int brow = nt * 32 + arow - s_row0;
      f32x16 acc = {};
#pragma unroll 4
      for (int kc = 0; kc < D / 8; ++kc) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(&rhat[swz<D>(arow, kh + 4 * kc)]);
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(&S_l[swz<D>(brow, kh + 4 * kc)]);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[0], b4[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[1], b4[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[2], b4[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[3], b4[3], acc, 0, 0, 0);
      }
      // register r of lane l holds u[vector 8(r/4) + 4(l/32) + r%4][32 nt + l%32]
      uint32_t sword = 0;
      uint64_t gmask[16];
      bool any_guard = false;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int m0 = 8 * (rr >> 2) + (rr & 3);
        const uint64_t sg = __ballot(acc[rr] >= 0.0f);
        gmask[rr] = __ballot(fabsf(acc[rr]) < kGuard);
        any_guard |= gmask[rr] != 0;
        if (lane == m0) sword = (uint32_t)sg;
        if (lane == m0 + 4) sword = (uint32_t)(sg >> 32);
      }
      const int sw_off = word_off_s[nt] + blk_bits_s[nt];
      if (lane < 32) stage[lane * 32 + sw_off] = sword;
      if (any_guard) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          uint64_t gm = gmask[rr];
          while (gm) {
            const int L = __builtin_ctzll(gm);
            gm &= gm - 1;
            const int m = 8 * (rr >> 2) + (rr & 3) + ((L >> 5) << 2);
            const int64_t v = v0 + m;
            if (v >= p.n) continue;
            cnt_guard += (lane == 0);
            guard_fix<D>(p, v, m, nt * 32 + (L & 31), S_l, s_row0, stage, snorm, cent_lds,
                         word_off_s, blk_bits_s, cnt_zero);
          }
        }
      }
    }
    if (!active) continue;
    // ---------------- store the tile: records (contiguous) and norms
    const int nvalid = (int)((p.n - v0) < 32 ? (p.n - v0) : 32);
    uint32_t* dst = p.codes + v0 * p.words;
    for (int i = lane; i < nvalid * p.words; i += 64) dst[i] = stage[(i / p.words) * 32 + (i % p.words)];
    if (lane < nvalid) p.norms[v0 + lane] = snorm[lane];
  }
  if (p.counters) {
    // cnt_amb is per lane; the others were counted on lane 0 or uniformly
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
  const size_t lds = sizeof(float) * (size_t)(C::kSRows * D + C::NW * wave_lds_words<D>());
  static bool attr_set = false;  // per template instance
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)quantize_kernel<D, BLO, BHI>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return TQ_ERR_HIP;
    attr_set = true;
  }
  const int64_t ntiles = (p.n + 31) / 32;
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
