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
// A format without QJL (MSE-only) skips the residual split and phase 2; ||r|| is still
// stored.
//
// Per tile:
//   staging:  the 16 input rows arrive in LDS through coalesced 16-byte loads; the next
//             tile's rows are fetched into registers while this tile is on the MFMA pipe.
//   phase 1 (VALU): two vectors per pass, one per 32-lane half, two passes interleaved.
//             Lane c holds coordinates 32*s + c (s = 0 .. D/32-1), so FWHT stages on
//             coordinate bits >= 5 are in-lane and bits 0..4 are DPP / ds_swizzle
//             butterflies.  One ballot per compare yields a code bit-plane word of both
//             vectors; lane 0 drops the 64-bit ballots into an LDS table and the records
//             are assembled from it when the tile is stored.  ||x|| is accumulated in fp64
//             (so the fp16 norm is correctly rounded); rotation, codes and residual run in
//             fp32.  The unit residual is split into fp16 hi + lo (scaled by 2^12).
//   phase 2 (MFMA): U = R^ S^T, the one dense contraction of the path, as three fp16
//             products (hi.hi + hi.lo + lo.hi, S scaled by 2^10 and split the same way) on
//             v_mfma_f32_16x16x32_f16 with fp32 accumulation: relative error ~2^-22 per
//             term.  Sign bits come from ballots over each 16x16 accumulator block; every
//             entry with |u| < 1e-5 is recomputed in fp64 from x, so each stored sign is the
//             sign of the exact projection.
// With 8 waves per workgroup (2 per SIMD) one wave's VALU phase overlaps another's MFMA.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tq_device.h"
#include "tq_internal.h"

namespace tqk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kGuard = 1e-5f;   // projections below this are rechecked in fp64
constexpr float kWindow = 1e-6f;  // ambiguity window reported through the counters
constexpr float kRScale = 4096.0f;   // unit residual scale before the fp16 split
constexpr float kSScale = 1024.0f;   // S scale before the fp16 split
constexpr float kUScale = kRScale * kSScale;

template <int D>
struct QCfg {
  static constexpr int NB = D / 32;                  // 32-coordinate blocks
  static constexpr int TV = 16;                      // vectors per wave tile
  static constexpr int NW = (D == 128) ? 8 : 4;      // waves per workgroup
  static constexpr bool kResidentS = (D == 128);     // S stays in LDS (else 32-row slices)
  static constexpr int kSRows = kResidentS ? D : 32;
  static constexpr int kRowB = 4 * D;                // bytes of one [hi | lo] fp16 row
  static constexpr int kBal = (TV / 2) * NB * 4;     // code-plane ballots per tile (uint64)
  static constexpr int kSBal = NB * 8;               // sign ballots per tile (uint64)
  // per wave: r^ tile (doubles as input staging), ballots, sign ballots, norms
  static constexpr int kWaveB = TV * kRowB + 8 * (kBal + kSBal) + 4 * TV;
  static constexpr int MAXC = TV * D * 4 / 16 / 64;  // 16-byte input chunks per lane
  static constexpr int PG = 2;                       // passes interleaved in phase 1
};

// Byte offset of fp16 element (row, col) of half `lo` (0 = hi, 1 = lo) in a tile whose
// rows are [hi D fp16 | lo D fp16]; 16-byte units swizzled by (row & 15) so 16 lanes
// reading one column unit of 16 rows (MFMA operand reads) hit distinct banks.
template <int D>
__device__ __forceinline__ int hoff(int row, int col, int lo) {
  return row * (4 * D) + lo * (2 * D) + ((((col >> 3) ^ (row & 15))) << 4) + 2 * (col & 7);
}

template <int B>
struct Thermo {
  static constexpr int H = 1 << (B - 1);  // positive centroids
};

struct QParams {
  const void* x;
  const float* S;
  uint32_t* codes;
  uint32_t* norms;
  unsigned long long* counters;
  int64_t n;
  int64_t ld_x;          // elements
  int32_t d_in;
  int32_t esize;         // bytes per input element
  int32_t staged;        // rows are 16-byte aligned with a 16-byte multiple of valid bytes
  int32_t cpr;           // 16-byte chunks per row (staged path)
  int32_t split_blocks;  // blocks using the lo table
  int32_t words;         // words per vector
  uint32_t sign_mask[8]; // bit j set: coordinate j is multiplied by -1
  float cpos_lo[8], tpos_lo[8], cpos_hi[8], tpos_hi[8];  // positive halves; tpos[0] unused
  float cent_lo[16], cent_hi[16];
  // Paged output (slots == nullptr: record and norm of vector v at index v).  Vector
  // v = token * page_heads + head goes to row (page * page_heads + head) * page_size + off
  // of the cache, with page, off = slots[token] / page_size, % page_size; a negative slot or
  // one at or past num_pages * page_size is not written.
  const int64_t* slots;
  int64_t num_pages;
  int32_t page_heads, page_log2;
  // slots == nullptr and block_table set: token i sits at position pos0 + i of the sequence
  // whose pages block_table lists (max_blocks entries), i.e. slot
  // block_table[pos / page_size] * page_size + pos % page_size
  const int32_t* block_table;
  int64_t pos0;
  int32_t max_blocks;
  // Re-encoding (XT 3): the source record of each row, so that the rare fp64 rechecks
  // (norm near an fp16 rounding boundary, projection near zero) use the exact fp64
  // reconstruction instead of the fp32 row: record of row v at src_codes + v * src_words,
  // its norms (fp16 n16 | r16 << 16) at src_norms[v], the source JL matrix, codebooks
  // (lo table, then hi table) and widths.
  const uint32_t* src_codes;
  const uint32_t* src_norms;
  const float* src_S;
  int32_t src_words, src_split_blocks, src_blo, src_bhi, src_qjl;
  float src_cent[16];
  double src_gamma;   // sqrt(pi / 2) / d
};

// Re-encoding: coordinates j0 .. j0 + N - 1 (N = 2 or 4, j0 a multiple of N, so all in one
// block of 32) of row v's reconstruction in fp64 from its source record,
// y~_j = n16 c[idx_j] + (gamma r16) sum_i S_in[i][j] (2 sigma_i - 1).  The N columns of a row
// of S_in are one vector load; the 32 rows of a sign block are loaded before they are summed
// (a rare path: 128 loads per lane, 16 rows in flight at a time).
template <int N>
__device__ __forceinline__ void src_coords(const QParams& p, int64_t v, int j0, double* y) {
  static_assert(N == 2 || N == 4, "re-encoding runs at d = 128");
  typedef float fN __attribute__((ext_vector_type(N)));
  const uint32_t* rec = p.src_codes + v * p.src_words;
  const uint32_t nr = p.src_norms[v];
  const int sb = p.src_split_blocks, Q = p.src_qjl ? 1 : 0;
  auto off = [&](int b) {
    return b < sb ? b * (p.src_blo + Q) : sb * (p.src_blo + Q) + (b - sb) * (p.src_bhi + Q);
  };
  const int blk = j0 >> 5, bit0 = j0 & 31;
  const int nb = blk < sb ? p.src_blo : p.src_bhi;
  const double n16 = (double)f16_bits_to_f32(nr & 0xFFFFu);
  int idx[N];
#pragma unroll
  for (int e = 0; e < N; ++e) idx[e] = 0;
  for (int q = 0; q < nb; ++q) {
    const uint32_t w = rec[off(blk) + q];
#pragma unroll
    for (int e = 0; e < N; ++e) idx[e] |= (int)((w >> (bit0 + e)) & 1u) << q;
  }
#pragma unroll
  for (int e = 0; e < N; ++e) y[e] = n16 * (double)p.src_cent[(blk < sb ? 0 : 8) + idx[e]];
  if (p.src_qjl) {
    double st[N];
#pragma unroll
    for (int e = 0; e < N; ++e) st[e] = 0.0;
    for (int b2 = 0; b2 < 4; ++b2) {
      const uint32_t sw = rec[off(b2) + (b2 < sb ? p.src_blo : p.src_bhi)];
      const fN* col = reinterpret_cast<const fN*>(p.src_S + (int64_t)(32 * b2) * 128 + j0);
#pragma unroll
      for (int i0 = 0; i0 < 32; i0 += 16) {
        fN sv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[i] = col[(i0 + i) * (128 / N)];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool one = (sw >> (i0 + i)) & 1u;
#pragma unroll
          for (int e = 0; e < N; ++e) st[e] += one ? (double)sv[i][e] : -(double)sv[i][e];
        }
      }
    }
    const double gr = p.src_gamma * (double)f16_bits_to_f32(nr >> 16);
#pragma unroll
    for (int e = 0; e < N; ++e) y[e] += gr * st[e];
  }
}

// Destination row of vector vg (or -1: not written).
__device__ __forceinline__ int64_t dest_row(const QParams& p, int64_t vg) {
  if (!p.slots && !p.block_table) return vg;
  const int64_t tok = vg / p.page_heads;
  const int head = (int)(vg - tok * p.page_heads);
  int64_t sl;
  if (p.slots) {
    sl = p.slots[tok];
  } else {
    const int64_t pos = p.pos0 + tok, blk = pos >> p.page_log2;
    sl = blk < p.max_blocks ? ((int64_t)p.block_table[blk] << p.page_log2) + (pos & ((1ll << p.page_log2) - 1)) : -1;
  }
  const int64_t page = sl >> p.page_log2;
  if (sl < 0 || page >= p.num_pages) return -1;
  return ((page * p.page_heads + head) << p.page_log2) + (sl & ((1ll << p.page_log2) - 1));
}

// 16-bit input element -> fp32 (bf16 or fp16)
template <int XT>
__device__ __forceinline__ float cvt16(uint32_t h) {
  if constexpr (XT == 1) return __uint_as_float(h << 16);
  else return f16_bits_to_f32(h);
}

// Encode one slot (block) of the two vectors of a pass.  Returns the signed centroid of
// this lane's coordinate; the B code-plane ballots go to planes[] (plane q = bit q of idx).
// idx = #{m : t_m < z}: with a' = |z| nudged one float up when z <= 0, one strict compare
// t_j < a' per positive boundary gives k = #{j : t_j < a'} and idx = z > 0 ? H + k : H-1-k;
// bit q of k is the XOR of the thermometer ballots over multiples of 2^q.
template <int B, bool COUNT>
__device__ __forceinline__ float encode_slot(float z, const float* cpos, const float* tpos,
                                             uint64_t* planes, int& amb) {
  constexpr int H = Thermo<B>::H;
  const bool pos = z > 0.0f;
  const float az = fabsf(z);
  const float a = as_f(as_u(az) + (pos ? 0u : 1u));
  uint64_t T[H > 1 ? H : 2];
  float cv = cpos[0];  // the thresholds ascend, so the last true compare picks the centroid
#pragma unroll
  for (int j = 1; j < H; ++j) {
    const bool cj = tpos[j] < a;
    T[j] = __ballot(cj);
    cv = cj ? cpos[j] : cv;
    asm("" : "+v"(cv));  // keeps the chain of selects (no indexed read of a private copy)
  }
  const uint64_t P = __ballot(pos);
#pragma unroll
  for (int q = 0; q + 1 < B; ++q) {
    uint64_t kq = 0;
#pragma unroll
    for (int j = (1 << q); j < H; j += (1 << q)) kq ^= T[j];
    planes[q] = ~(kq ^ P);
  }
  planes[B - 1] = P;
  if constexpr (COUNT) {
    float dmin = az;
#pragma unroll
    for (int j = 1; j < H; ++j) dmin = fminf(dmin, fabsf(az - tpos[j]));
    amb += dmin < kWindow ? 1 : 0;
  }
  return pos ? cv : -cv;
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1 (compile-time loop index).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// fp64 recomputation of projection n of local vector m (rare path, whole wave).  Codes are
// read back from the tile's ballot table; S from global memory (exact fp32 values).
template <int D, int XT>
__device__ void guard_fix(const QParams& p, int64_t v, int m, int n, const uint64_t* bal,
                          uint64_t* sbal, const uint32_t* snorm, const float* cent_lds, int blo,
                          int bhi, unsigned long long& cnt_zero) {
  constexpr int NE = D / 64;
  constexpr int NB = D / 32;
  constexpr bool PRE = (XT == 3);  // input already in the rotated domain
  const int lane = lane_id();
  // coordinate of element e of this lane: lane + 64 e, which the FWHT below assumes; for
  // re-encoded rows (no FWHT) NE lane + e, so that one vector load reads a row of S_in
  auto jof = [&](int e) { return PRE ? NE * lane + e : lane + 64 * e; };
  double xd[NE];
  if constexpr (PRE) {
    src_coords<NE>(p, v, NE * lane, xd);   // re-encoding: every coordinate is < d_in = D
  } else {
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int j = lane + 64 * e;
      float xv = (j < p.d_in) ? load_elem(p.x, v * p.ld_x + j, XT) : 0.0f;
      xd[e] = (double)xv;
    }
  }
#pragma unroll
  for (int e = 0; e < NE && !PRE; ++e) {
    const uint32_t sw = (lane & 32) ? uniform_u32(p.sign_mask[2 * e + 1]) : uniform_u32(p.sign_mask[2 * e]);
    if ((sw >> (lane & 31)) & 1u) xd[e] = -xd[e];
  }
  if constexpr (!PRE) {
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
  }
  const double isd = PRE ? 1.0 : 1.0 / sqrt((double)D);
  const double n16 = (double)f16_bits_to_f32(snorm[m] & 0xFFFFu);
  const int pass = m >> 1, half = m & 1;
  double dot = 0.0, rr = 0.0;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int j = jof(e);
    const int blk = j >> 5, bit = j & 31;
    const int nb = blk < p.split_blocks ? blo : bhi;
    int idx = 0;
    for (int q = 0; q < nb; ++q)
      idx |= (int)((bal[(pass * NB + blk) * 4 + q] >> (32 * half + bit)) & 1u) << q;
    const float c = cent_lds[(blk < p.split_blocks ? 0 : 16) + idx];
    const double r = xd[e] * isd - n16 * (double)c;
    dot += (double)p.S[(int64_t)n * D + j] * r;
    rr += r * r;
  }
  dot = wave_sum_d(dot);
  rr = wave_sum_d(rr);
  if (lane == 0) {
    // sign ballot of (block, t, r): bit 16 (m / 4) + n % 16 of entry ((n/32)*2 + t)*4 + m%4
    uint64_t* w = &sbal[((n >> 5) * 2 + ((n >> 4) & 1)) * 4 + (m & 3)];
    const uint64_t bitmask = 1ull << (16 * (m >> 2) + (n & 15));
    *w = (dot >= 0.0) ? (*w | bitmask) : (*w & ~bitmask);
  }
  if (rr == 0.0 || fabs(dot) < (double)kWindow * sqrt(rr)) cnt_zero += 1;
}

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
                                           char* tile) {
#pragma unroll
  for (int i = 0; i < QCfg<D>::MAXC; ++i)
    if (cp.loff[i] >= 0) *reinterpret_cast<u32x4*>(tile + cp.loff[i]) = buf[i];
}

// XT: 0 fp32, 1 bf16, 2 fp16 input; 3 fp32 rows already in the rotated domain (re-encoding
// stored records: no sign flip, no Hadamard transform, no 1/sqrt(d)).  COUNT: accumulate the diagnostic counters.  QJ: the
// records carry QJL sign words (else MSE-only: no residual split, no projection).
template <int D, int BLO, int BHI, int XT, bool COUNT, bool QJ>
__global__ __launch_bounds__(64 * QCfg<D>::NW) void quantize_kernel(QParams p) {
  using C = QCfg<D>;
  constexpr int NB = C::NB;
  constexpr int NW = C::NW;
  constexpr int TV = C::TV;
  constexpr int PG = C::PG;
  constexpr bool UNI = (BLO == BHI);
  extern __shared__ __attribute__((aligned(16))) char lds_b[];
  char* S_l = lds_b;                                   // [kSRows] rows of [hi | lo] fp16
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  char* wl = lds_b + C::kSRows * C::kRowB + wave * C::kWaveB;
  char* tileb = wl;                                                  // [TV][hi|lo]
  uint64_t* bal = reinterpret_cast<uint64_t*>(wl + TV * C::kRowB);   // [pass][blk][4]
  uint64_t* sbal = bal + C::kBal;                                    // [blk][t][r]
  uint32_t* snorm = reinterpret_cast<uint32_t*>(sbal + C::kSBal);   // [TV]
  __shared__ float cent_lds[32];
  __shared__ float cpos_lds[16];  // positive centroids: lo table, then hi table
  __shared__ int wmap[32];        // record word -> (block << 8) | plane, plane 0xFF = signs

  if (threadIdx.x == 0) {  // constant indices: scalar reads of the kernel arguments
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      cent_lds[k] = p.cent_lo[k];
      cent_lds[16 + k] = p.cent_hi[k];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      cpos_lds[k] = p.cpos_lo[k];
      cpos_lds[8 + k] = p.cpos_hi[k];
    }
  }
  if (threadIdx.x == 0) {
    int w = 0;
    for (int b = 0; b < NB; ++b) {
      const int bb = b < p.split_blocks ? BLO : BHI;
      for (int q = 0; q < bb; ++q) wmap[w++] = (b << 8) | q;
      if (QJ) wmap[w++] = (b << 8) | 0xFF;
    }
  }
  auto load_s_rows = [&](int row0, int nrows) {
    // fp32 S rows -> scaled fp16 hi / lo halves, swizzled
    for (int i = threadIdx.x; i < nrows * D / 4; i += blockDim.x) {
      const int row = (4 * i) / D, col = (4 * i) % D;
      const f32x4 v = reinterpret_cast<const f32x4*>(p.S + (int64_t)row0 * D)[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sv = v[e] * kSScale;
        const _Float16 hi = (_Float16)sv;
        const _Float16 lo = (_Float16)(sv - (float)hi);
        *reinterpret_cast<_Float16*>(S_l + hoff<D>(row, col + e, 0)) = hi;
        *reinterpret_cast<_Float16*>(S_l + hoff<D>(row, col + e, 1)) = lo;
      }
    }
  };
  if constexpr (C::kResidentS && QJ) load_s_rows(0, D);
  __syncthreads();
  // record store mapping: lane -> (vector sv of a group of vpi, word sw); fixed per kernel
  const int vpi = 64 / p.words;
  const int sv = lane / p.words, sw = lane - sv * p.words;
  const bool s_lane = sv < vpi;
  const int swm = wmap[s_lane ? sw : 0], s_blk = swm >> 8, s_q = swm & 0xFF;

  const int h = lane >> 5, c = lane & 31;
  float dsg[NB];
#pragma unroll
  for (int s = 0; s < NB; ++s) dsg[s] = ((p.sign_mask[s] >> c) & 1u) ? -1.0f : 1.0f;
  constexpr bool PRE = (XT == 3);  // rows already rotated: no sign flip, no FWHT
  const float bs1 = (c & 1) ? -1.0f : 1.0f, bs2 = (c & 2) ? -1.0f : 1.0f;
  const float bs4 = (c & 4) ? -1.0f : 1.0f, bs8 = (c & 8) ? -1.0f : 1.0f;
  const float bs16 = (c & 16) ? -1.0f : 1.0f;
  const float inv_sqrt_d = PRE ? 1.0f : 1.0f / sqrtf((float)D);
  const float sqrt_d = PRE ? 1.0f : sqrtf((float)D);
  float tpl[8], tph[8], cpl[8], cph[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    tpl[k] = p.tpos_lo[k];
    tph[k] = p.tpos_hi[k];
    cpl[k] = p.cpos_lo[k];
    cph[k] = p.cpos_hi[k];
  }

  ChunkPlan<D> cp;
#pragma unroll
  for (int i = 0; i < C::MAXC; ++i) {
    const int ci = lane + 64 * i;
    const int row = p.staged ? ci / p.cpr : 0;
    const int cc = p.staged ? ci % p.cpr : 0;
    const bool ok = p.staged && row < TV;
    cp.row[i] = row;
    cp.goff[i] = (int64_t)row * p.ld_x * p.esize + 16 * cc;
    cp.loff[i] = ok ? row * C::kRowB + 16 * cc : -1;
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
      if (p.staged) stash_tile<D>(cp, pre, tileb);
      // ---------------- phase 1: rotation, norm, codes, residual (PG passes at once)
      for (int pp0 = 0; pp0 < TV / 2; pp0 += PG) {
        float xv[PG][NB];
        float ss[PG];
        bool valid[PG];
        int vloc[PG];
        float xin[PG][NB];
#pragma unroll
        for (int gg = 0; gg < PG; ++gg) {
          vloc[gg] = 2 * (pp0 + gg) + h;
          valid[gg] = v0 + vloc[gg] < p.n;
        }
        // one uniform branch per pass group, so that the LDS reads issue back to back
        if (p.staged) {
          // this lane's element of the first row, kept opaque so that the row and slot
          // offsets fold into the reads' immediate offsets
          constexpr int esz = (XT == 0 || XT == 3) ? 4 : 2;
          int roff = (int)(tileb - lds_b) + vloc[0] * C::kRowB + esz * c;
          asm volatile("" : "+v"(roff));
          const char* r0 = lds_b + roff;
#pragma unroll
          for (int gg = 0; gg < PG; ++gg) {
            const char* rowp = r0 + 2 * gg * C::kRowB;  // vloc[gg] = vloc[0] + 2 gg
#pragma unroll
            for (int s = 0; s < NB; ++s) {
              if constexpr (XT == 0 || XT == 3) xin[gg][s] = *reinterpret_cast<const float*>(rowp + 4 * 32 * s);
              else xin[gg][s] = cvt16<XT>(*reinterpret_cast<const uint16_t*>(rowp + 2 * 32 * s));
            }
          }
        } else {
#pragma unroll
          for (int gg = 0; gg < PG; ++gg)
#pragma unroll
            for (int s = 0; s < NB; ++s) {
              const int j = 32 * s + c;
              xin[gg][s] = (valid[gg] && j < p.d_in)
                               ? load_elem(p.x, (v0 + vloc[gg]) * p.ld_x + j, XT) : 0.0f;
            }
        }
#pragma unroll
        for (int gg = 0; gg < PG; ++gg) {
          float sq[NB];
#pragma unroll
          for (int s = 0; s < NB; ++s) {
            const int j = 32 * s + c;
            const float x = (valid[gg] && j < p.d_in) ? xin[gg][s] : 0.0f;
            sq[s] = x * x;
            xv[gg][s] = PRE ? x : x * dsg[s];
          }
#pragma unroll
          for (int hh = 1; hh < NB; hh <<= 1)  // pairwise (tree) sum of the squares
#pragma unroll
            for (int s = 0; s < NB; s += 2 * hh) sq[s] += sq[s + hh];
          ss[gg] = sq[0];
        }
#pragma unroll
        for (int gg = 0; gg < PG; ++gg) {
          ss[gg] = half_sum(ss[gg]);
#pragma unroll
          for (int hh = 1; hh < NB && !PRE; hh <<= 1)
#pragma unroll
            for (int s = 0; s < NB; ++s)
              if (!(s & hh)) {
                const float a = xv[gg][s], b = xv[gg][s + hh];
                xv[gg][s] = a + b;
                xv[gg][s + hh] = a - b;
              }
        }
        if constexpr (!PRE) {
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
        }

        float r[PG][NB];
        float rsq[PG];
        uint32_t n16[PG];
#pragma unroll
        for (int gg = 0; gg < PG; ++gg) {
          // ||x||: the squares are summed as a tree of depth log2(D) in fp32, so the relative
          // error is below (log2(D) + 2) 2^-24 < 6e-7: z = y / ||x|| stays within 3e-7 of
          // exact.  The stored fp16 norm must be the correctly rounded one: when a 1e-6
          // relative interval around the estimate straddles an fp16 rounding boundary the
          // norm is recomputed in fp64 from the input row (still in the tile).
          float nf = __builtin_amdgcn_sqrtf(ss[gg]);
          n16[gg] = f32_to_f16_bits(nf);
          // re-encoded rows carry the fp32 error of their reconstruction (about 1e-7
          // relative per coordinate, a few 1e-7 of the norm at most, on top of the 6e-7
          // above): a wider interval there, rechecked from the record
          constexpr float kMid = PRE ? 2e-6f : 1e-6f;
          const bool near_mid =
              f32_to_f16_bits(nf * (1.0f - kMid)) != f32_to_f16_bits(nf * (1.0f + kMid));
          if (__ballot(near_mid)) {
            const char* rowp = tileb + vloc[gg] * C::kRowB;
            double sd = 0.0;
            if constexpr (PRE) {   // coordinates NB c .. NB c + NB - 1 of the row (all < d_in)
              if (valid[gg]) {     // uniform within the half-wave; a row past n has no record
                double y[NB];
                src_coords<NB>(p, v0 + vloc[gg], NB * c, y);
#pragma unroll
                for (int s = 0; s < NB; ++s) sd = fma(y[s], y[s], sd);
              }
            }
#pragma unroll
            for (int s = 0; s < NB && !PRE; ++s) {
              const int j = 32 * s + c;
              double x;
              if (p.staged) {
                float xf;
                if constexpr (XT == 0) xf = *reinterpret_cast<const float*>(rowp + 4 * j);
                else xf = cvt16<XT>(*reinterpret_cast<const uint16_t*>(rowp + 2 * j));
                x = (valid[gg] && j < p.d_in) ? (double)xf : 0.0;
              } else {
                x = (valid[gg] && j < p.d_in) ? (double)load_elem(p.x, (v0 + vloc[gg]) * p.ld_x + j, XT) : 0.0;
              }
              sd = fma(x, x, sd);
            }
            sd = half_sum_d(sd);
            const double nrm = sqrt(sd);
            if (near_mid) {  // uniform within the half-wave (one vector)
              n16[gg] = f64_to_f16_bits(nrm);
              nf = (float)nrm;
            }
          }
          const float n16f = f16_bits_to_f32(n16[gg]);
          const float zinv = nf > 0.0f ? __builtin_amdgcn_rcpf(nf * sqrt_d) : 0.0f;
          rsq[gg] = 0.0f;
          int amb = 0;
          uint64_t pls[NB][3];  // this pass's plane ballots, stored by lane 0 below
          static_for<0, NB>([&](auto sc) __attribute__((always_inline)) {
            constexpr int s = decltype(sc)::value;
            const float z = xv[gg][s] * zinv;
            float cv;
            if constexpr (UNI) {
              cv = encode_slot<BLO, COUNT>(z, cpl, tpl, pls[s], amb);
            } else {  // mixed widths (run-time split): lane 0 stores this slot right away
              uint64_t pl[3];
              int nb;
              if (s < p.split_blocks) {
                cv = encode_slot<BLO, COUNT>(z, cpl, tpl, pl, amb);
                nb = BLO;
              } else {
                cv = encode_slot<BHI, COUNT>(z, cph, tph, pl, amb);
                nb = BHI;
              }
              if (lane == 0) {
#pragma unroll
                for (int q = 0; q < 3; ++q)
                  if (q < nb) bal[((pp0 + gg) * NB + s) * 4 + q] = pl[q];
              }
            }
            r[gg][s] = fmaf(xv[gg][s], inv_sqrt_d, -n16f * cv);
            rsq[gg] = fmaf(r[gg][s], r[gg][s], rsq[gg]);
          });
          if constexpr (UNI) {
            if (lane == 0) {
#pragma unroll
              for (int s = 0; s < NB; ++s)
#pragma unroll
                for (int q = 0; q < BLO; ++q) bal[((pp0 + gg) * NB + s) * 4 + q] = pls[s][q];
            }
          }
          if constexpr (COUNT) cnt_amb += valid[gg] ? (unsigned long long)amb : 0ull;
        }
#pragma unroll
        for (int gg = 0; gg < PG; ++gg) {
          const float rs = half_sum(rsq[gg]);
          const float rn = __builtin_amdgcn_sqrtf(rs);  // 1 ulp: r16 tolerates it at midpoints
          const uint32_t r16 = f32_to_f16_bits(rn);
          // any positive scale of r leaves the projection signs unchanged
          const float rinv = rn > 0.0f ? kRScale * __builtin_amdgcn_rcpf(rn) : 0.0f;
          // hoff(row, 32 s + c, lo): the 16-byte unit 4 s + (c >> 3) is XORed with row & 15,
          // i.e. s with (row >> 2) & 3 and c >> 3 with row & 3
          const int row = vloc[gg];
          const int abase = row * (4 * D) + ((((c >> 3) ^ (row & 3))) << 4) + 2 * (c & 7);
          const int rx2 = (row >> 2) & 3;
          if constexpr (QJ) {
#pragma unroll
            for (int s = 0; s < NB; ++s) {
              const float rv = r[gg][s] * rinv;
              const _Float16 hi = (_Float16)rv;
              const _Float16 lo = (_Float16)(rv - (float)hi);
              _Float16* dst = reinterpret_cast<_Float16*>(tileb + abase + ((s ^ rx2) << 6));
              dst[0] = hi;
              dst[D] = lo;  // lo half: 2 D bytes further
            }
          }
          if (c == 0) snorm[vloc[gg]] = n16[gg] | (r16 << 16);
          if constexpr (COUNT)
            if (c == 0 && valid[gg] && n16[gg] == 0x7C00u) cnt_ovf += 1;  // lanes 0, 32
        }
      }
      // next tile's input is fetched while this one is on the MFMA pipe
      const int64_t gn = g + gridDim.x;
      if (p.staged && gn < ngroups && gn * NW + wave < ntiles) fetch_tile<D>(p, cp, (gn * NW + wave) * TV, pre);
    }
    // ---------------- phase 2: JL projection on MFMA (3 fp16 products), sign ballots
    constexpr bool kHoistA = (D == 128);
    f16x8 a_h[kHoistA ? D / 32 : 1], a_l[kHoistA ? D / 32 : 1];
    if constexpr (kHoistA && QJ) {
      if (active) {
        const int arow = lane & 15, kg = 8 * (lane >> 4);
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          a_h[ks] = *reinterpret_cast<const f16x8*>(tileb + hoff<D>(arow, 32 * ks + kg, 0));
          a_l[ks] = *reinterpret_cast<const f16x8*>(tileb + hoff<D>(arow, 32 * ks + kg, 1));
        }
      }
    }
    for (int blk = 0; QJ && blk < NB; ++blk) {
      if constexpr (!C::kResidentS) {
        __syncthreads();
        load_s_rows(blk * 32, 32);
        __syncthreads();
      }
      if (!active) continue;
      const int s_row0 = C::kResidentS ? 0 : blk * 32;
      const int arow = lane & 15, kg = 8 * (lane >> 4);
      const int brow = blk * 32 + arow - s_row0;
      f32x4 acc0 = {}, acc1 = {};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const int col = 32 * ks + kg;
        f16x8 ah, al;
        if constexpr (kHoistA) {
          ah = a_h[ks];
          al = a_l[ks];
        } else {
          ah = *reinterpret_cast<const f16x8*>(tileb + hoff<D>(arow, col, 0));
          al = *reinterpret_cast<const f16x8*>(tileb + hoff<D>(arow, col, 1));
        }
        const f16x8 bh0 = *reinterpret_cast<const f16x8*>(S_l + hoff<D>(brow, col, 0));
        const f16x8 bl0 = *reinterpret_cast<const f16x8*>(S_l + hoff<D>(brow, col, 1));
        const f16x8 bh1 = *reinterpret_cast<const f16x8*>(S_l + hoff<D>(brow + 16, col, 0));
        const f16x8 bl1 = *reinterpret_cast<const f16x8*>(S_l + hoff<D>(brow + 16, col, 1));
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh1, acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl1, acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh1, acc1, 0, 0, 0);
      }
      // acc_t[r] of lane l: kUScale * u[vector 4(l/16) + r][32 blk + 16 t + l%16]
      uint64_t sg[2][4], gm[2][4];
      bool any_guard = false;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        sg[0][rr] = __ballot(acc0[rr] >= 0.0f);
        sg[1][rr] = __ballot(acc1[rr] >= 0.0f);
        gm[0][rr] = __ballot(fabsf(acc0[rr]) < kGuard * kUScale);
        gm[1][rr] = __ballot(fabsf(acc1[rr]) < kGuard * kUScale);
        any_guard |= (gm[0][rr] | gm[1][rr]) != 0;
      }
      if (lane == 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) sbal[(blk * 2 + t) * 4 + rr] = sg[t][rr];
      }
      if (any_guard) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            uint64_t gmk = gm[t][rr];
            while (gmk) {
              const int L = __builtin_ctzll(gmk);
              gmk &= gmk - 1;
              const int m = 4 * (L >> 4) + rr;
              const int64_t v = v0 + m;
              if (v >= p.n) continue;
              cnt_guard += (lane == 0);
              guard_fix<D, XT>(p, v, m, blk * 32 + 16 * t + (L & 15), bal, sbal, snorm, cent_lds,
                           BLO, BHI, cnt_zero);
            }
          }
      }
    }
    if (!active) continue;
    // ---------------- store the tile: assemble record words from the ballot tables
    const int nvalid = (int)((p.n - v0) < TV ? (p.n - v0) : TV);
    const uint32_t* b32 = reinterpret_cast<const uint32_t*>(bal);
    const uint16_t* s16 = reinterpret_cast<const uint16_t*>(sbal);
    // a record has at most 4 NB words, so a group of vpi >= 16 / NB vectors covers a lane's
    // share of the tile in at most NB passes: every word is read from the tables first and
    // then stored, so the table reads do not wait on one another
    uint32_t wv[NB];
    int64_t rv[NB];
#pragma unroll
    for (int it = 0; it < NB; ++it) {
      const int v = it * vpi + sv;
      rv[it] = -1;
      wv[it] = 0u;
      if (s_lane && v < nvalid) {
        if (s_q != 0xFF) {
          wv[it] = b32[(((v >> 1) * NB + s_blk) * 4 + s_q) * 2 + (v & 1)];
        } else {
          const int rr = v & 3, gq = v >> 2;
          wv[it] = (uint32_t)s16[((s_blk * 2 + 0) * 4 + rr) * 4 + gq] |
                   ((uint32_t)s16[((s_blk * 2 + 1) * 4 + rr) * 4 + gq] << 16);
        }
        rv[it] = dest_row(p, v0 + v);
      }
    }
#pragma unroll
    for (int it = 0; it < NB; ++it)
      if (rv[it] >= 0) p.codes[rv[it] * p.words + sw] = wv[it];
    if (lane < nvalid) {
      const int64_t row = dest_row(p, v0 + lane);
      if (row >= 0) p.norms[row] = snorm[lane];
    }
  }
  if constexpr (COUNT) {
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

// Host: the format- and table-dependent parameters (record layout, sign flips, codebook
// halves and thresholds).
inline void fill_format_params(const tq_format* f, const tq_tables* t, QParams& p) {
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
}

template <int D, int BLO, int BHI, int XT, bool COUNT, bool QJ>
static int launch_q(const QParams& p, hipStream_t stream, int num_cu) {
  using C = QCfg<D>;
  const size_t lds = (size_t)C::kSRows * C::kRowB + (size_t)C::NW * C::kWaveB;
  static bool attr_set = false;  // per template instance
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)quantize_kernel<D, BLO, BHI, XT, COUNT, QJ>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return TQ_ERR_HIP;
    attr_set = true;
  }
  const int64_t ntiles = (p.n + C::TV - 1) / C::TV;
  const int64_t ngroups = (ntiles + C::NW - 1) / C::NW;
  const int64_t grid = ngroups < (int64_t)num_cu ? ngroups : (int64_t)num_cu;
  hipLaunchKernelGGL((quantize_kernel<D, BLO, BHI, XT, COUNT, QJ>), dim3((unsigned)grid),
                     dim3(64 * C::NW), lds, stream, p);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

template <int D, int BLO, int BHI, bool QJ>
static int launch_xt(const QParams& p, int xt, hipStream_t stream, int num_cu) {
  const bool count = p.counters != nullptr;
  if (xt == 0) return count ? launch_q<D, BLO, BHI, 0, true, QJ>(p, stream, num_cu)
                            : launch_q<D, BLO, BHI, 0, false, QJ>(p, stream, num_cu);
  if (xt == 1) return count ? launch_q<D, BLO, BHI, 1, true, QJ>(p, stream, num_cu)
                            : launch_q<D, BLO, BHI, 1, false, QJ>(p, stream, num_cu);
  return count ? launch_q<D, BLO, BHI, 2, true, QJ>(p, stream, num_cu)
               : launch_q<D, BLO, BHI, 2, false, QJ>(p, stream, num_cu);
}

// Launches the kernel of one (head dim, widths) pair; instantiated in the per-format
// translation units (tq_quantize_*.hip) so that they compile in parallel.
template <int D, int BLO, int BHI>
int launch_quantize(const QParams& p, int xt, bool qjl, hipStream_t stream, int num_cu) {
  return qjl ? launch_xt<D, BLO, BHI, true>(p, xt, stream, num_cu)
             : launch_xt<D, BLO, BHI, false>(p, xt, stream, num_cu);
}

}  // namespace tqk

