// Re-encoding stored records at another format (temporal decay: older tokens move to fewer
// bits; zhidx turboquant_plus article, section "01 turboquant_plus：介绍与详解").
//
// What is computed: each record's reconstruction in the rotated domain,
//   y~ = n16 c[idx] + gamma r16 S^T (2 sigma - 1)   (the sign term only with QJL),
// is encoded again by the quantize steps that follow the rotation (norm, codes, residual,
// QJL signs), in the rotation both formats share.  Two launches per chunk of vectors:
//   source:    y~ rows (fp32) into the caller's workspace.  S^T (2 sigma - 1) is the dense
//              contraction of this step: 16 records x 128 projections x 128 coordinates per
//              wave tile on v_mfma_f32_16x16x32_f16, with the +-1 signs exact in fp16 and S
//              split into scaled fp16 hi + lo (the same 2^-22 relative accuracy as the
//              quantize projection); S^T stays resident in LDS.
//   quantize:  quantize_kernel with pre-rotated fp32 rows (XT 3).  The rows carry the fp32
//              error of the reconstruction, about 1e-7 relative per coordinate; its rare
//              fp64 rechecks (a norm near an fp16 rounding boundary, a projection near
//              zero) recompute the reconstruction exactly in fp64 from the source record,
//              so those decisions are the ones the exact reconstruction gives.
// The source kernel also copies each chunk's records and norms into the workspace, where
// the rechecks read them.  In place: a chunk's rows and copies are complete before its
// records are rewritten, and a narrower record never reaches the next chunk's input, so
// codes_out may equal codes_in.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.h"
#include "tq_internal.h"
#include "tq_quantize_kernel.h"

namespace tqk {

constexpr int kRqD = 128;
constexpr int kRqWaves = 8;
constexpr int kRqRowB = 4 * kRqD;  // bytes of one [hi | lo] fp16 row of S^T

struct RqParams {
  const uint32_t* codes;  // source records of this chunk
  const uint32_t* norms;  // source norms of this chunk (fp16 n16 | fp16 r16 << 16)
  const float* S;         // source JL matrix [projection i][coordinate j]
  float* out;             // y~ rows [n][128]
  uint32_t* rec_copy;     // copies of the records [n][words] and norms [n] (for the rechecks)
  uint32_t* nrm_copy;
  int64_t n;
  int32_t words, split_blocks, bits_lo, bits_hi;
  float gamma;            // sqrt(pi/2) / d
  float cent[16];         // source codebooks: lo table, then hi table
};

// y~ of 16 records per wave tile.  BLO / BHI: source codebook widths below / above the
// split (run time); QJ: the source records carry sign words.
template <int BLO, int BHI, bool QJ>
__global__ __launch_bounds__(64 * kRqWaves) void requant_source(RqParams p) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  constexpr int Q = QJ ? 1 : 0;
  constexpr int BMAX = BLO > BHI ? BLO : BHI;
  extern __shared__ __attribute__((aligned(16))) char lds_r[];
  char* St = lds_r;                                          // [128 rows j][hi | lo] fp16
  uint32_t* recs = reinterpret_cast<uint32_t*>(lds_r + (QJ ? kRqD * kRqRowB : 0));
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  uint32_t* wrec = recs + wave * (16 * 16 + 16);             // 16 records (<= 16 words) + norms
  uint32_t* wnrm = wrec + 16 * 16;
  __shared__ float cent[16];
  if (tid < 16) cent[tid] = p.cent[tid];
  if constexpr (QJ) {
    // S^T scaled by 2^10, split hi / lo; the 16-byte units of a row are swizzled by j & 15
    for (int e = tid; e < kRqD * kRqD; e += blockDim.x) {
      const int i = e / kRqD, j = e % kRqD;
      const float sv = p.S[e] * 1024.0f;
      const _Float16 hi = (_Float16)sv;
      const _Float16 lo = (_Float16)(sv - (float)hi);
      const int unit = ((i >> 3) ^ (j & 15));
      *reinterpret_cast<_Float16*>(St + j * kRqRowB + (unit << 4) + 2 * (i & 7)) = hi;
      *reinterpret_cast<_Float16*>(St + j * kRqRowB + 2 * kRqD + (unit << 4) + 2 * (i & 7)) = lo;
    }
  }
  __syncthreads();
  const int W = p.words, sb = p.split_blocks;
  auto off = [&](int b) { return b < sb ? b * (BLO + Q) : sb * (BLO + Q) + (b - sb) * (BHI + Q); };
  const float scaleq = p.gamma * (1.0f / 1024.0f);
  const int64_t ntiles = (p.n + 15) / 16;
  const int64_t stride = (int64_t)gridDim.x * kRqWaves;
  // register prefetch of a tile: record words lane + 64 k (k < 4) and, lanes < 16, a norm
  uint32_t pw[4], pn = 0;
  auto fetch = [&](int64_t tile) {
    const int64_t v0 = tile * 16;
    const int nv = (int)((p.n - v0) < 16 ? (p.n - v0) : 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = lane + 64 * k;
      pw[k] = (tile < ntiles && i < nv * W) ? p.codes[v0 * W + i] : 0u;
    }
    pn = (tile < ntiles && lane < nv) ? p.norms[v0 + lane] : 0u;
  };
  int64_t tile = (int64_t)blockIdx.x * kRqWaves + wave;
  fetch(tile);
  for (; tile < ntiles; tile += stride) {
    const int64_t v0 = tile * 16;
    const int nv = (int)((p.n - v0) < 16 ? (p.n - v0) : 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (lane + 64 * k < 16 * W) wrec[lane + 64 * k] = pw[k];
      if (lane + 64 * k < nv * W) p.rec_copy[v0 * W + lane + 64 * k] = pw[k];
    }
    if (lane < 16) wnrm[lane] = pn;
    if (lane < nv) p.nrm_copy[v0 + lane] = pn;
    fetch(tile + stride);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile's rows are visible to the wave
    f32x4 acc[8];
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) acc[jb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (QJ) {
      // operand A: row m = record lane & 15, k = 8 (lane >> 4) .. + 7 of block ks as +-1
      const int m = lane & 15, kg = lane >> 4;
      f16x8 a[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint32_t sw = wrec[m * W + off(ks) + (ks < sb ? BLO : BHI)];
        const uint32_t b8 = (sw >> (8 * kg)) & 0xFFu;
        u32x4 u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // fp16 -1 is 0xBC00, +1 is 0x3C00: flip bit 15 of each half for a set bit
          const uint32_t lo = (b8 >> (2 * q)) & 1u, hi = (b8 >> (2 * q + 1)) & 1u;
          u[q] = 0xBC00BC00u ^ (lo << 15) ^ (hi << 31);
        }
        a[ks] = __builtin_bit_cast(f16x8, u);
      }
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) {
        const int j = 16 * jb + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int unit = ((4 * ks + kg) ^ (j & 15));
          const f16x8 bh = *reinterpret_cast<const f16x8*>(St + j * kRqRowB + (unit << 4));
          const f16x8 bl = *reinterpret_cast<const f16x8*>(St + j * kRqRowB + 2 * kRqD + (unit << 4));
          acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ks], bh, acc[jb], 0, 0, 0);
          acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ks], bl, acc[jb], 0, 0, 0);
        }
      }
    }
    // acc[jb][r] of lane l: 2^10 (S^T sigma) of record 4 (l >> 4) + r, coordinate 16 jb + l % 16
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * (lane >> 4) + r;
      const uint32_t nr = wnrm[m];
      const float n16 = f16_bits_to_f32(nr & 0xFFFFu);
      const float g = scaleq * f16_bits_to_f32(nr >> 16);
      float* orow = p.out + (v0 + m) * kRqD + (lane & 15);
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const bool lo = blk < sb;
        const uint32_t* rw = wrec + m * W + off(blk);
        uint32_t pl[BMAX];
#pragma unroll
        for (int q = 0; q < BMAX; ++q) pl[q] = (q < (lo ? BLO : BHI)) ? rw[q] : 0u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int bit = 16 * h + (lane & 15);
          int idx = 0;
#pragma unroll
          for (int q = 0; q < BMAX; ++q) idx |= (int)((pl[q] >> bit) & 1u) << q;
          float y = n16 * cent[(lo ? 0 : 8) + idx];
          if constexpr (QJ) y = fmaf(g, acc[2 * blk + h][r], y);
          if (m < nv) orow[32 * blk + 16 * h] = y;
        }
      }
    }
  }
}

template <int BLO, int BHI>
static int launch_reencode(const QParams& q, bool count, bool qjl, hipStream_t s, int ncu) {
  if (count) return qjl ? launch_q<128, BLO, BHI, 3, true, true>(q, s, ncu)
                        : launch_q<128, BLO, BHI, 3, true, false>(q, s, ncu);
  return qjl ? launch_q<128, BLO, BHI, 3, false, true>(q, s, ncu)
             : launch_q<128, BLO, BHI, 3, false, false>(q, s, ncu);
}

}  // namespace tqk

// ---------------------------------------------------------------------------------------
int tq_launch_requant(const tq_format* fi, const tq_tables* ti, const void* codes_in,
                      const uint16_t* norms_in, int64_t n, const tq_format* fo,
                      const tq_tables* to, void* codes_out, uint16_t* norms_out,
                      int64_t* counters, void* workspace, int64_t workspace_bytes,
                      hipStream_t stream) {
  using namespace tqk;
  const int ncu = tq_num_cus();
  if (ncu <= 0) return TQ_ERR_HIP;
  // workspace per vector of a chunk: its fp32 row, a copy of its record (at most 16 words)
  // and of its norms
  const int64_t chunk = workspace_bytes / tq_requant_vector_bytes();
  const int wi = (int)(tq_record_bytes(fi) / 4), wo = (int)(tq_record_bytes(fo) / 4);
  char* wsb = reinterpret_cast<char*>(workspace);
  RqParams rp{};
  rp.S = ti->S;
  rp.out = reinterpret_cast<float*>(wsb);
  rp.rec_copy = reinterpret_cast<uint32_t*>(wsb + chunk * kRqD * 4);
  rp.nrm_copy = reinterpret_cast<uint32_t*>(wsb + chunk * (kRqD * 4 + 64));
  rp.words = wi;
  rp.split_blocks = fi->split / 32;
  rp.bits_lo = fi->bits_lo;
  rp.bits_hi = fi->split == fi->d ? fi->bits_lo : fi->bits_hi;
  rp.gamma = (float)(std::sqrt(M_PI / 2.0) / kRqD);
  for (int k = 0; k < 8; ++k) {
    rp.cent[k] = k < (1 << rp.bits_lo) ? ti->centroids_lo[k] : 0.0f;
    rp.cent[8 + k] = k < (1 << rp.bits_hi) ? ti->centroids_hi[k] : 0.0f;
  }
  QParams q{};
  fill_format_params(fo, to, q);
  q.S = to->S;
  q.counters = reinterpret_cast<unsigned long long*>(counters);
  q.ld_x = kRqD;
  q.d_in = kRqD;
  q.esize = 4;
  q.staged = 1;  // workspace rows: 16-byte aligned, 512 bytes
  q.cpr = kRqD * 4 / 16;
  q.x = workspace;
  q.src_codes = rp.rec_copy;
  q.src_norms = rp.nrm_copy;
  q.src_S = ti->S;
  q.src_words = wi;
  q.src_split_blocks = rp.split_blocks;
  q.src_blo = rp.bits_lo;
  q.src_bhi = rp.bits_hi;
  q.src_qjl = fi->qjl;
  for (int k = 0; k < 16; ++k) q.src_cent[k] = rp.cent[k];
  q.src_gamma = std::sqrt(M_PI / 2.0) / kRqD;
  const size_t src_lds = (fi->qjl ? (size_t)kRqD * kRqRowB : 0) + (size_t)kRqWaves * (16 * 16 + 16) * 4;
  const int ilo = rp.bits_lo, ihi = rp.bits_hi;
  const void* src_fn = nullptr;
#define TQ_RQ_PICK(a, b)                                                                   \
  if (ilo == a && ihi == b)                                                                \
    src_fn = fi->qjl ? (const void*)requant_source<a, b, true> : (const void*)requant_source<a, b, false>;
  TQ_RQ_PICK(1, 1) TQ_RQ_PICK(2, 2) TQ_RQ_PICK(3, 3) TQ_RQ_PICK(3, 2) TQ_RQ_PICK(2, 1)
#undef TQ_RQ_PICK
  if (!src_fn) return TQ_ERR_SHAPE;
  if (hipFuncSetAttribute(src_fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)src_lds) != hipSuccess)
    return TQ_ERR_HIP;
  const int lo = fo->bits_lo, hi = fo->split == fo->d ? fo->bits_lo : fo->bits_hi;
  for (int64_t c0 = 0; c0 < n; c0 += chunk) {
    const int64_t m = (n - c0) < chunk ? (n - c0) : chunk;
    rp.codes = reinterpret_cast<const uint32_t*>(codes_in) + c0 * wi;
    rp.norms = reinterpret_cast<const uint32_t*>(norms_in) + c0;
    rp.n = m;
    const int64_t tiles = (m + 15) / 16;
    int64_t grid = (tiles + kRqWaves - 1) / kRqWaves;
    if (grid > ncu) grid = ncu;
    void* args[] = {&rp};
    if (hipLaunchKernel(src_fn, dim3((unsigned)grid), dim3(64 * kRqWaves), args, src_lds, stream) != hipSuccess ||
        hipGetLastError() != hipSuccess)
      return TQ_ERR_HIP;
    q.n = m;
    q.codes = reinterpret_cast<uint32_t*>(codes_out) + c0 * wo;
    q.norms = reinterpret_cast<uint32_t*>(norms_out) + c0;
    int rc = TQ_ERR_SHAPE;
    const bool cnt = counters != nullptr, qj = fo->qjl != 0;
    if (lo == 1 && hi == 1) rc = launch_reencode<1, 1>(q, cnt, qj, stream, ncu);
    else if (lo == 2 && hi == 2) rc = launch_reencode<2, 2>(q, cnt, qj, stream, ncu);
    else if (lo == 3 && hi == 3) rc = launch_reencode<3, 3>(q, cnt, qj, stream, ncu);
    else if (lo == 3 && hi == 2) rc = launch_reencode<3, 2>(q, cnt, qj, stream, ncu);
    else if (lo == 2 && hi == 1) rc = launch_reencode<2, 1>(q, cnt, qj, stream, ncu);
    if (rc != TQ_OK) return rc;
  }
  return TQ_OK;
}
