// Token-sliced cache layout (tq_format.layout == 1).  The per-vector record puts the bits of
// 32 coordinates of one vector in a word (the block-32 layout of the zhidx turboquant_plus
// article, section "01 turboquant_plus：介绍与详解").  The token-sliced layout keeps the same
// bits, sliced across tokens: for each group of 32 consecutive vectors and each coordinate j,
// the words of j (its code bit-planes, then its QJL sign) hold bit t = that bit of vector
// 32 * group + t.  A decode step sums w_t * value_t over tokens, so with this layout the bits
// of one coordinate over 32 tokens arrive as one word: the operand shape of an MFMA whose
// contraction runs over tokens.
//
// tile_values rewrites quantized records in place: each half-wave loads the 32 records of one
// group, every record word position k is a 32 x 32 bit matrix (token x bit), transposed across
// the 32 lanes in five exchange stages (ds_swizzle xor 16, 8, 4, 2, 1; at each stage lane t
// and lane t ^ J swap the halves of their words selected by bit J of the bit position), and
// lane t then holds coordinate 32 * block + t of every plane of that block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tqt {

template <int J>
__device__ __forceinline__ uint32_t transpose_stage(uint32_t r, int lane) {
  constexpr uint32_t HI = J == 16 ? 0xFFFF0000u
                        : J == 8  ? 0xFF00FF00u
                        : J == 4  ? 0xF0F0F0F0u
                        : J == 2  ? 0xCCCCCCCCu
                                  : 0xAAAAAAAAu;  // bit positions i with (i & J) != 0
  const uint32_t p = (uint32_t)__builtin_amdgcn_ds_swizzle((int)r, (J << 10) | 0x1F);
  // lane with bit J clear keeps its low positions and takes the partner's low positions
  // shifted up; the partner keeps its high positions and takes ours shifted down
  const uint32_t lo_lane = (r & ~HI) | ((p << J) & HI);
  const uint32_t hi_lane = (r & HI) | ((p >> J) & ~HI);
  return (lane & J) ? hi_lane : lo_lane;
}

__device__ __forceinline__ uint32_t transpose32(uint32_t r, int lane) {
  r = transpose_stage<16>(r, lane);
  r = transpose_stage<8>(r, lane);
  r = transpose_stage<4>(r, lane);
  r = transpose_stage<2>(r, lane);
  return transpose_stage<1>(r, lane);
}

// d = 128; blocks below SPLITB use BLO code bits, the others BHI; Q sign words (0 or 1).
// Records are read and written in the widest aligned units their word counts allow (16 or
// 8 bytes), so that a wave issues few, dense memory instructions.
template <int BLO, int BHI, int SPLITB, int Q>
__global__ __launch_bounds__(256) void tile_values(uint32_t* __restrict__ codes, int64_t n_groups) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  constexpr int WLO = BLO + Q, WHI = BHI + Q;
  constexpr int W = SPLITB * WLO + (4 - SPLITB) * WHI;   // words per record
  const int lane = threadIdx.x & 63, t = lane & 31;
  const int64_t grp = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  const bool valid = grp < n_groups;
  uint32_t r[W];
  uint32_t* gbase = codes + grp * 32 * W;
  if (valid) {
    const uint32_t* rec = gbase + (int64_t)t * W;   // 4 W bytes from a 128-byte aligned group
    if constexpr (W % 4 == 0) {
#pragma unroll
      for (int i = 0; i < W / 4; ++i) {
        const u32x4 x = reinterpret_cast<const u32x4*>(rec)[i];
        r[4 * i] = x[0]; r[4 * i + 1] = x[1]; r[4 * i + 2] = x[2]; r[4 * i + 3] = x[3];
      }
    } else if constexpr (W % 2 == 0) {
#pragma unroll
      for (int i = 0; i < W / 2; ++i) {
        const u32x2 x = reinterpret_cast<const u32x2*>(rec)[i];
        r[2 * i] = x[0]; r[2 * i + 1] = x[1];
      }
    } else {
#pragma unroll
      for (int k = 0; k < W; ++k) r[k] = rec[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < W; ++k) r[k] = 0u;
  }
  // every load of the group lands before any store overwrites it (in place)
  __syncthreads();
#pragma unroll
  for (int k = 0; k < W; ++k) r[k] = transpose32(r[k], lane);
  if (!valid) return;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int wb = b < SPLITB ? WLO : WHI;
    const int k0 = b < SPLITB ? b * WLO : SPLITB * WLO + (b - SPLITB) * WHI;  // first word of block b
    const int j = 32 * b + t;                                                  // coordinate
    const int64_t off = j < 32 * SPLITB ? (int64_t)j * WLO
                                        : (int64_t)32 * SPLITB * WLO + (int64_t)(j - 32 * SPLITB) * WHI;
    if (wb == 4) {          // 16-byte aligned: off is a multiple of 4 words
      *reinterpret_cast<u32x4*>(gbase + off) = (u32x4){r[k0], r[k0 + 1], r[k0 + 2], r[k0 + 3]};
    } else if (wb == 2) {   // 8-byte aligned: off is even
      *reinterpret_cast<u32x2*>(gbase + off) = (u32x2){r[k0], r[k0 + 1]};
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p)
        if (p < wb) gbase[off + p] = r[k0 + p];
    }
  }
}

template <int BLO, int BHI, int SPLITB, int Q>
int launch_tiles(uint32_t* codes, int64_t n_groups, hipStream_t stream) {
  const int64_t wgs = (n_groups + 7) / 8;
  hipLaunchKernelGGL((tile_values<BLO, BHI, SPLITB, Q>), dim3((unsigned)wgs), dim3(256), 0, stream,
                     codes, n_groups);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

}  // namespace tqt

// Rewrite n (a multiple of 32) freshly quantized d = 128 records as token-sliced groups.
int tq_launch_tiles(const tq_format* f, void* codes, int64_t n, hipStream_t stream) {
  using namespace tqt;
  if (n <= 0) return TQ_OK;
  uint32_t* c = reinterpret_cast<uint32_t*>(codes);
  const int64_t ng = n / 32;
  const int lo = f->bits_lo, hi = f->split == f->d ? f->bits_lo : f->bits_hi;
  const int sb = f->split == f->d ? 4 : f->split / 32;
#define TQ_TILE_CASE(BL, BH, SB)                                                   \
  if (lo == BL && hi == BH && (SB == 4 ? sb == 4 : sb == SB))                      \
    return f->qjl ? launch_tiles<BL, BH, SB, 1>(c, ng, stream)                     \
                  : launch_tiles<BL, BH, SB, 0>(c, ng, stream);
  TQ_TILE_CASE(1, 1, 4)
  TQ_TILE_CASE(2, 2, 4)
  TQ_TILE_CASE(3, 3, 4)
  TQ_TILE_CASE(3, 2, 1)
  TQ_TILE_CASE(3, 2, 2)
  TQ_TILE_CASE(3, 2, 3)
  TQ_TILE_CASE(2, 1, 1)
  TQ_TILE_CASE(2, 1, 2)
  TQ_TILE_CASE(2, 1, 3)
#undef TQ_TILE_CASE
  return TQ_ERR_SHAPE;
}
