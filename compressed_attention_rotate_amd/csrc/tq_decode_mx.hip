// Decode attention over a cache whose values are token-sliced (tq_format.layout == 1) with
// both dot products of the step on gfx950's block-scaled matrix cores
// (v_mfma_scale_f32_16x16x128_f8f6f4 with an fp6 e2m3 A operand of 16 x 128 and an fp4 e2m1
// B operand of 128 x 16, one E8M0 scale per row and 32-element block, fp32 accumulation).
//
// What is computed is the decode step of the 163.com explainer
// (m.163.com/dy/article/KOV7P8JI0556C3J2, sections "第二步：QJL" and "速度"):
//   logit_t = scale * (n16_t <q_rot, c[idx_t]> + gamma r16_t <S q_rot, sigma_t>),
//   softmax over t < seq_len, value rows summed in the rotated domain and mapped back once.
//
// Sign dot products on MFMA.  A symmetric codebook is an odd function of the code bits, so
// c[idx] = sum_k alpha_k s_k over the odd Walsh monomials s_k of the bit-planes (s = 2b - 1;
// for 3 bits: s0, s1, s2, s0 s1 s2, the last one the XOR of the three planes).  Every term
// of the step is then a dot product of real weights with +-1 signs: <q_rot, s_k> and
// <S q_rot, sigma> for the keys (contraction over coordinates), sum_t u_t s_k,t,j and
// sum_t u'_t sigma_t,j for the values (contraction over tokens).  A 32-bit plane word w
// becomes the fp4 B operand of 32 contraction indices with one AND per dword: dword D keeps
// bit D of every nibble, so nibble i of dword D is bit 4i + D of w, an e2m1 value 0.5 b,
// b or 2 b (D = 0, 1, 2); for D = 3 the bit lands on the nibble's sign and OR-ing 0001
// gives -+0.5 s.  Scaling the matching A entries by 4, 2, 1, -+2 turns every product into
// a (s + 1) or a s, and the constant sum over the first three nibble positions is removed
// after the product.
//
// Block floating point digits.  The matrix core sums each 32-element contraction block in a
// fixed-point window about 14 bits below the block's largest product, so real-valued
// operands lose small products next to large ones.  A operands are therefore written as
// integers: for each row of weights and 32-element block, an exponent e from the block's
// largest magnitude and x = |v| 2^-e in [0, 1) as base-16 digits; digit l is one row of A,
// stored as d / 2 (every half-integer 0 .. 7.5 is exact in e2m3), with the E8M0 block scale
// 2^(e - 4(l + 1) + 1).  Products are multiples of 1/4 below 16, every block sum is exact,
// and each row comes out of the product in absolute units.  Keys use 8 digits (x truncated
// to 32 bits: two products per plane, digits 0-3 and 4-7 of the same 4 heads), values 4
// (x rounded to 16 bits); the constants removed after the products are built from the same
// rounded weights.  An fp6 x fp4 product issues in half the cycles of an fp8 x fp4 one.
//
// Keys: lane (g, n) loads block g (32 coordinates, 16 bytes at b = 4) of token n of a
// 16-token group; the codebook and sign products give, in lane (h, n), head h's logit for
// token n.  Values: with the token-sliced layout, lane (g, n) loads the words of coordinate
// 16 c + n for 32-token group g of the tile; one product per plane and block of 16
// coordinates sums 128 tokens.  The softmax weights, produced in the logit lanes as 16-bit
// integers with a block exponent, are handed to the A layout through LDS.
//
// Grid (split, batch * KV head * chunk of 4 query heads); 4 waves per workgroup, one per
// SIMD; each wave walks 128-token tiles of the split, the next tile's records in flight
// while the current one is computed.  The waves' partials (m, l, A, Q) merge in LDS and go
// to the split-combine kernel of the per-vector path (same partial format).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "tq_decode_kernel.h"

namespace tqx {
using namespace tqk;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

constexpr int kXWaves = 4;
constexpr int kXThreads = 64 * kXWaves;
constexpr int kXTile = 128;      // tokens per wave tile

struct MxParams {
  const void* q;
  const uint32_t* codes_k;   // per-vector key records
  const uint32_t* norms_k;   // per vector: fp16 ||x|| | fp16 ||r|| << 16
  const uint32_t* codes_v;   // token-sliced value groups
  const uint32_t* norms_v;
  const int32_t* seq_lens;
  const float* S_k;
  float* ws_part;            // [batch * hq][n_split][kPartFloats]
  float* logits;             // nullable [batch][hq][capacity]
  unsigned long long* skipped;
  int64_t capacity, tokens_per_split;
  int32_t hq, hkv, group, q_dtype, n_split;
  float scale, tau, gamma;
  uint32_t sign_k[4];
  float alpha_k[2][4];       // Walsh coefficients of the key codebooks (lo, hi width)
  float alpha_v[2][4];
};

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));

// A (fp6 e2m3 digit rows, E8M0 scale byte `sa` of this lane's row and block) x B (fp4) + C
__device__ __forceinline__ f32x4 mma(const i32x8& a, const i32x4& b, f32x4 c, int sa) {
  const i32x8 bb = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, c, 2, 4, 0, sa, 0, 127);
}

// fp4 B operand of one plane word (see the file comment); the nibble-sign dword gives -0.5 s
__device__ __forceinline__ i32x4 fp4_of(uint32_t w) {
  i32x4 b;
  b[0] = (int)(w & 0x11111111u);
  b[1] = (int)(w & 0x22222222u);
  b[2] = (int)(w & 0x44444444u);
  b[3] = (int)((w & 0x88888888u) | 0x11111111u);
  return b;
}

// the same with +0.5 s for the nibble-sign dword (every A weight of the value sums >= 0)
__device__ __forceinline__ i32x4 fp4_pos(uint32_t w) {
  i32x4 b;
  b[0] = (int)(w & 0x11111111u);
  b[1] = (int)(w & 0x22222222u);
  b[2] = (int)(w & 0x44444444u);
  b[3] = (int)(((w ^ 0x88888888u) & 0x88888888u) | 0x11111111u);
  return b;
}

// A row of 32 digits (element p = K index 32 g + p of this lane) as fp6 e2m3 values d / 2;
// the packed conversion interleaves its two sources (element 2 i from ev[i], 2 i + 1 from od[i])
// and divides by its scale operand.  It writes its first result dwords before it has read the
// last source registers, so the result must not share registers with the sources: written
// as an instruction with an early-clobber result (the compiler's builtin may overlap them).
__device__ __forceinline__ i32x8 fp6_row(const f32x16& ev, const f32x16& od) {
  u32x6 r;
  asm volatile("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(r) : "v"(ev), "v"(od), "v"(2.0f));
  return (i32x8){(int)r[0], (int)r[1], (int)r[2], (int)r[3], (int)r[4], (int)r[5], 0, 0};
}

// Block exponent: e with |x| 2^-e in [0.5, 1); blocks below 2^-80 count as zero (e = -100)
constexpr int kZeroExp = -100;
__device__ __forceinline__ int block_exp(float amax) {
  return amax >= 8.271806125530277e-25f ? __builtin_amdgcn_frexp_expf(amax) : kZeroExp;
}

// E8M0 scale byte of digit row l (digits stored as d / 2) of a block with exponent e:
// 2^(e - 4(l + 1) + 1); zero blocks (all digits 0) get any valid byte
__device__ __forceinline__ int digit_scale(int e, int l) {
  return e == kZeroExp ? 127 : e - 4 * (l + 1) + 128;
}

// Format helpers (d = 128, four blocks of 32 coordinates; SB = first block of the hi width).
template <int LO, int HI, int SB>
struct Fmt {
  static constexpr int bits(int blk) { return blk < SB ? LO : HI; }
  static constexpr int words(int blk) { return bits(blk) + 1; }  // planes + QJL sign
  static constexpr int off(int blk) {                             // first word of a block
    return blk < SB ? blk * (LO + 1) : SB * (LO + 1) + (blk - SB) * (HI + 1);
  }
  static constexpr int RW = off(4);                               // words per record
  static constexpr int planes(int bits_) { return bits_ == 3 ? 4 : bits_; }  // Walsh terms
  static constexpr int NP = planes(LO) > planes(HI) ? planes(LO) : planes(HI);
};

// Column n of a key group k (0..7) of the tile: token 32 (2x + g0) + 16 s + 4 i + dd with
// k = 4x + i and n = 8 g0 + 4 s + dd.  Lane (h, n) then holds, for each x, the weights of
// 4 tokens that form one dword of the value A operand (see exchange below).
__device__ __forceinline__ int key_token(int k, int n) {
  return 32 * (2 * (k >> 2) + (n >> 3)) + 16 * ((n >> 2) & 1) + 4 * (k & 3) + (n & 3);
}

template <int KLO, int KHI, int KSB, int VLO, int VHI, int VSB>
__global__ __launch_bounds__(kXThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mx_scan(MxParams p) {
  using FK = Fmt<KLO, KHI, KSB>;
  using FV = Fmt<VLO, VHI, VSB>;
  constexpr int NPK = FK::NP;
  constexpr int VGW = 32 * FV::RW;   // words per value group

  __shared__ float s_qrot[4][kD];
  __shared__ float s_sq[4][kD];
  __shared__ float s_hc[4][2];                            // per head: constants Cc, Cs
  __shared__ uint32_t s_ak[NPK + 1][2][6][64];            // key A operands [plane][digits 0-3 / 4-7]
  __shared__ int s_ke[NPK + 1][64];                       // key block exponent of each A lane
  __shared__ int s_ve[kXWaves][2][4][4];                  // value block exponents [type][group][head]
  __shared__ uint32_t s_x[kXWaves][2][4][kXTile];         // rounded weights [type][head][K]
  __shared__ float s_m[kXWaves][4][2];
  __shared__ float s_red[kXWaves][4][2 * kD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x;
  const int unit = blockIdx.y;
  const int nchunk = p.group >> 2;
  const int bkv = unit / nchunk;                  // batch * hkv + kv head
  const int b = bkv / p.hkv;
  const int h0 = (bkv % p.hkv) * p.group + (unit % nchunk) * 4;  // first query head
  const int len = (int)min((int64_t)p.seq_lens[b], p.capacity);
  const int64_t t_beg = (int64_t)split * p.tokens_per_split;
  const int64_t t_end = min(t_beg + p.tokens_per_split, (int64_t)len);
  const int64_t vbase = (int64_t)bkv * p.capacity;   // first vector of this (batch, KV head)

  // lane roles
  const int n = lane & 15, g = lane >> 4;          // B operand: column n, K block g
  const int hh = lane >> 4;                        // C layout: head of this lane
  const int dd = n & 3;                            // token position mod 4 of this lane's tokens
  const float fd = dd == 0 ? 4.0f : dd == 1 ? 2.0f : dd == 2 ? 1.0f : -2.0f;

  // ---- tile loads
  auto tile_start = [&](int it) -> int64_t { return t_beg + (int64_t)(wave + kXWaves * it) * kXTile; };
  uint32_t kw[8][4];       // key block g of token key_token(k, n)
  uint32_t kn[8], vn[8];   // key / value norms of token key_token(k, n) (logit lanes)
  uint32_t vw[8][4];       // value words: coordinate 16 c + n of group g
  auto fetch = [&](int64_t t0, uint32_t (&kw_)[8][4], uint32_t (&kn_)[8], uint32_t (&vn_)[8],
                   uint32_t (&vw_)[8][4]) {
    const int64_t last = p.capacity - 1;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int64_t t = t0 + key_token(k, n);
      t = t > last ? last : t;
      const uint32_t* rec = p.codes_k + (vbase + t) * FK::RW + FK::off(g);
      if constexpr (KLO == KHI) {
        if constexpr (KLO == 3) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(rec);
          kw_[k][0] = w[0]; kw_[k][1] = w[1]; kw_[k][2] = w[2]; kw_[k][3] = w[3];
        } else if constexpr (KLO == 2) {
          kw_[k][0] = rec[0]; kw_[k][1] = rec[1]; kw_[k][2] = rec[2]; kw_[k][3] = 0;
        } else {
          kw_[k][0] = rec[0]; kw_[k][1] = rec[1]; kw_[k][2] = 0; kw_[k][3] = 0;
        }
      } else {
        kw_[k][0] = rec[0]; kw_[k][1] = rec[1]; kw_[k][2] = rec[2];
        kw_[k][3] = FK::bits(g) >= 3 ? rec[3] : 0;
      }
      kn_[k] = p.norms_k[vbase + t];
      vn_[k] = p.norms_v[vbase + t];
    }
    int64_t grp = (vbase + t0) / 32 + g;
    const int64_t glast = (vbase + p.capacity) / 32 - 1;
    grp = grp > glast ? glast : grp;
    const uint32_t* gw = p.codes_v + grp * VGW;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int blk = c >> 1;                     // 32-coordinate block of coordinate 16 c + n
      const int j = 16 * c + n;
      const uint32_t* w = gw + (blk < VSB ? j * (VLO + 1) : 32 * VSB * (VLO + 1) + (j - 32 * VSB) * (VHI + 1));
      const int nb = FV::words(blk);
      if (nb == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(w);
        vw_[c][0] = v[0]; vw_[c][1] = v[1]; vw_[c][2] = v[2]; vw_[c][3] = v[3];
      } else if (nb == 3) {
        vw_[c][0] = w[0]; vw_[c][1] = w[1]; vw_[c][2] = w[2]; vw_[c][3] = 0;
      } else {
        vw_[c][0] = w[0]; vw_[c][1] = w[1]; vw_[c][2] = 0; vw_[c][3] = 0;
      }
    }
  };

  int it = 0;
  const bool has_tile0 = tile_start(0) < t_end;
  if (has_tile0) fetch(tile_start(0), kw, kn, vn, vw);

  // ---- query prologue: q_rot = H D q / sqrt(d), S q_rot, scales, constants, key operands
  {
    const int hd = wave;  // head h0 + wave
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = lane + 64 * e;
      float x = load_elem(p.q, ((int64_t)b * p.hq + h0 + hd) * kD + j, p.q_dtype);
      const uint32_t sw = (lane & 32) ? uniform_u32(p.sign_k[2 * e + 1]) : uniform_u32(p.sign_k[2 * e]);
      if ((sw >> (j & 31)) & 1u) x = -x;
      v[e] = x;
    }
    fwht128(v, lane);
    const float isd = 1.0f / sqrtf((float)kD);
    s_qrot[hd][lane] = v[0] * isd;
    s_qrot[hd][lane + 64] = v[1] * isd;
  }
  __syncthreads();
  {  // S q_rot: wave w rows 32 w .. 32 w + 31; lane (row, half of the columns)
    const int row = 32 * wave + (lane >> 1), half = lane & 1;
    const f32x4* src = reinterpret_cast<const f32x4*>(p.S_k + (int64_t)row * kD + 64 * half);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const f32x4 s = src[c];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const f32x4 qv = *reinterpret_cast<const f32x4*>(&s_qrot[h][64 * half + 4 * c]);
        acc[h] = fmaf(s[0], qv[0], acc[h]);
        acc[h] = fmaf(s[1], qv[1], acc[h]);
        acc[h] = fmaf(s[2], qv[2], acc[h]);
        acc[h] = fmaf(s[3], qv[3], acc[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float tot = acc[h] + __shfl_xor(acc[h], 1, 64);
      if (!half) s_sq[h][row] = tot;
    }
  }
  __syncthreads();
  {  // per head (wave): the constants removed after the products
    const int hd = wave;
    float cc = 0.f, cs = 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = lane + 64 * e;
      if ((j & 3) != 3) {
        const int wsel = (j >> 5) < KSB ? 0 : 1;
        float a = 0.f;
#pragma unroll
        for (int k = 0; k < NPK; ++k) a += p.alpha_k[wsel][k];
        cc = fmaf(a, s_qrot[hd][j], cc);
        cs += s_sq[hd][j];
      }
    }
    cc = wave_sum(cc);
    cs = wave_sum(cs);
    if (lane == 0) {
      s_hc[hd][0] = cc;
      s_hc[hd][1] = cs;
    }
  }
  // key A operands, wave w building planes w, w + 4: A lane (g, m) holds row m = (head m / 4,
  // digit m % 4) for K = 32 g .. 32 g + 31.  K = 32 g + p is coordinate j = 32 g + 4 (p % 8) +
  // p / 8 (nibble p % 8 of dword p / 8 of the B operand), whose nibble weight is f_{p / 8}.
  // a_j = f alpha_k q_rot_j (codebook planes) or f (S q_rot)_j (sign plane); x = |a| 2^-e is
  // truncated to 32 bits: digits 0-3 in one operand, 4-7 in the other.
  {
    const int ga = lane >> 4, m = lane & 15, hd = m >> 2, l = m & 3;
    for (int k = wave; k <= NPK; k += kXWaves) {
      const float alpha = k < NPK ? p.alpha_k[ga < KSB ? 0 : 1][k] : 1.0f;
      const float* src = k < NPK ? &s_qrot[hd][32 * ga] : &s_sq[hd][32 * ga];
      float av[32];
      float amax = 0.f;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        const int D = q >> 3;
        const float f = D == 0 ? 4.0f : D == 1 ? 2.0f : D == 2 ? 1.0f : -2.0f;
        av[q] = f * (alpha * src[4 * (q & 7) + D]);
        amax = fmaxf(amax, fabsf(av[q]));
      }
      const int e = block_exp(amax);
      f32x16 hev, hod, lev, lod;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        const float x = e == kZeroExp ? 0.0f : ldexpf(fabsf(av[q]), -e);
        // digit n of x: floor(x 16^(n+1)) - 16 floor(x 16^n), exact in fp32
        const float t0 = floorf(ldexpf(x, 4 * l)), t1 = floorf(ldexpf(x, 4 * l + 4));
        const float t4 = floorf(ldexpf(x, 4 * l + 16)), t5 = floorf(ldexpf(x, 4 * l + 20));
        float dh = fmaf(-16.0f, t0, t1), dl = fmaf(-16.0f, t4, t5);
        if (av[q] < 0.0f) {
          dh = -dh;
          dl = -dl;
        }
        if (q & 1) {
          hod[q >> 1] = dh;
          lod[q >> 1] = dl;
        } else {
          hev[q >> 1] = dh;
          lev[q >> 1] = dl;
        }
      }
      const i32x8 ah = fp6_row(hev, hod), al = fp6_row(lev, lod);
#pragma unroll
      for (int r = 0; r < 6; ++r) {
        s_ak[k][0][r][lane] = (uint32_t)ah[r];
        s_ak[k][1][r][lane] = (uint32_t)al[r];
      }
      s_ke[k][lane] = e;
    }
  }
  __syncthreads();
  i32x8 akh[NPK + 1], akl[NPK + 1];
  int ksh[NPK + 1], ksl[NPK + 1];   // this lane's row scales (row lane & 15, block lane >> 4)
#pragma unroll
  for (int k = 0; k <= NPK; ++k) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      akh[k][r] = r < 6 ? (int)s_ak[k][0][r][lane] : 0;
      akl[k][r] = r < 6 ? (int)s_ak[k][1][r][lane] : 0;
    }
    const int e = s_ke[k][lane];
    ksh[k] = digit_scale(e, lane & 3);
    ksl[k] = digit_scale(e, 4 + (lane & 3));
  }
  const float lscale = p.scale * 1.4426950408889634f;   // logits in the log2 domain
  const float cc_h = s_hc[hh][0], cs_h = s_hc[hh][1];
  const float lsg = lscale * p.gamma;

  // ---- running state (lane (hh, n))
  float m_run = -INFINITY, l_part = 0.f, u3 = 0.f, u3s = 0.f;
  unsigned long long n_skip = 0;
  // value sums: arun[c] = sum_k alpha_k (products of plane k), one fp32 sum per digit row,
  // updated after each tile; accs[c] = sign products (one plane, kept on the MFMA)
  f32x4 arun[8], accs[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    accs[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
    arun[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  uint32_t* xw = &s_x[wave][0][0][0];
  const int g0 = n >> 3, sx = (n >> 2) & 1;
  const int gA_w = 2 * g0 + (dd >> 1);            // value A lane group of this lane's tokens
  const float fv = dd == 0 ? 4.0f : dd == 1 ? 2.0f : dd == 2 ? 1.0f : 2.0f;  // value A weights
  const float fvi = 1.0f / fv;
  int* ve = &s_ve[wave][0][0][0];

  for (; tile_start(it) < t_end; ++it) {
    const int64_t t0 = tile_start(it);
    // next tile in flight while this one is computed
    uint32_t nkw[8][4], nkn[8], nvn[8], nvw[8][4];
    const bool more = tile_start(it + 1) < t_end;
    if (more) fetch(tile_start(it + 1), nkw, nkn, nvn, nvw);

    // -- keys: logits of head hh for tokens key_token(k, n)
    float lg[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t p0 = kw[k][0], p1 = kw[k][1];
      uint32_t p2, sg;
      if constexpr (KLO == KHI) {
        p2 = KLO >= 3 ? kw[k][2] : 0u;
        sg = kw[k][KLO];
      } else {
        const bool w3 = FK::bits(g) >= 3;
        p2 = w3 ? kw[k][2] : 0u;
        sg = w3 ? kw[k][3] : kw[k][2];
      }
      f32x4 ac = {0.f, 0.f, 0.f, 0.f}, as = {0.f, 0.f, 0.f, 0.f};
      {
        const i32x4 b0 = fp4_of(p0);
        ac = mma(akh[0], b0, ac, ksh[0]);
        ac = mma(akl[0], b0, ac, ksl[0]);
      }
      if constexpr (NPK >= 2) {
        const i32x4 b1 = fp4_of(p1);
        ac = mma(akh[1], b1, ac, ksh[1]);
        ac = mma(akl[1], b1, ac, ksl[1]);
      }
      if constexpr (NPK >= 3) {
        const i32x4 b2 = fp4_of(p2), b3 = fp4_of(p0 ^ p1 ^ p2);
        ac = mma(akh[2], b2, ac, ksh[2]);
        ac = mma(akl[2], b2, ac, ksl[2]);
        ac = mma(akh[3], b3, ac, ksh[3]);
        ac = mma(akl[3], b3, ac, ksl[3]);
      }
      {
        const i32x4 bs = fp4_of(sg);
        as = mma(akh[NPK], bs, as, ksh[NPK]);
        as = mma(akl[NPK], bs, as, ksl[NPK]);
      }
      const float dc = ((ac[0] + ac[1]) + (ac[2] + ac[3]) - cc_h) * lscale;
      const float ds = ((as[0] + as[1]) + (as[2] + as[3]) - cs_h) * lsg;
      const float n16 = f16_bits_to_f32(kn[k]), r16 = f16_bits_to_f32(kn[k] >> 16);
      const int64_t t = t0 + key_token(k, n);
      lg[k] = t < t_end ? fmaf(n16, dc, r16 * ds) : -INFINITY;
    }
    if (p.logits) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t t = t0 + key_token(k, n);
        if (t < t_end)
          p.logits[((int64_t)b * p.hq + h0 + hh) * p.capacity + t] = lg[k] * 0.6931471805599453f;
      }
    }
    // -- online softmax (head hh spans the 16 lanes of its row)
    float tm = lg[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) tm = fmaxf(tm, lg[k]);
    tm = fmaxf(tm, __shfl_xor(tm, 1, 64));
    tm = fmaxf(tm, __shfl_xor(tm, 2, 64));
    tm = fmaxf(tm, __shfl_xor(tm, 4, 64));
    tm = fmaxf(tm, __shfl_xor(tm, 8, 64));
    const float m_new = fmaxf(m_run, tm);
    const bool rescale_m = m_new > m_run && m_run != -INFINITY;
    if (__ballot(rescale_m) != 0) {
      const float fm = rescale_m ? exp2f(m_run - m_new) : 1.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        accs[c] *= fm;
        arun[c] *= fm;
      }
      l_part *= fm;
      u3 *= fm;
      u3s *= fm;
    }
    m_run = m_new;
    float w[8];
    float tsum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      w[k] = lg[k] == -INFINITY ? 0.0f : exp2f(lg[k] - m_run);
      tsum += w[k];
    }
    l_part += tsum;
    if (p.tau > 0.0f) {  // Sparse V: drop weights below tau times the running sum (an upper bound)
      float lrun = l_part;
      lrun += __shfl_xor(lrun, 1, 64);
      lrun += __shfl_xor(lrun, 2, 64);
      lrun += __shfl_xor(lrun, 4, 64);
      lrun += __shfl_xor(lrun, 8, 64);
      const float thr = p.tau * lrun;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool drop = w[k] < thr;
        const unsigned long long bm = __ballot(drop && t0 + key_token(k, n) < t_end);
        const unsigned long long all4 = bm & (bm >> 16) & (bm >> 32) & (bm >> 48) & 0xFFFFull;
        n_skip += __builtin_popcountll(all4);
        if (drop) w[k] = 0.0f;
      }
    }
    // -- value weights u = w n16_v and u' = w r16_v (gamma applied after the sums), times the
    // nibble weight f_D, as 16-bit integers x 2^(e - 16) with a block exponent e per head and
    // 32-token group; K index of token 16 sx + 4 i + dd of a group: 8 dd + 4 sx + i
    {
      float u[8], us[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float n16 = f16_bits_to_f32(vn[k]), r16 = f16_bits_to_f32(vn[k] >> 16);
        u[k] = w[k] > 0.0f ? w[k] * n16 * fv : 0.0f;
        us[k] = w[k] > 0.0f ? w[k] * r16 * fv : 0.0f;
      }
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        // group 2x + g0 of the tile: its 32 tokens sit in the 8 lanes n = 8 g0 .. 8 g0 + 7
        float mu = fmaxf(fmaxf(u[4 * x], u[4 * x + 1]), fmaxf(u[4 * x + 2], u[4 * x + 3]));
        float ms = fmaxf(fmaxf(us[4 * x], us[4 * x + 1]), fmaxf(us[4 * x + 2], us[4 * x + 3]));
        mu = fmaxf(mu, xchg<1>(mu));
        ms = fmaxf(ms, xchg<1>(ms));
        mu = fmaxf(mu, xchg<2>(mu));
        ms = fmaxf(ms, xchg<2>(ms));
        mu = fmaxf(mu, xchg<4>(mu));
        ms = fmaxf(ms, xchg<4>(ms));
        const int eu = block_exp(mu), es = block_exp(ms);
        u32x4 ru, rs;
        float su = 0.f, ss = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = eu == kZeroExp ? 0.0f : fminf(__builtin_rintf(ldexpf(u[4 * x + i], 16 - eu)), 65535.0f);
          const float c = es == kZeroExp ? 0.0f : fminf(__builtin_rintf(ldexpf(us[4 * x + i], 16 - es)), 65535.0f);
          ru[i] = (uint32_t)a;
          rs[i] = (uint32_t)c;
          su += a;
          ss += c;
        }
        // the constant removed after the products: sum over positions D < 3 of the rounded
        // weights divided by f_D (exact: integers below 2^18 times powers of two)
        if (dd != 3) {
          u3 += eu == kZeroExp ? 0.0f : ldexpf(su, eu - 16) * fvi;
          u3s += es == kZeroExp ? 0.0f : ldexpf(ss, es - 16) * fvi;
        }
        const int kk = 32 * (2 * x + g0) + 8 * dd + 4 * sx;
        *reinterpret_cast<u32x4*>(&xw[(0 * 4 + hh) * kXTile + kk]) = ru;
        *reinterpret_cast<u32x4*>(&xw[(1 * 4 + hh) * kXTile + kk]) = rs;
        if ((n & 7) == 0) {
          ve[(0 * 4 + 2 * x + g0) * 4 + hh] = eu;
          ve[(1 * 4 + 2 * x + g0) * 4 + hh] = es;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // A lane (g, m): row m = (head m / 4, digit m % 4) of the 32 tokens of group g
    i32x8 au, as_;
    int vsu, vss;
    {
      const int ga = lane >> 4, ha = (lane & 15) >> 2, sh = 12 - 4 * (lane & 3);
#pragma unroll
      for (int type = 0; type < 2; ++type) {
        const uint32_t* src = &xw[(type * 4 + ha) * kXTile + 32 * ga];
        f32x16 ev, od;
#pragma unroll
        for (int c4 = 0; c4 < 8; ++c4) {
          const u32x4 r = *reinterpret_cast<const u32x4*>(src + 4 * c4);
          ev[2 * c4] = (float)((r[0] >> sh) & 15u);
          od[2 * c4] = (float)((r[1] >> sh) & 15u);
          ev[2 * c4 + 1] = (float)((r[2] >> sh) & 15u);
          od[2 * c4 + 1] = (float)((r[3] >> sh) & 15u);
        }
        const i32x8 op = fp6_row(ev, od);
        const int sc = digit_scale(ve[(type * 4 + ga) * 4 + ha], lane & 3);
        if (type == 0) {
          au = op;
          vsu = sc;
        } else {
          as_ = op;
          vss = sc;
        }
      }
    }
    // -- values: one product per plane and 16-coordinate block over the 128 tokens; the
    // codebook planes' products are folded with their Walsh coefficients right away
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int bits = FV::bits(c >> 1);
      const int wsel = (c >> 1) < VSB ? 0 : 1;
      const uint32_t p0 = vw[c][0], p1 = vw[c][1];
      const uint32_t p2 = bits >= 3 ? vw[c][2] : 0u;
      const uint32_t sg = vw[c][bits];
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 t0 = mma(au, fp4_pos(p0), z, vsu);
      f32x4 a = arun[c] + p.alpha_v[wsel][0] * t0;
      if (bits >= 2) {
        const f32x4 t1 = mma(au, fp4_pos(p1), z, vsu);
        a += p.alpha_v[wsel][1] * t1;
      }
      if (bits >= 3) {
        const f32x4 t2 = mma(au, fp4_pos(p2), z, vsu);
        const f32x4 t3 = mma(au, fp4_pos(p0 ^ p1 ^ p2), z, vsu);
        a += p.alpha_v[wsel][2] * t2;
        a += p.alpha_v[wsel][3] * t3;
      }
      arun[c] = a;
      accs[c] = mma(as_, fp4_pos(sg), accs[c], vss);
    }
    if (more) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        kn[k] = nkn[k];
        vn[k] = nvn[k];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kw[k][i] = nkw[k][i];
          vw[k][i] = nvw[k][i];
        }
      }
    }
  }

  // ---- wave partial: per head the running max, the sum of weights and the rotated-domain
  // sums A[j] = sum_k alpha_k (sum_t u_t s_k,t,j), Q[j] = sum_t u'_t sigma_t,j
  float lh = l_part, u3h = u3, u3sh = u3s;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    lh += __shfl_xor(lh, o, 64);
    u3h += __shfl_xor(u3h, o, 64);
    u3sh += __shfl_xor(u3sh, o, 64);
  }
  if (n == 0) {
    s_m[wave][hh][0] = m_run;
    s_m[wave][hh][1] = lh;
  }
  {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int bits = FV::bits(c >> 1);
      const int wsel = (c >> 1) < VSB ? 0 : 1;
      float asum = 0.f;   // sum of the Walsh coefficients: the constant's weight in A
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < FV::planes(bits)) asum += p.alpha_v[wsel][k];
      const f32x4 ra = arun[c];
      const float a = ((ra[0] + ra[1]) + (ra[2] + ra[3])) - asum * u3h;
      const f32x4 r = accs[c];
      const float qv = ((r[0] + r[1]) + (r[2] + r[3])) - u3sh;
      s_red[wave][hh][16 * c + n] = a;
      s_red[wave][hh][kD + 16 * c + n] = qv * p.gamma;
    }
  }
  __syncthreads();
  // ---- merge the 4 waves; one partial per (query head, split): m, l, then A and Q
  {
    float* part0 = p.ws_part + (((int64_t)b * p.hq + h0) * p.n_split + split) * kPartFloats;
    const int64_t hstride = (int64_t)p.n_split * kPartFloats;
    for (int o = tid; o < 4 * 2 * kD; o += kXThreads) {
      const int hd = o >> 8, f = o & 255;
      const float m0 = s_m[0][hd][0], m1 = s_m[1][hd][0], m2 = s_m[2][hd][0], m3 = s_m[3][hd][0];
      const float M = fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
      float acc_o = 0.f;
#pragma unroll
      for (int w = 0; w < kXWaves; ++w) {
        const float mw = w == 0 ? m0 : w == 1 ? m1 : w == 2 ? m2 : m3;
        const float sc = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
        acc_o = fmaf(sc, s_red[w][hd][f], acc_o);
      }
      part0[hd * hstride + 2 + f] = acc_o;
    }
    if (tid < 4) {
      const int hd = tid;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kXWaves; ++w) M = fmaxf(M, s_m[w][hd][0]);
      float l_o = 0.f;
#pragma unroll
      for (int w = 0; w < kXWaves; ++w) {
        const float mw = s_m[w][hd][0];
        l_o = fmaf((mw == -INFINITY) ? 0.0f : exp2f(mw - M), s_m[w][hd][1], l_o);
      }
      part0[hd * hstride] = M;
      part0[hd * hstride + 1] = l_o;
    }
  }
  if (p.skipped && p.tau > 0.0f && lane == 0 && n_skip) atomicAdd(p.skipped, n_skip);
}

template <int KLO, int KHI, int KSB, int VLO, int VHI, int VSB>
int launch_mx(const MxParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_mx_scan<KLO, KHI, KSB, VLO, VHI, VSB>), grid, dim3(kXThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

}  // namespace tqx

// (key lo, key hi, key split block, value lo, value hi, value split block); split block 4 =
// one width.  These are the format pairs with a token-sliced value path.
#define TQ_MX_PAIRS(X)   \
  X(3, 3, 4, 3, 3, 4)    \
  X(3, 3, 4, 2, 2, 4)    \
  X(3, 2, 2, 3, 2, 2)    \
  X(2, 2, 4, 2, 2, 4)

namespace {
void mx_shape(const tq_format* f, int& lo, int& hi, int& sb) {
  lo = f->bits_lo;
  hi = f->split == f->d ? f->bits_lo : f->bits_hi;
  sb = lo == hi ? 4 : f->split / 32;
}
}  // namespace

bool tq_decode_mx_supported(const tq_format* fk, const tq_format* fv) {
  if (!fk->qjl || !fv->qjl || fk->layout != 0 || fv->layout != 1) return false;
  int kl, kh, ks, vl, vh, vs;
  mx_shape(fk, kl, kh, ks);
  mx_shape(fv, vl, vh, vs);
#define TQ_MX_MATCH(a, b_, c, d, e, f) \
  if (kl == a && kh == b_ && ks == c && vl == d && vh == e && vs == f) return true;
  TQ_MX_PAIRS(TQ_MX_MATCH)
#undef TQ_MX_MATCH
  return false;
}

// The split plan of the per-vector path (same split count and workspace, so
// tq_attend_workspace_bytes covers both), with splits rounded to whole workgroup steps.
tq_decode_plan tq_plan_decode_mx(int32_t batch, int32_t hq, int32_t hkv, int64_t capacity) {
  using namespace tqx;
  tq_decode_plan p = tq_plan_decode(batch, hq, hkv, capacity, 128);
  const int64_t per_wg = (int64_t)kXTile * kXWaves;
  p.tokens_per_split = (p.tokens_per_split + per_wg - 1) / per_wg * per_wg;
  p.waves = kXWaves;
  return p;
}

int tq_launch_decode_mx(const tq_format* fk, const tq_tables* tk, const tq_format* fv,
                        const tq_tables* tv, const void* q, int32_t q_dtype, int32_t batch,
                        int32_t hq, int32_t hkv, const void* codes_k, const uint16_t* norms_k,
                        const void* codes_v, const uint16_t* norms_v, int64_t capacity,
                        const int32_t* seq_lens, float scale, float tau, float* out,
                        float* logits, int64_t* skipped, void* workspace,
                        const tq_decode_plan& plan, hipStream_t stream) {
  using namespace tqx;
  MxParams p{};
  p.q = q;
  p.codes_k = reinterpret_cast<const uint32_t*>(codes_k);
  p.norms_k = reinterpret_cast<const uint32_t*>(norms_k);
  p.codes_v = reinterpret_cast<const uint32_t*>(codes_v);
  p.norms_v = reinterpret_cast<const uint32_t*>(norms_v);
  p.seq_lens = seq_lens;
  p.S_k = tk->S;
  p.ws_part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + plan.ws_part_off);
  p.logits = logits;
  p.skipped = reinterpret_cast<unsigned long long*>(skipped);
  p.capacity = capacity;
  p.tokens_per_split = plan.tokens_per_split;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  p.q_dtype = q_dtype;
  p.n_split = plan.n_split;
  p.scale = scale;
  p.tau = tau;
  p.gamma = (float)(std::sqrt(M_PI / 2.0) / fk->d);
  for (int i = 0; i < 4; ++i) p.sign_k[i] = 0;
  for (int j = 0; j < 128; ++j)
    if (tk->signs[j] < 0) p.sign_k[j >> 5] |= 1u << (j & 31);
  tq_walsh_coeffs(fk->bits_lo, tk->centroids_lo, p.alpha_k[0]);
  tq_walsh_coeffs(fk->split == fk->d ? fk->bits_lo : fk->bits_hi,
                  fk->split == fk->d ? tk->centroids_lo : tk->centroids_hi, p.alpha_k[1]);
  tq_walsh_coeffs(fv->bits_lo, tv->centroids_lo, p.alpha_v[0]);
  tq_walsh_coeffs(fv->split == fv->d ? fv->bits_lo : fv->bits_hi,
                  fv->split == fv->d ? tv->centroids_lo : tv->centroids_hi, p.alpha_v[1]);
  const dim3 grid((unsigned)plan.n_split, (unsigned)(batch * hkv * (hq / hkv / 4)));
  int kl, kh, ks, vl, vh, vs;
  mx_shape(fk, kl, kh, ks);
  mx_shape(fv, vl, vh, vs);
  int rc = TQ_ERR_SHAPE;
#define TQ_MX_LAUNCH(a, b_, c, d, e, f)                                  \
  if (kl == a && kh == b_ && ks == c && vl == d && vh == e && vs == f)   \
    rc = launch_mx<a, b_, c, d, e, f>(p, grid, stream);                   \
  else
  TQ_MX_PAIRS(TQ_MX_LAUNCH) {}
#undef TQ_MX_LAUNCH
  if (rc != TQ_OK) return rc;
  // split merge and rotation back: the per-vector path's combine (same partial format)
  tqk::DecodeParams c{};
  c.S_v = tv->S;
  c.out = out;
  c.ws_part = p.ws_part;
  c.n_split = plan.n_split;
  for (int i = 0; i < 4; ++i) c.sign_v[i] = 0;
  for (int j = 0; j < 128; ++j)
    if (tv->signs[j] < 0) c.sign_v[j >> 5] |= 1u << (j & 31);
  return tqk::launch_decode_combine(c, batch * hq, stream);
}
