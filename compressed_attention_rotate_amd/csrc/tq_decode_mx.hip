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
// gives -0.5 s.  Scaling the matching A entries by 4, 2, 1, -2 turns every product into
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
#include <type_traits>

#include "tq_decode_kernel.h"
#include "tq_mx.h"

namespace tqx {
using namespace tqk;

typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

constexpr int kXWaves = 4;
constexpr int kXThreads = 64 * kXWaves;
constexpr int kXTile = 128;      // tokens per wave tile
// hand-off rows of 32 16-bit weights (one head, type and 32-token group; two per dword, K order)
// padded to 20 dwords, so the 16 rows one A-operand read touches start on 16 different 4-bank
// groups
constexpr int kXRow = 20;

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

// acc += A (fp6 digit rows, scale byte sa) x B (fp4) with acc held in accumulation registers
// (AGPRs) across the whole scan: value sums that are only read after the last tile never take
// vector registers or instructions.  Written as an instruction because the rest of this file
// keeps its MFMA results in VGPRs; the leading s_nop gives the two wait states an MFMA needs
// after a VALU write of its A or B registers (hazards the compiler does not see inside asm).
// Readers of acc must come at least 20 wait states after the last accumulation.
__device__ __forceinline__ void mma_acc(f32x4& acc, const i32x8& a, const i32x4& b, int sa) {
  const i32x6 a6 = {a[0], a[1], a[2], a[3], a[4], a[5]};
  asm("s_nop 1\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:2 blgp:4"
      : "+a"(acc)
      : "v"(a6), "v"(b), "v"(sa), "v"(127));
}

// The value of the other quad of this lane's 8-lane group (DPP row_half_mirror: lane i and
// lane 7 - i of each half row): the xor-4 partner's value once the value is uniform within
// each quad, as it is after exchanges at distances 1 and 2.  A DPP move, not an LDS swizzle.
__device__ __forceinline__ float quad_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
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
// 4 tokens with consecutive K indices of the value A operand (see the hand-off below).
__device__ __forceinline__ int key_token(int k, int n) {
  return 32 * (2 * (k >> 2) + (n >> 3)) + 16 * ((n >> 2) & 1) + 4 * (k & 3) + (n & 3);
}

typedef int i32x4s __attribute__((ext_vector_type(4)));
constexpr int kRsrcFlags = 0x00020000;   // raw (unformatted) 32-bit buffer, gfx9 family

// A buffer resource (V#) over [base, base + bytes), wave-uniform: loads past the end return
// zero.  base and bytes must be the same in every lane.
__device__ __forceinline__ i32x4s make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return (i32x4s){__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                  __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu)),
                  __builtin_amdgcn_readfirstlane(n), kRsrcFlags};
}

// Buffer loads straight to LDS: lane L's SZ bytes from rsrc at voffset + soffset land at the
// LDS address m0 + L * 16 (SZ = 16, 12) or m0 + L * 4 (SZ = 4).  Written as instructions so
// that the compiler, which cannot tell the LDS image from the rest of LDS, does not wait
// for them before every LDS access; the caller waits (vmcnt) before reading the image.
// The LDS address is lds_base + LOFF and the scalar offset SOFF, both compile-time constants
// added inside the statement (kept as operands, the 40-odd constants of a tile's loads would
// occupy scalar registers for the whole scan and push others out to vector-register lanes).
// No vector register is written.
template <int SZ, int LOFF, int SOFF>
__device__ __forceinline__ void load_lds(const i32x4s& rsrc, uint32_t lds_base, int voffset) {
  int so;
  if constexpr (SZ == 16)
    asm volatile("s_add_u32 m0, %1, %4\n\ts_mov_b32 %0, %5\n\tbuffer_load_dwordx4 %2, %3, %0 offen lds"
                 : "=&s"(so) : "s"(lds_base), "v"(voffset), "s"(rsrc), "i"(LOFF), "i"(SOFF)
                 : "memory", "m0", "scc");
  else if constexpr (SZ == 12)
    asm volatile("s_add_u32 m0, %1, %4\n\ts_mov_b32 %0, %5\n\tbuffer_load_dwordx3 %2, %3, %0 offen lds"
                 : "=&s"(so) : "s"(lds_base), "v"(voffset), "s"(rsrc), "i"(LOFF), "i"(SOFF)
                 : "memory", "m0", "scc");
  else
    asm volatile("s_add_u32 m0, %1, %4\n\ts_mov_b32 %0, %5\n\tbuffer_load_dword %2, %3, %0 offen lds"
                 : "=&s"(so) : "s"(lds_base), "v"(voffset), "s"(rsrc), "i"(LOFF), "i"(SOFF)
                 : "memory", "m0", "scc");
}

// Calls f(std::integral_constant<int, I>) for I = B .. E - 1 (a loop with a compile-time index).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS image of one 128-token tile, filled by buffer loads straight to LDS (lane L's bytes of
// one load land at L * 16 for 16- and 12-byte loads, L * 4 for 4-byte loads): dword offsets
constexpr int kTKw = 0;                 // [8 key groups][64 lanes][4]
constexpr int kTKn = kTKw + 8 * 64 * 4;  // [8][64] key norms
constexpr int kTVn = kTKn + 8 * 64;      // [8][64] value norms
constexpr int kTVw = kTVn + 8 * 64;      // [8 coordinate blocks][64 lanes][4]
constexpr int kTileDw = kTVw + 8 * 64 * 4;

// s_waitcnt immediates (gfx9 encoding): all vector memory done / all LDS operations done
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

// The records of one 128-token tile as this lane reads them.
struct TileRegs {
  u32x4 kw[8];        // key block g of token key_token(k, n)
  uint32_t kn[8];     // key norms (fp16 ||x|| | fp16 ||r|| << 16) of the same tokens
  uint32_t vn[8];     // value norms of the same tokens
  u32x4 vw[8];        // value words of coordinate 16 c + n, 32-token group g of the tile
};

// LA (long scans, many tiles per wave): the value products of every codebook plane keep their
// own accumulators over the whole scan, folded with the Walsh coefficients once at the end;
// otherwise each tile's products are folded right away (cheaper set-up and end for a few tiles).
template <int KLO, int KHI, int KSB, int VLO, int VHI, int VSB, bool LA>
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
  __shared__ __align__(16) uint32_t s_x[kXWaves][2 * 4 * 4 * kXRow];   // rounded weights [type][head][group][K / 2]
  __shared__ float s_m[kXWaves][4][2];
  __shared__ float s_red[kXWaves][4][2 * kD];
  __shared__ __align__(16) uint32_t s_tile[kXWaves][kTileDw];   // next tile, in flight

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform in the wave
  const int split = blockIdx.x;
  const int unit = blockIdx.y;
  const int nchunk = p.group >> 2;
  const int bkv = unit / nchunk;                  // batch * hkv + kv head
  const int b = bkv / p.hkv;
  const int h0 = (bkv % p.hkv) * p.group + (unit % nchunk) * 4;  // first query head
  const int len = __builtin_amdgcn_readfirstlane((int)min((int64_t)p.seq_lens[b], p.capacity));
  const int64_t t_beg = (int64_t)split * p.tokens_per_split;
  const int64_t t_end = min(t_beg + p.tokens_per_split, (int64_t)len);
  const int64_t vbase = (int64_t)bkv * p.capacity;   // first vector of this (batch, KV head)

  // lane roles
  const int n = lane & 15, g = lane >> 4;          // B operand: column n, K block g
  const int hh = lane >> 4;                        // C layout: head of this lane
  const int dd = n & 3;                            // token position mod 4 of this lane's tokens

  // ---- query and S loads first, all in flight together (the tile loads are issued once they
  // have arrived): the query elements lane and lane + 64 as raw bits from one uniform branch
  // on the type, converted after the S loads are issued, so that no wait splits them
  uint32_t qraw[2];
  {
    const int64_t qi = ((int64_t)b * p.hq + h0 + wave) * kD + lane;
    if (p.q_dtype == 0 || p.q_dtype == 3) {
      const uint32_t* qp = reinterpret_cast<const uint32_t*>(p.q) + qi;
      qraw[0] = qp[0];
      qraw[1] = qp[64];
    } else {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + qi;
      qraw[0] = qp[0];
      qraw[1] = qp[64];
    }
  }
  // S rows 32 wave .. 32 wave + 31: srow[4 r + c] holds row 32 wave + 8 r + lane / 8, columns
  // 32 c + 4 (lane % 8) .. + 3, so the eight lanes of a row read one whole 128-byte line
  f32x4 srow[16];
  {
    const float* src = p.S_k + (int64_t)(32 * wave + (lane >> 3)) * kD + 4 * (lane & 7);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      srow[i] = *reinterpret_cast<const f32x4*>(src + (i >> 2) * 8 * kD + (i & 3) * 32);
  }

  float qx[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    qx[e] = (p.q_dtype == 0 || p.q_dtype == 3) ? __uint_as_float(qraw[e])
            : p.q_dtype == 1                  ? __uint_as_float(qraw[e] << 16)
                                              : f16_bits_to_f32(qraw[e]);

  // ---- tile loads through buffer resources based at the tile: per-lane offsets are
  // constants, the tile start only moves the (scalar) base
  auto tile_start = [&](int i) -> int64_t { return t_beg + (int64_t)(wave + kXWaves * i) * kXTile; };
  const int tok0 = key_token(0, n);                         // + 64 (k >> 2) + 4 (k & 3)
  const int koff = tok0 * FK::RW * 4 + FK::off(g) * 4;
  const int noff = tok0 * 4;
  // value words of coordinate j = 16 c + n in group g: the lo-width region for j < 32 VSB
  const int voff_lo = g * VGW * 4 + n * (VLO + 1) * 4;
  const int voff_hi = g * VGW * 4 + (32 * VSB * (VLO + 1) + n * (VHI + 1)) * 4;
  uint32_t* tl = &s_tile[wave][0];
  const uint32_t tl_addr = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)reinterpret_cast<uintptr_t>((lds_ptr_t)tl));   // LDS byte address
  // the loads of the tile at t0 into this wave's LDS image (no registers), through buffer
  // resources over the records from t0 on; with valid false the resources are empty, so the
  // loads read nothing from memory (the image gets zeros)
  struct TileRes {
    i32x4s rk, rnk, rnv, rv;
  };
  auto tile_res = [&](int64_t t0, bool valid) {
    const int64_t left = valid ? p.capacity - t0 : 0;   // tokens of this (batch, KV head) from t0 on
    TileRes r;
    r.rk = make_rsrc(p.codes_k + (vbase + t0) * FK::RW, left * FK::RW * 4);
    r.rnk = make_rsrc(p.norms_k + vbase + t0, left * 4);
    r.rnv = make_rsrc(p.norms_v + vbase + t0, left * 4);
    r.rv = make_rsrc(p.codes_v + ((vbase + t0) >> 5) * VGW, (left >> 5) * VGW * 4);
    return r;
  };
  auto dma_keys = [&](const TileRes& r, auto kc) {   // key group k: records and both norms
    constexpr int k = decltype(kc)::value;
    constexpr int dt = 64 * (k >> 2) + 4 * (k & 3);     // token offset of key group k
    load_lds<16, 4 * (kTKw + k * 256), dt * FK::RW * 4>(r.rk, tl_addr, koff);
    load_lds<4, 4 * (kTKn + k * 64), dt * 4>(r.rnk, tl_addr, noff);
    load_lds<4, 4 * (kTVn + k * 64), dt * 4>(r.rnv, tl_addr, noff);
  };
  auto dma_values = [&](const TileRes& r) {
    static_for<0, 8>([&](auto cc) __attribute__((always_inline)) {
      constexpr int c = decltype(cc)::value;
      constexpr int blk = c >> 1;
      constexpr int so = blk < VSB ? 16 * c * (VLO + 1) * 4 : (16 * c - 32 * VSB) * (VHI + 1) * 4;
      const int vo = blk < VSB ? voff_lo : voff_hi;
      if constexpr (FV::words(blk) == 4)
        load_lds<16, 4 * (kTVw + c * 256), so>(r.rv, tl_addr, vo);
      else
        load_lds<12, 4 * (kTVw + c * 256), so>(r.rv, tl_addr, vo);
    });
  };
  auto dma = [&](int64_t t0) {
    const TileRes r = tile_res(t0, true);
    static_for<0, 8>([&](auto kc) __attribute__((always_inline)) { dma_keys(r, kc); });
    dma_values(r);
  };
  // this lane's part of the LDS image into registers (after the tile's loads completed)
  auto read_tile = [&](TileRegs& T) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      T.kw[k] = *reinterpret_cast<const u32x4*>(tl + kTKw + k * 256 + 4 * lane);
      T.kn[k] = tl[kTKn + k * 64 + lane];
      T.vn[k] = tl[kTVn + k * 64 + lane];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(tl + kTVw + c * 256 + 4 * lane);
      T.vw[c] = FV::words(c >> 1) == 4 ? w : (u32x4){w[0], w[1], w[2], 0u};
    }
  };

  // the query and S rows first, then the first tile in flight while the prologue runs
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  asm volatile("" ::: "memory");
  if (tile_start(0) < t_end) dma(tile_start(0));

  // ---- query prologue: q_rot = H D q / sqrt(d) (wave = head), then S q_rot
  {
    const int hd = wave;
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = lane + 64 * e;
      const uint32_t sw = (lane & 32) ? uniform_u32(p.sign_k[2 * e + 1]) : uniform_u32(p.sign_k[2 * e]);
      v[e] = ((sw >> (j & 31)) & 1u) ? -qx[e] : qx[e];
    }
    fwht128(v, lane);
    const float isd = 1.0f / sqrtf((float)kD);
    s_qrot[hd][lane] = v[0] * isd;
    s_qrot[hd][lane + 64] = v[1] * isd;
  }
  __syncthreads();
  {  // S q_rot: wave w rows 32 w .. 32 w + 31; eight lanes per row, summed across them
    float acc[4][4];   // [row group r][head]
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int h = 0; h < 4; ++h) acc[r][h] = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const f32x4 qv = *reinterpret_cast<const f32x4*>(&s_qrot[h][32 * c + 4 * (lane & 7)]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4 sv = srow[4 * r + c];
          acc[r][h] = fmaf(sv[0], qv[0], acc[r][h]);
          acc[r][h] = fmaf(sv[1], qv[1], acc[r][h]);
          acc[r][h] = fmaf(sv[2], qv[2], acc[r][h]);
          acc[r][h] = fmaf(sv[3], qv[3], acc[r][h]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        float t = acc[r][h];
        t += xchg<1>(t);
        t += xchg<2>(t);
        t += quad_swap(t);
        if ((lane & 7) == 0) s_sq[h][32 * wave + 8 * r + (lane >> 3)] = t;
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
    cc = wave_sum_fast(cc);
    cs = wave_sum_fast(cs);
    if (lane == 0) {
      s_hc[hd][0] = cc;
      s_hc[hd][1] = cs;
    }
  }
  // key A operands, wave w building plane w (and, for a fifth plane, waves 0 and 1 its digit
  // rows 0-3 and 4-7): A lane (g, m) holds row m = (head m / 4,
  // digit m % 4) for K = 32 g .. 32 g + 31.  K = 32 g + p is coordinate j = 32 g + 4 (p % 8) +
  // p / 8 (nibble p % 8 of dword p / 8 of the B operand), whose nibble weight is f_{p / 8}.
  // a_j = f alpha_k q_rot_j (codebook planes) or f (S q_rot)_j (sign plane); x = |a| 2^-e is
  // truncated to 32 bits (x 2^32 as an integer): digits 0-3 in one operand, 4-7 in the other.
  {
    const int ga = lane >> 4, m = lane & 15, hd = m >> 2, l = m & 3;
    auto build = [&](int k, bool hi, bool lo) {
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
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        if (part == 0 ? !hi : !lo) continue;
        const int sh = (part == 0 ? 28 : 12) - 4 * l;   // digit l (or 4 + l) of x 2^32
        // digits as f16 bit patterns, two per dword, signs in bits 15 and 31 (see fp6_row_f16)
        u32x16 hd16;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float a0 = av[2 * i], a1 = av[2 * i + 1];
          const uint32_t r0 = e == kZeroExp ? 0u : (uint32_t)ldexpf(fabsf(a0), 32 - e);
          const uint32_t r1 = e == kZeroExp ? 0u : (uint32_t)ldexpf(fabsf(a1), 32 - e);
          hd16[i] = ((r0 >> sh) & 15u) | (((r1 >> sh) & 15u) << 16) |
                    ((__float_as_uint(a0) >> 16) & 0x8000u) | (__float_as_uint(a1) & 0x80000000u);
        }
        const i32x8 a = fp6_row_f16(hd16);
#pragma unroll
        for (int r = 0; r < 6; ++r) s_ak[k][part][r][lane] = (uint32_t)a[r];
      }
      if (hi) s_ke[k][lane] = e;
    };
    if (wave <= NPK) build(wave, true, true);
    if (NPK == 4 && wave < 2) build(4, wave == 0, wave == 1);
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
  // the constants removed after the key products seed their accumulators instead
  const f32x4 c0_c = {-s_hc[hh][0], 0.f, 0.f, 0.f}, c0_s = {-s_hc[hh][1], 0.f, 0.f, 0.f};
  const float lsg = lscale * p.gamma;
  const uint32_t ones = __builtin_amdgcn_readfirstlane(0x11111111);   // operand of the sign dword

  // ---- running state (lane (hh, n)).  The running max moves only when a tile's max
  // exceeds it by more than kLazy (log2 units): weights then stay below 2^kLazy and the
  // accumulators are rescaled rarely.
  constexpr float kLazy = 8.0f;
  float m_run = -INFINITY, l_part = 0.f, u3 = 0.f, u3s = 0.f;
  unsigned long long n_skip = 0;
  // value sums of head hh at coordinate 16 c + n.  accs[c]: sign products, one fp32 sum per
  // digit row, kept on the matrix cores.  Codebook planes: with LA, acv[k][c] = products of
  // plane k, likewise per digit row, in accumulation registers; otherwise arun[c] = sum_k
  // alpha_k (product of plane k, its 4 digit rows added), folded after each tile.
  f32x4 acv[4][8], accs[8];
  float arun[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if constexpr (LA) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < FV::planes(FV::bits(c >> 1))) acv[k][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
    } else {
      arun[c] = 0.f;
    }
    accs[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  uint32_t* xw = &s_x[wave][0];
  const int g0 = n >> 3, sx = (n >> 2) & 1;
  const float fv = dd == 0 ? 4.0f : dd == 1 ? 2.0f : dd == 2 ? 1.0f : 2.0f;  // |value A weights|
  const float fvi = 1.0f / fv;
  int* ve = &s_ve[wave][0][0][0];

  // nr: the resources of the next tile, whose loads are spread over this tile's key groups
  // and softmax, so that the load queue never holds the wave up for long
  auto process = [&](const TileRegs& T, const int64_t t0, const TileRes& nr) {
    // tokens of the tile before the end of the split (key_token(k, n) < rem is valid)
    const int rem = (int)min(t_end - t0, (int64_t)kXTile);
    // -- keys: logits of head hh for tokens key_token(k, n)
    float lg[8];
    static_for<0, 8>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      dma_keys(nr, kc);
      const uint32_t p0 = T.kw[k][0], p1 = T.kw[k][1];
      uint32_t p2, sg;
      if constexpr (KLO == KHI) {
        p2 = KLO >= 3 ? T.kw[k][2] : 0u;
        sg = T.kw[k][KLO];
      } else {
        const bool w3 = FK::bits(g) >= 3;
        p2 = w3 ? T.kw[k][2] : 0u;
        sg = w3 ? T.kw[k][3] : T.kw[k][2];
      }
      // digits 0-3 and 4-7 of every plane into one accumulator per term (the 8 key groups
      // give the scheduler independent chains)
      f32x4 ac = c0_c, as = c0_s;
      const i32x4 b0 = fp4_of(p0, ones);
      ac = mma(akh[0], b0, ac, ksh[0]);
      ac = mma(akl[0], b0, ac, ksl[0]);
      const i32x4 b1 = fp4_of(p1, ones);
      if constexpr (NPK >= 2) {
        ac = mma(akh[1], b1, ac, ksh[1]);
        ac = mma(akl[1], b1, ac, ksl[1]);
      }
      if constexpr (NPK >= 3) {
        const i32x4 b2 = fp4_of(p2, ones), b3 = fp4_xor3(b0, b1, b2);
        ac = mma(akh[2], b2, ac, ksh[2]);
        ac = mma(akl[2], b2, ac, ksl[2]);
        ac = mma(akh[3], b3, ac, ksh[3]);
        ac = mma(akl[3], b3, ac, ksl[3]);
      }
      {
        const i32x4 bs = fp4_of(sg, ones);
        as = mma(akh[NPK], bs, as, ksh[NPK]);
        as = mma(akl[NPK], bs, as, ksl[NPK]);
      }
      const float dc = ((ac[0] + ac[1]) + (ac[2] + ac[3])) * lscale;
      const float ds = ((as[0] + as[1]) + (as[2] + as[3])) * lsg;
      const float n16 = f16_bits_to_f32(T.kn[k]), r16 = f16_bits_to_f32(T.kn[k] >> 16);
      float v = fmaf(n16, dc, r16 * ds);
      // computed in every lane before the mask: the products must not move under a branch
      // on the token index (their B operands come from other lanes)
      asm volatile("" : "+v"(v));
      lg[k] = key_token(k, n) < rem ? v : -INFINITY;
    });
    if (p.logits) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (key_token(k, n) < rem)
          p.logits[((int64_t)b * p.hq + h0 + hh) * p.capacity + t0 + key_token(k, n)] = lg[k] * 0.6931471805599453f;
      }
    }
    dma_values(nr);
    // -- online softmax (head hh spans the 16 lanes of its DPP row)
    float tm = fmaxf(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])), fmaxf(fmaxf(lg[4], lg[5]), fmaxf(lg[6], lg[7])));
    tm = fmaxf(tm, xchg<1>(tm));
    tm = fmaxf(tm, xchg<2>(tm));
    tm = fmaxf(tm, quad_swap(tm));
    tm = fmaxf(tm, xchg<8>(tm));
    const bool grow = tm > m_run + kLazy;   // also the first finite max
    if (__ballot(grow) != 0) {
      const float m_new = grow ? tm : m_run;
      // the sums only need rescaling where a finite max moved (they are zero before it)
      const bool resc = grow && m_run != -INFINITY;
      if (__ballot(resc) != 0) {
        const float fm = resc ? exp2f(m_run - m_new) : 1.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if constexpr (LA) {
            // (the barriers keep the reads of the accumulation registers inside this rarely
            // taken branch)
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (k < FV::planes(FV::bits(c >> 1))) {
                asm volatile("" : "+a"(acv[k][c]));
                acv[k][c] *= fm;
                asm volatile("" : "+a"(acv[k][c]));
              }
            asm volatile("" : "+a"(accs[c]));
            accs[c] *= fm;
            asm volatile("" : "+a"(accs[c]));
          } else {
            arun[c] *= fm;
            accs[c] *= fm;
          }
        }
        l_part *= fm;
        u3 *= fm;
        u3s *= fm;
      }
      m_run = m_new;
    }
    float w[8];
    float tsum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // m_run is finite here (the tile holds a valid token), so a masked token gives 0; the
      // hardware exp2 (results below 2^-126, i.e. weights below 2^-126 of the largest one,
      // flush to zero) instead of the library's denormal-preserving expansion
      w[k] = __builtin_amdgcn_exp2f(lg[k] - m_run);
      tsum += w[k];
    }
    l_part += tsum;
    if (p.tau > 0.0f) {  // Sparse V: drop weights below tau times the running sum (an upper bound)
      float lrun = l_part;
      lrun += xchg<1>(lrun);
      lrun += xchg<2>(lrun);
      lrun += quad_swap(lrun);
      lrun += xchg<8>(lrun);
      const float thr = p.tau * lrun;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool drop = w[k] < thr;
        const unsigned long long bm = __ballot(drop && key_token(k, n) < rem);
        const unsigned long long all4 = bm & (bm >> 16) & (bm >> 32) & (bm >> 48) & 0xFFFFull;
        n_skip += __builtin_popcountll(all4);
        if (drop) w[k] = 0.0f;
      }
      // a tile whose every weight was dropped adds nothing to the value sums
      bool kept = false;
#pragma unroll
      for (int k = 0; k < 8; ++k) kept |= w[k] > 0.0f;
      if (__ballot(kept) == 0) return;
    }
    // -- value weights u = w n16_v and u' = w r16_v (gamma applied after the sums), times the
    // nibble weight f_D, as 16-bit integers x 2^(e - 16) with a block exponent e per head and
    // 32-token group; K index of token 16 sx + 4 i + dd of a group: 8 dd + 4 sx + i
    {
      float u[8], us[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // computed first and then selected, so that no branch is taken per token; records of
        // masked tokens may hold any norm, infinite ones included, so the products of a zero
        // weight can be NaN: the selection is made on the bits (this file is compiled on the
        // assumption that float values are not NaN, which must not remove it)
        const float n16 = f16_bits_to_f32(T.vn[k]), r16 = f16_bits_to_f32(T.vn[k] >> 16);
        const float wf = w[k] * fv;
        const bool keep = w[k] > 0.0f;
        u[k] = __uint_as_float(keep ? __float_as_uint(wf * n16) : 0u);
        us[k] = __uint_as_float(keep ? __float_as_uint(wf * r16) : 0u);
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
        mu = fmaxf(mu, quad_swap(mu));
        ms = fmaxf(ms, quad_swap(ms));
        const int eu = block_exp(mu), es = block_exp(ms);
        // x 2^(16 - e) is at most 2^16: rounded half up and kept below 2^16 (zero blocks: 0)
        const float scu = eu == kZeroExp ? 0.0f : ldexpf(1.0f, 16 - eu);
        const float scs = es == kZeroExp ? 0.0f : ldexpf(1.0f, 16 - es);
        u32x4 ru, rs;
        uint32_t su = 0u, ss = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ru[i] = min((uint32_t)fmaf(u[4 * x + i], scu, 0.5f), 65535u);
          rs[i] = min((uint32_t)fmaf(us[4 * x + i], scs, 0.5f), 65535u);
          su += ru[i];
          ss += rs[i];
        }
        // the constant removed after the products: sum over positions D < 3 of the rounded
        // weights divided by f_D (exact: integers below 2^18 times powers of two)
        if (dd != 3) {
          u3 += ldexpf((float)su, eu - 16) * fvi;
          u3s += ldexpf((float)ss, es - 16) * fvi;
        }
        // two weights per dword (K order): K = 8 dd + 4 sx + i is half i & 1 of dword
        // 4 dd + 2 sx + i / 2 of the row
        const int kk = (2 * x + g0) * kXRow + 4 * dd + 2 * sx;
        *reinterpret_cast<u32x2*>(&xw[(0 * 4 + hh) * 4 * kXRow + kk]) = (u32x2){ru[0] | (ru[1] << 16), ru[2] | (ru[3] << 16)};
        *reinterpret_cast<u32x2*>(&xw[(1 * 4 + hh) * 4 * kXRow + kk]) = (u32x2){rs[0] | (rs[1] << 16), rs[2] | (rs[3] << 16)};
        if ((n & 7) == 0) {
          ve[(0 * 4 + 2 * x + g0) * 4 + hh] = eu;
          ve[(1 * 4 + 2 * x + g0) * 4 + hh] = es;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_sched_barrier(0);
    // A lane (g, m): row m = (head m / 4, digit m % 4) of the 32 tokens of group g
    i32x8 au, as_;
    int vsu, vss;
    {
      const int ga = lane >> 4, ha = (lane & 15) >> 2, sh = 12 - 4 * (lane & 3);
#pragma unroll
      for (int type = 0; type < 2; ++type) {
        const uint32_t* src = &xw[((type * 4 + ha) * 4 + ga) * kXRow];
        u32x16 hd;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          // K = 8 D + i: the last 8 positions (dwords 12 .. 15) are D = 3, whose A weight is
          // -2 (the B nibble gives -0.5 s there): the f16 sign bit set
          const u32x4 r = *reinterpret_cast<const u32x4*>(src + 4 * c4);
          const uint32_t sgn = c4 == 3 ? 0x80008000u : 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) hd[4 * c4 + i] = ((r[i] >> sh) & 0x000F000Fu) | sgn;
        }
        const i32x8 op = fp6_row_f16(hd);
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
    // -- values: one product per plane and 16-coordinate block over the 128 tokens
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int bits = FV::bits(c >> 1);
      const uint32_t p0 = T.vw[c][0], p1 = T.vw[c][1];
      const uint32_t p2 = bits >= 3 ? T.vw[c][2] : 0u;
      const uint32_t sg = T.vw[c][bits];
      const i32x4 b0 = fp4_of(p0, ones), b1 = fp4_of(p1, ones);
      if constexpr (LA) {   // each plane into its own accumulator
        mma_acc(acv[0][c], au, b0, vsu);
        if (bits >= 2) mma_acc(acv[1][c], au, b1, vsu);
        if (bits >= 3) {
          const i32x4 b2 = fp4_of(p2, ones);
          mma_acc(acv[2][c], au, b2, vsu);
          mma_acc(acv[3][c], au, fp4_xor3(b0, b1, b2), vsu);
        }
        mma_acc(accs[c], as_, fp4_of(sg, ones), vss);
      } else {              // the planes' products folded with their Walsh coefficients now
        const int wsel = (c >> 1) < VSB ? 0 : 1;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        auto rows = [](const f32x4& t) { return (t[0] + t[1]) + (t[2] + t[3]); };
        const f32x4 t0v = mma(au, b0, z, vsu);
        float a = fmaf(p.alpha_v[wsel][0], rows(t0v), arun[c]);
        if (bits >= 2) {
          const f32x4 t1 = mma(au, b1, z, vsu);
          a = fmaf(p.alpha_v[wsel][1], rows(t1), a);
        }
        if (bits >= 3) {
          const i32x4 b2 = fp4_of(p2, ones);
          const f32x4 t2 = mma(au, b2, z, vsu);
          const f32x4 t3 = mma(au, fp4_xor3(b0, b1, b2), z, vsu);
          a = fmaf(p.alpha_v[wsel][2], rows(t2), a);
          a = fmaf(p.alpha_v[wsel][3], rows(t3), a);
        }
        arun[c] = a;
        accs[c] = mma(as_, fp4_of(sg, ones), accs[c], vss);
      }
    }
  };

  // ---- main loop: take the tile out of LDS, put the next one in flight, compute
  for (int it = 0; tile_start(it) < t_end; ++it) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);      // this tile's loads (the only ones in flight)
    asm volatile("" ::: "memory");
    TileRegs T;
    read_tile(T);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);    // reads done before the image is overwritten
    asm volatile("" ::: "memory");
    const int64_t tn = tile_start(it + 1);
    process(T, tile_start(it), tile_res(tn, tn < t_end));
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the last tile's (empty) loads
  asm volatile("" ::: "memory");
  // the last accumulations complete before the sums are read
  if constexpr (LA) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // ---- wave partial: per head the running max, the sum of weights and the rotated-domain
  // sums A[j] = sum_k alpha_k (sum_t u_t s_k,t,j), Q[j] = sum_t u'_t sigma_t,j
  float lh = l_part, u3h = u3, u3sh = u3s;
  lh += xchg<1>(lh);
  u3h += xchg<1>(u3h);
  u3sh += xchg<1>(u3sh);
  lh += xchg<2>(lh);
  u3h += xchg<2>(u3h);
  u3sh += xchg<2>(u3sh);
  lh += quad_swap(lh);
  u3h += quad_swap(u3h);
  u3sh += quad_swap(u3sh);
  lh += xchg<8>(lh);
  u3h += xchg<8>(u3h);
  u3sh += xchg<8>(u3sh);
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
      float a = LA ? 0.f : arun[c];
      auto rows = [](const f32x4& t) { return (t[0] + t[1]) + (t[2] + t[3]); };
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < FV::planes(bits)) {
          asum += p.alpha_v[wsel][k];
          if constexpr (LA) a = fmaf(p.alpha_v[wsel][k], rows(acv[k][c]), a);
        }
      a -= asum * u3h;
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
        const float sc = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
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
        l_o = fmaf((mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M), s_m[w][hd][1], l_o);
      }
      part0[hd * hstride] = M;
      part0[hd * hstride + 1] = l_o;
    }
  }
  if (p.skipped && p.tau > 0.0f && lane == 0 && n_skip) atomicAdd(p.skipped, n_skip);
}

template <int KLO, int KHI, int KSB, int VLO, int VHI, int VSB>
int launch_mx(const MxParams& p, dim3 grid, bool long_scan, hipStream_t stream) {
  if (long_scan)
    hipLaunchKernelGGL((decode_mx_scan<KLO, KHI, KSB, VLO, VHI, VSB, true>), grid, dim3(kXThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_mx_scan<KLO, KHI, KSB, VLO, VHI, VSB, false>), grid, dim3(kXThreads), 0, stream, p);
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
  // per-plane accumulators pay off from about 8 tiles per wave (their set-up and final fold
  // cost about as much as 4 tiles' folds)
  const bool long_scan = plan.tokens_per_split >= 8 * (int64_t)kXTile * kXWaves;
  int kl, kh, ks, vl, vh, vs;
  mx_shape(fk, kl, kh, ks);
  mx_shape(fv, vl, vh, vs);
  int rc = TQ_ERR_SHAPE;
#define TQ_MX_LAUNCH(a, b_, c, d, e, f)                                  \
  if (kl == a && kh == b_ && ks == c && vl == d && vh == e && vs == f)   \
    rc = launch_mx<a, b_, c, d, e, f>(p, grid, long_scan, stream);        \
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
