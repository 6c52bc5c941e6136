// Device helpers shared by the quantize, decode and search kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tqk {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// ---------------------------------------------------------------------------------------
// Lane exchange x -> value of lane (lane ^ M), for M < 32 (never crosses a 32-lane half).
// xor 1 / 2: DPP quad_perm; xor 8: DPP row_ror:8 (within a 16-lane row i+8 == i^8);
// xor 4 / 16: ds_swizzle in bitmask mode (and 0x1f, xor M).
// ---------------------------------------------------------------------------------------
template <int M>
__device__ __forceinline__ float xchg(float v) {
  int x = __float_as_int(v);
  if constexpr (M == 1) {
    x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);
  } else if constexpr (M == 2) {
    x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);
  } else if constexpr (M == 8) {
    x = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);
  } else if constexpr (M == 4) {
    x = __builtin_amdgcn_ds_swizzle(x, (4 << 10) | 0x1F);
  } else {
    static_assert(M == 16, "xchg: M must be 1, 2, 4, 8 or 16");
    x = __builtin_amdgcn_ds_swizzle(x, (16 << 10) | 0x1F);
  }
  return __int_as_float(x);
}

// Hadamard butterfly across lanes for lane bit M: lower lane gets a + b, upper lane a - b
// (a = value of the lower lane, b = value of the upper lane).
template <int M>
__device__ __forceinline__ float butterfly(float mine, float sgn) {
  float t = xchg<M>(mine);
  return fmaf(sgn, mine, t);
}

// Sum over the 32 lanes of each half-wave (result in every lane of the half).
__device__ __forceinline__ float half_sum(float v) {
  v += xchg<1>(v);
  v += xchg<2>(v);
  v += xchg<4>(v);
  v += xchg<8>(v);
  v += xchg<16>(v);
  return v;
}

__device__ __forceinline__ double shfl_xor_d(double v, int m) { return __shfl_xor(v, m, 64); }

template <int M>
__device__ __forceinline__ double xchg_d(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __float_as_uint(xchg<M>(__uint_as_float((uint32_t)u)));
  const uint32_t hi = __float_as_uint(xchg<M>(__uint_as_float((uint32_t)(u >> 32))));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sum over the 32 lanes of each half-wave in fp64 (DPP / ds_swizzle exchanges).
__device__ __forceinline__ double half_sum_d(double v) {
  v += xchg_d<1>(v);
  v += xchg_d<2>(v);
  v += xchg_d<4>(v);
  v += xchg_d<8>(v);
  v += xchg_d<16>(v);
  return v;
}

// Reductions over all 64 lanes: DPP / swizzle within each half, then the two halves
// combined through readlane (result is wave-uniform).
__device__ __forceinline__ float wave_sum_fast(float v) {
  v = half_sum(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
}

__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, xchg<1>(v));
  v = fmaxf(v, xchg<2>(v));
  v = fmaxf(v, xchg<4>(v));
  v = fmaxf(v, xchg<8>(v));
  v = fmaxf(v, xchg<16>(v));
  return v;
}

__device__ __forceinline__ float wave_max_fast(float v) {
  v = half_max(v);
  return fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
               __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)));
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += shfl_xor_d(v, m);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// fp32 -> fp16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}

// Deposit a ballot: lane `slot` of the lower half receives the low 32 bits of `mask`,
// lane 32 + slot the high 32 bits (one vector per half-wave).
__device__ __forceinline__ uint32_t deposit(uint32_t old, uint64_t mask, int slot) {
  const int lane = lane_id();
  const uint32_t v = (lane & 32) ? (uint32_t)(mask >> 32) : (uint32_t)mask;
  return ((lane & 31) == slot) ? v : old;
}

// fp64 -> fp16 bits with one correct rounding (nearest, ties to even).  Round to odd
// into fp32 first (24 >= 11 + 2 significant bits), then round to nearest into fp16;
// this double rounding is exact.  Only used for non-negative finite inputs.
__device__ __forceinline__ uint32_t f64_to_f16_bits(double v) {
  float f = (float)v;
  double back = (double)f;
  if (back != v) {
    uint32_t b = __float_as_uint(f);
    if (back > v) b -= 1;  // v >= 0: step the magnitude down to the truncated value
    b |= 1u;
    f = __uint_as_float(b);
  }
  return f32_to_f16_bits(f);
}

// A wave-uniform 32-bit value (a kernel-argument word read with a constant index) kept
// in an SGPR and opaque to the optimizer.  Selecting among such values per lane avoids a
// per-lane indexed read of kernel-argument memory, which would become a vector load from
// the argument segment instead of scalar loads.
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}

__device__ __forceinline__ float load_elem(const void* base, int64_t i, int dtype) {
  if (dtype == 0 || dtype == 3) return reinterpret_cast<const float*>(base)[i];  // 3: fp32 rows, pre-rotated
  uint32_t h = reinterpret_cast<const uint16_t*>(base)[i];
  if (dtype == 1) return __uint_as_float(h << 16);  // bf16
  return f16_bits_to_f32(h);                       // fp16
}

// ---------------------------------------------------------------------------------------
// Subset-sum table reads (decode key scan over per-vector records): entry idx of a table with one
// float per head (GC heads side by side).
typedef float tq_f32x4 __attribute__((ext_vector_type(4)));
typedef float tq_f32x2 __attribute__((ext_vector_type(2)));

template <int GC>
__device__ __forceinline__ void table_read(const float* T, int idx, float (&out)[GC]) {
  if constexpr (GC == 4) {
    const tq_f32x4 v = *reinterpret_cast<const tq_f32x4*>(T + 4 * idx);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  } else if constexpr (GC == 2) {
    const tq_f32x2 v = *reinterpret_cast<const tq_f32x2*>(T + 2 * idx);
    out[0] = v[0]; out[1] = v[1];
  } else {
    out[0] = T[idx];
  }
}

// acc += alpha * (byte-table reads of one 32-bit plane word, byte groups g0 .. g0+3); the
// four reads are summed pairwise first so every read is consumed right away.
template <int GC>
__device__ __forceinline__ void lut_byte(const float* Tq, int g0, uint32_t w, float alpha,
                                         float (&acc)[GC]) {
  float t0[GC], t1[GC], t2[GC], t3[GC];
  table_read<GC>(Tq, (g0 + 0) * 256 + (w & 0xFFu), t0);
  table_read<GC>(Tq, (g0 + 1) * 256 + ((w >> 8) & 0xFFu), t1);
  table_read<GC>(Tq, (g0 + 2) * 256 + ((w >> 16) & 0xFFu), t2);
  table_read<GC>(Tq, (g0 + 3) * 256 + (w >> 24), t3);
#pragma unroll
  for (int h = 0; h < GC; ++h) acc[h] = fmaf(alpha, (t0[h] + t1[h]) + (t2[h] + t3[h]), acc[h]);
}

// acc += nibble-table reads of one 32-bit sign word (nibble groups g0 .. g0+7), summed as
// a tree.
template <int GC>
__device__ __forceinline__ void lut_nib(const float* Ts, int g0, uint32_t w, float (&acc)[GC]) {
  float t[8][GC];
#pragma unroll
  for (int i = 0; i < 8; ++i) table_read<GC>(Ts, (g0 + i) * 16 + ((w >> (4 * i)) & 0xFu), t[i]);
#pragma unroll
  for (int h = 0; h < GC; ++h)
    acc[h] += ((t[0][h] + t[1][h]) + (t[2][h] + t[3][h])) + ((t[4][h] + t[5][h]) + (t[6][h] + t[7][h]));
}

}  // namespace tqk
