// Seeded draws of the random rotation: the +-1 diagonal D applied before the Walsh-Hadamard
// transform and the d x d Gaussian JL matrix S of the residual sketch (163.com explainer,
// m.163.com/dy/article/KOV7P8JI0556C3J2, sections "第一步：PolarQuant" (random rotation) and
// "第二步：QJL" (JL transform); zhidx turboquant_plus article, intro: a sign flip then the
// Walsh-Hadamard transform).  The pages fix no generator; this one is counter-based so a
// (d, seed) pair names the same tables on every machine:
//   x_k  = SplitMix64 output k of the state started at `seed` (Steele, Lea and Flood, 2014);
//   u(x) = (x >> 11) * 2^-53, uniform on [0, 1);
//   D_i  = +1 if the top bit of draw i is 0, else -1, for i = 0 .. d-1;
//   then for each pair of S entries in row-major order, two draws x_a, x_b give
//   u1 = 1 - u(x_a) in (0, 1], u2 = u(x_b) and, by Box and Muller (1958), in fp64,
//   r = sqrt(-2 ln u1), a = (2 pi) u2, S_2k = fp32(r cos a), S_2k+1 = fp32(r sin a),
//   each rounded to nearest even.
#include <stdint.h>

#include <cmath>

#include "tq.h"

namespace {
struct SplitMix64 {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

double unit(uint64_t x) { return (double)(x >> 11) * 0x1.0p-53; }
}  // namespace

extern "C" int tq_make_rotation(int32_t d, uint64_t seed, int8_t* signs, float* S) {
  if (d < 8 || d > 4096 || (d & (d - 1))) return TQ_ERR_SHAPE;
  if (!signs || !S) return TQ_ERR_ARG;
  SplitMix64 g{seed};
  for (int i = 0; i < d; ++i) signs[i] = (g.next() >> 63) ? -1 : 1;
  const int64_t n = (int64_t)d * d;
  const double two_pi = 2.0 * M_PI;
  for (int64_t k = 0; k < n; k += 2) {
    const double u1 = 1.0 - unit(g.next());
    const double u2 = unit(g.next());
    const double r = std::sqrt(-2.0 * std::log(u1));
    const double a = two_pi * u2;
    S[k] = (float)(r * std::cos(a));
    S[k + 1] = (float)(r * std::sin(a));
  }
  return TQ_OK;
}
