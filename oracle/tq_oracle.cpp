// CPU oracle of the TurboQuant hot path in plain C++, fp64: the same definitions as
// oracle/tq_oracle.py, written out again for timing on the host cores and cross-checked
// against it.
//
// TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the cpu_baseline leg
// of bench.py load this library.  It shares no code, table or constant with the HIP path.
// The codebooks, the +/-1 diagonal and the Gaussian S come in as arguments, made by the
// Python oracle.
//
// What is computed (the pages, as cited in oracle/tq_oracle.py):
//  * rotation y = H (D x) / sqrt(d), with H the natural-order Sylvester Hadamard matrix,
//    H_ij = (-1)^popcount(i & j), summed entry by entry (163.com explainer, section
//    "第一步：PolarQuant"; zhidx article, section "01 turboquant_plus：介绍与详解");
//  * n = ||x||, stored as fp16 (round to nearest even) n16; z = y / n; idx_j = the number
//    of boundaries t_m < z_j in the coordinate's table;
//  * residual r = y - n16 c[idx] in the rotated domain, r16 = fp16(||r||),
//    u = S (r / ||r||), sign bit 1 where u >= 0 (163.com explainer, section "第二步：QJL");
//  * block-32 packing: per block of 32 coordinates the code bit-planes, then one word of
//    sign bits, bit i of a word belonging to coordinate 32 block + i (zhidx article);
//  * dequantize x~ = D H (n16 c[idx] + gamma r16 S^T (2 sigma - 1)) / sqrt(d) with
//    gamma = sqrt(pi / 2) / d, and decode attention as textbook softmax attention over the
//    dequantized keys and values (163.com explainer, section "速度").
// Work is split over rows (vectors, or query heads) among std::thread workers; each row's
// arithmetic is the same whatever the thread count.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

struct Fmt {
  int d, bits_lo, bits_hi, split, qjl;
  int bits_of_block(int blk) const { return 32 * blk < split ? bits_lo : bits_hi; }
  int words() const {
    int w = 0;
    for (int b = 0; b < d / 32; ++b) w += bits_of_block(b) + (qjl ? 1 : 0);
    return w;
  }
};

struct Book {
  const double* centroids;   // 2^bits ascending
  const double* bounds;      // 2^bits - 1 ascending
  int bits;
};

// fp64 -> fp16 bit pattern, round to nearest, ties to even (IEEE 754 binary16)
uint16_t fp16_bits(double v) {
  uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  double a = std::fabs(v);
  if (std::isnan(v)) return 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00;   // rounds to infinity
  if (a < std::ldexp(1.0, -25)) {
    // below half the smallest subnormal (exactly half rounds to 0, the even neighbour)
    return sign;
  }
  int e;
  std::frexp(a, &e);                       // a = f 2^e, f in [0.5, 1)
  int exp16 = e - 1 + 15;                  // biased exponent of a normal fp16
  double q;                                // a in units of the last place
  uint32_t mant;
  if (exp16 <= 0) {                        // subnormal: units of 2^-24
    q = std::ldexp(a, 24);
    exp16 = 0;
  } else {
    q = std::ldexp(a, 10 - (e - 1));       // in [1024, 2048)
  }
  double fl = std::floor(q);
  double rem = q - fl;
  uint64_t m = (uint64_t)fl;
  if (rem > 0.5 || (rem == 0.5 && (m & 1))) ++m;
  if (exp16 == 0) {
    // m in [0, 1024]; 1024 is the smallest normal
    return sign | (uint16_t)m;
  }
  if (m == 2048) {                         // carried into the next binade
    m = 1024;
    ++exp16;
    if (exp16 >= 31) return sign | 0x7C00;
  }
  mant = (uint32_t)(m - 1024);
  return sign | (uint16_t)(exp16 << 10) | (uint16_t)mant;
}

double fp16_value(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = std::ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp(1024.0 + m, e - 25);
  return s ? -v : v;
}

double hadamard_entry(int i, int j) { return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1.0 : 1.0; }

void rotate(const double* x, const int8_t* signs, int d, double* y) {
  const double isd = 1.0 / std::sqrt((double)d);
  for (int i = 0; i < d; ++i) {
    double acc = 0.0;
    for (int j = 0; j < d; ++j) acc += hadamard_entry(i, j) * (signs[j] * x[j]);
    y[i] = acc * isd;
  }
}

void unrotate(const double* y, const int8_t* signs, int d, double* x) {
  const double isd = 1.0 / std::sqrt((double)d);
  for (int j = 0; j < d; ++j) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += y[i] * hadamard_entry(i, j);
    x[j] = acc * isd * signs[j];
  }
}

const Book& book_of(const Fmt& f, const Book& lo, const Book& hi, int j) {
  return j < f.split ? lo : hi;
}

// One vector: x [d_in] (zero-padded to d) -> record words, n16, r16.
void quantize_one(const Fmt& f, const Book& lo, const Book& hi, const int8_t* signs,
                  const double* S, const double* x, int d_in, uint32_t* rec, uint16_t* n16b,
                  uint16_t* r16b) {
  const int d = f.d;
  std::vector<double> xp(d, 0.0), y(d), r(d), u(d);
  std::vector<int> idx(d);
  for (int j = 0; j < d_in; ++j) xp[j] = x[j];
  rotate(xp.data(), signs, d, y.data());
  double ss = 0.0;
  for (int j = 0; j < d; ++j) ss += xp[j] * xp[j];
  const double nrm = std::sqrt(ss);
  const uint16_t nb = fp16_bits(nrm);
  const double n16 = fp16_value(nb);
  for (int j = 0; j < d; ++j) {
    const Book& bk = book_of(f, lo, hi, j);
    const double z = nrm > 0.0 ? y[j] / nrm : 0.0;
    int c = 0;
    for (int m = 0; m < (1 << bk.bits) - 1; ++m)
      if (bk.bounds[m] < z) ++c;
    idx[j] = c;
    r[j] = y[j] - n16 * bk.centroids[c];
  }
  double rs = 0.0;
  for (int j = 0; j < d; ++j) rs += r[j] * r[j];
  const double rn = std::sqrt(rs);
  const uint16_t rb = fp16_bits(rn);
  for (int i = 0; i < d; ++i) {
    double acc = 0.0;
    if (rn > 0.0)
      for (int j = 0; j < d; ++j) acc += S[(size_t)i * d + j] * (r[j] / rn);
    u[i] = acc;
  }
  int k = 0;
  for (int blk = 0; blk < d / 32; ++blk) {
    const int B = f.bits_of_block(blk);
    for (int p = 0; p < B; ++p) {
      uint32_t w = 0;
      for (int i = 0; i < 32; ++i) w |= (uint32_t)((idx[32 * blk + i] >> p) & 1) << i;
      rec[k++] = w;
    }
    if (f.qjl) {
      uint32_t w = 0;
      for (int i = 0; i < 32; ++i) w |= (uint32_t)(u[32 * blk + i] >= 0.0 ? 1 : 0) << i;
      rec[k++] = w;
    }
  }
  *n16b = nb;
  *r16b = rb;
}

// One record -> the dequantized vector in the original domain.
void dequantize_one(const Fmt& f, const Book& lo, const Book& hi, const int8_t* signs,
                    const double* S, const uint32_t* rec, uint16_t n16b, uint16_t r16b, double* x) {
  const int d = f.d;
  std::vector<int> idx(d, 0);
  std::vector<double> pm(d, -1.0), y(d);
  int k = 0;
  for (int blk = 0; blk < d / 32; ++blk) {
    const int B = f.bits_of_block(blk);
    for (int p = 0; p < B; ++p) {
      const uint32_t w = rec[k++];
      for (int i = 0; i < 32; ++i) idx[32 * blk + i] |= (int)((w >> i) & 1) << p;
    }
    if (f.qjl) {
      const uint32_t w = rec[k++];
      for (int i = 0; i < 32; ++i) pm[32 * blk + i] = ((w >> i) & 1) ? 1.0 : -1.0;
    }
  }
  const double n16 = fp16_value(n16b), r16 = fp16_value(r16b);
  const double gam = std::sqrt(M_PI / 2.0) / d;
  for (int j = 0; j < d; ++j) {
    const Book& bk = book_of(f, lo, hi, j);
    double v = n16 * bk.centroids[idx[j]];
    if (f.qjl) {
      double st = 0.0;   // (S^T pm)_j
      for (int i = 0; i < d; ++i) st += S[(size_t)i * d + j] * pm[i];
      v += gam * r16 * st;
    }
    y[j] = v;
  }
  unrotate(y.data(), signs, d, x);
}

template <class F>
void parallel_rows(int64_t n, int threads, F fn) {
  if (threads <= 0) threads = (int)std::thread::hardware_concurrency();
  if (threads < 1) threads = 1;
  if ((int64_t)threads > n) threads = (int)(n > 0 ? n : 1);
  if (threads == 1) {
    for (int64_t i = 0; i < n; ++i) fn(i);
    return;
  }
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t)
    pool.emplace_back([=]() {
      for (int64_t i = t; i < n; i += threads) fn(i);
    });
  for (auto& th : pool) th.join();
}

Fmt fmt_of(const int32_t* fmt5) { return Fmt{fmt5[0], fmt5[1], fmt5[2], fmt5[3], fmt5[4]}; }

}  // namespace

extern "C" {

// Threads the calls below use when passed 0.
int tqo_hardware_threads() { return (int)std::thread::hardware_concurrency(); }

// fp64 -> fp16 bit patterns (round to nearest even), for the rounding pins.
void tqo_fp16_bits(const double* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = fp16_bits(v[i]);
}

// Quantize n rows of x [n][d_in] (fp64).  fmt5 = {d, bits_lo, bits_hi, split, qjl};
// cents_lo / bounds_lo: the codebook of bits_lo bits (2^b and 2^b - 1 values), the same
// for hi; signs [d] (+1 / -1), S [d][d].  Outputs: records [n][words] uint32, n16 / r16 [n]
// fp16 bit patterns.  threads = 0: all hardware threads.
void tqo_quantize(const int32_t* fmt5, const double* cents_lo, const double* bounds_lo,
                  const double* cents_hi, const double* bounds_hi, const int8_t* signs,
                  const double* S, const double* x, int64_t n, int32_t d_in, uint32_t* records,
                  uint16_t* n16, uint16_t* r16, int32_t threads) {
  const Fmt f = fmt_of(fmt5);
  const Book lo{cents_lo, bounds_lo, f.bits_lo}, hi{cents_hi, bounds_hi, f.bits_hi};
  const int W = f.words();
  parallel_rows(n, threads, [&](int64_t i) {
    quantize_one(f, lo, hi, signs, S, x + i * d_in, d_in, records + i * W, n16 + i, r16 + i);
  });
}

// Dequantize n records into x [n][d] (fp64, original domain).
void tqo_dequantize(const int32_t* fmt5, const double* cents_lo, const double* cents_hi,
                    const int8_t* signs, const double* S, const uint32_t* records,
                    const uint16_t* n16, const uint16_t* r16, int64_t n, double* x,
                    int32_t threads) {
  const Fmt f = fmt_of(fmt5);
  const Book lo{cents_lo, nullptr, f.bits_lo}, hi{cents_hi, nullptr, f.bits_hi};
  const int W = f.words();
  parallel_rows(n, threads, [&](int64_t i) {
    dequantize_one(f, lo, hi, signs, S, records + i * W, n16[i], r16[i], x + i * f.d);
  });
}

// Decode one step: for each (batch b, query head h) softmax attention of q [batch][hq][d]
// over the first lens[b] dequantized keys / values of KV head h / (hq / hkv).  kt / vt:
// dequantized caches [batch][hkv][cap][d] (fp64, from tqo_dequantize).  out [batch][hq][d],
// logits [batch][hq][cap] (entries t >= lens[b] untouched).  With tau > 0 the value rows whose
// final softmax weight is below tau are left out of the sum (no renormalization: the Sparse-V
// gate of the zhidx article, section "01 turboquant_plus：介绍与详解"), and dropped[bh] (when
// not null) receives the number of rows left out for that (batch, query head).
void tqo_attend(const double* q, const double* kt, const double* vt, const int32_t* lens,
                int32_t batch, int32_t hq, int32_t hkv, int64_t cap, int32_t d, double scale,
                double tau, double* out, double* logits, int64_t* dropped, int32_t threads) {
  const int G = hq / hkv;
  parallel_rows((int64_t)batch * hq, threads, [&](int64_t bh) {
    const int64_t b = bh / hq, h = bh % hq, kh = h / G;
    const int64_t L = lens[b];
    const double* qv = q + bh * d;
    const double* K = kt + (b * hkv + kh) * cap * d;
    const double* V = vt + (b * hkv + kh) * cap * d;
    double* lg = logits + bh * cap;
    double m = -INFINITY;
    for (int64_t t = 0; t < L; ++t) {
      double acc = 0.0;
      for (int j = 0; j < d; ++j) acc += K[t * d + j] * qv[j];
      lg[t] = acc * scale;
      if (lg[t] > m) m = lg[t];
    }
    double* o = out + bh * d;
    for (int j = 0; j < d; ++j) o[j] = 0.0;
    int64_t n_drop = 0;
    if (L > 0) {
      double sum = 0.0;
      for (int64_t t = 0; t < L; ++t) sum += std::exp(lg[t] - m);
      for (int64_t t = 0; t < L; ++t) {
        const double p = std::exp(lg[t] - m) / sum;
        if (tau > 0.0 && p < tau) {
          ++n_drop;
          continue;
        }
        for (int j = 0; j < d; ++j) o[j] += p * V[t * d + j];
      }
    }
    if (dropped) dropped[bh] = n_drop;
  });
}

// Inner-product top-k (163.com explainer, section "向量搜索"): for each query i of
// q [nq][d], the k rows of x [n][d] with the largest <q_i, x_t>, in descending order of the
// score; equal scores are ranked by the lower row index.  ids [nq][k] (-1 and -inf past n),
// scores [nq][k].  With x the dequantized database this is the estimator's top-k; with the
// raw vectors it is the exact one.
void tqo_topk_ip(const double* q, const double* x, int64_t n, int64_t nq, int32_t d, int32_t k,
                 int64_t* ids, double* scores, int32_t threads) {
  parallel_rows(nq, threads, [&](int64_t i) {
    const double* qv = q + i * d;
    std::vector<double> sc(n);
    for (int64_t t = 0; t < n; ++t) {
      double acc = 0.0;
      for (int j = 0; j < d; ++j) acc += x[t * d + j] * qv[j];
      sc[t] = acc;
    }
    std::vector<int64_t> idx(n);
    for (int64_t t = 0; t < n; ++t) idx[t] = t;
    const int64_t kk = std::min<int64_t>(k, n);
    std::partial_sort(idx.begin(), idx.begin() + kk, idx.end(), [&](int64_t a, int64_t b) {
      return sc[a] > sc[b] || (sc[a] == sc[b] && a < b);
    });
    for (int r = 0; r < k; ++r) {
      ids[i * k + r] = r < kk ? idx[r] : -1;
      scores[i * k + r] = r < kk ? sc[idx[r]] : -INFINITY;
    }
  });
}

}  // extern "C"
