// Host entry of the quantize path: packs the kernel parameters and dispatches on the
// format.  The kernel itself is in tq_quantize_kernel.h; its instances are compiled in the
// tq_quantize_*.hip translation units.
#include "tq_quantize_kernel.h"

namespace tqk {
extern template int launch_quantize<128, 1, 1>(const QParams&, int, bool, hipStream_t, int);
extern template int launch_quantize<128, 2, 2>(const QParams&, int, bool, hipStream_t, int);
extern template int launch_quantize<128, 3, 3>(const QParams&, int, bool, hipStream_t, int);
extern template int launch_quantize<128, 3, 2>(const QParams&, int, bool, hipStream_t, int);
extern template int launch_quantize<128, 2, 1>(const QParams&, int, bool, hipStream_t, int);
extern template int launch_quantize<256, 2, 2>(const QParams&, int, bool, hipStream_t, int);
extern template int launch_quantize<256, 3, 3>(const QParams&, int, bool, hipStream_t, int);
}  // namespace tqk

// ---------------------------------------------------------------------------------------
int tq_launch_quantize(const tq_format* f, const tq_tables* t, const void* x, int32_t x_dtype,
                       int64_t n, int32_t d_in, int64_t ld_x, void* codes, uint16_t* norms,
                       int64_t* counters, hipStream_t stream, const tq_paged_dst* paged) {
  using namespace tqk;
  QParams p{};
  if (paged) {
    p.slots = paged->slots;
    p.num_pages = paged->num_pages;
    p.page_heads = paged->page_heads;
    p.page_log2 = paged->page_log2;
    p.block_table = paged->block_table;
    p.pos0 = paged->pos0;
    p.max_blocks = paged->max_blocks;
  }
  p.x = x;
  p.S = t->S;
  p.codes = reinterpret_cast<uint32_t*>(codes);
  p.norms = reinterpret_cast<uint32_t*>(norms);
  p.counters = reinterpret_cast<unsigned long long*>(counters);
  p.n = n;
  p.ld_x = ld_x;
  p.d_in = d_in;
  p.esize = x_dtype == TQ_F32 ? 4 : 2;
  const int64_t row_bytes = (int64_t)d_in * p.esize;
  p.staged = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && ((ld_x * p.esize) % 16 == 0) &&
             (row_bytes % 16 == 0);
  p.cpr = p.staged ? (int32_t)(row_bytes / 16) : 1;
  fill_format_params(f, t, p);
  const int ncu = tq_num_cus();
  if (ncu <= 0) return TQ_ERR_HIP;
  const int lo = f->bits_lo, hi = f->bits_hi, xt = x_dtype;
  const bool q = f->qjl != 0;
  if (f->d == 128) {
    if (lo == 1 && hi == 1) return launch_quantize<128, 1, 1>(p, xt, q, stream, ncu);
    if (lo == 2 && hi == 2) return launch_quantize<128, 2, 2>(p, xt, q, stream, ncu);
    if (lo == 3 && hi == 3) return launch_quantize<128, 3, 3>(p, xt, q, stream, ncu);
    if (lo == 3 && hi == 2) return launch_quantize<128, 3, 2>(p, xt, q, stream, ncu);
    if (lo == 2 && hi == 1) return launch_quantize<128, 2, 1>(p, xt, q, stream, ncu);
  } else if (f->d == 256) {
    if (lo == 2 && hi == 2) return launch_quantize<256, 2, 2>(p, xt, q, stream, ncu);
    if (lo == 3 && hi == 3) return launch_quantize<256, 3, 3>(p, xt, q, stream, ncu);
  }
  return TQ_ERR_SHAPE;
}
