// Quantize kernel instances: d 128 / 3+2 bits, d 128 / 2+1 bits (every input type, with and without
// counters and QJL sign words).
#include "tq_quantize_kernel.h"

namespace tqk {
template int launch_quantize<128, 3, 2>(const QParams&, int, bool, hipStream_t, int);
template int launch_quantize<128, 2, 1>(const QParams&, int, bool, hipStream_t, int);
}  // namespace tqk
