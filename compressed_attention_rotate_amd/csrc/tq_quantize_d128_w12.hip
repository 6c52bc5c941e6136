// Quantize kernel instances: d 128 / 1 bits, d 128 / 2 bits (every input type, with and without
// counters and QJL sign words).
#include "tq_quantize_kernel.h"

namespace tqk {
template int launch_quantize<128, 1, 1>(const QParams&, int, bool, hipStream_t, int);
template int launch_quantize<128, 2, 2>(const QParams&, int, bool, hipStream_t, int);
}  // namespace tqk
