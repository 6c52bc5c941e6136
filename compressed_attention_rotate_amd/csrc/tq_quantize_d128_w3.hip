// Quantize kernel instances: d 128 / 3 bits (every input type, with and without
// counters and QJL sign words).
#include "tq_quantize_kernel.h"

namespace tqk {
template int launch_quantize<128, 3, 3>(const QParams&, int, bool, hipStream_t, int);
}  // namespace tqk
