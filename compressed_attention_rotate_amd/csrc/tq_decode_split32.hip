// Decode scan instances: 3+2-bit split formats (3.25, 3.5 bit), every
// query-head chunk size, values with and without QJL.
#include "tq_decode_kernel.h"

namespace tqk {
template int launch_pair<3, 2, 1, 3, 2, 1>(const DecodeParams&, bool, int, dim3, hipStream_t);
template int launch_pair<3, 2, 2, 3, 2, 2>(const DecodeParams&, bool, int, dim3, hipStream_t);
}  // namespace tqk
