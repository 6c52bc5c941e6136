// Decode scan instances: 2+1-bit split formats (2.25, 2.5, 2.75 bit), every
// query-head chunk size, values with and without QJL.
#include "tq_decode_kernel.h"

namespace tqk {
template int launch_pair<2, 1, 1, 2, 1, 1>(const DecodeParams&, bool, int, dim3, hipStream_t);
template int launch_pair<2, 1, 2, 2, 1, 2>(const DecodeParams&, bool, int, dim3, hipStream_t);
template int launch_pair<2, 1, 3, 2, 1, 3>(const DecodeParams&, bool, int, dim3, hipStream_t);
}  // namespace tqk
