// Decode scan instances: asymmetric pairs with split formats (b4 / b2.5, b3.5 / b2.5, b3.5 / b3), every
// query-head chunk size, values with and without QJL.
#include "tq_decode_kernel.h"

namespace tqk {
template int launch_pair<3, 3, 4, 2, 1, 2>(const DecodeParams&, bool, int, dim3, hipStream_t);
template int launch_pair<3, 2, 2, 2, 1, 2>(const DecodeParams&, bool, int, dim3, hipStream_t);
template int launch_pair<3, 2, 2, 2, 2, 4>(const DecodeParams&, bool, int, dim3, hipStream_t);
}  // namespace tqk
