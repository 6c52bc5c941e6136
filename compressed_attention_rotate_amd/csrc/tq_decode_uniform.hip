// Decode scan instances: one-width formats (b4, b3, b2 and asymmetric pairs of them), every
// query-head chunk size, values with and without QJL.
#include "tq_decode_kernel.h"

namespace tqk {
template int launch_pair<3, 3, 4, 3, 3, 4>(const DecodeParams&, bool, int, dim3, hipStream_t);
template int launch_pair<3, 3, 4, 2, 2, 4>(const DecodeParams&, bool, int, dim3, hipStream_t);
template int launch_pair<2, 2, 4, 2, 2, 4>(const DecodeParams&, bool, int, dim3, hipStream_t);
template int launch_pair<1, 1, 4, 1, 1, 4>(const DecodeParams&, bool, int, dim3, hipStream_t);
template int launch_pair<2, 2, 4, 1, 1, 4>(const DecodeParams&, bool, int, dim3, hipStream_t);
}  // namespace tqk
