// Instances of the fused two-segment decode scan (decode over a decayed cache in one
// launch), one per combination in TQ_DECAY_PAIRS; compiled apart so the instances build in
// parallel with the other decode files.
#include "tq_decode_kernel.h"

namespace tqk {

template <int A0, int A1, int A2, int A3, int A4, int A5, int B0, int B1, int B2, int B3, int B4,
          int B5>
int launch_scan_pair(const DecodeParams& p0, const DecodeParams& p1, int n0, dim3 grid,
                     hipStream_t s) {
  hipLaunchKernelGGL((decode_scan_pair<A0, A1, A2, A3, A4, A5, B0, B1, B2, B3, B4, B5, 4>), grid,
                     dim3(kThreads), 0, s, p0, p1, n0);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

#define TQ_DECAY_INSTANCE(a0, a1, a2, a3, a4, a5, b0, b1, b2, b3, b4, b5)                      \
  template int launch_scan_pair<a0, a1, a2, a3, a4, a5, b0, b1, b2, b3, b4, b5>(               \
      const DecodeParams&, const DecodeParams&, int, dim3, hipStream_t);
TQ_DECAY_PAIRS(TQ_DECAY_INSTANCE)
#undef TQ_DECAY_INSTANCE

}  // namespace tqk
