// Decode attention over the packed cache (placeholder until the kernels land).
#include "tq_internal.h"

tq_decode_plan tq_plan_decode(int32_t batch, int32_t hq, int32_t hkv, int64_t capacity, int32_t d) {
  tq_decode_plan p{};
  p.n_split = 1;
  p.waves = 1;
  p.parts = 1;
  p.tokens_per_split = capacity;
  p.ws_qrot_off = 0;
  p.ws_part_off = 0;
  p.ws_bytes = 256;
  return p;
}

int tq_launch_decode(const tq_format*, const tq_tables*, const tq_format*, const tq_tables*,
                     const void*, int32_t, int32_t, int32_t, int32_t, const void*, const uint16_t*,
                     const void*, const uint16_t*, int64_t, const int32_t*, float, float, float*,
                     float*, int64_t*, void*, const tq_decode_plan&, hipStream_t) {
  return TQ_ERR_SHAPE;
}
