// Compressed inner-product search (placeholder until the kernels land).
#include "tq_internal.h"

tq_search_plan tq_plan_search(int64_t n_q, int32_t k, int64_t n_db, int32_t d) {
  tq_search_plan p{};
  p.n_chunks = 1;
  p.chunk_len = n_db;
  p.ws_bytes = 256;
  return p;
}

int tq_launch_search(const tq_format*, const tq_tables*, const void*, const uint16_t*, int64_t,
                     const float*, int32_t, int64_t, int32_t, int64_t*, float*, void*,
                     const tq_search_plan&, hipStream_t) {
  return TQ_ERR_SHAPE;
}
