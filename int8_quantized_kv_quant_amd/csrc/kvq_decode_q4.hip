// kv_decode_attn_splitk for layouts with a 4-bit store (q4_0, k8v4).
#include "kvq_internal.h"

namespace kvq {

int launch_partial_q4(const kvq_layout&, const void*, const void*, const uint16_t*, const uint16_t*,
                      const uint16_t*, int32_t, int32_t, const int32_t*, int32_t, float, const kvq_plan_t&, void*,
                      void*) {
  return KVQ_ERR_UNSUPPORTED;
}

}  // namespace kvq
