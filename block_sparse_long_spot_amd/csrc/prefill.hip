// Prefill-tile variant: tile block scoring and causal block-sparse attention.
#include "device_common.h"
#include "spot_internal.h"

namespace spot {

hipError_t launch_prefill_select_score(const void*, const float*, const void*, float*, int, int,
                                       int, int, int, int, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_prefill_attn(const void*, const void*, const void*, const int32_t*,
                               const int32_t*, int, void*, int, int, int, int, int, int, int,
                               float, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace spot
