// Decode attention over the packed cache (filled in below) and top-k search.
#include "tq_device.h"
#include "tq_kernels.h"

namespace tq {

int64_t attend_ws_bytes(const tq_quantizer*, const tq_quantizer*, int, int, int, int64_t, int) { return 256; }

hipError_t launch_attend(const tq_quantizer*, const tq_quantizer*, const void*, int, int, int, int, const uint32_t*,
                         const float*, const float*, const uint32_t*, const float*, int64_t, const uint16_t*,
                         const uint16_t*, int, float, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

int64_t topk_ws_bytes(const tq_quantizer*, int, int, int, int64_t, int) { return 256; }

hipError_t launch_topk(const tq_quantizer*, const void*, int, int, int, int, const uint32_t*, const float*, const float*,
                       int64_t, int, float*, int64_t*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace tq
