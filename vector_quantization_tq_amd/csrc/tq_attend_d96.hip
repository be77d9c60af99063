// Decode-attention chunk kernels for head dimension 96 (every key and value
// width; the kernel and its launch are in tq_attend_impl.h, the rest of the
// attention path in tq_attend.hip).
#include "tq_attend_impl.h"

namespace tq {
namespace attn {
template hipError_t launch_chunks_d<96, false>(const AttendSegment&, int64_t, int, int, float, float, const uint8_t*,
                                               const float*, float*, int64_t, int64_t, int64_t, int64_t, hipStream_t);
}  // namespace attn
}  // namespace tq
