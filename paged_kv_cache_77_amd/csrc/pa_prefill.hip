// Varlen chunked prefill (rows of requests with q_len > 1): not built yet.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
