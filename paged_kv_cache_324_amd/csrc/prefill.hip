// Chunked prefill over the paged cache (MFMA kernel lands here).
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
hipError_t launch_prefill(const PrefillArgs&, int, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace pa
