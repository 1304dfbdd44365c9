// Instantiations of the MFMA chunked-prefill kernel (head_dim 64 and 128).
#include "prefill_impl.h"

namespace pa {
PA_LAYOUT_PROBE(prefill)

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int block_size, int group,
                          hipStream_t s) {
  if (head_dim == 128)
    return dtype == DT_BF16 ? launch_prefill_dt<DT_BF16, 128>(a, block_size, group, s)
                            : launch_prefill_dt<DT_F16, 128>(a, block_size, group, s);
  if (head_dim == 64)
    return dtype == DT_BF16 ? launch_prefill_dt<DT_BF16, 64>(a, block_size, group, s)
                            : launch_prefill_dt<DT_F16, 64>(a, block_size, group, s);
  return hipErrorInvalidValue;
}
}  // namespace pa
