// bf16 instantiations of the paged-attention decode kernels.
#include "decode_mfma_impl.h"

namespace pa {
PA_LAYOUT_PROBE(decode_bf16)

hipError_t launch_decode_bf16(const DecodeArgs& a, int head_dim, int block_size, int group,
                              int phases, hipStream_t s) {
  return launch_decode_dt<DT_BF16>(a, head_dim, block_size, group, phases, s);
}
}  // namespace pa
