// Matrix-core decode instantiations: head_dim 128, cacheable K/V loads.
#include "decode_gqa_mfma.h"

namespace pa {
hipError_t launch_gqa_mfma_128_t(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
  return launch_gqa_mfma_d<128, false>(s, a, stream);
}
}  // namespace pa
