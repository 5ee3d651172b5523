// Matrix-core decode instantiations: head_dim 64, cacheable K/V loads.
#include "decode_gqa_mfma.h"

namespace pa {
hipError_t launch_gqa_mfma_64_t(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
  return launch_gqa_mfma_d<64, false>(s, a, stream);
}
}  // namespace pa
