// Decode-kernel instantiations: head_dim 64, cached K/V loads.
#include "decode_kernel.h"

namespace pa {
hipError_t launch_decode_64_t(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
  return launch_decode_d<64, false>(s, a, stream);
}
}  // namespace pa
