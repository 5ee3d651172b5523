// Decode-kernel instantiations: head_dim 64, non-temporal K/V loads.
#include "decode_kernel.h"

namespace pa {
hipError_t launch_decode_64_nt(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
  return launch_decode_d<64, true>(s, a, stream);
}
}  // namespace pa
