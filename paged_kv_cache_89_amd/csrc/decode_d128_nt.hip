// Decode-kernel instantiations: head_dim 128, non-temporal K/V loads.
#include "decode_kernel.h"

namespace pa {
hipError_t launch_decode_128_nt(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
  return launch_decode_d<128, true>(s, a, stream);
}
}  // namespace pa
