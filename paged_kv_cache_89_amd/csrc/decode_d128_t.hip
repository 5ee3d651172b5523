// Decode-kernel instantiations: head_dim 128, cached K/V loads.
#include "decode_kernel.h"

namespace pa {
hipError_t launch_decode_128_t(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
  return launch_decode_d<128, false>(s, a, stream);
}
}  // namespace pa
