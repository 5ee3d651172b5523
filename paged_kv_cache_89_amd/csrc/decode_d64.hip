// Decode-kernel instantiations for head_dim 64.
#include "decode_kernel.h"

namespace pa {
hipError_t launch_decode_64(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
  return launch_decode_d<64>(s, a, stream);
}
}  // namespace pa
