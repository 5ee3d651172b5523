// Decode-kernel instantiations for head_dim 128.
#include "decode_kernel.h"

namespace pa {
hipError_t launch_decode_128(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
  return launch_decode_d<128>(s, a, stream);
}
}  // namespace pa
