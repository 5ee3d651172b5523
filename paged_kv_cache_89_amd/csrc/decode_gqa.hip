// Dispatch of the matrix-core GQA decode (fp16/bf16 Q; same-type or e4m3 cache; B = 16;
// G in {2, 4, 8, 16}, 16 only reached by shared-prefix units).  The instantiations live
// in decode_gqa_d{64,128}_{nt,t}.hip.
#include "launch.h"

namespace pa {
hipError_t launch_gqa_mfma_64_nt(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_gqa_mfma_64_t(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_gqa_mfma_128_nt(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_gqa_mfma_128_t(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream);

bool gqa_mfma_supported(const DecodeShape& s) {
  return (s.head_dim == 64 || s.head_dim == 128) && s.block_size == 16 &&
         (s.group == 2 || s.group == 4 || s.group == 8 || s.group == 16) &&
         (s.q_kind == KIND_F16 || s.q_kind == KIND_BF16) &&
         (s.kv_kind == s.q_kind || s.kv_kind == KIND_E4M3);
}

hipError_t launch_decode_gqa_mfma(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
  if (s.head_dim == 128)
    return s.nontemporal ? launch_gqa_mfma_128_nt(s, a, stream) : launch_gqa_mfma_128_t(s, a, stream);
  if (s.head_dim == 64)
    return s.nontemporal ? launch_gqa_mfma_64_nt(s, a, stream) : launch_gqa_mfma_64_t(s, a, stream);
  return hipErrorInvalidValue;
}
}  // namespace pa
