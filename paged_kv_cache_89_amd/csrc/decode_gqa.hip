// Instantiations of the matrix-core GQA decode (fp16/bf16 Q; same-type or e4m3 cache;
// B = 16; G in {2, 4, 8}).
#include "decode_gqa_mfma.h"

namespace pa {
bool gqa_mfma_supported(const DecodeShape& s) {
  return (s.head_dim == 64 || s.head_dim == 128) && s.block_size == 16 &&
         (s.group == 2 || s.group == 4 || s.group == 8) &&
         (s.q_kind == KIND_F16 || s.q_kind == KIND_BF16) &&
         (s.kv_kind == s.q_kind || s.kv_kind == KIND_E4M3);
}

hipError_t launch_decode_gqa_mfma(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
  if (s.head_dim == 128)
    return s.nontemporal ? launch_gqa_mfma_d<128, true>(s, a, stream)
                         : launch_gqa_mfma_d<128, false>(s, a, stream);
  return s.nontemporal ? launch_gqa_mfma_d<64, true>(s, a, stream)
                       : launch_gqa_mfma_d<64, false>(s, a, stream);
}
}  // namespace pa
