// Shared-prefix decode of e4m3 caches in one launch: the prefix units (matrix-core kernel
// body, per-column masks) take the first workgroups of the grid and the per-sequence
// units (vector kernel body) the rest.  Both bodies and their unit maps are those of the
// two separate launches (each reads its own DecodeArgs, whose wg_base / wg_count place
// its workgroups in the grid); only the kernel boundary between them goes, so the launch
// ramps up and drains once.  The long prefix units are dispatched first; with the plan's
// 1024-token prefix partitions they take about half of the wavefront slots and the short
// per-sequence units stream through the rest, then through the slots the prefix units
// free.
//
// e4m3 caches only: their prefix units need 32 KiB of LDS per workgroup and four waves
// per SIMD, which the vector body fits too; a 16-bit prefix workgroup needs 64 KiB, which
// would halve the vector body's occupancy.  One query head per KV head only (the
// per-sequence units then run the vector kernel).
#include "decode_gqa_mfma.h"
#include "decode_kernel.h"

namespace pa {

static_assert(PA_GQA_WAVES == PA_DECODE_WAVES, "both bodies run 64 * waves threads");

template <int D, int QK, int K, bool NT_OWN>
__global__ __launch_bounds__(64 * PA_GQA_WAVES, gqa_min_waves(KIND_E4M3, true, K)) void cascade_fp8_kernel(
    const DecodeArgs pre, const DecodeArgs own) {
  if ((int)blockIdx.x < own.wg_base)
    gqa_body<D, QK, KIND_E4M3, K, true, true, false>(pre);
  else
    decode_body<D, 16, QK, KIND_E4M3, 1, NT_OWN, false, false>(own);
}

template <int D, int QK, int K>
hipError_t launch_cascade_k(const DecodeArgs& pre, const DecodeArgs& own, bool nt_own, hipStream_t stream) {
  const dim3 grid(own.wg_base + own.wg_count), block(64 * PA_GQA_WAVES);
  if (nt_own)
    hipLaunchKernelGGL((cascade_fp8_kernel<D, QK, K, true>), grid, block, 0, stream, pre, own);
  else
    hipLaunchKernelGGL((cascade_fp8_kernel<D, QK, K, false>), grid, block, 0, stream, pre, own);
  return hipGetLastError();
}

template <int D, int QK>
hipError_t launch_cascade_q(int K, const DecodeArgs& pre, const DecodeArgs& own, bool nt_own,
                            hipStream_t stream) {
  switch (K) {
    case 2: return launch_cascade_k<D, QK, 2>(pre, own, nt_own, stream);
    case 4: return launch_cascade_k<D, QK, 4>(pre, own, nt_own, stream);
    case 8: return launch_cascade_k<D, QK, 8>(pre, own, nt_own, stream);
    case 16: return launch_cascade_k<D, QK, 16>(pre, own, nt_own, stream);
    default: return hipErrorInvalidValue;
  }
}

bool cascade_fp8_supported(const DecodeShape& pre_shape, int heads_per_kv) {
  return pre_shape.kv_kind == KIND_E4M3 && heads_per_kv == 1 && pre_shape.block_size == 16 &&
         (pre_shape.head_dim == 64 || pre_shape.head_dim == 128) &&
         (pre_shape.q_kind == KIND_F16 || pre_shape.q_kind == KIND_BF16) &&
         (pre_shape.group == 2 || pre_shape.group == 4 || pre_shape.group == 8 ||
          pre_shape.group == 16);
}

hipError_t launch_cascade_fp8(const DecodeShape& pre_shape, const DecodeArgs& pre,
                              const DecodeArgs& own, bool nt_own, hipStream_t stream) {
  const int K = pre_shape.group;
  if (pre_shape.head_dim == 128)
    return pre_shape.q_kind == KIND_BF16 ? launch_cascade_q<128, KIND_BF16>(K, pre, own, nt_own, stream)
                                         : launch_cascade_q<128, KIND_F16>(K, pre, own, nt_own, stream);
  if (pre_shape.head_dim == 64)
    return pre_shape.q_kind == KIND_BF16 ? launch_cascade_q<64, KIND_BF16>(K, pre, own, nt_own, stream)
                                         : launch_cascade_q<64, KIND_F16>(K, pre, own, nt_own, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
