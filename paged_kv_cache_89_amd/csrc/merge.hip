// Log-sum-exp merge of decode partitions.
//
// A sequence longer than one partition is decoded as independent partitions of P tokens,
// each leaving (m_p, l_p, acc_p): its running maximum (log2 units), denominator and
// unnormalised output.  They combine with the same rescaling the online softmax uses
// between blocks ("PagedAttention: Mathematical Foundations, ..." sec. 7 pseudocode):
//   M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  o = sum_p acc_p 2^(m_p - M) / L.
// One wavefront per (sequence, query head); lane k owns D/64 consecutive output elements.
// Cascade partials (shared prefix + own suffix) fill every slot of a row, some of them
// empty (m = -inf, l = 0, acc not written): those are skipped.
#include "device_common.h"
#include "launch.h"

namespace pa {

template <int D, int QK>
__global__ __launch_bounds__(256) void merge_partitions_kernel(const MergeArgs a) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * 4 + wave;  // s * Hq + h
  if (row >= a.num_seqs * a.num_heads) return;
  const int s = row / a.num_heads;
  int n = a.ctx[s];
  n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
  const int np = a.all_slots ? (n > 0 ? a.num_parts : 0) : (n + a.partition_size - 1) / a.partition_size;
  uint16_t* o = (uint16_t*)a.out + (size_t)row * D + lane * EPL;
  const float* ml = a.part_ml + (size_t)row * a.num_parts * 2;
  const float* pacc = a.part_acc + (size_t)row * a.num_parts * D + lane * EPL;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ml[2 * p]);
  if (M == -INFINITY) {  // n == 0: no token, zero row
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0;
    return;
  }
  float L = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int p = 0; p < np; ++p) {
    const float mp = ml[2 * p];
    if (a.all_slots && mp == -INFINITY) continue;  // empty slot (wave-uniform)
    const float w = fast_exp2(mp - M);
    L = fmaf(w, ml[2 * p + 1], L);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w, pacc[(size_t)p * D + e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = f32_to_store<QK>(acc[e] / L * a.v_scale);
}

hipError_t launch_merge(int head_dim, int q_kind, const MergeArgs& a, hipStream_t stream) {
  const dim3 grid((a.num_seqs * a.num_heads + 3) / 4);
  if (head_dim == 128 && q_kind == KIND_F16)
    hipLaunchKernelGGL((merge_partitions_kernel<128, KIND_F16>), grid, dim3(256), 0, stream, a);
  else if (head_dim == 128 && q_kind == KIND_BF16)
    hipLaunchKernelGGL((merge_partitions_kernel<128, KIND_BF16>), grid, dim3(256), 0, stream, a);
  else if (head_dim == 64 && q_kind == KIND_F16)
    hipLaunchKernelGGL((merge_partitions_kernel<64, KIND_F16>), grid, dim3(256), 0, stream, a);
  else if (head_dim == 64 && q_kind == KIND_BF16)
    hipLaunchKernelGGL((merge_partitions_kernel<64, KIND_BF16>), grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
