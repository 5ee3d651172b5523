// Log-sum-exp merge of decode partitions.
//
// A sequence longer than one partition is decoded as independent partitions of P tokens,
// each leaving (m_p, l_p, acc_p): its running maximum (log2 units), denominator and
// unnormalised output.  They combine with the same rescaling the online softmax uses
// between blocks ("PagedAttention: Mathematical Foundations, ..." sec. 7 pseudocode):
//   M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  o = sum_p acc_p 2^(m_p - M) / L.
// One wavefront per (sequence, query head); lane k owns D/64 consecutive output elements.
// Cascade partials (shared prefix + own suffix) fill every slot of a row, some of them
// empty (m = -inf, l = 0, acc not written): those are skipped.  Under the flat split a
// row's slots are the chunks its sequence's blocks fall into (see launch.h).
#include "device_common.h"
#include "launch.h"

namespace pa {

// Wave-wide max / sum (every lane gets the result), halves first, by VALU lane moves.
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = xor_combine<32>(v, op);
  v = xor_combine<16>(v, op);
  v = xor_combine<8>(v, op);
  v = xor_combine<4>(v, op);
  v = xor_combine<2>(v, op);
  return xor_combine<1>(v, op);
}
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, MaxOp{}); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, AddOp{}); }

// PF: partial outputs loaded per batch; the first batch goes out with the row's length and
// its (m, l) pairs, so a row of at most PF slots costs one round trip to memory.
template <int D, int QK, int PF>
__global__ __launch_bounds__(256) void merge_partitions_kernel(const MergeArgs a) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * 4 + wave;  // s * Hq + h
  if (row >= a.num_seqs * a.num_heads) return;
  const int s = row / a.num_heads;
  const int P = a.num_parts;
  uint16_t* o = (uint16_t*)a.out + (size_t)row * D + lane * EPL;
  const float2* ml = (const float2*)(a.part_ml + (size_t)row * P * 2);
  const float* pacc = a.part_acc + (size_t)row * P * D + lane * EPL;

  // Loads that do not depend on the length: slot `lane`'s (m, l) and the first PF slots'
  // outputs (indices clamped into the row's slots).  Slots at or past the row's own count
  // hold stale data; they are masked below and never enter the arithmetic.
  int n = a.ctx[s];
  const float2 ml0 = ml[min(lane, P - 1)];
  float x[PF][EPL];
#pragma unroll
  for (int k = 0; k < PF; ++k)
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[k][e] = pacc[(size_t)min(k, P - 1) * D + e];

  n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
  int np;
  if (a.flat) {
    // flat split: the row's slots are the chunks its sequence's blocks fall into
    const int B = a.block_size;
    int before = 0;  // blocks of the sequences before s
#pragma unroll
    for (int k = 0; k < kFlatK; ++k) {
      const int t = lane + 64 * k;
      int nt = t < s ? a.ctx[t] : 0;
      nt = nt < 0 ? 0 : (nt > a.max_ctx ? a.max_ctx : nt);
      before += (nt + B - 1) / B;
    }
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) before += __shfl_xor(before, k);
    const int C = a.flat_meta[0];
    const int nb = (n + B - 1) / B;
    np = nb > 0 ? (before + nb - 1) / C - before / C + 1 : 0;
  } else {
    np = a.all_slots ? (n > 0 ? P : 0) : (n + a.partition_size - 1) / a.partition_size;
  }

  // M = max over the row's slots (64 per pass; empty cascade slots carry m = -inf)
  float M = -INFINITY;
  for (int base = 0; base < np; base += 64) {
    const int p = base + lane;
    const float m = base == 0 ? ml0.x : (p < P ? ml[p].x : -INFINITY);
    M = fmaxf(M, wave_max(p < np ? m : -INFINITY));
  }
  if (M == -INFINITY) {  // n == 0: no token, zero row
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = 0;
    return;
  }
  float L = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int base = 0; base < np; base += 64) {
    const int p = base + lane;
    const float2 v = base == 0 ? ml0 : (p < P ? ml[p] : make_float2(-INFINITY, 0.f));
    const bool live = p < np && v.x != -INFINITY;
    const float w = live ? fast_exp2(v.x - M) : 0.f;  // this lane's slot weight
    L += wave_sum(live ? w * v.y : 0.f);
    const int cnt = min(64, np - base);
    int q = 0;
    if (base == 0) {
#pragma unroll
      for (int k = 0; k < PF; ++k) {
        if (k < cnt) {
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wk, wk != 0.f ? x[k][e] : 0.f, acc[e]);
        }
      }
      q = PF;
    }
    for (; q < cnt; q += PF) {  // further slots, PF loads in flight at a time; of cascade
                                // rows (many empty slots) only those that carry weight
      float y[PF][EPL];
#pragma unroll
      for (int k = 0; k < PF; ++k) {
        const bool want = !a.all_slots ||
                          (q + k < cnt && __builtin_amdgcn_readlane(__float_as_int(w), q + k) != 0);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          y[k][e] = want ? pacc[(size_t)min(base + q + k, P - 1) * D + e] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < PF; ++k) {
        if (q + k < cnt) {
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), q + k));
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wk, wk != 0.f ? y[k][e] : 0.f, acc[e]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = f32_to_store<QK>(acc[e] / L * a.v_scale);
}

template <int D, int QK>
hipError_t launch_merge_pf(const MergeArgs& a, dim3 grid, hipStream_t stream) {
  // The flat split sizes its slots for the shortest chunk, and cascade rows hold empty
  // slots: most rows fill a few of their slots, so the first batch stays small.
  if (a.num_parts <= 4 || a.flat || a.all_slots)
    hipLaunchKernelGGL((merge_partitions_kernel<D, QK, 4>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((merge_partitions_kernel<D, QK, 16>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(int head_dim, int q_kind, const MergeArgs& a, hipStream_t stream) {
  const dim3 grid((a.num_seqs * a.num_heads + 3) / 4);
  if (a.num_parts < 1) return hipErrorInvalidValue;
  if (head_dim == 128 && q_kind == KIND_F16) return launch_merge_pf<128, KIND_F16>(a, grid, stream);
  if (head_dim == 128 && q_kind == KIND_BF16) return launch_merge_pf<128, KIND_BF16>(a, grid, stream);
  if (head_dim == 64 && q_kind == KIND_F16) return launch_merge_pf<64, KIND_F16>(a, grid, stream);
  if (head_dim == 64 && q_kind == KIND_BF16) return launch_merge_pf<64, KIND_BF16>(a, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
