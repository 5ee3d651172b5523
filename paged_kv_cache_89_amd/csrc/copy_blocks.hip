// Batched copy of physical blocks ("PagedAttention: Mathematical Foundations, ..." sec. 7,
// fusion 3 "Batched Block Copy-on-Write"; sec. 5, parallel sampling): every copy-on-write
// of one decoding step -- block src duplicated into block dst, all KV heads, K and V --
// runs in one launch instead of one small memcpy per block.
//
// The same kernel moves blocks between two pools (sec. 6, swapping: a preempted request's
// blocks go to host RAM and come back on resume); either pool may be pinned host memory
// mapped into the device's address space, the other the device pool.
//
// One work-item moves 16 bytes; a block of Hkv * B * d * e bytes is a contiguous run in
// both pools ([NB][Hkv][B][d] layout), so reads and writes are fully coalesced.  Pairs with
// an id outside its pool's [0, blocks) are skipped.
#include "device_common.h"
#include "launch.h"

namespace pa {

__global__ __launch_bounds__(256) void copy_blocks_kernel(const CopyArgs a) {
  const int64_t chunks = a.block_bytes / 16;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = gid / chunks;
  if (pair >= a.num_pairs) return;
  const int64_t ch = gid % chunks;
  const int src = a.pairs[2 * pair], dst = a.pairs[2 * pair + 1];
  if ((unsigned)src >= (unsigned)a.src_blocks || (unsigned)dst >= (unsigned)a.dst_blocks) return;
  const size_t so = (size_t)src * a.block_bytes + ch * 16, d_o = (size_t)dst * a.block_bytes + ch * 16;
  *(u32x4*)((char*)a.dst_k + d_o) = *(const u32x4*)((const char*)a.src_k + so);
  *(u32x4*)((char*)a.dst_v + d_o) = *(const u32x4*)((const char*)a.src_v + so);
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
  if (a.num_pairs == 0) return hipSuccess;
  const int64_t items = (int64_t)a.num_pairs * (a.block_bytes / 16);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pa
