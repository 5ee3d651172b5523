// KV write into the paged cache ("PagedAttention: Mathematical Foundations, ..." sec. 7,
// "Fused Reshape and Block Write"; sec. 4, "Decoding Step"): the new key and value rows
// of token t go straight to slot pos % B of physical block block_tables[seq][pos / B].
//
// One work-item moves 16 source bytes (8 fp16/bf16 elements) of one (token, KV head)
// row, so a row of D elements is D/8 consecutive lanes and both the source read and the
// cache write are contiguous 16-byte (or, for e4m3, 8-byte) accesses.  An e4m3 cache
// stores e4m3(float(x) * inv_scale) (binary32 product, round to nearest even,
// saturating), the per-tensor-scale fp8 storage of the 10100.com article's sec. 4.
#include "device_common.h"
#include "launch.h"

namespace pa {

template <int D, int BS, int SK, int CK>
__global__ __launch_bounds__(256) void write_kv_kernel(const WriteArgs a) {
  constexpr int CH = D / 8;  // 16-byte source chunks per row
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long rowi = gid / CH;
  const int ch = (int)(gid % CH);
  if (rowi >= (long)a.num_tokens * a.num_kv_heads) return;
  const int t = (int)(rowi / a.num_kv_heads);
  const int h = (int)(rowi % a.num_kv_heads);
  // The source rows go out with the token's sequence and position, ahead of the checks
  // (row t < num_tokens is in bounds whatever they find), and the empty asm takes all four
  // as operands, so they share one round trip (the compiler would otherwise load them one
  // after another, the rows last); the table lookup is the only other one before the store.
  const size_t src = ((size_t)t * a.num_kv_heads + h) * D + ch * 8;
  u32x4 kx = *(const u32x4*)((const uint16_t*)a.k_src + src);
  u32x4 vx = *(const u32x4*)((const uint16_t*)a.v_src + src);
  int seq = a.seq_ids[t];
  int pos = a.positions[t];
  asm volatile("" : "+v"(kx), "+v"(vx), "+v"(seq), "+v"(pos));
  if (seq < 0 || seq >= a.num_seqs || pos < 0 || pos / BS >= a.max_blocks) return;
  const int blk = a.tables[(size_t)seq * a.max_blocks + pos / BS];
  if (blk < 0 || blk >= a.num_blocks) return;
  const size_t dst = (((size_t)blk * a.num_kv_heads + h) * BS + pos % BS) * D + ch * 8;
  if constexpr (CK == SK) {
    *(u32x4*)((uint16_t*)a.k_cache + dst) = kx;
    *(u32x4*)((uint16_t*)a.v_cache + dst) = vx;
  } else {
    static_assert(CK == KIND_E4M3, "fp16/bf16 sources go to a same-type or e4m3 cache");
    const u32x2 ko = src8_to_e4m3<SK>(kx, a.k_inv_scale);
    const u32x2 vo = src8_to_e4m3<SK>(vx, a.v_inv_scale);
    *(u32x2*)((uint8_t*)a.k_cache + dst) = ko;
    *(u32x2*)((uint8_t*)a.v_cache + dst) = vo;
  }
}

bool write_supported(int head_dim, int block_size, int src_kind, int cache_kind) {
  if (head_dim != 64 && head_dim != 128) return false;
  if (block_size != 8 && block_size != 16 && block_size != 32) return false;
  if (src_kind != KIND_F16 && src_kind != KIND_BF16) return false;
  return cache_kind == src_kind || cache_kind == KIND_E4M3;
}

template <int D, int BS, int SK, int CK>
static hipError_t launch_w(const WriteArgs& a, hipStream_t stream) {
  const long items = (long)a.num_tokens * a.num_kv_heads * (D / 8);
  const dim3 grid((unsigned)((items + 255) / 256));
  hipLaunchKernelGGL((write_kv_kernel<D, BS, SK, CK>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, int BS>
static hipError_t launch_w_bs(int sk, int ck, const WriteArgs& a, hipStream_t stream) {
  if (sk == KIND_F16 && ck == KIND_F16) return launch_w<D, BS, KIND_F16, KIND_F16>(a, stream);
  if (sk == KIND_BF16 && ck == KIND_BF16) return launch_w<D, BS, KIND_BF16, KIND_BF16>(a, stream);
  if (sk == KIND_F16 && ck == KIND_E4M3) return launch_w<D, BS, KIND_F16, KIND_E4M3>(a, stream);
  if (sk == KIND_BF16 && ck == KIND_E4M3) return launch_w<D, BS, KIND_BF16, KIND_E4M3>(a, stream);
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_w_d(int bs, int sk, int ck, const WriteArgs& a, hipStream_t stream) {
  switch (bs) {
    case 8: return launch_w_bs<D, 8>(sk, ck, a, stream);
    case 16: return launch_w_bs<D, 16>(sk, ck, a, stream);
    case 32: return launch_w_bs<D, 32>(sk, ck, a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_write_kv(int head_dim, int block_size, int src_kind, int cache_kind,
                           const WriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  if (head_dim == 128) return launch_w_d<128>(block_size, src_kind, cache_kind, a, stream);
  if (head_dim == 64) return launch_w_d<64>(block_size, src_kind, cache_kind, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
