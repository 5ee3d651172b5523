// Grouped-query paged decode on gfx950 matrix cores (one wavefront per work unit).
//
// The operation is the decode of "PagedAttention: Mathematical Foundations, ..." (sec. 3
// eqs. for S_ij / A_ij / o_i, sec. 7 pseudocode) for G query heads that share one KV head:
// per block j the G x B logits are a small dense contraction Q_g . K_j^T, and the output
// update is another, P . V_j.  Both run on MFMA with fp32 accumulation:
//
//   logits   C[16 tokens x 16 heads] = K_j[16 x D] . Q^T[D x 16]   (D/32 x v_mfma 16x16x32)
//            rows are the block's tokens, columns the query heads (G real, the rest zero)
//   output   acc[16 heads x 16 dims] += P[16 heads x 16 tokens] . V_j[16 x 16 dims]
//            (D/16 x v_mfma 16x16x16, one per 16-wide slice of the head dimension)
//
// Operand placement (lane l, r = l / 16, c = l % 16):
//   * K and V are read from HBM in fully coalesced 1 KiB wave loads and written row-major
//     into this wavefront's two LDS tiles (bank-swizzled 16-byte chunks).  K's A operand
//     (token c, dims 32kk + 8r .. +8) comes back with one ds_read_b128 per k-step.
//     Reading K straight into that operand layout from HBM would touch 16 rows x 64 bytes
//     per load instruction; measured, the coalesced route is 13 % faster;
//   * Q^T is loaded once: lane l holds head c's dims 32kk + 8r .. +8 (zero for c >= G);
//   * the logit result leaves in lane l the scores of head c for tokens 4r .. 4r+3, which
//     is exactly the A-operand layout of the P . V contraction, so softmax weights never
//     move between lanes;
//   * V is read back from its LDS tile with ds_read_b64_tr_b16, which hands each lane the
//     four tokens of one head-dimension column that the P . V B-operand needs.
// Softmax statistics use a lazily moved reference maximum: weights are 2^(z - m_ref) and
// m_ref (and with it acc and the denominator) is only moved when a block's maximum exceeds
// it by more than 8 (log2 units), so weights stay <= 256 and the usual per-block rescale
// of the accumulator is skipped in the common case.  The result is the same function.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int QK> struct MfmaOps;

template <> struct MfmaOps<KIND_BF16> {
  __device__ static f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static f32x4 pv(u32x2 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), b, c, 0, 0, 0);
  }
  // two fp32 weights -> packed bf16 pair (round to nearest even) and their rounded values
  __device__ static uint32_t pack2(float x, float y, float* rx, float* ry) {
    // gfx950 converts fp32 -> bf16 in hardware (round to nearest even)
    const uint32_t a = __builtin_bit_cast(uint16_t, (__bf16)x);
    const uint32_t b = __builtin_bit_cast(uint16_t, (__bf16)y);
    *rx = __uint_as_float(a << 16);
    *ry = __uint_as_float(b << 16);
    return a | (b << 16);
  }
};

template <> struct MfmaOps<KIND_F16> {
  __device__ static f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static f32x4 pv(u32x2 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack2(float x, float y, float* rx, float* ry) {
    const _Float16 a = (_Float16)x, b = (_Float16)y;
    *rx = (float)a;
    *ry = (float)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
};

constexpr float kLazyRescaleLog2 = 8.0f;  // weights stay <= 2^8 between reference moves

// Supported: D in {64, 128}, B = 16 (one MFMA token tile per block), fp16 or bf16 Q/K/V,
// 2 <= G <= 16.
template <int D, int QK, int G, bool NT>
__global__ __launch_bounds__(256) void paged_decode_gqa_mfma_kernel(const DecodeArgs a) {
  constexpr int BS = 16;
  constexpr int KSTEPS = D / 32;             // 16x16x32 steps over the head dimension
  constexpr int NTILES = D / 16;             // 16-wide output slices
  constexpr int LPT = D / 8;                 // lanes per token row in a 16-byte-per-lane load
  constexpr int TPL = 64 / LPT;              // token rows per 1 KiB wave load
  constexpr int NLDV = BS / TPL;             // wave loads per V tile
  constexpr int PITCH = D * 2;               // LDS row pitch (bytes)
  constexpr int RPB = 256 / PITCH;           // rows per 256-byte bank period
  constexpr int TILE = BS * D * 2;           // bytes of one (block, KV head) tile
  static_assert(G >= 2 && G <= 16, "group size");
  using Ops = MfmaOps<QK>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_tiles[4][TILE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_ktiles[4][TILE];

  // 16-byte chunk x of LDS row `row` holds chunk x ^ swz(row) of the V row: the two
  // chunks every ds_read_b64_tr_b16 takes from each of 16 rows then fall on distinct
  // banks (2 passes for 512 bytes), and each ds_write_b128 covers whole bank periods.
  auto swz = [](int row) { return 2 * ((row / RPB) % (D / 16)); };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int wg = blockIdx.x;
  if (a.xcd_remap) {
    const int G8 = gridDim.x, x = wg % 8, loc = wg / 8, per = G8 / 8, rem = G8 % 8;
    wg = (x < rem) ? x * (per + 1) + loc : rem * (per + 1) + (x - rem) * per + loc;
  }
  const int unit = wg * 4 + wave;
  if (unit >= a.num_units) return;
  int s, kvh, part;
  if (a.seq_fastest == 0) {
    kvh = unit % a.num_kv_heads;
    const int rest = unit / a.num_kv_heads;
    part = rest % a.num_parts;
    s = rest / a.num_parts;
  } else {
    s = unit % a.num_seqs;
    const int rest = unit / a.num_seqs;
    kvh = rest % a.num_kv_heads;
    part = rest / a.num_kv_heads;
  }
  const int h0 = kvh * G;
  int n = a.ctx[s];
  n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
  const int nblk = (n + BS - 1) / BS;
  const int j0 = part * a.blocks_per_part;
  const int j1 = min(nblk, j0 + a.blocks_per_part);
  const int r = lane >> 4;
  const int c = lane & 15;

  if (j0 >= j1) {
    if (a.num_parts == 1) {  // n == 0: zero rows
      uint16_t* o = (uint16_t*)a.out + ((size_t)s * a.num_heads + h0) * D;
      for (int e = lane; e < G * D; e += 64) o[e] = 0;
    }
    return;
  }

  // Q^T operand: lane (r, c) holds head c's dims 32kk + 8r .. +8 (zero for padding heads)
  u32x4 qop[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    if (c < G)
      qop[kk] = *(const u32x4*)((const uint16_t*)a.q + ((size_t)s * a.num_heads + h0 + c) * D +
                                32 * kk + 8 * r);
    else
      qop[kk] = u32x4{0, 0, 0, 0};
  }

  // Output accumulators (matrix-core C operands) hold P . V relative to the reference
  // maximum; they are rescaled only when the reference moves.
  f32x4 cacc[NTILES];
#pragma unroll
  for (int t = 0; t < NTILES; ++t) cacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference maximum of head c (log2 units), same in its 4 lanes
  float l_part = 0.f;       // this lane's share of head c's denominator

  const size_t blk_stride = (size_t)a.num_kv_heads * TILE;
  const char* kbase = (const char*)a.k + (size_t)kvh * TILE;
  const char* vbase = (const char*)a.v + (size_t)kvh * TILE;
  const uint32_t voff = (uint32_t)lane * 16;  // natural 1 KiB wave loads (K and V)
  uint8_t* vt = lds_tiles[wave];
  uint8_t* kt = lds_ktiles[wave];
  const float qk_scale = a.qk_scale;
  // LDS byte offsets: where this lane's V chunk of wave load i goes, and where its
  // ds_read_b64_tr_b16 of output slice t reads (row 4r + c/4, dims 16t + 4(c%4) .. +4)
  uint32_t vw_off[NLDV];
#pragma unroll
  for (int i = 0; i < NLDV; ++i) {
    const int row = i * TPL + lane / LPT;
    vw_off[i] = row * PITCH + (((lane % LPT) ^ swz(row)) * 16);
  }
  const int trow = 4 * r + c / 4;

  auto load_k = [&](int phys, u32x4 (&kr)[NLDV]) {
    const char* kp = kbase + (size_t)phys * blk_stride;
#pragma unroll
    for (int i = 0; i < NLDV; ++i) {
      if constexpr (NT) kr[i] = __builtin_nontemporal_load((const u32x4*)(kp + voff + 1024 * i));
      else kr[i] = *(const u32x4*)(kp + voff + 1024 * i);
    }
  };
  // K rows into their LDS tile: 16-byte chunk x of row t sits at chunk x ^ (t mod LPT), so
  // the A-operand reads (row c, chunk 4kk + r) of 16 lanes hit 16 different bank groups
  uint32_t kw_off[NLDV];
#pragma unroll
  for (int i = 0; i < NLDV; ++i) {
    const int row = i * TPL + lane / LPT;
    kw_off[i] = row * PITCH + (((lane % LPT) ^ (row % LPT)) * 16);
  }
  auto stage_k = [&](const u32x4 (&kr)[NLDV]) {
#pragma unroll
    for (int i = 0; i < NLDV; ++i) *(u32x4*)(kt + kw_off[i]) = kr[i];
  };
  auto load_v = [&](int phys, u32x4 (&vr)[NLDV]) {
    const char* vp = vbase + (size_t)phys * blk_stride;
#pragma unroll
    for (int i = 0; i < NLDV; ++i) {
      if constexpr (NT) vr[i] = __builtin_nontemporal_load((const u32x4*)(vp + voff + 1024 * i));
      else vr[i] = *(const u32x4*)(vp + voff + 1024 * i);
    }
  };
  // V rows into LDS; slots at or beyond n become zeros (their bytes may be NaN and the
  // matrix core would turn 0 * NaN into NaN)
  auto stage_v = [&](bool mask, int j, const u32x4 (&vr)[NLDV]) {
#pragma unroll
    for (int i = 0; i < NLDV; ++i) {
      u32x4 v = vr[i];
      if (mask && j * BS + i * TPL + lane / LPT >= n) v = u32x4{0, 0, 0, 0};
      *(u32x4*)(vt + vw_off[i]) = v;
    }
  };

  // logits of block j: C[token 4r+i][head c]
  auto logits = [&]() {
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const int chunk = (4 * kk + r) ^ (c % LPT);
      const u32x4 kop = *(const u32x4*)(kt + c * PITCH + chunk * 16);
      sc = Ops::qk(kop, qop[kk], sc);
    }
    return sc;
  };

  // online-softmax weights and P . V for block j (MASK: the block holds slots >= n)
  auto finish = [&](int j, f32x4 sc) {
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = (c < G) && (j * BS + 4 * r + i < n);
      z[i] = ok ? sc[i] * qk_scale : -INFINITY;
    }
    float bm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const bool move = bm > m_ref + kLazyRescaleLog2;  // false for padding heads (bm = -inf)
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float mn = move ? bm : m_ref;
      const float f = move ? ((m_ref == -INFINITY) ? 0.f : fast_exp2(m_ref - mn)) : 1.f;
      l_part *= f;
      m_ref = mn;
      // accumulator row 4r + i belongs to head 4r + i, whose factor sits in lane 4r + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float fi = __shfl(f, 4 * r + i);
#pragma unroll
        for (int t = 0; t < NTILES; ++t) cacc[t][i] *= fi;
      }
    }
    const float ms = (m_ref == -INFINITY) ? 0.f : m_ref;
    float rp[4];
    const uint32_t p01 = Ops::pack2(fast_exp2(z[0] - ms), fast_exp2(z[1] - ms), &rp[0], &rp[1]);
    const uint32_t p23 = Ops::pack2(fast_exp2(z[2] - ms), fast_exp2(z[3] - ms), &rp[2], &rp[3]);
    l_part += (rp[0] + rp[1]) + (rp[2] + rp[3]);
    const u32x2 pop = u32x2{p01, p23};
    // P . V over the 16 tokens, one 16-wide slice of the head dimension at a time
#pragma unroll
    for (int t = 0; t < NTILES; ++t) {
      const uint32_t chunk = (2 * t + (c % 4) / 2) ^ swz(trow);
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(vt + trow * PITCH + chunk * 16 + 8 * (c % 2)));
      cacc[t] = Ops::pv(pop, vb, cacc[t]);
    }
  };

  // Pipeline: the K and V loads of block j+1 are issued before block j is consumed (two
  // register sets each, as in the vector kernel); consuming block j moves V(j) into the
  // LDS tile, runs the logit contraction on K(j), the softmax update and P . V.  The mask
  // of slots >= n is applied branch-free (it only bites in a unit's last block).
  auto process = [&](int j, const u32x4 (&kr)[NLDV], const u32x4 (&vr)[NLDV]) {
    stage_k(kr);
    stage_v(true, j, vr);
    finish(j, logits());
  };
  TableSlice ts;
  ts.init(a.tables + (size_t)s * a.max_blocks, j0, j1, a.num_blocks, lane);
  u32x4 ka[NLDV], va[NLDV], kb[NLDV], vb[NLDV];
  {
    const int p0 = ts.get(j0);
    load_k(p0, ka);
    load_v(p0, va);
  }
  auto fetch = [&](int jj, u32x4 (&kr)[NLDV], u32x4 (&vr)[NLDV]) {
    const int p = ts.get(jj);
    load_k(p, kr);
    load_v(p, vr);
  };
  // steady state: every load in the loop is unconditional (see the vector kernel)
  int j = j0;
  while (j + 2 < j1) {
    fetch(j + 1, kb, vb);
    process(j, ka, va);
    fetch(j + 2, ka, va);
    process(j + 1, kb, vb);
    j += 2;
  }
  if (j + 1 < j1) {
    fetch(j + 1, kb, vb);
    process(j, ka, va);
    process(j + 1, kb, vb);
  } else {
    process(j, ka, va);
  }

  // head c's denominator: sum of its four lanes' shares
  float L = l_part + __shfl_xor(l_part, 16);
  L += __shfl_xor(L, 32);
  // accumulator row 4r + i (lane c holds dim 16t + c of slice t) belongs to head 4r + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * r + i;
    const float Li = __shfl(L, hh);
    const float Mi = __shfl(m_ref, hh);
    if (hh < G) {
      const int h = h0 + hh;
      if (a.num_parts == 1) {
        uint16_t* o = (uint16_t*)a.out + ((size_t)s * a.num_heads + h) * D + c;
#pragma unroll
        for (int t = 0; t < NTILES; ++t)
          o[16 * t] = f32_to_store<QK>(cacc[t][i] / Li);
      } else {
        const size_t pi = ((size_t)s * a.num_heads + h) * a.num_parts + part;
        float* pa_ = a.part_acc + pi * D + c;
#pragma unroll
        for (int t = 0; t < NTILES; ++t) pa_[16 * t] = cacc[t][i];
        if (c == 0) {
          a.part_ml[pi * 2] = Mi;
          a.part_ml[pi * 2 + 1] = Li;
        }
      }
    }
  }
}

template <int D, int QK, int G, bool NT>
hipError_t launch_gqa_mfma_t(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((a.num_units + 3) / 4);
  hipLaunchKernelGGL((paged_decode_gqa_mfma_kernel<D, QK, G, NT>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool NT>
hipError_t launch_gqa_mfma_d(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
#define PA_GQ(QK)                                                     \
  switch (s.group) {                                                  \
    case 2: return launch_gqa_mfma_t<D, QK, 2, NT>(a, stream);        \
    case 4: return launch_gqa_mfma_t<D, QK, 4, NT>(a, stream);        \
    case 8: return launch_gqa_mfma_t<D, QK, 8, NT>(a, stream);        \
    default: return hipErrorInvalidValue;                             \
  }
  if (s.q_kind == KIND_BF16 && s.kv_kind == KIND_BF16) { PA_GQ(KIND_BF16) }
  if (s.q_kind == KIND_F16 && s.kv_kind == KIND_F16) { PA_GQ(KIND_F16) }
  return hipErrorInvalidValue;
#undef PA_GQ
}

}  // namespace pa
