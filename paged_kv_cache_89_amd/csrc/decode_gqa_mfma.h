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
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

// Minimum waves per SIMD the register allocation must allow (compile-time tuning knob).
#ifndef PA_GQA_MIN_WAVES
#define PA_GQA_MIN_WAVES 1
#endif
// Wavefronts (independent work units) per workgroup (compile-time tuning knob).
#ifndef PA_GQA_WAVES
#define PA_GQA_WAVES 4
#endif

// e4m3 caches: 1 = contract the codes on the fp8 matrix cores (no widening); 0 = widen
// them to the query's 16-bit type while staging (compile-time switch for measurements).
#ifndef PA_FP8_NATIVE
#define PA_FP8_NATIVE 1
#endif

// fp8 MFMA with per-operand power-of-two scales (E8M0 exponents, 127 = 2^0); operands are
// e4m3 (format code 0).  16 x 16 output, 128-long contraction, 32 codes per lane.
__device__ __forceinline__ f32x4 mfma_e4m3(v8i a, v8i b, f32x4 c, int a_exp, int b_exp) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, a_exp, 0, b_exp);
}

// Four floats -> four e4m3 codes (round to nearest even; |x| <= 448 here), and back.
__device__ __forceinline__ uint32_t e4m3x4_pack(float x0, float x1, float x2, float x3) {
  int d = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  d = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, d, true);
  return (uint32_t)d;
}

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

// e4m3 codes -> values of the query's 16-bit type (exact: every e4m3 value is
// representable in bf16 and in fp16); 16 codes in, 16 values (two 16-byte chunks) out.
template <int QK>
__device__ __forceinline__ void e4m3x16_widen(const u32x4 src, u32x4 (&dst)[2]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float f[4];
    e4m3x4_to_f32(src[w], f);
    uint32_t lo, hi;
    if constexpr (QK == KIND_BF16) {
      lo = __builtin_bit_cast(uint16_t, (__bf16)f[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f[1]) << 16);
      hi = __builtin_bit_cast(uint16_t, (__bf16)f[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f[3]) << 16);
    } else {
      lo = __builtin_bit_cast(uint16_t, (_Float16)f[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f[1]) << 16);
      hi = __builtin_bit_cast(uint16_t, (_Float16)f[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f[3]) << 16);
    }
    dst[(2 * w) / 4][(2 * w) % 4] = lo;
    dst[(2 * w + 1) / 4][(2 * w + 1) % 4] = hi;
  }
}

// e4m3 caches (PA_FP8_NATIVE): K and V stay 1-byte codes in LDS and both contractions run
// on the fp8 matrix core (v_mfma_scale_f32_16x16x128_f8f6f4).  e4m3 keeps 4 significant
// bits, so the 16-bit query enters as three e4m3 terms (q = hi + mid + lo, each the
// rounding residual of the one before; about 12 bits together) after scaling each head by
// a power of two 2^e that puts its largest element in [128, 256); the operand scale 2^-e
// of the matrix core undoes it exactly.  The softmax weights enter as hi + lo under a
// per-(head, block) power of two that lifts the block's largest weight into [128, 256)
// (the operand scale undoes it), so small weights do not fall below e4m3's range; the
// denominator sums the unrounded fp32 weights.  Lane layouts (measured on the device with
// an in-bounds probe): lane (r, c) supplies row / column c and 32 codes of the contraction
// for both operands alike; the scale of row / column c comes from a lane of column c,
// which is why the scales here are per head.  V's operand is built with
// ds_read_b64_tr_b8: 16 lanes each name 8 bytes of one of 8 rows, and lane c receives
// byte c of each row.
//
// Supported: D in {64, 128}, B = 16 (one MFMA token tile per block), fp16 or bf16 Q with a
// cache of the same type or e4m3 (contracted as e4m3, or widened to Q's type while it is
// staged into LDS), 2 <= G <= 16.
// LANE: per-column visibility (each query column has its own token range and draft
// mask), needed by the prefix units of the shared-prefix decode and by multi-token
// queries; plain and suffix units share one token count and use the cheaper mask.
// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one matrix-core column's four
// row groups), by the row swaps of xor_combine; every lane ends with the same value.
__device__ __forceinline__ float rows_max(float x) { return across_lanes<16>(x, MaxOp{}); }
__device__ __forceinline__ float rows_sum(float x) { return across_lanes<16>(x, AddOp{}); }

// e4m3 tiles on the fp8 matrix cores: 1 = K/V go from HBM straight into two LDS stages per
// wave (global_load_lds; no register staging, about 110 VGPRs, four waves per SIMD);
// 0 = through registers like the 16-bit tiles (compile-time switch for measurements).
#ifndef PA_FP8_LDS_DMA
#define PA_FP8_LDS_DMA 1
#endif
// fp16/bf16 tiles: 1 = the same two-stage LDS ring (64 KiB per workgroup: two workgroups
// per CU, two waves per SIMD, about 120 VGPRs); 0 = through registers, the block fetched two
// ahead (196 VGPRs, also two waves per SIMD).  Measured on the GQA workload (three pairs on
// one box): the ring 0.5 % faster per step, equal on four-token drafts.  A three-slot ring
// per wave (K and V tiles in turn, 48 KiB per workgroup, three waves per SIMD, 8 KiB in
// flight per wave) measured 0.5 % slower than the register path and was dropped.
#ifndef PA_LDS_DMA_16
#define PA_LDS_DMA_16 1
#endif

// One 16-byte-per-lane load from global memory into LDS: lane l's 16 bytes land at LDS
// byte lds + 16 l (the wave fills 1 KiB).  The LDS address travels in M0; the statement
// saves M0 first and restores it after, so whatever the compiler keeps there survives.
// (M0 is a reserved register: clang treats naming it as clobbered as undefined behaviour,
// and never assigns reserved registers to asm operands, so saving it is the sound form.)
// vmcnt drops once the bytes are in LDS (wait_vmcnt).  The stage being refilled was read by
// the block before: lgkmcnt(0) first, so those reads have returned before the new bytes can
// land.  (The compiler's global_load_lds builtin is not used: the compiler then waits for
// every outstanding load, the next block's included, before the first LDS read after it.)
template <bool NT>
__device__ __forceinline__ void load_lds_x4(const void* src, uint32_t lds) {
  uint32_t saved;
  if constexpr (NT)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\t"
                 "global_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(src), "s"(lds) : "memory");
  else
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\t"
                 "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(src), "s"(lds) : "memory");
}
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Waves per SIMD the register allocation must allow.  e4m3 blocks carry half the bytes of
// 16-bit ones, so each wave keeps half as much in flight and occupancy matters: with the
// LDS ring every e4m3 instantiation fits four waves per SIMD (the ring's 32 KiB per
// workgroup allows five); through registers, the per-column-mask e4m3 units (G <= 8) fit
// three without spilling.  The 16-bit instantiations are left to the compiler (they run at
// the same speed with two or three).
constexpr int gqa_min_waves(int kvk, bool lane, int g) {
  return kvk == KIND_E4M3 ? ((PA_FP8_NATIVE != 0 && PA_FP8_LDS_DMA != 0) ? 4
                             : (lane && g <= 8)                        ? 3
                                                                       : PA_GQA_MIN_WAVES)
                          : (PA_LDS_DMA_16 != 0 ? 2 : PA_GQA_MIN_WAVES);
}

// The kernel body, also run by the one-launch cascade (decode_cascade.hip).
template <int D, int QK, int KVK, int G, bool NT, bool LANE, bool FLAT>
__device__ __forceinline__ void gqa_body(const DecodeArgs& a) {
  constexpr int BS = 16;
  constexpr int KSTEPS = D / 32;             // 16x16x32 steps over the head dimension
  constexpr int NTILES = D / 16;             // 16-wide output slices
  constexpr int E = (KVK == KIND_E4M3) ? 1 : 2;  // cache bytes per element
  constexpr int EPLS = 16 / E;               // cache elements per lane per 16-byte load
  constexpr int LPTS = D / EPLS;             // lanes per token row of a 1 KiB wave load
  constexpr int TPLS = 64 / LPTS;            // token rows per 1 KiB wave load
  constexpr int STILE = BS * D * E;          // cache bytes of one (block, KV head) tile
  constexpr int NLDS = STILE / 1024;         // wave loads per cache tile
  constexpr bool NATIVE = PA_FP8_NATIVE && KVK == KIND_E4M3;  // e4m3 codes on the fp8 MFMA
  constexpr int LE = NATIVE ? 1 : 2;         // LDS bytes per element
  constexpr int CPL = NATIVE ? 1 : EPLS / 8; // 16-byte LDS chunks one lane's load becomes
  constexpr int CPR = D * LE / 16;           // 16-byte chunks per LDS row
  constexpr int PITCH = D * LE;              // LDS row pitch (bytes)
  constexpr int RPB = 256 / PITCH;           // rows per 256-byte bank period
  constexpr int TILE = BS * D * LE;          // LDS bytes of one tile
  constexpr int QD = D / 4;                  // native: query elements per lane
  static_assert(NLDS * 1024 == STILE, "tile must be covered by whole wave loads");
  static_assert(G >= 2 && G <= 16, "group size");
  using Ops = MfmaOps<QK>;
  // per wave: NST stages of (K tile, V tile)
  constexpr bool DMA = NATIVE ? PA_FP8_LDS_DMA != 0 : (KVK != KIND_E4M3 && PA_LDS_DMA_16 != 0);
  // LDS tiles of each wave: two-stage ring, slot 2 * stage + (0 = K, 1 = V); register
  // path, slot 0 = K, 1 = V
  constexpr int NSLOT = DMA ? 4 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds_buf[PA_GQA_WAVES][NSLOT][TILE];

  // 16-byte chunk x of LDS row `row` holds chunk x ^ swz(row) of the V row: the two
  // chunks every ds_read_b64_tr_b16 takes from each of 16 rows then fall on distinct
  // banks (2 passes for 512 bytes), and each ds_write_b128 covers whole bank periods.
  // Native e4m3 V tiles: chunk x of row t at x ^ (t mod CPR).
  auto swz = [](int row) {
    if constexpr (NATIVE) return row % CPR;
    else return 2 * ((row / RPB) % (D / 16));
  };
  // K tiles: chunk x of row t sits at x ^ kswz(t).  The logit operand reads (ds_read_b128)
  // of lanes c = 0..15 take one 16-byte chunk from each of rows 0..15.  e4m3 rows are 128
  // (64) bytes, so rows one 128-byte bank period apart start on the same bank: rotating by
  // the row's index within its 8-row (4-row) run, xor its run, puts every 8 consecutive lanes
  // on 8 different 16-byte bank groups of a 128-byte period and all 16 on different groups
  // of a 256-byte period (conflict-free whether a pass serves 8 or 16 lanes).  16-bit rows
  // are 256 bytes or more: t mod CPR.
  auto kswz = [](int row) {
    if constexpr (NATIVE) return ((row / (128 / PITCH)) ^ (row / 8)) % CPR;
    else return row % CPR;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool prefix = LANE && a.mode == MODE_PREFIX;
  const bool multi = LANE && a.mode == MODE_MULTI;
  const int rows = prefix ? a.num_groups : a.num_seqs;
  const int r = lane >> 4;
  const int c = lane & 15;
  // Query column cc < G of a unit of sequence (or group) s and KV head kvh reads and writes
  // row row_at(s, kvh, cc) of the [rows, D] query / output arrays.  Plain and suffix units:
  // the G heads of sequence s that share KV head kvh.  Prefix units: head cc % Gr of member
  // cc / Gr of group s; multi-token units: head cc % Gr of query token cc / Gr of sequence
  // s (Gr = query heads per KV head; G = Gr * members or Gr * query tokens).
  const int Gr = a.num_heads / a.num_kv_heads;
  const int outer_n = prefix ? a.seq_group : a.query_len;
  auto row_at = [&](int s_, int kvh_, int cc) -> size_t {
    if (LANE && (prefix || multi))
      return ((size_t)s_ * outer_n + cc / Gr) * a.num_heads + kvh_ * Gr + cc % Gr;
    return (size_t)s_ * a.num_heads + kvh_ * G + cc;
  };
  auto clamp_len = [&](int v) { return v < 0 ? 0 : (v > a.max_ctx ? a.max_ctx : v); };
  // Lane (r, c) loads head c's query elements (zeros for c >= G): dims QD*r .. +QD for the
  // e4m3 contraction, dims 32kk + 8r .. +8 otherwise.
  constexpr int QL = NATIVE ? QD / 8 : KSTEPS;  // 16-byte query loads per lane
  auto load_query = [&](int s_, int kvh_, u32x4 (&qr)[QL]) {
    if (c < G) {
      const uint16_t* qrow = (const uint16_t*)a.q + row_at(s_, kvh_, c) * D;
#pragma unroll
      for (int k = 0; k < QL; ++k)
        qr[k] = *(const u32x4*)(qrow + (NATIVE ? QD * r + 8 * k : 32 * k + 8 * r));
    } else {
#pragma unroll
      for (int k = 0; k < QL; ++k) qr[k] = u32x4{0, 0, 0, 0};
    }
  };
  // multi-token units: the draft positions query column c sees
  auto load_mask = [&](int s_) -> uint32_t {
    const int t = c / Gr;
    return (c >= G) ? 0u
           : a.tree_masks ? a.tree_masks[(size_t)s_ * a.query_len + t]
                          : (uint32_t)((2ull << t) - 1);
  };

  using Slice = std::conditional_t<FLAT, TableSliceN<kFlatMaxChunkMatrix / 64>, TableSlice>;
  const size_t blk_stride = (size_t)a.num_kv_heads * STILE;
  // LDS-ring path: block j sits in stage (j - j0) mod 2.  Byte 16 * lane of 1 KiB piece i
  // of a tile is row i * TPLS + lane / LPTS, chunk lane % LPTS, which must hold the row's
  // chunk (lane % LPTS) ^ kswz(row) (K) or ^ swz(row) (V) of the swizzled layouts: that is
  // what the lane fetches, so the wave still reads whole 1 KiB pieces.
  uint32_t goffk[NLDS], goffv[NLDS];
#pragma unroll
  for (int i = 0; i < NLDS; ++i) {
    const int row = i * TPLS + lane / LPTS;
    const uint32_t base = i * 1024 + (lane / LPTS) * (D * E);
    goffk[i] = base + (((lane % LPTS) ^ kswz(row)) * 16);
    goffv[i] = base + (((lane % LPTS) ^ swz(row)) * 16);
  }
  // block jj of the table slice t, KV head kvh_, into stage st of the ring
  auto issue_at = [&](const Slice& t, int kvh_, int jj, int st) {
    const size_t boff = (size_t)t.get(jj) * blk_stride + (size_t)kvh_ * STILE;
    const uint32_t kl = __builtin_amdgcn_readfirstlane(lds_offset(lds_buf[wave][2 * st]));
    const uint32_t vl = __builtin_amdgcn_readfirstlane(lds_offset(lds_buf[wave][2 * st + 1]));
#pragma unroll
    for (int i = 0; i < NLDS; ++i) load_lds_x4<NT>((const char*)a.k + boff + goffk[i], kl + 1024 * i);
#pragma unroll
    for (int i = 0; i < NLDS; ++i) load_lds_x4<NT>((const char*)a.v + boff + goffv[i], vl + 1024 * i);
  };

  // Work: the one unit of unit_coords, or under the flat split (plain and multi-token
  // decodes) this wavefront's walk.  The walk loads the next segment's set-up (table slice,
  // query, draft masks) while the current segment streams, right behind the
  // current segment's first block, so a segment starts by requesting its first block.
  constexpr bool flat = FLAT;  // plain and multi-token decodes only (never prefix units)
  FlatWalk walk;
  FlatSeg nx{0, 0, 0, 0, 0, 0};
  bool nx_ok = false;
  Slice nx_ts;
  u32x4 nx_q[QL];
  uint32_t nx_tm = 0;
  auto prefetch = [&]() {
    nx_ok = walk.next(nx);
    if (!nx_ok) return;
    nx_ts.init(a.tables + (size_t)nx.s * a.max_blocks, nx.j0, nx.j1, a.num_blocks, lane);
    load_query(nx.s, nx.kvh, nx_q);
    if (multi) nx_tm = load_mask(nx.s);
  };
  bool pre_issued = false;  // the segment's first block went out before the last one's partials
  // (m, L, acc) of rows 4r + i, i < 4, of unit (s_, kvh_) into partial slot slot_
  auto store_partials = [&](int s_, int kvh_, int slot_, const f32x4 (&acc)[NTILES],
                            const float (&L_)[4], const float (&M_)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * r + i;
      if (hh < G) {
        const size_t pi = row_at(s_, kvh_, hh) * a.num_slots + slot_;
        float* pa_ = a.part_acc + pi * D + c;
        // Units of 8 or more query rows store their partials with the non-temporal hint
        // (measured: four draft tokens over the GQA workload, 16 rows per unit, decode
        // 392.5 vs 400.7 us, merge 14.9 vs 13.8 us); fewer rows keep ordinary stores
        // (plain GQA even, the fp8 prefix units 0.9 % slower with the hint).
        if constexpr (G >= 8) {
#pragma unroll
          for (int t = 0; t < NTILES; ++t) __builtin_nontemporal_store(acc[t][i], &pa_[16 * t]);
          if (c == 0) {
            __builtin_nontemporal_store(M_[i], &a.part_ml[pi * 2]);
            __builtin_nontemporal_store(L_[i], &a.part_ml[pi * 2 + 1]);
          }
        } else {
#pragma unroll
          for (int t = 0; t < NTILES; ++t) pa_[16 * t] = acc[t][i];
          if (c == 0) {
            a.part_ml[pi * 2] = M_[i];
            a.part_ml[pi * 2 + 1] = L_[i];
          }
        }
      }
    }
  };
  // the flat walk's pending partials (one segment's, stored at the next segment's end)
  bool pd_ok = false;
  int pd_s = 0, pd_kvh = 0, pd_slot = 0;
  f32x4 pd_acc[FLAT ? NTILES : 1];
  float pd_L[4], pd_M[4];
  UnitCoords uc{0, 0, 0, true};
  if constexpr (flat) {
    walk.init(a, BS, PA_GQA_WAVES, wave, lane, kFlatMaxChunkMatrix);
    prefetch();
  } else {
    uc = unit_coords(a, PA_GQA_WAVES, wave, rows, BS);
    if (!uc.ok) return;
  }
  // (one pass over the unit without the flat split: the trip count stays in the loop
  // condition, where the compiler sees it)
  for (int iter = 0; flat || iter < 1; ++iter) {
    int s, kvh, j0, j1, slot;  // s: the sequence, or in prefix mode the group
    // n: tokens the unit's block range covers; jb: first block of the walk.  Column c
    // sees token t iff t < lo or (t < hi and bit t - lo of tm is set).
    int n, jb = 0, lo = 0, hi = 0;
    uint32_t tm = 0;
    Slice ts;
    u32x4 qraw[QL];
    if constexpr (flat) {
      if (!nx_ok) break;
      s = nx.s;
      kvh = nx.kvh;
      j0 = nx.j0;
      j1 = nx.j1;
      slot = nx.slot;
      n = nx.n;
      tm = nx_tm;
      ts = nx_ts;
#pragma unroll
      for (int k = 0; k < QL; ++k) qraw[k] = nx_q[k];
    } else {
      s = uc.s;
      kvh = uc.kvh;
      slot = a.slot_base + uc.part;
      const int32_t* table_row;
      if (prefix) {
        n = 0;
        for (int k = 0; k < a.seq_group; ++k)
          n = max(n, prefix_tokens(a, s, BS, clamp_len(a.ctx[s * a.seq_group + k])));
        lo = hi = (c < G) ? prefix_tokens(a, s, BS, clamp_len(a.ctx[s * a.seq_group + c / Gr])) : 0;
        table_row = a.tables + (size_t)s * a.seq_group * a.max_blocks;  // the group's first member
      } else {
        n = clamp_len(a.ctx[s]);
        if (multi) tm = load_mask(s);
        if (a.mode == MODE_SUFFIX) jb = (prefix_tokens(a, s / a.seq_group, BS, n) + BS - 1) / BS;
        table_row = a.tables + (size_t)s * a.max_blocks;
      }
      const int nblk = (n + BS - 1) / BS;
      const int bpp = part_share_blocks(a, jb, nblk);
      j0 = jb + uc.part * bpp;
      j1 = min(nblk, j0 + bpp);
      if (j0 >= j1) {
        if (a.num_slots == 0) {  // direct output of an n == 0 sequence: zero rows
          for (int cc = 0; cc < G; ++cc) {
            uint16_t* o = (uint16_t*)a.out + row_at(s, kvh, cc) * D;
            for (int e = lane; e < D; e += 64) o[e] = 0;
          }
        } else if (a.mode != MODE_PLAIN && r == 0 && c < G) {  // empty slot of a cascade row
          const size_t pi = row_at(s, kvh, c) * a.num_slots + slot;
          a.part_ml[pi * 2] = -INFINITY;
          a.part_ml[pi * 2 + 1] = 0.f;
        }
        continue;
      }
      // the query's loads go out together with the table-slice load (neither depends on
      // the other), and the first block's loads before the query is converted
      ts.init(table_row, j0, j1, a.num_blocks, lane);
      if constexpr (!DMA) load_query(s, kvh, qraw);  // register path: with the table slice
    }
    if (!prefix) {
      if (multi) {
        lo = (c < G) ? n - a.query_len : 0;
        hi = (c < G) ? n : 0;
      } else {
        lo = hi = (c < G) ? n : 0;
      }
    }
    // Every query column (c < G) sees all tokens below lo_min: a block that ends there
    // needs only the column mask (the per-column bounds matter at a segment's edges only).
    int lo_min = n;
    if constexpr (LANE) {
      int v = (c < G) ? lo : 0x7fffffff;  // columns of lanes 0..15 (the rows repeat them)
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) v = min(v, __shfl_xor(v, off));
      lo_min = __builtin_amdgcn_readfirstlane(v);
    }
    auto row_of = [&](int cc) -> size_t { return row_at(s, kvh, cc); };
    auto issue = [&](int jj, int st) { issue_at(ts, kvh, jj, st); };
    if constexpr (DMA) {
      // The segment's first block goes out before anything else it needs (unless the walk
      // requested it before the last segment's partials); then the next segment's set-up,
      // then (fixed partitions) this one's query.
      if (!pre_issued) issue(j0, 0);
      pre_issued = false;
      if constexpr (flat) prefetch();
      if constexpr (!flat) load_query(s, kvh, qraw);
    }
    const char* kbase = (const char*)a.k + (size_t)kvh * STILE;
    const char* vbase = (const char*)a.v + (size_t)kvh * STILE;
    const uint32_t voff = (uint32_t)lane * 16;  // natural 1 KiB wave loads (K and V)
    auto load_tile = [&](const char* base, int phys, u32x4 (&t)[NLDS]) {
      const char* p = base + (size_t)phys * blk_stride;
#pragma unroll
      for (int i = 0; i < NLDS; ++i) {
        if constexpr (NT) t[i] = __builtin_nontemporal_load((const u32x4*)(p + voff + 1024 * i));
        else t[i] = *(const u32x4*)(p + voff + 1024 * i);
      }
    };
    // Appending decode (the unit that walks the sequence's last block, whose table entry lies
    // in the pool -- an entry outside it skips the write, as the KV write does).  LDS-ring
    // path: once block jn has landed, lane x < CPR writes 16-byte chunk x of the new K and V
    // rows (in the cache's type: e4m3 codes of x * inv_scale, the KV write's conversion)
    // into slot tn of the staged tiles, and the rows go to the cache after the epilogue, so
    // no load waits for the store.  Register path: the rows are stored first.
    const int jn = (n - 1) / BS, tn = (n - 1) % BS;
    bool app = a.append && a.mode == MODE_PLAIN && n > 0 && j1 == (n + BS - 1) / BS;
    int app_phys = 0;
    u32x4 nk = u32x4{0, 0, 0, 0}, nv = u32x4{0, 0, 0, 0};
    if constexpr (DMA) {
      if (app && lane < CPR) {  // loaded whatever the table entry says (checked below)
        const size_t src = ((size_t)s * a.num_kv_heads + kvh) * D + (size_t)lane * (16 / LE);
        const u32x4* ks = (const u32x4*)((const uint16_t*)a.k_new + src);
        const u32x4* vs = (const u32x4*)((const uint16_t*)a.v_new + src);
        if constexpr (LE == 1) {
          const u32x2 k0 = src8_to_e4m3<QK>(ks[0], a.k_inv_scale), k1 = src8_to_e4m3<QK>(ks[1], a.k_inv_scale);
          const u32x2 v0 = src8_to_e4m3<QK>(vs[0], a.v_inv_scale), v1 = src8_to_e4m3<QK>(vs[1], a.v_inv_scale);
          nk = u32x4{k0[0], k0[1], k1[0], k1[1]};
          nv = u32x4{v0[0], v0[1], v1[0], v1[1]};
        } else {
          nk = ks[0];
          nv = vs[0];
        }
      }
    }
    if (app) {
      app_phys = ts.raw(jn);
      app = (unsigned)app_phys < (unsigned)a.num_blocks;
    }
    if constexpr (!DMA) {
      if (app) append_new_row<D, BS, QK, KVK>(a, s, kvh, app_phys, tn, lane, jn - j0 < 2);
    }
    u32x4 ka[NLDS], va[NLDS], kb[NLDS], vb[NLDS];
    // The barrier keeps the scheduler from hoisting the next block's LDS staging (and its
    // wait for that block's loads) above these loads: the loads of block j+1 must be in
    // flight before the wave waits for block j.
    auto fetch = [&](int jj, u32x4 (&kr)[NLDS], u32x4 (&vr)[NLDS]) {
      const int p = ts.get(jj);
      load_tile(kbase, p, kr);
      load_tile(vbase, p, vr);
      __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (!DMA) {
      fetch(j0, ka, va);
      if constexpr (flat) prefetch();  // the next segment's set-up, behind this first block
    }

    // Q^T operand: lane (r, c) holds head c's dims 32kk + 8r .. +8 (zero for padding heads)
    u32x4 qop[NATIVE ? 1 : KSTEPS];
    // native: head c's dims QD*r .. +QD as three e4m3 terms (zero for padding heads), and
    // the E8M0 exponent 127 - e of the operand scale 2^-e that undoes the head's 2^e
    v8i qn[NATIVE ? 3 : 1];
    int q_exp = 127;
    if constexpr (NATIVE) {
      float qv[QD];
#pragma unroll
      for (int k = 0; k < QD / 8; ++k) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          qv[8 * k + 2 * w] = (QK == KIND_BF16) ? bf16_lo(qraw[k][w]) : f16_lo(qraw[k][w]);
          qv[8 * k + 2 * w + 1] = (QK == KIND_BF16) ? bf16_hi(qraw[k][w]) : f16_hi(qraw[k][w]);
        }
      }
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < QD; ++i) mx = fmaxf(mx, fabsf(qv[i]));
      mx = rows_max(mx);
      // mx in [2^(x-1), 2^x) -> scale by 2^(8-x): the largest element lands in [128, 256)
      int e = (mx > 0.f) ? 8 - __builtin_amdgcn_frexp_expf(mx) : 0;
      e = e > 127 ? 127 : e;
      q_exp = 127 - e;
#pragma unroll
      for (int t = 0; t < 3; ++t) qn[t] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < QD / 4; ++w) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __builtin_amdgcn_ldexpf(qv[4 * w + i], e);
#pragma unroll
        for (int t = 0; t < 3; ++t) {  // each term takes the rounding residual of the last
          const uint32_t code = e4m3x4_pack(x[0], x[1], x[2], x[3]);
          qn[t][w] = (int)code;
          float back[4];
          e4m3x4_to_f32(code, back);
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] -= back[i];
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qop[kk] = qraw[kk];
    }

    // Output accumulators (matrix-core C operands) hold P . V relative to the reference
    // maximum; they are rescaled only when the reference moves.
    f32x4 cacc[NTILES];
#pragma unroll
    for (int t = 0; t < NTILES; ++t) cacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY;  // reference maximum of head c (log2 units), same in its 4 lanes
    float l_part = 0.f;       // this lane's share of head c's denominator

    uint8_t* kt = lds_buf[wave][0];
    uint8_t* vt = lds_buf[wave][1];
    const float qk_scale = a.qk_scale;
    // This lane's share of a tile: wave load i, token row i*TPLS + lane/LPTS, elements
    // (lane % LPTS) * EPLS .. +EPLS, i.e. LDS chunks (lane % LPTS) * CPL .. +CPL of that row.
    // K's chunk x of row t sits at x ^ kswz(t): the operand reads (row c, one chunk) of 16
    // lanes hit 16 different bank groups.  V's chunk x sits at x ^ swz(t).
    uint32_t kw_off[NLDS][CPL], vw_off[NLDS][CPL];
#pragma unroll
    for (int i = 0; i < NLDS; ++i) {
      const int row = i * TPLS + lane / LPTS;
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const int chunk = (lane % LPTS) * CPL + q;
        kw_off[i][q] = row * PITCH + ((chunk ^ kswz(row)) * 16);
        vw_off[i][q] = row * PITCH + ((chunk ^ swz(row)) * 16);
      }
    }
    const int trow = 4 * r + c / 4;

    // widen (e4m3) and write one tile into LDS; rows at or beyond n become zeros when
    // `mask` (their bytes may be NaN and the matrix core would turn 0 * NaN into NaN)
    auto stage = [&](uint8_t* dst, const uint32_t (&off)[NLDS][CPL], bool mask, int j,
                     const u32x4 (&t)[NLDS]) {
#pragma unroll
      for (int i = 0; i < NLDS; ++i) {
        u32x4 w[CPL];
        if constexpr (NATIVE) {
          w[0] = t[i];
        } else if constexpr (KVK == KIND_E4M3) {
          u32x4 two[2];
          e4m3x16_widen<QK>(t[i], two);
          w[0] = two[0];
          w[CPL - 1] = two[1];
        } else {
          w[0] = t[i];
        }
        const bool dead = mask && j * BS + i * TPLS + lane / LPTS >= n;
#pragma unroll
        for (int q = 0; q < CPL; ++q) *(u32x4*)(dst + off[i][q]) = dead ? u32x4{0, 0, 0, 0} : w[q];
      }
    };

    // logits of block j: C[token 4r+i][head c]
    auto logits = [&]() {
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (NATIVE) {
        // K's operand: token c, the same dims QD*r .. +QD that lane (r, c) holds of Q
        const uint8_t* row = kt + c * PITCH;
        const u32x4 lo = *(const u32x4*)(row + ((((QD / 16) * r) ^ kswz(c)) * 16));
        u32x4 hi = u32x4{0, 0, 0, 0};
        if constexpr (QD == 32) hi = *(const u32x4*)(row + (((2 * r + 1) ^ kswz(c)) * 16));
        const v8i kop = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
        for (int t = 0; t < 3; ++t) sc = mfma_e4m3(kop, qn[t], sc, 127, q_exp);
      } else {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const int chunk = (4 * kk + r) ^ kswz(c);
          const u32x4 kop = *(const u32x4*)(kt + c * PITCH + chunk * 16);
          sc = Ops::qk(kop, qop[kk], sc);
        }
      }
      return sc;
    };

    // online-softmax weights and P . V for block j (MASK: the block holds slots >= n)
    auto finish = [&](int j, f32x4 sv) {
      float z[4];
      if (j * BS + BS <= lo_min) {  // (wave-uniform) the block lies below every bound
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = c < G ? sv[i] * qk_scale : -INFINITY;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = j * BS + 4 * r + i;
          const bool ok = LANE ? (t < lo || (t < hi && ((tm >> ((t - lo) & 31)) & 1u)))
                               : (c < G && t < n);
          z[i] = ok ? sv[i] * qk_scale : -INFINITY;
        }
      }
      float bm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      bm = rows_max(bm);
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
      if constexpr (NATIVE) {
        // weights 2^(z - ms) <= 2^8, lifted by 2^kb so the block's largest is in [2^7, 2^8)
        const float rel = bm - ms;
        int kb = 0;
        if (rel > -INFINITY) {
          kb = 7 - (int)floorf(rel);
          kb = kb > 126 ? 126 : kb;
        }
        float p[4], pp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = fast_exp2(z[i] - ms);
          pp[i] = __builtin_amdgcn_ldexpf(p[i], kb);  // exact
        }
        const uint32_t hi = e4m3x4_pack(pp[0], pp[1], pp[2], pp[3]);
        float back[4];
        e4m3x4_to_f32(hi, back);
        const uint32_t lo = e4m3x4_pack(pp[0] - back[0], pp[1] - back[1], pp[2] - back[2],
                                        pp[3] - back[3]);
        // P's operand: head c, tokens 4r .. 4r+3 as hi then lo; V's operand repeats those
        // four tokens so both halves meet the same values; the A-operand scale 2^-kb undoes
        // the lift.  The operands carry 8 codes of the 32 the instruction takes (the rest
        // zero); issuing one tile at a time keeps a single zero-padded V operand live (about
        // 30 fewer VGPRs at D = 128 than letting the compiler build all eight up front).
        const v8i pop8 = v8i{(int)hi, (int)lo, 0, 0, 0, 0, 0, 0};
        l_part += (p[0] + p[1]) + (p[2] + p[3]);
        const int rho = 4 * r + ((c >> 1) & 3);
#pragma unroll
        for (int t = 0; t < NTILES; ++t) {
          const v2i vv = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_v2i*)(vt + rho * PITCH + ((t ^ swz(rho)) * 16) + 8 * (c & 1)));
          const v8i vop = v8i{vv[0], vv[1], 0, 0, 0, 0, 0, 0};
          cacc[t] = mfma_e4m3(pop8, vop, cacc[t], 127 - kb, 127);
          __builtin_amdgcn_sched_barrier(0);
        }
        return;
      }
      float p[4], rp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(z[i] - ms);
      const uint32_t p01 = Ops::pack2(p[0], p[1], &rp[0], &rp[1]);
      const uint32_t p23 = Ops::pack2(p[2], p[3], &rp[2], &rp[3]);
      const u32x2 pop = u32x2{p01, p23};
      // A weight rounded to the operand type is off by up to 2^-9 (bf16) or 2^-12 (fp16) of
      // itself, which a few dominant tokens with distant values turn into output errors of
      // the order of the 2e-3 bar.  So P goes in as hi + lo (the second MFMA takes the
      // rounding residual, exact to about 2^-17 / 2^-23) and the denominator sums the
      // unrounded weights.
      float unused[4];
      const u32x2 plo = u32x2{Ops::pack2(p[0] - rp[0], p[1] - rp[1], &unused[0], &unused[1]),
                              Ops::pack2(p[2] - rp[2], p[3] - rp[3], &unused[2], &unused[3])};
      l_part += (p[0] + p[1]) + (p[2] + p[3]);
      // P . V over the 16 tokens, one 16-wide slice of the head dimension at a time
#pragma unroll
      for (int t = 0; t < NTILES; ++t) {
        const uint32_t chunk = (2 * t + (c % 4) / 2) ^ swz(trow);
        const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vt + trow * PITCH + chunk * 16 + 8 * (c % 2)));
        cacc[t] = Ops::pv(pop, vb, cacc[t]);
        cacc[t] = Ops::pv(plo, vb, cacc[t]);
      }
    };

    // Pipeline (register path): two register sets of K and V tiles, as in the vector kernel;
    // consuming block j moves K(j) and V(j) into the LDS tiles, runs the logit contraction,
    // the softmax update and P . V.  The mask of slots >= n is applied branch-free (it only
    // bites in a unit's last block).
    if constexpr (DMA) {
      constexpr int PER = 2 * NLDS;  // vector-memory operations per block
      int st = 0;
      for (int j = j0; j < j1; ++j) {
        // fill the other stage (read by block j - 1) with block j + 1, then wait for block j
        if (j + 1 < j1) {
          issue(j + 1, st ^ 1);
          wait_vmcnt<PER>();
        } else {
          wait_vmcnt<0>();
        }
        kt = lds_buf[wave][2 * st];
        vt = lds_buf[wave][2 * st + 1];
        if (app && j == jn && lane < CPR) {  // the new token's rows into slot tn
          *(u32x4*)(kt + tn * PITCH + ((lane ^ kswz(tn)) * 16)) = nk;
          *(u32x4*)(vt + tn * PITCH + ((lane ^ swz(tn)) * 16)) = nv;
        }
        if (j * BS + BS > n) {  // V rows at or beyond n become zeros (their bytes may be NaN)
#pragma unroll
          for (int x = lane; x < TILE / 16; x += 64)
            if (j * BS + x / CPR >= n) *(u32x4*)(vt + x * 16) = u32x4{0, 0, 0, 0};
        }
        finish(j, logits());
        st ^= 1;
      }
    } else {
      // A block's registers are free once it sits in LDS, so the block two ahead is fetched
      // into them before the block's contractions run: two blocks stay in flight while one
      // is consumed.  Steady state: blocks j .. j+3 exist, ka/va hold block j and kb/vb
      // block j + 1, and every load in the loop is unconditional (see the vector kernel).
      auto stage_kv = [&](int j, const u32x4 (&kr)[NLDS], const u32x4 (&vr)[NLDS]) {
        stage(kt, kw_off, false, j, kr);
        stage(vt, vw_off, true, j, vr);
      };
      int j = j0;
      if (j + 1 < j1) fetch(j + 1, kb, vb);
      while (j + 3 < j1) {
        stage_kv(j, ka, va);
        fetch(j + 2, ka, va);
        finish(j, logits());
        stage_kv(j + 1, kb, vb);
        fetch(j + 3, kb, vb);
        finish(j + 1, logits());
        j += 2;
      }
      // one to three blocks left: ka/va hold block j, kb/vb block j + 1 when it exists
      stage_kv(j, ka, va);
      if (j + 2 < j1) fetch(j + 2, ka, va);
      finish(j, logits());
      if (j + 1 < j1) {
        stage_kv(j + 1, kb, vb);
        finish(j + 1, logits());
      }
      if (j + 2 < j1) {
        stage_kv(j + 2, ka, va);
        finish(j + 2, logits());
      }
    }

    // flat walk: the next segment's first block goes out before this segment's partials
    // (its table slice is already here), into stage 0, where that segment starts
    if constexpr (flat && DMA) {
      if (nx_ok) {
        issue_at(nx_ts, nx.kvh, nx.j0, 0);
        pre_issued = true;
      }
    }
    // head c's denominator: sum of its four lanes' shares; accumulator row 4r + i (lane c
    // holds dim 16t + c of slice t) belongs to head 4r + i, whose (m, L) sit in lane 4r + i
    const float L = rows_sum(l_part);
    float Lr[4], Mr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Lr[i] = __shfl(L, 4 * r + i);
      Mr[i] = __shfl(m_ref, 4 * r + i);
    }
    if (a.num_slots == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = 4 * r + i;
        if (hh < G) {
          uint16_t* o = (uint16_t*)a.out + row_of(hh) * D + c;
          // a column that sees no token (possible under a draft mask) gives a zero row
          const float inv = (Lr[i] > 0.f) ? a.v_scale / Lr[i] : 0.f;
#pragma unroll
          for (int t = 0; t < NTILES; ++t) o[16 * t] = f32_to_store<QK>(cacc[t][i] * inv);
        }
      }
    } else if constexpr (flat) {
      // The walk's partials leave one segment late: the previous segment's now, this one's
      // at the next segment's end or after the walk.  (A wave's next wait on its loads also
      // waits for every store it issued before them, and stores issued among a full-rate
      // read stream are slow to complete: storing each segment's partials at its end cost
      // the four-draft-token GQA decode 22 us of 393.)
      if (pd_ok) store_partials(pd_s, pd_kvh, pd_slot, pd_acc, pd_L, pd_M);
      pd_ok = true;
      pd_s = s;
      pd_kvh = kvh;
      pd_slot = slot;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pd_L[i] = Lr[i];
        pd_M[i] = Mr[i];
#pragma unroll
        for (int t = 0; t < NTILES; ++t) pd_acc[t][i] = cacc[t][i];
      }
    } else {
      store_partials(s, kvh, slot, cacc, Lr, Mr);
    }
    // appending decode, LDS-ring path: the new rows into the cache, after everything that
    // read the block
    if (DMA && app && lane < CPR) {
      const size_t dst = (((size_t)app_phys * a.num_kv_heads + kvh) * BS + tn) * (D * E) +
                         (size_t)lane * 16;
      *(u32x4*)((char*)a.k + dst) = nk;
      *(u32x4*)((char*)a.v + dst) = nv;
    }
  }
  if constexpr (flat) {
    if (pd_ok) store_partials(pd_s, pd_kvh, pd_slot, pd_acc, pd_L, pd_M);
  }
}

template <int D, int QK, int KVK, int G, bool NT, bool LANE, bool FLAT>
__global__ __launch_bounds__(64 * PA_GQA_WAVES, gqa_min_waves(KVK, LANE, G)) void paged_decode_gqa_mfma_kernel(
    const DecodeArgs a) {
  gqa_body<D, QK, KVK, G, NT, LANE, FLAT>(a);
}

template <int D, int QK, int KVK, int G, bool NT>
hipError_t launch_gqa_mfma_t(const DecodeArgs& a, hipStream_t stream) {
  const dim3 block(64 * PA_GQA_WAVES);
  const bool lane_masks = a.mode == MODE_PREFIX || a.mode == MODE_MULTI;
  if (a.flat_min_blocks > 0) {
    // the flat split: plain and multi-token decodes over 16-bit caches only (the host never
    // asks it otherwise)
    if (a.mode != MODE_PLAIN && a.mode != MODE_MULTI) return hipErrorInvalidValue;
    if constexpr (KVK == KIND_E4M3) {
      return hipErrorInvalidValue;
    } else {
      static std::atomic<int> resident[2][kMaxCachedDevices];
      if (lane_masks)
        hipLaunchKernelGGL((paged_decode_gqa_mfma_kernel<D, QK, KVK, G, NT, true, true>),
                           decode_grid(a, PA_GQA_WAVES,
                                       (const void*)paged_decode_gqa_mfma_kernel<D, QK, KVK, G, NT, true, true>,
                                       resident[1]),
                           block, 0, stream, a);
      else
        hipLaunchKernelGGL((paged_decode_gqa_mfma_kernel<D, QK, KVK, G, NT, false, true>),
                           decode_grid(a, PA_GQA_WAVES,
                                       (const void*)paged_decode_gqa_mfma_kernel<D, QK, KVK, G, NT, false, true>,
                                       resident[0]),
                           block, 0, stream, a);
      return hipGetLastError();
    }
  }
  const dim3 grid = decode_grid(a, PA_GQA_WAVES);
  if (lane_masks)
    hipLaunchKernelGGL((paged_decode_gqa_mfma_kernel<D, QK, KVK, G, NT, true, false>), grid, block, 0,
                       stream, a);
  else
    hipLaunchKernelGGL((paged_decode_gqa_mfma_kernel<D, QK, KVK, G, NT, false, false>), grid, block, 0,
                       stream, a);
  return hipGetLastError();
}

template <int D, bool NT>
hipError_t launch_gqa_mfma_d(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
#define PA_GQ(QK, KVK)                                                     \
  switch (s.group) {                                                       \
    case 2: return launch_gqa_mfma_t<D, QK, KVK, 2, NT>(a, stream);        \
    case 4: return launch_gqa_mfma_t<D, QK, KVK, 4, NT>(a, stream);        \
    case 8: return launch_gqa_mfma_t<D, QK, KVK, 8, NT>(a, stream);        \
    case 16: return launch_gqa_mfma_t<D, QK, KVK, 16, NT>(a, stream);      \
    default: return hipErrorInvalidValue;                                  \
  }
  if (s.q_kind == KIND_BF16 && s.kv_kind == KIND_BF16) { PA_GQ(KIND_BF16, KIND_BF16) }
  if (s.q_kind == KIND_F16 && s.kv_kind == KIND_F16) { PA_GQ(KIND_F16, KIND_F16) }
  if (s.q_kind == KIND_BF16 && s.kv_kind == KIND_E4M3) { PA_GQ(KIND_BF16, KIND_E4M3) }
  if (s.q_kind == KIND_F16 && s.kv_kind == KIND_E4M3) { PA_GQ(KIND_F16, KIND_E4M3) }
  return hipErrorInvalidValue;
#undef PA_GQ
}

}  // namespace pa
