// Device-side helpers shared by the gfx950 kernels of libpaged_attn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---- DPP cross-lane moves inside a 16-lane row -------------------------------------
// Control words of the GFX9 DPP encoding.
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over groups of N consecutive lanes (N in {2,4,8,16}); every lane of a group gets
// the group's total.  xor-1 and xor-2 are quad permutes; the 8- and 16-lane steps use
// the half-row and row mirrors, which pair lane i with its reflection, i.e. the other
// half of the group, after the smaller groups have been summed.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group size");
  x += dpp_mov<DPP_QUAD_XOR1>(x);
  if constexpr (N >= 4) x += dpp_mov<DPP_QUAD_XOR2>(x);
  if constexpr (N >= 8) x += dpp_mov<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp_mov<DPP_ROW_MIRROR>(x);
  return x;
}

// op(x, x of lane ^ OFF) for a commutative op, OFF in {1, 2, 4, 8, 16, 32}, by VALU lane
// moves rather than an LDS-crossbar permute (which costs an LDS round trip and a wait per
// step): quad permutes for 1 and 2, two bank-masked row shifts for 4 (banks 0 and 2 take
// the lanes 4 above, banks 1 and 3 the lanes 4 below), a half-row rotate for 8, and the
// gfx950 permlane16 / permlane32 swaps for 16 and 32.  Measured lane layout:
// permlane16_swap(x, x) returns rows (0, 0, 2, 2) and (1, 1, 3, 3) of x (16-lane rows),
// permlane32_swap(x, x) halves (0, 0) and (1, 1); each lane so holds its own value and
// its partner's, in one order or the other, and op(first, second) is op(own, partner)
// bit for bit.
constexpr int DPP_ROW_SHL4 = 0x104;
constexpr int DPP_ROW_SHR4 = 0x114;
constexpr int DPP_ROW_ROR8 = 0x128;

template <int OFF, typename Op>
__device__ __forceinline__ float xor_combine(float x, Op op) {
  static_assert(OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8 || OFF == 16 || OFF == 32,
                "lane distance");
  const int xi = __float_as_int(x);
  if constexpr (OFF == 1) {
    return op(x, dpp_mov<DPP_QUAD_XOR1>(x));
  } else if constexpr (OFF == 2) {
    return op(x, dpp_mov<DPP_QUAD_XOR2>(x));
  } else if constexpr (OFF == 4) {
    int p = __builtin_amdgcn_update_dpp(0, xi, DPP_ROW_SHL4, 0xF, 0x5, false);
    p = __builtin_amdgcn_update_dpp(p, xi, DPP_ROW_SHR4, 0xF, 0xA, false);
    return op(x, __int_as_float(p));
  } else if constexpr (OFF == 8) {
    return op(x, dpp_mov<DPP_ROW_ROR8>(x));
  } else if constexpr (OFF == 16) {
    const auto s = __builtin_amdgcn_permlane16_swap((unsigned)xi, (unsigned)xi, false, false);
    return op(__uint_as_float(s[0]), __uint_as_float(s[1]));
  } else {
    const auto s = __builtin_amdgcn_permlane32_swap((unsigned)xi, (unsigned)xi, false, false);
    return op(__uint_as_float(s[0]), __uint_as_float(s[1]));
  }
}

struct AddOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// op over the lanes whose indices differ from this lane's only in bits FROM .. 32 (FROM a
// power of two), combined from the lowest of those bits up; every lane gets the result.
template <int FROM, typename Op>
__device__ __forceinline__ float across_lanes(float x, Op op) {
  if constexpr (FROM >= 64) {
    return x;
  } else {
    return across_lanes<FROM * 2>(xor_combine<FROM>(x, op), op);
  }
}

// Reduce-scatter of N values over the lanes whose indices differ from this lane's only in
// bits FROM .. 32 (FROM in {4, 8, 16}): afterwards v[0 .. N * FROM / 64) hold the sums of
// values rs_first<FROM, N>(lane) onwards.  Each step pairs lane l with l ^ OFF; the lane
// with bit OFF clear keeps the lower half of its live values, the other the upper half,
// and each adds what its partner sends of its own half (DPP moves inside a row for 4 and
// 8, the permlane swaps for 16 and 32, which bring both lanes' values in one move).  Every
// sum is own + partner at each step, from the lowest bit up, as across_lanes forms it, so
// the results are the same bits, with N/2 + N/4 + ... lane moves instead of N per step.
template <int OFF>
__device__ __forceinline__ float xor_partner(float x) {
  static_assert(OFF == 4 || OFF == 8, "DPP lane distance");
  if constexpr (OFF == 8) {
    return dpp_mov<DPP_ROW_ROR8>(x);
  } else {
    const int xi = __float_as_int(x);
    int p = __builtin_amdgcn_update_dpp(0, xi, DPP_ROW_SHL4, 0xF, 0x5, false);
    p = __builtin_amdgcn_update_dpp(p, xi, DPP_ROW_SHR4, 0xF, 0xA, false);
    return __int_as_float(p);
  }
}

template <int OFF, int LIVE, int N>
__device__ __forceinline__ void rs_steps(float (&v)[N], int lane) {
  if constexpr (OFF < 64) {
    constexpr int H = LIVE / 2;
    static_assert(H >= 1, "more lanes than values");
    if constexpr (OFF == 16 || OFF == 32) {
#pragma unroll
      for (int k = 0; k < H; ++k) {
        const unsigned lo = __float_as_uint(v[k]), hi = __float_as_uint(v[k + H]);
        if constexpr (OFF == 16) {
          const auto t = __builtin_amdgcn_permlane16_swap(lo, hi, false, false);
          v[k] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
        } else {
          const auto t = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
          v[k] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
        }
      }
    } else {
      const bool upper = (lane & OFF) != 0;
#pragma unroll
      for (int k = 0; k < H; ++k) {
        const float keep = upper ? v[k + H] : v[k];
        const float send = upper ? v[k] : v[k + H];
        v[k] = keep + xor_partner<OFF>(send);
      }
    }
    rs_steps<OFF * 2, H, N>(v, lane);
  }
}

template <int FROM, int N>
__device__ __forceinline__ void reduce_scatter(float (&v)[N], int lane) {
  static_assert(N * FROM / 64 >= 1, "more lanes than values");
  rs_steps<FROM, N, N>(v, lane);
}

template <int FROM, int N>
__device__ __forceinline__ int rs_first(int lane) {
  int first = 0, live = N;
#pragma unroll
  for (int off = FROM; off < 64; off <<= 1) {
    live /= 2;
    if (lane & off) first += live;
  }
  return first;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- conversions ---------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[1];
}

// binary32 -> bfloat16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32 under the default round-to-nearest-even mode
  return __builtin_bit_cast(uint16_t, h);
}

template <int K>
__device__ __forceinline__ uint16_t f32_to_store(float f) {
  if constexpr (K == KIND_BF16) return f32_to_bf16_rne(f);
  else return f32_to_f16_rne(f);
}

// Four e4m3 codes of a dword -> four floats (OCP E4M3 decode by the gfx950 converter).
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* o) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = lo[0]; o[1] = lo[1]; o[2] = hi[0]; o[3] = hi[1];
}

// Four e4m3 codes of a dword -> their values as two dwords of packed fp16 or bf16 pairs
// (codes 0, 1 and 2, 3), by the gfx950 scaled converter at scale 1.  Exact: every E4M3
// value (at most 448 in magnitude, subnormals down to 2^-9) is an fp16 and a bf16 value.
template <int K>
__device__ __forceinline__ u32x2 e4m3x4_to_16(uint32_t w) {
  if constexpr (K == KIND_BF16)
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
  else
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))};
}

// c + a.x * b.x + a.y * b.y over packed fp16 or bf16 pairs, fp32 result.
template <int K>
__device__ __forceinline__ float dot2_16(uint32_t a, uint32_t b, float c) {
  if constexpr (K == KIND_BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

// binary32 -> OCP E4M3 code, round to nearest even, saturating at +-448, NaN -> NaN.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;          // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;         // |x| >= 448 (and inf): largest finite
  if (a >= 0x3C800000u) {                             // |x| >= 2^-6: normal E4M3 range
    // keep 3 of the 23 fraction bits, ties to even; a carry bumps the exponent
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));                  // rebias exponent 127 -> 7
  }
  // subnormal range: multiples of 2^-9; 8 * 2^-9 is the smallest normal (code 0x08)
  const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
  return sign | (uint32_t)m;
}

// Eight fp16/bf16 source elements (16 bytes) of a new K or V row -> their eight e4m3 cache
// codes (8 bytes): e4m3(float(x) * inv_scale), the binary32 product rounded to nearest even
// and saturated.  The one conversion both the KV write and the appending decode use.
template <int SK>
__device__ __forceinline__ u32x2 src8_to_e4m3(u32x4 x, float inv_scale) {
  u32x2 o;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    uint32_t b = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t xw = x[2 * w + e / 2];
      const float f = (SK == KIND_BF16) ? ((e & 1) ? bf16_hi(xw) : bf16_lo(xw))
                                        : ((e & 1) ? f16_hi(xw) : f16_lo(xw));
      b |= f32_to_e4m3_sat(f * inv_scale) << (8 * e);
    }
    o[w] = b;
  }
  return o;
}

// Wait until at most N vector-memory operations (loads and stores) of this wave are
// outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Appending decode: store the new token's K and V rows (row `slot` of block `phys`, KV head
// kvh) into the cache, as the KV write would: lane x < D * E / 16 stores 16 cache bytes of
// chunk x, copied from a source of the cache's type or converted to e4m3 (src8_to_e4m3).
// The caller loads that block afterwards (nothing cached it before: only this unit reads
// it), so the stores must be done before that load is issued.  vmcnt counts loads and
// stores together and retires them in order, so once the caller has waited for a load
// issued after these stores they are done as well; `wait` is for the caller whose load of
// the block goes out before any such wait (the block is among its first two).
template <int D, int BS, int QK, int KVK>
__device__ __forceinline__ void append_new_row(const DecodeArgs& a, int s, int kvh, int phys,
                                               int slot, int lane, bool wait) {
  constexpr int E = (KVK == KIND_E4M3) ? 1 : 2;
  constexpr int CH = D * E / 16;  // 16-byte chunks of a cache row
  if (lane < CH) {
    const size_t src = ((size_t)s * a.num_kv_heads + kvh) * D + (size_t)lane * (16 / E);
    const u32x4* ks = (const u32x4*)((const uint16_t*)a.k_new + src);
    const u32x4* vs = (const u32x4*)((const uint16_t*)a.v_new + src);
    u32x4 nk, nv;
    if constexpr (E == 1) {
      const u32x2 k0 = src8_to_e4m3<QK>(ks[0], a.k_inv_scale), k1 = src8_to_e4m3<QK>(ks[1], a.k_inv_scale);
      const u32x2 v0 = src8_to_e4m3<QK>(vs[0], a.v_inv_scale), v1 = src8_to_e4m3<QK>(vs[1], a.v_inv_scale);
      nk = u32x4{k0[0], k0[1], k1[0], k1[1]};
      nv = u32x4{v0[0], v0[1], v1[0], v1[1]};
    } else {
      nk = ks[0];
      nv = vs[0];
    }
    const size_t dst = (((size_t)phys * a.num_kv_heads + kvh) * BS + slot) * (D * E) + (size_t)lane * 16;
    *(u32x4*)((char*)a.k + dst) = nk;
    *(u32x4*)((char*)a.v + dst) = nv;
  }
  if (wait) wait_vmcnt<0>();
}

// A work unit walks at most 64 blocks, so its slice of the block table fits one VGPR:
// lane k holds entry j0 + k (loaded once, unconditionally, with the index clamped into the
// unit's range), and the physical id of block j is read with v_readlane into a scalar
// register.  Entries outside [0, num_blocks) are replaced by block 0 so a malformed table
// can never fault.  Keeping every load of the block loop unconditional also lets the
// compiler's in-order load counters wait for exactly the block being consumed.
struct TableSlice {
  int j0, nb, ids;

  __device__ __forceinline__ void init(const int32_t* row, int j0_, int j1, int nb_, int lane) {
    j0 = j0_;
    nb = nb_;
    const int jj = j0 + lane < j1 ? j0 + lane : j1 - 1;
    ids = row[jj];
  }
  // j is wave-uniform, j0 <= j < j0 + 64
  __device__ __forceinline__ int raw(int j) const { return __builtin_amdgcn_readlane(ids, j - j0); }
  __device__ __forceinline__ int get(int j) const {
    const int p = raw(j);
    return ((unsigned)p < (unsigned)nb) ? p : 0;
  }
};

// The same over at most 64 * NS blocks in NS VGPRs (entry j0 + 64 q + lane in ids[q]): the
// flat walk's chunks may be that long.
template <int NS>
struct TableSliceN {
  int j0, nb, ids[NS];

  __device__ __forceinline__ void init(const int32_t* row, int j0_, int j1, int nb_, int lane) {
    j0 = j0_;
    nb = nb_;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      const int jj = j0 + 64 * q + lane;
      ids[q] = row[jj < j1 ? jj : j1 - 1];
    }
  }
  // j is wave-uniform, j0 <= j < j0 + 64 * NS
  __device__ __forceinline__ int raw(int j) const {
    const int d = j - j0;
    int v = 0;
#pragma unroll
    for (int q = 0; q < NS; ++q)
      if (d >> 6 == q) v = __builtin_amdgcn_readlane(ids[q], d & 63);
    return v;
  }
  __device__ __forceinline__ int get(int j) const {
    const int p = raw(j);
    return ((unsigned)p < (unsigned)nb) ? p : 0;
  }
};

// Work-unit coordinates (row s, KV head, partition) of wavefront `wave` of this
// workgroup (`waves` per workgroup); false when the wavefront has no unit.
//   xcd_remap 1: the hardware deals workgroups to the 8 XCDs round-robin; they are
//     renumbered so that XCD x runs a contiguous range of logical workgroups (a bijection
//     for any grid size).  0: launch order.  2: work-balanced ranges (balanced_coords).
//   seq_fastest 0: units in (row, partition, KV head) order, neighbouring heads of the
//     same blocks side by side; 1: (partition, KV head, row), the rows that share blocks
//     side by side.
struct UnitCoords {
  int s, kvh, part;
  bool ok;
};

__device__ __forceinline__ UnitCoords remapped_coords(const DecodeArgs& a, int waves, int wave,
                                                      int rows) {
  // (a launch's workgroups may be a range of a larger grid: the one-launch cascade)
  int wg = (int)blockIdx.x - a.wg_base;
  if (a.xcd_remap != 0) {
    const int G8 = a.wg_count > 0 ? a.wg_count : (int)gridDim.x;
    const int x = wg % 8, loc = wg / 8, per = G8 / 8, rem = G8 % 8;
    wg = (x < rem) ? x * (per + 1) + loc : rem * (per + 1) + (x - rem) * per + loc;
  }
  const int unit = wg * waves + wave;
  UnitCoords u;
  u.ok = unit < a.num_units;
  if (a.seq_fastest == 0) {
    u.kvh = unit % a.num_kv_heads;
    const int rest = unit / a.num_kv_heads;
    u.part = rest % a.num_parts;
    u.s = rest / a.num_parts;
  } else {
    u.s = unit % rows;
    const int rest = unit / rows;
    u.kvh = rest % a.num_kv_heads;
    u.part = rest / a.num_kv_heads;
  }
  return u;
}

// Work-balanced XCD ranges (xcd_remap 2; units in (row, partition, KV head) order; at most
// kBalancedMaxSeqs rows).  The row-partitions that hold blocks are laid out in row order;
// XCD x takes those whose first block lies in the x-th eighth of all the rows' blocks, KV
// heads fastest, so every XCD reads the same amount of K/V (to within one partition) and
// still works through a few neighbouring rows at a time; partitions past a row's end get
// no unit at all.  Workgroup i runs on XCD i % 8 (round-robin dealing); the grid has
// rows * num_parts * num_kv_heads units, and the workgroups of an XCD beyond its range's
// units find none and exit.  If some XCD's range has more units than the XCD has
// wavefronts, every wavefront falls back to the contiguous mapping (the decision is the
// same in all of them: it depends only on the lengths).  Every cross-lane chain below is
// independent of the others, so they overlap.
__device__ __forceinline__ UnitCoords balanced_coords(const DecodeArgs& a, int waves, int wave,
                                                      int block_size) {
  const int lane = threadIdx.x & 63;
  const int S = a.num_seqs, bpp = a.blocks_per_part, H = a.num_kv_heads;
  if (S > kBalancedMaxSeqs) return remapped_coords(a, waves, wave, S);
  constexpr int K = kBalancedMaxSeqs / 64;
  // lane's rows s = lane + 64 k: blocks and non-empty partitions
  int nb[K], np[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int s = lane + 64 * k;
    int n = s < S ? a.ctx[s] : 0;
    n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
    nb[k] = (n + block_size - 1) / block_size;
    np[k] = (nb[k] + bpp - 1) / bpp;
  }
  // exclusive prefix sums in row order: wb = blocks before the row, wp = row-partitions
  int ib[K], ip[K];
#pragma unroll
  for (int k = 0; k < K; ++k) { ib[k] = nb[k]; ip[k] = np[k]; }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int yb = __shfl_up(ib[k], off), yp = __shfl_up(ip[k], off);
      if (lane >= off) { ib[k] += yb; ip[k] += yp; }
    }
  }
  int wb[K], wp[K], cb = 0, cp = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    wb[k] = cb + ib[k] - nb[k];
    wp[k] = cp + ip[k] - np[k];
    cb += __builtin_amdgcn_readlane(ib[k], 63);
    cp += __builtin_amdgcn_readlane(ip[k], 63);
  }
  // row-partitions whose first block lies before block y * total / 8, y = 1..7
  int c[7];
#pragma unroll
  for (int y = 0; y < 7; ++y) {
    const int t = (int)(((long long)cb * (y + 1)) / 8);
    c[y] = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int d = t - wb[k];
      const int m = d <= 0 ? 0 : (d + bpp - 1) / bpp;
      c[y] += m < np[k] ? m : np[k];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int y = 0; y < 7; ++y) c[y] += __shfl_xor(c[y], off);
  const int G8 = gridDim.x, x = blockIdx.x % 8, loc = blockIdx.x / 8;
  const int per_lo = G8 / 8, rem = G8 % 8;
  bool fits = true;
  int r_lo = 0, r_hi = 0, prev = 0;
#pragma unroll
  for (int y = 0; y < 8; ++y) {
    const int r = y == 7 ? cp : __builtin_amdgcn_readfirstlane(c[y]);
    fits = fits && (r - prev) * H <= (per_lo + (y < rem ? 1 : 0)) * waves;
    if (y == x) { r_lo = prev; r_hi = r; }
    prev = r;
  }
  if (!fits) return remapped_coords(a, waves, wave, S);
  UnitCoords u;
  const int unit = r_lo * H + loc * waves + wave;
  const int rp = unit / H;
  u.kvh = unit % H;
  u.s = 0;
  u.part = 0;
  // the row holding row-partition rp
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const uint64_t hit = __ballot(np[k] > 0 && rp >= wp[k] && rp < wp[k] + np[k]);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      u.s = 64 * k + l;
      u.part = rp - __builtin_amdgcn_readlane(wp[k], l);
    }
  }
  u.ok = unit < r_hi * H;
  return u;
}

__device__ __forceinline__ UnitCoords unit_coords(const DecodeArgs& a, int waves, int wave,
                                                  int rows, int block_size) {
  if (a.xcd_remap == 2) return balanced_coords(a, waves, wave, block_size);
  return remapped_coords(a, waves, wave, rows);
}

// ---- flat split (DecodeArgs::flat_min_blocks > 0) -----------------------------------
constexpr int kFlatK = kFlatMaxSeqs / 64;  // sequences per lane in the scans below

// Block counts of sequences 0 .. S-1 as an inclusive prefix sum: cend[k] of lane l holds the
// blocks of sequences 0 .. 64k + l (sequences at or past S count none), shifted left by 5,
// with (n - 1) mod block_size of sequence 64k + l in the low 5 bits (block_size <= 32), so
// that a sequence's length comes back from the scan too (flat_len).  Returns the total T.
__device__ __forceinline__ int flat_scan(const int32_t* ctx, int S, int max_ctx, int block_size,
                                         int lane, int (&cend)[kFlatK]) {
  int nb[kFlatK], rem[kFlatK];
#pragma unroll
  for (int k = 0; k < kFlatK; ++k) {
    const int s = lane + 64 * k;
    int n = s < S ? ctx[s] : 0;
    n = n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
    nb[k] = (n + block_size - 1) / block_size;
    rem[k] = n > 0 ? (n - 1) % block_size : 0;
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < kFlatK; ++k) {
      const int y = __shfl_up(nb[k], off);
      if (lane >= off) nb[k] += y;
    }
  }
  int carry = 0;
#pragma unroll
  for (int k = 0; k < kFlatK; ++k) {
    cend[k] = ((carry + nb[k]) << 5) | rem[k];
    carry += __builtin_amdgcn_readlane(nb[k], 63);
  }
  return carry;
}

// Chunk length for a stream of T blocks, H KV heads and a grid of `waves` wavefronts: with
// R = floor(waves / H) chunks per round, the fewest rounds k for which C = ceil(T / (k R))
// is at most max_chunk, and C no shorter than min_blocks (<= max_chunk).  Then
// ceil(T / C) <= k R chunks: every wavefront walks at most k units.
__device__ __forceinline__ int flat_chunk(int T, int H, int waves, int min_blocks, int max_chunk) {
  const int R = waves / H > 0 ? waves / H : 1;
  const int per = max_chunk * R;  // blocks one round covers at the longest chunk
  int k = T > per ? (T + per - 1) / per : 1;
  while ((T + k * R - 1) / (k * R) > max_chunk) ++k;  // guards the rounding above
  const int C = (T + k * R - 1) / (k * R);
  return C > min_blocks ? C : (min_blocks > 0 ? min_blocks : 1);
}

// Units (chunk, KV head) of this wavefront out of U: XCD x (workgroup i runs on XCD i % 8)
// takes the contiguous share of [0, U) proportional to its wavefronts, and its wavefronts
// take every (wavefronts on x)-th unit of it from their own index on.
__device__ __forceinline__ void flat_units(long long U, int waves, int wave, int* first,
                                           int* step, int* end) {
  const int G8 = gridDim.x, x = blockIdx.x % 8, loc = blockIdx.x / 8;
  const int per = G8 / 8, rem = G8 % 8;
  const long long total = (long long)G8 * waves;
  const long long before = (long long)(x * per + (x < rem ? x : rem)) * waves;
  const int mine = (per + (x < rem ? 1 : 0)) * waves;
  const long long lo = U * before / total, hi = U * (before + mine) / total;
  *first = (int)(lo + (long long)loc * waves + wave);
  *step = mine;
  *end = (int)hi;
}

// The scan's word for sequence s (wave-uniform).
__device__ __forceinline__ int flat_word(const int (&cend)[kFlatK], int s) {
  int v = 0;
#pragma unroll
  for (int k = 0; k < kFlatK; ++k)
    if (s >> 6 == k) v = __builtin_amdgcn_readlane(cend[k], s & 63);
  return v;
}

// Inclusive block end of sequence s (wave-uniform), read from the scan.
__device__ __forceinline__ int flat_end(const int (&cend)[kFlatK], int s) {
  return flat_word(cend, s) >> 5;
}

// The sequence holding stream position p (0 <= p < T): the first whose inclusive end
// exceeds p (the scan does not decrease, and empty sequences end where their predecessor
// does, so they are never chosen).
__device__ __forceinline__ int flat_seq(const int (&cend)[kFlatK], int p) {
  int s = 0;
  bool found = false;
  const int key = (p << 5) | 31;  // word > key  <=>  block end > p
#pragma unroll
  for (int k = 0; k < kFlatK; ++k) {
    const uint64_t m = __ballot(cend[k] > key);
    if (!found && m) {
      s = 64 * k + __builtin_ctzll(m);
      found = true;
    }
  }
  return s;
}

// One segment of the flat walk: blocks [j0, j1) of sequence s (n tokens, clamped) for KV
// head kvh, ending in partial slot `slot` of the sequence's rows.
struct FlatSeg {
  int s, n, kvh, j0, j1, slot;
};

// The flat walk of one wavefront: its units (chunk, KV head) in turn (flat_units), each
// as one segment per sequence it touches.  init() runs the scan and stores the chunk
// length (and the grid's wavefronts) for the merge; next() yields the segments in order.
struct FlatWalk {
  int cend[kFlatK];
  int T, C, H, unit, ustep, uend, pos, pend, chunk, ukvh;

  int B;

  __device__ __forceinline__ void init(const DecodeArgs& a, int block_size, int waves, int wave,
                                       int lane, int max_chunk) {
    B = block_size;
    T = flat_scan(a.ctx, a.num_seqs, a.max_ctx, block_size, lane, cend);
    H = a.num_kv_heads;
    C = flat_chunk(T, H, gridDim.x * waves, a.flat_min_blocks, max_chunk);
    flat_units((long long)((T + C - 1) / C) * H, waves, wave, &unit, &ustep, &uend);
    pos = pend = chunk = ukvh = 0;
    if (blockIdx.x == 0 && wave == 0 && lane == 0) {  // for the merge, and for the record
      a.flat_meta[0] = C;
      a.flat_meta[1] = (int)gridDim.x * waves;
    }
  }

  __device__ __forceinline__ bool next(FlatSeg& g) {
    if (pos >= pend) {  // next unit
      if (unit >= uend) return false;
      chunk = unit / H;
      ukvh = unit % H;
      pos = chunk * C;
      pend = min(pos + C, T);
      unit += ustep;
    }
    // (all wave-uniform: read into scalar registers, so what they index is loaded with
    // scalar loads)
    g.s = __builtin_amdgcn_readfirstlane(flat_seq(cend, pos));
    const int cum = g.s > 0 ? flat_end(cend, g.s - 1) : 0;
    const int w = flat_word(cend, g.s);
    g.n = __builtin_amdgcn_readfirstlane(((w >> 5) - cum - 1) * B + (w & 31) + 1);
    g.kvh = __builtin_amdgcn_readfirstlane(ukvh);
    g.j0 = __builtin_amdgcn_readfirstlane(pos - cum);
    g.j1 = __builtin_amdgcn_readfirstlane(min(pend, w >> 5) - cum);
    g.slot = __builtin_amdgcn_readfirstlane(chunk - cum / C);
    pos = cum + g.j1;
    return true;
  }
};

// Blocks per unit of a row whose units walk blocks [jb, nblk): the fixed partition, or
// under a balanced split an equal share of them, at least part_min_blocks.
__device__ __forceinline__ int part_share_blocks(const DecodeArgs& a, int jb, int nblk) {
  if (a.part_min_blocks <= 0) return a.blocks_per_part;
  const int share = (nblk - jb + a.num_parts - 1) / a.num_parts;
  return share > a.part_min_blocks ? share : a.part_min_blocks;
}

// Tokens of its group's shared prefix that a sequence of length n attends (cascade modes):
// the group's shared blocks, clamped to [0, max_prefix_blocks], in tokens, capped at n.
__device__ __forceinline__ int prefix_tokens(const DecodeArgs& a, int group, int block_size, int n) {
  if (a.max_prefix_blocks <= 0) return 0;  // prefix_blocks may then be null
  int pb = a.prefix_blocks[group];
  pb = pb < 0 ? 0 : (pb > a.max_prefix_blocks ? a.max_prefix_blocks : pb);
  const int t = pb * block_size;
  return t < n ? t : n;
}

}  // namespace pa
