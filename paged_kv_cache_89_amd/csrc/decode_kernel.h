// Paged decode attention for gfx950: one wavefront per work unit (sequence, KV head,
// context partition), single pass over K and V with online softmax.
//
// What is computed ([P1] = "PagedAttention: Mathematical Foundations, Virtual Memory Block
// Allocation, and Zero-Waste KV Cache Serving"):
//   sec. 3, eq. for a_ij / o_i and the block-wise forms S_ij, A_ij: the output is the
//   softmax-weighted sum of the value rows over the sequence's first n tokens, scored by
//   scale * q.k; the last block may be partial and its empty slots do not count;
//   sec. 7 pseudocode: blocks are visited through the block table one at a time, the
//   running maximum / denominator / output are rescaled by exp(old max - new max).
// The partition split and its merge are this library's addition (the same rescaling
// applied across partitions); see merge.hip.
//
// How it maps to CDNA4:
//   * a (block, KV head) tile is B x D contiguous elements (cache layout
//     [NB][Hkv][B][D]); one wave load instruction covers 1 KiB (16 B per lane, or 512 B at
//     8 B per lane for tiles smaller than 1 KiB) of the tile, so every load is a fully
//     coalesced run of consecutive bytes;
//   * with that mapping LPT = D / (elements per lane) consecutive lanes hold one token row
//     and a load covers TPL = 64 / LPT token rows; the q.k partial sums of a token are
//     combined with DPP quad-permute / mirror moves inside the lane group, never through
//     LDS;
//   * each lane group (one "row" of the wave) keeps its own running max, denominator and
//     output slice for the tokens it holds, so the per-block softmax update needs no
//     cross-group traffic at all; the TPL group states are merged once per unit with
//     the same rescaling rule;
//   * the lane holds exactly the K/V elements its arithmetic needs, so tiles go straight
//     from HBM into registers (no LDS round trip); the next block's K and V loads are
//     issued before the current block is consumed (register double buffering), and the
//     unit's slice of the block table (at most 64 entries) sits in one VGPR, read with
//     v_readlane into scalar registers so the address of the next tile never waits on
//     memory;
//   * GQA (G query heads per KV head) reuses each loaded tile for all G heads;
//   * e4m3 tiles are decoded in registers by the hardware fp8 converters: K codes to the
//     query's 16-bit type (exact), contracted with the same dot2 as a 16-bit cache, V
//     codes to fp32; k_scale is folded into the logit scale and v_scale into the epilogue.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "launch.h"

// Compile-time tuning knobs (defaults are the measured best on MI355X).
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4        // wavefronts (independent work units) per workgroup
#endif

namespace pa {

template <int D, int BS, int KVK>
struct TileGeometry {
  static constexpr int E = (KVK == KIND_E4M3) ? 1 : 2;   // bytes per element
  static constexpr int TILE = BS * D * E;                // bytes of one (block, KV head) tile
  static constexpr int LB = TILE >= 1024 ? 16 : 8;       // bytes per lane per load
  static constexpr int W = LB / 4;                       // dwords per lane per load
  static constexpr int EPL = LB / E;                     // elements per lane per load
  static constexpr int LPT = D / EPL;                    // lanes sharing a token row
  static constexpr int TPL = 64 / LPT;                   // token rows per load
  static constexpr int NLD = BS / TPL;                   // loads per tile
  static constexpr int SPAN = 64 * LB;                   // bytes per wave load
  static_assert(NLD * SPAN == TILE, "tile must be covered by whole wave loads");
  static_assert(LPT >= 2 && LPT <= 16, "token row must fit in a 16-lane DPP row");
};

template <int W> struct LoadVec;
template <> struct LoadVec<4> { using T = u32x4; };
template <> struct LoadVec<2> { using T = u32x2; };


// NT: K/V loads carry the non-temporal hint (data read once per step).  APP: the appending
// decode, FLAT: the flat split (separate instantiations, so the plain decode over fixed
// partitions carries none of their registers).
// The kernel body, also run by the one-launch cascade (decode_cascade.hip).
template <int D, int BS, int QK, int KVK, int G, bool NT, bool APP, bool FLAT>
__device__ __forceinline__ void decode_body(const DecodeArgs& a) {
  using Geo = TileGeometry<D, BS, KVK>;
  using LT = typename LoadVec<Geo::W>::T;
  constexpr int W = Geo::W, EPL = Geo::EPL, LPT = Geo::LPT, TPL = Geo::TPL, NLD = Geo::NLD;
  constexpr bool F8 = (KVK == KIND_E4M3);
  static_assert(F8 || QK == KVK, "fp16/bf16 caches are read with a query of the same type");
  // Partials leave with the non-temporal hint for 32-token blocks (measured on the
  // long-context workload, 512-token partitions: decode 632.7 vs 650.8 us, merge 10.4 vs
  // 8.7 us); 16-token blocks keep ordinary stores (the OPT-13B layer and the fp8
  // shared-prompt per-sequence units ran 0.1 % and 2.2 % slower with the hint).
  constexpr bool NT_PARTIALS = BS >= 32;
  typedef float f32x4v __attribute__((ext_vector_type(4)));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPT;   // token row of this lane inside a load
  const int c = lane % LPT;   // element slice [c*EPL, c*EPL + EPL) of the head dimension
  // the query slices of the G heads that share KV head kvh, as loaded
  auto load_query = [&](int s_, int kvh_, u32x4 (&qr)[G][EPL / 8]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const u32x4* qp = (const u32x4*)((const uint16_t*)a.q +
                                       ((size_t)s_ * a.num_heads + kvh_ * G + g) * D + c * EPL);
#pragma unroll
      for (int k = 0; k < EPL / 8; ++k) qr[g][k] = qp[k];
    }
  };

  const size_t blk_stride = (size_t)a.num_kv_heads * Geo::TILE;
  const uint32_t loff = (uint32_t)lane * Geo::LB;
  // block `phys` of KV head kvh_ into (kr, vr)
  auto issue_at = [&](int phys, int kvh_, LT (&kr)[NLD], LT (&vr)[NLD]) {
    const char* kp = (const char*)a.k + (size_t)kvh_ * Geo::TILE + loff;
    const char* vp = (const char*)a.v + (size_t)kvh_ * Geo::TILE + loff;
    const size_t off = (size_t)phys * blk_stride;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      if constexpr (NT) kr[i] = __builtin_nontemporal_load((const LT*)(kp + off + i * Geo::SPAN));
      else kr[i] = *(const LT*)(kp + off + i * Geo::SPAN);
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      if constexpr (NT) vr[i] = __builtin_nontemporal_load((const LT*)(vp + off + i * Geo::SPAN));
      else vr[i] = *(const LT*)(vp + off + i * Geo::SPAN);
    }
  };

  // Work: the one unit of unit_coords, or under the flat split this wavefront's walk.  The
  // walk loads the next segment's set-up (table slice, query) while the current
  // segment streams, right behind the current segment's first block, so a segment starts
  // by requesting its first block.
  constexpr bool flat = FLAT;
  FlatWalk walk;
  FlatSeg nx{0, 0, 0, 0, 0, 0};
  bool nx_ok = false;
  using Slice = std::conditional_t<FLAT, TableSliceN<kFlatMaxChunkVector / 64>, TableSlice>;
  Slice nx_ts;
  u32x4 nx_q[G][EPL / 8];
  auto prefetch = [&]() {
    nx_ok = walk.next(nx);
    if (!nx_ok) return;
    nx_ts.init(a.tables + (size_t)nx.s * a.max_blocks, nx.j0, nx.j1, a.num_blocks, lane);
    load_query(nx.s, nx.kvh, nx_q);
  };
  // Partial stores: a row's accumulator and its (m, L) (lane 0).  A unit's row: after the
  // end-of-unit reduce-scatter every lane holds NV consecutive elements of the row, from
  // element rs_first of its slice c on, so the row leaves in one store instruction of the
  // whole wave.  A flat-walk segment's row: slice c of lanes < LPT (the walk keeps the
  // full lane-group merge: the reduce-scatter's lane selects would cost those kernels an
  // occupancy step, measured in VGPRs).
  constexpr int NV = EPL * LPT / 64;
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  auto store_slice = [&](size_t pi, const float (&v)[EPL]) {
    float* pa_ = a.part_acc + pi * D + c * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const f32x4v t = f32x4v{v[e], v[e + 1], v[e + 2], v[e + 3]};
      if constexpr (NT_PARTIALS) __builtin_nontemporal_store(t, (f32x4v*)(pa_ + e));
      else *(f32x4v*)(pa_ + e) = t;
    }
  };
  auto store_acc = [&](size_t pi, const float (&v)[NV]) {
    float* pa_ = a.part_acc + pi * D + c * EPL + rs_first<LPT, EPL>(lane);
    if constexpr (NV == 2) {
      if constexpr (NT_PARTIALS) __builtin_nontemporal_store(f32x2v{v[0], v[1]}, (f32x2v*)pa_);
      else *(f32x2v*)pa_ = f32x2v{v[0], v[1]};
    } else {
      static_assert(NV == 1, "elements per lane");
      if constexpr (NT_PARTIALS) __builtin_nontemporal_store(v[0], pa_);
      else *pa_ = v[0];
    }
  };
  auto store_ml = [&](size_t pi, float M_, float L_) {
    if constexpr (NT_PARTIALS) {
      __builtin_nontemporal_store(M_, &a.part_ml[pi * 2]);
      __builtin_nontemporal_store(L_, &a.part_ml[pi * 2 + 1]);
    } else {
      a.part_ml[pi * 2] = M_;
      a.part_ml[pi * 2 + 1] = L_;
    }
  };
  // The flat walk's partials leave one segment late: a segment's wait in LDS (never in
  // registers, which would cost occupancy) and go out at the next segment's end or after
  // the walk.  A wave's next wait on its loads also waits for every store it issued
  // before them, and stores issued among a full-rate read stream are slow to complete.
  [[maybe_unused]] bool pd_ok = false;
  [[maybe_unused]] int pd_s = 0, pd_h0 = 0, pd_slot = 0;
  __shared__ __attribute__((aligned(16))) float pend_acc[PA_DECODE_WAVES][FLAT ? G * D : 4];
  __shared__ float pend_ml[PA_DECODE_WAVES][FLAT ? 2 * G : 2];
  [[maybe_unused]] auto flush_pending = [&]() {
    if (!pd_ok) return;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const size_t pi = ((size_t)pd_s * a.num_heads + pd_h0 + g) * a.num_slots + pd_slot;
      if (lane < LPT) {
        float v[EPL];
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
          const f32x4v t = *(const f32x4v*)&pend_acc[wave][g * D + c * EPL + e];
          v[e] = t[0];
          v[e + 1] = t[1];
          v[e + 2] = t[2];
          v[e + 3] = t[3];
        }
        store_slice(pi, v);
      }
      if (lane == 0) store_ml(pi, pend_ml[wave][2 * g], pend_ml[wave][2 * g + 1]);
    }
    pd_ok = false;
  };
  // the pipeline's first register set: under the flat split it can already hold the next
  // segment's first block, requested before the last segment's epilogue
  LT ka[NLD], va[NLD];
  bool pre_issued = false;
  UnitCoords uc{0, 0, 0, true};
  if constexpr (flat) {
    walk.init(a, BS, PA_DECODE_WAVES, wave, lane, kFlatMaxChunkVector);
    prefetch();
  } else {
    uc = unit_coords(a, PA_DECODE_WAVES, wave, a.num_seqs, BS);
    if (!uc.ok) return;
  }
  // (one pass over the unit without the flat split: the trip count stays in the loop
  // condition, where the compiler sees it)
  for (int iter = 0; flat || iter < 1; ++iter) {
    int s, kvh, j0, j1, slot, n;
    Slice ts;
    u32x4 qraw[G][EPL / 8];
    if constexpr (flat) {
      if (!nx_ok) break;
      s = nx.s;
      kvh = nx.kvh;
      j0 = nx.j0;
      j1 = nx.j1;
      slot = nx.slot;
      n = nx.n;
      ts = nx_ts;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < EPL / 8; ++k) qraw[g][k] = nx_q[g][k];
    } else {
      s = uc.s;
      kvh = uc.kvh;
      slot = a.slot_base + uc.part;
      n = a.ctx[s];
    }
    n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
    const int h0 = kvh * G;
    const int nblk = (n + BS - 1) / BS;
    if constexpr (!flat) {
      // suffix of a shared-prefix group: start after the blocks the prefix units cover
      const int jb = (a.mode == MODE_SUFFIX)
                         ? (prefix_tokens(a, s / a.seq_group, BS, n) + BS - 1) / BS : 0;
      const int bpp = part_share_blocks(a, jb, nblk);
      j0 = jb + uc.part * bpp;
      j1 = min(nblk, j0 + bpp);
    }

    if (j0 >= j1) {
      // Nothing to read.  Direct output: this is the n == 0 row, write zeros.  Cascade
      // partials: mark the slot empty (the merge skips it).
      if (a.num_slots == 0 && lane < LPT) {
        for (int g = 0; g < G; ++g) {
          uint16_t* o = (uint16_t*)a.out + ((size_t)s * a.num_heads + h0 + g) * D + c * EPL;
          for (int e = 0; e < EPL; ++e) o[e] = 0;
        }
      } else if (a.mode != MODE_PLAIN && lane < G) {
        const size_t pi = ((size_t)s * a.num_heads + h0 + lane) * a.num_slots + slot;
        a.part_ml[pi * 2] = -INFINITY;
        a.part_ml[pi * 2 + 1] = 0.f;
      }
      continue;
    }

    // The segment's first block goes out before anything else it needs (unless the walk
    // requested it before the last segment's epilogue); then the next segment's set-up.
    if constexpr (!flat) ts.init(a.tables + (size_t)s * a.max_blocks, j0, j1, a.num_blocks, lane);
    if (!pre_issued) issue_at(ts.get(j0), kvh, ka, va);
    pre_issued = false;
    if constexpr (flat) prefetch();

    // ---- query slice, kept packed (fp16/bf16 caches) or widened to fp32 (e4m3 caches)
    if constexpr (!flat) load_query(s, kvh, qraw);
    uint32_t qw[G][EPL / 2];
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int k = 0; k < EPL / 8; ++k) {
        const u32x4 t = qraw[g][k];
#pragma unroll
        for (int w = 0; w < 4; ++w) qw[g][4 * k + w] = t[w];
      }
    }

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }

    const float qk_scale = a.qk_scale;
    auto issue = [&](int phys, LT (&kr)[NLD], LT (&vr)[NLD]) { issue_at(phys, kvh, kr, vr); };

    // Fold one block into the running state.  MASK: the block holds slots >= n.
    auto consume = [&](auto mask_tag, int j, const LT (&kr)[NLD], const LT (&vr)[NLD]) {
      constexpr bool MASK = decltype(mask_tag)::value;
      float sc[G][NLD];
      // q.k partial sums over this lane's slice
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        if constexpr (F8) {
          // the codes widened to the query's 16-bit type (exact: every E4M3 value is an
          // fp16 and a bf16 value), then the dot2 of a 16-bit cache
          uint32_t kh[EPL / 2];
#pragma unroll
          for (int w = 0; w < W; ++w) {
            const u32x2 t = e4m3x4_to_16<QK>(kr[i][w]);
            kh[2 * w] = t[0];
            kh[2 * w + 1] = t[1];
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float d0 = 0.f, d1 = 0.f;
#pragma unroll
            for (int w = 0; w < EPL / 2; w += 2) {
              d0 = dot2_16<QK>(qw[g][w], kh[w], d0);
              d1 = dot2_16<QK>(qw[g][w + 1], kh[w + 1], d1);
            }
            sc[g][i] = d0 + d1;
          }
        } else {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float d = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) d = dot2_16<KVK>(qw[g][w], (uint32_t)kr[i][w], d);
            sc[g][i] = d;
          }
        }
      }
      // finish the dot products inside each token's lane group; scale into log2 units
      bool valid[NLD];
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        valid[i] = !MASK || (j * BS + i * TPL + r < n);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float z = group_sum<LPT>(sc[g][i]) * qk_scale;
          sc[g][i] = valid[i] ? z : -INFINITY;
        }
      }
      // online softmax update per head
      float p[G][NLD];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float bm = sc[g][0];
#pragma unroll
        for (int i = 1; i < NLD; ++i) bm = fmaxf(bm, sc[g][i]);
        const float mn = fmaxf(m[g], bm);
        const float ms = (mn == -INFINITY) ? 0.f : mn;  // row has seen no valid token yet
        const float rs = fast_exp2(m[g] - ms);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          p[g][i] = fast_exp2(sc[g][i] - ms);
          ps += p[g][i];
        }
        l[g] = l[g] * rs + ps;
        m[g] = mn;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= rs;
      }
      // weighted value rows
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        float vf[EPL];
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const uint32_t x = vr[i][w];
          if constexpr (F8) {
            e4m3x4_to_f32(x, &vf[4 * w]);
          } else if constexpr (KVK == KIND_BF16) {
            vf[2 * w] = bf16_lo(x);
            vf[2 * w + 1] = bf16_hi(x);
          } else {
            vf[2 * w] = f16_lo(x);
            vf[2 * w + 1] = f16_hi(x);
          }
        }
        if constexpr (MASK) {
          // never let an unused slot's bytes (possibly NaN) reach the FMA: 0 * NaN = NaN
#pragma unroll
          for (int e = 0; e < EPL; ++e) vf[e] = valid[i] ? vf[e] : 0.f;
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p[g][i], vf[e], acc[g][e]);
      }
    };

    // Appending decode (the unit that walks the sequence's last block, whose table entry lies
    // in the pool -- an entry outside it skips the write, as the KV write does): the new
    // token's rows take slot tn of block jn in place of the loaded bytes, and are stored into
    // the cache after the unit's epilogue, so no load waits for the store.  Lanes of token
    // row tn % TPL hold its slice c in load tn / TPL, in the cache's type (e4m3: the code of
    // x * inv_scale, the conversion the KV write uses).
    // (The rows are loaded whatever the table entry says; whether the entry lies in the pool
    // is read from the unit's table slice once it is there, so nothing waits for it here.)
    const int jn = (n - 1) / BS, tn = (n - 1) % BS;
    bool app = APP && a.mode == MODE_PLAIN && n > 0 && j1 == nblk;
    int app_phys = 0;
    LT nk{}, nv{};
    if (app) {
      const size_t src = ((size_t)s * a.num_kv_heads + kvh) * D + (size_t)c * EPL;
      const uint16_t* ks = (const uint16_t*)a.k_new + src;
      const uint16_t* vs = (const uint16_t*)a.v_new + src;
      if constexpr (F8) {
        if constexpr (W == 4) {  // 16 codes from 16 source elements
          const u32x2 k0 = src8_to_e4m3<QK>(((const u32x4*)ks)[0], a.k_inv_scale);
          const u32x2 k1 = src8_to_e4m3<QK>(((const u32x4*)ks)[1], a.k_inv_scale);
          const u32x2 v0 = src8_to_e4m3<QK>(((const u32x4*)vs)[0], a.v_inv_scale);
          const u32x2 v1 = src8_to_e4m3<QK>(((const u32x4*)vs)[1], a.v_inv_scale);
          nk = LT{k0[0], k0[1], k1[0], k1[1]};
          nv = LT{v0[0], v0[1], v1[0], v1[1]};
        } else {  // 8 codes from 8 source elements
          nk = src8_to_e4m3<QK>(*(const u32x4*)ks, a.k_inv_scale);
          nv = src8_to_e4m3<QK>(*(const u32x4*)vs, a.v_inv_scale);
        }
      } else {
        nk = *(const LT*)ks;
        nv = *(const LT*)vs;
      }
    }

    auto process = [&](int j, LT (&kr)[NLD], LT (&vr)[NLD]) {
      if (app && j == jn && r == tn % TPL) {
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          if (i == tn / TPL) {
            kr[i] = nk;
            vr[i] = nv;
          }
      }
      if ((j + 1) * BS <= n) consume(std::false_type{}, j, kr, vr);
      else consume(std::true_type{}, j, kr, vr);
    };

    // Software pipeline: the K/V loads of block j+1 are issued before block j is consumed
    // (two register sets).  The steady-state loop always has a next block to request, so every
    // load in it is unconditional and the compiler's in-order load counter waits for exactly
    // the block being consumed; the last one or two blocks are peeled off the loop.
    if (app) {
      app_phys = ts.raw(jn);
      app = (unsigned)app_phys < (unsigned)a.num_blocks;
    }
    LT kb[NLD], vb[NLD];
    int j = j0;
    while (j + 2 < j1) {
      issue(ts.get(j + 1), kb, vb);
      process(j, ka, va);
      issue(ts.get(j + 2), ka, va);
      process(j + 1, kb, vb);
      j += 2;
    }
    if (j + 1 < j1) {
      issue(ts.get(j + 1), kb, vb);
      process(j, ka, va);
      process(j + 1, kb, vb);
    } else {
      process(j, ka, va);
    }
    // flat walk: the next segment's first block goes out before this segment's epilogue
    // (its table slice is already here)
    if constexpr (flat) {
      if (nx_ok) {
        issue_at(nx_ts.get(nx.j0), nx.kvh, ka, va);
        pre_issued = true;
      }
    }

    if constexpr (flat) flush_pending();
    // ---- merge the TPL lane-group states of the wave (same rescaling rule)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float M = across_lanes<LPT>(m[g], MaxOp{});
      const float f = (m[g] == -INFINITY) ? 0.f : fast_exp2(m[g] - M);
      float L = l[g] * f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= f;
      L = across_lanes<LPT>(L, AddOp{});
      const int h = h0 + g;
      if constexpr (flat) {
        // this segment's partials wait in LDS until the next segment ends (the previous
        // segment's went out at the top of this epilogue); the walk always has slots
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = across_lanes<LPT>(acc[g][e], AddOp{});
        if (lane < LPT) {
#pragma unroll
          for (int e = 0; e < EPL; e += 4)
            *(f32x4v*)&pend_acc[wave][g * D + c * EPL + e] =
                f32x4v{acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]};
        }
        if (lane == 0) {
          pend_ml[wave][2 * g] = M;
          pend_ml[wave][2 * g + 1] = L;
        }
        continue;
      }
      reduce_scatter<LPT>(acc[g], lane);  // acc[g][0 .. NV): elements fst.. of slice c
      const int fst = rs_first<LPT, EPL>(lane);
      float ov[NV];
#pragma unroll
      for (int e = 0; e < NV; ++e) ov[e] = acc[g][e];
      if (a.num_slots == 0) {
        uint16_t* op = (uint16_t*)a.out + ((size_t)s * a.num_heads + h) * D + c * EPL + fst;
        uint16_t ob[NV];
#pragma unroll
        for (int e = 0; e < NV; ++e) {
          float o = ov[e] / L;
          if constexpr (F8) o = o * a.v_scale;
          ob[e] = f32_to_store<QK>(o);
        }
        if constexpr (NV == 2) *(uint32_t*)op = (uint32_t)ob[0] | ((uint32_t)ob[1] << 16);
        else *op = ob[0];
      } else {
        const size_t pi = ((size_t)s * a.num_heads + h) * a.num_slots + slot;
        store_acc(pi, ov);
        if (lane == 0) store_ml(pi, M, L);
      }
    }
    if constexpr (flat) {
      pd_ok = a.num_slots > 0;
      pd_s = s;
      pd_h0 = h0;
      pd_slot = slot;
    }
    // appending decode: the new rows into the cache, after everything that read the block
    if (app && r == tn % TPL) {
      const size_t dst = (((size_t)app_phys * a.num_kv_heads + kvh) * BS + tn) * (Geo::TILE / BS) +
                         (size_t)c * Geo::LB;
      *(LT*)((char*)a.k + dst) = nk;
      *(LT*)((char*)a.v + dst) = nv;
    }
  }
  if constexpr (flat) flush_pending();
}

template <int D, int BS, int QK, int KVK, int G, bool NT, bool APP, bool FLAT>
__global__ __launch_bounds__(64 * PA_DECODE_WAVES) void paged_decode_kernel(const DecodeArgs a) {
  decode_body<D, BS, QK, KVK, G, NT, APP, FLAT>(a);
}

template <int D, int BS, int QK, int KVK, int G, bool NT>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const dim3 block(64 * PA_DECODE_WAVES);
  if (a.flat_min_blocks > 0) {
    // the flat split: 16-bit caches only (the host never asks it for e4m3 caches)
    if constexpr (KVK == KIND_E4M3) {
      return hipErrorInvalidValue;
    } else {
      // The grid (and so the chunk length the walk derives from it) is the plain decode's
      // for the appending one too, so both split the stream alike and give the same bits.
      static std::atomic<int> resident[kMaxCachedDevices];
      const dim3 grid = decode_grid(
          a, PA_DECODE_WAVES, (const void*)paged_decode_kernel<D, BS, QK, KVK, G, NT, false, true>,
          resident);
      if (a.append)
        hipLaunchKernelGGL((paged_decode_kernel<D, BS, QK, KVK, G, NT, true, true>), grid, block,
                           0, stream, a);
      else
        hipLaunchKernelGGL((paged_decode_kernel<D, BS, QK, KVK, G, NT, false, true>), grid, block,
                           0, stream, a);
      return hipGetLastError();
    }
  }
  if (a.append)
    hipLaunchKernelGGL((paged_decode_kernel<D, BS, QK, KVK, G, NT, true, false>),
                       decode_grid(a, PA_DECODE_WAVES), block, 0, stream, a);
  else
    hipLaunchKernelGGL((paged_decode_kernel<D, BS, QK, KVK, G, NT, false, false>),
                       decode_grid(a, PA_DECODE_WAVES), block, 0, stream, a);
  return hipGetLastError();
}

// Instantiate every (block size, dtype pair, group) for one head_dim and load policy.
template <int D, bool NT>
hipError_t launch_decode_d(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
#define PA_G(BS, QK, KVK)                                                  \
  switch (s.group) {                                                       \
    case 1: return launch_decode_t<D, BS, QK, KVK, 1, NT>(a, stream);      \
    case 2: return launch_decode_t<D, BS, QK, KVK, 2, NT>(a, stream);      \
    case 4: return launch_decode_t<D, BS, QK, KVK, 4, NT>(a, stream);      \
    case 8: return launch_decode_t<D, BS, QK, KVK, 8, NT>(a, stream);      \
    default: return hipErrorInvalidValue;                                  \
  }
#define PA_DT(BS)                                                                     \
  if (s.q_kind == KIND_F16 && s.kv_kind == KIND_F16) { PA_G(BS, KIND_F16, KIND_F16) } \
  if (s.q_kind == KIND_BF16 && s.kv_kind == KIND_BF16) { PA_G(BS, KIND_BF16, KIND_BF16) } \
  if (s.q_kind == KIND_F16 && s.kv_kind == KIND_E4M3) { PA_G(BS, KIND_F16, KIND_E4M3) } \
  if (s.q_kind == KIND_BF16 && s.kv_kind == KIND_E4M3) { PA_G(BS, KIND_BF16, KIND_E4M3) } \
  return hipErrorInvalidValue;
  // 16-token blocks with G >= 2 always run on the matrix-core kernel: only G = 1 here.
#define PA_G1(BS, QK, KVK) \
  if (s.group == 1) return launch_decode_t<D, BS, QK, KVK, 1, NT>(a, stream); \
  return hipErrorInvalidValue;
#define PA_DT16                                                                            \
  if (s.q_kind == KIND_F16 && s.kv_kind == KIND_F16) { PA_G1(16, KIND_F16, KIND_F16) }     \
  if (s.q_kind == KIND_BF16 && s.kv_kind == KIND_BF16) { PA_G1(16, KIND_BF16, KIND_BF16) } \
  if (s.q_kind == KIND_F16 && s.kv_kind == KIND_E4M3) { PA_G1(16, KIND_F16, KIND_E4M3) }   \
  if (s.q_kind == KIND_BF16 && s.kv_kind == KIND_E4M3) { PA_G1(16, KIND_BF16, KIND_E4M3) } \
  return hipErrorInvalidValue;
  switch (s.block_size) {
    case 8: { PA_DT(8) }
    case 16: { PA_DT16 }
    case 32: { PA_DT(32) }
    default: return hipErrorInvalidValue;
  }
#undef PA_DT16
#undef PA_G1
#undef PA_DT
#undef PA_G
}

}  // namespace pa
