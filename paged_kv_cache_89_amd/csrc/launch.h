// Internal interface between the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace pa {

// Storage kinds used as template parameters.
enum Kind : int { KIND_F16 = 0, KIND_BF16 = 1, KIND_E4M3 = 2 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxUnitBlocks = 64;  // blocks one work unit (wavefront) walks at most
constexpr int kBalancedMaxSeqs = 128;  // rows the work-balanced XCD ranges handle (xcd_remap 2)
constexpr int kFlatMaxSeqs = 256;      // sequences the flat split handles (flat_min_blocks > 0)
// blocks of a flat-split chunk at most: the vector kernel's table slice takes two VGPRs, the
// matrix-core kernel's four (it is held to two waves per SIMD by its LDS, not its registers)
constexpr int kFlatMaxChunkVector = 128;
constexpr int kFlatMaxChunkMatrix = 256;

// Decode over work units (sequence, KV head, partition).  A unit walks blocks
// [part * blocks_per_part, min(ceil(n / B), (part + 1) * blocks_per_part)) of its
// sequence for the num_heads / num_kv_heads query heads that share the KV head.
//
// Shared-prefix (cascade) modes: the batch is cut into groups of seq_group consecutive
// sequences whose first prefix_blocks[g] table entries are the same physical blocks.
//   MODE_PREFIX: units are (group, KV head, partition) over the group's shared prefix; the
//     unit's query heads are the G heads of every member (seq_group * G of them), and head
//     c of member k sees min(prefix tokens, n_k) of those tokens.
//   MODE_SUFFIX: units are (sequence, KV head, partition) over the tokens after the
//     sequence's shared prefix; the walk starts at block ceil(min(prefix tokens, n) / B).
// In both modes every unit writes its (m, l, acc) partial, empty or not, into slot
// slot_base + part of the num_slots slots of each of its rows.
//
// Flat split (flat_min_blocks > 0; plain and multi-token decodes of at most kFlatMaxSeqs
// sequences): instead of fixed partitions per sequence, the blocks of all sequences,
// sequence after sequence, form one stream of T blocks cut into chunks of C blocks, and a
// unit is (chunk, KV head), so every unit reads the same number of blocks however the
// lengths fall.  A chunk that runs from one sequence into the next is walked as one segment
// per sequence, each ending in a partial of its own: the segment of sequence s that starts
// at stream position p fills slot floor(p / C) - floor(cum_s / C) of the sequence's rows
// (cum_s: blocks of the sequences before s), so the slots of a sequence are consecutive
// from 0.  The grid holds exactly the wavefronts that run at once (W); with T known, C is
// the shortest chunk for which k rounds of W units cover the stream, k the fewest rounds
// that keep C within the kernel's table slice (kFlatMaxChunk*), and C >= flat_min_blocks
// (flat_chunk).  The decode stores
// C at flat_meta[0] for the merge, which finds each row's slot count from the same scan,
// and W at flat_meta[1].
//
// MODE_MULTI: query_len tokens per sequence (q and out are [S, query_len, Hq, D]); a
// unit's query heads are its KV head's G heads for every query token, and query token
// t sees the positions before n - query_len plus the draft positions n - query_len + u
// whose bit u is set in tree_masks[s][t] (causal, bits 0..t, when tree_masks is null).
enum DecodeMode : int32_t { MODE_PLAIN = 0, MODE_PREFIX = 1, MODE_SUFFIX = 2, MODE_MULTI = 3 };

struct DecodeArgs {
  void* out;                 // [S, Hq, D] q dtype (written when num_slots == 0)
  const void* q;             // [S, Hq, D]
  const void* k;             // [NB, Hkv, B, D]
  const void* v;
  const int32_t* tables;     // [S, MB]
  const int32_t* ctx;        // [S]
  float* part_acc;           // [S, Hq, num_slots, D]   (num_slots > 0)
  float* part_ml;            // [S, Hq, num_slots, 2]   running max (log2 units) and sum
  int32_t num_seqs, num_heads, num_kv_heads, max_blocks, num_blocks, max_ctx;
  int32_t num_parts, blocks_per_part, num_units;
  // > 0: balanced split instead -- each of the num_parts units of a row takes an equal
  // share of the row's blocks [jb, ceil(n / B)), at least part_min_blocks of them
  // (part_share_blocks); the host keeps num_parts * 64 >= ceil(max_ctx / B)
  int32_t part_min_blocks = 0;
  int32_t num_slots, slot_base;  // partial slots per row (0: write the output directly)
  float qk_scale;            // scale * log2(e) * k_scale
  float v_scale;
  int32_t seq_fastest;       // unit order: 0 = (seq, part, kv head), 1 = (part, kv head, seq)
  int32_t xcd_remap;         // 1 = each XCD runs a contiguous range of workgroups; 2 = of
                             // row-partitions, balanced by blocks (balanced_coords)
  int32_t mode;              // DecodeMode
  int32_t seq_group, num_groups, max_prefix_blocks;
  const int32_t* prefix_blocks;  // [num_groups] shared leading blocks of each group
  int32_t query_len;             // MODE_MULTI: query tokens per sequence
  const uint32_t* tree_masks;    // MODE_MULTI: [S, query_len] or null (causal)
  // Appending decode (MODE_PLAIN only): the new token of sequence s sits at position n - 1
  // of its (clamped) length n; its K/V rows are k_new / v_new [S, Hkv, D] in the query's
  // type.  The unit that walks the sequence's last block stores them into the cache
  // (e4m3 caches: code of x * inv_scale) and uses them in place of what it loaded.
  int32_t append = 0;
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  float k_inv_scale = 1.f, v_inv_scale = 1.f;
  // flat split (see above): shortest chunk in blocks (0: fixed partitions), and where the
  // decode leaves the chunk length it chose
  int32_t flat_min_blocks = 0;
  int32_t* flat_meta = nullptr;
  // Fixed partitions inside a larger grid (the one-launch cascade): this part's workgroups
  // are [wg_base, wg_base + wg_count) of the grid; wg_base is a multiple of 8, so each keeps
  // its XCD (0 / 0: the whole grid)
  int32_t wg_base = 0, wg_count = 0;
};

struct DecodeShape {
  int head_dim, block_size, q_kind, kv_kind, group;
  bool nontemporal;          // K/V loads with the non-temporal hint
};

// Workgroups of `kernel` (`threads` each) that fit on the current device at once:
// occupancy per compute unit times the compute units, looked up once per device and kept
// in `cache` (kMaxCachedDevices entries, zero-initialised).
constexpr int kMaxCachedDevices = 64;
int resident_workgroups(const void* kernel, int threads, std::atomic<int>* cache);

// Grid of a decode launch with `waves` units per workgroup; the flat split takes the
// workgroups that fit at once (`cache` as above).
inline dim3 decode_grid(const DecodeArgs& a, int waves, const void* kernel = nullptr,
                        std::atomic<int>* cache = nullptr) {
  if (a.flat_min_blocks > 0 && kernel) return dim3(resident_workgroups(kernel, 64 * waves, cache));
  return dim3((a.num_units + waves - 1) / waves);
}

bool decode_supported(const DecodeShape& s);
hipError_t launch_decode(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream);
// The shared-prefix decode of an e4m3 cache with one query head per KV head in one launch:
// `pre` (prefix units, workgroups [0, own.wg_base)) and `own` (per-sequence units,
// workgroups [own.wg_base, own.wg_base + own.wg_count)); own.wg_base is a multiple of 8.
bool cascade_fp8_supported(const DecodeShape& pre_shape, int heads_per_kv);
hipError_t launch_cascade_fp8(const DecodeShape& pre_shape, const DecodeArgs& pre,
                              const DecodeArgs& own, bool nt_own, hipStream_t stream);
// The matrix-core kernel alone (the only one that runs shared-prefix units).
bool gqa_mfma_supported(const DecodeShape& s);
hipError_t launch_decode_gqa_mfma(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream);

struct MergeArgs {
  void* out;
  const float* part_acc;
  const float* part_ml;
  const int32_t* ctx;
  int32_t num_seqs, num_heads, num_parts, partition_size, max_ctx;
  float v_scale;
  int32_t all_slots;         // 1: merge every slot, skipping empty ones (cascade partials)
  // flat split: a row's slots follow from the chunk length at flat_meta[0] and the blocks
  // of the sequences before it (block_size tokens each); 0 / null otherwise
  int32_t flat = 0, block_size = 0;
  const int32_t* flat_meta = nullptr;
};
hipError_t launch_merge(int head_dim, int q_kind, const MergeArgs& a, hipStream_t stream);

struct WriteArgs {
  const void* k_src;
  const void* v_src;
  void* k_cache;
  void* v_cache;
  const int32_t* tables;
  const int32_t* seq_ids;
  const int32_t* positions;
  int32_t num_seqs, max_blocks, num_tokens, num_blocks, num_kv_heads;
  float k_inv_scale, v_inv_scale;
};
bool write_supported(int head_dim, int block_size, int src_kind, int cache_kind);
hipError_t launch_write_kv(int head_dim, int block_size, int src_kind, int cache_kind,
                           const WriteArgs& a, hipStream_t stream);

struct CopyArgs {
  const void* src_k;         // source pools (may equal the destination pools)
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const int32_t* pairs;      // [num_pairs][2]: (src, dst) block ids
  int32_t num_pairs, src_blocks, dst_blocks;
  int64_t block_bytes;       // Hkv * B * d * e, a multiple of 16
};
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);

}  // namespace pa
