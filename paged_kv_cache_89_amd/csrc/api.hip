// C-ABI layer of libpaged_attn: argument checks, launch planning, error reporting.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "launch.h"
#include "paged_attn.h"
#include "validate.h"

static thread_local std::string g_last_error;

void pa_set_error(const std::string& msg) { g_last_error = msg; }

namespace {

using namespace pa;

bool dtype_kind(pa_dtype d, int* kind) {
  switch (d) {
    case PA_F16: *kind = KIND_F16; return true;
    case PA_BF16: *kind = KIND_BF16; return true;
    case PA_FP8_E4M3: *kind = KIND_E4M3; return true;
  }
  return false;
}

pa_status fail(pa_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

pa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PA_OK;
  return fail(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("PA_LOG");
    return v && *v && *v != '0';
  }();
  return on;
}

struct Plan {
  int32_t partition_size;  // 0 = whole context in one unit (or the flat split)
  int32_t num_parts;       // partial slots per row
  int32_t flat_min_blocks = 0;  // > 0: flat split with chunks of at least this many blocks
};

// Library choice of the partition length.  A unit is one wavefront.  Contexts of at most
// 256 tokens run unsplit (the merge launch would cost more than it balances).  Otherwise
// partitions of `base` tokens keep units long enough to stream efficiently while cutting
// ragged batches into near-uniform pieces; when that leaves too few units to fill the
// chip's wave slots (256 CUs), the partition is halved while it stays at least 128 tokens.
// Measured on MI355X: 768-token partitions beat 512 by 0.5-1 % on the OPT-13B workload
// (and 1024 by 3.5-5 %); grouped queries take 1024 (below); the shared-prefix decode keeps
// 512, which splits its block-aligned prompts evenly (768 measured 4 % slower there).
constexpr int32_t kAutoPartition = 768;
// Grouped queries over 16-token blocks run on the matrix-core kernel, whose row-partitions
// are spread over the XCDs by their blocks: there 64-block partitions measured 0.55 % faster
// per GQA step than 768 tokens (0.2 % for four draft tokens; 512 tokens 3-4 % slower).
constexpr int32_t kAutoPartitionMfma = 1024;
// 1: matrix-core decodes (grouped queries, multi-token) of at most kBalancedMaxSeqs rows
// spread the row-partitions over the XCDs by their blocks (balanced_coords); compile-time
// switch for measurements.  Measured against contiguous ranges of rows, three pairs on one
// box: GQA workload 1.1 % faster per step, four-token drafts over it 2.1 %; the vector
// kernel's OPT-13B layer 5.7 % slower and the long-context workload 0.5 % slower, so the
// vector kernel keeps contiguous ranges.
#ifndef PA_BALANCED_XCD
#define PA_BALANCED_XCD 1
#endif
constexpr int32_t kCascadePartition = 512;
// The one-launch e4m3 cascade starts from 1024-token prefix partitions: its prefix units
// then fill about half of the wavefront slots and per-sequence units the rest from the
// start (measured on the fp8 shared-prompt workload: 184.9 vs 192.5 us, merge 5.3 vs 5.6 us).
constexpr int32_t kCascadeFusedPartition = 1024;
// 1: e4m3 shared-prefix decodes with one query head per KV head run their prefix and
// per-sequence units in one launch (compile-time switch for measurements)
#ifndef PA_CASCADE_ONE_LAUNCH
#define PA_CASCADE_ONE_LAUNCH 1
#endif
// Partials are stored and merged with 8- and 16-byte vector accesses.
constexpr uintptr_t kWorkspaceAlign = 16;
// Shortest share of a row's own blocks in the shared-prefix decode's per-sequence launch.
constexpr int32_t kSuffixMinBlocks = 8;

// Long contexts (the bound spans at least 16 base partitions): the partial last partition
// of a sequence is a small share of its work, so partitions take the 64-block maximum while
// the grid keeps at least 4096 units; fewer unit boundaries mean fewer set-ups and partial
// writes (measured +3 % on 32K-token contexts against 768).
int32_t auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx, int32_t base,
                       int32_t block_size) {
  if (max_ctx <= 256) return 0;
  const int64_t want_units = 4096;
  if ((int64_t)max_ctx >= 16 * (int64_t)base) {
    const int64_t big = (int64_t)kMaxUnitBlocks * block_size;
    if ((int64_t)num_seqs * num_kv_heads * ((max_ctx + big - 1) / big) >= want_units)
      return (int32_t)big;
  }
  int32_t P = base;
  while (P / 2 >= 128 &&
         (int64_t)num_seqs * num_kv_heads * ((max_ctx + P - 1) / P) < want_units)
    P /= 2;
  return P;
}

// Flat split (see launch.h): the library's choice for plain and multi-token decodes of at
// most kFlatMaxSeqs sequences whose contexts it would split, when the caller leaves the
// partition size to it.  Every unit then reads the same number of blocks whatever the
// lengths: measured on MI355X, partitions of unequal length (each sequence's last one
// short) cost 6-7 % against equal ones on the same bytes.  Chunks are at least
// kFlatMinBlocks long, which bounds a row's slots at ceil(blocks / kFlatMinBlocks) + 1.
// 32-token blocks keep fixed partitions: the flat walk would take their vector kernel from
// three waves per SIMD to two (and their one workload has equal lengths).
constexpr int32_t kFlatMinBlocks = 16;

pa_status make_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_context_len, int32_t partition_size,
                    Plan* plan, int32_t base_partition = kAutoPartition, bool flat_ok = false) {
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 ||
      max_context_len < 0 || partition_size < 0)
    return fail(PA_ERR_INVALID_ARG, "decode plan: negative or zero size");
  if (partition_size % block_size != 0)
    return fail(PA_ERR_INVALID_ARG, "decode plan: partition_size must be a multiple of block_size");
  const int32_t G = num_heads / num_kv_heads;
  if (base_partition == kAutoPartition && block_size == 16 && (G == 2 || G == 4 || G == 8) &&
      (head_dim == 64 || head_dim == 128))
    base_partition = kAutoPartitionMfma;
  int32_t P = partition_size > 0 ? partition_size
                                  : auto_partition(num_seqs, num_kv_heads, max_context_len,
                                                   base_partition, block_size);
  if (P > 0 && P % block_size != 0) P = ((P + block_size - 1) / block_size) * block_size;
  // A work unit walks at most kMaxUnitBlocks blocks (its table slice lives in one VGPR).
  const int64_t cap = (int64_t)kMaxUnitBlocks * block_size;
  if (P == 0 && max_context_len > cap) P = (int32_t)cap;
  if (P > cap) P = (int32_t)cap;
  plan->flat_min_blocks = 0;
  if (P == 0 || P >= max_context_len) {
    plan->partition_size = 0;
    plan->num_parts = 1;
  } else if (flat_ok && partition_size == 0 && num_seqs <= kFlatMaxSeqs && block_size <= 16 &&
             (int64_t)num_seqs * (((int64_t)max_context_len + block_size - 1) / block_size) <
                 ((int64_t)1 << 26)) {  // the walk's scan keeps block ends in 26 bits
    const int64_t max_blk = ((int64_t)max_context_len + block_size - 1) / block_size;
    plan->partition_size = 0;
    plan->num_parts = (int32_t)((max_blk + kFlatMinBlocks - 1) / kFlatMinBlocks + 1);
    plan->flat_min_blocks = kFlatMinBlocks;
  } else {
    plan->partition_size = P;
    plan->num_parts = (max_context_len + P - 1) / P;
  }
  return PA_OK;
}

// Partials: acc [rows, num_parts, D] then (m, l) [rows, num_parts, 2] (fp32); the flat
// split adds one 16-byte word after them for the chunk length the decode chose.
size_t workspace_bytes(const Plan& p, int32_t num_seqs, int32_t num_heads, int32_t head_dim) {
  if (p.num_parts <= 1 && p.flat_min_blocks == 0) return 0;
  const size_t rows = (size_t)num_seqs * num_heads * p.num_parts;
  return rows * head_dim * sizeof(float) + rows * 2 * sizeof(float) +
         (p.flat_min_blocks > 0 ? 16 : 0);
}

// Where the flat split's chunk length sits in a workspace laid out as above.
int32_t* flat_meta_ptr(const Plan& p, void* workspace, int32_t num_seqs, int32_t num_heads,
                       int32_t head_dim) {
  const size_t rows = (size_t)num_seqs * num_heads * p.num_parts;
  return (int32_t*)((char*)workspace + rows * head_dim * sizeof(float) + rows * 2 * sizeof(float));
}

// Shared-prefix decode: one partition length P for both launches (pa_decode's choice,
// or the whole context up to the 64-block cap when that choice is "no split"); the prefix
// launch owns slots [0, pre_parts) of every row, the per-sequence launch the next
// suf_parts.  Both counts come from host bounds, so some slots stay empty.
struct CascadePlan {
  int32_t partition_size, pre_parts, suf_parts;
  int32_t suf_min_blocks;  // > 0: the per-sequence launch splits each row's blocks evenly
};

pa_status make_cascade_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t max_context_len,
                            int32_t max_prefix_blocks, int32_t partition_size,
                            CascadePlan* cp, bool one_launch = false) {
  if (max_prefix_blocks < 0) return fail(PA_ERR_INVALID_ARG, "shared-prefix plan: max_prefix_blocks < 0");
  Plan p;
  const pa_status st = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                 max_context_len, partition_size, &p,
                                 one_launch ? kCascadeFusedPartition : kCascadePartition);
  if (st != PA_OK) return st;
  int64_t P = p.partition_size;
  if (P == 0) {
    const int64_t cap = (int64_t)kMaxUnitBlocks * block_size;
    const int64_t whole = ((int64_t)(max_context_len > 0 ? max_context_len : 1) + block_size - 1) /
                          block_size * block_size;
    P = whole < cap ? whole : cap;
  }
  const int64_t pre_tokens = std::min<int64_t>((int64_t)max_prefix_blocks * block_size, max_context_len);
  cp->partition_size = (int32_t)P;
  cp->pre_parts = (int32_t)((pre_tokens + P - 1) / P);
  cp->suf_parts = (int32_t)std::max<int64_t>(1, (max_context_len + P - 1) / P);
  cp->suf_min_blocks = 0;
  if (partition_size == 0) {
    // Library choice: the per-sequence tokens are what remains after the shared prefix,
    // anything from none to the whole context, so fixed partitions sized for the whole
    // context leave many per-sequence units short or empty.  Each row's own blocks are
    // split instead into suf_parts equal shares of at least kSuffixMinBlocks blocks: two
    // shares, or more where a share would exceed two partitions (64 blocks at most).
    // Measured on the fp8 shared-prompt workload (own tokens U[0, 512]): 2 % faster than
    // 512-token partitions, 1 % faster than three shares.
    const int64_t max_blk = ((int64_t)std::max(max_context_len, 1) + block_size - 1) / block_size;
    const int64_t cap = std::min<int64_t>(kMaxUnitBlocks, 2 * (P / block_size));
    const int64_t split = std::min<int64_t>(2, (max_blk + kSuffixMinBlocks - 1) / kSuffixMinBlocks);
    cp->suf_parts = (int32_t)std::max<int64_t>(split, (max_blk + cap - 1) / cap);
    cp->suf_min_blocks = kSuffixMinBlocks;
  }
  return PA_OK;
}

// Whether pa_decode_shared_prefix runs its prefix and per-sequence units in one launch:
// an e4m3 cache with one query head per KV head (the shapes pa_decode_shared_prefix
// supports otherwise), with a shared prefix to read.
bool cascade_one_launch(int32_t num_heads, int32_t num_kv_heads, int32_t block_size,
                        int32_t head_dim, int kv_kind, int32_t max_prefix_blocks) {
  return PA_CASCADE_ONE_LAUNCH && kv_kind == KIND_E4M3 && num_heads == num_kv_heads &&
         block_size == 16 && (head_dim == 64 || head_dim == 128) && max_prefix_blocks > 0;
}

size_t cascade_workspace_bytes(const CascadePlan& cp, int32_t num_seqs, int32_t num_heads,
                               int32_t head_dim) {
  const size_t rows = (size_t)num_seqs * num_heads * (cp.pre_parts + cp.suf_parts);
  return rows * head_dim * sizeof(float) + rows * 2 * sizeof(float);
}

}  // namespace

static pa_status decode_impl(const char* who, void* out, const void* query, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                    int32_t num_blocks, int32_t max_context_len, float scale,
                    pa_dtype q_dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
                    int32_t partition_size, uint32_t flags, void* workspace,
                    size_t workspace_bytes_given, void* stream, const void* k_new,
                    const void* v_new, float k_inv_scale, float v_inv_scale,
                    bool flat_ok = true) {
  g_last_error.clear();
  int qk, kk;
  if (!dtype_kind(q_dtype, &qk) || !dtype_kind(kv_dtype, &kk))
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": unknown dtype");
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 ||
      max_blocks_per_seq < 1 || num_blocks < 1 || max_context_len < 0 || partition_size < 0)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": bad size");
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": num_heads must be a multiple of num_kv_heads");
  if (partition_size % block_size != 0)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": partition_size must be a multiple of block_size");
  if (!std::isfinite(scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": non-finite scale");
  if (flags & ~(uint32_t)PA_DECODE_SHARED_KV)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": unknown flag bits");
  const bool shared = (flags & PA_DECODE_SHARED_KV) != 0;
  // Read-once K/V streams with the non-temporal hint; blocks shared between sequences of
  // the batch stay cacheable and the sharing sequences are visited together.
  DecodeShape shape{head_dim, block_size, qk, kk, num_heads / num_kv_heads, !shared};
  if (!decode_supported(shape))
    return fail(PA_ERR_UNSUPPORTED, std::string(who) + ": unsupported head_dim/block_size/group/dtype pair");
  const bool append = k_new != nullptr || v_new != nullptr;
  if (append && kk == KIND_E4M3 && !(std::isfinite(k_inv_scale) && std::isfinite(v_inv_scale)))
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": non-finite inverse scale");
  if (num_seqs == 0) return PA_OK;
  if (append && (!k_new || !v_new)) return fail(PA_ERR_INVALID_ARG, std::string(who) + ": NULL pointer");
  if (!out || !query || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": NULL pointer");

  // Tokens beyond the table's reach can never be addressed.
  const int64_t reach = (int64_t)max_blocks_per_seq * block_size;
  const int32_t max_ctx = (int32_t)(max_context_len < reach ? max_context_len : reach);
  // Plan from the caller's bound, exactly as pa_decode_workspace_size does; units beyond
  // the table's reach find no blocks and exit.
  Plan plan;
  pa_status st = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, partition_size, &plan, kAutoPartition,
                           flat_ok && !shared && kk != KIND_E4M3);
  if (st != PA_OK) return st;
  const size_t need = workspace_bytes(plan, num_seqs, num_heads, head_dim);
  if (need > 0 && (!workspace || workspace_bytes_given < need))
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": workspace needs " + std::to_string(need) +
                                        " bytes, got " + std::to_string(workspace_bytes_given));
  if (need > 0 && ((uintptr_t)workspace & (kWorkspaceAlign - 1)) != 0)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": workspace must be " +
                                        std::to_string(kWorkspaceAlign) + "-byte aligned");
  if (validate_enabled()) {
    std::string err;
    if (!validate_decode(who, block_tables, context_lens, num_seqs, max_blocks_per_seq,
                         num_blocks, block_size, max_context_len, 0, stream, &err))
      return fail(PA_ERR_INVALID_ARG, err);
    if (append && !validate_append_blocks(who, block_tables, context_lens, num_seqs,
                                          max_blocks_per_seq, num_blocks, block_size, stream,
                                          &err))
      return fail(PA_ERR_INVALID_ARG, err);
  }

  DecodeArgs a;
  a.out = out; a.q = query; a.k = k_cache; a.v = v_cache;
  a.tables = block_tables; a.ctx = context_lens;
  a.part_acc = need ? (float*)workspace : nullptr;
  a.part_ml = need ? (float*)workspace + (size_t)num_seqs * num_heads * plan.num_parts * head_dim
                   : nullptr;
  a.num_seqs = num_seqs; a.num_heads = num_heads; a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq; a.num_blocks = num_blocks; a.max_ctx = max_ctx;
  a.num_parts = plan.num_parts;
  a.blocks_per_part = plan.num_parts > 1 ? plan.partition_size / block_size
                                         : (int32_t)((reach + block_size - 1) / block_size);
  const int64_t units = (int64_t)num_seqs * num_kv_heads * plan.num_parts;
  if (units > (int64_t)1 << 30) return fail(PA_ERR_UNSUPPORTED, std::string(who) + ": grid too large");
  a.num_units = (int32_t)units;
  const bool f8 = kk == KIND_E4M3;
  a.qk_scale = scale * kLog2e * (f8 ? k_scale : 1.0f);
  a.v_scale = f8 ? v_scale : 1.0f;
  a.seq_fastest = shared ? 1 : 0;
  a.xcd_remap = (PA_BALANCED_XCD && gqa_mfma_supported(shape) && !shared &&
                 num_seqs <= kBalancedMaxSeqs) ? 2 : 1;
  a.num_slots = plan.num_parts > 1 ? plan.num_parts : 0;
  a.slot_base = 0;
  a.mode = MODE_PLAIN;
  a.seq_group = 1; a.num_groups = num_seqs; a.max_prefix_blocks = 0; a.prefix_blocks = nullptr;
  a.query_len = 1; a.tree_masks = nullptr;
  a.append = append ? 1 : 0;
  a.k_new = k_new; a.v_new = v_new;
  a.k_inv_scale = k_inv_scale; a.v_inv_scale = v_inv_scale;
  a.flat_min_blocks = plan.flat_min_blocks;
  a.flat_meta = plan.flat_min_blocks > 0
                    ? flat_meta_ptr(plan, workspace, num_seqs, num_heads, head_dim) : nullptr;
  if (plan.flat_min_blocks > 0) a.num_slots = plan.num_parts;
  if (log_enabled())
    std::fprintf(stderr, "[paged_attn] decode S=%d Hq=%d Hkv=%d D=%d B=%d max_ctx=%d P=%d parts=%d units=%lld flat=%d\n",
                 num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_ctx,
                 plan.partition_size, plan.num_parts, (long long)units, plan.flat_min_blocks);
  st = hip_status(launch_decode(shape, a, (hipStream_t)stream), (std::string(who) + " launch").c_str());
  if (st != PA_OK || a.num_slots == 0) return st;
  MergeArgs m;
  m.out = out; m.part_acc = a.part_acc; m.part_ml = a.part_ml; m.ctx = context_lens;
  m.num_seqs = num_seqs; m.num_heads = num_heads; m.num_parts = plan.num_parts;
  m.partition_size = plan.partition_size; m.max_ctx = max_ctx;
  m.v_scale = a.v_scale; m.all_slots = 0;
  m.flat = plan.flat_min_blocks > 0 ? 1 : 0; m.block_size = block_size; m.flat_meta = a.flat_meta;
  return hip_status(launch_merge(head_dim, qk, m, (hipStream_t)stream), (std::string(who) + " merge launch").c_str());
}

// ---- scratch of pa_decode_noalloc --------------------------------------------------
// A fixed device array for the partition partials of the no-allocation decode: the HIP
// runtime gives every GPU the library runs on its own copy, at its own address, held until
// the process ends.  Host code never uses the array's name as an address (on the host it
// only names the symbol): the device address of each GPU's copy is looked up once, with that
// GPU current, and kept in g_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's copy of `scratch`.
pa_status scratch_address(const char* who, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, (std::string(who) + ": hipGetDevice").c_str());
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, std::string(who) + ": device ordinal " + std::to_string(dev) +
                                        " beyond the " + std::to_string(kMaxDevices) + " supported");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, (std::string(who) + ": hipGetSymbolAddress").c_str());
    if (!p) return fail(PA_ERR_HIP, std::string(who) + ": no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_last_error.c_str(); }

const char* pa_version(void) { return "0.1.0"; }

int32_t pa_set_validate(int32_t on) { return set_validate(on != 0); }

uint64_t pa_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                               pa_dtype kv_dtype) {
  int kind;
  if (!dtype_kind(kv_dtype, &kind) || num_layers < 0 || num_kv_heads < 0 || head_dim < 0) return 0;
  const uint64_t e = kind == KIND_E4M3 ? 1 : 2;
  // one key and one value vector of num_kv_heads * head_dim elements per layer
  return 2ull * (uint64_t)num_layers * (uint64_t)num_kv_heads * (uint64_t)head_dim * e;
}

pa_status pa_write_kv(const void* k_src, const void* v_src, void* k_cache, void* v_cache,
                      const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                      const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                      int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, pa_dtype src_dtype, pa_dtype cache_dtype,
                      float k_inv_scale, float v_inv_scale, void* stream) {
  g_last_error.clear();
  int sk, ck;
  if (!dtype_kind(src_dtype, &sk) || !dtype_kind(cache_dtype, &ck))
    return fail(PA_ERR_INVALID_ARG, "pa_write_kv: unknown dtype");
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 1 || num_blocks < 1 ||
      num_kv_heads < 1 || head_dim < 1 || block_size < 1)
    return fail(PA_ERR_INVALID_ARG, "pa_write_kv: bad size");
  if (!write_supported(head_dim, block_size, sk, ck))
    return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: unsupported head_dim/block_size/dtype pair");
  if (num_tokens == 0) return PA_OK;
  if (!k_src || !v_src || !k_cache || !v_cache || !block_tables || !seq_ids || !positions)
    return fail(PA_ERR_INVALID_ARG, "pa_write_kv: NULL pointer");
  if (ck == KIND_E4M3 && !(std::isfinite(k_inv_scale) && std::isfinite(v_inv_scale)))
    return fail(PA_ERR_INVALID_ARG, "pa_write_kv: non-finite inverse scale");
  if (validate_enabled()) {
    std::string err;
    if (!validate_write(block_tables, seq_ids, positions, num_seqs, max_blocks_per_seq, num_tokens,
                        num_blocks, block_size, stream, &err))
      return fail(PA_ERR_INVALID_ARG, err);
  }
  WriteArgs a;
  a.k_src = k_src; a.v_src = v_src; a.k_cache = k_cache; a.v_cache = v_cache;
  a.tables = block_tables; a.seq_ids = seq_ids; a.positions = positions;
  a.num_seqs = num_seqs; a.max_blocks = max_blocks_per_seq; a.num_tokens = num_tokens;
  a.num_blocks = num_blocks; a.num_kv_heads = num_kv_heads;
  a.k_inv_scale = k_inv_scale; a.v_inv_scale = v_inv_scale;
  return hip_status(launch_write_kv(head_dim, block_size, sk, ck, a, (hipStream_t)stream),
                    "pa_write_kv launch");
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs,
                         int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads,
                         int32_t block_size, int32_t head_dim, pa_dtype cache_dtype,
                         void* stream) {
  g_last_error.clear();
  int ck;
  if (!dtype_kind(cache_dtype, &ck)) return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: unknown dtype");
  if (num_pairs < 0 || num_blocks < 1 || num_kv_heads < 1 || block_size < 1 || head_dim < 1)
    return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: bad size");
  const int64_t bytes = (int64_t)num_kv_heads * block_size * head_dim * (ck == KIND_E4M3 ? 1 : 2);
  if (bytes % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: block size in bytes must be a multiple of 16");
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: NULL pointer");
  if (validate_enabled()) {
    std::string err;
    if (!validate_pairs("pa_copy_blocks", block_pairs, num_pairs, num_blocks, num_blocks, true,
                        stream, &err))
      return fail(PA_ERR_INVALID_ARG, err);
  }
  CopyArgs a{k_cache, v_cache, k_cache, v_cache, block_pairs, num_pairs, num_blocks, num_blocks,
             bytes};
  return hip_status(launch_copy_blocks(a, (hipStream_t)stream), "pa_copy_blocks launch");
}

// Device-visible address of a pool: device memory as is; pinned host memory through its
// mapping.  Anything else (pageable host memory, unknown pointers) is refused, so the
// kernel never touches an address the device cannot reach.
static pa_status device_view(const void* p, const char* name, void** out) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PA_ERR_INVALID_ARG, std::string("pa_swap_blocks: ") + name +
                                        " is neither device memory nor pinned host memory");
  }
  if (attr.type == hipMemoryTypeDevice) {
    *out = const_cast<void*>(p);
    return PA_OK;
  }
  if (attr.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess || !d) {
      (void)hipGetLastError();
      return fail(PA_ERR_INVALID_ARG, std::string("pa_swap_blocks: ") + name +
                                          " is host memory without a device mapping");
    }
    *out = d;
    return PA_OK;
  }
  return fail(PA_ERR_INVALID_ARG, std::string("pa_swap_blocks: ") + name +
                                      " is neither device memory nor pinned host memory (type " +
                                      std::to_string((int)attr.type) + ")");
}

pa_status pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                         const int32_t* block_pairs, int32_t num_pairs, int32_t src_blocks,
                         int32_t dst_blocks, int32_t num_kv_heads, int32_t block_size,
                         int32_t head_dim, pa_dtype cache_dtype, void* stream) {
  g_last_error.clear();
  int ck;
  if (!dtype_kind(cache_dtype, &ck)) return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: unknown dtype");
  if (num_pairs < 0 || src_blocks < 1 || dst_blocks < 1 || num_kv_heads < 1 || block_size < 1 ||
      head_dim < 1)
    return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: bad size");
  const int64_t bytes = (int64_t)num_kv_heads * block_size * head_dim * (ck == KIND_E4M3 ? 1 : 2);
  if (bytes % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "pa_swap_blocks: block size in bytes must be a multiple of 16");
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !block_pairs)
    return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: NULL pointer");
  void *sk, *sv, *dk, *dv, *pp;
  pa_status st;
  if ((st = device_view(src_k, "src_k", &sk)) != PA_OK) return st;
  if ((st = device_view(src_v, "src_v", &sv)) != PA_OK) return st;
  if ((st = device_view(dst_k, "dst_k", &dk)) != PA_OK) return st;
  if ((st = device_view(dst_v, "dst_v", &dv)) != PA_OK) return st;
  if ((st = device_view(block_pairs, "block_pairs", &pp)) != PA_OK) return st;
  if (validate_enabled()) {
    std::string err;
    if (!validate_pairs("pa_swap_blocks", block_pairs, num_pairs, src_blocks, dst_blocks, false,
                        stream, &err))
      return fail(PA_ERR_INVALID_ARG, err);
  }
  CopyArgs a{sk, sv, dk, dv, (const int32_t*)pp, num_pairs, src_blocks, dst_blocks, bytes};
  return hip_status(launch_copy_blocks(a, (hipStream_t)stream), "pa_swap_blocks launch");
}

pa_status pa_decode_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t max_context_len,
                         int32_t partition_size, pa_dtype kv_dtype,
                         int32_t* used_partition_size, int32_t* num_partitions,
                         int32_t* flat_min_blocks) {
  g_last_error.clear();
  int kk;
  if (!dtype_kind(kv_dtype, &kk)) return fail(PA_ERR_INVALID_ARG, "pa_decode_plan: unknown dtype");
  Plan p;
  const pa_status st = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                 max_context_len, partition_size, &p, kAutoPartition,
                                 kk != KIND_E4M3);
  if (st != PA_OK) return st;
  if (used_partition_size) *used_partition_size = p.partition_size;
  if (num_partitions) *num_partitions = p.num_parts;
  if (flat_min_blocks) *flat_min_blocks = p.flat_min_blocks;
  return PA_OK;
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                int32_t partition_size) {
  // Enough for either split pa_decode may take: the flat split, or fixed partitions
  // (PA_DECODE_SHARED_KV, e4m3 caches).
  Plan flat, fixed;
  if (make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                partition_size, &flat, kAutoPartition, true) != PA_OK ||
      make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                partition_size, &fixed) != PA_OK)
    return 0;
  return std::max(workspace_bytes(flat, num_seqs, num_heads, head_dim),
                  workspace_bytes(fixed, num_seqs, num_heads, head_dim));
}

pa_status pa_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                    int32_t num_blocks, int32_t max_context_len, float scale,
                    pa_dtype q_dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
                    int32_t partition_size, uint32_t flags, void* workspace,
                    size_t workspace_bytes_given, void* stream) {
  return decode_impl("pa_decode", out, query, k_cache, v_cache, block_tables, context_lens,
                     num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, max_context_len, scale, q_dtype, kv_dtype, k_scale, v_scale,
                     partition_size, flags, workspace, workspace_bytes_given, stream, nullptr,
                     nullptr, 1.0f, 1.0f);
}

pa_status pa_decode_noalloc(void* out, const void* query, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t max_blocks_per_seq, int32_t num_blocks,
                            int32_t max_context_len, float scale, pa_dtype q_dtype,
                            pa_dtype kv_dtype, float k_scale, float v_scale,
                            int32_t partition_size, uint32_t flags, void* stream) {
  g_last_error.clear();
  const char* who = "pa_decode_noalloc";
  // The same plan pa_decode makes (and pa_decode_workspace_size sizes); refused before
  // anything else when its partials do not fit the fixed array.
  // The flat split where its partials fit the array, else fixed partitions.
  int kk;
  if (!dtype_kind(kv_dtype, &kk)) return fail(PA_ERR_INVALID_ARG, std::string(who) + ": unknown dtype");
  const bool shared = (flags & PA_DECODE_SHARED_KV) != 0;
  bool flat_ok = !shared && kk != KIND_E4M3;
  Plan plan;
  pa_status st = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, partition_size, &plan, kAutoPartition, flat_ok);
  if (st != PA_OK) return st;
  if (plan.flat_min_blocks > 0 &&
      workspace_bytes(plan, num_seqs, num_heads, head_dim) > (size_t)PA_NOALLOC_SCRATCH_BYTES) {
    flat_ok = false;
    st = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                   partition_size, &plan);
    if (st != PA_OK) return st;
  }
  const size_t need = workspace_bytes(plan, num_seqs, num_heads, head_dim);
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_ERR_UNSUPPORTED, std::string(who) + ": the partition partials need " +
                                        std::to_string(need) + " bytes, more than the " +
                                        std::to_string((size_t)PA_NOALLOC_SCRATCH_BYTES) +
                                        "-byte scratch array; call pa_decode with a workspace");
  void* ws = nullptr;
  if (need > 0 && num_seqs > 0) {
    st = scratch_address(who, &ws);
    if (st != PA_OK) return st;
  }
  return decode_impl(who, out, query, k_cache, v_cache, block_tables, context_lens, num_seqs,
                     num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, max_context_len, scale, q_dtype, kv_dtype, k_scale, v_scale,
                     partition_size, flags, ws, ws ? (size_t)PA_NOALLOC_SCRATCH_BYTES : 0,
                     stream, nullptr, nullptr, 1.0f, 1.0f, flat_ok);
}

pa_status pa_decode_append(void* out, const void* query, const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int32_t num_blocks,
                           int32_t max_context_len, float scale, pa_dtype q_dtype,
                           pa_dtype kv_dtype, float k_scale, float v_scale, float k_inv_scale,
                           float v_inv_scale, int32_t partition_size, uint32_t flags,
                           void* workspace, size_t workspace_bytes_given, void* stream) {
  g_last_error.clear();
  if (num_seqs > 0 && (!k_new || !v_new))
    return fail(PA_ERR_INVALID_ARG, "pa_decode_append: NULL pointer");
  return decode_impl("pa_decode_append", out, query, k_cache, v_cache, block_tables,
                     context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, num_blocks, max_context_len, scale, q_dtype, kv_dtype,
                     k_scale, v_scale, partition_size, flags, workspace, workspace_bytes_given,
                     stream, k_new, v_new, k_inv_scale, v_inv_scale);
}

size_t pa_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t block_size, int32_t max_context_len,
                                              int32_t max_prefix_blocks,
                                              int32_t partition_size) {
  // enough for either plan (the cache dtype is not an argument): the one-launch plan's
  // longer prefix partitions never need more slots than the two-launch plan's
  CascadePlan two, one;
  if (make_cascade_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_context_len, max_prefix_blocks, partition_size, &two) != PA_OK ||
      make_cascade_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_context_len, max_prefix_blocks, partition_size, &one, true) != PA_OK)
    return 0;
  return std::max(cascade_workspace_bytes(two, num_seqs, num_heads, head_dim),
                  cascade_workspace_bytes(one, num_seqs, num_heads, head_dim));
}

pa_status pa_decode_shared_prefix_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size,
                                       int32_t max_context_len, int32_t max_prefix_blocks,
                                       int32_t partition_size, pa_dtype kv_dtype,
                                       int32_t* prefix_partition_size, int32_t* prefix_slots,
                                       int32_t* suffix_slots, int32_t* suffix_min_blocks,
                                       int32_t* decode_launches) {
  g_last_error.clear();
  int kk;
  if (!dtype_kind(kv_dtype, &kk)) return fail(PA_ERR_INVALID_ARG, "shared-prefix plan: unknown dtype");
  const bool one = cascade_one_launch(num_heads, num_kv_heads, block_size, head_dim, kk,
                                      max_prefix_blocks);
  CascadePlan cp;
  const pa_status st = make_cascade_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                         max_context_len, max_prefix_blocks, partition_size, &cp,
                                         one);
  if (st != PA_OK) return st;
  if (prefix_partition_size) *prefix_partition_size = cp.partition_size;
  if (prefix_slots) *prefix_slots = cp.pre_parts;
  if (suffix_slots) *suffix_slots = cp.suf_parts;
  if (suffix_min_blocks) *suffix_min_blocks = cp.suf_min_blocks;
  if (decode_launches) *decode_launches = (one && cp.pre_parts > 0) ? 1 : (cp.pre_parts > 0 ? 2 : 1);
  return PA_OK;
}

pa_status pa_decode_shared_prefix(void* out, const void* query, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* prefix_blocks,
                                  int32_t num_seqs, int32_t seq_group, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, int32_t num_blocks,
                                  int32_t max_context_len, int32_t max_prefix_blocks,
                                  float scale, pa_dtype q_dtype, pa_dtype kv_dtype,
                                  float k_scale, float v_scale, int32_t partition_size,
                                  uint32_t flags, void* workspace,
                                  size_t workspace_bytes_given, void* stream) {
  g_last_error.clear();
  const char* who = "pa_decode_shared_prefix";
  int qk, kk;
  if (!dtype_kind(q_dtype, &qk) || !dtype_kind(kv_dtype, &kk))
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": unknown dtype");
  if (num_seqs < 0 || seq_group < 1 || num_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
      block_size < 1 || max_blocks_per_seq < 1 || num_blocks < 1 || max_context_len < 0 ||
      max_prefix_blocks < 0 || partition_size < 0)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": bad size");
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": num_heads must be a multiple of num_kv_heads");
  if (num_seqs % seq_group != 0)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": num_seqs must be a multiple of seq_group");
  if (partition_size % block_size != 0)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": partition_size must be a multiple of block_size");
  if (!std::isfinite(scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": non-finite scale");
  if (flags & ~(uint32_t)PA_DECODE_SHARED_KV)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": unknown flag bits");
  const bool shared = (flags & PA_DECODE_SHARED_KV) != 0;
  const int32_t G = num_heads / num_kv_heads;
  const int64_t vgroup = (int64_t)G * seq_group;
  // The prefix launch: one matrix-core unit holds every member's G heads.
  DecodeShape pre_shape{head_dim, block_size, qk, kk, (int)std::min<int64_t>(vgroup, 1 << 20), true};
  DecodeShape suf_shape{head_dim, block_size, qk, kk, G, !shared};
  if (!gqa_mfma_supported(pre_shape) || !decode_supported(suf_shape))
    return fail(PA_ERR_UNSUPPORTED, std::string(who) +
                ": needs block_size 16, head_dim 64/128, fp16/bf16 queries and "
                "(num_heads/num_kv_heads)*seq_group in {2,4,8,16}");
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !context_lens ||
      (max_prefix_blocks > 0 && !prefix_blocks))
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": NULL pointer");

  const int64_t reach = (int64_t)max_blocks_per_seq * block_size;
  const int32_t max_ctx = (int32_t)(max_context_len < reach ? max_context_len : reach);
  const bool one_launch = cascade_one_launch(num_heads, num_kv_heads, block_size, head_dim, kk,
                                            max_prefix_blocks);
  CascadePlan cp;
  pa_status st = make_cascade_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                   max_context_len, max_prefix_blocks, partition_size, &cp,
                                   one_launch);
  if (st != PA_OK) return st;
  const size_t need = cascade_workspace_bytes(cp, num_seqs, num_heads, head_dim);
  if (!workspace || workspace_bytes_given < need)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": workspace needs " + std::to_string(need) +
                                        " bytes, got " + std::to_string(workspace_bytes_given));
  if (need > 0 && ((uintptr_t)workspace & (kWorkspaceAlign - 1)) != 0)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": workspace must be " +
                                        std::to_string(kWorkspaceAlign) + "-byte aligned");
  if (validate_enabled()) {
    std::string err;
    if (!validate_decode(who, block_tables, context_lens, num_seqs, max_blocks_per_seq, num_blocks,
                         block_size, max_context_len, 0, stream, &err) ||
        !validate_prefix(who, block_tables, context_lens, prefix_blocks, num_seqs, seq_group,
                         max_blocks_per_seq, num_blocks, block_size, max_prefix_blocks, stream,
                         &err))
      return fail(PA_ERR_INVALID_ARG, err);
  }
  const int32_t slots = cp.pre_parts + cp.suf_parts;
  const int32_t groups = num_seqs / seq_group;
  const int64_t pre_units = (int64_t)groups * num_kv_heads * cp.pre_parts;
  const int64_t suf_units = (int64_t)num_seqs * num_kv_heads * cp.suf_parts;
  if (pre_units > (int64_t)1 << 30 || suf_units > (int64_t)1 << 30)
    return fail(PA_ERR_UNSUPPORTED, std::string(who) + ": grid too large");

  DecodeArgs a;
  a.out = out; a.q = query; a.k = k_cache; a.v = v_cache;
  a.tables = block_tables; a.ctx = context_lens;
  a.part_acc = (float*)workspace;
  a.part_ml = (float*)workspace + (size_t)num_seqs * num_heads * slots * head_dim;
  a.num_seqs = num_seqs; a.num_heads = num_heads; a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq; a.num_blocks = num_blocks; a.max_ctx = max_ctx;
  a.blocks_per_part = cp.partition_size / block_size;
  a.num_slots = slots;
  const bool f8 = kk == KIND_E4M3;
  a.qk_scale = scale * kLog2e * (f8 ? k_scale : 1.0f);
  a.v_scale = f8 ? v_scale : 1.0f;
  a.xcd_remap = 1;
  a.seq_group = seq_group; a.num_groups = groups;
  a.max_prefix_blocks = max_prefix_blocks;
  a.prefix_blocks = prefix_blocks;
  a.query_len = 1; a.tree_masks = nullptr;
  if (log_enabled())
    std::fprintf(stderr, "[paged_attn] shared-prefix decode S=%d K=%d Hq=%d Hkv=%d D=%d B=%d max_ctx=%d "
                 "max_prefix_blocks=%d P=%d prefix_parts=%d suffix_parts=%d\n",
                 num_seqs, seq_group, num_heads, num_kv_heads, head_dim, block_size, max_ctx,
                 max_prefix_blocks, cp.partition_size, cp.pre_parts, cp.suf_parts);
  // The per-sequence units' arguments.  The remaining tokens are mostly private:
  // neighbouring units take neighbouring heads of the same blocks (contiguous lines);
  // PA_DECODE_SHARED_KV only keeps the loads cacheable.
  DecodeArgs own = a;
  own.mode = MODE_SUFFIX; own.slot_base = cp.pre_parts; own.num_parts = cp.suf_parts;
  own.part_min_blocks = cp.suf_min_blocks;
  own.num_units = (int32_t)suf_units; own.seq_fastest = 0;
  if (cp.pre_parts > 0) {
    a.mode = MODE_PREFIX; a.slot_base = 0; a.num_parts = cp.pre_parts;
    a.num_units = (int32_t)pre_units; a.seq_fastest = 0;
    if (one_launch && cascade_fp8_supported(pre_shape, G)) {
      // e4m3, one query head per KV head: both kinds of unit in one launch, prefix units'
      // workgroups first (their count rounded up to a multiple of 8, so the per-sequence
      // workgroups keep their XCDs)
      const int64_t pre_wg = ((pre_units + 3) / 4 + 7) / 8 * 8;
      const int64_t own_wg = (suf_units + 3) / 4;
      if (pre_wg + own_wg > (int64_t)1 << 30)
        return fail(PA_ERR_UNSUPPORTED, std::string(who) + ": grid too large");
      a.wg_base = 0; a.wg_count = (int32_t)pre_wg;
      own.wg_base = (int32_t)pre_wg; own.wg_count = (int32_t)own_wg;
      st = hip_status(launch_cascade_fp8(pre_shape, a, own, suf_shape.nontemporal, (hipStream_t)stream),
                      "pa_decode_shared_prefix launch");
      if (st != PA_OK) return st;
    } else {
      st = hip_status(launch_decode_gqa_mfma(pre_shape, a, (hipStream_t)stream),
                      "pa_decode_shared_prefix prefix launch");
      if (st != PA_OK) return st;
      st = hip_status(launch_decode(suf_shape, own, (hipStream_t)stream),
                      "pa_decode_shared_prefix suffix launch");
      if (st != PA_OK) return st;
    }
  } else {
    st = hip_status(launch_decode(suf_shape, own, (hipStream_t)stream),
                    "pa_decode_shared_prefix suffix launch");
    if (st != PA_OK) return st;
  }
  MergeArgs m;
  m.out = out; m.part_acc = a.part_acc; m.part_ml = a.part_ml; m.ctx = context_lens;
  m.num_seqs = num_seqs; m.num_heads = num_heads; m.num_parts = slots;
  m.partition_size = cp.partition_size; m.max_ctx = max_ctx;
  m.v_scale = a.v_scale; m.all_slots = 1;
  return hip_status(launch_merge(head_dim, qk, m, (hipStream_t)stream),
                    "pa_decode_shared_prefix merge launch");
}

size_t pa_decode_multi_workspace_size(int32_t num_seqs, int32_t query_len, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int32_t max_context_len, int32_t partition_size) {
  // Enough for either split pa_decode_multi may take (see pa_decode_workspace_size).
  Plan flat, fixed;
  if (query_len < 1 ||
      make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                partition_size, &flat, kAutoPartition, true) != PA_OK ||
      make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                partition_size, &fixed) != PA_OK)
    return 0;
  return std::max(workspace_bytes(flat, num_seqs * query_len, num_heads, head_dim),
                  workspace_bytes(fixed, num_seqs * query_len, num_heads, head_dim));
}

pa_status pa_decode_multi(void* out, const void* query, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const uint32_t* tree_masks, int32_t num_seqs, int32_t query_len,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                          int32_t max_context_len, float scale, pa_dtype q_dtype,
                          pa_dtype kv_dtype, float k_scale, float v_scale,
                          int32_t partition_size, uint32_t flags, void* workspace,
                          size_t workspace_bytes_given, void* stream) {
  g_last_error.clear();
  const std::string who = "pa_decode_multi";
  int qk, kk;
  if (!dtype_kind(q_dtype, &qk) || !dtype_kind(kv_dtype, &kk))
    return fail(PA_ERR_INVALID_ARG, who + ": unknown dtype");
  if (num_seqs < 0 || query_len < 1 || num_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
      block_size < 1 || max_blocks_per_seq < 1 || num_blocks < 1 || max_context_len < 0 ||
      partition_size < 0)
    return fail(PA_ERR_INVALID_ARG, who + ": bad size");
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, who + ": num_heads must be a multiple of num_kv_heads");
  if (partition_size % block_size != 0)
    return fail(PA_ERR_INVALID_ARG, who + ": partition_size must be a multiple of block_size");
  if (!std::isfinite(scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_INVALID_ARG, who + ": non-finite scale");
  if (flags & ~(uint32_t)PA_DECODE_SHARED_KV)
    return fail(PA_ERR_INVALID_ARG, who + ": unknown flag bits");
  const bool shared = (flags & PA_DECODE_SHARED_KV) != 0;
  const int64_t cols = (int64_t)query_len * (num_heads / num_kv_heads);
  DecodeShape shape{head_dim, block_size, qk, kk, (int)std::min<int64_t>(cols, 1 << 20), !shared};
  if (!gqa_mfma_supported(shape))
    return fail(PA_ERR_UNSUPPORTED, who + ": needs block_size 16, head_dim 64/128, fp16/bf16 "
                "queries and query_len*(num_heads/num_kv_heads) in {2,4,8,16}");
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, who + ": NULL pointer");

  const int64_t reach = (int64_t)max_blocks_per_seq * block_size;
  const int32_t max_ctx = (int32_t)(max_context_len < reach ? max_context_len : reach);
  Plan plan;
  pa_status st = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, partition_size, &plan, kAutoPartition,
                           !shared && kk != KIND_E4M3);
  if (st != PA_OK) return st;
  const int32_t qrows = num_seqs * query_len;  // rows of [S, T] query tokens
  const size_t need = workspace_bytes(plan, qrows, num_heads, head_dim);
  if (need > 0 && (!workspace || workspace_bytes_given < need))
    return fail(PA_ERR_INVALID_ARG, who + ": workspace needs " + std::to_string(need) +
                                        " bytes, got " + std::to_string(workspace_bytes_given));
  if (need > 0 && ((uintptr_t)workspace & (kWorkspaceAlign - 1)) != 0)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": workspace must be " +
                                        std::to_string(kWorkspaceAlign) + "-byte aligned");
  if (validate_enabled()) {
    std::string err;
    if (!validate_decode(who.c_str(), block_tables, context_lens, num_seqs, max_blocks_per_seq,
                         num_blocks, block_size, max_context_len, query_len, stream, &err))
      return fail(PA_ERR_INVALID_ARG, err);
  }
  DecodeArgs a;
  a.out = out; a.q = query; a.k = k_cache; a.v = v_cache;
  a.tables = block_tables; a.ctx = context_lens;
  a.part_acc = need ? (float*)workspace : nullptr;
  a.part_ml = need ? (float*)workspace + (size_t)qrows * num_heads * plan.num_parts * head_dim
                   : nullptr;
  a.num_seqs = num_seqs; a.num_heads = num_heads; a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq; a.num_blocks = num_blocks; a.max_ctx = max_ctx;
  a.num_parts = plan.num_parts;
  a.blocks_per_part = plan.num_parts > 1 ? plan.partition_size / block_size
                                         : (int32_t)((reach + block_size - 1) / block_size);
  const int64_t units = (int64_t)num_seqs * num_kv_heads * plan.num_parts;
  if (units > (int64_t)1 << 30) return fail(PA_ERR_UNSUPPORTED, who + ": grid too large");
  a.num_units = (int32_t)units;
  a.num_slots = plan.num_parts > 1 ? plan.num_parts : 0;
  a.slot_base = 0;
  const bool f8 = kk == KIND_E4M3;
  a.qk_scale = scale * kLog2e * (f8 ? k_scale : 1.0f);
  a.v_scale = f8 ? v_scale : 1.0f;
  a.seq_fastest = shared ? 1 : 0;
  a.xcd_remap = (PA_BALANCED_XCD && !shared && num_seqs <= kBalancedMaxSeqs) ? 2 : 1;
  a.mode = MODE_MULTI;
  a.seq_group = 1; a.num_groups = num_seqs; a.max_prefix_blocks = 0; a.prefix_blocks = nullptr;
  a.query_len = query_len; a.tree_masks = tree_masks;
  a.flat_min_blocks = plan.flat_min_blocks;
  a.flat_meta = plan.flat_min_blocks > 0
                    ? flat_meta_ptr(plan, workspace, qrows, num_heads, head_dim) : nullptr;
  if (plan.flat_min_blocks > 0) a.num_slots = plan.num_parts;
  st = hip_status(launch_decode_gqa_mfma(shape, a, (hipStream_t)stream), "pa_decode_multi launch");
  if (st != PA_OK || a.num_slots == 0) return st;
  MergeArgs m;
  m.out = out; m.part_acc = a.part_acc; m.part_ml = a.part_ml; m.ctx = context_lens;
  m.num_seqs = num_seqs; m.num_heads = query_len * num_heads; m.num_parts = plan.num_parts;
  m.partition_size = plan.partition_size; m.max_ctx = max_ctx;
  m.v_scale = a.v_scale; m.all_slots = 0;
  m.flat = plan.flat_min_blocks > 0 ? 1 : 0; m.block_size = block_size; m.flat_meta = a.flat_meta;
  return hip_status(launch_merge(head_dim, qk, m, (hipStream_t)stream), "pa_decode_multi merge launch");
}

}  // extern "C"

namespace pa {

hipError_t launch_decode_64_nt(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_64_t(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_128_nt(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_128_t(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream);

bool decode_supported(const DecodeShape& s) {
  if (s.head_dim != 64 && s.head_dim != 128) return false;
  if (s.block_size != 8 && s.block_size != 16 && s.block_size != 32) return false;
  if (s.group != 1 && s.group != 2 && s.group != 4 && s.group != 8) return false;
  if (s.q_kind == KIND_E4M3) return false;
  return s.kv_kind == s.q_kind || s.kv_kind == KIND_E4M3;
}


int resident_workgroups(const void* kernel, int threads, std::atomic<int>* cache) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const bool cached = dev >= 0 && dev < kMaxCachedDevices && cache;
  if (cached) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) {
    (void)hipGetLastError();  // a failed query must not surface as the launch's error
    per_cu = 1;
  }
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    cus = 1;
  }
  const int r = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  if (cached) cache[dev].store(r, std::memory_order_relaxed);
  return r;
}

// Grouped-query shapes with 16-token blocks run the matrix-core kernel (fp16/bf16 caches on
// the 16-bit MFMA, e4m3 caches on the fp8 MFMA); every other shape runs the vector kernel.
hipError_t launch_decode(const DecodeShape& s, const DecodeArgs& a, hipStream_t stream) {
  if (gqa_mfma_supported(s))
    return launch_decode_gqa_mfma(s, a, stream);
  if (s.head_dim == 128)
    return s.nontemporal ? launch_decode_128_nt(s, a, stream) : launch_decode_128_t(s, a, stream);
  if (s.head_dim == 64)
    return s.nontemporal ? launch_decode_64_nt(s, a, stream) : launch_decode_64_t(s, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
