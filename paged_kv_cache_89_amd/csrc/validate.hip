// Validation mode of libpaged_attn (PA_VALIDATE=1 or pa_set_validate(1)).
//
// The device operations trust the index data that lives in device memory (context lengths,
// block tables, token slots, block pairs): an entry outside its range is skipped or
// clamped by the kernels, never dereferenced, so a bad table gives wrong numbers rather
// than a fault.  In validation mode every such entry point first copies that data to the
// host on the caller's stream (after all work queued before it), synchronises, and checks
// it; the first violation is returned as PA_ERR_INVALID_ARG with the offending index, and
// nothing is launched.  This costs a host round trip per call and is meant for debugging.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <string>
#include <unordered_set>
#include <vector>

#include "validate.h"

namespace pa {
namespace {

std::atomic<int> g_validate{-1};  // -1: not yet read from the environment

bool fetch_i32(const void* p, size_t count, void* stream, std::vector<int32_t>* out,
               const char* what, std::string* err) {
  out->assign(count, 0);
  if (count == 0) return true;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(out->data(), p, count * sizeof(int32_t), hipMemcpyDefault, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *err = std::string("validation: reading ") + what + ": " + hipGetErrorString(e);
    return false;
  }
  return true;
}

std::string at2(const char* name, int64_t i, int64_t j) {
  return std::string(name) + "[" + std::to_string(i) + "][" + std::to_string(j) + "]";
}

}  // namespace

bool validate_enabled() {
  int v = g_validate.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("PA_VALIDATE");
    v = (e && *e && *e != '0') ? 1 : 0;
    int expected = -1;
    g_validate.compare_exchange_strong(expected, v);
    v = g_validate.load(std::memory_order_relaxed);
  }
  return v == 1;
}

int set_validate(int on) {
  const int prev = validate_enabled() ? 1 : 0;
  g_validate.store(on ? 1 : 0);
  return prev;
}

bool validate_decode(const char* who, const int32_t* tables, const int32_t* ctx, int32_t num_seqs,
                     int32_t max_blocks, int32_t num_blocks, int32_t block_size,
                     int32_t max_context_len, int32_t min_len, void* stream, std::string* err) {
  std::vector<int32_t> n, t;
  if (!fetch_i32(ctx, (size_t)num_seqs, stream, &n, "context_lens", err)) return false;
  if (!fetch_i32(tables, (size_t)num_seqs * max_blocks, stream, &t, "block_tables", err)) return false;
  const int64_t reach = (int64_t)max_blocks * block_size;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t ns = n[s];
    const std::string head = std::string(who) + ": context_lens[" + std::to_string(s) + "] = " +
                             std::to_string(ns);
    if (ns < 0) return *err = head + " is negative", false;
    if (ns < min_len) return *err = head + " is below query_len " + std::to_string(min_len), false;
    if (ns > max_context_len)
      return *err = head + " exceeds max_context_len " + std::to_string(max_context_len), false;
    if (ns > reach)
      return *err = head + " exceeds max_blocks_per_seq * block_size = " + std::to_string(reach), false;
    const int64_t nb = (ns + block_size - 1) / block_size;
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t id = t[(size_t)s * max_blocks + j];
      if (id < 0 || id >= num_blocks)
        return *err = std::string(who) + ": " + at2("block_tables", s, j) + " = " +
                      std::to_string(id) + " is outside [0, " + std::to_string(num_blocks) +
                      ") (sequence length " + std::to_string(ns) + ")",
               false;
    }
  }
  return true;
}

bool validate_append_blocks(const char* who, const int32_t* tables, const int32_t* ctx,
                            int32_t num_seqs, int32_t max_blocks, int32_t num_blocks,
                            int32_t block_size, void* stream, std::string* err) {
  std::vector<int32_t> n, t;
  if (!fetch_i32(ctx, (size_t)num_seqs, stream, &n, "context_lens", err)) return false;
  if (!fetch_i32(tables, (size_t)num_seqs * max_blocks, stream, &t, "block_tables", err)) return false;
  // every read of a block: how many entries name it, and the first two of them
  std::vector<int32_t> refs((size_t)num_blocks, 0);
  std::vector<int64_t> first((size_t)num_blocks, -1), second((size_t)num_blocks, -1);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t nb = ((int64_t)n[s] + block_size - 1) / block_size;
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t id = t[(size_t)s * max_blocks + j];
      if (id < 0 || id >= num_blocks) continue;  // reported by validate_decode
      const int64_t at = (int64_t)s * max_blocks + j;
      if (refs[id]++ == 0) first[id] = at; else if (second[id] < 0) second[id] = at;
    }
  }
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (n[s] <= 0) continue;
    const int64_t j = ((int64_t)n[s] - 1) / block_size;
    const int32_t id = t[(size_t)s * max_blocks + j];
    if (id < 0 || id >= num_blocks || refs[id] == 1) continue;
    const int64_t other = first[id] == (int64_t)s * max_blocks + j ? second[id] : first[id];
    return *err = std::string(who) + ": the new token of sequence " + std::to_string(s) +
                  " goes to block " + std::to_string(id) + " (" + at2("block_tables", s, j) +
                  "), which " + at2("block_tables", other / max_blocks, other % max_blocks) +
                  " also reads (a race)",
           false;
  }
  return true;
}

bool validate_prefix(const char* who, const int32_t* tables, const int32_t* ctx,
                     const int32_t* prefix_blocks, int32_t num_seqs, int32_t seq_group,
                     int32_t max_blocks, int32_t num_blocks, int32_t block_size,
                     int32_t max_prefix_blocks, void* stream, std::string* err) {
  const int32_t groups = num_seqs / seq_group;
  std::vector<int32_t> n, t, pb;
  if (!fetch_i32(ctx, (size_t)num_seqs, stream, &n, "context_lens", err)) return false;
  if (!fetch_i32(tables, (size_t)num_seqs * max_blocks, stream, &t, "block_tables", err)) return false;
  if (max_prefix_blocks > 0 &&
      !fetch_i32(prefix_blocks, (size_t)groups, stream, &pb, "prefix_blocks", err))
    return false;
  for (int32_t g = 0; g < groups && max_prefix_blocks > 0; ++g) {
    const int32_t p = pb[g];
    if (p < 0 || p > max_prefix_blocks)
      return *err = std::string(who) + ": prefix_blocks[" + std::to_string(g) + "] = " +
                    std::to_string(p) + " is outside [0, max_prefix_blocks = " +
                    std::to_string(max_prefix_blocks) + "]",
             false;
    const int32_t first = g * seq_group;
    // the shared blocks are read through the first member's row, up to the longest member
    int64_t longest = 0;
    for (int32_t k = 0; k < seq_group; ++k) longest = std::max<int64_t>(longest, n[first + k]);
    const int64_t shared = std::min<int64_t>(
        std::min<int64_t>(p, max_blocks), (longest + block_size - 1) / block_size);
    for (int64_t j = 0; j < shared; ++j) {
      const int32_t id = t[(size_t)first * max_blocks + j];
      if (id < 0 || id >= num_blocks)
        return *err = std::string(who) + ": " + at2("block_tables", first, j) + " = " +
                      std::to_string(id) + " (a shared block of group " + std::to_string(g) +
                      ") is outside [0, " + std::to_string(num_blocks) + ")",
               false;
    }
    for (int32_t k = 1; k < seq_group; ++k) {
      const int32_t m = first + k;
      const int64_t used = std::min<int64_t>(
          std::min<int64_t>(p, max_blocks), ((int64_t)std::max(n[m], 0) + block_size - 1) / block_size);
      for (int64_t j = 0; j < used; ++j)
        if (t[(size_t)m * max_blocks + j] != t[(size_t)first * max_blocks + j])
          return *err = std::string(who) + ": " + at2("block_tables", m, j) + " = " +
                        std::to_string(t[(size_t)m * max_blocks + j]) +
                        " differs from the group's first member (" +
                        std::to_string(t[(size_t)first * max_blocks + j]) + ") inside prefix_blocks[" +
                        std::to_string(g) + "] = " + std::to_string(p),
                 false;
    }
  }
  return true;
}

bool validate_write(const int32_t* tables, const int32_t* seq_ids, const int32_t* positions,
                    int32_t num_seqs, int32_t max_blocks, int32_t num_tokens, int32_t num_blocks,
                    int32_t block_size, void* stream, std::string* err) {
  std::vector<int32_t> t, sid, pos;
  if (!fetch_i32(seq_ids, (size_t)num_tokens, stream, &sid, "seq_ids", err)) return false;
  if (!fetch_i32(positions, (size_t)num_tokens, stream, &pos, "positions", err)) return false;
  if (!fetch_i32(tables, (size_t)num_seqs * max_blocks, stream, &t, "block_tables", err)) return false;
  const int64_t reach = (int64_t)max_blocks * block_size;
  std::unordered_set<int64_t> slots;
  for (int32_t i = 0; i < num_tokens; ++i) {
    const std::string tok = "pa_write_kv: token " + std::to_string(i);
    if (sid[i] < 0 || sid[i] >= num_seqs)
      return *err = tok + ": seq_ids = " + std::to_string(sid[i]) + " is outside [0, " +
                    std::to_string(num_seqs) + ")",
             false;
    if (pos[i] < 0 || pos[i] >= reach)
      return *err = tok + ": positions = " + std::to_string(pos[i]) + " is outside [0, " +
                    std::to_string(reach) + ")",
             false;
    const int64_t j = pos[i] / block_size;
    const int32_t id = t[(size_t)sid[i] * max_blocks + j];
    if (id < 0 || id >= num_blocks)
      return *err = tok + ": " + at2("block_tables", sid[i], j) + " = " + std::to_string(id) +
                    " is outside [0, " + std::to_string(num_blocks) + ")",
             false;
    const int64_t slot = (int64_t)id * block_size + pos[i] % block_size;
    if (!slots.insert(slot).second)
      return *err = tok + " writes block " + std::to_string(id) + " slot " +
                    std::to_string(pos[i] % block_size) + ", as an earlier token does (a race)",
             false;
  }
  return true;
}

bool validate_pairs(const char* who, const int32_t* pairs, int32_t num_pairs, int32_t src_blocks,
                    int32_t dst_blocks, bool same_pool, void* stream, std::string* err) {
  std::vector<int32_t> p;
  if (!fetch_i32(pairs, (size_t)num_pairs * 2, stream, &p, "block_pairs", err)) return false;
  std::unordered_set<int32_t> dsts, srcs;
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int32_t s = p[2 * i], d = p[2 * i + 1];
    const std::string pr = std::string(who) + ": pair " + std::to_string(i) + " (" +
                           std::to_string(s) + ", " + std::to_string(d) + ")";
    if (s < 0 || s >= src_blocks)
      return *err = pr + ": source outside [0, " + std::to_string(src_blocks) + ")", false;
    if (d < 0 || d >= dst_blocks)
      return *err = pr + ": destination outside [0, " + std::to_string(dst_blocks) + ")", false;
    if (!dsts.insert(d).second) return *err = pr + ": destination written twice (a race)", false;
    if (same_pool) srcs.insert(s);
  }
  if (same_pool)
    for (int32_t i = 0; i < num_pairs; ++i)
      if (srcs.count(p[2 * i + 1]))
        return *err = std::string(who) + ": pair " + std::to_string(i) + " writes block " +
                      std::to_string(p[2 * i + 1]) + ", which another pair reads (a race)",
               false;
  return true;
}

}  // namespace pa
