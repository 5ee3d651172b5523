// CPU block manager: free list, block tables and reference counts.
//
// "PagedAttention: Mathematical Foundations, ..." sec. 4 (allocation lifecycle: a prompt
// of N tokens takes ceil(N/B) physical blocks from the free list; a finished sequence
// drops one reference on each of its blocks and blocks at zero go back to the pool) and
// sec. 5 (parallel sampling / system-prompt sharing: the prompt's blocks are stored once
// with reference count K).  "Pytorch implementation of paper ..." sec. 3 fixes the order:
// blocks leave from the front of the free list and return at its back.
//
// The free list is a ring buffer of capacity num_blocks (it can never hold more), so both
// ends are O(1) and the list keeps its exact order.
//
// Swapping (same page, sec. 6: a preempted request's blocks are evicted to host RAM and
// brought back on resume): an optional host pool of slots with its own free list and
// reference counts.  A swapped-out sequence's table holds host slot ids.
#include <stdint.h>

#include <string>
#include <vector>

#include "paged_attn.h"

void pa_set_error(const std::string& msg);  // defined in api.hip

// FIFO free list over ids 0..capacity-1 (ring buffer).
struct FreeRing {
  std::vector<int32_t> ring;     // free ids, ring[(head + k) % capacity], k < count
  int64_t head = 0;
  int64_t count = 0;
  int32_t pop_front() {
    const int32_t id = ring[head];
    head = (head + 1) % (int64_t)ring.size();
    --count;
    return id;
  }
  void push_back(int32_t id) {
    ring[(head + count) % (int64_t)ring.size()] = id;
    ++count;
  }
  int32_t at(int64_t k) const { return ring[(head + k) % (int64_t)ring.size()]; }
};

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  FreeRing dev;                  // device free list
  std::vector<int32_t> refs;     // references per physical block
  FreeRing host;                 // host slot free list (empty until pa_bm_host_pool)
  std::vector<int32_t> host_refs;
  struct Seq {
    std::vector<int32_t> blocks; // logical block j -> physical id (host slot if swapped)
    int32_t context_len = 0;
    bool live = false;
    bool swapped = false;
  };
  std::vector<Seq> seqs;         // indexed by handle

  int64_t free_count() const { return dev.count; }
  int32_t pop_front() { return dev.pop_front(); }
  void push_back(int32_t id) { dev.push_back(id); }
  bool resident(int32_t h) const {
    return h >= 0 && h < (int32_t)seqs.size() && seqs[h].live && !seqs[h].swapped;
  }
};

static int32_t blocks_for(int64_t tokens, int32_t bs) { return (int32_t)((tokens + bs - 1) / bs); }

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       pa_block_manager** out) {
  if (!out || num_blocks < 1 || block_size < 1) {
    pa_set_error("pa_bm_create: need out != NULL, num_blocks >= 1, block_size >= 1");
    return PA_ERR_INVALID_ARG;
  }
  std::vector<int32_t> ring(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t k = 0; k < num_blocks; ++k) {
      const int32_t id = free_order[k];
      if (id < 0 || id >= num_blocks || seen[id]) {
        pa_set_error("pa_bm_create: free_order is not a permutation of 0..num_blocks-1");
        return PA_ERR_INVALID_ARG;
      }
      seen[id] = 1;
      ring[k] = id;
    }
  } else {
    for (int32_t k = 0; k < num_blocks; ++k) ring[k] = k;
  }
  auto* bm = new pa_block_manager();
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->dev.ring = std::move(ring);
  bm->dev.count = num_blocks;
  bm->refs.assign(num_blocks, 0);
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status pa_alloc_tables(pa_block_manager* bm, int32_t num_seqs, const int32_t* context_lens,
                          const int32_t* prefix_group, const int32_t* prefix_lens,
                          int32_t num_groups, int32_t max_blocks_per_seq,
                          int32_t* block_tables, int32_t* seq_handles) {
  if (!bm || num_seqs < 0 || max_blocks_per_seq < 1 || num_groups < 0 ||
      (num_seqs > 0 && (!context_lens || !block_tables || !seq_handles)) ||
      (prefix_group && num_groups > 0 && !prefix_lens)) {
    pa_set_error("pa_alloc_tables: invalid arguments");
    return PA_ERR_INVALID_ARG;
  }
  const int32_t B = bm->block_size;
  // Validate everything and count the blocks before touching any state.
  std::vector<int32_t> group_shared(num_groups, -1);  // shared block count once met
  int64_t need = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t n = context_lens[s];
    if (n < 0) {
      pa_set_error("pa_alloc_tables: negative context length");
      return PA_ERR_INVALID_ARG;
    }
    const int32_t nb = blocks_for(n, B);
    if (nb > max_blocks_per_seq) {
      pa_set_error("pa_alloc_tables: sequence " + std::to_string(s) + " needs " +
                   std::to_string(nb) + " blocks > max_blocks_per_seq " +
                   std::to_string(max_blocks_per_seq));
      return PA_ERR_TABLE_OVERFLOW;
    }
    int32_t shared = 0;
    const int32_t g = prefix_group ? prefix_group[s] : -1;
    if (g >= 0) {
      if (g >= num_groups || prefix_lens[g] < 0 || prefix_lens[g] > n) {
        pa_set_error("pa_alloc_tables: bad prefix group or prefix longer than the sequence");
        return PA_ERR_INVALID_ARG;
      }
      shared = prefix_lens[g] / B;
      if (group_shared[g] < 0) {
        group_shared[g] = shared;
        need += shared;
      }
    } else if (g < -1) {
      pa_set_error("pa_alloc_tables: prefix group ids must be >= -1");
      return PA_ERR_INVALID_ARG;
    }
    need += nb - shared;
  }
  if (need > bm->free_count()) {
    pa_set_error("pa_alloc_tables: need " + std::to_string(need) + " blocks, " +
                 std::to_string(bm->free_count()) + " free");
    return PA_ERR_NO_BLOCKS;
  }
  // Commit.
  std::vector<std::vector<int32_t>> group_blocks(num_groups);
  std::vector<char> group_done(num_groups, 0);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t n = context_lens[s];
    const int32_t nb = blocks_for(n, B);
    pa_block_manager::Seq seq;
    seq.context_len = n;
    seq.live = true;
    seq.blocks.reserve(nb);
    const int32_t g = prefix_group ? prefix_group[s] : -1;
    if (g >= 0) {
      if (!group_done[g]) {
        const int32_t shared = prefix_lens[g] / B;
        for (int32_t k = 0; k < shared; ++k) group_blocks[g].push_back(bm->pop_front());
        group_done[g] = 1;
      }
      for (int32_t id : group_blocks[g]) seq.blocks.push_back(id);
    }
    while ((int32_t)seq.blocks.size() < nb) seq.blocks.push_back(bm->pop_front());
    int32_t* row = block_tables + (size_t)s * max_blocks_per_seq;
    for (int32_t j = 0; j < max_blocks_per_seq; ++j)
      row[j] = j < nb ? seq.blocks[j] : -1;
    for (int32_t id : seq.blocks) bm->refs[id] += 1;
    seq_handles[s] = (int32_t)bm->seqs.size();
    bm->seqs.push_back(std::move(seq));
  }
  return PA_OK;
}

pa_status pa_bm_free(pa_block_manager* bm, int32_t n, const int32_t* seq_handles) {
  if (!bm || n < 0 || (n > 0 && !seq_handles)) {
    pa_set_error("pa_bm_free: invalid arguments");
    return PA_ERR_INVALID_ARG;
  }
  std::vector<char> hit(bm->seqs.size(), 0);
  for (int32_t k = 0; k < n; ++k) {
    const int32_t h = seq_handles[k];
    if (h < 0 || h >= (int32_t)bm->seqs.size() || !bm->seqs[h].live || hit[h]) {
      pa_set_error("pa_bm_free: handle " + std::to_string(h) + " is not a live sequence");
      return PA_ERR_INVALID_ARG;
    }
    hit[h] = 1;
  }
  for (int32_t k = 0; k < n; ++k) {
    auto& seq = bm->seqs[seq_handles[k]];
    if (seq.swapped) {  // its blocks live in host slots
      for (int32_t id : seq.blocks)
        if (--bm->host_refs[id] == 0) bm->host.push_back(id);
    } else {
      for (int32_t id : seq.blocks)
        if (--bm->refs[id] == 0) bm->push_back(id);
    }
    seq.swapped = false;
    seq.blocks.clear();
    seq.blocks.shrink_to_fit();
    seq.live = false;
  }
  return PA_OK;
}

pa_status pa_bm_stats(const pa_block_manager* bm, int32_t* refcounts, int32_t* num_free,
                      int64_t* waste_slots) {
  if (!bm) {
    pa_set_error("pa_bm_stats: NULL manager");
    return PA_ERR_INVALID_ARG;
  }
  if (refcounts)
    for (int32_t b = 0; b < bm->num_blocks; ++b) refcounts[b] = bm->refs[b];
  if (num_free) *num_free = (int32_t)bm->free_count();
  if (waste_slots) {
    int64_t w = 0;
    for (const auto& seq : bm->seqs)
      if (seq.live && !seq.swapped)
        w += (int64_t)seq.blocks.size() * bm->block_size - seq.context_len;
    *waste_slots = w;
  }
  return PA_OK;
}

pa_status pa_bm_free_list(const pa_block_manager* bm, int32_t* out, int32_t capacity,
                          int32_t* count) {
  if (!bm || !count || (capacity > 0 && !out) || capacity < 0) {
    pa_set_error("pa_bm_free_list: invalid arguments");
    return PA_ERR_INVALID_ARG;
  }
  *count = (int32_t)bm->free_count();
  const int64_t k_end = bm->free_count() < capacity ? bm->free_count() : capacity;
  for (int64_t k = 0; k < k_end; ++k) out[k] = bm->dev.at(k);
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t n, int32_t* child_handles) {
  if (!bm || n < 0 || (n > 0 && !child_handles) || !bm->resident(parent)) {
    pa_set_error("pa_bm_fork: invalid arguments or parent is not a live, resident sequence");
    return PA_ERR_INVALID_ARG;
  }
  for (int32_t k = 0; k < n; ++k) {
    pa_block_manager::Seq child;
    child.blocks = bm->seqs[parent].blocks;  // copied before push_back may reallocate
    child.context_len = bm->seqs[parent].context_len;
    child.live = true;
    for (int32_t id : child.blocks) bm->refs[id] += 1;
    child_handles[k] = (int32_t)bm->seqs.size();
    bm->seqs.push_back(std::move(child));
  }
  return PA_OK;
}

pa_status pa_bm_append(pa_block_manager* bm, int32_t n, const int32_t* seq_handles,
                       int32_t* slot_blocks, int32_t* slot_offsets, int32_t* copies,
                       int32_t max_copies, int32_t* num_copies) {
  if (!bm || n < 0 || max_copies < 0 || !num_copies ||
      (n > 0 && (!seq_handles || !slot_blocks || !slot_offsets)) || (max_copies > 0 && !copies)) {
    pa_set_error("pa_bm_append: invalid arguments");
    return PA_ERR_INVALID_ARG;
  }
  const int32_t B = bm->block_size;
  for (int32_t k = 0; k < n; ++k) {
    const int32_t h = seq_handles[k];
    if (!bm->resident(h)) {
      pa_set_error("pa_bm_append: handle " + std::to_string(h) +
                   " is not a live, resident sequence");
      return PA_ERR_INVALID_ARG;
    }
  }
  // Dry run: count new blocks and copies without touching the manager.  Appends are
  // applied in order, so a block shared by two sequences of the same call is copied only
  // for the first of them (the second then holds the last reference).
  std::vector<int32_t> ref_delta;   // sparse: block ids whose count dropped in the dry run
  std::vector<int32_t> len(n), fresh_tail(n, 0);
  auto dry_ref = [&](int32_t id) {
    int32_t r = bm->refs[id];
    for (int32_t x : ref_delta) r -= (x == id);
    return r;
  };
  int64_t need = 0, ncopy = 0;
  for (int32_t k = 0; k < n; ++k) {
    const int32_t h = seq_handles[k];
    int32_t cur = bm->seqs[h].context_len;
    bool tail_private = false;  // this call already gave the sequence a private tail block
    for (int32_t q = 0; q < k; ++q)
      if (seq_handles[q] == h) {
        cur += 1;
        tail_private = tail_private || fresh_tail[q];
      }
    if (cur % B == 0) {
      need += 1;
      fresh_tail[k] = 1;
    } else if (!tail_private) {
      const int32_t last = bm->seqs[h].blocks[cur / B];
      if (dry_ref(last) > 1) {
        need += 1;
        ncopy += 1;
        ref_delta.push_back(last);
        fresh_tail[k] = 1;
      }
    } else {
      fresh_tail[k] = 1;
    }
  }
  if (need > bm->free_count()) {
    pa_set_error("pa_bm_append: need " + std::to_string(need) + " blocks, " +
                 std::to_string(bm->free_count()) + " free");
    return PA_ERR_NO_BLOCKS;
  }
  if (ncopy > max_copies) {
    pa_set_error("pa_bm_append: " + std::to_string(ncopy) + " block copies exceed max_copies");
    return PA_ERR_INVALID_ARG;
  }
  // Commit.
  int32_t nc = 0;
  for (int32_t k = 0; k < n; ++k) {
    auto& seq = bm->seqs[seq_handles[k]];
    const int32_t j = seq.context_len / B, off = seq.context_len % B;
    if (off == 0) {  // overflow: the token opens a new block
      const int32_t id = bm->pop_front();
      bm->refs[id] = 1;
      seq.blocks.push_back(id);
    } else if (bm->refs[seq.blocks[j]] > 1) {  // copy-on-write of a shared partial block
      const int32_t src = seq.blocks[j];
      const int32_t id = bm->pop_front();
      bm->refs[src] -= 1;
      bm->refs[id] = 1;
      seq.blocks[j] = id;
      copies[2 * nc] = src;
      copies[2 * nc + 1] = id;
      ++nc;
    }
    slot_blocks[k] = seq.blocks[j];
    slot_offsets[k] = off;
    seq.context_len += 1;
  }
  *num_copies = nc;
  return PA_OK;
}

pa_status pa_bm_table(const pa_block_manager* bm, int32_t n, const int32_t* seq_handles,
                      int32_t max_blocks_per_seq, int32_t* block_tables, int32_t* context_lens) {
  if (!bm || n < 0 || max_blocks_per_seq < 1 || (n > 0 && (!seq_handles || !block_tables))) {
    pa_set_error("pa_bm_table: invalid arguments");
    return PA_ERR_INVALID_ARG;
  }
  for (int32_t k = 0; k < n; ++k) {
    const int32_t h = seq_handles[k];
    if (!bm->resident(h)) {
      pa_set_error("pa_bm_table: handle " + std::to_string(h) +
                   " is not a live, resident sequence");
      return PA_ERR_INVALID_ARG;
    }
    if ((int32_t)bm->seqs[h].blocks.size() > max_blocks_per_seq) {
      pa_set_error("pa_bm_table: sequence needs more than max_blocks_per_seq entries");
      return PA_ERR_TABLE_OVERFLOW;
    }
  }
  for (int32_t k = 0; k < n; ++k) {
    const auto& seq = bm->seqs[seq_handles[k]];
    int32_t* row = block_tables + (size_t)k * max_blocks_per_seq;
    for (int32_t j = 0; j < max_blocks_per_seq; ++j)
      row[j] = j < (int32_t)seq.blocks.size() ? seq.blocks[j] : -1;
    if (context_lens) context_lens[k] = seq.context_len;
  }
  return PA_OK;
}

pa_status pa_bm_host_pool(pa_block_manager* bm, int32_t num_host_blocks) {
  if (!bm || num_host_blocks < 0) {
    pa_set_error("pa_bm_host_pool: invalid arguments");
    return PA_ERR_INVALID_ARG;
  }
  for (int32_t r : bm->host_refs)
    if (r != 0) {
      pa_set_error("pa_bm_host_pool: host slots are in use");
      return PA_ERR_INVALID_ARG;
    }
  bm->host.ring.resize(num_host_blocks);
  for (int32_t k = 0; k < num_host_blocks; ++k) bm->host.ring[k] = k;
  bm->host.head = 0;
  bm->host.count = num_host_blocks;
  bm->host_refs.assign(num_host_blocks, 0);
  return PA_OK;
}

pa_status pa_bm_host_stats(const pa_block_manager* bm, int32_t* host_refcounts,
                           int32_t* num_host_free) {
  if (!bm) {
    pa_set_error("pa_bm_host_stats: NULL manager");
    return PA_ERR_INVALID_ARG;
  }
  if (host_refcounts)
    for (size_t k = 0; k < bm->host_refs.size(); ++k) host_refcounts[k] = bm->host_refs[k];
  if (num_host_free) *num_host_free = (int32_t)bm->host.count;
  return PA_OK;
}

// Move a gang of sequences between the device pool and the host pool.  Every distinct
// block the gang references (first appearance in handle order, then table order) gets one
// new block on the other side; sharing inside the gang is kept, references from outside
// the gang stay on the old side.  All-or-nothing.
static pa_status swap_gang(pa_block_manager* bm, bool out, int32_t n, const int32_t* handles,
                           int32_t* pairs, int32_t max_pairs, int32_t* num_pairs) {
  const char* who = out ? "pa_bm_swap_out" : "pa_bm_swap_in";
  if (!bm || n < 0 || max_pairs < 0 || !num_pairs || (n > 0 && !handles) ||
      (max_pairs > 0 && !pairs)) {
    pa_set_error(std::string(who) + ": invalid arguments");
    return PA_ERR_INVALID_ARG;
  }
  std::vector<char> hit(bm->seqs.size(), 0);
  for (int32_t k = 0; k < n; ++k) {
    const int32_t h = handles[k];
    if (h < 0 || h >= (int32_t)bm->seqs.size() || !bm->seqs[h].live || hit[h] ||
        bm->seqs[h].swapped != !out) {
      pa_set_error(std::string(who) + ": handle " + std::to_string(h) + " is not a live " +
                   (out ? "resident" : "swapped-out") + " sequence (or is repeated)");
      return PA_ERR_INVALID_ARG;
    }
    hit[h] = 1;
  }
  std::vector<int32_t>& from_refs = out ? bm->refs : bm->host_refs;
  std::vector<int32_t>& to_refs = out ? bm->host_refs : bm->refs;
  FreeRing& from_free = out ? bm->dev : bm->host;
  FreeRing& to_free = out ? bm->host : bm->dev;
  std::vector<int32_t> order;               // distinct old ids, first appearance
  std::vector<int32_t> slot(from_refs.size(), -1);
  for (int32_t k = 0; k < n; ++k)
    for (int32_t id : bm->seqs[handles[k]].blocks)
      if (slot[id] == -1) {
        slot[id] = (int32_t)order.size();
        order.push_back(id);
      }
  if ((int64_t)order.size() > to_free.count) {
    pa_set_error(std::string(who) + ": need " + std::to_string(order.size()) + " " +
                 (out ? "host slots" : "blocks") + ", " + std::to_string(to_free.count) + " free");
    return PA_ERR_NO_BLOCKS;
  }
  if ((int64_t)order.size() > max_pairs) {
    pa_set_error(std::string(who) + ": " + std::to_string(order.size()) +
                 " block moves exceed max_pairs");
    return PA_ERR_INVALID_ARG;
  }
  std::vector<int32_t> target(order.size());
  for (size_t q = 0; q < order.size(); ++q) {
    target[q] = to_free.pop_front();
    to_refs[target[q]] = 0;
    pairs[2 * q] = order[q];
    pairs[2 * q + 1] = target[q];
  }
  for (int32_t k = 0; k < n; ++k) {
    auto& seq = bm->seqs[handles[k]];
    for (int32_t& id : seq.blocks) {
      const int32_t nid = target[slot[id]];
      if (--from_refs[id] == 0) from_free.push_back(id);
      to_refs[nid] += 1;
      id = nid;
    }
    seq.swapped = out;
  }
  *num_pairs = (int32_t)order.size();
  return PA_OK;
}

pa_status pa_bm_swap_out(pa_block_manager* bm, int32_t n, const int32_t* seq_handles,
                         int32_t* block_pairs, int32_t max_pairs, int32_t* num_pairs) {
  return swap_gang(bm, true, n, seq_handles, block_pairs, max_pairs, num_pairs);
}

pa_status pa_bm_swap_in(pa_block_manager* bm, int32_t n, const int32_t* seq_handles,
                        int32_t* block_pairs, int32_t max_pairs, int32_t* num_pairs) {
  return swap_gang(bm, false, n, seq_handles, block_pairs, max_pairs, num_pairs);
}

}  // extern "C"
