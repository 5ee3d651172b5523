/*
 * libpaged_attn — paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Every call returns a pa_status (0 = OK,
 * negative = error) unless stated otherwise; pa_last_error() then gives a message.
 *
 * The operation and its vocabulary come from:
 *   [P1] "PagedAttention: Mathematical Foundations, Virtual Memory Block Allocation,
 *        and Zero-Waste KV Cache Serving" (llms.blog)
 *   [P2] "Pytorch implementation of paper: Efficient Memory Management for Large
 *        Language Model Serving with PagedAttention (2023)" (aishastr.live)
 *   [P3] the 10100.com article on the retirement of vLLM's PagedAttention kernel
 *
 * Conventions for the device calls (pa_write_kv, pa_copy_blocks, pa_decode*):
 *   - every pointer is device memory owned by the caller, every tensor is contiguous
 *     row-major with the shape written beside it;
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream);
 *     the call only enqueues work and never synchronises; argument errors are found
 *     on the host before anything is launched and leave device memory untouched;
 *   - device-resident tables and lengths are read by the kernels as given; entries
 *     outside [0, num_blocks) are never dereferenced (the decode clamps them to block 0,
 *     the writer skips them) so malformed tables give wrong numbers, not faults;
 *   - the library allocates no device memory: scratch space is a caller-provided
 *     workspace sized by pa_decode_workspace_size();
 *   - a call enqueues kernels only (no allocation, memset or host wait), so it can be
 *     captured into a HIP graph and replayed; validation mode (pa_set_validate) waits on
 *     the stream and must be off while a stream is captured.
 *
 * Cache layout (both K and V, every dtype): [num_blocks][num_kv_heads][block_size][head_dim],
 * i.e. the per-block [block_size, head_dim] key and value tiles of [P1] sec. 3 (eq. for
 * K_j, V_j) and sec. 7 (pseudocode), one tile per KV head.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,     /* null pointer, inconsistent sizes, bad handle, short workspace */
  PA_ERR_UNSUPPORTED = -2,     /* shape or dtype outside the compiled set */
  PA_ERR_NO_BLOCKS = -3,       /* the free list cannot satisfy the request (state unchanged) */
  PA_ERR_TABLE_OVERFLOW = -4,  /* a sequence needs more than max_blocks_per_seq blocks */
  PA_ERR_HIP = -5              /* the HIP runtime reported an error at launch */
} pa_status;

/* Storage / arithmetic types.  PA_FP8_E4M3 is the OCP 8-bit E4M3 format (no infinities,
 * S.1111.111 = NaN, largest finite 448), stored one byte per element. */
typedef enum { PA_F16 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

typedef struct pa_block_manager pa_block_manager; /* opaque, host memory only */

/* Message for the last error on the calling thread ("" if none).  Owned by the library,
 * valid until the next call on the same thread. */
const char* pa_last_error(void);

/* Library version string, e.g. "0.1.0". */
const char* pa_version(void);

/* Validation mode (off by default; on when the environment has PA_VALIDATE=1 at the first
 * call, or after pa_set_validate(1)).  The device operations read index data that lives in
 * device memory -- context_lens, block_tables, prefix_blocks, seq_ids / positions, block
 * pairs -- and trust it: out-of-range entries are skipped or clamped as each operation
 * documents, never dereferenced.  In validation mode each of pa_write_kv, pa_copy_blocks,
 * pa_swap_blocks, pa_decode, pa_decode_shared_prefix and pa_decode_multi first copies that
 * data to the host on its stream (after everything queued before it), synchronises and
 * checks it: ids inside their pools, context_lens in [0, max_context_len] and within the
 * table's reach (at least query_len for pa_decode_multi), the table entries a sequence
 * reads, prefix_blocks in [0, max_prefix_blocks] with every member's prefix entries equal
 * to the first member's, no cache slot or destination block written twice in one call,
 * and (pa_copy_blocks) no destination that another pair reads.  The first violation is
 * returned as PA_ERR_INVALID_ARG with its index in pa_last_error(), and nothing is
 * launched (pa_decode_append is checked as pa_decode, and its new tokens' blocks must be
 * named by no other table entry the decode reads).  A debugging aid: every call then
 * costs a host round trip.
 * Returns the previous setting (0 or 1). */
int32_t pa_set_validate(int32_t on);

/* ------------------------------------------------------------------------------------
 * CPU block manager.
 * [P1] sec. 4 "Allocation Lifecycle": a prompt of N tokens takes ceil(N / B) blocks from
 * the free list; blocks whose reference count drops to zero return to the pool.
 * [P2] sec. 3 "The Block Manager": the free list is consumed from its front and returned
 * blocks are appended at its back.
 * [P1] sec. 5 "Parallel Sampling" / "System Prompt Prefix Sharing": the prompt of K
 * sequences is stored once, in blocks whose reference count is K.
 * ------------------------------------------------------------------------------------ */

/* Create a manager over num_blocks physical blocks of block_size tokens (any block_size
 * >= 1).  free_order: host [num_blocks], a permutation of 0..num_blocks-1 giving the
 * initial free-list order (NULL = ascending).  *out receives the handle. */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       pa_block_manager** out);

/* Destroy a manager (NULL is ignored). */
void pa_bm_destroy(pa_block_manager* bm);

/* Allocate block tables for num_seqs new sequences, in index order.
 *   context_lens  host [num_seqs], each >= 0 tokens;
 *   prefix_group  host [num_seqs] or NULL: group id in [0, num_groups) or -1 for none;
 *   prefix_lens   host [num_groups] tokens: the group's first floor(len / B) blocks are
 *                 shared by all its members (taken from the free list when the group is
 *                 first met; reference count = number of members).  A member needs
 *                 context_len >= its prefix length.  The prompt's remaining tokens, and
 *                 everything after, go in private blocks;
 *   block_tables  host out [num_seqs, max_blocks_per_seq] int32, row s = physical ids of
 *                 sequence s's logical blocks, unused entries -1;
 *   seq_handles   host out [num_seqs]: handles for pa_bm_free.
 * All-or-nothing: on PA_ERR_NO_BLOCKS / PA_ERR_TABLE_OVERFLOW / PA_ERR_INVALID_ARG the
 * manager is unchanged and the outputs are untouched. */
pa_status pa_alloc_tables(pa_block_manager* bm, int32_t num_seqs, const int32_t* context_lens,
                          const int32_t* prefix_group, const int32_t* prefix_lens,
                          int32_t num_groups, int32_t max_blocks_per_seq,
                          int32_t* block_tables, int32_t* seq_handles);

/* Release sequences: each of their blocks loses one reference; blocks reaching zero are
 * appended to the back of the free list in table order ([P1] sec. 4 "Completion").
 * A handle that is not live (never issued, or already freed) gives PA_ERR_INVALID_ARG and
 * nothing is released. */
pa_status pa_bm_free(pa_block_manager* bm, int32_t n, const int32_t* seq_handles);

/* Counters.  refcounts: host [num_blocks] or NULL; num_free, waste_slots: may be NULL.
 * waste_slots = sum over live sequences of (blocks * B - context_len), the internal
 * fragmentation that [P1] sec. 4 bounds by B - 1 slots per sequence. */
pa_status pa_bm_stats(const pa_block_manager* bm, int32_t* refcounts, int32_t* num_free,
                      int64_t* waste_slots);

/* Copy the current free list (front first) into out[capacity]; *count = its length. */
pa_status pa_bm_free_list(const pa_block_manager* bm, int32_t* out, int32_t capacity,
                          int32_t* count);

/* Fork ([P1] sec. 5 "Parallel Sampling"): create n sequences that share every block of the
 * live sequence `parent` (each shared block gains n references) and have its length.
 * child_handles: host out [n]. */
pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t n, int32_t* child_handles);

/* Reserve the slot of the next token of each sequence, in the order given ([P1] sec. 4
 * "Decoding Step" / "Block Overflow"; sec. 5 copy-on-write).  For a sequence of length L:
 *   - L % B == 0: the token opens a new block, taken from the front of the free list;
 *   - otherwise, if the last block is shared (reference count > 1): copy-on-write -- a new
 *     block is taken, the pair (shared id, new id) is recorded for pa_copy_blocks, the
 *     shared block loses one reference and the sequence's table points at the new block;
 *   - the length becomes L + 1.
 * slot_blocks / slot_offsets: host out [n], where the token goes (the block id and slot to
 * hand to pa_write_kv via the updated table and position L).  copies: host out
 * [max_copies][2]; *num_copies receives the number of pairs.  All-or-nothing: if the free
 * list is too short (PA_ERR_NO_BLOCKS), max_copies too small or a handle not live
 * (PA_ERR_INVALID_ARG), nothing changes.  The copies must run (pa_copy_blocks) before the
 * new tokens are written. */
pa_status pa_bm_append(pa_block_manager* bm, int32_t n, const int32_t* seq_handles,
                       int32_t* slot_blocks, int32_t* slot_offsets, int32_t* copies,
                       int32_t max_copies, int32_t* num_copies);

/* ------------------------------------------------------------------------------------
 * Swapping ([P1] sec. 6, preemption by swapping: a preempted request's blocks are evicted
 * from HBM to host RAM and brought back when it resumes; the cost is bounded by the host
 * link).  The manager keeps an optional pool of host slots with its own FIFO free list
 * (ascending ids) and reference counts; the data moves with pa_swap_blocks.
 *
 * pa_bm_host_pool: (re)size the host pool to num_host_blocks slots; refused while any slot
 * is referenced. */
pa_status pa_bm_host_pool(pa_block_manager* bm, int32_t num_host_blocks);

/* host_refcounts host out [num_host_blocks] (may be NULL), num_host_free (may be NULL). */
pa_status pa_bm_host_stats(const pa_block_manager* bm, int32_t* host_refcounts,
                           int32_t* num_host_free);

/* Swap out a gang of live, resident sequences (e.g. all samples of one request): every
 * distinct block they reference (first appearance in handle order, then table order)
 * takes a host slot from the front of the host free list; the gang's tables then name host
 * slots (sharing inside the gang is kept), each device block loses the gang's references
 * and returns to the back of the device free list at zero.  block_pairs host out
 * [max_pairs][2] receives (device block, host slot) for every move, *num_pairs their
 * count: copy them (pa_swap_blocks, device pools -> host pools) before the released
 * device blocks are written again.  Swapped-out sequences can only be swapped in or freed
 * (pa_bm_free releases their host slots).  All-or-nothing: too few host slots
 * (PA_ERR_NO_BLOCKS), max_pairs too small or a handle that is not a live resident
 * sequence or is repeated (PA_ERR_INVALID_ARG) change nothing. */
pa_status pa_bm_swap_out(pa_block_manager* bm, int32_t n, const int32_t* seq_handles,
                         int32_t* block_pairs, int32_t max_pairs, int32_t* num_pairs);

/* Swap a gang of swapped-out sequences back in: every distinct host slot they reference
 * takes a block from the front of the device free list; block_pairs receives (host slot,
 * device block) per move (copy host pools -> device pools with pa_swap_blocks before the
 * sequences are decoded).  Same rules and errors as pa_bm_swap_out, roles exchanged. */
pa_status pa_bm_swap_in(pa_block_manager* bm, int32_t n, const int32_t* seq_handles,
                        int32_t* block_pairs, int32_t max_pairs, int32_t* num_pairs);

/* Current table rows and lengths of live, resident sequences: block_tables host out
 * [n, max_blocks_per_seq] (-1 padded), context_lens host out [n] (may be NULL).
 * PA_ERR_TABLE_OVERFLOW if a row does not fit. */
pa_status pa_bm_table(const pa_block_manager* bm, int32_t n, const int32_t* seq_handles,
                      int32_t max_blocks_per_seq, int32_t* block_tables, int32_t* context_lens);

/* ------------------------------------------------------------------------------------
 * KV write: [P1] sec. 7 "Fused Reshape and Block Write" and sec. 4 "Decoding Step".
 * Token t (sequence seq_ids[t], position positions[t]) is stored in block
 * block_tables[seq][pos / B] at slot pos % B, for every KV head.
 *   k_src, v_src      [num_tokens, num_kv_heads, head_dim] in src_dtype (PA_F16 / PA_BF16)
 *   k_cache, v_cache  [num_blocks, num_kv_heads, block_size, head_dim] in cache_dtype
 *   block_tables      [num_seqs, max_blocks_per_seq] int32; seq_ids, positions [num_tokens]
 * cache_dtype == src_dtype: the source bits are copied unchanged.
 * cache_dtype == PA_FP8_E4M3: byte = e4m3(float(src) * inv_scale), the product rounded to
 * binary32 and then to E4M3 round-to-nearest-even, saturating at +-448 (NaN stays NaN);
 * [P3] sec. 4: K/V stored in fp8 with per-tensor scales.
 * A token whose sequence id is outside [0, num_seqs), whose position is negative or at or
 * beyond max_blocks_per_seq * block_size, or whose table entry is outside [0, num_blocks),
 * is skipped.  Two tokens naming the same slot race (last writer wins, unordered).
 * Supported: head_dim in {64, 128}, block_size in {8, 16, 32}. */
pa_status pa_write_kv(const void* k_src, const void* v_src, void* k_cache, void* v_cache,
                      const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                      const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                      int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, pa_dtype src_dtype, pa_dtype cache_dtype,
                      float k_inv_scale, float v_inv_scale, void* stream);

/* ------------------------------------------------------------------------------------
 * Batched block copy: [P1] sec. 7 "Batched Block Copy-on-Write" -- all copy-on-write
 * duplications of a step in one launch.  block_pairs: device [num_pairs][2] int32 of
 * (src, dst) physical ids (as produced by pa_bm_append); block dst of both pools receives
 * block src, all KV heads.  Pairs naming an id outside [0, num_blocks) are skipped; a dst
 * that is also a src of the same call races.  Any head_dim/block_size whose block is a
 * multiple of 16 bytes. */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs,
                         int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads,
                         int32_t block_size, int32_t head_dim, pa_dtype cache_dtype,
                         void* stream);

/* Batched move of blocks between two pools (swap-out: device -> host; swap-in: host ->
 * device), [P1] sec. 6.  Pools are [blocks][num_kv_heads][block_size][head_dim] of
 * cache_dtype, K and V each; src_blocks / dst_blocks give their sizes in blocks (the
 * caller guarantees the allocations hold that many).  block_pairs: [num_pairs][2] int32 of
 * (src block, dst block), e.g. from pa_bm_swap_out / pa_bm_swap_in.  Every pointer must be
 * device memory or pinned host memory mapped for the device (hipHostMalloc, torch
 * pin_memory); anything else is refused with PA_ERR_INVALID_ARG before any launch.  One
 * launch moves all pairs; a work-item copies 16 bytes, so host memory is written or read
 * directly over the host link (no staging copy).  Pairs naming an id outside its pool are
 * skipped. */
pa_status pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                         const int32_t* block_pairs, int32_t num_pairs, int32_t src_blocks,
                         int32_t dst_blocks, int32_t num_kv_heads, int32_t block_size,
                         int32_t head_dim, pa_dtype cache_dtype, void* stream);

/* ------------------------------------------------------------------------------------
 * Decode attention.
 * [P1] sec. 3: for sequence s and query head h, with n = context_lens[s],
 *   o = sum_{t<n} softmax_t(scale * q . k_t) v_t,
 * where token t's key/value rows sit in block block_tables[s][t / B], slot t % B, of KV
 * head h / (num_heads / num_kv_heads).  Slots at or beyond n are never read into the
 * arithmetic (the partial-last-block rule of [P1] sec. 3); only table entries
 * j < ceil(n / B) are read ([P2] sec. 2).  n = 0 gives a zero row.
 * The kernel walks the table block by block with the online rescaling of [P1] sec. 7,
 * one pass over K and V ([P3] sec. 3), accumulating in fp32.  Long contexts are cut into
 * partitions of partition_size tokens whose partial (max, sum, output) triples are
 * combined by a second, log-sum-exp merge kernel; with partition_size 0, fp16/bf16 caches
 * and at most 256 sequences the split is instead the flat one pa_decode_plan describes.
 *   out           [num_seqs, num_heads, head_dim] in q_dtype (round to nearest even)
 *   query         [num_seqs, num_heads, head_dim] in q_dtype
 *   k/v_cache     [num_blocks, num_kv_heads, block_size, head_dim] in kv_dtype
 *   block_tables  [num_seqs, max_blocks_per_seq] int32;  context_lens [num_seqs] int32
 *   max_context_len  host upper bound of context_lens (sizes the grid; larger values in
 *                 context_lens are clamped to it and to max_blocks_per_seq * block_size)
 *   k_scale, v_scale  dequantisation scales of an e4m3 cache (value = code * scale);
 *                 ignored for fp16/bf16 caches
 *   partition_size 0 = library choice, else a positive multiple of block_size; a
 *                 partition never spans more than 64 blocks (larger values, and unsplit
 *                 contexts longer than 64 blocks, are cut into 64-block partitions)
 *   flags         0, or PA_DECODE_SHARED_KV when some physical blocks are referenced by
 *                 several sequences of the batch (shared prompts, [P1] sec. 5): K/V loads
 *                 then stay cacheable and sequences are visited together so that a shared
 *                 block is fetched from HBM once; without it K/V loads are streamed with
 *                 the non-temporal hint.  At a given partition_size results are identical
 *                 either way; under the library's choice the flag keeps fixed partitions
 *                 (the flat split does not visit sharing sequences together), so results
 *                 then agree to rounding.
 *   workspace     device scratch of at least pa_decode_workspace_size(...) bytes, 16-byte
 *                 aligned (hipMalloc gives 256); may be NULL when that size is 0.  The
 *                 same holds for every workspace argument below.
 * Supported: head_dim in {64, 128}; block_size in {8, 16, 32}; num_heads / num_kv_heads in
 * {1, 2, 4, 8}; (q, kv) in {(f16, f16), (bf16, bf16), (f16, e4m3), (bf16, e4m3)}. */
#define PA_DECODE_SHARED_KV 1u

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                int32_t partition_size);

/* The split pa_decode (flags 0) will use for these arguments and cache type.  Fixed partitions:
 * used_partition_size tokens each (0 = no split) and num_partitions of them per sequence;
 * *flat_min_blocks = 0.  Flat split (the library's choice for fp16/bf16 caches and at most
 * 256 sequences whose contexts it splits): the blocks of all sequences, one sequence after another, are cut
 * into equal chunks of at least *flat_min_blocks blocks (the length itself is chosen on the
 * device from context_lens, so that every wavefront walks the same number of blocks), and
 * a chunk crossing into the next sequence leaves one partial per sequence; then
 * used_partition_size = 0 and num_partitions is the most partials a row can have.  Any
 * output pointer may be NULL. */
pa_status pa_decode_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t max_context_len,
                         int32_t partition_size, pa_dtype kv_dtype,
                         int32_t* used_partition_size, int32_t* num_partitions,
                         int32_t* flat_min_blocks);

pa_status pa_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                    int32_t num_blocks, int32_t max_context_len, float scale,
                    pa_dtype q_dtype, pa_dtype kv_dtype, float k_scale, float v_scale,
                    int32_t partition_size, uint32_t flags, void* workspace,
                    size_t workspace_bytes, void* stream);

/* No-allocation decode, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Computes what
 * pa_decode computes, with the same arguments minus the workspace, and launches the same
 * kernels: the partition partials go to a fixed device array of PA_NOALLOC_SCRATCH_BYTES
 * bytes inside the library (one copy per GPU, held until the process ends; its address on
 * the current GPU is looked up on the first call there).  The call allocates nothing.  It
 * takes pa_decode's split, bit for bit the same output, except where the flat split's
 * partials would not fit the array: then it takes fixed partitions (the same result to
 * within the decode's tolerance).  A plan whose fixed partitions do not fit either (more
 * than about 64,000 (sequence, query head, partition) triples at head_dim 128) returns
 * PA_ERR_UNSUPPORTED before anything is launched; call pa_decode with a workspace
 * instead.  Every call on a
 * GPU shares that GPU's array, which keeps whatever the last call left there (nothing in
 * it needs to start at zero): calls that overlap on one GPU -- on several streams, or from
 * several host threads -- race on it and must be serialised by the caller.  Errors and
 * support as for pa_decode. */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)
pa_status pa_decode_noalloc(void* out, const void* query, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t max_blocks_per_seq, int32_t num_blocks,
                            int32_t max_context_len, float scale, pa_dtype q_dtype,
                            pa_dtype kv_dtype, float k_scale, float v_scale,
                            int32_t partition_size, uint32_t flags, void* stream);

/* Decode step with the new token written in the same launch: pa_write_kv of one new token
 * per sequence followed by pa_decode ([P1] sec. 4 "Decoding Step": the new token's key and
 * value go to their slot, then every query attends the sequence including it).  The new
 * token of sequence s is at position n - 1 of its length n = context_lens[s] (clamped as
 * pa_decode clamps it); the unit of the decode that walks that block stores the rows first,
 * so results and cache contents equal those of the two calls.
 *   k_new, v_new  device [num_seqs, num_kv_heads, head_dim] in q_dtype: the new rows
 *   k_inv_scale, v_inv_scale  as for pa_write_kv (e4m3 caches: code of x * inv_scale)
 *   Other arguments as for pa_decode; a sequence with n = 0 gets no row and a zero output.
 * A table entry outside [0, num_blocks) for the new token's block skips the write (as
 * pa_write_kv skips it).  Precondition: no other sequence of the batch reads the block the
 * new token goes to (after pa_bm_append's copy-on-write a shared last block has been
 * replaced by a private one); otherwise that sequence may see the block before or after
 * the store.  Same support as pa_decode. */
pa_status pa_decode_append(void* out, const void* query, const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int32_t num_blocks,
                           int32_t max_context_len, float scale, pa_dtype q_dtype,
                           pa_dtype kv_dtype, float k_scale, float v_scale, float k_inv_scale,
                           float v_inv_scale, int32_t partition_size, uint32_t flags,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * Shared-prefix (cascade) decode.  Same result as pa_decode (the attention definition of
 * [P1] sec. 3) for batches in which groups of sequences share their leading blocks: the
 * K samples of one prompt ([P1] sec. 5, parallel sampling) or the sessions behind one
 * pinned system prompt ([P1] sec. 5, prefix sharing).  The shared blocks are read from HBM
 * once per group: prefix units attend the queries of all members to the group's prefix
 * (the member queries become the columns of one matrix-core contraction per block),
 * per-sequence units attend every sequence to its own remaining tokens, and the partial
 * (max, sum, output) triples are combined by the log-sum-exp merge (the rescaling of [P1]
 * sec. 7).  The two kinds of unit run as two launches, or as one (prefix units' workgroups
 * first) for an e4m3 cache with num_heads == num_kv_heads; the merge is one more launch.
 *   Arguments as for pa_decode, plus:
 *   seq_group      sequences per group; the batch is num_seqs / seq_group groups of
 *                  consecutive sequences (group g = sequences g*seq_group .. +seq_group-1)
 *   prefix_blocks  device [num_seqs / seq_group] int32: blocks shared by the group's
 *                  members (may be NULL when max_prefix_blocks is 0: nothing is shared
 *                  and no launch reads it).  Precondition: the first prefix_blocks[g] entries of the
 *                  members' table rows are the same physical ids; the prefix units read
 *                  the first member's row only, so a violation gives that member's blocks
 *                  to every member (wrong numbers, no fault).  Values are clamped to
 *                  [0, max_prefix_blocks]; a member shorter than the prefix attends its
 *                  own n tokens of it, so any value gives the pa_decode result when the
 *                  precondition holds.
 *   max_prefix_blocks  host upper bound of prefix_blocks (sizes the prefix grid)
 *   flags          0, or PA_DECODE_SHARED_KV when blocks after the group prefixes are still
 *                  shared (e.g. between beams): the per-sequence units then keep their K/V
 *                  loads cacheable.  The prefix units always stream (they read each shared
 *                  block once).  Results are identical either way.
 *   partition_size 0 = library choice: prefix partitions of a planned size, and each
 *                  row's own blocks split into equal shares (at least 8 blocks each);
 *                  else a positive multiple of block_size used by both kinds of unit
 *   workspace      at least pa_decode_shared_prefix_workspace_size(...) bytes (never 0
 *                  for num_seqs > 0: both kinds of unit always leave partials)
 * Supported: what the matrix-core decode covers for the group's queries: block_size 16,
 * head_dim in {64, 128}, (num_heads / num_kv_heads) * seq_group in {2, 4, 8, 16}, q in
 * {f16, bf16} with a cache of the same type or e4m3; the per-sequence units then follow
 * pa_decode's support.  Other shapes return PA_ERR_UNSUPPORTED (use pa_decode). */
size_t pa_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t block_size, int32_t max_context_len,
                                              int32_t max_prefix_blocks,
                                              int32_t partition_size);

/* The plan pa_decode_shared_prefix makes for these arguments and a cache of kv_dtype (host
 * only, nothing launched): the partition length of the prefix units (tokens), the partial
 * slots per row that the prefix units and the per-sequence units own (prefix_slots +
 * suffix_slots in all, the merge's input), the shortest share of a row's own blocks in the
 * per-sequence units (0 = fixed partitions of prefix_partition_size tokens instead of equal
 * shares), and the decode launches before the merge (1: both kinds of unit in one launch,
 * e4m3 caches with num_heads == num_kv_heads and a prefix to share; else 2, or 1 when
 * max_prefix_blocks is 0).  Any output pointer may be NULL. */
pa_status pa_decode_shared_prefix_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size,
                                       int32_t max_context_len, int32_t max_prefix_blocks,
                                       int32_t partition_size, pa_dtype kv_dtype,
                                       int32_t* prefix_partition_size, int32_t* prefix_slots,
                                       int32_t* suffix_slots, int32_t* suffix_min_blocks,
                                       int32_t* decode_launches);

pa_status pa_decode_shared_prefix(void* out, const void* query, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* prefix_blocks,
                                  int32_t num_seqs, int32_t seq_group, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, int32_t num_blocks,
                                  int32_t max_context_len, int32_t max_prefix_blocks,
                                  float scale, pa_dtype q_dtype, pa_dtype kv_dtype,
                                  float k_scale, float v_scale, int32_t partition_size,
                                  uint32_t flags, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* ------------------------------------------------------------------------------------
 * Multi-token decode: query_len > 1 query tokens per sequence, as when a draft of several
 * tokens (a chain or a tree, [P1] sec. 9 speculative decoding trees) is verified in one
 * pass.  The query tokens of sequence s are its last query_len positions, whose K/V rows
 * are already in the cache (n = context_lens[s] counts them).  Query token t attends
 * every position before n - query_len and the draft position n - query_len + u when bit
 * u of its mask is set; with tree_masks == NULL the mask is causal (bits 0..t).  Each
 * (s, t, h) output row is the [P1] sec. 3 softmax-weighted sum over its visible
 * positions; a row with no visible position is zero.
 *   out, query     [num_seqs, query_len, num_heads, head_dim] in q_dtype
 *   tree_masks     device [num_seqs, query_len] uint32, or NULL (causal)
 *   Other arguments, planning, flags and the workspace as for pa_decode (the workspace
 *   holds partials for num_seqs * query_len * num_heads rows).
 * One matrix-core tile holds the query_len * (num_heads / num_kv_heads) query columns of
 * a KV head, so each K/V tile is read once for all draft tokens.
 * Supported: block_size 16, head_dim in {64, 128}, query_len * (num_heads / num_kv_heads)
 * in {2, 4, 8, 16}, q in {f16, bf16} with a cache of the same type or e4m3. */
size_t pa_decode_multi_workspace_size(int32_t num_seqs, int32_t query_len, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int32_t max_context_len, int32_t partition_size);

pa_status pa_decode_multi(void* out, const void* query, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const uint32_t* tree_masks, int32_t num_seqs, int32_t query_len,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                          int32_t max_context_len, float scale, pa_dtype q_dtype,
                          pa_dtype kv_dtype, float k_scale, float v_scale,
                          int32_t partition_size, uint32_t flags, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * Footprint: [P1] sec. 1 "KV Cache Memory Footprint" — a token stores one key and one
 * value vector per layer, so it costs 2 * num_layers * num_kv_heads * head_dim * e bytes
 * (e = 2 for fp16/bf16, 1 for e4m3); with fp16 and num_kv_heads * head_dim = d_model this
 * is the page's 4 * L * d_model.  Returns 0 for a bad dtype or negative size. */
uint64_t pa_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                               pa_dtype kv_dtype);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
