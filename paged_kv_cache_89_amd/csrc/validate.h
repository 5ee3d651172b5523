// Validation mode: host-side checks of the index data the device operations read.  Each
// check copies that data to the host on `stream`, synchronises, and returns false with a
// message naming the first violation.
#pragma once

#include <stdint.h>

#include <string>

namespace pa {

bool validate_enabled();
int set_validate(int on);  // returns the previous setting

// context_lens in [min_len, max_context_len] and within max_blocks * block_size; table
// entries j < ceil(n / block_size) in [0, num_blocks)
bool validate_decode(const char* who, const int32_t* tables, const int32_t* ctx, int32_t num_seqs,
                     int32_t max_blocks, int32_t num_blocks, int32_t block_size,
                     int32_t max_context_len, int32_t min_len, void* stream, std::string* err);
// the block each sequence's new token goes to (entry (n - 1) / block_size, n > 0) is named
// by no other table entry that the decode reads, of this or another sequence
bool validate_append_blocks(const char* who, const int32_t* tables, const int32_t* ctx,
                            int32_t num_seqs, int32_t max_blocks, int32_t num_blocks,
                            int32_t block_size, void* stream, std::string* err);
// prefix_blocks[g] in [0, max_prefix_blocks]; the group's shared entries (first member's
// row) in range; every member's entries inside the prefix equal to the first member's
bool validate_prefix(const char* who, const int32_t* tables, const int32_t* ctx,
                     const int32_t* prefix_blocks, int32_t num_seqs, int32_t seq_group,
                     int32_t max_blocks, int32_t num_blocks, int32_t block_size,
                     int32_t max_prefix_blocks, void* stream, std::string* err);
// seq_ids, positions and the table entries they name in range; no slot written twice
bool validate_write(const int32_t* tables, const int32_t* seq_ids, const int32_t* positions,
                    int32_t num_seqs, int32_t max_blocks, int32_t num_tokens, int32_t num_blocks,
                    int32_t block_size, void* stream, std::string* err);
// block pairs in range; no destination twice; within one pool, no destination that is
// also a source
bool validate_pairs(const char* who, const int32_t* pairs, int32_t num_pairs, int32_t src_blocks,
                    int32_t dst_blocks, bool same_pool, void* stream, std::string* err);

}  // namespace pa
