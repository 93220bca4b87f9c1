// Internal interface between the C ABI (capi.cpp) and the prefix-cache
// kernels (prefix_cache.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Chained full-block hashes of a batch of token sequences; mul_block is
// base^block_size mod 2^61 - 1.
hipError_t launch_prefix_hash(const int32_t *tokens, const int32_t *token_start,
                              const int32_t *block_start, int num_seqs, int total_tokens,
                              int total_blocks, int block_size, uint64_t seed, uint64_t base,
                              uint64_t mul_block, uint64_t *block_hashes, hipStream_t stream);
hipError_t launch_prefix_insert(const uint64_t *hashes, const int32_t *blocks, int n,
                                uint64_t *table_keys, int32_t *table_blocks, int capacity_log2,
                                int32_t *stored, hipStream_t stream);
hipError_t launch_prefix_match(const uint64_t *block_hashes, const int32_t *block_start,
                               int num_seqs, int total_blocks, const uint64_t *table_keys,
                               const int32_t *table_blocks, int capacity_log2,
                               int32_t *matched_blocks, int32_t *matched_len,
                               hipStream_t stream);

}  // namespace pkv
