// Internal interface between the C ABI (capi.cpp) and the KV cache bit-copy
// kernels (kv_cache_ops.hip): the write, the gather and the block copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

hipError_t launch_kv_cache_write(const void *key, const void *value, const int32_t *slot_mapping,
                                 void *key_cache, void *value_cache, int num_tokens,
                                 int row_bytes, int64_t num_slots, hipStream_t stream);

// Block copy from a source pool pair into a destination pool pair (the
// same pair for copy-on-write; device and host pools for a swap).
hipError_t launch_copy_blocks(const void *src_key, const void *src_value, int num_src_blocks,
                              void *dst_key, void *dst_value, int num_dst_blocks,
                              const int32_t *block_mapping, int num_pairs, int64_t block_bytes,
                              hipStream_t stream);

hipError_t launch_paged_kv_gather(const void *key_cache, const void *value_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  void *out_key, void *out_value, int num_seqs,
                                  int max_blocks_per_seq, int block_size, int num_blocks,
                                  int max_context_len, int row_bytes, int elem_bytes,
                                  hipStream_t stream);

}  // namespace pkv
