// Internal interface between the C ABI (capi.cpp) and the multi-token
// (chunked-prefill) attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct PrefillParams {
    const void *query;            // [total_q, Hq, D]
    const char *key_cache;        // [num_blocks, bs, Hkv, D]
    const char *value_cache;      // [num_blocks, bs, Hkv, D]
    const int32_t *block_tables;  // [S, max_blocks_per_seq]
    const int32_t *context_lens;  // [S]
    const int32_t *query_start;   // [S + 1]
    void *out;                    // [total_q, Hq, D]
    float score_scale;            // |scale| * log2(e)
    int negate_query;             // scale < 0: the query enters with its sign flipped
    int num_seqs;
    int total_q;
    int num_q_heads;
    int num_kv_heads;
    int group;                    // num_q_heads / num_kv_heads
    int block_size;
    int block_shift;              // log2(block_size)
    int num_blocks;
    int max_blocks_per_seq;
    int max_query_len;            // rows of a sequence beyond this are not computed
    int max_context_len;          // every valid context_len is <= this
    int row_blocks;               // ceil(max_query_len * group / rows per workgroup)
    int64_t block_stride_bytes;   // bs * Hkv * D * elem bytes
    int row_stride_bytes;         // Hkv * D * elem bytes
    // Shared-prefix pass only (launch_shared_prefix): the rows are the
    // decode batch's (sequence, query head) pairs, query [num_seqs, Hq, D];
    // positions [0, prefix_len) are read through block_tables' first row,
    // in prefix_parts partitions of prefix_part positions; partition q of
    // row (s, h) leaves its running max, sum and unnormalised output in slot
    // (s * Hq + h) * num_slots + q of the decode's split scratch.
    int prefix_len;
    int prefix_part;
    int prefix_parts;
    int num_slots;
    float *part_max;
    float *part_sum;
    float *part_out;
};

// Query rows (new token, query head) one prefill workgroup covers.
int prefill_rows_per_block(int head_dim);
int prefill_f32_rows_per_block();
// dtype codes match paged_kv_dtype: the 16-bit kernel (f16, bf16) ...
hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_dim, hipStream_t stream);
// ... and the fp32 kernel.
hipError_t launch_prefill_f32(const PrefillParams &p, int head_dim, hipStream_t stream);
// The shared-prefix pass of the shared-prefix decode on the prefill
// kernels: grid num_kv_heads * row_blocks * prefix_parts (rows per block:
// prefill_rows_per_block, for fp32 prefill_f32_rows_per_block).
hipError_t launch_shared_prefix(const PrefillParams &p, int dtype, int head_dim,
                                hipStream_t stream);
hipError_t launch_shared_prefix_f32(const PrefillParams &p, int head_dim, hipStream_t stream);

}  // namespace pkv
