// Internal interface between the C ABI (capi.cpp) and the decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Block ids of one context partition are staged in LDS; a partition may span
// at most this many blocks.
constexpr int kBtLds = 1024;
// A decode workgroup has one wave of 64 lanes per kv head of its group, at
// most this many.
constexpr int kMaxDecodeWaves = 8;
constexpr int kMaxDecodeThreads = kMaxDecodeWaves * 64;

struct DecodeParams {
    const void *query;          // [S, Hq, D]
    const char *key_cache;      // [num_blocks, bs, Hkv, D]
    const char *value_cache;    // [num_blocks, bs, Hkv, D]
    const int32_t *block_tables;  // [S, max_blocks_per_seq]
    const int32_t *context_lens;  // [S]
    void *out;                  // [S, Hq, D]
    float *part_max;            // [S, Hq, P_max]   running max (log2 domain)
    float *part_sum;            // [S, Hq, P_max]   running sum
    float *part_out;            // [S, Hq, P_max, D] unnormalised output
    float scale_log2;           // scale * log2(e)
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int block_size;
    int block_shift;            // log2(block_size)
    int num_blocks;
    int max_blocks_per_seq;
    int max_context_len;        // every valid context_len is <= this
    int partition_size;         // tokens per partition
    int num_partitions;         // P_max = ceil(max_context_len / partition_size)
    int heads_per_group;        // kv heads (= waves) per workgroup
    int num_head_groups;        // num_kv_heads / heads_per_group
    int64_t block_stride_bytes; // bs * Hkv * D * elem bytes
    int row_stride_bytes;       // Hkv * D * elem bytes
};

// dtype codes match paged_kv_dtype; kernel = 0 VALU, 1 MFMA.
hipError_t launch_decode(const DecodeParams &p, int dtype, int head_dim, int group, int kernel,
                         hipStream_t stream);
// Compute units of the current device and decode workgroups of this shape
// one of them holds at once; 0 where unknown (no device).
struct DeviceOccupancy {
    int compute_units;
    int workgroups_per_cu;
};
DeviceOccupancy decode_occupancy(int dtype, int head_dim, int group, int block_size,
                                 int heads_per_group);
// Which decode kernel launch_decode uses for this shape.
int decode_kernel_choice(int dtype, int head_dim, int group);

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
