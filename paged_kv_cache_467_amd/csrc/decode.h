// Internal interface between the C ABI (capi.cpp) and the decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Block ids of one context partition are staged in LDS; a partition may span
// at most this many blocks.
constexpr int kBtLds = 1024;
// A decode workgroup has one wave of 64 lanes per kv head of its group, at
// most this many.
constexpr int kMaxDecodeWaves = 8;
constexpr int kMaxDecodeThreads = kMaxDecodeWaves * 64;
// Balanced split: every workgroup keeps the padded start of every sequence
// in LDS, so a batch may hold at most this many sequences.
constexpr int kBalancedMaxSeqs = 1024;

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
    // Balanced split (num_chunks > 0): the positions of all sequences, each
    // padded to a multiple of 16, end to end, cut into num_chunks chunks of
    // equal size; partition_size and num_partitions are then unused, and
    // the partials are indexed by chunk (two slots per chunk).
    int num_chunks;
    // Shared-prefix decode (0 and 0 otherwise): every sequence's positions
    // [0, prefix_len) were computed by the shared-prefix pass into partial
    // slots [0, prefix_parts); this launch covers [prefix_len, L) in
    // partitions of partition_size, partition q in slot prefix_parts + q.
    int prefix_len;
    int prefix_parts;
    int heads_per_group;        // kv heads (= waves) per workgroup
    int num_head_groups;        // num_kv_heads / heads_per_group
    int64_t block_stride_bytes; // bs * Hkv * D * elem bytes
    int row_stride_bytes;       // Hkv * D * elem bytes
    // Fused KV write (null new_key: none): sequence s's new token's rows
    // new_key/new_value [S, Hkv, D] go to pool cell slot_mapping[s], and the
    // sequence's attention sees them at position L - 1 (the VALU kernel
    // stores them before reading its history; the MFMA kernel's fused
    // instance reads them from new_key/new_value and stores them after).
    const char *new_key;
    const char *new_value;
    const int32_t *slot_mapping;
    int64_t num_slots;          // num_blocks * block_size
    // Multi-token decode (launch_decode_multiquery only; null otherwise):
    // sequence s's new tokens are query rows query_start[s] ..
    // query_start[s + 1] - 1 (at most max_query_len of them), token i seeing
    // positions 0 .. L - q_len + i; mq_group = num_q_heads / num_kv_heads.
    const int32_t *query_start;
    int total_q;                // query rows in all
    int max_query_len;
    int mq_group;
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
// The multi-token decode: paged_attn_prefill's computation for a batch with
// max_query_len * group <= 32 and no split, on the decode MFMA kernel (one
// wave per kv head, the (new token, query head) rows of the kv head in one
// or two 16-row tiles).  16-bit types only.
hipError_t launch_decode_multiquery(const DecodeParams &p, int dtype, int head_dim,
                                    hipStream_t stream);
constexpr int kMultiQueryRows = 16;
// Which decode kernel launch_decode uses for this shape.
int decode_kernel_choice(int dtype, int head_dim, int group);

// Host-side plan of one decode launch (decode_plan.cpp): status, the
// context bound, the partition size and count, and kv heads per workgroup.
struct DecodePlan {
    int status;
    int max_context_len;
    int partition_size;
    int num_partitions;
    int heads_per_group;  // kv heads per decode workgroup (one wave each)
    int num_chunks;       // > 0: balanced split into this many chunks
};
DecodePlan plan_decode(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       int block_size, int max_blocks_per_seq, int max_context_len,
                       int partition_size, int dtype);
// Host-side plan of the shared-prefix decode (decode_plan.cpp).  With
// prefix_len 0 it is paged_attn_decode's plan (suffix, prefix_parts 0).
struct SharedPrefixPlan {
    int status;
    DecodePlan suffix;  // the per-sequence pass over [prefix_len, L): its
                        // partition size and heads per group; num_partitions
                        // counts every partial slot (prefix and suffix)
    int prefix_len;
    int prefix_part;    // positions per prefix partition
    int prefix_parts;   // prefix partitions (0: plain decode)
    int row_blocks;     // workgroups of (sequence, query head) rows per kv head
    size_t workspace_bytes;
};
SharedPrefixPlan plan_shared_prefix(int num_seqs, int num_q_heads, int num_kv_heads,
                                    int head_dim, int block_size, int max_blocks_per_seq,
                                    int max_context_len, int prefix_len,
                                    int prefix_partition_size, int partition_size, int dtype);
// Floats per partition in each split-scratch array (rounded for alignment),
// and the workspace bytes the plan needs (0 without a split).
int plan_partition_for_lengths(const int32_t *lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_dim, int block_size,
                               int max_blocks_per_seq, int dtype);
size_t decode_partial_floats(int num_seqs, int num_q_heads);
// Entries of each split-scratch array (running max, running sum; the
// output array holds head_dim times as many).
size_t decode_partial_slots(const DecodePlan &pl, int num_seqs, int num_q_heads);
size_t decode_workspace_bytes(const DecodePlan &pl, int num_seqs, int num_q_heads, int head_dim);

// The decode entry points' common path (capi.cpp): host checks, then the
// launch; with new_key non-null the launch also stores the new tokens (the
// fused KV write, in the same kernels).  With
// static_scratch the split's scratch is noalloc_scratch() (workspace and
// workspace_bytes are ignored) and a split that needs more than it holds
// returns PAGED_KV_ERR_SCRATCH_LIMIT.  Returns a paged_kv_status.
int run_decode(const void *query, const void *new_key, const void *new_value,
               const int32_t *slot_mapping, const void *key_cache, const void *value_cache,
               const int32_t *block_tables, const int32_t *context_lens, float scale, void *out,
               int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
               int num_blocks, int max_blocks_per_seq, int max_context_len, int partition_size,
               int dtype, void *workspace, size_t workspace_bytes, void *stream,
               bool static_scratch);
// Device address of the current device's copy of the library's static
// scratch (PAGED_KV_NOALLOC_SCRATCH_BYTES bytes, decode_noalloc.hip), looked
// up on the first call on each device; nullptr if the runtime fails.
void *noalloc_scratch();

}  // namespace pkv
