// C ABI of the paged-KV library: host-side argument checks and kernel
// launches on the caller's stream (the decode's partition choice and
// workspace sizing are in decode_plan.cpp).  Nothing here reads device
// memory or allocates.

#include "../../include/paged_kv.h"

#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "decode.h"
#include "kv_ops.h"
#include "prefill.h"
#include "prefix_cache.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}
int elem_bytes(int dtype) { return dtype == PAGED_KV_F32 ? 4 : 2; }

}  // namespace

extern "C" {

const char *paged_kv_status_string(int status) {
    switch (status) {
        case PAGED_KV_OK: return "ok";
        case PAGED_KV_ERR_NULL_POINTER: return "null pointer";
        case PAGED_KV_ERR_BAD_SHAPE: return "bad shape, size or alignment";
        case PAGED_KV_ERR_UNSUPPORTED: return "unsupported dtype or shape";
        case PAGED_KV_ERR_WORKSPACE: return "workspace missing or too small";
        case PAGED_KV_ERR_HIP: return "HIP runtime error";
        case PAGED_KV_ERR_HOST_MEMORY: return "host buffer is not pinned, device-mapped memory";
        case PAGED_KV_ERR_SCRATCH_LIMIT:
            return "the split needs more scratch than the library's static buffer holds";
        default: return "unknown status";
    }
}

int paged_attn_decode_partition_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                     int head_dim, int block_size, int max_blocks_per_seq,
                                     int max_context_len, int partition_size, int dtype) {
    const pkv::DecodePlan pl = pkv::plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, max_context_len, partition_size, dtype);
    return pl.status == PAGED_KV_OK ? pl.partition_size : -pl.status;
}

int paged_attn_decode_partition_size_for_lengths(const int32_t *host_context_lens,
                                                 int num_seqs, int num_q_heads,
                                                 int num_kv_heads, int head_dim, int block_size,
                                                 int max_blocks_per_seq, int dtype) {
    if (num_seqs < 0) return -PAGED_KV_ERR_BAD_SHAPE;
    if (num_seqs > 0 && !host_context_lens) return -PAGED_KV_ERR_NULL_POINTER;
    return pkv::plan_partition_for_lengths(host_context_lens, num_seqs, num_q_heads,
                                           num_kv_heads, head_dim, block_size,
                                           max_blocks_per_seq, dtype);
}

size_t paged_attn_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                         int head_dim, int block_size, int max_blocks_per_seq,
                                         int max_context_len, int partition_size, int dtype) {
    const pkv::DecodePlan pl = pkv::plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, max_context_len, partition_size, dtype);
    if (pl.status != PAGED_KV_OK) return (size_t)-1;
    return pkv::decode_workspace_bytes(pl, num_seqs, num_q_heads, head_dim);
}

}  // extern "C"

namespace pkv {
namespace {

// Pointer and value checks common to the decode entry points.
int check_decode_args(const void *query, const void *key_cache, const void *value_cache,
                      const int32_t *block_tables, const int32_t *context_lens, float scale,
                      const void *out, int num_blocks) {
    if (num_blocks < 1 || !isfinite(scale)) return PAGED_KV_ERR_BAD_SHAPE;
    if (!query || !key_cache || !value_cache || !block_tables || !context_lens || !out)
        return PAGED_KV_ERR_NULL_POINTER;
    if (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
        !aligned16(out) || !aligned4(block_tables) || !aligned4(context_lens))
        return PAGED_KV_ERR_BAD_SHAPE;
    return PAGED_KV_OK;
}

// The decode kernels' parameters for plan pl (no fused write, no shared
// prefix); ws holds nph entries per partial array.
DecodeParams decode_params(const void *query, const void *key_cache, const void *value_cache,
                           const int32_t *block_tables, const int32_t *context_lens, float scale,
                           void *out, int num_seqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                           const DecodePlan &pl, float *ws, size_t nph, int dtype) {
    const int e = elem_bytes(dtype);
    DecodeParams p;
    p.query = query;
    p.key_cache = static_cast<const char *>(key_cache);
    p.value_cache = static_cast<const char *>(value_cache);
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.out = out;
    p.part_max = ws;
    p.part_sum = ws ? ws + nph : nullptr;
    p.part_out = ws ? ws + 2 * nph : nullptr;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);  // scale * log2(e)
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.block_size = block_size;
    p.block_shift = log2i(block_size);
    p.num_blocks = num_blocks;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.max_context_len = pl.max_context_len;
    p.partition_size = pl.partition_size;
    p.num_partitions = pl.num_partitions;
    p.num_chunks = pl.num_chunks;
    p.prefix_len = 0;
    p.prefix_parts = 0;
    p.heads_per_group = pl.heads_per_group;
    p.num_head_groups = num_kv_heads / pl.heads_per_group;
    p.row_stride_bytes = num_kv_heads * head_dim * e;
    p.block_stride_bytes = (int64_t)block_size * p.row_stride_bytes;
    p.new_key = nullptr;
    p.new_value = nullptr;
    p.slot_mapping = nullptr;
    p.num_slots = (int64_t)num_blocks * block_size;
    p.query_start = nullptr;
    p.total_q = 0;
    p.max_query_len = 0;
    p.mq_group = 0;
    return p;
}

}  // namespace

// The decode, with (new_key non-null) or without the fused KV write; with
// static_scratch the split's scratch is the library's own buffer
// (decode_noalloc.hip) instead of the caller's workspace.
int run_decode(const void *query, const void *new_key, const void *new_value,
               const int32_t *slot_mapping, const void *key_cache, const void *value_cache,
               const int32_t *block_tables, const int32_t *context_lens, float scale, void *out,
               int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
               int num_blocks, int max_blocks_per_seq, int max_context_len, int partition_size,
               int dtype, void *workspace, size_t workspace_bytes, void *stream,
               bool static_scratch) {
    const pkv::DecodePlan pl = pkv::plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, max_context_len, partition_size, dtype);
    if (pl.status != PAGED_KV_OK) return pl.status;
    if (num_blocks < 1 || !isfinite(scale)) return PAGED_KV_ERR_BAD_SHAPE;
    if (num_seqs == 0) return PAGED_KV_OK;
    const int chk = check_decode_args(query, key_cache, value_cache, block_tables, context_lens,
                                      scale, out, num_blocks);
    if (chk != PAGED_KV_OK) return chk;
    if (new_key && (!new_value || !slot_mapping)) return PAGED_KV_ERR_NULL_POINTER;
    if (new_key && pl.num_chunks > 0) return PAGED_KV_ERR_UNSUPPORTED;
    if (new_key && (!aligned16(new_key) || !aligned16(new_value) || !aligned4(slot_mapping)))
        return PAGED_KV_ERR_BAD_SHAPE;
    const int e = elem_bytes(dtype);
    // The kernels address a block's rows with 32-bit offsets.
    if ((int64_t)block_size * num_kv_heads * head_dim * e > INT_MAX) return PAGED_KV_ERR_BAD_SHAPE;
    const size_t need = pkv::decode_workspace_bytes(pl, num_seqs, num_q_heads, head_dim);
    if (static_scratch) {
        if (need > PAGED_KV_NOALLOC_SCRATCH_BYTES) return PAGED_KV_ERR_SCRATCH_LIMIT;
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0) {
            workspace = noalloc_scratch();
            if (!workspace) return PAGED_KV_ERR_HIP;
            workspace_bytes = PAGED_KV_NOALLOC_SCRATCH_BYTES;
        }
    }
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return PAGED_KV_ERR_WORKSPACE;

    const size_t nph = pkv::decode_partial_slots(pl, num_seqs, num_q_heads);
    pkv::DecodeParams p = decode_params(
        query, key_cache, value_cache, block_tables, context_lens, scale, out, num_seqs,
        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, pl,
        need ? static_cast<float *>(workspace) : nullptr, nph, dtype);
    p.new_key = static_cast<const char *>(new_key);
    p.new_value = static_cast<const char *>(new_value);
    p.slot_mapping = slot_mapping;

    const int group = num_q_heads / num_kv_heads;
    const int kernel = pkv::decode_kernel_choice(dtype, head_dim, group);
    const hipError_t err = pkv::launch_decode(p, dtype, head_dim, group, kernel,
                                              static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PAGED_KV_OK : PAGED_KV_ERR_HIP;
}

// The shared-prefix decode: the prefix pass (the prefill kernel over the
// shared blocks, all sequences' query rows at once), then the decode
// kernels over each sequence's positions after the prefix, then the merge.
int run_shared_prefix_decode(const void *query, const void *key_cache, const void *value_cache,
                             const int32_t *block_tables, const int32_t *context_lens,
                             float scale, void *out, int num_seqs, int num_q_heads,
                             int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             int max_blocks_per_seq, int max_context_len, int prefix_len,
                             int prefix_partition_size, int partition_size, int dtype,
                             void *workspace, size_t workspace_bytes, void *stream) {
    const SharedPrefixPlan sp = plan_shared_prefix(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
        max_context_len, prefix_len, prefix_partition_size, partition_size, dtype);
    if (sp.status != PAGED_KV_OK) return sp.status;
    if (sp.prefix_parts == 0)
        return run_decode(query, nullptr, nullptr, nullptr, key_cache, value_cache, block_tables,
                          context_lens, scale, out, num_seqs, num_q_heads, num_kv_heads,
                          head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                          partition_size, dtype, workspace, workspace_bytes, stream, false);
    if (num_blocks < 1 || !isfinite(scale)) return PAGED_KV_ERR_BAD_SHAPE;
    if (num_seqs == 0) return PAGED_KV_OK;
    const int chk = check_decode_args(query, key_cache, value_cache, block_tables, context_lens,
                                      scale, out, num_blocks);
    if (chk != PAGED_KV_OK) return chk;
    const int e = elem_bytes(dtype);
    if ((int64_t)block_size * num_kv_heads * head_dim * e > INT_MAX) return PAGED_KV_ERR_BAD_SHAPE;
    if (!workspace || workspace_bytes < sp.workspace_bytes || !aligned16(workspace))
        return PAGED_KV_ERR_WORKSPACE;

    const size_t nph = decode_partial_floats(num_seqs, num_q_heads) * sp.suffix.num_partitions;
    float *ws = static_cast<float *>(workspace);
    DecodeParams p = decode_params(query, key_cache, value_cache, block_tables, context_lens,
                                   scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                   block_size, num_blocks, max_blocks_per_seq, sp.suffix, ws,
                                   nph, dtype);
    p.prefix_len = sp.prefix_len;
    p.prefix_parts = sp.prefix_parts;

    PrefillParams q{};
    q.query = query;
    q.key_cache = p.key_cache;
    q.value_cache = p.value_cache;
    q.block_tables = block_tables;
    q.context_lens = context_lens;
    q.score_scale = (float)(fabs((double)scale) * 1.4426950408889634);
    q.negate_query = scale < 0.0f;
    q.num_seqs = num_seqs;
    q.num_q_heads = num_q_heads;
    q.num_kv_heads = num_kv_heads;
    q.group = num_q_heads / num_kv_heads;
    q.block_size = block_size;
    q.block_shift = p.block_shift;
    q.num_blocks = num_blocks;
    q.max_blocks_per_seq = max_blocks_per_seq;
    q.max_context_len = sp.suffix.max_context_len;
    q.row_blocks = sp.row_blocks;
    q.block_stride_bytes = p.block_stride_bytes;
    q.row_stride_bytes = p.row_stride_bytes;
    q.prefix_len = sp.prefix_len;
    q.prefix_part = sp.prefix_part;
    q.prefix_parts = sp.prefix_parts;
    q.num_slots = sp.suffix.num_partitions;
    q.part_max = p.part_max;
    q.part_sum = p.part_sum;
    q.part_out = p.part_out;

    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t err = dtype == PAGED_KV_F32 ? launch_shared_prefix_f32(q, head_dim, st)
                                           : launch_shared_prefix(q, dtype, head_dim, st);
    if (err != hipSuccess) return PAGED_KV_ERR_HIP;
    const int group = num_q_heads / num_kv_heads;
    err = launch_decode(p, dtype, head_dim, group, decode_kernel_choice(dtype, head_dim, group), st);
    return err == hipSuccess ? PAGED_KV_OK : PAGED_KV_ERR_HIP;
}

}  // namespace pkv

extern "C" {

int paged_attn_decode_shared_prefix(const void *query, const void *key_cache,
                                    const void *value_cache, const int32_t *block_tables,
                                    const int32_t *context_lens, float scale, void *out,
                                    int num_seqs, int num_q_heads, int num_kv_heads,
                                    int head_dim, int block_size, int num_blocks,
                                    int max_blocks_per_seq, int max_context_len, int prefix_len,
                                    int prefix_partition_size, int partition_size, int dtype,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    return pkv::run_shared_prefix_decode(
        query, key_cache, value_cache, block_tables, context_lens, scale, out, num_seqs,
        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
        max_context_len, prefix_len, prefix_partition_size, partition_size, dtype, workspace,
        workspace_bytes, stream);
}

size_t paged_attn_decode_shared_prefix_workspace_bytes(
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
    int max_blocks_per_seq, int max_context_len, int prefix_len, int prefix_partition_size,
    int partition_size, int dtype) {
    const pkv::SharedPrefixPlan sp = pkv::plan_shared_prefix(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
        max_context_len, prefix_len, prefix_partition_size, partition_size, dtype);
    return sp.status == PAGED_KV_OK ? sp.workspace_bytes : (size_t)-1;
}

int paged_attn_decode(const void *query, const void *key_cache, const void *value_cache,
                      const int32_t *block_tables, const int32_t *context_lens, float scale,
                      void *out, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, int max_blocks_per_seq,
                      int max_context_len, int partition_size, int dtype, void *workspace,
                      size_t workspace_bytes, void *stream) {
    return pkv::run_decode(query, nullptr, nullptr, nullptr, key_cache, value_cache,
                           block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                           num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                           max_context_len, partition_size, dtype, workspace, workspace_bytes,
                           stream, false);
}

int paged_attn_decode_write(const void *query, const void *new_key, const void *new_value,
                            const int32_t *slot_mapping, void *key_cache, void *value_cache,
                            const int32_t *block_tables, const int32_t *context_lens,
                            float scale, void *out, int num_seqs, int num_q_heads,
                            int num_kv_heads, int head_dim, int block_size, int num_blocks,
                            int max_blocks_per_seq, int max_context_len, int partition_size,
                            int dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (num_seqs > 0 && (!new_key || !new_value || !slot_mapping))
        return PAGED_KV_ERR_NULL_POINTER;
    return pkv::run_decode(query, new_key, new_value, slot_mapping, key_cache, value_cache,
                           block_tables, context_lens, scale, out, num_seqs, num_q_heads,
                           num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                           max_context_len, partition_size, dtype, workspace, workspace_bytes,
                           stream, false);
}

int kv_cache_write(const void *key, const void *value, const int32_t *slot_mapping,
                   void *key_cache, void *value_cache, int num_tokens, int num_kv_heads,
                   int head_dim, int block_size, int num_blocks, int dtype, void *stream) {
    if (dtype != PAGED_KV_F32 && dtype != PAGED_KV_F16 && dtype != PAGED_KV_BF16)
        return PAGED_KV_ERR_UNSUPPORTED;
    if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
        return PAGED_KV_ERR_BAD_SHAPE;
    const int64_t row = (int64_t)num_kv_heads * head_dim * elem_bytes(dtype);
    if (row % 16 != 0 || row > INT_MAX) return PAGED_KV_ERR_BAD_SHAPE;
    if (num_tokens == 0) return PAGED_KV_OK;
    if (!key || !value || !slot_mapping || !key_cache || !value_cache)
        return PAGED_KV_ERR_NULL_POINTER;
    if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) ||
        !aligned16(value_cache) || !aligned4(slot_mapping))
        return PAGED_KV_ERR_BAD_SHAPE;
    const hipError_t err =
        pkv::launch_kv_cache_write(key, value, slot_mapping, key_cache, value_cache, num_tokens,
                                   (int)row, (int64_t)num_blocks * block_size,
                                   static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PAGED_KV_OK : PAGED_KV_ERR_HIP;
}

int paged_attn_prefill(const void *query, const void *key_cache, const void *value_cache,
                       const int32_t *block_tables, const int32_t *context_lens,
                       const int32_t *query_start, float scale, void *out, int num_seqs,
                       int total_q, int num_q_heads, int num_kv_heads, int head_dim,
                       int block_size, int num_blocks, int max_blocks_per_seq,
                       int max_query_len, int max_context_len, int dtype, void *stream) {
    if (dtype != PAGED_KV_F32 && dtype != PAGED_KV_F16 && dtype != PAGED_KV_BF16)
        return PAGED_KV_ERR_UNSUPPORTED;
    if (num_seqs < 0 || total_q < 0 || num_q_heads < 1 || num_kv_heads < 1 ||
        num_q_heads % num_kv_heads != 0 || num_blocks < 1 || max_blocks_per_seq < 1 ||
        max_query_len < 0 || max_context_len < 0)
        return PAGED_KV_ERR_BAD_SHAPE;
    const int group = num_q_heads / num_kv_heads;
    if (!(head_dim == 64 || head_dim == 128 || head_dim == 256) ||
        !(group == 1 || group == 2 || group == 4 || group == 8) || !pow2(block_size) ||
        block_size > 256)
        return PAGED_KV_ERR_UNSUPPORTED;
    const int64_t table_tokens = (int64_t)max_blocks_per_seq * block_size;
    if (table_tokens > INT_MAX) return PAGED_KV_ERR_BAD_SHAPE;
    const int max_ctx = max_context_len == 0 ? (int)table_tokens : max_context_len;
    if (max_ctx > table_tokens || !isfinite(scale)) return PAGED_KV_ERR_BAD_SHAPE;
    const int e = elem_bytes(dtype);
    if ((int64_t)block_size * num_kv_heads * head_dim * e > INT_MAX) return PAGED_KV_ERR_BAD_SHAPE;
    const int rpb = dtype == PAGED_KV_F32 ? pkv::prefill_f32_rows_per_block()
                                          : pkv::prefill_rows_per_block(head_dim);
    const int64_t row_blocks = ((int64_t)max_query_len * group + rpb - 1) / rpb;
    if ((int64_t)num_seqs * num_kv_heads * row_blocks > INT_MAX) return PAGED_KV_ERR_BAD_SHAPE;
    if (num_seqs == 0 || total_q == 0 || max_query_len == 0) return PAGED_KV_OK;
    if (!query || !key_cache || !value_cache || !block_tables || !context_lens ||
        !query_start || !out)
        return PAGED_KV_ERR_NULL_POINTER;
    if (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
        !aligned16(out) || !aligned4(block_tables) || !aligned4(context_lens) ||
        !aligned4(query_start))
        return PAGED_KV_ERR_BAD_SHAPE;
    // A few new tokens per sequence -- the (new token, query head) rows of a
    // kv head in one or two 16-row tiles -- and no split: the decode kernel's
    // structure (one wave per kv head, the context read once per kv head)
    // computes them, with a causal limit per row.
    const int mq_max_rows = head_dim <= 128 ? 2 * pkv::kMultiQueryRows : pkv::kMultiQueryRows;
    if (dtype != PAGED_KV_F32 && (int64_t)max_query_len * group <= mq_max_rows) {
        const pkv::DecodePlan pl =
            pkv::plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             max_blocks_per_seq, max_ctx, 0, dtype);
        if (pl.status == PAGED_KV_OK && pl.num_partitions == 1 && pl.num_chunks == 0) {
            pkv::DecodeParams d = pkv::decode_params(
                query, key_cache, value_cache, block_tables, context_lens, scale, out, num_seqs,
                num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                pl, nullptr, 0, dtype);
            d.query_start = query_start;
            d.total_q = total_q;
            d.max_query_len = max_query_len;
            d.mq_group = group;
            const hipError_t err = pkv::launch_decode_multiquery(
                d, dtype, head_dim, static_cast<hipStream_t>(stream));
            return err == hipSuccess ? PAGED_KV_OK : PAGED_KV_ERR_HIP;
        }
    }
    pkv::PrefillParams p;
    p.query = query;
    p.key_cache = static_cast<const char *>(key_cache);
    p.value_cache = static_cast<const char *>(value_cache);
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.query_start = query_start;
    p.out = out;
    // scale * dot(q, k) == |scale| * dot(-q, k) exactly, so the kernel keeps
    // a non-negative score scale and flips the query's sign bits instead
    p.score_scale = (float)(fabs((double)scale) * 1.4426950408889634);  // |scale| * log2(e)
    p.negate_query = scale < 0.0f;
    p.num_seqs = num_seqs;
    p.total_q = total_q;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = group;
    p.block_size = block_size;
    p.block_shift = log2i(block_size);
    p.num_blocks = num_blocks;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.max_query_len = max_query_len;
    p.max_context_len = max_ctx;
    p.row_blocks = (int)row_blocks;
    p.row_stride_bytes = num_kv_heads * head_dim * e;
    p.block_stride_bytes = (int64_t)block_size * p.row_stride_bytes;
    const hipError_t err =
        dtype == PAGED_KV_F32
            ? pkv::launch_prefill_f32(p, head_dim, static_cast<hipStream_t>(stream))
            : pkv::launch_prefill(p, dtype, head_dim, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PAGED_KV_OK : PAGED_KV_ERR_HIP;
}

int paged_kv_copy_blocks(void *key_cache, void *value_cache, const int32_t *block_mapping,
                         int num_pairs, int num_kv_heads, int head_dim, int block_size,
                         int num_blocks, int dtype, void *stream) {
    if (dtype != PAGED_KV_F32 && dtype != PAGED_KV_F16 && dtype != PAGED_KV_BF16)
        return PAGED_KV_ERR_UNSUPPORTED;
    if (num_pairs < 0 || num_pairs > 0x7fffffff / 2 || num_kv_heads < 1 || head_dim < 1 ||
        block_size < 1 || num_blocks < 1)
        return PAGED_KV_ERR_BAD_SHAPE;
    const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * elem_bytes(dtype);
    if (block_bytes % 16 != 0 || block_bytes / 65536 > 65535) return PAGED_KV_ERR_BAD_SHAPE;
    if (num_pairs == 0) return PAGED_KV_OK;
    if (!key_cache || !value_cache || !block_mapping) return PAGED_KV_ERR_NULL_POINTER;
    if (!aligned16(key_cache) || !aligned16(value_cache) || !aligned4(block_mapping))
        return PAGED_KV_ERR_BAD_SHAPE;
    const hipError_t err = pkv::launch_copy_blocks(key_cache, value_cache, num_blocks, key_cache,
                                                   value_cache, num_blocks, block_mapping,
                                                   num_pairs, block_bytes,
                                                   static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PAGED_KV_OK : PAGED_KV_ERR_HIP;
}

namespace {

// The device address of pinned, device-mapped host memory (hipHostMalloc, or
// a pinned torch tensor), or nullptr for any other pointer.
void *host_device_view(const void *host) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, host) != hipSuccess) {
        (void)hipGetLastError();  // an unknown pointer is an answer, not a failure
        return nullptr;
    }
    return attr.type == hipMemoryTypeHost ? attr.devicePointer : nullptr;
}

// Shared checks and launch of both swap directions; device_to_host picks
// which pools are the source.
int swap_blocks(const void *dev_key, const void *dev_value, const void *host_key,
                const void *host_value, const int32_t *block_mapping, int num_pairs,
                int num_kv_heads, int head_dim, int block_size, int num_blocks,
                int num_host_blocks, int dtype, void *stream, bool device_to_host) {
    if (dtype != PAGED_KV_F32 && dtype != PAGED_KV_F16 && dtype != PAGED_KV_BF16)
        return PAGED_KV_ERR_UNSUPPORTED;
    if (num_pairs < 0 || num_pairs > 0x7fffffff / 2 || num_kv_heads < 1 || head_dim < 1 ||
        block_size < 1 || num_blocks < 1 || num_host_blocks < 1)
        return PAGED_KV_ERR_BAD_SHAPE;
    const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * elem_bytes(dtype);
    if (block_bytes % 16 != 0 || block_bytes / 65536 > 65535) return PAGED_KV_ERR_BAD_SHAPE;
    if (num_pairs == 0) return PAGED_KV_OK;
    if (!dev_key || !dev_value || !host_key || !host_value || !block_mapping)
        return PAGED_KV_ERR_NULL_POINTER;
    if (!aligned16(dev_key) || !aligned16(dev_value) || !aligned16(host_key) ||
        !aligned16(host_value) || !aligned4(block_mapping))
        return PAGED_KV_ERR_BAD_SHAPE;
    void *hk = host_device_view(host_key);
    void *hv = host_device_view(host_value);
    if (!hk || !hv) return PAGED_KV_ERR_HOST_MEMORY;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t err =
        device_to_host
            ? pkv::launch_copy_blocks(dev_key, dev_value, num_blocks, hk, hv, num_host_blocks,
                                      block_mapping, num_pairs, block_bytes, st)
            : pkv::launch_copy_blocks(hk, hv, num_host_blocks, const_cast<void *>(dev_key),
                                      const_cast<void *>(dev_value), num_blocks, block_mapping,
                                      num_pairs, block_bytes, st);
    return err == hipSuccess ? PAGED_KV_OK : PAGED_KV_ERR_HIP;
}

}  // namespace

int paged_kv_swap_out(const void *key_cache, const void *value_cache, void *host_key_cache,
                      void *host_value_cache, const int32_t *block_mapping, int num_pairs,
                      int num_kv_heads, int head_dim, int block_size, int num_blocks,
                      int num_host_blocks, int dtype, void *stream) {
    return swap_blocks(key_cache, value_cache, host_key_cache, host_value_cache, block_mapping,
                       num_pairs, num_kv_heads, head_dim, block_size, num_blocks,
                       num_host_blocks, dtype, stream, true);
}

int paged_kv_swap_in(const void *host_key_cache, const void *host_value_cache,
                     void *key_cache, void *value_cache, const int32_t *block_mapping,
                     int num_pairs, int num_kv_heads, int head_dim, int block_size,
                     int num_blocks, int num_host_blocks, int dtype, void *stream) {
    return swap_blocks(key_cache, value_cache, host_key_cache, host_value_cache, block_mapping,
                       num_pairs, num_kv_heads, head_dim, block_size, num_blocks,
                       num_host_blocks, dtype, stream, false);
}

int paged_kv_gather(const void *key_cache, const void *value_cache,
                    const int32_t *block_tables, const int32_t *context_lens, void *out_key,
                    void *out_value, int num_seqs, int num_kv_heads, int head_dim,
                    int block_size, int num_blocks, int max_blocks_per_seq,
                    int max_context_len, int dtype, void *stream) {
    if (dtype != PAGED_KV_F32 && dtype != PAGED_KV_F16 && dtype != PAGED_KV_BF16)
        return PAGED_KV_ERR_UNSUPPORTED;
    if (num_seqs < 0 || num_seqs > 65535 || num_kv_heads < 1 || head_dim < 1 ||
        !pow2(block_size) || num_blocks < 1 || max_blocks_per_seq < 1 || max_context_len < 0 ||
        (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
        return PAGED_KV_ERR_BAD_SHAPE;
    const int64_t row = (int64_t)num_kv_heads * head_dim * elem_bytes(dtype);
    if (row % 16 != 0 || row * block_size > INT_MAX) return PAGED_KV_ERR_BAD_SHAPE;
    if (num_seqs == 0 || max_context_len == 0) return PAGED_KV_OK;
    if (!key_cache || !value_cache || !block_tables || !context_lens || !out_key || !out_value)
        return PAGED_KV_ERR_NULL_POINTER;
    if (!aligned16(key_cache) || !aligned16(value_cache) || !aligned16(out_key) ||
        !aligned16(out_value) || !aligned4(block_tables) || !aligned4(context_lens))
        return PAGED_KV_ERR_BAD_SHAPE;
    const hipError_t err = pkv::launch_paged_kv_gather(
        key_cache, value_cache, block_tables, context_lens, out_key, out_value, num_seqs,
        max_blocks_per_seq, block_size, num_blocks, max_context_len, (int)row,
        elem_bytes(dtype), static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PAGED_KV_OK : PAGED_KV_ERR_HIP;
}


int paged_kv_prefix_hash(const int32_t *tokens, const int32_t *token_start,
                         const int32_t *block_start, int num_seqs, int total_tokens,
                         int total_blocks, int block_size, uint64_t seed, uint64_t *block_hashes,
                         void *stream) {
    if (num_seqs < 0 || num_seqs > 0x7fffffff - 1 || total_tokens < 0 || total_blocks < 0 ||
        block_size < 1 || block_size > 4096)
        return PAGED_KV_ERR_BAD_SHAPE;
    if (num_seqs == 0) return PAGED_KV_OK;
    if (!token_start || !block_start || (total_tokens > 0 && !tokens) ||
        (total_blocks > 0 && !block_hashes))
        return PAGED_KV_ERR_NULL_POINTER;
    if (!aligned4(tokens) || !aligned4(token_start) || !aligned4(block_start) ||
        (reinterpret_cast<uintptr_t>(block_hashes) & 7u) != 0)
        return PAGED_KV_ERR_BAD_SHAPE;
    // base^block_size mod 2^61 - 1, the factor that carries a hash over one block
    const unsigned __int128 p = (((unsigned __int128)1) << 61) - 1;
    unsigned __int128 m = 1;
    for (int i = 0; i < block_size; ++i) m = m * PAGED_KV_PREFIX_HASH_BASE % p;
    const hipError_t err = pkv::launch_prefix_hash(
        tokens, token_start, block_start, num_seqs, total_tokens, total_blocks, block_size, seed,
        PAGED_KV_PREFIX_HASH_BASE, (uint64_t)m, block_hashes, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PAGED_KV_OK : PAGED_KV_ERR_HIP;
}

int paged_kv_prefix_insert(const uint64_t *hashes, const int32_t *blocks, int num_entries,
                           uint64_t *table_keys, int32_t *table_blocks, int capacity_log2,
                           int32_t *stored, void *stream) {
    if (num_entries < 0 || capacity_log2 < 1 || capacity_log2 > 30) return PAGED_KV_ERR_BAD_SHAPE;
    if (num_entries == 0) return PAGED_KV_OK;
    if (!hashes || !blocks || !table_keys || !table_blocks) return PAGED_KV_ERR_NULL_POINTER;
    if ((reinterpret_cast<uintptr_t>(hashes) & 7u) != 0 ||
        (reinterpret_cast<uintptr_t>(table_keys) & 7u) != 0 || !aligned4(blocks) ||
        !aligned4(table_blocks) || !aligned4(stored))
        return PAGED_KV_ERR_BAD_SHAPE;
    const hipError_t err =
        pkv::launch_prefix_insert(hashes, blocks, num_entries, table_keys, table_blocks,
                                  capacity_log2, stored, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PAGED_KV_OK : PAGED_KV_ERR_HIP;
}

int paged_kv_prefix_match(const uint64_t *block_hashes, const int32_t *block_start,
                          int num_seqs, int total_blocks, const uint64_t *table_keys,
                          const int32_t *table_blocks, int capacity_log2, int32_t *matched_blocks,
                          int32_t *matched_len, void *stream) {
    if (num_seqs < 0 || num_seqs > 0x7fffffff - 1 || total_blocks < 0 || capacity_log2 < 1 ||
        capacity_log2 > 30)
        return PAGED_KV_ERR_BAD_SHAPE;
    if (num_seqs == 0) return PAGED_KV_OK;
    if (!block_start || !table_keys || !table_blocks || !matched_len ||
        (total_blocks > 0 && (!block_hashes || !matched_blocks)))
        return PAGED_KV_ERR_NULL_POINTER;
    if ((reinterpret_cast<uintptr_t>(block_hashes) & 7u) != 0 ||
        (reinterpret_cast<uintptr_t>(table_keys) & 7u) != 0 || !aligned4(block_start) ||
        !aligned4(table_blocks) || !aligned4(matched_blocks) || !aligned4(matched_len))
        return PAGED_KV_ERR_BAD_SHAPE;
    const hipError_t err = pkv::launch_prefix_match(
        block_hashes, block_start, num_seqs, total_blocks, table_keys, table_blocks, capacity_log2,
        matched_blocks, matched_len, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PAGED_KV_OK : PAGED_KV_ERR_HIP;
}

}  // extern "C"
