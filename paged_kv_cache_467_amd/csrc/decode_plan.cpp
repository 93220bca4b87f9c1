// Host-side planning of a decode launch: shape checks, the context
// partition and the split workspace.  Shared by the C ABI entry points.

#include "../../include/paged_kv.h"

#include <limits.h>
#include <stdint.h>

#include "decode.h"

namespace pkv {
namespace {

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Context partitions.  HBM reads run fastest on this part with about eight
// streaming waves per compute unit: more concurrent streams lower DRAM
// efficiency, fewer leave bandwidth unused.  So the decode aims for
// 8 / heads_per_group workgroups per compute unit (never more than fit).
// Contexts are not split when the batch already has that many (sequence,
// kv-head group) units; otherwise the split aims to reach it in one round.
// A partition holds between kMinSplitTokens and kMaxAutoTokens tokens, so
// that one very long context cannot hold up the whole launch.  When the
// device cannot be queried (no GPU), assume 256 compute units.
constexpr int kMinSplitTokens = 256;
constexpr int kMaxAutoTokens = 1024;
constexpr int kTargetWavesPerCu = 8;
constexpr int kFallbackComputeUnits = 256;


// Kv heads per workgroup: the largest power of two up to PKV_HEADS_PER_GROUP
// that divides num_kv_heads.
#ifndef PKV_HEADS_PER_GROUP
#define PKV_HEADS_PER_GROUP 4
#endif
static_assert(PKV_HEADS_PER_GROUP >= 1 && PKV_HEADS_PER_GROUP <= kMaxDecodeWaves,
              "heads per group");
int heads_per_group_for(int num_kv_heads) {
    for (int h = PKV_HEADS_PER_GROUP; h > 1; h /= 2)
        if (num_kv_heads % h == 0) return h;
    return 1;
}

}  // namespace

// Shape checks shared by the decode entry points, and the partition choice.
DecodePlan plan_decode(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                 int max_blocks_per_seq, int max_context_len, int partition_size, int dtype) {
    DecodePlan pl{PAGED_KV_OK, 0, 0, 1, 1};
    if (dtype != PAGED_KV_F32 && dtype != PAGED_KV_F16 && dtype != PAGED_KV_BF16) {
        pl.status = PAGED_KV_ERR_UNSUPPORTED;
        return pl;
    }
    if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_blocks_per_seq < 1 ||
        max_context_len < 0 || partition_size < 0 || num_q_heads % num_kv_heads != 0) {
        pl.status = PAGED_KV_ERR_BAD_SHAPE;
        return pl;
    }
    const int group = num_q_heads / num_kv_heads;
    if (!(head_dim == 64 || head_dim == 128 || head_dim == 256) ||
        !(group == 1 || group == 2 || group == 4 || group == 8) || !pow2(block_size) ||
        block_size > 256) {
        pl.status = PAGED_KV_ERR_UNSUPPORTED;
        return pl;
    }
    const int64_t table_tokens = (int64_t)max_blocks_per_seq * block_size;
    if (table_tokens > INT_MAX) {
        pl.status = PAGED_KV_ERR_BAD_SHAPE;
        return pl;
    }
    const int max_ctx = max_context_len == 0 ? (int)table_tokens : max_context_len;
    if (max_ctx > table_tokens) {
        pl.status = PAGED_KV_ERR_BAD_SHAPE;
        return pl;
    }
    const int align = block_size > 16 ? block_size : 16;
    const int64_t max_part = (int64_t)kBtLds * block_size;
    int64_t P;
    if (partition_size > 0) {
        if (partition_size % 16 != 0 || partition_size % block_size != 0 ||
            partition_size > max_part) {
            pl.status = PAGED_KV_ERR_BAD_SHAPE;
            return pl;
        }
        P = partition_size;
    } else {
        const int hpg = heads_per_group_for(num_kv_heads);
        const int64_t units = (int64_t)num_seqs * (num_kv_heads / hpg);
        const DeviceOccupancy occ =
            decode_occupancy(dtype, head_dim, group, block_size, hpg);
        int64_t per_cu = kTargetWavesPerCu / hpg;
        if (occ.workgroups_per_cu > 0 && per_cu > occ.workgroups_per_cu)
            per_cu = occ.workgroups_per_cu;
        if (per_cu < 1) per_cu = 1;
        const int64_t target =
            (occ.compute_units > 0 ? occ.compute_units : kFallbackComputeUnits) * per_cu;
        if (units >= target || max_ctx <= kMinSplitTokens) {
            P = max_ctx;  // enough units already, or nothing worth splitting
        } else {
            const int64_t parts = units > 0 ? target / units : 1;
            P = (max_ctx + parts - 1) / parts;
            if (P > kMaxAutoTokens) P = kMaxAutoTokens;
            if (P < kMinSplitTokens) P = kMinSplitTokens;
        }
        P = round_up(P, align);
        if (P < align) P = align;
        if (P > max_part) P = max_part;
    }
    const int64_t nparts = max_ctx == 0 ? 1 : (max_ctx + P - 1) / P;
    if ((int64_t)num_seqs * num_kv_heads * nparts > INT_MAX ||
        (int64_t)num_seqs * num_q_heads > INT_MAX) {
        pl.status = PAGED_KV_ERR_BAD_SHAPE;
        return pl;
    }
    pl.max_context_len = max_ctx;
    pl.partition_size = (int)P;
    pl.num_partitions = (int)nparts;
    pl.heads_per_group = heads_per_group_for(num_kv_heads);
    return pl;
}

size_t decode_partial_floats(int num_seqs, int num_q_heads) {
    return round_up((int64_t)num_seqs * num_q_heads, 4);  // keeps the o array 16-byte aligned
}

size_t decode_workspace_bytes(const DecodePlan &pl, int num_seqs, int num_q_heads, int head_dim) {
    if (pl.num_partitions <= 1) return 0;
    const size_t n = decode_partial_floats(num_seqs, num_q_heads) * pl.num_partitions;
    return n * (2 + (size_t)head_dim) * sizeof(float);
}

// The partition for a batch whose lengths the caller holds on the host.  A
// split sized by the longest context suits contexts of similar length; with
// very uneven lengths (the longest more than 1.5 times the mean) the
// workgroups of the long contexts would finish far behind the rest, so the
// split is the finest one, kMinSplitTokens (256-token partitions measured
// 169 us against 192 us for 1024 on a batch of 50 contexts of 1..2048
// tokens; 1024 stays best for contexts of 24K..32K tokens).
int plan_partition_for_lengths(const int32_t *lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_dim, int block_size,
                               int max_blocks_per_seq, int dtype) {
    int64_t sum = 0;
    int longest = 0;
    for (int s = 0; s < num_seqs; ++s) {
        const int L = lens[s] > 0 ? lens[s] : 0;
        sum += L;
        if (L > longest) longest = L;
    }
    const int64_t table_tokens = (int64_t)max_blocks_per_seq * block_size;
    if (longest > table_tokens) return -PAGED_KV_ERR_BAD_SHAPE;
    const DecodePlan pl = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_blocks_per_seq, longest > 0 ? longest : 1, 0, dtype);
    if (pl.status != PAGED_KV_OK) return -pl.status;
    if (pl.num_partitions > 1 && 2 * (int64_t)longest * num_seqs > 3 * sum) {
        const int align = block_size > 16 ? block_size : 16;
        return (int)round_up(kMinSplitTokens, align);
    }
    return pl.partition_size;
}

}  // namespace pkv
