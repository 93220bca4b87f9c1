// Host-side planning of a decode launch: shape checks, the context
// partition and the split workspace.  Shared by the C ABI entry points.

#include "../../include/paged_kv.h"

#include <limits.h>
#include <stdint.h>

#include "decode.h"
#include "prefill.h"

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

// Workgroups of hpg kv heads the device should have running at once.
int64_t target_workgroups(int dtype, int head_dim, int group, int block_size, int hpg) {
    const DeviceOccupancy occ = decode_occupancy(dtype, head_dim, group, block_size, hpg);
    int64_t per_cu = kTargetWavesPerCu / hpg;
    if (occ.workgroups_per_cu > 0 && per_cu > occ.workgroups_per_cu)
        per_cu = occ.workgroups_per_cu;
    if (per_cu < 1) per_cu = 1;
    return (occ.compute_units > 0 ? occ.compute_units : kFallbackComputeUnits) * per_cu;
}

// Balanced split: chunks per group of kv heads.  Two chunks per workgroup
// slot the device holds at once (on a 13B-shaped MHA batch of 50 contexts of
// 7..1965 tokens: 154.6 us against 165.4 us for one chunk per slot, 158.9 us
// for four and 161.2 us for six), and enough chunks that one chunk's blocks
// fit in a workgroup's block-id staging (a chunk of C tokens spans at most
// C / block_size + 2 blocks).
#ifndef PKV_BALANCED_ROUNDS
#define PKV_BALANCED_ROUNDS 2
#endif
int64_t balanced_chunks(int64_t padded_positions, int num_head_groups, int64_t target,
                        int block_size) {
    int64_t w = (target * PKV_BALANCED_ROUNDS + num_head_groups - 1) / num_head_groups;
    const int64_t per_chunk = (int64_t)(kBtLds - 2) * block_size - 16;
    const int64_t w_min = (padded_positions + per_chunk - 1) / per_chunk;
    if (w < w_min) w = w_min;
    return w < 1 ? 1 : w;
}

}  // namespace

// Shape checks shared by the decode entry points, and the partition choice.
DecodePlan plan_decode(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                 int max_blocks_per_seq, int max_context_len, int partition_size, int dtype) {
    DecodePlan pl{PAGED_KV_OK, 0, 0, 1, 1, 0};
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
    const int hpg = heads_per_group_for(num_kv_heads);
    if (partition_size == PAGED_KV_BALANCED_SPLIT) {
        const int64_t padded = (int64_t)num_seqs * round_up(max_ctx, 16);
        if (num_seqs > kBalancedMaxSeqs || padded > INT_MAX - 16) {
            pl.status = PAGED_KV_ERR_UNSUPPORTED;
            return pl;
        }
        const int64_t w = balanced_chunks(padded, num_kv_heads / hpg,
                                          target_workgroups(dtype, head_dim, group, block_size,
                                                            hpg),
                                          block_size);
        if (w * (num_kv_heads / hpg) > INT_MAX || 2 * w * (int64_t)num_q_heads > INT_MAX) {
            pl.status = PAGED_KV_ERR_BAD_SHAPE;
            return pl;
        }
        pl.max_context_len = max_ctx;
        pl.partition_size = PAGED_KV_BALANCED_SPLIT;
        pl.num_partitions = 1;
        pl.heads_per_group = hpg;
        pl.num_chunks = (int)w;
        return pl;
    }
    int64_t P;
    if (partition_size > 0) {
        if (partition_size % 16 != 0 || partition_size % block_size != 0 ||
            partition_size > max_part) {
            pl.status = PAGED_KV_ERR_BAD_SHAPE;
            return pl;
        }
        P = partition_size;
    } else {
        const int64_t units = (int64_t)num_seqs * (num_kv_heads / hpg);
        const int64_t target = target_workgroups(dtype, head_dim, group, block_size, hpg);
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
    pl.heads_per_group = hpg;
    // A batch that needs no split and whose workgroups are all resident at
    // once (one round) ends when the most loaded compute unit does; with 2
    // kv heads per workgroup instead of 4 each unit holds twice as many,
    // smaller workgroups and the units' loads come out more even (the same
    // waves per unit).  Only where the 2 heads' share of a token row stays
    // at least 512 contiguous bytes.  Measured with 256 contexts of ~580
    // tokens, 8 kv heads, bf16, head_dim 128: -2.0% (G = 4), -1.9% (G = 8),
    // -1.1% (G = 2), -1.7% (f16, G = 1), and -1.9% with 384 contexts of ~390
    // (three workgroups of 4 heads per unit); batches of more than one round
    // gained nothing or lost up to 1.8%, and head_dim 64 (256-byte
    // pieces) lost 2.7%.
    if (nparts == 1 && hpg == 4 && (int64_t)head_dim * (dtype == PAGED_KV_F32 ? 4 : 2) >= 256) {
        const DeviceOccupancy occ = decode_occupancy(dtype, head_dim, group, block_size, hpg);
        const int64_t cus = occ.compute_units > 0 ? occ.compute_units : kFallbackComputeUnits;
        const int64_t units = (int64_t)num_seqs * (num_kv_heads / hpg);
        if (occ.workgroups_per_cu > 0 && units <= cus * occ.workgroups_per_cu)
            pl.heads_per_group = 2;
    }
    return pl;
}

// The shared-prefix decode.  The prefix pass gets about one workgroup per
// two compute units, the prefix cut into partitions of whole 64-position
// tiles: every partition leaves a partial result per (sequence, query
// head), which the pass writes and the merge reads, so finer partitions
// cost more than the parallelism they add (on the 64-sequence batch with a
// 2000-token prefix, 16 x 128 rows x 8 kv heads: 33.3 us per call with
// 256-position partitions, 35.1 with 128, 38.3 with 512, 40.2 with 64).  The suffix pass (positions after
// the prefix: a few hundred at most in the workloads this is for) is split
// for latency rather than bandwidth: its partitions are sized so that its
// workgroups fill the device once, with no 256-token minimum.
SharedPrefixPlan plan_shared_prefix(int num_seqs, int num_q_heads, int num_kv_heads,
                                    int head_dim, int block_size, int max_blocks_per_seq,
                                    int max_context_len, int prefix_len,
                                    int prefix_partition_size, int partition_size, int dtype) {
    SharedPrefixPlan sp{};
    const DecodePlan base = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                        max_blocks_per_seq, max_context_len, 0, dtype);
    if (base.status != PAGED_KV_OK) {
        sp.status = base.status;
        return sp;
    }
    const int max_ctx = base.max_context_len;
    if (partition_size < 0 || prefix_partition_size < 0 || prefix_len < 0 ||
        prefix_len % 16 != 0 || prefix_len % block_size != 0 || prefix_len > max_ctx ||
        prefix_partition_size % 64 != 0) {
        sp.status = PAGED_KV_ERR_BAD_SHAPE;
        return sp;
    }
    if (partition_size == PAGED_KV_BALANCED_SPLIT && prefix_len > 0) {
        sp.status = PAGED_KV_ERR_UNSUPPORTED;
        return sp;
    }
    sp.prefix_len = prefix_len;
    if (prefix_len == 0) {  // nothing shared: the plain decode, balanced split included
        sp.suffix = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, max_context_len, partition_size, dtype);
        sp.status = sp.suffix.status;
        if (sp.status == PAGED_KV_OK)
            sp.workspace_bytes = decode_workspace_bytes(sp.suffix, num_seqs, num_q_heads, head_dim);
        return sp;
    }
    const int group = num_q_heads / num_kv_heads;
    const int hpg = base.heads_per_group;
    const int64_t rows = (int64_t)num_seqs * group;
    const int64_t rpb = dtype == PAGED_KV_F32 ? prefill_f32_rows_per_block()
                                              : prefill_rows_per_block(head_dim);
    const int64_t row_blocks = (rows + rpb - 1) / rpb;
    const DeviceOccupancy occ = decode_occupancy(dtype, head_dim, group, block_size, hpg);
    const int64_t cus = occ.compute_units > 0 ? occ.compute_units : kFallbackComputeUnits;
    int64_t pp;
    if (prefix_partition_size > 0) {
        pp = prefix_partition_size;
    } else {
        const int64_t units = row_blocks * num_kv_heads;
        int64_t parts = units > 0 ? cus / (2 * units) : 1;
        if (parts < 1) parts = 1;
        pp = round_up((prefix_len + parts - 1) / parts, 64);
    }
    const int64_t prefix_parts = (prefix_len + pp - 1) / pp;

    // the suffix pass
    const int suffix_max = max_ctx - prefix_len;
    int64_t P = 16, suffix_parts = 0;
    if (suffix_max > 0) {
        const int align = block_size > 16 ? block_size : 16;
        const int64_t max_part = (int64_t)kBtLds * block_size;
        if (partition_size > 0) {
            if (partition_size % 16 != 0 || partition_size % block_size != 0 ||
                partition_size > max_part) {
                sp.status = PAGED_KV_ERR_BAD_SHAPE;
                return sp;
            }
            P = partition_size;
        } else {
            const int64_t units = (int64_t)num_seqs * (num_kv_heads / hpg);
            const int64_t target = target_workgroups(dtype, head_dim, group, block_size, hpg);
            int64_t parts = units > 0 ? target / units : 1;
            if (parts < 1) parts = 1;
            P = round_up((suffix_max + parts - 1) / parts, align);
            if (P > kMaxAutoTokens) P = round_up(kMaxAutoTokens, align);
            if (P > max_part) P = max_part;
        }
        suffix_parts = (suffix_max + P - 1) / P;
    }
    const int64_t slots = prefix_parts + suffix_parts;
    if (row_blocks * num_kv_heads * prefix_parts > INT_MAX ||
        (int64_t)num_seqs * num_kv_heads * suffix_parts > INT_MAX || slots > INT_MAX ||
        (int64_t)num_seqs * num_q_heads > INT_MAX) {
        sp.status = PAGED_KV_ERR_BAD_SHAPE;
        return sp;
    }
    sp.status = PAGED_KV_OK;
    sp.suffix = base;
    sp.suffix.partition_size = (int)P;
    sp.suffix.num_partitions = (int)slots;
    sp.prefix_part = (int)pp;
    sp.prefix_parts = (int)prefix_parts;
    sp.row_blocks = (int)row_blocks;
    sp.workspace_bytes = decode_partial_floats(num_seqs, num_q_heads) * (size_t)slots *
                         (2 + (size_t)head_dim) * sizeof(float);
    return sp;
}

size_t decode_partial_floats(int num_seqs, int num_q_heads) {
    return round_up((int64_t)num_seqs * num_q_heads, 4);  // keeps the o array 16-byte aligned
}

size_t decode_partial_slots(const DecodePlan &pl, int num_seqs, int num_q_heads) {
    if (pl.num_chunks > 0) return round_up(2 * (int64_t)pl.num_chunks * num_q_heads, 4);
    if (pl.num_partitions <= 1) return 0;
    return decode_partial_floats(num_seqs, num_q_heads) * pl.num_partitions;
}

size_t decode_workspace_bytes(const DecodePlan &pl, int num_seqs, int num_q_heads, int head_dim) {
    return decode_partial_slots(pl, num_seqs, num_q_heads) * (2 + (size_t)head_dim) *
           sizeof(float);
}

// The partition for a batch whose lengths the caller holds on the host.  A
// split sized by the longest context suits contexts of similar length; with
// very uneven lengths (the longest more than 1.5 times the mean) the
// workgroups of the long contexts would finish far behind the rest, so the
// split is the balanced one, or where that does not apply the finest
// partition, kMinSplitTokens (256-token partitions measured 169 us against
// 192 us for 1024 on a batch of 50 contexts of 1..2048 tokens; 1024 stays
// best for contexts of 24K..32K tokens).
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
        const DecodePlan bal = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           block_size, max_blocks_per_seq, longest,
                                           PAGED_KV_BALANCED_SPLIT, dtype);
        if (bal.status == PAGED_KV_OK) return PAGED_KV_BALANCED_SPLIT;
        const int align = block_size > 16 ? block_size : 16;
        return (int)round_up(kMinSplitTokens, align);
    }
    return pl.partition_size;
}

}  // namespace pkv
