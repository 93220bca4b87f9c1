// Paged-attention decode kernels for gfx950 (CDNA4).
//
// What is computed: for every sequence s and query head h, the one new query
// attends over the L = context_lens[s] cached tokens; token j is read from
// physical block block_tables[s][j / block_size] at offset j % block_size of
// the pool [num_blocks, block_size, num_kv_heads, head_dim]
// ("大模型推理框架 vllm 源码解析 一", §三, the paged_attention_v1
// description), with a scaled dot-product softmax.  Long contexts are split
// into partitions whose partial results are merged by log-sum-exp; the pages
// only name this as segmented attention over scattered blocks
// ("23.1 vLLM：高吞吐推理框架原理与部署", §二.2 step 3).
//
// Work decomposition: one workgroup per (sequence, group of kv heads,
// context partition), one wave per kv head of the group -- or, with the
// balanced split (for batches whose context lengths are very uneven), one
// workgroup per (chunk, group of kv heads), a chunk being an equal share of
// all the batch's positions laid end to end, which it walks sequence piece
// by sequence piece.  The workgroup
// stages the partition's block ids in LDS once (checking each against the
// pool size); then every wave walks the whole partition for its kv head, one
// tile of at most 16 tokens at a time, keeping the online-softmax state
// (running max m, running sum l, fp32 output accumulator) of the G query
// heads that share that kv head, so every K/V byte is read once for all G
// heads.  The waves of a workgroup read the same token rows side by side (a
// block of all kv heads is one contiguous stretch of the pool), and a wave's
// result needs no merge with other waves.  K/V tiles are loaded one tile
// ahead of the one being consumed, with non-temporal loads.
//
// Addressing: tiles never cross a 16-token boundary, so with block_size >= 16
// a tile lies in one block and its base address is wave-uniform (block id
// read once from LDS into a scalar register); each lane adds a fixed offset.
// Smaller blocks and the last, partial tile of a partition use per-lane
// addresses with bounds guards.
//
// Two per-tile inner loops:
//  * decode_mfma_kernel (f16/bf16, G >= 2): the scores of a 16-token tile for
//    all G heads are one 16x16x32 MFMA chain.  K and V rows are both loaded
//    whole-row coalesced (consecutive lanes read consecutive 16-byte chunks
//    of one row); K goes through a wave-private LDS slice to the B operand
//    layout (lane = token), the query rows (repeated 16/G times) form the A
//    operand.  With G >= 4 the value product is a matrix product too:
//    O^T += V^T P^T, v_mfma_f32_16x16x16 per 16-wide block of head_dim, V^T
//    read from the V slice with the gfx950 transposing LDS read and the
//    weights (through LDS, rounded to the element type) as the B operand;
//    with G = 2 the weights go through LDS to the lanes that hold the V rows
//    and PV is accumulated with fp32 FMAs.
//  * decode_valu_kernel (all dtypes, any G): each row of head_dim elements is
//    spread over head_dim * bytes / 16 lanes, 16 bytes each; scores are dot
//    products (packed 16-bit dot instructions for f16/bf16, fp32 FMAs for
//    f32) reduced across those lanes with DPP.
// Online softmax: the running max only moves when some score of the tile
// exceeds it; each lane checks its own scores, and the cross-lane max
// reduction and the rescale of l and the accumulator run only when one did.
//
// Fused KV write (paged_attn_decode_write: each sequence's new token goes to
// its pool cell, position L - 1, in the same launch): the VALU kernel stores
// the new rows before it reads the context; the MFMA kernel has an instance
// of its own (FW) that takes the rows from the new-token input, uses them in
// place of the pool's in the tile that holds position L - 1, and stores them
// in the cell after its loop.

#include "decode.h"
#include "device_utils.h"

#include <math.h>

#include <atomic>

namespace pkv {
namespace {

// K/V tiles held in registers per wave by the VALU kernel: one being
// consumed, the rest in flight.  For 16-bit types (the multi-head decode)
// three tiles of look-ahead measured best (on a 13B-shaped f16 batch: 0.9%
// faster with two than with one, 0.4% more with three, five no better),
// though it halves the waves a SIMD holds; f32 keeps one, which fits
// without spilling at every group size.  The MFMA kernel keeps one tile in
// registers and one in LDS instead.
constexpr int kValuDepth16 = 4;
constexpr int kValuDepth32 = 2;

struct WorkItem {
    int s, kvh0, part;  // sequence, first kv head of the workgroup, partition
    int kvh;            // this wave's kv head
    int context_len;
    int tok_begin, tok_end;  // this partition's token range [begin, end)
    bool bad_len;            // context_len < 0 or > max_context_len
    bool final;              // the range is the whole context: write the output
};

__device__ inline WorkItem work_item(const DecodeParams &p) {
    WorkItem w;
    const int id = blockIdx.x;
    const int hg = id % p.num_head_groups;
    const int rest = id / p.num_head_groups;
    const int parts = p.num_partitions - p.prefix_parts;  // partitions in the grid
    const int q = rest % parts;
    w.part = p.prefix_parts + q;
    w.s = rest / parts;
    w.kvh0 = hg * p.heads_per_group;
    w.kvh = w.kvh0 + (int)(threadIdx.x / kWave);
    w.context_len = p.context_lens[w.s];
    w.bad_len = w.context_len < 0 || w.context_len > p.max_context_len;
    w.tok_begin = p.prefix_len + q * p.partition_size;
    const int end = w.tok_begin + p.partition_size;
    w.tok_end = end < w.context_len ? end : w.context_len;
    w.final = p.num_partitions == 1;
    return w;
}

// ------------------------------------------------------------------------
// Balanced split.  The positions of all sequences, each padded to a
// multiple of 16 (a length outside [0, max_context_len] counts 0), are laid
// end to end and cut into num_chunks chunks of C positions, C a multiple of
// 16; workgroup (chunk w, kv-head group) computes every piece of a sequence
// that falls in chunk w (a segment).  A sequence whose positions lie in one
// chunk is finished there.  The others leave one partial result per chunk
// they touch, in slot 2 w + 1 of the chunk they start in and in slot 2 w of
// every later one (a chunk holds at most one sequence that continues from
// the chunk before and one that continues into the next), and the reduce
// merges them.
// ------------------------------------------------------------------------
__device__ inline int padded_len(const DecodeParams &p, int L) {
    return (L > 0 && L <= p.max_context_len) ? (L + 15) & ~15 : 0;
}

__device__ inline int chunk_size(int total, int num_chunks) {
    const int64_t c = ((int64_t)total + num_chunks - 1) / num_chunks;
    const int r = (int)((c + 15) & ~(int64_t)15);
    return r < 16 ? 16 : r;
}

__device__ inline int scan_inclusive_wave(int x) {
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    return x;
}

// start[s] for s = 0 .. num_seqs: exclusive prefix sums of the padded
// lengths, written to LDS by the whole workgroup (start[num_seqs] = total).
__device__ inline void padded_starts(const DecodeParams &p, int32_t *start, int32_t *wave_tot) {
    const int S = p.num_seqs;
    const int nt = blockDim.x;
    const int t = threadIdx.x;
    const int k = (S + nt - 1) / nt;  // consecutive sequences per thread
    const int s0 = t * k;
    int local = 0;
    for (int i = 0; i < k; ++i)
        if (s0 + i < S) local += padded_len(p, p.context_lens[s0 + i]);
    const int incl = scan_inclusive_wave(local);
    const int wave = t / kWave;
    if (t % kWave == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int v = 0; v < wave; ++v) before += wave_tot[v];
    int run = before + incl - local;
    for (int i = 0; i < k; ++i) {
        if (s0 + i < S) {
            start[s0 + i] = run;
            run += padded_len(p, p.context_lens[s0 + i]);
        }
    }
    if (t == nt - 1) start[S] = before + incl;
    __syncthreads();
}

// Runs body(work item) for each segment of this workgroup's chunk, with a
// workgroup barrier after each (the segments reuse the block-id staging).
template <class Body>
__device__ inline void for_each_segment(const DecodeParams &p, int32_t *start,
                                        int32_t *wave_tot, Body &&body) {
    padded_starts(p, start, wave_tot);
    const int S = p.num_seqs;
    const int total = start[S];
    const int C = chunk_size(total, p.num_chunks);
    const int chunk = blockIdx.x / p.num_head_groups;
    const int hg = blockIdx.x % p.num_head_groups;
    const int lo = (int)((int64_t)chunk * C < total ? (int64_t)chunk * C : total);
    if (lo >= total) return;
    const int hi = total - lo < C ? total : lo + C;
    // the last sequence starting at or before lo: the one holding position lo
    int a = 0, b = S - 1;
    while (a < b) {
        const int mid = (a + b + 1) / 2;
        if (start[mid] <= lo) a = mid; else b = mid - 1;
    }
    for (int s = a; s < S && start[s] < hi; ++s) {
        if (start[s + 1] == start[s]) continue;  // empty or invalid length
        const int L = p.context_lens[s];
        const int begin = (lo > start[s] ? lo : start[s]) - start[s];
        const int e0 = (hi < start[s + 1] ? hi : start[s + 1]) - start[s];
        const int end = e0 < L ? e0 : L;
        if (begin >= end) continue;               // only padding of s in this chunk
        const int first = start[s] / C, last = (start[s] + L - 1) / C;
        WorkItem w;
        w.s = s;
        w.kvh0 = hg * p.heads_per_group;
        w.kvh = w.kvh0 + (int)(threadIdx.x / kWave);
        w.part = chunk == first ? 2 * chunk + 1 : 2 * chunk;  // partial slot
        w.context_len = L;
        w.tok_begin = begin;
        w.tok_end = end;
        w.bad_len = false;
        w.final = first == last;
        body(w);
        __syncthreads();
    }
}

// Index of the partial result of query head h for work item w.
__device__ inline int64_t partial_index(const DecodeParams &p, const WorkItem &w, int h) {
    if (p.num_chunks > 0) return (int64_t)w.part * p.num_q_heads + h;
    return ((int64_t)w.s * p.num_q_heads + h) * p.num_partitions + w.part;
}

// Copies the block ids covering tokens [begin, end) into LDS.  Returns true
// (for every thread) if any of them is outside [0, num_blocks).
__device__ inline bool stage_block_table(const DecodeParams &p, const WorkItem &w,
                                         int32_t *bt_lds) {
    const int b0 = w.tok_begin >> p.block_shift;
    const int b1 = (w.tok_end - 1) >> p.block_shift;
    const int32_t *row = p.block_tables + (int64_t)w.s * p.max_blocks_per_seq;
    int bad = b1 - b0 + 1 > kBtLds;  // never with the host's split (kept in bounds regardless)
    for (int i = threadIdx.x; i <= b1 - b0 && i < kBtLds; i += blockDim.x) {
        int id = row[b0 + i];
        if (id < 0 || id >= p.num_blocks) {
            bad = 1;
            id = 0;
        }
        bt_lds[i] = id;
    }
    return __syncthreads_or(bad) != 0;
}

// Stages the block table like stage_block_table, and when `early` also
// issues the partition's first tile in the middle of it: the ids' load goes
// out first, the tile's own block id is read on its own (a scalar load:
// the table is never written by a decode, so it is read as constant
// memory), issue_first(base) issues the tile, and only then does the
// staging wait for the ids.  Memory loads complete in order, so that wait
// does not cover the tile, and the code is straight-line, so the compiler
// can count the tile's loads as still in flight.  `early` requires
// block_size >= 16, a whole first tile and at most one id per thread.  An
// id outside the pool gives base of block 0 (in bounds, never used: the
// staging flags the partition, and the caller then waits for the loads).
template <class IssueFirst>
__device__ inline bool stage_block_table_early(const DecodeParams &p, const WorkItem &w,
                                               int32_t *bt_lds, bool early,
                                               IssueFirst &&issue_first) {
    if (!early) return stage_block_table(p, w, bt_lds);
    const int b0 = w.tok_begin >> p.block_shift;
    const int nb = ((w.tok_end - 1) >> p.block_shift) - b0 + 1;
    const int32_t *row = p.block_tables + (int64_t)w.s * p.max_blocks_per_seq;
    const int tid = threadIdx.x;
    const int id = tid < nb ? row[b0 + tid] : 0;
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    int blk = ((const_i32 *)row)[b0];
    blk = blk >= 0 && blk < p.num_blocks ? blk : 0;
    issue_first((int64_t)blk * p.block_stride_bytes +
                (int64_t)(w.tok_begin & (p.block_size - 1)) * p.row_stride_bytes);
    const bool ok = id >= 0 && id < p.num_blocks;
    if (tid < nb) bt_lds[tid] = ok ? id : 0;
    return __syncthreads_or(tid < nb && !ok) != 0;
}

// Whether stage_block_table_early may issue the first tile of `tile` tokens.
template <bool BT>
__device__ inline bool first_tile_early(const DecodeParams &p, const WorkItem &w, int tile) {
    const int b0 = w.tok_begin >> p.block_shift;
    const int nb = ((w.tok_end - 1) >> p.block_shift) - b0 + 1;
    return BT && w.tok_end - w.tok_begin >= tile && nb <= (int)blockDim.x;
}

// Byte offset of (token, kv head) in the pool; token must be in the staged
// range.
__device__ inline int64_t row_offset(const DecodeParams &p, const int32_t *bt_lds, int b0,
                                     int token, int head_bytes) {
    const int blk = bt_lds[(token >> p.block_shift) - b0];
    const int off = token & (p.block_size - 1);
    return (int64_t)blk * p.block_stride_bytes + (int64_t)(off * p.row_stride_bytes + head_bytes);
}

// Byte offset of the row of token t0 (kv head 0) for a wave-uniform t0 when
// block_size >= 16: the block id goes through a scalar register, so the
// address arithmetic is scalar.
__device__ inline int64_t uniform_row_offset(const DecodeParams &p, const int32_t *bt_lds, int b0,
                                             int t0) {
    const int blk = __builtin_amdgcn_readfirstlane(bt_lds[(t0 >> p.block_shift) - b0]);
    const int off = t0 & (p.block_size - 1);
    return (int64_t)blk * p.block_stride_bytes + (int64_t)off * p.row_stride_bytes;
}

// Output of a workgroup that reads nothing: zeros for an empty sequence, NaN
// for an invalid one; covers every query head of the workgroup's kv heads.
template <class T, int D, int G>
__device__ void store_constant(const DecodeParams &p, const WorkItem &w, bool nan) {
    const int n = p.heads_per_group * G * D;
    const int64_t base = ((int64_t)w.s * p.num_q_heads + (int64_t)w.kvh0 * G) * D;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        if (nan)
            T::store_nan(p.out, base + i);
        else
            T::store(p.out, base + i, 0.0f);
    }
}

// Fused KV write, store first (the VALU kernel; the MFMA kernel's fused
// instance only for a context that reads nothing; the plain instances are
// launched with new_key null): the new token of sequence s (position L - 1)
// goes to its pool cell before the sequence's attention reads it.  The
// workgroup whose partition holds position L - 1 (partition 0 when L is 0 or
// invalid: then nothing is read) writes the rows of its kv heads, each wave
// its own head's row -- the row that wave alone reads back -- and fences it.
// A slot outside the pool writes nothing.
template <class T, int D>
__device__ inline void write_new_token(const DecodeParams &p, const WorkItem &w) {
    if (p.new_key == nullptr) return;
    const bool reads = !w.bad_len && w.context_len >= 1;
    const int owner = reads ? (w.context_len - 1) / p.partition_size : 0;
    if (w.part != owner) return;
    const int slot = p.slot_mapping[w.s];
    if (slot < 0 || slot >= p.num_slots) return;
    constexpr int kRowBytes = D * T::kBytes;
    const int lane = threadIdx.x % kWave;
    const int64_t src = ((int64_t)w.s * p.num_kv_heads + w.kvh) * kRowBytes;
    const int64_t dst = (int64_t)(slot >> p.block_shift) * p.block_stride_bytes +
                        (int64_t)(slot & (p.block_size - 1)) * p.row_stride_bytes +
                        (int64_t)w.kvh * kRowBytes;
    char *kc = const_cast<char *>(p.key_cache);
    char *vc = const_cast<char *>(p.value_cache);
    for (int b = lane * 16; b < kRowBytes; b += kWave * 16) {
        store16(kc + dst + b, load16(p.new_key + src + b));
        store16(vc + dst + b, load16(p.new_value + src + b));
    }
    __threadfence_block();
}

// Common prologue.  Returns false when the workgroup has nothing to read (it
// has then already written whatever it owes).
template <class T, int D, int G>
__device__ bool prologue(const DecodeParams &p, const WorkItem &w) {
    if (w.bad_len || w.tok_begin >= w.context_len) {
        // Without a split this workgroup owns the output (zeros when L == 0,
        // NaN when L is invalid).  With a split the reduce kernel owns it.
        if (p.num_partitions == 1) store_constant<T, D, G>(p, w, w.bad_len);
        return false;
    }
    return true;
}

// Writes one wave's result for query head h: the 16-byte chunk of output
// elements starting at d0 (T::kPerChunk of them), from fp32 accumulators acc
// (unnormalised), with the head's final running max m and sum l.  Without a
// split the normalised output is stored in the output dtype; with a split
// the partial (m, l, acc) is.
template <class T, int D>
__device__ inline void write_result(const DecodeParams &p, const WorkItem &w, int h, int d0,
                                    const float *acc, float m, float l, bool bad,
                                    bool write_ml) {
    constexpr int EPC = T::kPerChunk;
    if (w.final) {
        const int64_t o = ((int64_t)w.s * p.num_q_heads + h) * D + d0;
        u32x4 c;
        if (bad) {
            c = u32x4{T::kNanPair, T::kNanPair, T::kNanPair, T::kNanPair};
        } else {
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            float v[EPC];
#pragma unroll
            for (int e = 0; e < EPC; ++e) v[e] = acc[e] * inv;
            c = T::narrow_chunk(v);
        }
        store16(static_cast<char *>(p.out) + o * T::kBytes, c);
    } else {
        const int64_t ph = partial_index(p, w, h);
        float *po = p.part_out + ph * D + d0;
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
            u32x4 c;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                c[k] = bad ? 0x7FC00000u : __builtin_bit_cast(uint32_t, acc[e + k]);
            store16(po + e, c);
        }
        if (write_ml) {
            p.part_max[ph] = bad ? 0.0f : m;
            p.part_sum[ph] = bad ? NAN : l;
        }
    }
}

// Runs the tile pipeline of one wave: tiles [0, ntiles), of which the first
// nfull are complete; load(t, slot, full) fills register slot `slot` with
// tile t, consume(t, slot, full) folds it into the softmax state.  Slots are
// compile-time indices after unrolling, so the buffers stay in registers.
// With first_issued, tile 0 is already in flight in slot 0.
template <int DEPTH, class Load, class Consume>
__device__ inline void run_tiles(int ntiles, int nfull, Load &&load, Consume &&consume,
                                 bool first_issued = false) {
#pragma unroll
    for (int j = 0; j < DEPTH - 1; ++j)
        if (j < ntiles && !(first_issued && j == 0)) load(j, j, j < nfull);
    for (int t0 = 0; t0 < ntiles; t0 += DEPTH) {
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) {
            const int t = t0 + j;
            if (t < ntiles) {
                const int ahead = t + DEPTH - 1;
                if (ahead < ntiles && !(first_issued && ahead == 0))
                    load(ahead, (j + DEPTH - 1) % DEPTH, ahead < nfull);
                consume(t, j, t < nfull);
            }
        }
    }
}

// ------------------------------------------------------------------------
// VALU kernel
// ------------------------------------------------------------------------
template <class T, int D, int G, bool BT, bool BAL>
__global__ __launch_bounds__(kMaxDecodeThreads) void decode_valu_kernel(DecodeParams p) {
    constexpr int EPC = T::kPerChunk;   // elements per 16-byte chunk
    constexpr int CPR = D / EPC;        // lanes holding one row
    constexpr int TPI = kWave / CPR;    // tokens per load instruction
    // loads per lane per tile (K and V each); fewer with many fp32 accumulators
    constexpr int NL = TPI > 4 ? 16 / TPI : G * EPC >= 32 ? 2 : 4;
    constexpr int TILE = TPI * NL;      // tokens per tile: 2 to 16, divides 16
    static_assert(CPR >= 4 && CPR <= 64 && kWave % CPR == 0, "row layout");
    static_assert(16 % TILE == 0, "tiles must not cross a 16-token boundary");
    // wide rows or many fp32 accumulators: no room for a second tile
    constexpr int DEPTH =
        (D >= 256 || G * EPC >= 32) ? 1 : T::kBytes == 2 ? kValuDepth16 : kValuDepth32;

    __shared__ int32_t bt_lds[kBtLds];

    // one partition (or, with the balanced split, one segment) of a sequence
    auto segment = [&](const WorkItem &w) {
    const int b0 = w.tok_begin >> p.block_shift;

    const int lane = threadIdx.x % kWave;
    const int tg = lane / CPR;  // token slot within a load
    const int c = lane % CPR;   // 16-byte chunk of the row
    const int head_bytes = w.kvh * D * T::kBytes + c * 16;
    // offset of this lane's chunk from the row of the tile's first token
    const uint32_t lane_off = (uint32_t)(tg * p.row_stride_bytes + head_bytes);
    const uint32_t step_off = (uint32_t)(TPI * p.row_stride_bytes);  // per load of a tile

    u32x4 q[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        q[g] = load16(static_cast<const char *>(p.query) +
                      (((int64_t)w.s * p.num_q_heads + w.kvh * G + g) * D + c * EPC) * T::kBytes);

    float m[G], l[G], acc[G][EPC];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[g][e] = 0.0f;
    }

    const int span = w.tok_end - w.tok_begin;
    u32x4 kbuf[DEPTH][NL], vbuf[DEPTH][NL];

    // a whole tile at pool byte offset base (the row of its first token)
    auto load_full = [&](int64_t base, int j) {
        const char *kb = p.key_cache + base;
        const char *vb = p.value_cache + base;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            kbuf[j][i] = load16_stream(kb + (lane_off + i * step_off));
            vbuf[j][i] = load16_stream(vb + (lane_off + i * step_off));
        }
    };
    auto load = [&](int tile, int slot, bool full) {
        const int t0 = w.tok_begin + tile * TILE;
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) {
            if (j != slot) continue;
            if (BT && full) {
                load_full(uniform_row_offset(p, bt_lds, b0, t0), j);
            } else {
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    const int t = t0 + i * TPI + tg;
                    if (t < w.tok_end) {
                        const int64_t o = row_offset(p, bt_lds, b0, t, head_bytes);
                        kbuf[j][i] = load16_stream(p.key_cache + o);
                        vbuf[j][i] = load16_stream(p.value_cache + o);
                    } else {
                        kbuf[j][i] = u32x4{0, 0, 0, 0};
                        vbuf[j][i] = u32x4{0, 0, 0, 0};
                    }
                }
            }
        }
    };

    auto consume = [&](int tile, int slot, bool full) {
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) {
            if (j != slot) continue;
            const int t0 = w.tok_begin + tile * TILE;
            float sc[NL][G];
            bool up = false;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const bool valid = full || t0 + i * TPI + tg < w.tok_end;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float d = group_sum<CPR>(T::dot_chunk(q[g], kbuf[j][i], 0.0f));
                    sc[i][g] = valid ? d * p.scale_log2 : -INFINITY;
                    up |= sc[i][g] > m[g];
                }
            }
            if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float x = sc[0][g];
#pragma unroll
                    for (int i = 1; i < NL; ++i) x = vmax(x, sc[i][g]);
                    const float mn = vmax(m[g], across_groups_max<CPR>(x));
                    const float alpha = fast_exp2(m[g] - mn);  // 0 on the first tile
                    m[g] = mn;
                    l[g] *= alpha;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) acc[g][e] *= alpha;
                }
            }
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                float v[EPC];
                T::widen(vbuf[j][i], v);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float pr = fast_exp2(sc[i][g] - m[g]);
                    l[g] += pr;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) acc[g][e] = fmaf(pr, v[e], acc[g][e]);
                }
            }
        }
    };

    // the first tile goes out while the block ids are staged
    const bool early = first_tile_early<BT>(p, w, TILE);
    const bool bad = stage_block_table_early(p, w, bt_lds, early,
                                             [&](int64_t base) { load_full(base, 0); });
    // a flagged partition never consumes the first tile: let its loads land
    // before the wave moves on
    if (bad && early) __builtin_amdgcn_s_waitcnt(0);
    const int ntiles = bad ? 0 : (span + TILE - 1) / TILE;
    const int nfull = bad ? 0 : span / TILE;
    run_tiles<DEPTH>(ntiles, nfull, load, consume, early);

    // Combine the token groups of the wave: l and acc over the TPI groups.
#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = across_groups_sum<CPR>(l[g]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[g][e] = across_groups_sum<CPR>(acc[g][e]);
    }
    if (tg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
            write_result<T, D>(p, w, w.kvh * G + g, c * EPC, acc[g], m[g], l[g], bad, c == 0);
    }
    };

    if constexpr (BAL) {
        __shared__ int32_t seq_start[kBalancedMaxSeqs + 1];
        __shared__ int32_t wave_tot[kMaxDecodeWaves];
        for_each_segment(p, seq_start, wave_tot, segment);
    } else {
        const WorkItem w = work_item(p);
        write_new_token<T, D>(p, w);
        if (!prologue<T, D, G>(p, w)) return;
        segment(w);
    }
}

// ------------------------------------------------------------------------
// MFMA kernel (f16 / bf16, G in {2, 4, 8})
// ------------------------------------------------------------------------
template <class T>
__device__ inline f32x4 mfma16x16x32(const u32x4 &a, const u32x4 &b, const f32x4 &c);
template <>
__device__ inline f32x4 mfma16x16x32<BF16>(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ inline f32x4 mfma16x16x32<F16>(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Operand layout of v_mfma_f32_16x16x32_{bf16,f16} used here: lane l gives
// row (A) / column (B) l % 16 and 8 consecutive k values of k-group l / 16;
// lane l receives result rows 4 * (l / 16) + r, r = 0..3, of column l % 16.
// Any pairing of k values works as long as A and B use the same one, so the
// k-group of lane l in step ks is 16-byte chunk (l / 16) + 4 * ks of a row.
//
// K tiles: loading them straight in that B layout makes every load
// instruction touch 16 rows, 64 bytes each; on this part the same bytes read
// about 3% faster as whole rows (4 rows x 256 bytes per instruction at
// D = 128, the V layout).  So K is loaded like V and each wave turns its tile
// around in its own LDS slice: 16 rows of D * 2 bytes plus a 16-byte pad, so
// that the 16 rows a B-layout read touches start in different banks.
//
// V tiles go through LDS too, in the lanes' own order: a wave's registers
// are then free for the next tile's loads as soon as the current tile has
// arrived.
template <int D>
constexpr int k_lds_row_bytes() { return D * 2 + 16; }
template <int D>
constexpr int v_lds_offset() { return 16 * k_lds_row_bytes<D>(); }

// Value product on the matrix cores (groups of at least PKV_PV_MFMA_MIN_G
// query heads): O^T = V^T P^T with v_mfma_f32_16x16x16 per 16-wide d block,
// the A operand (V^T) read from the V slice with the transposing LDS read,
// the B operand the tile's weights rounded to the element type.  Otherwise
// fp32 FMAs on the vector unit.  Measured on a batch of 256 contexts of
// 522..638 tokens, 8 kv heads, bf16 (interleaved runs): G = 8 6.4% faster
// at head_dim 128 (97.5 against 104.1 us), 8.4% at 64; G = 4 0.9-1.9%;
// G = 2 0.5% slower, so it starts at G = 4.
#ifndef PKV_PV_MFMA_MIN_G
#define PKV_PV_MFMA_MIN_G 4
#endif
template <int G>
constexpr bool pv_mfma() { return G >= PKV_PV_MFMA_MIN_G; }
// V rows in the slice: D * 2 bytes, padded by 32 for the transposing reads
// (8 rows x 32 bytes per pass then start 8 banks apart)
template <int D, int G>
constexpr int v_lds_row_bytes() { return pv_mfma<G>() ? D * 2 + 32 : D * 2; }
template <int D, int G>
constexpr int kv_lds_wave_bytes() { return v_lds_offset<D>() + 16 * v_lds_row_bytes<D, G>(); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// 8-byte transposing LDS read: within each 16 lanes, lane i receives
// element i % 4 of the 8-byte vectors addressed by lanes 4 e + i / 4
// (e = 0..3); so if lane 4 r + c addresses row r, elements 4 c .. 4 c + 3
// of a 4 x 16 block, lane i receives column i of the block.
[[maybe_unused]] __device__ inline uint64_t lds_read_tr16(const char *p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3))) *)(p));
    return __builtin_bit_cast(uint64_t, v);
}

template <class T>
__device__ inline f32x4 mfma16x16x16(uint64_t a, uint64_t b, const f32x4 &c);
template <>
[[maybe_unused]] __device__ inline f32x4 mfma16x16x16<BF16>(uint64_t a, uint64_t b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
template <>
[[maybe_unused]] __device__ inline f32x4 mfma16x16x16<F16>(uint64_t a, uint64_t b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Four weights in [0, 1] rounded (nearest even) to the element type, packed
// low to high.
template <class T>
__device__ inline uint64_t narrow4(const f32x4 &w);
template <>
[[maybe_unused]] __device__ inline uint64_t narrow4<BF16>(const f32x4 &w) {
    const float a = w[0], b = w[1], c = w[2], d = w[3];
    const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{c, d}, bf16x2));
    return (uint64_t)lo | ((uint64_t)hi << 32);
}
template <>
[[maybe_unused]] __device__ inline uint64_t narrow4<F16>(const f32x4 &w) {
    const float a = w[0], b = w[1], c = w[2], d = w[3];
    const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
    const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{c, d}, f16x2));
    return (uint64_t)lo | ((uint64_t)hi << 32);
}

// Writes four consecutive output elements d0 .. d0 + 3 of query head h from
// fp32 accumulators (unnormalised), with the head's running max m and sum
// l: the normalised output in the element type without a split, else the
// partial (m, l, acc).
template <class T, int D>
__device__ inline void write_result4(const DecodeParams &p, const WorkItem &w, int h, int d0,
                                     const f32x4 &acc, float m, float l, bool bad,
                                     bool write_ml) {
    const float a0 = acc[0], a1 = acc[1], a2 = acc[2], a3 = acc[3];
    if (w.final) {
        const int64_t o = ((int64_t)w.s * p.num_q_heads + h) * D + d0;
        uint64_t c;
        if (bad) {
            c = ((uint64_t)T::kNanPair << 32) | T::kNanPair;
        } else {
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            const float v[8] = {a0 * inv, a1 * inv, a2 * inv, a3 * inv, 0.0f, 0.0f, 0.0f, 0.0f};
            const u32x4 n = T::narrow_chunk(v);
            c = (uint64_t)n[0] | ((uint64_t)n[1] << 32);
        }
        *reinterpret_cast<uint64_t *>(static_cast<char *>(p.out) + o * T::kBytes) = c;
    } else {
        const int64_t ph = partial_index(p, w, h);
        const u32x4 c = bad ? u32x4{0x7FC00000u, 0x7FC00000u, 0x7FC00000u, 0x7FC00000u}
                            : u32x4{__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1),
                                    __builtin_bit_cast(uint32_t, a2), __builtin_bit_cast(uint32_t, a3)};
        store16(p.part_out + ph * D + d0, c);
        if (write_ml) {
            p.part_max[ph] = bad ? 0.0f : m;
            p.part_sum[ph] = bad ? NAN : l;
        }
    }
}

// MQ: the multi-token decode (launch_decode_multiquery).  G is then the
// 16 rows of the tile, row v = (new token v / mq_group, query head
// v % mq_group of the kv head), each with its own last visible position;
// no split, no fused write.
template <class T, int D, int G, bool BT, bool BAL, bool FW = false, bool MQ = false>
__global__ __launch_bounds__(kMaxDecodeThreads) void decode_mfma_kernel(DecodeParams p) {
    static_assert(T::kBytes == 2, "MFMA path is for 16-bit element types");
    static_assert(!(FW && BAL), "the fused write takes the plain split");
    static_assert(MQ ? (G == kMultiQueryRows || G == 2 * kMultiQueryRows) && !FW && !BAL
                     : (G == 2 || G == 4 || G == 8),
                  "group size");
    // row tiles of 16 per wave: MQ with 32 rows holds two, each its own
    // score and value products over the same K and V operands
    constexpr int NT = MQ ? G / kMultiQueryRows : 1;
    constexpr int KS = D / 32;        // MFMA k-steps per tile
    constexpr int CPR = D / 8;        // 16-byte chunks per row
    constexpr int TPI = kWave / CPR;  // tokens per V load instruction
    constexpr int NV = 16 / TPI;      // V loads per lane per tile
    constexpr int TILE = 16;
    constexpr int HW = G < 4 ? G : 4;  // heads among a lane's four result rows
    constexpr int KRS = k_lds_row_bytes<D>();
    static_assert(NV == KS, "a K tile in row layout takes as many loads as MFMA steps");
    constexpr bool PVM = pv_mfma<G>();
    constexpr int VRS = v_lds_row_bytes<D, G>();
    constexpr int DB = D / 16;        // 16-wide d blocks of the value MFMA

    __shared__ int32_t bt_lds[kBtLds];
    // softmax weights of the tile (16-byte aligned: read and written as
    // f32x4); [token][head], or [head][token] for the value MFMA
    __shared__ __attribute__((aligned(16))) float pex[kMaxDecodeWaves][TILE][G];
    __shared__ float aex[kMaxDecodeWaves][G];  // rescale factors, then final m
    __shared__ float lex[kMaxDecodeWaves][G];  // final l
    // K tiles turned from row layout to the B layout, and V tiles: one slice
    // per wave, kv_lds_wave_bytes<D>() each (dynamic, sized by the launch)
    extern __shared__ __attribute__((aligned(16))) char k_lds[];

    // MQ: the sequence's first query row, its new tokens computed (at most
    // max_query_len) and the last position its first new token sees
    int mq_q0 = 0, mq_nq = 0, mq_lim0 = 0;

    // one partition (or, with the balanced split, one segment) of a sequence
    auto segment = [&](const WorkItem &w) {
    const int b0 = w.tok_begin >> p.block_shift;

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    // score layout (MFMA): token kt of the tile, k-group / row group rg
    const int kt = lane & 15;
    const int rg = lane >> 4;
    // value layout: token slot vtg, chunk vc
    const int vtg = lane / CPR;
    const int vc = lane % CPR;
    const int head_bytes = w.kvh * D * 2;
    // offset from the row of the tile's first token (K and V alike)
    const uint32_t v_off = (uint32_t)(vtg * p.row_stride_bytes + head_bytes + 16 * vc);
    const uint32_t v_step = (uint32_t)(TPI * p.row_stride_bytes);
    // this wave's K slice (row-layout writes, B-layout reads) and V slice
    char *k_slice = k_lds + wave * kv_lds_wave_bytes<D, G>();
    char *k_wr = k_slice + vtg * KRS + 16 * vc;
    const char *k_rd = k_slice + kt * KRS + 16 * rg;
    // V: without the value MFMA in the lanes' own order (row-major, 4 rows
    // x 256 bytes per load at D = 128), with it in padded rows
    char *v_slot = k_slice + v_lds_offset<D>() + (PVM ? vtg * VRS + 16 * vc : lane * 16);
    constexpr int v_wr_step = PVM ? TPI * VRS : kWave * 16;
    // value MFMA: this lane's column (query head) and k-group (4 tokens), the
    // transposing read's row and chunk within its 4 x 16 block
    const int ph = lane & 15;
    const int pkg = lane >> 4;
    const char *v_tr = k_slice + v_lds_offset<D>() + (4 * pkg + ((lane & 15) >> 2)) * VRS +
                       (lane & 3) * 8;
    float *pt = &pex[wave][0][0];  // [head][token] with the value MFMA
    // row group rg holds heads 4 * rg .. 4 * rg + HW - 1; groups with
    // 4 * rg >= G hold copies of those rows
    const bool owns_rows = 4 * rg < G;

    // A operand: query head (kt % G) of this kv head's group
    u32x4 qa[NT][KS];
    if constexpr (MQ) {
        // row 16 t + kt of tile t: new token (16 t + kt) / mq_group, query
        // head (16 t + kt) % mq_group; rows past the sequence's new tokens
        // are zero
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int v = kMultiQueryRows * t + kt, i = v / p.mq_group;
            const char *qrow = static_cast<const char *>(p.query) +
                               (((int64_t)(mq_q0 + i) * p.num_q_heads + w.kvh * p.mq_group +
                                 v % p.mq_group) * D) * 2;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qa[t][ks] = i < mq_nq ? load16(qrow + 16 * (rg + 4 * ks)) : u32x4{0, 0, 0, 0};
        }
    } else {
        const char *qrow = static_cast<const char *>(p.query) +
                           (((int64_t)w.s * p.num_q_heads + w.kvh * G + kt % G) * D) * 2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[0][ks] = load16(qrow + 16 * (rg + 4 * ks));
    }
    // result row 4 * rg + r (of tile t) holds query head (4 * rg + r) % G
    float m[NT][4], l[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            m[t][r] = -INFINITY;
            l[t][r] = 0.0f;
        }
    // MQ: the last position result row 16 t + 4 * rg + r sees (-1: a row past
    // the new tokens, which sees nothing and is not written)
    int lim[NT][4] = {};
    if constexpr (MQ) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = (kMultiQueryRows * t + 4 * rg + r) / p.mq_group;
                lim[t][r] = i < mq_nq ? mq_lim0 + i : -1;
            }
    }
    float acc[PVM ? 1 : G][8];
    f32x4 accm[NT][PVM ? DB : 1];
    if constexpr (PVM) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int b = 0; b < DB; ++b) accm[t][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = 0.0f;
    }

    const int span = w.tok_end - w.tok_begin;
    // K and V of the tile in flight, in row layout
    u32x4 kbuf[NV], vbuf[NV];

    // a whole tile at pool byte offset base (the row of its first token)
    auto load_full = [&](int64_t base) {
        const char *kb = p.key_cache + base;
        const char *vb = p.value_cache + base;
#pragma unroll
        for (int i = 0; i < NV; ++i) kbuf[i] = load16_stream(kb + (v_off + i * v_step));
#pragma unroll
        for (int i = 0; i < NV; ++i) vbuf[i] = load16_stream(vb + (v_off + i * v_step));
    };
    auto load = [&](int tile, bool full) {
        const int t0 = w.tok_begin + tile * TILE;
        if (BT && full) {
            load_full(uniform_row_offset(p, bt_lds, b0, t0));
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int tv = t0 + i * TPI + vtg;
                if (tv < w.tok_end) {
                    const int64_t o = row_offset(p, bt_lds, b0, tv, head_bytes) + 16 * vc;
                    kbuf[i] = load16_stream(p.key_cache + o);
                    vbuf[i] = load16_stream(p.value_cache + o);
                } else {
                    kbuf[i] = u32x4{0, 0, 0, 0};
                    vbuf[i] = u32x4{0, 0, 0, 0};
                }
            }
        }
    };

    // Fused write (FW): the partition that ends at the context's end holds
    // the new token, position L - 1, whose pool cell is slot_mapping[s] by
    // the entry point's contract.  Its rows are read from new_key /
    // new_value (each lane its chunk vc), put in place of the pool's rows in
    // the LDS copy of the tile that holds the position, and stored in the
    // cell after the loop; nothing else in the launch reads that cell.  The
    // slot and the rows are loaded before the first tile, so that waiting
    // for them overlaps the tile's loads.
    int nt_tile = -1, nt_row = 0;
    int64_t nt_dst = 0;
    u32x4 nk = {0, 0, 0, 0}, nv = {0, 0, 0, 0};
    const bool nt_part = FW && w.tok_end == w.context_len;
    int slot = -1;
    if constexpr (FW) {
        slot = p.slot_mapping[w.s];
        if (nt_part) {
            const int64_t src = ((int64_t)w.s * p.num_kv_heads + w.kvh) * (D * 2) + 16 * vc;
            nk = load16(p.new_key + src);
            nv = load16(p.new_value + src);
        }
    }

    // the first tile goes out while the block ids are staged
    const bool early = first_tile_early<BT>(p, w, TILE);
    const bool bad = stage_block_table_early(p, w, bt_lds, early, load_full);
    const int ntiles = bad ? 0 : (span + TILE - 1) / TILE;
    const int nfull = bad ? 0 : span / TILE;
    // a flagged partition never consumes the first tile: let its loads land
    // before the wave moves on
    if (bad && early) __builtin_amdgcn_s_waitcnt(0);

    if constexpr (FW) {
        if (nt_part && slot >= 0 && slot < p.num_slots) {
            const int rel = w.context_len - 1 - w.tok_begin;
            nt_tile = rel / TILE;
            nt_row = rel % TILE;
            nt_dst = (int64_t)(slot >> p.block_shift) * p.block_stride_bytes +
                     (int64_t)(slot & (p.block_size - 1)) * p.row_stride_bytes + head_bytes +
                     16 * vc;
        }
    }

    // Per tile: the tile's K and V go from registers to this wave's LDS
    // slices as soon as they arrive, which frees the registers for the next
    // tile's loads; those are issued before the tile's arithmetic, so every
    // wave keeps one tile in flight while it computes.  LDS executes a
    // wave's accesses in order, so only compiler ordering must be kept.
    if (ntiles > 0 && !early) load(0, 0 < nfull);
    for (int tile = 0; tile < ntiles; ++tile) {
        const bool full = tile < nfull;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            *reinterpret_cast<u32x4 *>(k_wr + i * TPI * KRS) = kbuf[i];
            *reinterpret_cast<u32x4 *>(v_slot + i * v_wr_step) = vbuf[i];
        }
        if constexpr (FW) {
            // the new token's rows over the pool's (LDS keeps a wave's
            // writes in order)
            if (tile == nt_tile && vtg == nt_row % TPI) {
                const int i = nt_row / TPI;
                *reinterpret_cast<u32x4 *>(k_wr + i * TPI * KRS) = nk;
                *reinterpret_cast<u32x4 *>(v_slot + i * v_wr_step) = nv;
            }
        }
        if (tile + 1 < ntiles) load(tile + 1, tile + 1 < nfull);
        __builtin_amdgcn_wave_barrier();
        // scores: K in the B layout
        u32x4 kb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kb[ks] = *reinterpret_cast<const u32x4 *>(k_rd + 64 * ks);
        f32x4 s[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            s[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) s[t] = mfma16x16x32<T>(qa[t][ks], kb[ks], s[t]);
        }

        const bool valid = full || w.tok_begin + tile * TILE + kt < w.tok_end;
        float sc[NT][4];
        bool up = false;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (MQ)  // causal: each row's own last position (always < tok_end)
                    sc[t][r] = w.tok_begin + tile * TILE + kt <= lim[t][r] ? s[t][r] * p.scale_log2
                                                                         : -INFINITY;
                else
                    sc[t][r] = valid ? s[t][r] * p.scale_log2 : -INFINITY;
                up |= sc[t][r] > m[t][r];
            }
        // Every head is held by some lane, so "no lane's score exceeds its
        // row's max" means no head's max moves in this tile.
        const bool rescale = __builtin_amdgcn_ballot_w64(up) != 0;
        if (rescale) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float mn = vmax(m[t][r], group_max<16>(sc[t][r]));  // 16 tokens
                    const float alpha = fast_exp2(m[t][r] - mn);  // 0 on the first tile
                    m[t][r] = mn;
                    l[t][r] *= alpha;
                    if (r < HW && owns_rows && kt == 0)
                        aex[wave][kMultiQueryRows * t + 4 * rg + r] = alpha;
                }
        }
        float pr[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // (MQ: a masked score is 0 also in a row that has seen nothing)
                pr[t][r] = MQ && sc[t][r] == -INFINITY ? 0.0f : fast_exp2(sc[t][r] - m[t][r]);
                l[t][r] += pr[t][r];
            }
        if (owns_rows) {
            if constexpr (PVM) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int r = 0; r < HW; ++r)
                        pt[(kMultiQueryRows * t + 4 * rg + r) * TILE + kt] = pr[t][r];
            } else if constexpr (HW == 4) {
                *reinterpret_cast<f32x4 *>(&pex[wave][kt][4 * rg]) =
                    f32x4{pr[0][0], pr[0][1], pr[0][2], pr[0][3]};
            } else {
#pragma unroll
                for (int r = 0; r < HW; ++r) pex[wave][kt][4 * rg + r] = pr[0][r];
            }
        }
        // The weights were written by this wave; LDS executes a wave's
        // accesses in order, so only compiler ordering must be kept.
        __builtin_amdgcn_wave_barrier();
        if constexpr (PVM) {
            // lane (head ph, tokens 4 pkg .. 4 pkg + 3): B = P^T; heads past
            // G (columns no result reads) get zero weights
            if (rescale) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int hr = kMultiQueryRows * t + ph;
                    const float a = hr < G ? aex[wave][hr] : 1.0f;
#pragma unroll
                    for (int b = 0; b < DB; ++b) accm[t][b] *= a;
                }
            }
            uint64_t bw[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int hr = kMultiQueryRows * t + ph;
                const f32x4 wq = hr < G
                                     ? *reinterpret_cast<const f32x4 *>(&pt[hr * TILE + 4 * pkg])
                                     : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                bw[t] = narrow4<T>(wq);
            }
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const uint64_t va = lds_read_tr16(v_tr + 32 * b);
#pragma unroll
                for (int t = 0; t < NT; ++t) accm[t][b] = mfma16x16x16<T>(va, bw[t], accm[t][b]);
            }
        } else {
            if (rescale) {
                float alpha[G];
#pragma unroll
                for (int g = 0; g < G; ++g) alpha[g] = aex[wave][g];
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[g][e] *= alpha[g];
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                float v[8];
                T::widen(*reinterpret_cast<const u32x4 *>(v_slot + i * (kWave * 16)), v);
                float pw[G];
#pragma unroll
                for (int g = 0; g < G; ++g) pw[g] = pex[wave][i * TPI + vtg][g];
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pw[g], v[e], acc[g][e]);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    if constexpr (FW) {
        // every read of the cell (the last tile's loads) has landed
        if (nt_tile >= 0 && vtg == 0) {
            store16(const_cast<char *>(p.key_cache) + nt_dst, nk);
            store16(const_cast<char *>(p.value_cache) + nt_dst, nv);
        }
    }

    // l: sum over the 16 tokens of each row; acc: over the value token
    // slots (the value MFMA sums over the tokens itself).
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) l[t][r] = group_sum<16>(l[t][r]);
    if constexpr (!PVM) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = across_groups_sum<CPR>(acc[g][e]);
    }
    if (kt == 0 && owns_rows) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < HW; ++r) {
                aex[wave][kMultiQueryRows * t + 4 * rg + r] = m[t][r];
                lex[wave][kMultiQueryRows * t + 4 * rg + r] = l[t][r];
            }
    }
    __builtin_amdgcn_wave_barrier();
    if constexpr (MQ) {
        // lane (row 16 t + ph, d group pkg) holds d = 16 b + 4 pkg .. + 3 of
        // new token (16 t + ph) / mq_group, query head (16 t + ph) %
        // mq_group; no split
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int v = kMultiQueryRows * t + ph, i = v / p.mq_group;
            if (i >= mq_nq) continue;
            const float lh = lex[wave][v];
            const float inv = lh > 0.0f ? 1.0f / lh : 0.0f;
            const int64_t o = ((int64_t)(mq_q0 + i) * p.num_q_heads + w.kvh * p.mq_group +
                               v % p.mq_group) * D;
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                uint64_t c;
                if (bad) {
                    c = ((uint64_t)T::kNanPair << 32) | T::kNanPair;
                } else {
                    const float x[8] = {accm[t][b][0] * inv, accm[t][b][1] * inv,
                                        accm[t][b][2] * inv, accm[t][b][3] * inv,
                                        0.0f, 0.0f, 0.0f, 0.0f};
                    const u32x4 n = T::narrow_chunk(x);
                    c = (uint64_t)n[0] | ((uint64_t)n[1] << 32);
                }
                *reinterpret_cast<uint64_t *>(static_cast<char *>(p.out) +
                                              (o + 16 * b + 4 * pkg) * T::kBytes) = c;
            }
        }
    } else if constexpr (PVM) {
        // lane (head ph, d group pkg) holds d = 16 b + 4 pkg .. + 3
        if (ph < G) {
            const float mh = aex[wave][ph], lh = lex[wave][ph];
#pragma unroll
            for (int b = 0; b < DB; ++b)
                write_result4<T, D>(p, w, w.kvh * G + ph, 16 * b + 4 * pkg, accm[0][b], mh, lh,
                                    bad, b == 0 && pkg == 0);
        }
    } else if (vtg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
            write_result<T, D>(p, w, w.kvh * G + g, vc * 8, acc[g], aex[wave][g], lex[wave][g],
                               bad, vc == 0);
    }
    };

    if constexpr (BAL) {
        __shared__ int32_t seq_start[kBalancedMaxSeqs + 1];
        __shared__ int32_t wave_tot[kMaxDecodeWaves];
        for_each_segment(p, seq_start, wave_tot, segment);
    } else if constexpr (MQ) {
        // the prefill's rules: rows of a sequence whose query range cannot be
        // identified are not written; a length outside [q_len,
        // max_context_len] gives NaN rows
        const WorkItem w = work_item(p);
        const int qs0 = p.query_start[w.s], qs1 = p.query_start[w.s + 1];
        if (qs0 < 0 || qs1 > p.total_q || qs1 < qs0) return;
        const int q_len = qs1 - qs0;
        mq_q0 = qs0;
        mq_nq = q_len < p.max_query_len ? q_len : p.max_query_len;
        mq_lim0 = w.context_len - q_len;
        if (mq_nq == 0) return;
        if (w.bad_len || w.context_len < q_len) {
            const int n = mq_nq * p.mq_group * D;  // this wave's kv head's rows
            for (int e = threadIdx.x % kWave; e < n; e += kWave) {
                const int i = e / (p.mq_group * D), rest = e % (p.mq_group * D);
                T::store_nan(p.out, ((int64_t)(qs0 + i) * p.num_q_heads +
                                     (int64_t)w.kvh * p.mq_group) * D + rest);
            }
            return;
        }
        segment(w);
    } else {
        const WorkItem w = work_item(p);
        if constexpr (FW) {
            // a context that reads nothing: the row goes straight to its cell
            if (w.bad_len || w.context_len < 1) write_new_token<T, D>(p, w);
        } else {
            write_new_token<T, D>(p, w);
        }
        if (!prologue<T, D, G>(p, w)) return;
        segment(w);
    }
}

// ------------------------------------------------------------------------
// Cross-partition reduce: out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p
// with M = max_p m_p.  One wave per (sequence, query head): the lanes split
// the partitions for M and the denominator, then each lane owns head_dim / 64
// output elements and walks the partitions, 16 loads in flight at a time.
// ------------------------------------------------------------------------
constexpr int kReduceThreads = 64;

template <class T, int D>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(DecodeParams p) {
    constexpr int EL = D / kReduceThreads;  // output elements per lane: 1, 2 or 4
    constexpr int R = 16;                   // partitions' outputs loaded per round
    const int sh = blockIdx.x;
    const int lane = threadIdx.x;
    const int s = sh / p.num_q_heads;
    const int64_t obase = (int64_t)sh * D + lane * EL;
    const int64_t pbase = (int64_t)sh * p.num_partitions;
    const float *pm = p.part_max + pbase;
    const float *ps = p.part_sum + pbase;
    const float *po = p.part_out + pbase * D + lane * EL;
    const int np = p.num_partitions;

    // The maxima and sums of the first 64 partitions are loaded with the
    // length (every index stays below num_partitions, inside the workspace;
    // what lies past this sequence's own partitions is masked below, and
    // shares cache lines with the partitions that are used).  The partial
    // outputs, 4 * head_dim bytes a partition, are loaded only for the
    // sequence's own partitions, once its length is known.
    const int L = p.context_lens[s];
    float mq = lane < np ? pm[lane] : -INFINITY;  // lane q holds partition q < 64
    float lq = lane < np ? ps[lane] : 0.0f;
    // (a context shorter than the shared prefix breaks the shared-prefix
    // decode's contract)
    if (L < 0 || L > p.max_context_len || L < p.prefix_len) {
#pragma unroll
        for (int e = 0; e < EL; ++e) T::store_nan(p.out, obase + e);
        return;
    }
    if (L == 0) {
#pragma unroll
        for (int e = 0; e < EL; ++e) T::store(p.out, obase + e, 0.0f);
        return;
    }
    const int nparts =
        p.prefix_parts + (L - p.prefix_len + p.partition_size - 1) / p.partition_size;
    float v[R][EL];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        // past the last partition: reread partition 0 (in bounds, finite, cached)
        const int q = u < nparts ? u : 0;
#pragma unroll
        for (int e = 0; e < EL; ++e) v[u][e] = po[(int64_t)q * D + e];
    }
    if (lane >= nparts) {
        mq = -INFINITY;
        lq = 0.0f;
    }
    float M = mq;
    for (int q = lane + kReduceThreads; q < nparts; q += kReduceThreads) M = vmax(M, pm[q]);
    M = group_max<kReduceThreads>(M);
    float Ls = lane < nparts ? lq * fast_exp2(mq - M) : 0.0f;
    for (int q = lane + kReduceThreads; q < nparts; q += kReduceThreads)
        Ls += ps[q] * fast_exp2(pm[q] - M);
    Ls = group_sum<kReduceThreads>(Ls);
    const float inv = 1.0f / Ls;

    // weight of partition q (q < 64 is held by lane q)
    const float wl = lane < nparts ? fast_exp2(mq - M) : 0.0f;
    auto weight = [&](int q) {
        return q < kReduceThreads
                   ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                   __builtin_bit_cast(int, wl), q))
                   : fast_exp2(pm[q] - M);
    };
    float o[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) o[e] = 0.0f;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        if (u < nparts) {
            const float wq = weight(u);
#pragma unroll
            for (int e = 0; e < EL; ++e) o[e] = fmaf(wq, v[u][e], o[e]);
        }
    }
    for (int q0 = R; q0 < nparts; q0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int q = q0 + u < nparts ? q0 + u : 0;
#pragma unroll
            for (int e = 0; e < EL; ++e) v[u][e] = po[(int64_t)q * D + e];
        }
#pragma unroll
        for (int u = 0; u < R; ++u) {
            if (q0 + u < nparts) {
                const float wq = weight(q0 + u);
#pragma unroll
                for (int e = 0; e < EL; ++e) o[e] = fmaf(wq, v[u][e], o[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < EL; ++e) T::store(p.out, obase + e, o[e] * inv);
}

// The reduce of the balanced split, one wave per (sequence, query head):
// the same merge over the sequence's partial results, which sit in slot
// 2 f + 1 (its first chunk f) and slots 2 c of its later chunks c.  A
// sequence that lies in one chunk was finished by the partition kernel.
__device__ inline int wave_sum_int(int x) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) x += __shfl_xor(x, d);
    return x;
}

template <class T, int D>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_balanced_kernel(DecodeParams p) {
    constexpr int EL = D / kReduceThreads;
    constexpr int R = 16;
    const int sh = blockIdx.x;
    const int lane = threadIdx.x;
    const int s = sh / p.num_q_heads;
    const int h = sh % p.num_q_heads;
    const int64_t obase = (int64_t)sh * D + lane * EL;
    const int L = p.context_lens[s];
    if (L < 0 || L > p.max_context_len) {
#pragma unroll
        for (int e = 0; e < EL; ++e) T::store_nan(p.out, obase + e);
        return;
    }
    if (L == 0) {
#pragma unroll
        for (int e = 0; e < EL; ++e) T::store(p.out, obase + e, 0.0f);
        return;
    }
    // this sequence's padded start and the padded total, as the partition
    // kernel lays them out
    int before = 0, total = 0;
    for (int i = lane; i < p.num_seqs; i += kReduceThreads) {
        const int pi = padded_len(p, p.context_lens[i]);
        total += pi;
        if (i < s) before += pi;
    }
    before = wave_sum_int(before);
    total = wave_sum_int(total);
    const int C = chunk_size(total, p.num_chunks);
    const int first = before / C;
    const int n = (before + L - 1) / C - first + 1;  // partial results
    if (n == 1) return;
    auto index = [&](int q) -> int64_t {
        const int slot = q == 0 ? 2 * first + 1 : 2 * (first + q);
        return (int64_t)slot * p.num_q_heads + h;
    };
    const float mq = lane < n ? p.part_max[index(lane)] : -INFINITY;  // lane q: partial q < 64
    const float lq = lane < n ? p.part_sum[index(lane)] : 0.0f;
    float v[R][EL];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int64_t o = index(u < n ? u : 0) * D + lane * EL;
#pragma unroll
        for (int e = 0; e < EL; ++e) v[u][e] = p.part_out[o + e];
    }
    float M = mq;
    for (int q = lane + kReduceThreads; q < n; q += kReduceThreads)
        M = vmax(M, p.part_max[index(q)]);
    M = group_max<kReduceThreads>(M);
    float Ls = lane < n ? lq * fast_exp2(mq - M) : 0.0f;
    for (int q = lane + kReduceThreads; q < n; q += kReduceThreads)
        Ls += p.part_sum[index(q)] * fast_exp2(p.part_max[index(q)] - M);
    Ls = group_sum<kReduceThreads>(Ls);
    const float inv = 1.0f / Ls;
    const float wl = lane < n ? fast_exp2(mq - M) : 0.0f;
    auto weight = [&](int q) {
        return q < kReduceThreads
                   ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                   __builtin_bit_cast(int, wl), q))
                   : fast_exp2(p.part_max[index(q)] - M);
    };
    float o[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) o[e] = 0.0f;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        if (u < n) {
            const float wq = weight(u);
#pragma unroll
            for (int e = 0; e < EL; ++e) o[e] = fmaf(wq, v[u][e], o[e]);
        }
    }
    for (int q0 = R; q0 < n; q0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int64_t oo = index(q0 + u < n ? q0 + u : 0) * D + lane * EL;
#pragma unroll
            for (int e = 0; e < EL; ++e) v[u][e] = p.part_out[oo + e];
        }
#pragma unroll
        for (int u = 0; u < R; ++u) {
            if (q0 + u < n) {
                const float wq = weight(q0 + u);
#pragma unroll
                for (int e = 0; e < EL; ++e) o[e] = fmaf(wq, v[u][e], o[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < EL; ++e) T::store(p.out, obase + e, o[e] * inv);
}

// Workgroups of this kernel instance one compute unit holds at once.
template <class T, int D, int G, bool BT>
int blocks_per_cu(int threads) {
    int n = 0;
    hipError_t e;
    if constexpr (T::kBytes == 2 && G >= 2)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void *>(&decode_mfma_kernel<T, D, G, BT, false>), threads,
            (threads / kWave) * kv_lds_wave_bytes<D, G>());
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void *>(&decode_valu_kernel<T, D, G, BT, false>), threads, 0);
    return e == hipSuccess ? n : 0;
}

template <class T, int D>
int blocks_per_cu_d(int group, bool bt, int threads) {
    switch (group) {
        case 1: return bt ? blocks_per_cu<T, D, 1, true>(threads) : blocks_per_cu<T, D, 1, false>(threads);
        case 2: return bt ? blocks_per_cu<T, D, 2, true>(threads) : blocks_per_cu<T, D, 2, false>(threads);
        case 4: return bt ? blocks_per_cu<T, D, 4, true>(threads) : blocks_per_cu<T, D, 4, false>(threads);
        case 8: return bt ? blocks_per_cu<T, D, 8, true>(threads) : blocks_per_cu<T, D, 8, false>(threads);
        default: return 0;
    }
}

template <class T>
int blocks_per_cu_t(int head_dim, int group, bool bt, int threads) {
    switch (head_dim) {
        case 64: return blocks_per_cu_d<T, 64>(group, bt, threads);
        case 128: return blocks_per_cu_d<T, 128>(group, bt, threads);
        case 256: return blocks_per_cu_d<T, 256>(group, bt, threads);
        default: return 0;
    }
}

template <class T, int D, int G, bool BT>
hipError_t launch_main(const DecodeParams &p, int kernel, hipStream_t stream) {
    const unsigned grid =
        p.num_chunks > 0
            ? (unsigned)((int64_t)p.num_chunks * p.num_head_groups)
            : (unsigned)((int64_t)p.num_seqs * p.num_head_groups *
                         (p.num_partitions - p.prefix_parts));
    if (grid == 0) return hipSuccess;  // a shared prefix that is the whole context
    const unsigned threads = (unsigned)(p.heads_per_group * kWave);
    // 16-bit types with grouped queries take the MFMA kernel, everything else
    // the VALU kernel (decode_kernel_choice); only those pairs are built.
    if constexpr (T::kBytes == 2 && G >= 2) {
        if (kernel != 1) return hipErrorInvalidValue;
        const size_t lds = p.heads_per_group * kv_lds_wave_bytes<D, G>();
        if (p.num_chunks > 0)
            hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, BT, true>), dim3(grid),
                               dim3(threads), lds, stream, p);
        else if (p.new_key != nullptr)
            hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, BT, false, true>), dim3(grid),
                               dim3(threads), lds, stream, p);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, BT, false>), dim3(grid),
                               dim3(threads), lds, stream, p);
    } else {
        if (kernel != 0) return hipErrorInvalidValue;
        if (p.num_chunks > 0)
            hipLaunchKernelGGL((decode_valu_kernel<T, D, G, BT, true>), dim3(grid),
                               dim3(threads), 0, stream, p);
        else
            hipLaunchKernelGGL((decode_valu_kernel<T, D, G, BT, false>), dim3(grid),
                               dim3(threads), 0, stream, p);
    }
    return hipGetLastError();
}

template <class T, int D, int G>
hipError_t launch_typed(const DecodeParams &p, int kernel, hipStream_t stream) {
    hipError_t e = p.block_size >= 16 ? launch_main<T, D, G, true>(p, kernel, stream)
                                      : launch_main<T, D, G, false>(p, kernel, stream);
    if (e != hipSuccess) return e;
    if (p.num_chunks > 0) {
        hipLaunchKernelGGL((decode_reduce_balanced_kernel<T, D>),
                           dim3(p.num_seqs * p.num_q_heads), dim3(kReduceThreads), 0, stream, p);
        e = hipGetLastError();
    } else if (p.num_partitions > 1 || p.prefix_parts > 0) {
        hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3(p.num_seqs * p.num_q_heads),
                           dim3(kReduceThreads), 0, stream, p);
        e = hipGetLastError();
    }
    return e;
}

template <class T, int D>
hipError_t launch_d(const DecodeParams &p, int group, int kernel, hipStream_t stream) {
    switch (group) {
        case 1: return launch_typed<T, D, 1>(p, kernel, stream);
        case 2: return launch_typed<T, D, 2>(p, kernel, stream);
        case 4: return launch_typed<T, D, 4>(p, kernel, stream);
        case 8: return launch_typed<T, D, 8>(p, kernel, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class T>
hipError_t launch_t(const DecodeParams &p, int head_dim, int group, int kernel,
                    hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_d<T, 64>(p, group, kernel, stream);
        case 128: return launch_d<T, 128>(p, group, kernel, stream);
        case 256: return launch_d<T, 256>(p, group, kernel, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int decode_kernel_choice(int dtype, int head_dim, int group) {
    (void)head_dim;
    // Grouped queries of a 16-bit type make each tile a real contraction
    // (G heads x head_dim x 16 tokens): MFMA.  Otherwise plain FMAs.
    return (dtype != 0 && group >= 2) ? 1 : 0;
}

DeviceOccupancy decode_occupancy(int dtype, int head_dim, int group, int block_size,
                                 int heads_per_group) {
    // Occupancy depends only on the kernel instance and the workgroup size;
    // cache it per (dtype, head_dim, group, block_size >= 16, heads_per_group).
    static std::atomic<int> cache[3][3][4][2][4];
    static std::atomic<int> cus{0};
    DeviceOccupancy r{0, 0};
    if (dtype < 0 || dtype > 2) return r;
    const int hi = head_dim == 64 ? 0 : head_dim == 128 ? 1 : 2;
    const int gi = group == 1 ? 0 : group == 2 ? 1 : group == 4 ? 2 : 3;
    const int bi = block_size >= 16 ? 1 : 0;
    const int wi = heads_per_group == 1 ? 0 : heads_per_group == 2 ? 1 : heads_per_group == 4 ? 2 : 3;
    int n_cu = cus.load(std::memory_order_relaxed);
    if (n_cu == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            n_cu = 0;
        if (n_cu > 0) cus.store(n_cu, std::memory_order_relaxed);
    }
    int per_cu = cache[dtype][hi][gi][bi][wi].load(std::memory_order_relaxed);
    if (per_cu == 0 && n_cu > 0) {
        const int threads = heads_per_group * kWave;
        switch (dtype) {
            case 0: per_cu = blocks_per_cu_t<F32>(head_dim, group, bi, threads); break;
            case 1: per_cu = blocks_per_cu_t<F16>(head_dim, group, bi, threads); break;
            default: per_cu = blocks_per_cu_t<BF16>(head_dim, group, bi, threads); break;
        }
        if (per_cu > 0) cache[dtype][hi][gi][bi][wi].store(per_cu, std::memory_order_relaxed);
    }
    if (n_cu <= 0 || per_cu <= 0) (void)hipGetLastError();  // no device here: clear the error
    r.compute_units = n_cu > 0 ? n_cu : 0;
    r.workgroups_per_cu = per_cu > 0 ? per_cu : 0;
    return r;
}

namespace {
template <class T, int D, int R>
hipError_t launch_multiquery_r(const DecodeParams &p, hipStream_t stream) {
    const unsigned grid = (unsigned)((int64_t)p.num_seqs * p.num_head_groups);
    if (grid == 0) return hipSuccess;
    const unsigned threads = (unsigned)(p.heads_per_group * kWave);
    const size_t lds = p.heads_per_group * kv_lds_wave_bytes<D, R>();
    if (p.block_size >= 16)
        hipLaunchKernelGGL((decode_mfma_kernel<T, D, R, true, false, false, true>), dim3(grid),
                           dim3(threads), lds, stream, p);
    else
        hipLaunchKernelGGL((decode_mfma_kernel<T, D, R, false, false, false, true>), dim3(grid),
                           dim3(threads), lds, stream, p);
    return hipGetLastError();
}
// one 16-row tile per wave, or two (17..32 rows; head_dim up to 128: at 256
// the two tiles' accumulators do not fit in registers)
template <class T, int D>
hipError_t launch_multiquery_d(const DecodeParams &p, hipStream_t stream) {
    if (p.mq_group * p.max_query_len <= kMultiQueryRows)
        return launch_multiquery_r<T, D, kMultiQueryRows>(p, stream);
    if constexpr (D <= 128)
        return launch_multiquery_r<T, D, 2 * kMultiQueryRows>(p, stream);
    return hipErrorInvalidValue;
}
template <class T>
hipError_t launch_multiquery_t(const DecodeParams &p, int head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_multiquery_d<T, 64>(p, stream);
        case 128: return launch_multiquery_d<T, 128>(p, stream);
        case 256: return launch_multiquery_d<T, 256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_decode_multiquery(const DecodeParams &p, int dtype, int head_dim,
                                    hipStream_t stream) {
    if (p.heads_per_group < 1 || p.heads_per_group > kMaxDecodeWaves || p.num_partitions != 1 ||
        p.num_chunks != 0 || p.mq_group < 1 ||
        p.mq_group * p.max_query_len > 2 * kMultiQueryRows)
        return hipErrorInvalidValue;
    switch (dtype) {
        case 1: return launch_multiquery_t<F16>(p, head_dim, stream);
        case 2: return launch_multiquery_t<BF16>(p, head_dim, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeParams &p, int dtype, int head_dim, int group, int kernel,
                         hipStream_t stream) {
    if (p.heads_per_group < 1 || p.heads_per_group > kMaxDecodeWaves) return hipErrorInvalidValue;
    switch (dtype) {
        case 0: return launch_t<F32>(p, head_dim, group, kernel, stream);
        case 1: return launch_t<F16>(p, head_dim, group, kernel, stream);
        case 2: return launch_t<BF16>(p, head_dim, group, kernel, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
