// Device-side pieces shared by the multi-token (chunked-prefill) attention
// kernels: the workgroup -> (sequence, kv head, row block) order, the
// cross-lane row reductions and the lazy-rescale threshold.
#pragma once

#include "device_utils.h"
#include "prefill.h"

namespace pkv {

constexpr int kXcds = 8;   // accelerator complex dies of the MI355X, each with its own L2
// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format):
// loads past the stated size return zero.
constexpr int kBufferConfig = 0x00020000;

// Maximum (sum) over lanes l, l ^ 16, l ^ 32 and l ^ 48 -- the four token
// groups holding one row -- with the gfx950 lane-swap instructions rather
// than LDS permutes: swapping a value with itself across 32-lane (16-lane)
// halves leaves each lane holding its own value in one result and its
// partner's in the other.  (The results are copied out as scalars: clang
// reads element 0 for a bit cast of an indexed vector element.)
template <bool MAX>
__device__ inline float row_reduce4(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t a0 = a[0], a1 = a[1];
    const float x0 = __builtin_bit_cast(float, a0), x1 = __builtin_bit_cast(float, a1);
    x = MAX ? vmax(x0, x1) : x0 + x1;
    u = __builtin_bit_cast(uint32_t, x);
    const auto b = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t b0 = b[0], b1 = b[1];
    const float y0 = __builtin_bit_cast(float, b0), y1 = __builtin_bit_cast(float, b1);
    return MAX ? vmax(y0, y1) : y0 + y1;
}

// The running max of a row is only moved (and the row's sum and
// accumulator rescaled) once a tile's max exceeds it by more than this many
// binary orders of magnitude: until then the weights stay below 2^8, well
// inside fp32 and the 16-bit weight formats, and the result is the same
// softmax up to rounding.
constexpr float kRescaleSlack = 8.0f;

// Units are dispatched longest sequence first, so that the launch ends on
// short ones (4% less time on the chunked-prefill workload, whose lengths
// range over a factor of two): the sequence at position r of that order,
// by descending context length, ties by index.  Lane i holds sequence i's
// length and ranks it against the others' (read across lanes; a strict
// total order, so the ranks are a permutation of 0 .. S - 1); with more
// than one wave's worth of sequences the batch order is kept.
constexpr int kSortedDispatchMaxSeqs = kWave;
__device__ inline int seq_by_length_rank(const int32_t *lens, int num_seqs, int r) {
    const int i = threadIdx.x % kWave;
    const int li = i < num_seqs ? lens[i] : 0;
    int rank = 0;
    for (int j = 0; j < num_seqs; ++j) {
        const int lj = __builtin_amdgcn_readlane(li, j);
        rank += (lj > li || (lj == li && j < i)) ? 1 : 0;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(i < num_seqs && rank == r);
    return hit != 0 ? (int)__builtin_ctzll(hit) : r;
}

struct PrefillWork {
    int s, kvh, rb;  // sequence, kv head, block of query rows
};

// Workgroup id -> (unit, row block) for n_units units of nrb row blocks
// each: the row blocks of one unit read the same K/V, so they get ids 8
// apart -- the same XCD, dispatched together, sharing that XCD's L2 --
// while consecutive units go to consecutive XCDs (the units left over
// after the last whole round of 8 are numbered plainly).  rb counts from
// 0 in dispatch order.
__device__ inline void xcd_grouped(int id, int n_units, int nrb, int &unit, int &rb) {
    const int full = n_units / kXcds * kXcds;  // units placed XCD by XCD
    if (id < full * nrb) {
        const int k = id / kXcds;
        rb = k % nrb;
        unit = (k / nrb) * kXcds + id % kXcds;
    } else {
        const int r = id - full * nrb;
        unit = full + r / nrb;
        rb = r % nrb;
    }
}

// Workgroups go to the 8 XCDs round-robin.  All row blocks of one
// (sequence, kv head) unit read the same K/V, so they get ids 8 apart: the
// same XCD, dispatched together, sharing that XCD's L2.  A unit's last row
// block sees the most positions, so its row blocks are dispatched last to
// first: the launch then ends on the lightest ones (3.5% faster on the
// chunked-prefill workload than first to last).  Units go longest sequence
// first (seq_by_length_rank).
__device__ inline PrefillWork prefill_work(const PrefillParams &p, int id) {
    const int nrb = p.row_blocks;
    int unit, k;
    xcd_grouped(id, p.num_seqs * p.num_kv_heads, nrb, unit, k);
    PrefillWork w;
    w.kvh = unit % p.num_kv_heads;
    w.s = p.num_seqs <= kSortedDispatchMaxSeqs
              ? seq_by_length_rank(p.context_lens, p.num_seqs, unit / p.num_kv_heads)
              : unit / p.num_kv_heads;
    w.rb = nrb - 1 - k;
    return w;
}

// The shared-prefix pass: a unit is (prefix partition, kv head), its row
// blocks are blocks of (sequence, query head) rows; every workgroup has the
// same work, so they go in plain order within the XCD grouping (with 8 kv
// heads, XCD x serves kv head x of every partition).
struct SharedPrefixWork {
    int kvh, rb, part;  // kv head, block of rows, prefix partition
};
__device__ inline SharedPrefixWork shared_prefix_work(const PrefillParams &p, int id) {
    int unit, rb;
    xcd_grouped(id, p.prefix_parts * p.num_kv_heads, p.row_blocks, unit, rb);
    SharedPrefixWork w;
    w.kvh = unit % p.num_kv_heads;
    w.part = unit / p.num_kv_heads;
    w.rb = rb;
    return w;
}

}  // namespace pkv
