// Prefix caching on gfx950: chained hashes of every full block of a batch of
// token sequences, an open-addressing table from hash to physical block, and
// the longest cached prefix of each sequence.
//
// Requests whose token prefix is identical reuse the KV blocks already
// computed for it; each full block's hash covers the block together with
// everything before it, so any change in a prompt changes the hashes from
// that block on and only whole identical prefixes hit
// ("大模型推理框架VLLM-0.7.3源码", §2.3 and §4.2).  The hash is the polynomial
// hash of the token prefix modulo the prime P = 2^61 - 1 from a seed:
// h(empty) = seed, h(prefix, t) = h(prefix) * B + t + 1 (t read as an
// unsigned 32-bit value), and full block k's hash is h of its sequence's
// first (k + 1) * block_size tokens.
//
// Block hashes form an affine recurrence, h_k = M * h_{k-1} + L_k with
// M = B^block_size and L_k the hash of block k's tokens alone (from 0), so
// a wave hashes 64 blocks at once (one per lane) and chains them with an
// inclusive scan of the maps x -> a x + b across its lanes.

#include "device_utils.h"
#include "prefix_cache.h"

namespace pkv {
namespace {

constexpr uint64_t kP = (uint64_t(1) << 61) - 1;
constexpr uint64_t kEmptyKey = ~uint64_t(0);
constexpr int kHashThreads = 64;  // one wave per sequence

// a * b mod P for a, b < P: the 122-bit product folded twice (2^61 = 1 mod P).
__device__ inline uint64_t mulmod(uint64_t a, uint64_t b) {
    const uint64_t lo = a * b;
    const uint64_t hi = __umul64hi(a, b);
    const uint64_t s = (lo & kP) + ((lo >> 61) | (hi << 3));
    const uint64_t r = (s & kP) + (s >> 61);
    return r >= kP ? r - kP : r;
}
__device__ inline uint64_t addmod(uint64_t a, uint64_t b) {
    const uint64_t s = a + b;
    return s >= kP ? s - kP : s;
}

// Checked range [lo, hi) of a prefix-sum array, or an empty one.
__device__ inline bool range_ok(const int32_t *start, int i, int limit, int &lo, int &hi) {
    lo = start[i];
    hi = start[i + 1];
    return lo >= 0 && hi >= lo && hi <= limit;
}

__global__ __launch_bounds__(kHashThreads) void prefix_hash_kernel(
    const int32_t *__restrict__ tokens, const int32_t *__restrict__ token_start,
    const int32_t *__restrict__ block_start, int total_tokens, int total_blocks, int block_size,
    uint64_t seed, uint64_t base, uint64_t mul_block, uint64_t *__restrict__ block_hashes) {
    const int s = blockIdx.x;
    const int lane = threadIdx.x;
    int t0, t1, b0, b1;
    if (!range_ok(token_start, s, total_tokens, t0, t1) ||
        !range_ok(block_start, s, total_blocks, b0, b1))
        return;
    const int full = (t1 - t0) / block_size;
    const int nblocks = full < b1 - b0 ? full : b1 - b0;
    uint64_t carry = seed % kP;
    for (int c = 0; c < nblocks; c += kHashThreads) {
        const int k = c + lane;
        uint64_t a = 1, b = 0;  // identity map past the last block
        if (k < nblocks) {
            const int32_t *tk = tokens + t0 + (int64_t)k * block_size;
            for (int j = 0; j < block_size; ++j)
                b = addmod(mulmod(b, base), (uint64_t)(uint32_t)tk[j] + 1);
            a = mul_block;
        }
        // inclusive scan of x -> a x + b over the lanes, lane 0 applied first
#pragma unroll
        for (int d = 1; d < kHashThreads; d *= 2) {
            const uint64_t pa = __shfl_up(a, d);
            const uint64_t pb = __shfl_up(b, d);
            if (lane >= d) {
                b = addmod(mulmod(a, pb), b);
                a = mulmod(a, pa);
            }
        }
        const uint64_t h = addmod(mulmod(a, carry), b);
        if (k < nblocks) block_hashes[b0 + k] = h;
        carry = __shfl(h, kHashThreads - 1);
    }
}

__global__ __launch_bounds__(256) void prefix_insert_kernel(
    const uint64_t *__restrict__ hashes, const int32_t *__restrict__ blocks, int n,
    uint64_t *table_keys, int32_t *table_blocks, uint64_t mask, int32_t *stored) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint64_t h = hashes[i];
    int32_t result = -1;  // no free slot, or not a hash value
    if (h < kP) {
        uint64_t slot = h & mask;
        for (uint64_t probe = 0; probe <= mask; ++probe) {
            const uint64_t old = atomicCAS((unsigned long long *)&table_keys[slot],
                                           (unsigned long long)kEmptyKey,
                                           (unsigned long long)h);
            if (old == kEmptyKey) {
                table_blocks[slot] = blocks[i];
                result = 1;
                break;
            }
            if (old == h) {
                result = 0;  // already cached: the block stored first stays
                break;
            }
            slot = (slot + 1) & mask;
        }
    }
    if (stored) stored[i] = result;
}

// The block cached under h, or -1.
__device__ inline int32_t lookup(const uint64_t *table_keys, const int32_t *table_blocks,
                                 uint64_t mask, uint64_t h) {
    if (h >= kP) return -1;
    uint64_t slot = h & mask;
    for (uint64_t probe = 0; probe <= mask; ++probe) {
        const uint64_t key = table_keys[slot];
        if (key == h) return table_blocks[slot];
        if (key == kEmptyKey) return -1;
        slot = (slot + 1) & mask;
    }
    return -1;
}

__global__ __launch_bounds__(kHashThreads) void prefix_match_kernel(
    const uint64_t *__restrict__ block_hashes, const int32_t *__restrict__ block_start,
    int total_blocks, const uint64_t *__restrict__ table_keys,
    const int32_t *__restrict__ table_blocks, uint64_t mask, int32_t *__restrict__ matched_blocks,
    int32_t *__restrict__ matched_len) {
    const int s = blockIdx.x;
    const int lane = threadIdx.x;
    int b0, b1;
    if (!range_ok(block_start, s, total_blocks, b0, b1)) {
        if (lane == 0) matched_len[s] = 0;
        return;
    }
    int matched = 0;
    for (int c = b0; c < b1; c += kHashThreads) {
        const int i = c + lane;
        const int32_t blk =
            i < b1 ? lookup(table_keys, table_blocks, mask, block_hashes[i]) : -1;
        const uint64_t miss = __builtin_amdgcn_ballot_w64(blk < 0);
        const int first = miss ? __builtin_ctzll(miss) : kHashThreads;  // first uncached block
        if (lane < first && i < b1) matched_blocks[i] = blk;
        matched += first < b1 - c ? first : b1 - c;
        if (first < kHashThreads) break;
    }
    if (lane == 0) matched_len[s] = matched;
}

}  // namespace

hipError_t launch_prefix_hash(const int32_t *tokens, const int32_t *token_start,
                              const int32_t *block_start, int num_seqs, int total_tokens,
                              int total_blocks, int block_size, uint64_t seed, uint64_t base,
                              uint64_t mul_block, uint64_t *block_hashes, hipStream_t stream) {
    if (num_seqs == 0) return hipSuccess;
    hipLaunchKernelGGL(prefix_hash_kernel, dim3(num_seqs), dim3(kHashThreads), 0, stream, tokens,
                       token_start, block_start, total_tokens, total_blocks, block_size, seed,
                       base, mul_block, block_hashes);
    return hipGetLastError();
}

hipError_t launch_prefix_insert(const uint64_t *hashes, const int32_t *blocks, int n,
                                uint64_t *table_keys, int32_t *table_blocks, int capacity_log2,
                                int32_t *stored, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const uint64_t mask = (uint64_t(1) << capacity_log2) - 1;
    hipLaunchKernelGGL(prefix_insert_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, hashes,
                       blocks, n, table_keys, table_blocks, mask, stored);
    return hipGetLastError();
}

hipError_t launch_prefix_match(const uint64_t *block_hashes, const int32_t *block_start,
                               int num_seqs, int total_blocks, const uint64_t *table_keys,
                               const int32_t *table_blocks, int capacity_log2,
                               int32_t *matched_blocks, int32_t *matched_len,
                               hipStream_t stream) {
    if (num_seqs == 0) return hipSuccess;
    const uint64_t mask = (uint64_t(1) << capacity_log2) - 1;
    hipLaunchKernelGGL(prefix_match_kernel, dim3(num_seqs), dim3(kHashThreads), 0, stream,
                       block_hashes, block_start, total_blocks, table_keys, table_blocks, mask,
                       matched_blocks, matched_len);
    return hipGetLastError();
}

}  // namespace pkv
