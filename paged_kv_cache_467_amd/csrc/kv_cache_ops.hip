// Paged KV cache write (slot_mapping scatter) and block-table gather.
//
// Write: each new token's K and V rows ([num_kv_heads, head_dim] contiguous)
// are copied to the pool cell named by slot_mapping, where a slot is
// physical_block * block_size + offset ("大模型推理框架VLLM-0.7.3源码", §2.1;
// the pool is [num_blocks, block_size, num_kv_heads, head_dim], so a cell's
// row starts at slot * num_kv_heads * head_dim elements).
// Gather: the inverse view used to check the addressing on its own -- each
// sequence's logical tokens are read through its block table
// ("大模型推理框架 vllm 源码解析 一", §三 pseudo-code) into a dense array.
//
// Block copy: copy-on-write of a shared block -- before a sequence writes
// into a block that other sequences still reference, the block's contents
// go to a block of its own ("23.1 vLLM：高吞吐推理框架原理与部署", §二.3);
// each (src, dst) pair copies all block_size slots of every kv head, in both
// pools.
//
// All three are bit copies done with 16-byte vector loads and stores.

#include "kv_ops.h"
#include "device_utils.h"

namespace pkv {
namespace {

constexpr int kCopyThreads = 256;

// One lane per 16-byte chunk of a token's row (K and V): the chunks of all
// tokens are numbered in one range, so a workgroup covers whole rows of
// several tokens when rows are short and part of one when they are long,
// and no lane idles but in the last workgroup.  Each lane issues its slot
// read and its two row loads together (the rows do not depend on the
// slot), so the write waits for one memory round trip before its stores.
// Slots outside [0, num_slots) write nothing.
__global__ __launch_bounds__(kCopyThreads) void kv_cache_write_kernel(
    const char *__restrict__ key, const char *__restrict__ value,
    const int32_t *__restrict__ slot_mapping, char *__restrict__ key_cache,
    char *__restrict__ value_cache, int row_chunks, int64_t num_chunks, int64_t num_slots) {
    const int64_t g = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x;
    if (g >= num_chunks) return;
    const int t = (int)(g / row_chunks);
    const int c = (int)(g - (int64_t)t * row_chunks);
    const int slot = slot_mapping[t];
    const u32x4 k = load16(key + g * 16);
    const u32x4 v = load16(value + g * 16);
    if (slot < 0 || (int64_t)slot >= num_slots) return;
    const int64_t dst = ((int64_t)slot * row_chunks + c) * 16;
    store16(key_cache + dst, k);
    store16(value_cache + dst, v);
}

// One workgroup per (sequence, logical block).  A block of the pool holds
// block_size consecutive token rows, so a logical block is one contiguous
// run of bytes in both the pool and the output.
__global__ __launch_bounds__(kCopyThreads) void paged_kv_gather_kernel(
    const char *__restrict__ key_cache, const char *__restrict__ value_cache,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    char *__restrict__ out_key, char *__restrict__ out_value, int max_blocks_per_seq,
    int block_size, int num_blocks, int max_context_len, int row_bytes, int elem_bytes) {
    const int s = blockIdx.y;
    const int lb = blockIdx.x;
    int L = context_lens[s];
    if (L > max_context_len) L = max_context_len;
    const int first = lb * block_size;
    if (first >= L) return;
    const int ntok = (L - first) < block_size ? (L - first) : block_size;
    const int blk = block_tables[(int64_t)s * max_blocks_per_seq + lb];
    const int64_t bytes = (int64_t)ntok * row_bytes;
    const int64_t dst = ((int64_t)s * max_context_len + first) * row_bytes;
    if (blk < 0 || blk >= num_blocks) {
        // out-of-range table entry: NaN rows, nothing read
        // f32 quiet NaN, or two bf16 quiet NaNs (also a NaN pattern as f16)
        const uint32_t bits = elem_bytes == 4 ? 0x7FC00000u : 0x7FC07FC0u;
        const u32x4 nan = u32x4{bits, bits, bits, bits};
        for (int64_t b = threadIdx.x * 16; b < bytes; b += kCopyThreads * 16) {
            store16(out_key + dst + b, nan);
            store16(out_value + dst + b, nan);
        }
        return;
    }
    const int64_t src = (int64_t)blk * block_size * row_bytes;
    for (int64_t b = threadIdx.x * 16; b < bytes; b += kCopyThreads * 16) {
        store16(out_key + dst + b, load16(key_cache + src + b));
        store16(out_value + dst + b, load16(value_cache + src + b));
    }
}

// Block copy from one pool pair into another of the same block shape (one
// pool pair for a copy-on-write copy; device and pinned host pools for a
// swap): grid (pair, pool, chunk of up to kCopyChunkBytes of the block).  A
// pair whose from or to id leaves its pool copies nothing.  Every byte is
// touched once, so loads and stores are non-temporal.
constexpr int kCopyChunkBytes = 64 * 1024;
constexpr int kCopyUnroll = 4;

struct BlockCopy {
    const char *src_key, *src_value;
    char *dst_key, *dst_value;
    int num_src_blocks, num_dst_blocks;
};

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    BlockCopy c, const int32_t *__restrict__ block_mapping, int64_t block_bytes) {
    const int pair = blockIdx.x;
    const int src = block_mapping[2 * pair];
    const int dst = block_mapping[2 * pair + 1];
    if (src < 0 || src >= c.num_src_blocks || dst < 0 || dst >= c.num_dst_blocks) return;
    const int64_t begin = (int64_t)blockIdx.z * kCopyChunkBytes;
    const int64_t end = begin + kCopyChunkBytes < block_bytes ? begin + kCopyChunkBytes : block_bytes;
    const char *from = (blockIdx.y == 0 ? c.src_key : c.src_value) + (int64_t)src * block_bytes;
    char *to = (blockIdx.y == 0 ? c.dst_key : c.dst_value) + (int64_t)dst * block_bytes;
    constexpr int kStep = kCopyThreads * 16;
    int64_t b = begin + threadIdx.x * 16;
    for (; b + (kCopyUnroll - 1) * kStep < end; b += kCopyUnroll * kStep) {
        u32x4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) v[u] = load16_stream(from + b + u * kStep);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) store16_stream(to + b + u * kStep, v[u]);
    }
    for (; b < end; b += kStep) store16_stream(to + b, load16_stream(from + b));
}

}  // namespace

hipError_t launch_copy_blocks(const void *src_key, const void *src_value, int num_src_blocks,
                              void *dst_key, void *dst_value, int num_dst_blocks,
                              const int32_t *block_mapping, int num_pairs, int64_t block_bytes,
                              hipStream_t stream) {
    if (num_pairs == 0) return hipSuccess;
    const unsigned chunks = (unsigned)((block_bytes + kCopyChunkBytes - 1) / kCopyChunkBytes);
    const BlockCopy c{static_cast<const char *>(src_key), static_cast<const char *>(src_value),
                      static_cast<char *>(dst_key), static_cast<char *>(dst_value),
                      num_src_blocks, num_dst_blocks};
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2, chunks), dim3(kCopyThreads), 0,
                       stream, c, block_mapping, block_bytes);
    return hipGetLastError();
}

hipError_t launch_kv_cache_write(const void *key, const void *value, const int32_t *slot_mapping,
                                 void *key_cache, void *value_cache, int num_tokens,
                                 int row_bytes, int64_t num_slots, hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    const int row_chunks = row_bytes / 16;  // row_bytes is a multiple of 16
    const int64_t chunks = (int64_t)num_tokens * row_chunks;
    const int64_t groups = (chunks + kCopyThreads - 1) / kCopyThreads;
    if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kv_cache_write_kernel, dim3((unsigned)groups), dim3(kCopyThreads), 0,
                       stream, static_cast<const char *>(key), static_cast<const char *>(value),
                       slot_mapping, static_cast<char *>(key_cache),
                       static_cast<char *>(value_cache), row_chunks, chunks, num_slots);
    return hipGetLastError();
}

hipError_t launch_paged_kv_gather(const void *key_cache, const void *value_cache,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  void *out_key, void *out_value, int num_seqs,
                                  int max_blocks_per_seq, int block_size, int num_blocks,
                                  int max_context_len, int row_bytes, int elem_bytes,
                                  hipStream_t stream) {
    const int nlb = (max_context_len + block_size - 1) / block_size;
    if (num_seqs == 0 || nlb == 0) return hipSuccess;
    hipLaunchKernelGGL(paged_kv_gather_kernel, dim3(nlb, num_seqs), dim3(kCopyThreads), 0,
                       stream, static_cast<const char *>(key_cache),
                       static_cast<const char *>(value_cache), block_tables, context_lens,
                       static_cast<char *>(out_key), static_cast<char *>(out_value),
                       max_blocks_per_seq, block_size, num_blocks, max_context_len, row_bytes,
                       elem_bytes);
    return hipGetLastError();
}

}  // namespace pkv
