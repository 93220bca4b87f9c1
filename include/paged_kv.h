/*
 * paged_kv.h -- C ABI of the MI355X (gfx950) paged-attention decode library.
 *
 * The library implements the decode step of PagedAttention: for every
 * sequence of a batch, the one new query token attends over the sequence's
 * whole cached history, whose keys and values live in fixed-size physical
 * blocks of a shared pool and are reached through a per-sequence block table
 * ("大模型推理框架 vllm 源码解析 一", §三, the paged_attention_v1 description;
 * "23.1 vLLM：高吞吐推理框架原理与部署", §二.2).  It also implements the
 * companion write that stores each new token's K/V in the cell named by
 * slot_mapping ("大模型推理框架VLLM-0.7.3源码", §2.1 and §3.3).
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers, owned by the caller, dense and
 *    row-major, 16-byte aligned.  The library never allocates memory and
 *    keeps no state between calls besides a cache of the device's compute
 *    unit count and of kernel occupancies, filled on first use; entry points
 *    are re-entrant.  (paged_attn_decode_noalloc also uses a fixed scratch
 *    array that the library's code object holds on each GPU.)
 *  - Element data are one dtype per call (paged_kv_dtype); index arrays are
 *    int32.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *    null stream).  A return of PAGED_KV_OK means the work was enqueued.
 *    Argument checks run on the host before anything is enqueued and never
 *    read device memory; an invalid argument returns an error code and
 *    enqueues nothing.  A failed kernel launch returns PAGED_KV_ERR_HIP.
 *  - Values that live in device memory (block ids, context lengths, slots)
 *    are checked by the kernels themselves, so a bad value never makes a
 *    kernel read or write outside the arrays described here; what the
 *    kernels do instead is stated per entry point.
 */
#ifndef PAGED_KV_H
#define PAGED_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Entry points are the library's only exported symbols. */
#define PAGED_KV_API __attribute__((visibility("default")))

typedef enum {
    PAGED_KV_F32 = 0,  /* IEEE binary32 */
    PAGED_KV_F16 = 1,  /* IEEE binary16 */
    PAGED_KV_BF16 = 2  /* bfloat16 (upper half of a binary32) */
} paged_kv_dtype;

typedef enum {
    PAGED_KV_OK = 0,
    PAGED_KV_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
    PAGED_KV_ERR_BAD_SHAPE = 2,    /* sizes inconsistent, out of range or misaligned */
    PAGED_KV_ERR_UNSUPPORTED = 3,  /* valid but not implemented (dtype, head_dim, ...) */
    PAGED_KV_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required */
    PAGED_KV_ERR_HIP = 5,          /* the HIP runtime reported an error */
    PAGED_KV_ERR_HOST_MEMORY = 6,  /* a host buffer is not pinned, device-mapped memory */
    PAGED_KV_ERR_SCRATCH_LIMIT = 7 /* needs more than the library's static scratch holds */
} paged_kv_status;

/* Human-readable name of a status code (static storage, never NULL). */
PAGED_KV_API const char *paged_kv_status_string(int status);

/*
 * Decode attention over a paged KV cache.
 *
 * For each sequence s < num_seqs and query head h < num_q_heads, with
 * L = context_lens[s], G = num_q_heads / num_kv_heads and kv head h / G:
 *   logical token j < L is read from physical block
 *   block_tables[s * max_blocks_per_seq + j / block_size] at offset
 *   j % block_size ("大模型推理框架 vllm 源码解析 一", §三 pseudo-code);
 *   x_j = scale * dot(query[s, h, :], key_cache[block, offset, h / G, :]);
 *   out[s, h, :] = sum_j softmax(x)_j * value_cache[block, offset, h / G, :].
 * Accumulation is in fp32; out is rounded to the element dtype (RNE).
 *
 * Arguments:
 *   query        [num_seqs, num_q_heads, head_dim]
 *   key_cache    [num_blocks, block_size, num_kv_heads, head_dim]
 *   value_cache  [num_blocks, block_size, num_kv_heads, head_dim]
 *   block_tables [num_seqs, max_blocks_per_seq] int32; entries at index
 *                >= ceil(L / block_size) are never read
 *   context_lens [num_seqs] int32
 *   scale        softmax scale (typically 1/sqrt(head_dim)); must be finite
 *   out          [num_seqs, num_q_heads, head_dim], written
 *   max_context_len  upper bound on every context_lens[s]; 0 means
 *                max_blocks_per_seq * block_size.  It sizes the split into
 *                context partitions and the workspace.
 *   partition_size   tokens per context partition; 0 picks one from the
 *                shape and the current device (its compute units and the
 *                decode kernel's occupancy), so query the split and the
 *                workspace size on the device that will run the decode.  An
 *                explicit value must be a positive multiple of 16 and of
 *                block_size with partition_size / block_size <= 1024.
 *                PAGED_KV_BALANCED_SPLIT asks for the balanced split instead
 *                of partitions per sequence: the positions of all sequences,
 *                each rounded up to a multiple of 16, are laid end to end
 *                and cut into equal chunks, one workgroup each (per group of
 *                kv heads), so that contexts of very different lengths still
 *                give every workgroup the same work; a sequence that lies
 *                in one chunk is finished there, the others are merged
 *                across chunks.  It takes num_seqs <= 1024 and num_seqs *
 *                (max_context_len rounded up to 16) < 2^31 (else
 *                PAGED_KV_ERR_UNSUPPORTED).
 *   workspace, workspace_bytes  device scratch of at least
 *                paged_attn_decode_workspace_bytes(...) bytes for the same
 *                arguments; may be NULL when that size is 0.  Its contents
 *                need no initialisation and are garbage afterwards.
 * Supported: dtype f32/f16/bf16; head_dim 64, 128, 256; block_size a power
 * of two in [1, 256]; num_q_heads / num_kv_heads in {1, 2, 4, 8}.
 * Device-side values: a sequence with context_len == 0 gets a zero output.
 * A sequence whose context_len is negative or above max_context_len, or one
 * of whose first ceil(L / block_size) table entries is outside
 * [0, num_blocks), gets NaN in every output element; nothing out of range
 * is read.
 * Pool size: num_blocks * block_size * num_kv_heads * head_dim may exceed
 * 2^31 elements (64-bit addressing); one block, block_size * num_kv_heads *
 * head_dim elements, must fit in 2^31 - 1 bytes (else PAGED_KV_ERR_BAD_SHAPE).
 */
#define PAGED_KV_BALANCED_SPLIT 1
PAGED_KV_API int paged_attn_decode(
    const void *query, const void *key_cache, const void *value_cache,
    const int32_t *block_tables, const int32_t *context_lens, float scale, void *out,
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
    int num_blocks, int max_blocks_per_seq, int max_context_len, int partition_size, int dtype,
    void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step in one launch: kv_cache_write of each sequence's new token
 * followed by paged_attn_decode, with the same results (pool bits and
 * output) as the two calls.  The worker writes each new token's K/V into its
 * pool cell and the kernel then reads the sequence's history, the new token
 * included ("大模型推理框架VLLM-0.7.3源码", §3.3).
 *   new_key, new_value  [num_seqs, num_kv_heads, head_dim]: sequence s's new
 *                token, same dtype as query
 *   slot_mapping [num_seqs] int32: its cell (physical_block * block_size +
 *                offset), which must be the cell of position
 *                context_lens[s] - 1 of sequence s (the only cell of the
 *                launch it then writes and reads); a negative slot, or one
 *                outside the pool, writes nothing
 *   key_cache, value_cache  updated in place
 * Every other argument, check and status is paged_attn_decode's, except
 * that partition_size PAGED_KV_BALANCED_SPLIT returns
 * PAGED_KV_ERR_UNSUPPORTED.
 */
PAGED_KV_API int paged_attn_decode_write(
    const void *query, const void *new_key, const void *new_value, const int32_t *slot_mapping,
    void *key_cache, void *value_cache, const int32_t *block_tables, const int32_t *context_lens,
    float scale, void *out, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int block_size, int num_blocks, int max_blocks_per_seq, int max_context_len,
    int partition_size, int dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_attn_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments (minus the workspace), checks, kernels and
 * results, bit for bit, as paged_attn_decode; the split-context partials go
 * to a scratch buffer the library itself holds in device memory, one per
 * GPU, PAGED_KV_NOALLOC_SCRATCH_BYTES bytes, kept until the process ends
 * (its address is looked up on a device's first call, with that device
 * current).  Nothing is allocated by the call, on the host or the device.
 *   A call whose split needs more scratch than that
 * (paged_attn_decode_workspace_bytes(...) > PAGED_KV_NOALLOC_SCRATCH_BYTES)
 * returns PAGED_KV_ERR_SCRATCH_LIMIT and enqueues nothing; pass a larger
 * partition_size, or use paged_attn_decode with a workspace.
 *   The current device must be the one `stream` runs on.  Every call on one
 * GPU shares that GPU's scratch: two calls that may run at the same time on
 * one GPU (different streams, or different host threads without ordering)
 * race on it and may return wrong results.  Calls ordered on one stream are
 * safe.  The scratch needs no initialisation: every value the merge reads
 * is written earlier in the same call.
 */
#define PAGED_KV_NOALLOC_SCRATCH_BYTES (32u << 20)
PAGED_KV_API int paged_attn_decode_noalloc(
    const void *query, const void *key_cache, const void *value_cache,
    const int32_t *block_tables, const int32_t *context_lens, float scale, void *out,
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
    int num_blocks, int max_blocks_per_seq, int max_context_len, int partition_size, int dtype,
    void *stream);

/*
 * paged_attn_decode for a batch whose sequences all begin with the same
 * prefix_len positions held in the same physical blocks: a common prompt,
 * parallel samples or beams of one prompt, whose blocks the sequences share
 * ("23.1 vLLM：高吞吐推理框架原理与部署", §二.3).  Same result as
 * paged_attn_decode up to rounding, computed in three launches on the
 * caller's stream:
 *   1. the prefix pass: for each kv head, every sequence's query rows at
 *      once against the shared positions, read once, as two matrix products
 *      on the matrix cores (the prefill kernel's tiles), in partitions of
 *      prefix_partition_size positions;
 *   2. the decode kernels over each sequence's positions [prefix_len, L), in
 *      partitions of partition_size;
 *   3. the merge of the two passes' partial results per (sequence, head).
 *   prefix_len   positions every sequence shares: a multiple of 16 and of
 *                block_size, at most max_context_len.  The caller promises
 *                that every sequence's first prefix_len / block_size table
 *                entries equal the first row's and that every context_len
 *                is at least prefix_len.  0 runs paged_attn_decode.
 *   prefix_partition_size  positions per partition of the prefix pass; 0
 *                picks one (about one workgroup per compute unit), else a
 *                positive multiple of 64.
 *   partition_size  positions per partition after the prefix; 0 picks one
 *                (enough workgroups to fill the device once), else as for
 *                paged_attn_decode; PAGED_KV_BALANCED_SPLIT is
 *                PAGED_KV_ERR_UNSUPPORTED when prefix_len > 0.
 *   workspace, workspace_bytes  device scratch of at least
 *                paged_attn_decode_shared_prefix_workspace_bytes(...) bytes
 *                (never 0 with a prefix), 16-byte aligned; no
 *                initialisation needed, garbage afterwards.
 * Every other argument is paged_attn_decode's.  Supported: f32, f16, bf16
 * (the prefix pass on fp32 matrix instructions for f32), head_dim 64, 128,
 * 256, num_q_heads / num_kv_heads in {1, 2, 4, 8}, block_size a power of two
 * in [1, 256].
 * Device-side values: a sequence whose context_len is below prefix_len
 * (0 included), negative or above max_context_len, or whose first
 * prefix_len / block_size table entries differ from the first row's, gets
 * NaN in every output element; a table entry outside [0, num_blocks) among
 * the shared ones makes every sequence's output NaN, one after the prefix
 * only its own sequence's.  Nothing out of range is read.
 */
PAGED_KV_API int paged_attn_decode_shared_prefix(
    const void *query, const void *key_cache, const void *value_cache,
    const int32_t *block_tables, const int32_t *context_lens, float scale, void *out,
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
    int num_blocks, int max_blocks_per_seq, int max_context_len, int prefix_len,
    int prefix_partition_size, int partition_size, int dtype, void *workspace,
    size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace paged_attn_decode_shared_prefix needs for these
 * arguments ((size_t)-1 for invalid ones): fp32 partial results (running
 * max, running sum, head_dim output values) per (sequence, query head) and
 * partition of either pass.
 */
PAGED_KV_API size_t paged_attn_decode_shared_prefix_workspace_bytes(
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
    int max_blocks_per_seq, int max_context_len, int prefix_len, int prefix_partition_size,
    int partition_size, int dtype);

/*
 * The context partition size paged_attn_decode uses for these arguments
 * (partition_size 0 = its automatic choice), or a negative paged_kv_status
 * code when the arguments are invalid.  A partition size >= max_context_len
 * means no split: one pass writes out directly; PAGED_KV_BALANCED_SPLIT
 * (when asked for) means the balanced split.
 */
PAGED_KV_API int paged_attn_decode_partition_size(
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
    int max_blocks_per_seq, int max_context_len, int partition_size, int dtype);

/*
 * A partition size to pass to paged_attn_decode when the caller holds the
 * batch's context lengths on the host (as the scheduler that builds the
 * batch does): host_context_lens [num_seqs] int32 in host memory, read here
 * and not kept.  The automatic choice sizes partitions from the longest
 * context; when the batch needs a split and its lengths are very uneven
 * (the longest above 1.5 times the mean) this returns
 * PAGED_KV_BALANCED_SPLIT instead (or, where that split does not apply, the
 * finest split), so that the long contexts' workgroups do not finish far
 * behind the rest.  A negative paged_kv_status code when the arguments are
 * invalid.
 */
PAGED_KV_API int paged_attn_decode_partition_size_for_lengths(
    const int32_t *host_context_lens, int num_seqs, int num_q_heads, int num_kv_heads,
    int head_dim, int block_size, int max_blocks_per_seq, int dtype);

/*
 * Bytes of workspace paged_attn_decode needs for these arguments (0 when the
 * context is not split); (size_t)-1 for invalid arguments.  The split-context
 * partials are fp32: per (sequence, query head, partition) -- or, with the
 * balanced split, per (chunk, 2 slots, query head) -- a running max, a
 * running sum and head_dim unnormalised output values.
 */
PAGED_KV_API size_t paged_attn_decode_workspace_bytes(
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
    int max_blocks_per_seq, int max_context_len, int partition_size, int dtype);

/*
 * Store new tokens' keys and values in the paged pool.
 *
 * For each t < num_tokens with slot = slot_mapping[t]:
 *   key_cache[slot / block_size, slot % block_size, :, :]   = key[t, :, :]
 *   value_cache[slot / block_size, slot % block_size, :, :] = value[t, :, :]
 * as a bit copy ("大模型推理框架VLLM-0.7.3源码", §2.1: slot_mapping tells the
 * operator which cell each token's KV goes to).
 *   key, value   [num_tokens, num_kv_heads, head_dim]
 *   slot_mapping [num_tokens] int32
 *   key_cache, value_cache  [num_blocks, block_size, num_kv_heads, head_dim]
 * Device-side values: a slot < 0 or >= num_blocks * block_size writes
 * nothing.  Two tokens with the same slot in one call leave either token's
 * row (unspecified which).  Writing into a block that several sequences
 * share is the caller's responsibility (copy it first).
 */
PAGED_KV_API int kv_cache_write(
    const void *key, const void *value, const int32_t *slot_mapping, void *key_cache,
    void *value_cache, int num_tokens, int num_kv_heads, int head_dim, int block_size,
    int num_blocks, int dtype, void *stream);

/*
 * Multi-token (chunked-prefill) attention over a paged KV cache.
 *
 * Sequence s holds L = context_lens[s] tokens in the pool, the last q_len of
 * which are new: a prompt, or a chunk of one, processed in the same batch as
 * decoding sequences ("23.1 vLLM：高吞吐推理框架原理与部署", §二.2;
 * "大模型推理框架VLLM-0.7.3源码", §3.2).  Their keys and values are already
 * in the pool (kv_cache_write), and their queries are rows
 * query_start[s] .. query_start[s+1] - 1 of query (q_len of them).  New
 * token i sits at position L - q_len + i and attends over positions
 * 0 .. L - q_len + i of its sequence -- every earlier token and itself:
 *   x_j = scale * dot(query[row, h, :], key_cache[block, offset, h / G, :]),
 *   out[row, h, :] = sum_j softmax(x)_j * value_cache[block, offset, h / G, :],
 * with position j at block block_tables[s][j / block_size], offset
 * j % block_size ("大模型推理框架 vllm 源码解析 一", §三).  With q_len = 1
 * this is paged_attn_decode.  Accumulation is fp32 (for f16 and bf16 the
 * weights enter the value product rounded to the element type; f32 runs
 * on the fp32 matrix instructions throughout); out is rounded to nearest
 * even.
 *
 * Arguments:
 *   query, out     [total_q, num_q_heads, head_dim]
 *   key_cache, value_cache  [num_blocks, block_size, num_kv_heads, head_dim]
 *   block_tables   [num_seqs, max_blocks_per_seq] int32
 *   context_lens   [num_seqs] int32, L including the new tokens
 *   query_start    [num_seqs + 1] int32, non-decreasing, query_start[0] = 0,
 *                  query_start[num_seqs] = total_q
 *   max_query_len  upper bound on every q_len (sizes the grid)
 *   max_context_len  upper bound on every L; 0 means
 *                  max_blocks_per_seq * block_size
 * Supported: dtype f32, f16, bf16; head_dim 64,
 * 128, 256; num_q_heads / num_kv_heads in {1, 2, 4, 8}; block_size a power
 * of two in [1, 256].  No workspace; nothing is allocated.
 * Device-side values: a sequence with q_len > L or L > max_context_len gets
 * NaN rows; a table entry outside [0, num_blocks) makes the rows that read
 * it NaN (every row of the sequence when few new tokens take the decode's
 * structure, below); rows past max_query_len are not written, nor are the
 * rows of a sequence whose query_start range leaves [0, total_q] or
 * decreases.  Nothing out of range is read or written.
 * Few new tokens (max_query_len * num_q_heads / num_kv_heads <= 32, or 16
 * at head_dim 256; f16 or bf16) in a batch the decode's plan does not split
 * run the decode kernel's structure, one wave per kv head (the multi-token
 * decode): the same results to rounding, with one new token the decode's
 * bits.
 */
PAGED_KV_API int paged_attn_prefill(
    const void *query, const void *key_cache, const void *value_cache,
    const int32_t *block_tables, const int32_t *context_lens, const int32_t *query_start,
    float scale, void *out, int num_seqs, int total_q, int num_q_heads, int num_kv_heads,
    int head_dim, int block_size, int num_blocks, int max_blocks_per_seq, int max_query_len,
    int max_context_len, int dtype, void *stream);

/*
 * Copy-on-write block copy: before a sequence writes into a block that other
 * sequences still reference (a shared prompt prefix, parallel samples or
 * beams), the block is copied to a block of the sequence's own
 * ("23.1 vLLM：高吞吐推理框架原理与部署", §二.3).
 *
 * For each pair i < num_pairs with src = block_mapping[2 * i] and
 * dst = block_mapping[2 * i + 1]: all block_size slots of all kv heads of
 * physical block dst, in both key_cache and value_cache, become a bit copy
 * of block src.
 *   key_cache, value_cache  [num_blocks, block_size, num_kv_heads, head_dim],
 *                updated in place
 *   block_mapping [num_pairs, 2] int32 (src, dst), device memory
 * Device-side values: a pair whose src or dst is outside [0, num_blocks)
 * copies nothing.  Pairs run in parallel: a dst that appears twice, or that
 * is also a src in the same call, leaves an unspecified result.
 * One block (block_size * num_kv_heads * head_dim elements) must be a
 * multiple of 16 bytes and at most 4 GiB (else PAGED_KV_ERR_BAD_SHAPE).
 */
PAGED_KV_API int paged_kv_copy_blocks(
    void *key_cache, void *value_cache, const int32_t *block_mapping, int num_pairs,
    int num_kv_heads, int head_dim, int block_size, int num_blocks, int dtype, void *stream);

/*
 * Block swap for preemption: when GPU memory runs short the scheduler moves
 * a preempted sequence's KV blocks out to CPU memory instead of refusing
 * work, and brings them back (into whatever device blocks are free) when
 * the sequence resumes ("大模型推理框架 vllm 源码解析 一", §三, and the CPU
 * swap-space option of §四; "大模型推理框架VLLM-0.7.3源码", §2.2 on the swapped
 * queue).
 *
 * Swap-out: for each pair i < num_pairs with from = block_mapping[2 * i]
 * (device block) and to = block_mapping[2 * i + 1] (host block), all
 * block_size slots of all kv heads of host block `to`, in both host pools,
 * become a bit copy of device block `from`.  Swap-in is the reverse: from is
 * a host block and to a device block.
 *   key_cache, value_cache  device pools [num_blocks, block_size,
 *                num_kv_heads, head_dim]
 *   host_key_cache, host_value_cache  host pools [num_host_blocks,
 *                block_size, num_kv_heads, head_dim] in pinned, device-mapped
 *                host memory (hipHostMalloc, or a pinned torch tensor); any
 *                other host memory returns PAGED_KV_ERR_HOST_MEMORY and
 *                enqueues nothing.  The kernel reads or writes it directly
 *                over the host link.
 *   block_mapping [num_pairs, 2] int32 (from, to), device memory
 * The destination pools are updated in place; the caller keeps the host
 * pools alive and unmodified until the stream has passed the call.
 * Device-side values: a pair with an id outside its pool copies nothing.
 * Pairs run in parallel: a `to` that appears twice leaves an unspecified
 * result.  One block must be a multiple of 16 bytes and at most 4 GiB (else
 * PAGED_KV_ERR_BAD_SHAPE).
 */
PAGED_KV_API int paged_kv_swap_out(
    const void *key_cache, const void *value_cache, void *host_key_cache,
    void *host_value_cache, const int32_t *block_mapping, int num_pairs, int num_kv_heads,
    int head_dim, int block_size, int num_blocks, int num_host_blocks, int dtype, void *stream);

PAGED_KV_API int paged_kv_swap_in(
    const void *host_key_cache, const void *host_value_cache, void *key_cache,
    void *value_cache, const int32_t *block_mapping, int num_pairs, int num_kv_heads,
    int head_dim, int block_size, int num_blocks, int num_host_blocks, int dtype, void *stream);

/*
 * Prefix caching: requests whose token prefix is identical reuse the KV
 * blocks already computed for it.  Each full block is identified by a hash
 * of the block together with everything before it, so any change in a
 * prompt changes the hashes from that block on and only whole identical
 * prefixes hit ("大模型推理框架VLLM-0.7.3源码", §2.3 and §4.2; the shared
 * system prompt of "23.1 vLLM：高吞吐推理框架原理与部署").
 *
 * The hash (the pages fix none): the polynomial hash of the token prefix
 * modulo the prime P = 2^61 - 1, from a seed, by Horner's rule:
 *   h(empty) = seed mod P,  h(prefix, t) = (h(prefix) * B + t + 1) mod P
 * with B = PAGED_KV_PREFIX_HASH_BASE and each token read as an unsigned
 * 32-bit value; full block k of a sequence hashes to h of the sequence's
 * first (k + 1) * block_size tokens.  Every hash is below 2^61 - 1.  The seed
 * keeps hashes of different namespaces (models, adapters) apart.
 */
#define PAGED_KV_PREFIX_HASH_BASE 0x1C6A8B2F3E5D7093ull
/* The key of an empty slot of a prefix table: every key slot starts as this. */
#define PAGED_KV_PREFIX_EMPTY_KEY 0xFFFFFFFFFFFFFFFFull

/*
 * Hashes of every full block of a batch of token sequences.
 *   tokens       [total_tokens] int32, the sequences one after another
 *   token_start  [num_seqs + 1] int32: sequence s holds tokens
 *                token_start[s] .. token_start[s+1] - 1
 *   block_start  [num_seqs + 1] int32: sequence s's hashes go to
 *                block_hashes[block_start[s] ..] (prefix sums of the full-block
 *                counts, computed by the caller)
 *   block_hashes [total_blocks] uint64, written: block_hashes[block_start[s]
 *                + k] for k < min(full blocks of s, block_start[s+1] -
 *                block_start[s]); a trailing partial block has no hash and
 *                other slots are left as they are
 * All device memory.  Device-side values: a sequence whose token_start or
 * block_start range leaves its array or decreases is skipped.
 * block_size in [1, 4096].
 */
PAGED_KV_API int paged_kv_prefix_hash(
    const int32_t *tokens, const int32_t *token_start, const int32_t *block_start, int num_seqs,
    int total_tokens, int total_blocks, int block_size, uint64_t seed, uint64_t *block_hashes,
    void *stream);

/*
 * Record cached blocks: entry i maps hashes[i] to physical block blocks[i]
 * in an open-addressing table of 2^capacity_log2 slots (linear probing from
 * slot hash mod capacity).  table_keys [capacity] uint64 (every slot starts
 * as PAGED_KV_PREFIX_EMPTY_KEY), table_blocks [capacity] int32, caller-owned
 * device memory, updated in place.  stored [num_entries] int32 (device,
 * optional): 1 = inserted, 0 = the hash was already there (the block stored
 * first stays), -1 = no free slot or not a hash value (>= 2^61 - 1).
 * Entries run in parallel: two entries with one hash leave either block.
 * capacity_log2 in [1, 30]; keep the table at most about half full.
 */
PAGED_KV_API int paged_kv_prefix_insert(
    const uint64_t *hashes, const int32_t *blocks, int num_entries, uint64_t *table_keys,
    int32_t *table_blocks, int capacity_log2, int32_t *stored, void *stream);

/*
 * The longest cached prefix of each sequence: matched_len[s] = the number of
 * leading blocks of s (block_hashes[block_start[s]], [block_start[s] + 1],
 * ...) whose hashes are all in the table, and matched_blocks[block_start[s]
 * + k] = the cached block for k < matched_len[s] (the entries after are
 * left as they are).  The walk stops at the first uncached block even when
 * later hashes are cached.  All device memory; matched_blocks [total_blocks]
 * int32, matched_len [num_seqs] int32.  A sequence whose block_start range
 * leaves the array or decreases matches nothing.
 */
PAGED_KV_API int paged_kv_prefix_match(
    const uint64_t *block_hashes, const int32_t *block_start, int num_seqs, int total_blocks,
    const uint64_t *table_keys, const int32_t *table_blocks, int capacity_log2,
    int32_t *matched_blocks, int32_t *matched_len, void *stream);

/*
 * Materialise each sequence's logical K/V through its block table (the
 * addressing of paged_attn_decode, as a bit copy); used to check the
 * addressing on its own.
 *   out_key, out_value [num_seqs, max_context_len, num_kv_heads, head_dim]
 * Position j < min(context_lens[s], max_context_len) receives logical token
 * j; later positions are left untouched.  A table entry outside
 * [0, num_blocks) fills the rows it would supply with NaN.
 */
PAGED_KV_API int paged_kv_gather(
    const void *key_cache, const void *value_cache, const int32_t *block_tables,
    const int32_t *context_lens, void *out_key, void *out_value, int num_seqs, int num_kv_heads,
    int head_dim, int block_size, int num_blocks, int max_blocks_per_seq, int max_context_len,
    int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H */
