/*
 * CPU oracle for paged-attention decode and the paged KV cache write.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
 * bench's CPU-baseline leg may load this library.  It shares no code with
 * the HIP path and is deliberately plain and slow: every result is computed
 * in fp64 straight from the definition, one (sequence, query head) at a time.
 *
 * What it computes, and where that is stated:
 *  - Paged addressing: logical token j of a sequence lives in physical block
 *    block_tables[s][j / block_size] at offset j % block_size of the pool
 *    key_cache/value_cache[num_blocks, block_size, num_heads, head_dim]
 *    ("大模型推理框架 vllm 源码解析 一", §三, the paged_attention_v1
 *    pseudo-code and the shape it gives for key_cache/value_cache).
 *  - Decode attention: the current token's query attends over all
 *    context_lens[s] cached tokens of its sequence (same passage; and
 *    "23.1 vLLM：高吞吐推理框架原理与部署", §二.2 step 3).  The pages only
 *    say "compute attention scores"; the score function used here is the
 *    standard scaled dot product followed by a softmax over the sequence's
 *    tokens, with the scale given by the caller.  Query head h reads kv head
 *    h / (num_q_heads / num_kv_heads), i.e. consecutive query heads share a
 *    kv head.
 *  - Split-context decode: partition p of a sequence covers tokens
 *    [p*P, min((p+1)*P, L)); each partition yields its running max m_p, sum
 *    l_p and unnormalised output o_p, and the partitions are merged with
 *    weights exp(m_p - M).  The pages name this only as segmented attention
 *    over scattered blocks ("23.1 vLLM", §二.2 step 3).
 *  - KV write: new token t's K and V rows go to the cell slot_mapping[t],
 *    read as physical_block * block_size + offset; a negative slot writes
 *    nothing ("大模型推理框架VLLM-0.7.3源码", §2.1 on slot_mapping).
 *  - Gather: materialise each sequence's logical K/V through its block
 *    table (the same addressing, as a bit copy).
 *  - Multi-token (chunked-prefill) attention: a sequence adds q_len new
 *    tokens at once (a prompt, or a chunk of one, processed together with
 *    decoding sequences in one batch: "23.1 vLLM：高吞吐推理框架原理与部署",
 *    §二.2 and continuous batching; "大模型推理框架VLLM-0.7.3源码", §3.2).
 *    Their keys and values are already in the pool at positions
 *    L - q_len .. L - 1 of the sequence, and new token i (position
 *    L - q_len + i) attends over positions 0 .. L - q_len + i -- every
 *    earlier token and itself, never a later one (causal).  With q_len = 1
 *    this is the decode above.
 *  - Block copy: copy-on-write of shared blocks -- before a sequence writes
 *    into a block it shares with others, the block's contents are copied to
 *    a block of its own ("23.1 vLLM：高吞吐推理框架原理与部署", §二.3).  Each
 *    (src, dst) pair copies every slot of physical block src to block dst,
 *    in both pools; a negative id skips the pair.
 *  - Prefix hashing: requests whose token prefix is identical reuse the KV
 *    blocks already computed for it; the prefix of each full block is
 *    hashed, chained to everything before it, so that any change anywhere
 *    in the prompt changes the hashes from that block on
 *    ("大模型推理框架VLLM-0.7.3源码", §2.3 and §4.2).  The pages fix no hash
 *    function; the one used here is the polynomial hash of the token
 *    sequence modulo the prime 2^61 - 1, evaluated by Horner's rule from a
 *    seed: h(empty) = seed, h(prefix, t) = h(prefix) * base + t + 1, and
 *    full block k's hash is h of the first (k + 1) * block_size tokens.
 *  - Block swap: when GPU memory runs short the scheduler preempts a
 *    sequence and moves its KV blocks out to CPU memory rather than
 *    refusing work, and a swapped sequence goes back to running first once
 *    memory allows ("大模型推理框架 vllm 源码解析 一", §三; the size of the
 *    CPU swap area is a serving option, §四; "大模型推理框架VLLM-0.7.3源码",
 *    §2.2 on the swapped queue).  Each (from, to) pair copies block `from`
 *    of a source pool pair to block `to` of a destination pool pair of the
 *    same block shape; swap-out and swap-in differ only in which pools are
 *    which.
 *
 * Element types: f32 (code 0), f16 (code 1, IEEE binary16), bf16 (code 2,
 * the upper half of a binary32).  Inputs are read as stored bits and widened
 * to double exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };

static int element_bytes(int dtype) { return dtype == ORACLE_F32 ? 4 : 2; }

/* binary16: sign, 5-bit exponent (bias 15), 10-bit fraction. */
static double half_bits_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exponent = (h >> 10) & 0x1f;
    int fraction = h & 0x3ff;
    double v;
    if (exponent == 0)
        v = ldexp((double)fraction, -24); /* subnormal: fraction * 2^-24 */
    else if (exponent == 31)
        v = fraction ? NAN : INFINITY;
    else
        v = ldexp((double)(fraction + 1024), exponent - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the high 16 bits of a binary32. */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double element(const void *base, int64_t index, int dtype)
{
    const unsigned char *p = (const unsigned char *)base + index * element_bytes(dtype);
    if (dtype == ORACLE_F32) {
        float f;
        memcpy(&f, p, sizeof f);
        return (double)f;
    }
    uint16_t b;
    memcpy(&b, p, sizeof b);
    return dtype == ORACLE_F16 ? half_bits_to_double(b) : bf16_bits_to_double(b);
}

/* Index (in elements) of the first element of row (block_id, offset, kv_head)
 * of a [num_blocks, block_size, num_kv_heads, head_dim] pool. */
static int64_t pool_row(int64_t block_id, int offset, int kv_head, int block_size,
                        int num_kv_heads, int head_dim)
{
    return ((block_id * block_size + offset) * num_kv_heads + kv_head) * (int64_t)head_dim;
}

void oracle_elements_to_double(const void *bits, int64_t n, int dtype, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = element(bits, i, dtype);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * out: [num_seqs, num_q_heads, head_dim] fp64.
 * weights (may be NULL): [num_seqs, num_q_heads, weights_stride] fp64; the
 * softmax weight of token j is stored at index j (j < context_lens[s]).
 * A sequence with context_len <= 0 gets an all-zero output.
 */
void oracle_paged_attention_decode(const void *query, const void *key_cache,
                                   const void *value_cache, const int32_t *block_tables,
                                   const int32_t *context_lens, float scale, int num_seqs,
                                   int num_q_heads, int num_kv_heads, int head_dim,
                                   int block_size, int max_blocks_per_seq, int dtype,
                                   double *out, double *weights, int weights_stride)
{
    const int group = num_q_heads / num_kv_heads;
    const int64_t units = (int64_t)num_seqs * num_q_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t unit = 0; unit < units; ++unit) {
        const int s = (int)(unit / num_q_heads);
        const int h = (int)(unit % num_q_heads);
        const int kv_head = h / group;
        const int context_len = context_lens[s];
        const int32_t *blocks = block_tables + (int64_t)s * max_blocks_per_seq;
        const int64_t q0 = ((int64_t)s * num_q_heads + h) * head_dim;
        double *o = out + unit * head_dim;
        for (int d = 0; d < head_dim; ++d)
            o[d] = 0.0;
        if (context_len <= 0)
            continue;

        /* attention scores x_j = scale * q . k_j */
        double *x = (double *)malloc(sizeof(double) * (size_t)context_len);
        for (int j = 0; j < context_len; ++j) {
            const int block_id = blocks[j / block_size];
            const int offset = j % block_size;
            const int64_t k0 = pool_row(block_id, offset, kv_head, block_size, num_kv_heads,
                                        head_dim);
            double dot = 0.0;
            for (int d = 0; d < head_dim; ++d)
                dot += element(query, q0 + d, dtype) * element(key_cache, k0 + d, dtype);
            x[j] = (double)scale * dot;
        }

        /* softmax over the sequence's tokens */
        double m = x[0];
        for (int j = 1; j < context_len; ++j)
            if (x[j] > m)
                m = x[j];
        double sum = 0.0;
        for (int j = 0; j < context_len; ++j)
            sum += exp(x[j] - m);

        /* weighted sum of the value rows */
        for (int j = 0; j < context_len; ++j) {
            const double w = exp(x[j] - m) / sum;
            if (weights)
                weights[unit * weights_stride + j] = w;
            const int block_id = blocks[j / block_size];
            const int offset = j % block_size;
            const int64_t v0 = pool_row(block_id, offset, kv_head, block_size, num_kv_heads,
                                        head_dim);
            for (int d = 0; d < head_dim; ++d)
                o[d] += w * element(value_cache, v0 + d, dtype);
        }
        free(x);
    }
}

/*
 * The same attention, computed partition by partition and merged.
 * partition_size > 0 tokens per partition.
 */
void oracle_paged_attention_decode_partitioned(
    const void *query, const void *key_cache, const void *value_cache,
    const int32_t *block_tables, const int32_t *context_lens, float scale, int num_seqs,
    int num_q_heads, int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
    int dtype, int partition_size, double *out)
{
    const int group = num_q_heads / num_kv_heads;
    const int64_t units = (int64_t)num_seqs * num_q_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t unit = 0; unit < units; ++unit) {
        const int s = (int)(unit / num_q_heads);
        const int h = (int)(unit % num_q_heads);
        const int kv_head = h / group;
        const int context_len = context_lens[s];
        const int32_t *blocks = block_tables + (int64_t)s * max_blocks_per_seq;
        const int64_t q0 = ((int64_t)s * num_q_heads + h) * head_dim;
        double *o = out + unit * head_dim;
        for (int d = 0; d < head_dim; ++d)
            o[d] = 0.0;
        if (context_len <= 0)
            continue;
        const int num_partitions = (context_len + partition_size - 1) / partition_size;
        double *m_p = (double *)malloc(sizeof(double) * (size_t)num_partitions);
        double *l_p = (double *)malloc(sizeof(double) * (size_t)num_partitions);
        double *o_p = (double *)calloc((size_t)num_partitions * head_dim, sizeof(double));
        double *x = (double *)malloc(sizeof(double) * (size_t)partition_size);

        for (int p = 0; p < num_partitions; ++p) {
            const int begin = p * partition_size;
            const int end = begin + partition_size < context_len ? begin + partition_size
                                                                 : context_len;
            for (int j = begin; j < end; ++j) {
                const int64_t k0 = pool_row(blocks[j / block_size], j % block_size, kv_head,
                                            block_size, num_kv_heads, head_dim);
                double dot = 0.0;
                for (int d = 0; d < head_dim; ++d)
                    dot += element(query, q0 + d, dtype) * element(key_cache, k0 + d, dtype);
                x[j - begin] = (double)scale * dot;
            }
            double m = x[0];
            for (int j = begin + 1; j < end; ++j)
                if (x[j - begin] > m)
                    m = x[j - begin];
            double l = 0.0;
            for (int j = begin; j < end; ++j) {
                const double e = exp(x[j - begin] - m);
                l += e;
                const int64_t v0 = pool_row(blocks[j / block_size], j % block_size, kv_head,
                                            block_size, num_kv_heads, head_dim);
                for (int d = 0; d < head_dim; ++d)
                    o_p[(int64_t)p * head_dim + d] += e * element(value_cache, v0 + d, dtype);
            }
            m_p[p] = m;
            l_p[p] = l;
        }

        /* merge: M = max m_p, total = sum l_p e^(m_p - M), out = sum e^(m_p - M) o_p / total */
        double M = m_p[0];
        for (int p = 1; p < num_partitions; ++p)
            if (m_p[p] > M)
                M = m_p[p];
        double total = 0.0;
        for (int p = 0; p < num_partitions; ++p)
            total += l_p[p] * exp(m_p[p] - M);
        for (int p = 0; p < num_partitions; ++p) {
            const double c = exp(m_p[p] - M) / total;
            for (int d = 0; d < head_dim; ++d)
                o[d] += c * o_p[(int64_t)p * head_dim + d];
        }
        free(m_p);
        free(l_p);
        free(o_p);
        free(x);
    }
}

/*
 * key/value: [num_tokens, num_kv_heads, head_dim]; each token's row of
 * num_kv_heads * head_dim elements is copied, as bits, to the pool cell
 * (slot / block_size, slot % block_size).  Slots < 0 are skipped.
 */
void oracle_kv_cache_write(const void *key, const void *value, const int32_t *slot_mapping,
                           void *key_cache, void *value_cache, int num_tokens,
                           int num_kv_heads, int head_dim, int block_size, int dtype)
{
    const size_t row_bytes = (size_t)num_kv_heads * head_dim * element_bytes(dtype);
    for (int t = 0; t < num_tokens; ++t) {
        const int slot = slot_mapping[t];
        if (slot < 0)
            continue;
        const int64_t block_id = slot / block_size;
        const int offset = slot % block_size;
        const int64_t dst = pool_row(block_id, offset, 0, block_size, num_kv_heads, head_dim);
        const int64_t src = (int64_t)t * num_kv_heads * head_dim;
        memcpy((char *)key_cache + dst * element_bytes(dtype),
               (const char *)key + src * element_bytes(dtype), row_bytes);
        memcpy((char *)value_cache + dst * element_bytes(dtype),
               (const char *)value + src * element_bytes(dtype), row_bytes);
    }
}

/*
 * out_k/out_v: [num_seqs, max_context_len, num_kv_heads, head_dim]; position
 * j < context_lens[s] receives the bits of logical token j; positions past
 * the context length are left untouched.
 */
void oracle_paged_kv_gather(const void *key_cache, const void *value_cache,
                            const int32_t *block_tables, const int32_t *context_lens,
                            void *out_k, void *out_v, int num_seqs, int num_kv_heads,
                            int head_dim, int block_size, int max_blocks_per_seq,
                            int max_context_len, int dtype)
{
    const size_t row_bytes = (size_t)num_kv_heads * head_dim * element_bytes(dtype);
    for (int s = 0; s < num_seqs; ++s) {
        const int32_t *blocks = block_tables + (int64_t)s * max_blocks_per_seq;
        for (int j = 0; j < context_lens[s]; ++j) {
            const int block_id = blocks[j / block_size];
            const int offset = j % block_size;
            const int64_t src = pool_row(block_id, offset, 0, block_size, num_kv_heads, head_dim);
            const int64_t dst = ((int64_t)s * max_context_len + j) * num_kv_heads * head_dim;
            memcpy((char *)out_k + dst * element_bytes(dtype),
                   (const char *)key_cache + src * element_bytes(dtype), row_bytes);
            memcpy((char *)out_v + dst * element_bytes(dtype),
                   (const char *)value_cache + src * element_bytes(dtype), row_bytes);
        }
    }
}

/*
 * block_mapping: [num_pairs, 2] int32 (src, dst).  Pairs are applied in
 * order; a pair with a negative src or dst copies nothing.
 */
void oracle_copy_blocks(void *key_cache, void *value_cache, const int32_t *block_mapping,
                        int num_pairs, int num_kv_heads, int head_dim, int block_size, int dtype)
{
    const size_t block_bytes =
        (size_t)block_size * num_kv_heads * head_dim * element_bytes(dtype);
    for (int i = 0; i < num_pairs; ++i) {
        const int src = block_mapping[2 * i];
        const int dst = block_mapping[2 * i + 1];
        if (src < 0 || dst < 0)
            continue;
        memmove((char *)key_cache + (size_t)dst * block_bytes,
                (const char *)key_cache + (size_t)src * block_bytes, block_bytes);
        memmove((char *)value_cache + (size_t)dst * block_bytes,
                (const char *)value_cache + (size_t)src * block_bytes, block_bytes);
    }
}

/*
 * Block swap between two pool pairs of the same block shape (device to host
 * or host to device).  block_mapping holds (from, to) pairs; a pair with an
 * id outside its pool copies nothing.
 */
void oracle_swap_blocks(const void *src_key, const void *src_value, int num_src_blocks,
                        void *dst_key, void *dst_value, int num_dst_blocks,
                        const int32_t *block_mapping, int num_pairs, int num_kv_heads,
                        int head_dim, int block_size, int dtype)
{
    const size_t bytes = (size_t)block_size * num_kv_heads * head_dim * element_bytes(dtype);
    for (int i = 0; i < num_pairs; ++i) {
        const int from = block_mapping[2 * i];
        const int to = block_mapping[2 * i + 1];
        if (from < 0 || from >= num_src_blocks || to < 0 || to >= num_dst_blocks)
            continue;
        memcpy((char *)dst_key + (size_t)to * bytes, (const char *)src_key + (size_t)from * bytes,
               bytes);
        memcpy((char *)dst_value + (size_t)to * bytes,
               (const char *)src_value + (size_t)from * bytes, bytes);
    }
}

/*
 * Prefix hashes of one token sequence: out[k] = h(tokens[0 .. (k+1)*bs - 1])
 * for every full block k (num_tokens / block_size of them), with
 * h(empty) = seed mod P and h(prefix, t) = (h(prefix) * base + t + 1) mod P,
 * P = 2^61 - 1, a token read as an unsigned 32-bit value.
 */
#define ORACLE_HASH_P ((((uint64_t)1) << 61) - 1)

static uint64_t mulmod_p61(uint64_t a, uint64_t b)
{
    return (uint64_t)(((unsigned __int128)a * b) % ORACLE_HASH_P);
}

void oracle_prefix_block_hashes(const int32_t *tokens, int num_tokens, int block_size,
                                uint64_t seed, uint64_t base, uint64_t *out)
{
    uint64_t h = seed % ORACLE_HASH_P;
    for (int i = 0; i < num_tokens; ++i) {
        h = (mulmod_p61(h, base % ORACLE_HASH_P) + (uint64_t)(uint32_t)tokens[i] + 1) %
            ORACLE_HASH_P;
        if ((i + 1) % block_size == 0)
            out[i / block_size] = h;
    }
}

/*
 * Multi-token attention.  query and out: [total_q, num_q_heads, head_dim],
 * the new tokens of all sequences one after another; query_start[num_seqs+1]
 * gives sequence s its rows query_start[s] .. query_start[s+1] - 1 (q_len).
 * context_lens[s] = L counts every cached token of s including its q_len new
 * ones.  Row i of sequence s attends over positions 0 .. L - q_len + i.
 * A sequence with q_len > L writes NaN rows (out is fp64 here).
 */
void oracle_paged_attention_prefill(const void *query, const void *key_cache,
                                    const void *value_cache, const int32_t *block_tables,
                                    const int32_t *context_lens, const int32_t *query_start,
                                    float scale, int num_seqs, int num_q_heads, int num_kv_heads,
                                    int head_dim, int block_size, int max_blocks_per_seq,
                                    int dtype, double *out)
{
    const int group = num_q_heads / num_kv_heads;
    const int64_t total_q = query_start[num_seqs];
    const int64_t units = total_q * num_q_heads;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t unit = 0; unit < units; ++unit) {
        const int64_t row = unit / num_q_heads; /* global new-token index */
        const int h = (int)(unit % num_q_heads);
        int s = 0;
        while (query_start[s + 1] <= row)
            ++s;
        const int q_len = query_start[s + 1] - query_start[s];
        const int i = (int)(row - query_start[s]);
        const int context_len = context_lens[s];
        const int kv_head = h / group;
        const int32_t *blocks = block_tables + (int64_t)s * max_blocks_per_seq;
        const int64_t q0 = (row * num_q_heads + h) * head_dim;
        double *o = out + unit * head_dim;
        if (q_len > context_len) {
            for (int d = 0; d < head_dim; ++d)
                o[d] = NAN;
            continue;
        }
        const int position = context_len - q_len + i;
        const int n = position + 1; /* positions 0 .. position */

        double *x = (double *)malloc(sizeof(double) * (size_t)n);
        for (int j = 0; j < n; ++j) {
            const int64_t k0 = pool_row(blocks[j / block_size], j % block_size, kv_head,
                                        block_size, num_kv_heads, head_dim);
            double dot = 0.0;
            for (int d = 0; d < head_dim; ++d)
                dot += element(query, q0 + d, dtype) * element(key_cache, k0 + d, dtype);
            x[j] = (double)scale * dot;
        }
        double m = x[0];
        for (int j = 1; j < n; ++j)
            if (x[j] > m)
                m = x[j];
        double sum = 0.0;
        for (int j = 0; j < n; ++j)
            sum += exp(x[j] - m);
        for (int d = 0; d < head_dim; ++d)
            o[d] = 0.0;
        for (int j = 0; j < n; ++j) {
            const double w = exp(x[j] - m) / sum;
            const int64_t v0 = pool_row(blocks[j / block_size], j % block_size, kv_head,
                                        block_size, num_kv_heads, head_dim);
            for (int d = 0; d < head_dim; ++d)
                o[d] += w * element(value_cache, v0 + d, dtype);
        }
        free(x);
    }
}
