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
// Work decomposition: one workgroup of 4 waves per (sequence, kv head,
// context partition).  The workgroup first stages the partition's block ids
// in LDS (checking each against the pool size), then its waves take 16-token
// tiles of the partition in turn.  Each wave keeps its own online-softmax
// state (running max m, running sum l, fp32 output accumulator) for the G
// query heads that share the kv head, so every K/V byte is read once for all
// G heads.  At the end the four waves are merged through LDS.
//
// Two per-tile inner loops:
//  * decode_mfma_kernel (f16/bf16, G >= 2): the scores of a 16-token tile for
//    all G heads are one 16x16x32 MFMA chain; the K rows are loaded straight
//    into the B operand (lane = token, 16 contiguous bytes per lane), the
//    query rows (repeated 16/G times) form the A operand.  The softmax
//    weights are passed through LDS to the lanes that hold the V rows and PV
//    is accumulated with fp32 FMAs.
//  * decode_valu_kernel (all dtypes, any G): each row of head_dim elements is
//    spread over head_dim * bytes / 16 lanes, 16 bytes each; scores are dot
//    products reduced across those lanes with DPP.
// Loads of the next tile are issued before the current tile is consumed.

#include "decode.h"
#include "device_utils.h"

#include <math.h>

namespace pkv {
namespace {

struct WorkItem {
    int s, kvh, part;
    int context_len;
    int tok_begin, tok_end;  // this partition's token range [begin, end)
    bool bad_len;            // context_len < 0 or > max_context_len
};

__device__ inline WorkItem work_item(const DecodeParams &p) {
    WorkItem w;
    const int id = blockIdx.x;
    // kv head fastest: consecutive workgroups go to consecutive XCDs, so all
    // workgroups of one kv head (which share any shared-prefix blocks) land
    // on the same XCD and its L2 when num_kv_heads is a multiple of 8.
    w.kvh = id % p.num_kv_heads;
    const int rest = id / p.num_kv_heads;
    w.part = rest % p.num_partitions;
    w.s = rest / p.num_partitions;
    w.context_len = p.context_lens[w.s];
    w.bad_len = w.context_len < 0 || w.context_len > p.max_context_len;
    w.tok_begin = w.part * p.partition_size;
    const int end = w.tok_begin + p.partition_size;
    w.tok_end = end < w.context_len ? end : w.context_len;
    return w;
}

// Copies the block ids covering tokens [begin, end) into LDS.  Returns true
// (for every thread) if any of them is outside [0, num_blocks).
__device__ inline bool stage_block_table(const DecodeParams &p, const WorkItem &w,
                                         int32_t *bt_lds) {
    const int b0 = w.tok_begin >> p.block_shift;
    const int b1 = (w.tok_end - 1) >> p.block_shift;
    const int32_t *row = p.block_tables + (int64_t)w.s * p.max_blocks_per_seq;
    int bad = 0;
    for (int i = threadIdx.x; i <= b1 - b0; i += kDecodeThreads) {
        int id = row[b0 + i];
        if (id < 0 || id >= p.num_blocks) {
            bad = 1;
            id = 0;
        }
        bt_lds[i] = id;
    }
    return __syncthreads_or(bad) != 0;
}

// Byte offset of (token, kv head) in the pool; token must be in the staged
// range.
__device__ inline int64_t row_offset(const DecodeParams &p, const int32_t *bt_lds, int b0,
                                     int token, int head_bytes) {
    const int blk = bt_lds[(token >> p.block_shift) - b0];
    const int off = token & (p.block_size - 1);
    return (int64_t)blk * p.block_stride_bytes + (int64_t)(off * p.row_stride_bytes + head_bytes);
}

// Output of a workgroup that reads nothing: zeros for an empty sequence, NaN
// for an invalid one.
template <class T, int D, int G>
__device__ void store_constant(const DecodeParams &p, const WorkItem &w, bool nan) {
    for (int i = threadIdx.x; i < G * D; i += kDecodeThreads) {
        const int g = i / D, d = i % D;
        const int64_t o = ((int64_t)w.s * p.num_q_heads + w.kvh * G + g) * D + d;
        if (nan)
            T::store_nan(p.out, o);
        else
            T::store(p.out, o, 0.0f);
    }
}

// Merges the per-wave states in LDS and writes either the final output (no
// split) or this partition's partial (m, l, unnormalised o).
template <class T, int D, int G>
__device__ void merge_waves(const DecodeParams &p, const WorkItem &w, const float (*mw)[G],
                            const float (*lw)[G], const float (*ow)[G][D], bool bad) {
    const bool split = p.num_partitions > 1;
    for (int i = threadIdx.x; i < G * D; i += kDecodeThreads) {
        const int g = i / D, d = i % D;
        float M = mw[0][g];
#pragma unroll
        for (int v = 1; v < kDecodeWaves; ++v) M = fmaxf(M, mw[v][g]);
        float Ls = 0.0f, O = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
            for (int v = 0; v < kDecodeWaves; ++v) {
                const float f = fast_exp2(mw[v][g] - M);  // 0 for a wave that saw no token
                Ls += lw[v][g] * f;
                O += ow[v][g][d] * f;
            }
        }
        const int h = w.kvh * G + g;
        if (!split) {
            const int64_t o = ((int64_t)w.s * p.num_q_heads + h) * D + d;
            if (bad)
                T::store_nan(p.out, o);
            else
                T::store(p.out, o, Ls > 0.0f ? O / Ls : 0.0f);
        } else {
            const int64_t ph = ((int64_t)w.s * p.num_q_heads + h) * p.num_partitions + w.part;
            p.part_out[ph * D + d] = bad ? NAN : O;
            if (d == 0) {
                p.part_max[ph] = bad ? 0.0f : M;
                p.part_sum[ph] = bad ? NAN : Ls;
            }
        }
    }
}

// Common prologue.  Returns false when the workgroup has nothing to read (it
// has then already written whatever it owes).
template <class T, int D, int G>
__device__ bool prologue(const DecodeParams &p, const WorkItem &w) {
    const bool split = p.num_partitions > 1;
    if (w.bad_len || w.tok_begin >= w.context_len) {
        // Without a split this workgroup owns the output (zeros when L == 0,
        // NaN when L is invalid).  With a split the reduce kernel owns it.
        if (!split) store_constant<T, D, G>(p, w, w.bad_len);
        return false;
    }
    return true;
}

// ------------------------------------------------------------------------
// VALU kernel
// ------------------------------------------------------------------------
template <class T, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_valu_kernel(DecodeParams p) {
    constexpr int EPC = T::kPerChunk;   // elements per 16-byte chunk
    constexpr int CPR = D / EPC;        // lanes holding one row
    constexpr int TPI = kWave / CPR;    // tokens per load instruction
    constexpr int NL = 4;               // loads per lane per tile (K and V each)
    constexpr int TILE = TPI * NL;      // tokens per tile
    static_assert(CPR >= 1 && CPR <= 64 && kWave % CPR == 0, "row layout");

    __shared__ int32_t bt_lds[kBtLds];
    __shared__ float mw[kDecodeWaves][G];
    __shared__ float lw[kDecodeWaves][G];
    __shared__ float ow[kDecodeWaves][G][D];

    const WorkItem w = work_item(p);
    if (!prologue<T, D, G>(p, w)) return;
    const bool bad = stage_block_table(p, w, bt_lds);
    const int b0 = w.tok_begin >> p.block_shift;

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int tg = lane / CPR;  // token slot within a load
    const int c = lane % CPR;   // 16-byte chunk of the row
    const int head_bytes = w.kvh * D * T::kBytes + c * 16;

    float q[G][EPC];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t qo = (((int64_t)w.s * p.num_q_heads + w.kvh * G + g) * D + c * EPC) *
                           T::kBytes;
        T::widen(load16(static_cast<const char *>(p.query) + qo), q[g]);
    }

    float m[G], l[G], acc[G][EPC];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[g][e] = 0.0f;
    }

    const int ntiles = bad ? 0 : (w.tok_end - w.tok_begin + TILE - 1) / TILE;
    u32x4 kb[NL], vb[NL];
    auto load_tile = [&](int tile, u32x4 *kd, u32x4 *vd) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int t = w.tok_begin + tile * TILE + i * TPI + tg;
            if (t < w.tok_end) {
                const int64_t o = row_offset(p, bt_lds, b0, t, head_bytes);
                kd[i] = load16(p.key_cache + o);
                vd[i] = load16(p.value_cache + o);
            } else {
                kd[i] = u32x4{0, 0, 0, 0};
                vd[i] = u32x4{0, 0, 0, 0};
            }
        }
    };

    int tile = wave;
    if (tile < ntiles) load_tile(tile, kb, vb);
    for (; tile < ntiles; tile += kDecodeWaves) {
        u32x4 kn[NL], vn[NL];
        const int next = tile + kDecodeWaves;
        if (next < ntiles) load_tile(next, kn, vn);

        float sc[NL][G];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            float k[EPC];
            T::widen(kb[i], k);
            const bool valid = w.tok_begin + tile * TILE + i * TPI + tg < w.tok_end;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.0f;
#pragma unroll
                for (int e = 0; e < EPC; ++e) d = fmaf(q[g][e], k[e], d);
                d = group_sum<CPR>(d);
                sc[i][g] = valid ? d * p.scale_log2 : -INFINITY;
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mt = sc[0][g];
#pragma unroll
            for (int i = 1; i < NL; ++i) mt = fmaxf(mt, sc[i][g]);
            mt = across_groups_max<CPR>(mt);
            const float mn = fmaxf(m[g], mt);
            const float alpha = fast_exp2(m[g] - mn);
            m[g] = mn;
            l[g] *= alpha;
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[g][e] *= alpha;
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            float v[EPC];
            T::widen(vb[i], v);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pr = fast_exp2(sc[i][g] - m[g]);
                l[g] += pr;
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc[g][e] = fmaf(pr, v[e], acc[g][e]);
            }
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            kb[i] = kn[i];
            vb[i] = vn[i];
        }
    }

    // Combine the token groups of the wave, then the waves.
#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = across_groups_sum<CPR>(l[g]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[g][e] = across_groups_sum<CPR>(acc[g][e]);
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            mw[wave][g] = m[g];
            lw[wave][g] = l[g];
        }
    }
    if (tg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < EPC; ++e) ow[wave][g][c * EPC + e] = acc[g][e];
    }
    __syncthreads();
    merge_waves<T, D, G>(p, w, mw, lw, ow, bad);
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
template <class T, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_mfma_kernel(DecodeParams p) {
    static_assert(T::kBytes == 2, "MFMA path is for 16-bit element types");
    static_assert(G == 2 || G == 4 || G == 8, "group size");
    constexpr int KS = D / 32;        // MFMA k-steps per tile
    constexpr int CPR = D / 8;        // 16-byte chunks per row
    constexpr int TPI = kWave / CPR;  // tokens per V load instruction
    constexpr int NV = 16 / TPI;      // V loads per lane per tile
    constexpr int TILE = 16;

    __shared__ int32_t bt_lds[kBtLds];
    __shared__ float pex[kDecodeWaves][TILE][G];  // softmax weights of the tile
    __shared__ float aex[kDecodeWaves][G];        // rescale factors of the tile
    __shared__ float mw[kDecodeWaves][G];
    __shared__ float lw[kDecodeWaves][G];
    __shared__ float ow[kDecodeWaves][G][D];

    const WorkItem w = work_item(p);
    if (!prologue<T, D, G>(p, w)) return;
    const bool bad = stage_block_table(p, w, bt_lds);
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

    // A operand: query head (kt % G) of this kv head's group
    u32x4 qa[KS];
    {
        const char *qrow = static_cast<const char *>(p.query) +
                           (((int64_t)w.s * p.num_q_heads + w.kvh * G + kt % G) * D) * 2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = load16(qrow + 16 * (rg + 4 * ks));
    }
    // result row 4 * rg + r holds query head (4 * rg + r) % G
    float m[4], l[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.0f;
    }
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.0f;

    const int ntiles = bad ? 0 : (w.tok_end - w.tok_begin + TILE - 1) / TILE;
    auto load_tile = [&](int tile, u32x4 *kd, u32x4 *vd) {
        const int base = w.tok_begin + tile * TILE;
        {
            const int t = base + kt;
            if (t < w.tok_end) {
                const char *row = p.key_cache + row_offset(p, bt_lds, b0, t, head_bytes);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kd[ks] = load16(row + 16 * (rg + 4 * ks));
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kd[ks] = u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int t = base + i * TPI + vtg;
            if (t < w.tok_end)
                vd[i] = load16(p.value_cache + row_offset(p, bt_lds, b0, t, head_bytes) + 16 * vc);
            else
                vd[i] = u32x4{0, 0, 0, 0};
        }
    };

    u32x4 kb[KS], vb[NV];
    int tile = wave;
    if (tile < ntiles) load_tile(tile, kb, vb);
    for (; tile < ntiles; tile += kDecodeWaves) {
        u32x4 kn[KS], vn[NV];
        const int next = tile + kDecodeWaves;
        if (next < ntiles) load_tile(next, kn, vn);

        f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = mfma16x16x32<T>(qa[ks], kb[ks], s);

        const bool valid = w.tok_begin + tile * TILE + kt < w.tok_end;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sc = valid ? s[r] * p.scale_log2 : -INFINITY;
            const float mt = group_max<16>(sc);  // over the 16 tokens of the tile
            const float mn = fmaxf(m[r], mt);
            const float alpha = fast_exp2(m[r] - mn);
            const float pr = fast_exp2(sc - mn);
            m[r] = mn;
            l[r] = l[r] * alpha + pr;
            const int head = 4 * rg + r;
            if (head < G) {
                pex[wave][kt][head] = pr;
                if (kt == 0) aex[wave][head] = alpha;
            }
        }
        // The weights were written by this wave; LDS executes a wave's
        // accesses in order, so only compiler ordering must be kept.
        __builtin_amdgcn_wave_barrier();

        float alpha[G];
#pragma unroll
        for (int g = 0; g < G; ++g) alpha[g] = aex[wave][g];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] *= alpha[g];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float v[8];
            T::widen(vb[i], v);
            float pw[G];
#pragma unroll
            for (int g = 0; g < G; ++g) pw[g] = pex[wave][i * TPI + vtg][g];
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pw[g], v[e], acc[g][e]);
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kb[ks] = kn[ks];
#pragma unroll
        for (int i = 0; i < NV; ++i) vb[i] = vn[i];
    }

    // l: sum over the 16 tokens of each row; acc: over the value token slots.
#pragma unroll
    for (int r = 0; r < 4; ++r) l[r] = group_sum<16>(l[r]);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = across_groups_sum<CPR>(acc[g][e]);
    if (kt == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int head = 4 * rg + r;
            if (head < G) {
                mw[wave][head] = m[r];
                lw[wave][head] = l[r];
            }
        }
    }
    if (vtg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) ow[wave][g][vc * 8 + e] = acc[g][e];
    }
    __syncthreads();
    merge_waves<T, D, G>(p, w, mw, lw, ow, bad);
}

// ------------------------------------------------------------------------
// Cross-partition reduce: out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p
// ------------------------------------------------------------------------
constexpr int kReduceThreads = 64;

template <class T, int D>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(DecodeParams p) {
    const int sh = blockIdx.x;
    const int s = sh / p.num_q_heads;
    const int L = p.context_lens[s];
    const int64_t obase = (int64_t)sh * D;
    if (L < 0 || L > p.max_context_len) {
        for (int d = threadIdx.x; d < D; d += kReduceThreads) T::store_nan(p.out, obase + d);
        return;
    }
    if (L == 0) {
        for (int d = threadIdx.x; d < D; d += kReduceThreads) T::store(p.out, obase + d, 0.0f);
        return;
    }
    const int nparts = (L + p.partition_size - 1) / p.partition_size;
    const int64_t pbase = (int64_t)sh * p.num_partitions;
    float M = -INFINITY;
    for (int q = 0; q < nparts; ++q) M = fmaxf(M, p.part_max[pbase + q]);
    float Ls = 0.0f;
    for (int q = 0; q < nparts; ++q) Ls += p.part_sum[pbase + q] * fast_exp2(p.part_max[pbase + q] - M);
    const float inv = 1.0f / Ls;
    for (int d = threadIdx.x; d < D; d += kReduceThreads) {
        float O = 0.0f;
        for (int q = 0; q < nparts; ++q)
            O += p.part_out[(pbase + q) * D + d] * fast_exp2(p.part_max[pbase + q] - M);
        T::store(p.out, obase + d, O * inv);
    }
}

template <class T, int D, int G>
hipError_t launch_typed(const DecodeParams &p, int kernel, hipStream_t stream) {
    const unsigned grid = (unsigned)((int64_t)p.num_seqs * p.num_kv_heads * p.num_partitions);
    if (kernel == 1) {
        if constexpr (T::kBytes == 2 && G >= 2) {
            hipLaunchKernelGGL((decode_mfma_kernel<T, D, G>), dim3(grid), dim3(kDecodeThreads), 0,
                               stream, p);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        hipLaunchKernelGGL((decode_valu_kernel<T, D, G>), dim3(grid), dim3(kDecodeThreads), 0,
                           stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.num_partitions > 1) {
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

hipError_t launch_decode(const DecodeParams &p, int dtype, int head_dim, int group, int kernel,
                         hipStream_t stream) {
    switch (dtype) {
        case 0: return launch_t<F32>(p, head_dim, group, kernel, stream);
        case 1: return launch_t<F16>(p, head_dim, group, kernel, stream);
        case 2: return launch_t<BF16>(p, head_dim, group, kernel, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
