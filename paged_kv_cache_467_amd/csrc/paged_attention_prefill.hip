// Multi-token (chunked-prefill) paged attention for gfx950 (CDNA4).
//
// What is computed: sequence s holds L = context_lens[s] tokens in the paged
// pool, the last q_len of which are new (a prompt, or a chunk of one, taken
// in the same batch as decoding sequences: "23.1 vLLM：高吞吐推理框架原理与
// 部署", §二.2; "大模型推理框架VLLM-0.7.3源码", §3.2).  New token i sits at
// position L - q_len + i and attends, with a scaled dot-product softmax,
// over positions 0 .. L - q_len + i of its sequence (every earlier token and
// itself); position j is read from block block_tables[s][j / block_size] at
// offset j % block_size ("大模型推理框架 vllm 源码解析 一", §三).
//
// With q_len new tokens and G query heads per kv head, each kv head serves
// q_len * G query rows: both products are real contractions, so both run on
// MFMA.  Work decomposition: one workgroup of 4 waves per (sequence, kv
// head, block of 64 rows), row r = (new token r / G, query head r % G);
// each wave owns 16 rows.  The workgroup walks the positions its rows can
// see in 16-token tiles, staged in LDS (double-buffered, one barrier per
// tile) and shared by its 4 waves:
//  * K rows are stored as they are ([token][d], rows padded against bank
//    conflicts); V rows are stored transposed ([d][token]).
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32: A = K (lane l: token l % 16, 8 consecutive d of
//    k-group l / 16), B = Q^T from registers (lane l: row l % 16, same d).
//    The result leaves lane l holding tokens 4 * (l / 16) + 0..3 of row
//    l % 16 -- exactly the B-operand layout of v_mfma_f32_16x16x16 with the
//    tokens as k, so after the online softmax the weights P^T feed the value
//    product O^T = V^T P^T straight from registers (A = V^T from LDS: lane l,
//    d = l % 16 of a 16-wide d block, 4 consecutive tokens).
//  * The accumulator O^T leaves lane l holding 4 consecutive d of row
//    l % 16, so each lane owns one row's running max, sum and rescale.
// Causal masking: position t is masked for a row whose position is below t;
// tiles past a wave's last row position are skipped by that wave.

#include "decode.h"
#include "device_utils.h"
#include "prefill.h"

#include <math.h>

namespace pkv {
namespace {

constexpr int kPrefillThreads = 256;
constexpr int kPrefillWaves = kPrefillThreads / 64;
constexpr int kRowsPerWave = 16;
constexpr int kRowsPerBlock = kPrefillWaves * kRowsPerWave;  // 64
constexpr int kTile = 16;                                     // tokens per tile

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

template <class T>
__device__ inline f32x4 mfma_k32(const u32x4 &a, const u32x4 &b, const f32x4 &c);
template <>
__device__ inline f32x4 mfma_k32<BF16>(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ inline f32x4 mfma_k32<F16>(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 16x16x16: a, b each hold 4 consecutive k values (two 32-bit words)
template <class T>
__device__ inline f32x4 mfma_k16(uint64_t a, uint64_t b, const f32x4 &c);
template <>
__device__ inline f32x4 mfma_k16<BF16>(uint64_t a, uint64_t b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
template <>
__device__ inline f32x4 mfma_k16<F16>(uint64_t a, uint64_t b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Round one weight in [0, 1] to the element type (nearest even).
template <class T>
__device__ inline uint32_t narrow_weight(float x);
template <>
__device__ inline uint32_t narrow_weight<BF16>(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
template <>
__device__ inline uint32_t narrow_weight<F16>(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <class T, int D>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillParams p) {
    static_assert(T::kBytes == 2, "MFMA path is for 16-bit element types");
    constexpr int KS = D / 32;            // k-steps of the score MFMA
    constexpr int DB = D / 16;            // 16-wide d blocks of the value MFMA
    constexpr int KSTR = D + 8;           // K tile row stride in elements (+16 bytes)
    constexpr int VSTR = kTile + 4;       // V^T row stride in elements (+8 bytes)
    constexpr int CHUNKS = kTile * D / 8;  // 16-byte chunks per tile and tensor
    constexpr int CPT = (CHUNKS + kPrefillThreads - 1) / kPrefillThreads;  // per thread
    constexpr int CPRW = D / 8;           // chunks per token row

    __shared__ __attribute__((aligned(16))) uint16_t ks_lds[2][kTile * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D * VSTR];

    // ---- work item
    const int nrb = p.row_blocks;
    const int rb = blockIdx.x % nrb;
    const int rest = blockIdx.x / nrb;
    const int kvh = rest % p.num_kv_heads;
    const int s = rest / p.num_kv_heads;
    const int G = p.group;
    const int qs0 = p.query_start[s];
    const int qs1 = p.query_start[s + 1];
    const int L = p.context_lens[s];
    if (qs0 < 0 || qs1 > p.total_q || qs1 < qs0) return;  // rows not identifiable: nothing written
    const int q_len = qs1 - qs0;
    const int nrows = (q_len < p.max_query_len ? q_len : p.max_query_len) * G;
    const int row0 = rb * kRowsPerBlock;
    if (row0 >= nrows) return;
    const bool bad_len = L < q_len || L > p.max_context_len;

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int lrow = lane & 15;   // this lane's row within the wave's 16
    const int kg = lane >> 4;     // k-group / token group
    const int row = row0 + wave * kRowsPerWave + lrow;
    const bool row_ok = row < nrows;
    const int tok = row / G;            // new token index within the sequence
    const int head = kvh * G + row % G;
    const int64_t qrow = (int64_t)qs0 + tok;
    const int pos = L - q_len + tok;     // this row's position

    if (bad_len) {
        if (row_ok) {
            const int64_t o = (qrow * p.num_q_heads + head) * D;
            for (int d = kg * 4; d < D; d += 16)
                *reinterpret_cast<uint64_t *>(static_cast<char *>(p.out) + (o + d) * 2) =
                    ((uint64_t)T::kNanPair << 32) | T::kNanPair;
        }
        return;
    }

    // positions the workgroup's rows can see: 0 .. pmax (the last valid row's)
    const int last_row = (row0 + kRowsPerBlock < nrows ? row0 + kRowsPerBlock : nrows) - 1;
    const int pmax = L - q_len + last_row / G;
    const int ntiles = pmax / kTile + 1;
    // this wave's rows: positions wave_pmin .. wave_pmax (none if the wave has no row)
    const int w_first = row0 + wave * kRowsPerWave;
    const int w_last = (w_first + kRowsPerWave < nrows ? w_first + kRowsPerWave : nrows) - 1;
    const bool wave_active = w_first < nrows;
    const int wave_pmax = L - q_len + w_last / G;
    const int wave_pmin = L - q_len + w_first / G;

    // B operand of the score MFMA: Q^T, lane = row, 16-byte chunk kg + 4 * ks
    u32x4 qb[KS];
    {
        const char *qp = static_cast<const char *>(p.query) + ((qrow * p.num_q_heads + head) * D) * 2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[ks] = row_ok ? load16(qp + 16 * (kg + 4 * ks)) : u32x4{0, 0, 0, 0};
    }

    // cooperative tile loader: thread -> (token of the tile, 16-byte chunk)
    const int32_t *bt_row = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    const int64_t head_off = (int64_t)kvh * D * 2;
    int bad = 0;
    u32x4 kreg[CPT], vreg[CPT];
    auto load_tile = [&](int tile) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int idx = threadIdx.x + c * kPrefillThreads;
            const int tt = idx / CPRW;
            const int ch = idx % CPRW;
            const int t = tile * kTile + tt;
            kreg[c] = u32x4{0, 0, 0, 0};
            vreg[c] = u32x4{0, 0, 0, 0};
            if (idx < CHUNKS && t <= pmax) {
                int blk = bt_row[t >> p.block_shift];
                if (blk < 0 || blk >= p.num_blocks) {
                    bad = 1;
                } else {
                    const int64_t o = (int64_t)blk * p.block_stride_bytes +
                                      (int64_t)(t & (p.block_size - 1)) * p.row_stride_bytes +
                                      head_off + ch * 16;
                    kreg[c] = load16_stream(p.key_cache + o);
                    vreg[c] = load16_stream(p.value_cache + o);
                }
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int idx = threadIdx.x + c * kPrefillThreads;
            if (idx >= CHUNKS) continue;
            const int tt = idx / CPRW;
            const int ch = idx % CPRW;
            *reinterpret_cast<u32x4 *>(&ks_lds[buf][tt * KSTR + ch * 8]) = kreg[c];
            // transpose V: element e of the chunk is d = 8 ch + e
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t word = vreg[c][w];
                vt_lds[buf][(ch * 8 + 2 * w) * VSTR + tt] = (uint16_t)(word & 0xFFFFu);
                vt_lds[buf][(ch * 8 + 2 * w + 1) * VSTR + tt] = (uint16_t)(word >> 16);
            }
        }
    };

    float m = -INFINITY, lsum = 0.0f;  // this lane's row (partial sum over its 4 tokens per tile)
    f32x4 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int tile = 0; tile < ntiles; ++tile) {
        const int buf = tile & 1;
        if (tile + 1 < ntiles) load_tile(tile + 1);
        const int t0 = tile * kTile;
        if (wave_active && t0 <= wave_pmax) {
            // S^T tile: lane holds tokens t0 + 4 kg + r of its row
            f32x4 st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 a =
                    *reinterpret_cast<const u32x4 *>(&ks_lds[buf][lrow * KSTR + (kg + 4 * ks) * 8]);
                st = mfma_k32<T>(a, qb[ks], st);
            }
            float sc[4];
            const bool need_mask = t0 + kTile - 1 > wave_pmin || !row_ok;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + 4 * kg + r;
                const bool vis = !need_mask || (row_ok && t <= pos);
                sc[r] = vis ? st[r] * p.scale_log2 : -INFINITY;
            }
            float mt = vmax(vmax(sc[0], sc[1]), vmax(sc[2], sc[3]));
            mt = vmax(mt, __shfl_xor(mt, 16));
            mt = vmax(mt, __shfl_xor(mt, 32));  // row max over the 16 tokens
            if (__builtin_amdgcn_ballot_w64(mt > m) != 0) {
                const float mn = vmax(m, mt);
                const float alpha = mn == -INFINITY ? 1.0f : fast_exp2(m - mn);
                m = mn;
                lsum *= alpha;
#pragma unroll
                for (int b = 0; b < DB; ++b) acc[b] *= alpha;
            }
            const float mref = m == -INFINITY ? 0.0f : m;  // rows that saw nothing: weights 0
            float pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pr[r] = fast_exp2(sc[r] - mref);
                lsum += pr[r];
            }
            const uint64_t pb =
                (uint64_t)(narrow_weight<T>(pr[0]) | (narrow_weight<T>(pr[1]) << 16)) |
                ((uint64_t)(narrow_weight<T>(pr[2]) | (narrow_weight<T>(pr[3]) << 16)) << 32);
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const uint64_t a = *reinterpret_cast<const uint64_t *>(
                    &vt_lds[buf][(b * 16 + lrow) * VSTR + 4 * kg]);
                acc[b] = mfma_k16<T>(a, pb, acc[b]);
            }
        }
        if (tile + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
    }
    bad = __syncthreads_or(bad);

    // row sum over the 4 token groups; the lane's accumulator holds d = 16 b + 4 kg + r
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (!row_ok) return;
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    char *op = static_cast<char *>(p.out) + ((qrow * p.num_q_heads + head) * D) * 2;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
        uint64_t v;
        if (bad) {
            v = ((uint64_t)T::kNanPair << 32) | T::kNanPair;
        } else {
            float o4[8] = {acc[b][0] * inv, acc[b][1] * inv, acc[b][2] * inv, acc[b][3] * inv,
                           0.0f, 0.0f, 0.0f, 0.0f};
            const u32x4 c = T::narrow_chunk(o4);
            v = (uint64_t)c[0] | ((uint64_t)c[1] << 32);
        }
        *reinterpret_cast<uint64_t *>(op + (b * 16 + 4 * kg) * 2) = v;
    }
}

template <class T>
hipError_t launch_t(const PrefillParams &p, int head_dim, hipStream_t stream) {
    const unsigned grid = (unsigned)((int64_t)p.num_seqs * p.num_kv_heads * p.row_blocks);
    switch (head_dim) {
        case 64:
            hipLaunchKernelGGL((prefill_kernel<T, 64>), dim3(grid), dim3(kPrefillThreads), 0,
                               stream, p);
            break;
        case 128:
            hipLaunchKernelGGL((prefill_kernel<T, 128>), dim3(grid), dim3(kPrefillThreads), 0,
                               stream, p);
            break;
        case 256:
            hipLaunchKernelGGL((prefill_kernel<T, 256>), dim3(grid), dim3(kPrefillThreads), 0,
                               stream, p);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int prefill_rows_per_block() { return kRowsPerBlock; }

hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_dim, hipStream_t stream) {
    switch (dtype) {
        case 1: return launch_t<F16>(p, head_dim, stream);
        case 2: return launch_t<BF16>(p, head_dim, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
