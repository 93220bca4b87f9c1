// Multi-token (chunked-prefill) paged attention for fp32 pools on gfx950.
//
// Computes what the 16-bit kernel (paged_attention_prefill.hip) computes --
// each new token of a sequence attends causally over the cached positions
// 0 .. L - q_len + i of its sequence ("23.1 vLLM：高吞吐推理框架原理与部署",
// §二.2; "大模型推理框架VLLM-0.7.3源码", §3.2), position j read from block
// block_tables[s][j / block_size] at offset j % block_size ("大模型推理框架
// vllm 源码解析 一", §三) -- with fp32 inputs and fp32 arithmetic throughout,
// on the fp32 matrix instruction v_mfma_f32_16x16x4_f32.
//
// One workgroup of 4 waves per (sequence, kv head, block of 64 query rows);
// each wave owns one 16-row block (row = (new token, query head) as in the
// 16-bit kernel).  Tiles of TT positions (64, 32 or 16 for head_dim 64, 128,
// 256: 16 KB per tensor) are staged in LDS as they lie in the pool, rows
// padded by 16 bytes, double-buffered with one barrier per tile.
//  * Scores transposed, S^T = K Q^T, per 16-token quarter: the contraction
//    over d is split among the four lane groups g = l / 16, group g taking
//    d in [g D/4, (g + 1) D/4) and step j its j-th element, so one 16-byte
//    LDS read gives a lane the K operands of four steps; the query operands
//    stay in registers.  Lane l then holds tokens 4 g + 0..3 of the quarter
//    for row l % 16 -- the layout of the 16-bit kernel, so the softmax is
//    the same.
//  * Value product O^T = V^T P^T, per quarter and 16-wide d block, in four
//    steps j over the tokens 4 g + j: the A operand is V[4 g + j][d] (one
//    4-byte LDS read per lane, 16 consecutive d per lane group) and the B
//    operand is the lane's own weight for token 4 g + j, in fp32.
// The row stride D + 4 floats keeps both reads free of bank conflicts: the
// K reads take 16 rows at one column, the V reads four rows 4 apart.

#include "device_utils.h"
#include "prefill.h"
#include "prefill_common.h"

#include <math.h>

namespace pkv {
namespace {

constexpr int kF32Threads = 256;
constexpr int kF32Waves = kF32Threads / 64;
constexpr int kF32Rows = kF32Waves * 16;  // query rows per workgroup
__host__ __device__ constexpr int f32_tile_tokens(int D) {
    return D >= 256 ? 16 : D >= 128 ? 32 : 64;
}

__device__ inline f32x4 mfma_k4(float a, float b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// SHARED: the shared-prefix pass of the shared-prefix decode (see
// launch_shared_prefix_f32) instead of the prefill.
template <int D, bool BT, bool SHARED>
__global__ __launch_bounds__(kF32Threads) void prefill_f32_kernel(PrefillParams p) {
    constexpr int TT = f32_tile_tokens(D);  // positions per tile
    constexpr int NQ = TT / 16;             // 16-token quarters of a tile
    constexpr int KJ = D / 4;               // score steps (4 d each); a lane group's d span
    constexpr int DB = D / 16;              // 16-wide d blocks of the value product
    constexpr int STR = D + 4;              // tile row stride in floats
    constexpr int CPRW = D / 4;             // 16-byte chunks per token row
    constexpr int CHUNKS = TT * CPRW;       // per tile and tensor
    constexpr int CPT = CHUNKS / kF32Threads;
    static_assert(CHUNKS % kF32Threads == 0, "every thread loads whole chunks");
    static_assert(16 * CPRW >= kF32Threads, "a thread's chunk c lies in quarter c * threads / (16 CPRW)");

    __shared__ __attribute__((aligned(16))) float k_lds[2][TT * STR];
    __shared__ __attribute__((aligned(16))) float v_lds[2][TT * STR];

    // ---- work item
    const int G = p.group;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int lrow = lane & 15;  // this lane's row within the wave's 16-row block
    const int g = lane >> 4;     // lane group: d span of the scores, token group of a quarter
    int kvh, row0, nrows;
    int tb = 0;     // the workgroup reads positions tb .. pmax (tb a multiple of 16)
    int pmax, wave_pmax, wave_pmin, pos;
    int part = 0;   // SHARED: the prefix partition
    int64_t obase;  // element offset of the row's output / query
    const int32_t *bt_row;
    if constexpr (SHARED) {
        // rows (sequence r / G, query head kvh * G + r % G) of the decode
        // batch, all seeing the partition's positions of the shared prefix
        const SharedPrefixWork sw = shared_prefix_work(p, blockIdx.x);
        kvh = sw.kvh;
        part = sw.part;
        nrows = p.num_seqs * G;
        row0 = sw.rb * kF32Rows;
        if (row0 >= nrows) return;
        tb = part * p.prefix_part;
        pmax = (tb + p.prefix_part < p.prefix_len ? tb + p.prefix_part : p.prefix_len) - 1;
        bt_row = p.block_tables;  // the first sequence's blocks: the shared ones
        const int row = row0 + wave * 16 + lrow;
        pos = row < nrows ? pmax : -1;
        obase = ((int64_t)(row / G) * p.num_q_heads + kvh * G + row % G) * D;
        wave_pmax = pmax;
        wave_pmin = row0 + wave * 16 + 16 <= nrows ? pmax : -1;
    } else {
        const PrefillWork wk = prefill_work(p, blockIdx.x);
        const int s = wk.s;
        kvh = wk.kvh;
        const int qs0 = p.query_start[s];
        const int qs1 = p.query_start[s + 1];
        const int L = p.context_lens[s];
        if (qs0 < 0 || qs1 > p.total_q || qs1 < qs0) return;  // rows not identifiable: nothing written
        const int q_len = qs1 - qs0;
        nrows = (q_len < p.max_query_len ? q_len : p.max_query_len) * G;
        row0 = wk.rb * kF32Rows;
        if (row0 >= nrows) return;
        const bool bad_len = L < q_len || L > p.max_context_len;
        const int w_first = row0 + wave * 16;
        const int row = w_first + lrow;
        pos = row < nrows ? L - q_len + row / G : -1;  // -1: a row past the end sees nothing
        obase = (((int64_t)qs0 + row / G) * p.num_q_heads + kvh * G + row % G) * D;

        if (bad_len) {
            if (row < nrows)
                for (int d = g * 4; d < D; d += 16)
                    *reinterpret_cast<u32x4 *>(static_cast<char *>(p.out) + (obase + d) * 4) =
                        u32x4{F32::kNanPair, F32::kNanPair, F32::kNanPair, F32::kNanPair};
            return;
        }

        // positions the workgroup's rows can see: 0 .. pmax (the last valid row's)
        const int last_row = (row0 + kF32Rows < nrows ? row0 + kF32Rows : nrows) - 1;
        pmax = L - q_len + last_row / G;
        const int w_last = (w_first + 16 < nrows ? w_first + 16 : nrows) - 1;
        wave_pmax = L - q_len + w_last / G;
        // tiles ending at or below this position need no causal mask
        wave_pmin = w_first + 16 <= nrows ? L - q_len + w_first / G : -1;
        bt_row = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    }
    const int w_first = row0 + wave * 16;
    const int row = w_first + lrow;
    const bool row_ok = row < nrows;
    const bool wave_active = w_first < nrows;
    const int ntiles = (pmax - tb) / TT + 1;

    // Shared prefix: a sequence whose table does not hold the first row's
    // blocks over this partition (the caller's promise broken) gets NaN
    // partial results.  The flags are cleared here, the first kCheckAhead
    // pairs (sequence, block) of each thread loaded with the first tile,
    // compared once the first barrier has passed and read back after the
    // tile loop's barriers.
    __shared__ int seq_bad[SHARED ? kF32Rows : 1];
    constexpr int kCheckAhead = SHARED ? 4 : 0;
    int s_first = 0, npairs = 0, nb = 1, b_first = 0;
    int chk_mine[kCheckAhead > 0 ? kCheckAhead : 1], chk_ref[kCheckAhead > 0 ? kCheckAhead : 1];
    if constexpr (SHARED) {
        s_first = row0 / G;
        const int ns = ((row0 + kF32Rows < nrows ? row0 + kF32Rows : nrows) - 1) / G - s_first + 1;
        b_first = tb >> p.block_shift;
        nb = (pmax >> p.block_shift) - b_first + 1;
        npairs = ns * nb;
        for (int i = threadIdx.x; i < ns; i += kF32Threads) seq_bad[i] = 0;
    }
    auto check_pair = [&](int i) {  // the pair's entry and the first row's
        const int si = i / nb, b = b_first + i % nb;
        return int2{p.block_tables[(int64_t)(s_first + si) * p.max_blocks_per_seq + b],
                    p.block_tables[b]};
    };

    // B operand of the score product: Q^T, this lane's row, d = g KJ + j
    float qv[KJ];
    {
        const float *qp = static_cast<const float *>(p.query) + obase + g * KJ;
#pragma unroll
        for (int c = 0; c < KJ / 4; ++c) {
            const u32x4 v = row_ok ? load16(qp + 4 * c) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t bits = v[e] ^ (p.negate_query ? 0x80000000u : 0u);
                qv[4 * c + e] = __builtin_bit_cast(float, bits);
            }
        }
    }

    // cooperative tile loader: thread -> (token of the tile, 16-byte chunk);
    // with block_size >= 16 the quarter of chunk c is the same for every
    // thread and lies in one block (a scalar block id per quarter)
    const int64_t head_off = (int64_t)kvh * D * 4;
    int bad = 0;
    u32x4 kreg[CPT], vreg[CPT];
    uint32_t chunk_off[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int idx = threadIdx.x + c * kF32Threads;
        chunk_off[c] = (uint32_t)(((idx / CPRW) % 16) * p.row_stride_bytes + head_off +
                                  (idx % CPRW) * 16);
    }
    const __amdgpu_buffer_rsrc_t bt_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t *>(bt_row), 0, p.max_blocks_per_seq * 4, kBufferConfig);
    int next_id[NQ];
    auto fetch_ids = [&](int tile) {  // one tile ahead; past pmax: pmax's block
#pragma unroll
        for (int h = 0; h < NQ; ++h) {
            const int th = min(tb + tile * TT + 16 * h, pmax);
            next_id[h] = __builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, (th >> p.block_shift) * 4,
                                                              0, 0);
        }
    };
    // every chunk is loaded from an in-bounds cell; tokens past pmax are
    // zeroed when the last tile is stored
    auto load_tile = [&](int tile) {
        const int t0 = tb + tile * TT;
        int64_t quarter_base[NQ] = {};
        if constexpr (BT) {
#pragma unroll
            for (int h = 0; h < NQ; ++h) {
                const int th = t0 + 16 * h;
                int blk = __builtin_amdgcn_readfirstlane(next_id[h]);
                if (blk < 0 || blk >= p.num_blocks) {
                    bad = 1;
                    blk = 0;
                }
                quarter_base[h] = (int64_t)blk * p.block_stride_bytes +
                                  (int64_t)(th & (p.block_size - 1)) * p.row_stride_bytes;
            }
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            int64_t o;
            if constexpr (BT) {
                o = quarter_base[c * kF32Threads / (16 * CPRW)] + chunk_off[c];
            } else {
                const int idx = threadIdx.x + c * kF32Threads;
                const int t = min(t0 + idx / CPRW, pmax);
                int blk = bt_row[t >> p.block_shift];
                if (blk < 0 || blk >= p.num_blocks) {
                    bad = 1;
                    blk = 0;
                }
                o = (int64_t)blk * p.block_stride_bytes +
                    (int64_t)(t & (p.block_size - 1)) * p.row_stride_bytes + head_off +
                    (idx % CPRW) * 16;
            }
            kreg[c] = load16_stream(p.key_cache + o);
            vreg[c] = load16_stream(p.value_cache + o);
        }
        if constexpr (BT) fetch_ids(tile + 1);
    };
    auto store_tile = [&](int buf, int tile) {
        const int t0 = tb + tile * TT;
        const bool last = t0 + TT - 1 > pmax;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int idx = threadIdx.x + c * kF32Threads;
            const int r = idx / CPRW, col = (idx % CPRW) * 4;
            const bool past = last && t0 + r > pmax;
            *reinterpret_cast<u32x4 *>(&k_lds[buf][r * STR + col]) =
                past ? u32x4{0, 0, 0, 0} : kreg[c];
            *reinterpret_cast<u32x4 *>(&v_lds[buf][r * STR + col]) =
                past ? u32x4{0, 0, 0, 0} : vreg[c];
        }
    };

    float m = -INFINITY, lsum = 0.0f;  // this lane's row; lsum is the lane's share
    f32x4 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    if constexpr (BT) fetch_ids(0);
    if constexpr (SHARED) {
#pragma unroll
        for (int k = 0; k < kCheckAhead; ++k) {
            const int i = threadIdx.x + k * kF32Threads;
            if (i < npairs) {
                const int2 e = check_pair(i);
                chk_mine[k] = e.x;
                chk_ref[k] = e.y;
            }
        }
    }
    load_tile(0);
    store_tile(0, 0);
    __syncthreads();
    if constexpr (SHARED) {  // the flags were cleared before the barrier
#pragma unroll
        for (int k = 0; k < kCheckAhead; ++k) {
            const int i = threadIdx.x + k * kF32Threads;
            if (i < npairs && chk_mine[k] != chk_ref[k]) seq_bad[i / nb] = 1;
        }
        for (int i = threadIdx.x + kCheckAhead * kF32Threads; i < npairs; i += kF32Threads) {
            const int2 e = check_pair(i);
            if (e.x != e.y) seq_bad[i / nb] = 1;
        }
    }
    for (int tile = 0; tile < ntiles; ++tile) {
        const int buf = tile & 1;
        const int t0 = tb + tile * TT;
        if (tile + 1 < ntiles) load_tile(tile + 1);
        if (wave_active && t0 <= wave_pmax) {
            const float *kt = k_lds[buf];
            const float *vt = v_lds[buf];
            // S^T of each quarter: lane holds tokens 4 g + r for row lrow
            f32x4 st[NQ];
#pragma unroll
            for (int u = 0; u < NQ; ++u) {
                st[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                const float *kr = kt + (16 * u + lrow) * STR + g * KJ;
#pragma unroll
                for (int c = 0; c < KJ / 4; ++c) {
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(kr + 4 * c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) st[u] = mfma_k4(a[e], qv[4 * c + e], st[u]);
                }
            }
            // online softmax; the scale (>= 0) enters with the exponent
            const bool need_mask = t0 + TT - 1 > wave_pmin;  // wave-uniform
            const int first = t0 + 4 * g;  // this lane's first token of quarter 0
            const float cs = p.score_scale;
            float sc[NQ][4];
#pragma unroll
            for (int u = 0; u < NQ; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sc[u][r] = st[u][r];
                    if (need_mask && first + 16 * u + r > pos) sc[u][r] = -INFINITY;
                }
            float mt = -INFINITY;
#pragma unroll
            for (int u = 0; u < NQ; ++u)
                mt = vmax(mt, vmax(vmax(sc[u][0], sc[u][1]), vmax(sc[u][2], sc[u][3])));
            mt = row_reduce4<true>(mt);
            mt = mt == -INFINITY ? -INFINITY : mt * cs;
            if (__builtin_amdgcn_ballot_w64(mt > m + kRescaleSlack) != 0) {
                const float mn = vmax(m, mt);
                const float alpha = mn == -INFINITY ? 1.0f : fast_exp2(m - mn);
                m = mn;
                lsum *= alpha;
#pragma unroll
                for (int b = 0; b < DB; ++b) acc[b] *= alpha;
            }
            const float nref = m == -INFINITY ? 0.0f : -m;  // rows that saw nothing
            float pw[NQ][4];
#pragma unroll
            for (int u = 0; u < NQ; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float a = __builtin_fmaf(sc[u][r], cs, nref);
                    if (need_mask && first + 16 * u + r > pos) a = -INFINITY;  // a zero scale
                    pw[u][r] = fast_exp2(a);
                    lsum += pw[u][r];
                }
            // O^T += V^T P^T: step j takes tokens 4 g + j of each quarter
#pragma unroll
            for (int u = 0; u < NQ; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float *vr = vt + (16 * u + 4 * g + j) * STR + lrow;
#pragma unroll
                    for (int b = 0; b < DB; ++b) acc[b] = mfma_k4(vr[16 * b], pw[u][j], acc[b]);
                }
        }
        if (tile + 1 < ntiles) store_tile(buf ^ 1, tile + 1);
        __syncthreads();
    }
    bad = __syncthreads_or(bad);

    // the accumulator holds d = 16 b + 4 g + r of row lrow
    lsum = row_reduce4<false>(lsum);
    if (!row_ok) return;
    if constexpr (SHARED) {
        // the partition's partial result for this row: running max (log2
        // domain), sum and unnormalised output, fp32 (NaN sum and output for
        // an invalid block id or a sequence that broke the sharing)
        const bool nan = bad || seq_bad[row / G - s_first] != 0;
        const int64_t slot = (obase / D) * p.num_slots + part;
        float *po = p.part_out + slot * D;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            // (through scalars: clang reads element 0 for a bit cast of an
            // indexed vector element)
            const float o0 = acc[b][0], o1 = acc[b][1], o2 = acc[b][2], o3 = acc[b][3];
            const u32x4 c = nan ? u32x4{0x7FC00000u, 0x7FC00000u, 0x7FC00000u, 0x7FC00000u}
                                : u32x4{__builtin_bit_cast(uint32_t, o0),
                                        __builtin_bit_cast(uint32_t, o1),
                                        __builtin_bit_cast(uint32_t, o2),
                                        __builtin_bit_cast(uint32_t, o3)};
            store16_stream(po + b * 16 + 4 * g, c);
        }
        if (g == 0) {
            __builtin_nontemporal_store(nan ? 0.0f : m, p.part_max + slot);
            __builtin_nontemporal_store(nan ? NAN : lsum, p.part_sum + slot);
        }
        return;
    }
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    char *op = static_cast<char *>(p.out) + obase * 4;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
        u32x4 v;
        if (bad) {
            v = u32x4{F32::kNanPair, F32::kNanPair, F32::kNanPair, F32::kNanPair};
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = __builtin_bit_cast(uint32_t, acc[b][r] * inv);
        }
        store16(op + (16 * b + 4 * g) * 4, v);
    }
}

template <int D>
void launch_d(const PrefillParams &p, hipStream_t stream) {
    const unsigned grid = (unsigned)((int64_t)p.num_seqs * p.num_kv_heads * p.row_blocks);
    if (p.block_size >= 16)
        hipLaunchKernelGGL((prefill_f32_kernel<D, true, false>), dim3(grid), dim3(kF32Threads),
                           0, stream, p);
    else
        hipLaunchKernelGGL((prefill_f32_kernel<D, false, false>), dim3(grid), dim3(kF32Threads),
                           0, stream, p);
}

template <int D>
void launch_shared_d(const PrefillParams &p, hipStream_t stream) {
    const unsigned grid = (unsigned)((int64_t)p.num_kv_heads * p.row_blocks * p.prefix_parts);
    if (p.block_size >= 16)
        hipLaunchKernelGGL((prefill_f32_kernel<D, true, true>), dim3(grid), dim3(kF32Threads), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((prefill_f32_kernel<D, false, true>), dim3(grid), dim3(kF32Threads),
                           0, stream, p);
}

}  // namespace

int prefill_f32_rows_per_block() { return kF32Rows; }

hipError_t launch_prefill_f32(const PrefillParams &p, int head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: launch_d<64>(p, stream); break;
        case 128: launch_d<128>(p, stream); break;
        case 256: launch_d<256>(p, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_shared_prefix_f32(const PrefillParams &p, int head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: launch_shared_d<64>(p, stream); break;
        case 128: launch_shared_d<128>(p, stream); break;
        case 256: launch_shared_d<256>(p, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
