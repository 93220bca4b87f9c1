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
// head, block of rows), row r = (new token r / G, query head r % G); each
// wave owns MB blocks of 16 rows (32 rows for head_dim <= 128, 16 for 256),
// so that every K/V operand read from LDS serves MB blocks.  The workgroup
// walks the positions its rows can see in tiles of 64 positions (32 for
// head_dim 256), staged in LDS as they lie in the pool ([token][d]; K rows
// padded by 16 bytes and V rows by 32, so that neither operand read meets a
// bank conflict), double-buffered with one barrier per tile and shared by
// its 4 waves.  At head_dim 128 with blocks of 16 tokens or more the tiles
// go from memory straight into LDS (global_load_lds, one 16-token quarter
// per wave, issued at the start of the tile before) with the chunks of each
// row placed by an XOR swizzle instead of padding:
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32 per 16-token quarter: A = K (lane l: token l % 16,
//    8 consecutive d of k-group l / 16), B = Q^T from registers (lane l: row
//    l % 16, same d).  Lane l then holds tokens 4 (l / 16) + 0..3 of each
//    quarter for row l % 16, and owns that row's running max, sum and
//    rescale.
//  * The value product O^T = V^T P^T also uses v_mfma_f32_16x16x32, once
//    per 32 tokens (two quarters), with k-group g of the 32 tokens being
//    {4g .. 4g+3} of the first quarter and {16+4g .. 16+4g+3} of the
//    second -- what each lane already holds of P^T
//    after the softmax, so the weights feed the MFMA from registers.  The
//    matching V^T operand (lane l: d = l % 16 of a 16-wide block, the same 8
//    tokens) comes from the row-major V tile through ds_read_b64_tr_b16:
//    within a group of 16 lanes, lane i receives element i % 4 of the 8-byte
//    vectors addressed by lanes 4e + i / 4 (e = 0..3), so lane 16g + 4r + c
//    addresses V[4g + r][4c ..] and lane 16g + i receives V[4g + 0..3][i].
//  * The accumulator O^T leaves lane l holding 4 consecutive d of row l % 16.
// Causal masking: position t is masked for a row whose position is below t;
// tiles past a wave's last row position are skipped by that wave.

#include "device_utils.h"
#include "prefill.h"
#include "prefill_common.h"

#include <math.h>

#include <type_traits>

namespace pkv {
namespace {

constexpr int kPrefillThreads = 256;
constexpr int kPrefillWaves = kPrefillThreads / 64;

// 16-row blocks per wave: two share each K/V operand read; head_dim 256
// keeps one (its accumulators and query operands double).
__host__ __device__ constexpr int blocks_per_wave(int D) { return D >= 256 ? 1 : 2; }
__host__ __device__ constexpr int rows_per_workgroup(int D) {
    return kPrefillWaves * 16 * blocks_per_wave(D);
}
// Positions per tile (one barrier each): 64 -- four 16-token quarters, two
// 32-token value-product groups -- and 32 for head_dim 256, whose tiles
// would otherwise leave room in LDS for one workgroup per compute unit.
__host__ __device__ constexpr int tile_tokens(int D) { return D >= 256 ? 32 : 64; }

typedef short s16x4 __attribute__((ext_vector_type(4)));

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

// Round two weights in [0, 1] to the element type (nearest even) and pack
// them into one word, the first in the low half.
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <class T>
__device__ inline uint32_t narrow_pair(float a, float b);
template <>
__device__ inline uint32_t narrow_pair<BF16>(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
template <>
__device__ inline uint32_t narrow_pair<F16>(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// Staging of the K/V tiles straight from memory into LDS at head_dim 128
// (see the kernel); 0 keeps the register staging everywhere.
#ifndef PKV_PREFILL_DMA
#define PKV_PREFILL_DMA 1
#endif
// s_waitcnt operand: vector memory count 0, the other counters untouched
constexpr int kWaitVmcnt0 = 0x0F70;

// K operands of the score products in flight ahead of their use (4 LDS
// reads cover their latency; measured 2-3% faster than 1 on the chunked-
// prefill workload, no faster at 2..8).
constexpr int kScoreReadAhead = 4;
// Instruction classes of __builtin_amdgcn_sched_group_barrier's mask.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedLdsRead = 0x100;

// One load straight into LDS: 64 lanes x 16 bytes, lane l's at LDS byte
// address lds + 16 l (M0 holds lds; one wait state after writing M0).
// Written out in assembly: through the builtin, the compiler cannot order
// the LDS write against the LDS reads in flight and waits for all of them
// (lgkmcnt(0)) wherever it needs one (2-3% slower on the chunked-prefill
// workload).  The caller waits for the load (vmcnt) itself before its
// barrier.  Default cache policy: the row blocks of a (sequence, kv head)
// unit read the same K/V tiles through L2, and the non-temporal hint
// measured 5% slower.  M0 is a reserved register that the compiler does
// not preserve around the statement; none of the code generated for these
// kernels uses it otherwise (a host test compiles this file and checks).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void load_to_lds16(const char *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ inline uint32_t lds_address(const uint16_t *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t *)p;
}

// Transposing 8-byte LDS read (see the layout note at the top of the file).
__device__ inline uint64_t lds_read_tr16(const uint16_t *p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3))) *)(p));
    return __builtin_bit_cast(uint64_t, v);
}

// SHARED: the shared-prefix pass of the shared-prefix decode (see
// launch_shared_prefix) instead of the prefill.
template <class T, int D, bool BT, bool SHARED>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillParams p) {
    static_assert(T::kBytes == 2, "MFMA path is for 16-bit element types");
    constexpr int MB = blocks_per_wave(D);
    constexpr int RPB = rows_per_workgroup(D);
    constexpr int KS = D / 32;            // k-steps of the score MFMA
    constexpr int DB = D / 16;            // 16-wide d blocks of the value MFMA
    constexpr int TT = tile_tokens(D);    // positions per tile
    constexpr int NQ = TT / 16;           // 16-token quarters of a tile
    constexpr int NG = TT / 32;           // 32-token groups of the value MFMA
    // Tile row strides in elements.  The score operand reads 16 rows x 16
    // bytes per pass: a 16-byte pad puts those rows 4 banks apart.  The
    // transposing value reads take 8 rows x 32 bytes per pass: a 32-byte pad
    // puts them 8 banks apart.  Either way no two lanes of a pass share a
    // bank (with 32 or with 64 four-byte banks).
    constexpr int KSTR = D + 8;
    constexpr int VSTR = D + 16;
    constexpr int CHUNKS = TT * D / 8;    // 16-byte chunks per tile and tensor
    constexpr int CPT = (CHUNKS + kPrefillThreads - 1) / kPrefillThreads;  // per thread
    constexpr int CPRW = D / 8;           // chunks per token row
    static_assert(CHUNKS % kPrefillThreads == 0, "every thread loads whole chunks");
    // At head_dim 128 with whole 16-token quarters per block, the tiles go
    // from memory straight into LDS (global_load_lds): each wave loads one
    // quarter of each tile, 1 KB (4 rows) per instruction, with no register
    // staging and no padding.  The 16-byte chunks are placed with an XOR
    // swizzle instead -- chunk c of tile row r at position c ^ (r mod 16) in
    // K and c ^ 2 (r mod 8) in V -- so that the score operand reads (16 rows,
    // one chunk each) and the transposing value reads (4 rows x 32 bytes)
    // still meet no bank conflict.
    constexpr bool DMA = PKV_PREFILL_DMA && D == 128 && BT && NQ == kPrefillWaves;
    constexpr int KROW = DMA ? D : KSTR;  // element stride of the LDS tile rows
    constexpr int VROW = DMA ? D : VSTR;

    // The two tile buffers.  With the loads straight to LDS each buffer is a
    // variable of its own and the tile loop names it by a compile-time
    // constant, so that every LDS address of a tile is a fixed offset from
    // one register; otherwise one array of two.
    constexpr int NKB = DMA ? 1 : 2;
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[NKB][DMA ? 8 : TT * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[NKB][DMA ? 8 : TT * VROW];
    __shared__ __attribute__((aligned(16))) uint16_t k_lds0[DMA ? TT * KROW : 8];
    __shared__ __attribute__((aligned(16))) uint16_t k_lds1[DMA ? TT * KROW : 8];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds0[DMA ? TT * VROW : 8];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds1[DMA ? TT * VROW : 8];
    auto kbuf = [&](int b) -> uint16_t * {
        if constexpr (DMA)
            return b ? k_lds1 : k_lds0;
        else
            return k_lds[b];
    };
    auto vbuf = [&](int b) -> uint16_t * {
        if constexpr (DMA)
            return b ? v_lds1 : v_lds0;
        else
            return v_lds[b];
    };

    // ---- work item
    const int G = p.group;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int lrow = lane & 15;   // this lane's row within each 16-row block
    const int kg = lane >> 4;     // k-group / token group
    int kvh, row0, nrows;
    int tb = 0;     // the workgroup reads positions tb .. pmax (tb a multiple of 16)
    int pmax;
    int wave_pmax;  // the last position any row of this wave sees
    int wave_pmin;  // tiles ending at or below this position need no mask
    int part = 0;   // SHARED: the prefix partition
    const int32_t *bt_row;
    bool row_ok[MB];
    int pos[MB];        // the row's last visible position; -1 for a row past the end
    int64_t obase[MB];  // element offset of the row's output / query
    if constexpr (SHARED) {
        // rows (sequence r / G, query head kvh * G + r % G) of the decode
        // batch, all seeing the partition's positions of the shared prefix
        const SharedPrefixWork sw = shared_prefix_work(p, blockIdx.x);
        kvh = sw.kvh;
        part = sw.part;
        nrows = p.num_seqs * G;
        row0 = sw.rb * RPB;
        if (row0 >= nrows) return;
        tb = part * p.prefix_part;
        pmax = (tb + p.prefix_part < p.prefix_len ? tb + p.prefix_part : p.prefix_len) - 1;
        bt_row = p.block_tables;  // the first sequence's blocks: the shared ones
        const int w_first = row0 + wave * 16 * MB;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int row = w_first + 16 * mb + lrow;
            row_ok[mb] = row < nrows;
            pos[mb] = row_ok[mb] ? pmax : -1;
            obase[mb] = ((int64_t)(row / G) * p.num_q_heads + kvh * G + row % G) * D;
        }
        wave_pmax = pmax;
        wave_pmin = w_first + 16 * MB <= nrows ? pmax : -1;
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
        row0 = wk.rb * RPB;
        if (row0 >= nrows) return;
        const bool bad_len = L < q_len || L > p.max_context_len;
        const int w_first = row0 + wave * 16 * MB;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int row = w_first + 16 * mb + lrow;
            row_ok[mb] = row < nrows;
            const int tok = row / G;
            pos[mb] = row_ok[mb] ? L - q_len + tok : -1;
            obase[mb] = (((int64_t)qs0 + tok) * p.num_q_heads + kvh * G + row % G) * D;
        }

        if (bad_len) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                if (row_ok[mb])
                    for (int d = kg * 4; d < D; d += 16)
                        *reinterpret_cast<uint64_t *>(static_cast<char *>(p.out) +
                                                      (obase[mb] + d) * 2) =
                            ((uint64_t)T::kNanPair << 32) | T::kNanPair;
            return;
        }

        // positions the workgroup's rows can see: 0 .. pmax (the last valid row's)
        const int last_row = (row0 + RPB < nrows ? row0 + RPB : nrows) - 1;
        pmax = L - q_len + last_row / G;
        const int w_last = (w_first + 16 * MB < nrows ? w_first + 16 * MB : nrows) - 1;
        wave_pmax = L - q_len + w_last / G;
        wave_pmin = w_first + 16 * MB <= nrows ? L - q_len + w_first / G : -1;
        bt_row = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    }
    const int w_first = row0 + wave * 16 * MB;
    const bool wave_active = w_first < nrows;
    const int ntiles = (pmax - tb) / TT + 1;

    // Shared prefix: a sequence whose table does not hold the first row's
    // blocks over this partition (the caller's promise broken) gets NaN
    // partial results.  The flags are cleared here; the table entries of
    // the first kCheckAhead pairs (sequence, block) of each thread are
    // loaded with the first tile's, compared once the first barrier has
    // passed, and read back after the tile loop's barriers.
    __shared__ int seq_bad[SHARED ? RPB : 1];
    constexpr int kCheckAhead = SHARED ? 4 : 0;
    int s_first = 0, npairs = 0, nb = 1, b_first = 0;
    int chk_mine[kCheckAhead > 0 ? kCheckAhead : 1], chk_ref[kCheckAhead > 0 ? kCheckAhead : 1];
    if constexpr (SHARED) {
        s_first = row0 / G;
        const int ns = ((row0 + RPB < nrows ? row0 + RPB : nrows) - 1) / G - s_first + 1;
        b_first = tb >> p.block_shift;
        nb = (pmax >> p.block_shift) - b_first + 1;
        npairs = ns * nb;
        for (int i = threadIdx.x; i < ns; i += kPrefillThreads) seq_bad[i] = 0;
    }
    auto check_pair = [&](int i) {  // the pair's entry and the first row's
        const int si = i / nb, b = b_first + i % nb;
        return int2{p.block_tables[(int64_t)(s_first + si) * p.max_blocks_per_seq + b],
                    p.block_tables[b]};
    };

    // B operand of the score MFMA: Q^T, lane = row, 16-byte chunk kg + 4 * ks
    u32x4 qb[MB][KS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const char *qp = static_cast<const char *>(p.query) + obase[mb] * 2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[mb][ks] = row_ok[mb] ? load16(qp + 16 * (kg + 4 * ks)) : u32x4{0, 0, 0, 0};
    }
    if (p.negate_query) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qb[mb][ks] ^= 0x80008000u;  // both sign bits
    }

    // cooperative tile loader: thread -> (token of the tile, 16-byte chunk).
    // With block_size >= 16 each 16-token quarter of a tile lies in one
    // block: its id is uniform (a scalar register) and each thread adds a
    // fixed offset; the quarter a chunk falls in is the same for a whole wave.
    const int64_t head_off = (int64_t)kvh * D * 2;
    int bad = 0;
    u32x4 kreg[CPT], vreg[CPT];
    uint32_t chunk_off[CPT];  // offset of the thread's chunk from its quarter's first row
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int idx = threadIdx.x + c * kPrefillThreads;
        chunk_off[c] = (uint32_t)(((idx / CPRW) % 16) * p.row_stride_bytes + head_off +
                                  (idx % CPRW) * 16);
    }
    // the 16-token quarter of a tile that chunk c of this thread falls in:
    // the same for the whole wave
    const int wave_s = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    auto half_of = [&](int c) {
        if constexpr (16 * CPRW >= kPrefillThreads)
            return c * kPrefillThreads / (16 * CPRW);
        else
            return (wave_s * kWave + c * kPrefillThreads) / (16 * CPRW);
    };
    // Block ids of the quarters of the next tile to load, fetched one tile
    // ahead with a vector (buffer) load, so that they are in registers when
    // the tile's loads are issued: a scalar load there would stall the wave
    // (its wait also covers every outstanding LDS access).  A quarter past
    // pmax takes pmax's block; its tokens are zeroed when the tile is stored.
    const __amdgpu_buffer_rsrc_t bt_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t *>(bt_row), 0, p.max_blocks_per_seq * 4, kBufferConfig);
    int next_id[NQ];
    auto fetch_ids = [&](int tile) {
        if constexpr (DMA) {  // this wave's quarter only
            const int th = min(tb + tile * TT + 16 * wave_s, pmax);
            next_id[0] = __builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, (th >> p.block_shift) * 4,
                                                              0, 0);
        } else {
#pragma unroll
            for (int h = 0; h < NQ; ++h) {
                const int th = min(tb + tile * TT + 16 * h, pmax);
                next_id[h] = __builtin_amdgcn_raw_buffer_load_b32(
                    bt_rsrc, (th >> p.block_shift) * 4, 0, 0);
            }
        }
    };
    // DMA: this lane's byte offset from its quarter's first row for each of
    // the 4 instructions per tensor: tile row r = 4 j + lane / 16 of the
    // quarter, LDS position lane % 16, holding the chunk the swizzle puts there
    uint32_t dma_k[4], dma_v[4];
    if constexpr (DMA) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * j + lane / 16, pos16 = lane % 16;
            const uint32_t row = (uint32_t)(r * p.row_stride_bytes + head_off);
            dma_k[j] = row + 16 * (pos16 ^ r);
            dma_v[j] = row + 16 * (pos16 ^ (2 * (r & 7)));
        }
    }
    // DMA: issues this wave's quarter of tile `tile` into LDS buffer buf
    // (block id from fetch_ids, then the next tile's id is fetched)
    auto dma_tile = [&](int buf, int tile) {
        const int th = tb + tile * TT + 16 * wave_s;
        int blk = __builtin_amdgcn_readfirstlane(next_id[0]);
        if (blk < 0 || blk >= p.num_blocks) {
            bad = 1;
            blk = 0;
        }
        const int64_t qb = (int64_t)blk * p.block_stride_bytes +
                           (int64_t)(th & (p.block_size - 1)) * p.row_stride_bytes;
        const char *kq = p.key_cache + qb;
        const char *vq = p.value_cache + qb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row0 = 16 * wave_s + 4 * j;  // the instruction's first tile row
            load_to_lds16(kq + dma_k[j], lds_address(&kbuf(buf)[row0 * KROW]));
            load_to_lds16(vq + dma_v[j], lds_address(&vbuf(buf)[row0 * VROW]));
        }
        fetch_ids(tile + 1);  // past the last tile: pmax's block again
    };
    // DMA: once this wave's loads of tile `tile` have landed, zero the rows
    // of its quarter past pmax (last tile only)
    auto dma_finish = [&](int buf, int tile) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        const int t0 = tb + tile * TT;
        if (t0 + TT - 1 > pmax) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * wave_s + 4 * j + lane / 16;
                if (t0 + r <= pmax) continue;
                *reinterpret_cast<u32x4 *>(&kbuf(buf)[r * KROW + 8 * (lane % 16)]) =
                    u32x4{0, 0, 0, 0};
                *reinterpret_cast<u32x4 *>(&vbuf(buf)[r * VROW + 8 * (lane % 16)]) =
                    u32x4{0, 0, 0, 0};
            }
        }
    };
    auto load_tile = [&](int tile) {
        const int t0 = tb + tile * TT;
        int64_t half_base[NQ] = {};
        if constexpr (BT) {
#pragma unroll
            for (int h = 0; h < NQ; ++h) {
                const int th = t0 + 16 * h;
                int blk = __builtin_amdgcn_readfirstlane(next_id[h]);
                if (blk < 0 || blk >= p.num_blocks) {
                    bad = 1;
                    blk = 0;
                }
                half_base[h] = (int64_t)blk * p.block_stride_bytes +
                               (int64_t)(th & (p.block_size - 1)) * p.row_stride_bytes;
            }
        }
        // Every chunk is loaded, so that the loads issue back to back; a
        // token past pmax reads an in-bounds cell (pmax's block for a quarter
        // past pmax, the same block otherwise, or token pmax with per-token
        // ids)
        // and is zeroed when the tile is stored.
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            int64_t o;
            if constexpr (BT) {
                o = half_base[half_of(c)] + chunk_off[c];
            } else {
                const int idx = threadIdx.x + c * kPrefillThreads;
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
        if constexpr (BT) fetch_ids(tile + 1);  // past the last tile: pmax's block again
    };
    auto store_tile = [&](int buf, int tile) {
        const int t0 = tb + tile * TT;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int idx = threadIdx.x + c * kPrefillThreads;
            const int row = idx / CPRW, col = (idx % CPRW) * 8;
            *reinterpret_cast<u32x4 *>(&kbuf(buf)[row * KROW + col]) = kreg[c];
            *reinterpret_cast<u32x4 *>(&vbuf(buf)[row * VROW + col]) = vreg[c];
        }
        if (t0 + TT - 1 > pmax) {  // the last tile: overwrite tokens past pmax
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const int idx = threadIdx.x + c * kPrefillThreads;
                if (t0 + idx / CPRW <= pmax) continue;
                const int row = idx / CPRW, col = (idx % CPRW) * 8;
                *reinterpret_cast<u32x4 *>(&kbuf(buf)[row * KROW + col]) = u32x4{0, 0, 0, 0};
                *reinterpret_cast<u32x4 *>(&vbuf(buf)[row * VROW + col]) = u32x4{0, 0, 0, 0};
            }
        }
    };

    float m[MB], lsum[MB];  // this lane's rows; lsum is the lane's share of the row sum
    f32x4 acc[MB][DB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        m[mb] = -INFINITY;
        lsum[mb] = 0.0f;
#pragma unroll
        for (int b = 0; b < DB; ++b) acc[mb][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // this lane's V^T addresses inside a tile (quarter 0); quarter q is 16 q rows down
    // (DMA: d block b of the lane's row sits at swizzled chunk pair b ^ vt_swz)
    const int vt_elem = DMA ? (4 * kg + lrow / 4) * VROW + 8 * ((lrow >> 1) & 1) +
                                  4 * (lrow & 1)
                            : (4 * kg + lrow / 4) * VSTR + 4 * (lrow % 4);
    const int vt_swz = (4 * kg + lrow / 4) & 7;

    if constexpr (BT) fetch_ids(0);
    if constexpr (SHARED) {
#pragma unroll
        for (int k = 0; k < kCheckAhead; ++k) {
            const int i = threadIdx.x + k * kPrefillThreads;
            if (i < npairs) {
                const int2 e = check_pair(i);
                chk_mine[k] = e.x;
                chk_ref[k] = e.y;
            }
        }
    }
    if constexpr (DMA) {
        dma_tile(0, 0);
        dma_finish(0, 0);
    } else {
        load_tile(0);
        store_tile(0, 0);
    }
    __syncthreads();
    if constexpr (SHARED) {  // the flags were cleared before the barrier
#pragma unroll
        for (int k = 0; k < kCheckAhead; ++k) {
            const int i = threadIdx.x + k * kPrefillThreads;
            if (i < npairs && chk_mine[k] != chk_ref[k]) seq_bad[i / nb] = 1;
        }
        for (int i = threadIdx.x + kCheckAhead * kPrefillThreads; i < npairs;
             i += kPrefillThreads) {
            const int2 e = check_pair(i);
            if (e.x != e.y) seq_bad[i / nb] = 1;
        }
    }
    // One tile: its scores, softmax and value product, with the next tile's
    // loads in flight.  The LDS buffer is bufc, a compile-time constant when
    // the loads go straight to LDS (the loop runs two tiles at a time).
    auto tile_step = [&](int tile, auto bufc) {
        const int buf = bufc;
        const int t0 = tb + tile * TT;
        bool prefetched = false;
        // DMA: the next tile goes out at once, into the buffer every wave
        // finished reading before the last barrier
        if constexpr (DMA) {
            if (tile + 1 < ntiles) dma_tile(buf ^ 1, tile + 1);
        }
        if (wave_active && t0 <= wave_pmax) {
            const uint16_t *kt = kbuf(buf);
            const uint16_t *vt = vbuf(buf);
            // S^T for every quarter and row block.  The K operands are read
            // kScoreReadAhead products ahead of their use (the schedule is
            // pinned below: left to itself the compiler reads each operand
            // just before its two products and waits for it every time).
            f32x4 st[MB][NQ];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int u = 0; u < NQ; ++u) st[mb][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            constexpr int NS = NQ * KS;  // (quarter, k-step) pairs
            constexpr int PD = kScoreReadAhead < NS ? kScoreReadAhead : NS;
            u32x4 ka[NS];
            auto kread = [&](int step) {
                const int u = step / KS, ks = step % KS;
                const int chunk = DMA ? (kg + 4 * ks) ^ lrow : kg + 4 * ks;
                ka[step] = *reinterpret_cast<const u32x4 *>(&kt[(16 * u + lrow) * KROW + chunk * 8]);
            };
#pragma unroll
            for (int step = 0; step < PD; ++step) kread(step);
#pragma unroll
            for (int step = 0; step < NS; ++step) {
                if (step + PD < NS) kread(step + PD);
                const int u = step / KS, ks = step % KS;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    st[mb][u] = mfma_k32<T>(ka[step], qb[mb][ks], st[mb][u]);
            }
            // order: PD reads, then per step one read and its MB products
            __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, PD, 0);
#pragma unroll
            for (int step = 0; step < NS; ++step) {
                if (step + PD < NS) __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, MB, 0);
            }
            // the next tile's loads, issued once this tile's K operands are in registers
            if constexpr (!DMA) {
                if (tile + 1 < ntiles) load_tile(tile + 1);
            }
            prefetched = true;
            const bool need_mask = t0 + TT - 1 > wave_pmin;  // wave-uniform
            const int first = t0 + 4 * kg;  // this lane's first token of quarter 0
            const float c = p.score_scale;
            u32x4 pb[MB][NG];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                // raw scores; the scale (>= 0) enters with the exponent
                float sc[NQ][4];
                const int lim = pos[mb] - first;  // tokens 16 u + r past it are masked
#pragma unroll
                for (int u = 0; u < NQ; ++u)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sc[u][r] = st[mb][u][r];
                if (need_mask) {
#pragma unroll
                    for (int u = 0; u < NQ; ++u)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (16 * u + r > lim) sc[u][r] = -INFINITY;
                }
                float mt = -INFINITY;
#pragma unroll
                for (int u = 0; u < NQ; ++u)
                    mt = vmax(mt, vmax(vmax(sc[u][0], sc[u][1]), vmax(sc[u][2], sc[u][3])));
                mt = row_reduce4<true>(mt);                     // row max over the tile
                mt = mt == -INFINITY ? -INFINITY : mt * c;      // scaled (log2 domain)
                if (__builtin_amdgcn_ballot_w64(mt > m[mb] + kRescaleSlack) != 0) {
                    const float mn = vmax(m[mb], mt);
                    const float alpha = mn == -INFINITY ? 1.0f : fast_exp2(m[mb] - mn);
                    m[mb] = mn;
                    lsum[mb] *= alpha;
#pragma unroll
                    for (int b = 0; b < DB; ++b) acc[mb][b] *= alpha;
                }
                const float nref = m[mb] == -INFINITY ? 0.0f : -m[mb];  // rows that saw nothing
                float arg[NQ][4];
#pragma unroll
                for (int u = 0; u < NQ; ++u)
#pragma unroll
                    for (int r = 0; r < 4; ++r) arg[u][r] = __builtin_fmaf(sc[u][r], c, nref);
                if (need_mask) {  // a zero scale turns a masked score into NaN above
#pragma unroll
                    for (int u = 0; u < NQ; ++u)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (16 * u + r > lim) arg[u][r] = -INFINITY;
                }
                uint32_t w[NQ][2];
#pragma unroll
                for (int u = 0; u < NQ; ++u) {
                    float pr[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pr[r] = fast_exp2(arg[u][r]);
                        lsum[mb] += pr[r];
                    }
                    w[u][0] = narrow_pair<T>(pr[0], pr[1]);
                    w[u][1] = narrow_pair<T>(pr[2], pr[3]);
                }
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    pb[mb][g] = u32x4{w[2 * g][0], w[2 * g][1], w[2 * g + 1][0], w[2 * g + 1][1]};
            }
#pragma unroll
            for (int g = 0; g < NG; ++g) {
#pragma unroll
                for (int b = 0; b < DB; ++b) {
                    const uint16_t *vg = vt + vt_elem + 32 * g * VROW +
                                         (DMA ? 16 * (b ^ vt_swz) : 16 * b);
                    const uint64_t lo = lds_read_tr16(vg);
                    const uint64_t hi = lds_read_tr16(vg + 16 * VROW);
                    const u32x4 a = u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi,
                                          (uint32_t)(hi >> 32)};
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb][b] = mfma_k32<T>(a, pb[mb][g], acc[mb][b]);
                }
            }
        }
        if constexpr (DMA) {
            if (tile + 1 < ntiles) dma_finish(buf ^ 1, tile + 1);
        } else {
            if (!prefetched && tile + 1 < ntiles) load_tile(tile + 1);
            if (tile + 1 < ntiles) store_tile(buf ^ 1, tile + 1);
        }
        __syncthreads();
    };
    if constexpr (DMA) {
        for (int tile = 0; tile < ntiles; tile += 2) {
            tile_step(tile, std::integral_constant<int, 0>{});
            if (tile + 1 < ntiles) tile_step(tile + 1, std::integral_constant<int, 1>{});
        }
    } else {
        for (int tile = 0; tile < ntiles; ++tile) tile_step(tile, tile & 1);
    }
    bad = __syncthreads_or(bad);

    // row sums over the 4 token groups; the accumulator holds d = 16 b + 4 kg + r
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        lsum[mb] = row_reduce4<false>(lsum[mb]);
    }
    if constexpr (SHARED) {
        // the partition's partial result per row: running max (log2
        // domain), sum and unnormalised output, fp32; NaN sum and output
        // for a row that read an invalid block id or broke the sharing.
        // (Non-temporal stores: 4% faster here, where the partials of 16
        // or more partitions per row are written at once at the end.)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (!row_ok[mb]) continue;
            const bool nan =
                bad || seq_bad[(w_first + 16 * mb + lrow) / G - s_first] != 0;
            const int64_t slot = (obase[mb] / D) * p.num_slots + part;
            float *po = p.part_out + slot * D;
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                // (through scalars: clang reads element 0 for a bit cast of
                // an indexed vector element)
                const float o0 = acc[mb][b][0], o1 = acc[mb][b][1], o2 = acc[mb][b][2],
                            o3 = acc[mb][b][3];
                const u32x4 c = nan ? u32x4{0x7FC00000u, 0x7FC00000u, 0x7FC00000u, 0x7FC00000u}
                                    : u32x4{__builtin_bit_cast(uint32_t, o0),
                                            __builtin_bit_cast(uint32_t, o1),
                                            __builtin_bit_cast(uint32_t, o2),
                                            __builtin_bit_cast(uint32_t, o3)};
                store16_stream(po + b * 16 + 4 * kg, c);
            }
            if (kg == 0) {
                __builtin_nontemporal_store(nan ? 0.0f : m[mb], p.part_max + slot);
                __builtin_nontemporal_store(nan ? NAN : lsum[mb], p.part_sum + slot);
            }
        }
        return;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        if (!row_ok[mb]) continue;
        const float inv = lsum[mb] > 0.0f ? 1.0f / lsum[mb] : 0.0f;
        char *op = static_cast<char *>(p.out) + obase[mb] * 2;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            uint64_t v;
            if (bad) {
                v = ((uint64_t)T::kNanPair << 32) | T::kNanPair;
            } else {
                float o4[8] = {acc[mb][b][0] * inv, acc[mb][b][1] * inv, acc[mb][b][2] * inv,
                               acc[mb][b][3] * inv, 0.0f, 0.0f, 0.0f, 0.0f};
                const u32x4 c = T::narrow_chunk(o4);
                v = (uint64_t)c[0] | ((uint64_t)c[1] << 32);
            }
            *reinterpret_cast<uint64_t *>(op + (b * 16 + 4 * kg) * 2) = v;
        }
    }
}

template <class T, int D>
void launch_d(const PrefillParams &p, hipStream_t stream) {
    const unsigned grid = (unsigned)((int64_t)p.num_seqs * p.num_kv_heads * p.row_blocks);
    if (p.block_size >= 16)
        hipLaunchKernelGGL((prefill_kernel<T, D, true, false>), dim3(grid),
                           dim3(kPrefillThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_kernel<T, D, false, false>), dim3(grid),
                           dim3(kPrefillThreads), 0, stream, p);
}

template <class T, int D>
void launch_shared_d(const PrefillParams &p, hipStream_t stream) {
    const unsigned grid = (unsigned)((int64_t)p.num_kv_heads * p.row_blocks * p.prefix_parts);
    if (p.block_size >= 16)
        hipLaunchKernelGGL((prefill_kernel<T, D, true, true>), dim3(grid),
                           dim3(kPrefillThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_kernel<T, D, false, true>), dim3(grid),
                           dim3(kPrefillThreads), 0, stream, p);
}

template <class T>
hipError_t launch_shared_t(const PrefillParams &p, int head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: launch_shared_d<T, 64>(p, stream); break;
        case 128: launch_shared_d<T, 128>(p, stream); break;
        case 256: launch_shared_d<T, 256>(p, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class T>
hipError_t launch_t(const PrefillParams &p, int head_dim, hipStream_t stream) {
    switch (head_dim) {
        case 64: launch_d<T, 64>(p, stream); break;
        case 128: launch_d<T, 128>(p, stream); break;
        case 256: launch_d<T, 256>(p, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int prefill_rows_per_block(int head_dim) { return rows_per_workgroup(head_dim); }

hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_dim, hipStream_t stream) {
    switch (dtype) {
        case 1: return launch_t<F16>(p, head_dim, stream);
        case 2: return launch_t<BF16>(p, head_dim, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_shared_prefix(const PrefillParams &p, int dtype, int head_dim,
                                hipStream_t stream) {
    switch (dtype) {
        case 1: return launch_shared_t<F16>(p, head_dim, stream);
        case 2: return launch_shared_t<BF16>(p, head_dim, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
