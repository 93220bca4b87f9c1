// Device helpers shared by the gfx950 kernels: element types, 16-byte
// chunks, wavefront reductions on DPP, exp2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- dtypes
// Each element type knows its size, how to widen a 16-byte chunk to fp32 and
// how to narrow one fp32 result (round to nearest even).
struct F32 {
    static constexpr int kBytes = 4;
    static constexpr int kPerChunk = 4;
    __device__ static inline void widen(const u32x4 &c, float *v) {
        // element copied to a scalar first: a bit cast straight from the
        // vector element lvalue reads element 0 with this compiler
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = c[i];
            v[i] = __builtin_bit_cast(float, w);
        }
    }
    // acc + sum over the chunk of q[e] * k[e]
    __device__ static inline float dot_chunk(const u32x4 &q, const u32x4 &k, float acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t a = q[i], b = k[i];
            acc = fmaf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b), acc);
        }
        return acc;
    }
    __device__ static inline u32x4 narrow_chunk(const float *v) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = __builtin_bit_cast(uint32_t, v[i]);
        return r;
    }
    __device__ static inline void store(void *base, int64_t i, float x) {
        static_cast<float *>(base)[i] = x;
    }
    __device__ static inline void store_nan(void *base, int64_t i) {
        static_cast<uint32_t *>(base)[i] = 0x7FC00000u;
    }
    static constexpr uint32_t kNanPair = 0x7FC00000u;  // one NaN element per word
};

struct F16 {
    static constexpr int kBytes = 2;
    static constexpr int kPerChunk = 8;
    __device__ static inline void widen(const u32x4 &c, float *v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = c[i];
            v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
            v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
        }
    }
    // acc + sum over the chunk of q[e] * k[e]: products of two f16 values are
    // exact in fp32, the dot instruction adds them in fp32.
    __device__ static inline float dot_chunk(const u32x4 &q, const u32x4 &k, float acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t a = q[i], b = k[i];
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b),
                                         acc, false);
        }
        return acc;
    }
    __device__ static inline u32x4 narrow_chunk(const float *v) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i]);
            const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1]);
            r[i] = lo | (hi << 16);
        }
        return r;
    }
    __device__ static inline void store(void *base, int64_t i, float x) {
        static_cast<_Float16 *>(base)[i] = (_Float16)x;
    }
    __device__ static inline void store_nan(void *base, int64_t i) {
        static_cast<uint16_t *>(base)[i] = 0x7E00u;
    }
    static constexpr uint32_t kNanPair = 0x7E007E00u;
};

struct BF16 {
    static constexpr int kBytes = 2;
    static constexpr int kPerChunk = 8;
    __device__ static inline void widen(const u32x4 &c, float *v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = c[i];
            v[2 * i] = __builtin_bit_cast(float, w << 16);
            v[2 * i + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
        }
    }
    __device__ static inline uint16_t narrow(float x) {
        const uint32_t u = __builtin_bit_cast(uint32_t, x);
        if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;  // NaN stays NaN
        return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    }
    // acc + sum over the chunk of q[e] * k[e]: products of two bf16 values
    // are exact in fp32, the dot instruction adds them in fp32.
    __device__ static inline float dot_chunk(const u32x4 &q, const u32x4 &k, float acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t a = q[i], b = k[i];
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                                  __builtin_bit_cast(bf16x2, b), acc, false);
        }
        return acc;
    }
    __device__ static inline u32x4 narrow_chunk(const float *v) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r[i] = (uint32_t)narrow(v[2 * i]) | ((uint32_t)narrow(v[2 * i + 1]) << 16);
        return r;
    }
    __device__ static inline void store(void *base, int64_t i, float x) {
        static_cast<uint16_t *>(base)[i] = narrow(x);
    }
    __device__ static inline void store_nan(void *base, int64_t i) {
        static_cast<uint16_t *>(base)[i] = 0x7FC0u;
    }
    static constexpr uint32_t kNanPair = 0x7FC07FC0u;
};

// ------------------------------------------------------------ memory ops
__device__ inline u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
// Streaming load for data read once (the K/V pool): the non-temporal hint
// keeps it from displacing reused lines and raises the achieved HBM read rate
// on this part (about 6.5 vs 5.8 TB/s for random 32 KB blocks).
__device__ inline u32x4 load16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ inline void store16(void *p, const u32x4 &v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}
// Streaming (non-temporal) 16-byte vector store, for data not read again soon.
__device__ inline void store16_stream(void *p, const u32x4 &v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// ------------------------------------------------------------------ DPP
// dpp_ctrl encodings (GFX9 DPP): quad_perm [1,0,3,2] swaps neighbours,
// [2,3,0,1] swaps pairs; row_half_mirror reverses each 8-lane half row;
// row_mirror reverses each 16-lane row.  Applied in this order after the
// lanes of every quad hold the same value, each step pairs lanes that hold
// disjoint partial results, so all lanes of the row end with the full result.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Every control used here reads a lane of the same row, so no lane reads out
// of bounds and the instruction needs no old value.
template <int CTRL>
__device__ inline float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// max(a, b) as IEEE 754-2019 maximum: one instruction on gfx950 (fmaxf also
// quiets signalling NaNs first, which costs a second one).  A NaN operand
// gives NaN; no NaN reaches these reductions from valid inputs.
__device__ inline float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Sum over groups of N consecutive lanes (N in 1, 2, 4, 8, 16, 32, 64);
// every lane receives its group's sum.
template <int N>
__device__ inline float group_sum(float x) {
    if constexpr (N >= 2) x += dpp<kDppQuadXor1>(x);
    if constexpr (N >= 4) x += dpp<kDppQuadXor2>(x);
    if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

template <int N>
__device__ inline float group_max(float x) {
    if constexpr (N >= 2) x = vmax(x, dpp<kDppQuadXor1>(x));
    if constexpr (N >= 4) x = vmax(x, dpp<kDppQuadXor2>(x));
    if constexpr (N >= 8) x = vmax(x, dpp<kDppRowHalfMirror>(x));
    if constexpr (N >= 16) x = vmax(x, dpp<kDppRowMirror>(x));
    if constexpr (N >= 32) x = vmax(x, __shfl_xor(x, 16));
    if constexpr (N >= 64) x = vmax(x, __shfl_xor(x, 32));
    return x;
}

// Sum / max across lanes that differ only in lane bits [log2(STRIDE), 6):
// combines the "token groups" of a wave whose lanes are laid out as
// (group, lane-in-group) with STRIDE lanes per group.
template <int STRIDE>
__device__ inline float across_groups_sum(float x) {
    if constexpr (STRIDE <= 1) x += dpp<kDppQuadXor1>(x);
    if constexpr (STRIDE <= 2) x += dpp<kDppQuadXor2>(x);
    if constexpr (STRIDE <= 4) x += __shfl_xor(x, 4);
    if constexpr (STRIDE <= 8) x += __shfl_xor(x, 8);
    if constexpr (STRIDE <= 16) x += __shfl_xor(x, 16);
    if constexpr (STRIDE <= 32) x += __shfl_xor(x, 32);
    return x;
}

template <int STRIDE>
__device__ inline float across_groups_max(float x) {
    if constexpr (STRIDE <= 1) x = vmax(x, dpp<kDppQuadXor1>(x));
    if constexpr (STRIDE <= 2) x = vmax(x, dpp<kDppQuadXor2>(x));
    if constexpr (STRIDE <= 4) x = vmax(x, __shfl_xor(x, 4));
    if constexpr (STRIDE <= 8) x = vmax(x, __shfl_xor(x, 8));
    if constexpr (STRIDE <= 16) x = vmax(x, __shfl_xor(x, 16));
    if constexpr (STRIDE <= 32) x = vmax(x, __shfl_xor(x, 32));
    return x;
}

// 2^x on the hardware transcendental unit (2^-inf = 0).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pkv
