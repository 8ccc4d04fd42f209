// Device-side helpers shared by the gfx950 kernels of the semi-CRF library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace semicrf {

// Stand-in for -inf in the log semiring: finite, so that max-subtraction of an
// all-impossible set gives exp2(0) instead of NaN, and far below any real score.
constexpr float NEG = -1.0e30f;
constexpr float NEG_HALF = -1.0e29f;
constexpr double LOG2E = 1.4426950408889634073599246810019;
constexpr double LN2 = 0.69314718055994530941723212145818;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- cross-lane all-reduce
// All-reduce over aligned groups of G lanes (G a power of two, <= 64) inside a
// wavefront, using DPP row permutations for the first four levels and the gfx950
// permlane16/32 swaps for the 16->32->64 levels.  Every lane of the group ends
// with the reduced value.

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}

constexpr int DPP_QUAD_1032 = 0xB1;   // quad_perm [1,0,3,2]: partner = lane ^ 1
constexpr int DPP_QUAD_2301 = 0x4E;   // quad_perm [2,3,0,1]: partner = lane ^ 2
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // partner = 7 - lane within 8 lanes
constexpr int DPP_ROW_MIRROR = 0x140;       // partner = 15 - lane within 16 lanes

struct OpMax {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpSum {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

template <int G, class Op>
__device__ __forceinline__ float group_reduce(float v, Op op) {
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "group size");
    if constexpr (G >= 2) v = op(v, dpp_f<DPP_QUAD_1032>(v));
    if constexpr (G >= 4) v = op(v, dpp_f<DPP_QUAD_2301>(v));
    if constexpr (G >= 8) v = op(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
    if constexpr (G >= 16) v = op(v, dpp_f<DPP_ROW_MIRROR>(v));
    if constexpr (G >= 32) {
        const int iv = __builtin_bit_cast(int, v);
        auto p = __builtin_amdgcn_permlane16_swap(iv, iv, false, false);
        v = op(__builtin_bit_cast(float, (int)p[0]), __builtin_bit_cast(float, (int)p[1]));
    }
    if constexpr (G >= 64) {
        const int iv = __builtin_bit_cast(int, v);
        auto p = __builtin_amdgcn_permlane32_swap(iv, iv, false, false);
        v = op(__builtin_bit_cast(float, (int)p[0]), __builtin_bit_cast(float, (int)p[1]));
    }
    return v;
}

template <int G>
__device__ __forceinline__ int group_min_int(int v) {
    if constexpr (G >= 2) v = min(v, dpp_i<DPP_QUAD_1032>(v));
    if constexpr (G >= 4) v = min(v, dpp_i<DPP_QUAD_2301>(v));
    if constexpr (G >= 8) v = min(v, dpp_i<DPP_ROW_HALF_MIRROR>(v));
    if constexpr (G >= 16) v = min(v, dpp_i<DPP_ROW_MIRROR>(v));
    if constexpr (G >= 32) {
        auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = min((int)p[0], (int)p[1]);
    }
    if constexpr (G >= 64) {
        auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = min((int)p[0], (int)p[1]);
    }
    return v;
}

// Block-wide sum of a double over blockDim.x threads (blockDim.x a multiple of 64,
// at most 1024).  `scratch` must hold 16 doubles.  Fixed reduction order.
__device__ __forceinline__ double block_sum_double(double v, double* scratch) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[w] = v;
    __syncthreads();
    double r = 0.0;
    const int nw = blockDim.x >> 6;
    for (int i = 0; i < nw; ++i) r += scratch[i];
    __syncthreads();
    return r;
}

}  // namespace semicrf
