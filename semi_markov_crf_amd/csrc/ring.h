// Per-label ring of recent recurrence values, held in LDS, shared by the log-semiring
// and max-plus sweeps.
//
// Lanes form groups of G per label.  For the "bulk" value of position tq (the terms with
// segment length k >= 3), lane j of the group owns k = 3 + j + i*G for i < KPL, i.e. the
// ring entries of positions tq - k.  Lanes whose k exceeds K read some finite slot and
// weight it by a duration of NEG (log space) or 0 (linear space), so no lane branches on k.
//
// Two layouts (chosen on the host from the LDS budget):
//   mirrored: position p is stored in slots (p & RMASK) and (p & RMASK) + RS, so every
//             window of up to RS consecutive positions is contiguous and a lane reads its
//             KPL terms at compile-time offsets from one base address;
//   plain:    one copy, every read masked.
#pragma once

#include <limits.h>

#include "common.h"

namespace semicrf {

constexpr int REBASE = 8;   // ring values move to a new per-label base every REBASE positions

// v[i] = ring value of position tq - (3 + j + i*G)
template <int G, int KPL, bool MIR>
__device__ __forceinline__ void ring_load(const float* row, int tq, int j, int RS, float* v) {
    if constexpr (MIR) {
        // lowest address of the window; term i sits (KPL-1-i)*G above it
        const float* w = row + (((tq - 3) & (RS - 1)) + RS - j - (KPL - 1) * G);
#pragma unroll
        for (int i = 0; i < KPL; ++i) v[KPL - 1 - i] = w[i * G];
    } else {
        const int t3 = tq - 3 - j;
#pragma unroll
        for (int i = 0; i < KPL; ++i) v[i] = row[(t3 - i * G) & (RS - 1)];
    }
}

// Writes v[i] to the ring slot(s) of position tq - (3 + j + i*G).
template <int G, int KPL, bool MIR>
__device__ __forceinline__ void ring_store(float* row, int tq, int j, int RS, const float* v) {
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int s0 = (tq - 3 - j - i * G) & (RS - 1);
        row[s0] = v[i];
        if constexpr (MIR) row[s0 + RS] = v[i];
    }
}

// Writes r to the ring slot(s) of position pos.
template <bool MIR>
__device__ __forceinline__ void ring_put(float* row, int pos, int RS, float r) {
    const int s0 = pos & (RS - 1);
    row[s0] = r;
    if constexpr (MIR) row[s0 + RS] = r;
}

// log2-sum-exp2 over the group of r[i] + d[i] (all lanes of the group get the result)
template <int G, int KPL>
__device__ __forceinline__ float group_lse(const float* r, const float* d) {
    float x[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) x[i] = r[i] + d[i];
    float m = x[0];
#pragma unroll
    for (int i = 1; i < KPL; ++i) m = fmaxf(m, x[i]);
    m = group_reduce<G>(m, OpMax());
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < KPL; ++i) s += fast_exp2(x[i] - m);
    s = group_reduce<G>(s, OpSum());
    return m + fast_log2(s);
}

// max over the group of r[i] + d[i]; *kbest = lowest k = 3 + j + i*G attaining it
template <int G, int KPL>
__device__ __forceinline__ float group_argmax(const float* r, const float* d, int j, int* kbest) {
    float x[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) x[i] = r[i] + d[i];
    float m = x[0];
#pragma unroll
    for (int i = 1; i < KPL; ++i) m = fmaxf(m, x[i]);
    m = group_reduce<G>(m, OpMax());
    int kk = INT_MAX;
#pragma unroll
    for (int i = KPL - 1; i >= 0; --i)
        if (x[i] == m) kk = 3 + j + i * G;
    *kbest = group_min_int<G>(kk);
    return m;
}

}  // namespace semicrf
