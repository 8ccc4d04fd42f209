// Posterior marginals and gradients of log Z on gfx950.
//
// The sweeps write, per position, the forward and backward messages before the
// transition step (natural log, each span in its own frame):
//   XF[s,c] = alpha[s,c]       (segments of label c ending at s, their end projection included)
//   XB[s,c] = beta_bar[s,c]    (suffixes whose first segment, label c, starts at s)
// k_trans_step takes the transition step once per position, in place, and leaves the
// start-side and end-side values in base 2, frame offsets added, shifted so that a
// segment's posterior is one exponential:
//   AF[s,c] = log2 e (log sum_c' exp(XF[s,c'] + trans[c',c]) - S[s,c] + P_start[s,c] + S[L,c] - logZ)
//             (s = 0: log2 e (P_start[0,c] + S[L,c] - logZ))
//   AB[u,c] = log2 e (log sum_c'' exp(XB[u,c''] + trans[c,c'']) + S[u,c] - S[L,c] + P_end[u-1,c])
//             (u = L: log2 e P_end[L-1,c])
//   p(s,k,c) = 2^(AF[s,c] + AB[s+k,c] + log2 e dur[k-1,c])
// and, from the messages before it, the transition posteriors
// exp(XF[s,c'] + trans[c',c] + XB[s,c] - logZ), summed per tile group.  Their sums are the
// gradients of log Z with respect to dur and trans, and the position marginal mu[t,c] (the
// probability that t lies in a segment of label c) is the mass of the segments covering
// t.  The pages validate exactly these quantities ("Streaming Structured Inference with
// Flash-SemiCRF", gist.science EN explainer, "4. Results and Benchmarks": marginals sum
// to 1, exact gradients).
//
// mu is formed as a prefix sum over positions of (start mass - end mass), where both
// masses are fp64 sums of the same per-segment values, so each segment's contribution
// cancels exactly once it has ended.  The prefix is kept as an fp32 prefix inside each
// tile plus an fp64 prefix of the tile totals.  mu is then divided by its sum over labels
// at each position (1 in exact arithmetic; the tests bound its distance from 1), which
// removes the slow drift between the forward and backward sweeps' rounding over
// 10^5..10^6 positions; the dur / trans partial sums of a tile are divided by the tile's
// mean normaliser.  The start and end masses at each position, divided by the same
// per-position normaliser, are the gradients with respect to the projections; their sum
// over labels at t is the probability that a segment boundary (a segment start) lies at t
// (the pages check that these boundary probabilities are valid at genome scale,
// "4. Results and Benchmarks").
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace semicrf {

// LDS of k_marginals for CL labels, tile TM and duration chunk KC: the tile's own start /
// end values, the two shifted windows of a chunk, start / end mass accumulators (fp64), the
// prefix scratch (256 doubles) and the chunk's durations (fp32).
static size_t marg_lds(int CL, int TM, int KC) {
    return (size_t)8 * CL * (6 * TM + 2 * KC) + (size_t)8 * 256 + (size_t)4 * KC * CL;
}

// Labels a k_marginals workgroup takes: all of them up to 16, else groups of 16.
int marg_labels(int C) { return C <= 16 ? C : 16; }

__host__ __device__ static inline int c4_of(int C) { return (C + 3) / 4 * 4; }
// LDS of k_trans_step_wide (more than 16 labels) for tile TM
static size_t step_lds_wide(int C, int TM) {
    const int C4 = c4_of(C);
    return (size_t)8 * (2 * TM * C + 2 * TM) + (size_t)4 * TM + (size_t)8 * TM * C4 +
           (size_t)4 * C4 * C4 + 32;
}

// Tile and duration chunk.  First choice: the largest tile of at least max(32, K/4)
// positions (the per-tile duration partials, K*C doubles, then take at most as much memory
// as the per-position input arrays) whose LDS, with a chunk of at least min(K, 64) durations, lets
// three workgroups share a CU (12 wavefronts to hide the latency of the exponentials and
// the fp64 sums).  Otherwise the largest tile that fits one workgroup per CU with such a
// chunk; the smallest tile takes any chunk.
static void marg_shape(int C, int K, int* tm, int* kc) {
    const int CL = marg_labels(C);
    // chunks of equal size (ceil(K / n) for the fewest chunks n that fit): no short last
    // chunk that stages a whole window for a few durations and leaves most lanes of the
    // duration partials idle
    auto chunks = [&](int t, int min_kc, size_t budget) {
        for (int n = 1; n <= K; ++n) {
            const int k = (K + n - 1) / n;
            if (k < min_kc) break;
            if (k <= 512 && marg_lds(CL, t, k) <= budget) return k;
        }
        return 0;
    };
    // above 16 labels the transition step shares the tile: keep its LDS within 150 KB
    int tmax = 512;
    while (C > 16 && tmax > 8 && step_lds_wide(C, tmax) > 150 * 1024) tmax >>= 1;
    int tmin = 32;
    while (tmin < 512 && 4 * tmin < K) tmin *= 2;
    for (int t = tmax; t >= tmin; t >>= 1) {
        const int k = chunks(t, std::min(K, 64), 52 * 1024);
        if (k > 0) {
            *tm = t;
            *kc = k;
            return;
        }
    }
    for (int t = tmax; t >= 8; t >>= 1) {
        const int k = chunks(t, t > 8 ? std::min(K, 64) : 1, 150 * 1024);
        if (k > 0) {
            *tm = t;
            *kc = k;
            return;
        }
    }
    *tm = 8;
    *kc = 1;
}

int marg_tile(int C, int K) {
    int tm, kc;
    marg_shape(C, K, &tm, &kc);
    return tm;
}

int marg_kchunk(int C, int K) {
    int tm, kc;
    marg_shape(C, K, &tm, &kc);
    return kc;
}

constexpr double DNEG = -1.0e300;

// LDS of k_trans_step for tile TM: both directions' messages (fp64) and their
// exponentials relative to the row maximum (fp32), the row maxima, the transitions in
// base 2 and as linear weights.
static size_t step_lds(int C, int TM) {
    return (size_t)TM * C * (2 * 8 + 2 * 4) + (size_t)2 * 8 * TM + (size_t)2 * 4 * C * C;
}

// grid (ngroups, B), block 256: the tiles g*tpg .. (g+1)*tpg - 1 of sequence b in order.
// Per tile: stage the messages of both directions (frame offsets added, base 2); the
// transition partials, lanes over (c', c) (an fp32 sum over the tile's rows, then fp64
// across the group's tiles); then the transition step of every row and direction, lanes
// over (row, label), as a linear sum of the row's exponentials (relative to the row
// maximum) against 2^(trans - max trans), redone exactly in log space where that sum
// leaves [2^-100, inf); written back over the messages.  CT > 0: C = CT known at compile
// time.
template <int CT>
__global__ __launch_bounds__(256) void k_trans_step(const TransStepArgs a) {
    extern __shared__ double lds[];
    const int C = CT ? CT : a.C, T = a.T, TM = a.tile;
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int L = abs(a.Leff[b]);
    const size_t rowC = (size_t)(T + 1) * C;
    double* X1 = lds;                                // [TM][C] forward messages
    double* X2 = X1 + (size_t)TM * C;                // [TM][C] backward messages
    double* m1 = X2 + (size_t)TM * C;                // [TM] row maxima
    double* m2 = m1 + TM;
    float* E1 = (float*)(m2 + TM);                   // [TM][C] 2^(X - row max)
    float* E2 = E1 + (size_t)TM * C;
    float* tr2 = E2 + (size_t)TM * C;                // [C][C] trans * log2 e
    float* trw = tr2 + (size_t)C * C;                // [C][C] 2^(tr2 - max tr2)

    for (int q = tid; q < C * C; q += 256) tr2[q] = fmaxf((float)((double)a.trans[q] * LOG2E), NEG);
    __syncthreads();
    float tmax = NEG;
    for (int q = 0; q < C * C; ++q) tmax = fmaxf(tmax, tr2[q]);
    for (int q = tid; q < C * C; q += 256) trw[q] = fast_exp2(tr2[q] - tmax);

    double* XF = a.XF + (size_t)b * rowC;
    double* XB = a.XB + (size_t)b * rowC;
    const double* Sb = a.S + (size_t)b * rowC;
    const float* Ps = a.proj_start ? a.proj_start + (size_t)b * T * C : nullptr;
    const float* Pe = a.proj_end ? a.proj_end + (size_t)b * T * C : nullptr;
    const double logZ = a.logz[b];
    // frame offsets of the spans that wrote each value (0 without speculative spans):
    // forward X of position s from span floor((s-1)/delta), backward X of s from the span
    // of the mirrored position L - s - 1
    const double* offF = a.off ? a.off + (size_t)b * a.nspans : nullptr;
    const double* offB = a.off ? a.off + ((size_t)a.B + b) * a.nspans : nullptr;
    auto oXF = [&](int s) { return offF ? offF[(s - 1) / a.delta] : 0.0; };
    auto oXB = [&](int s) { return offB ? offB[(L - s - 1) / a.delta] : 0.0; };
    double* part_trans = a.part_trans + ((size_t)b * a.ngroups + g) * C * C;

    const int tile_end = min(a.ntiles, (g + 1) * a.tpg);
    for (int tile = g * a.tpg; tile < tile_end; ++tile) {
        const int p0 = tile * TM;
        const bool first = tile == g * a.tpg;
        __syncthreads();   // the previous tile's LDS is read no more
        for (int q = tid; q < TM * C; q += 256) {
            const int r = q / C, c = q - r * C;
            const int s = p0 + r;
            const bool in = s >= 1 && s <= L - 1;
            X1[q] = in ? (XF[(size_t)s * C + c] + oXF(s)) * LOG2E : DNEG;
            X2[q] = in ? (XB[(size_t)s * C + c] + oXB(s)) * LOG2E : DNEG;
        }
        __syncthreads();
        // transition partials
        const double lz2 = logZ * LOG2E;
        for (int q = tid; q < C * C; q += 256) {
            const int cp = q / C, c = q - cp * C;
            const float tv = tr2[q];
            float acc = 0.0f;
            for (int r = 0; r < TM; ++r) {
                const double v = X1[(size_t)r * C + cp] + X2[(size_t)r * C + c] - lz2;
                acc += fast_exp2((float)v + tv);
            }
            part_trans[q] = first ? (double)acc : part_trans[q] + (double)acc;
        }
        // row maxima, then the exponentials relative to them
        for (int r = tid; r < 2 * TM; r += 256) {
            const double* x = (r < TM ? X1 : X2) + (size_t)(r % TM) * C;
            double m = DNEG;
            for (int c = 0; c < C; ++c) m = fmax(m, x[c]);
            (r < TM ? m1 : m2)[r % TM] = m;
        }
        __syncthreads();
        for (int q = tid; q < 2 * TM * C; q += 256) {
            const bool fw = q < TM * C;
            const int qq = fw ? q : q - TM * C;
            const int r = qq / C;
            (fw ? E1 : E2)[qq] = fast_exp2((float)((fw ? X1 : X2)[qq] - (fw ? m1 : m2)[r]));
        }
        __syncthreads();
        // the transition step; rows outside the sequence (and the unwritten message rows
        // 0 of XF and L of XB) take their boundary values
        for (int q = tid; q < 2 * TM * C; q += 256) {
            const bool fw = q < TM * C;
            const int qq = fw ? q : q - TM * C;
            const int r = qq / C, c = qq - r * C;
            const int s = p0 + r;
            if (s > T) continue;
            double out;
            if (fw) {
                if (s == 0) out = ((Ps ? (double)Ps[c] : 0.0) + (offF ? offF[0] : 0.0) +
                                   Sb[(size_t)L * C + c] - logZ) * LOG2E;
                else if (s > L - 1) out = DNEG;
                else {
                    const float* e = E1 + (size_t)r * C;
                    float acc = 0.0f;
                    for (int j = 0; j < C; ++j) acc = fmaf(e[j], trw[j * C + c], acc);
                    float lv = fast_log2(acc) + tmax;
                    if (!(acc >= 0x1p-100f)) {
                        const double* x = X1 + (size_t)r * C;
                        float m = NEG;
                        for (int j = 0; j < C; ++j) m = fmaxf(m, (float)(x[j] - m1[r]) + tr2[j * C + c]);
                        float z = 0.0f;
                        for (int j = 0; j < C; ++j) z += fast_exp2((float)(x[j] - m1[r]) + tr2[j * C + c] - m);
                        lv = m + fast_log2(z);
                    }
                    out = m1[r] + (double)lv +
                          ((Ps ? (double)Ps[(size_t)s * C + c] : 0.0) - Sb[(size_t)s * C + c] +
                           Sb[(size_t)L * C + c] - logZ) * LOG2E;
                }
                XF[(size_t)s * C + c] = out;
            } else {
                if (s == L) out = ((Pe ? (double)Pe[(size_t)(L - 1) * C + c] : 0.0) +
                                   (offB ? offB[0] : 0.0)) * LOG2E;
                else if (s < 1 || s > L) out = DNEG;
                else {
                    const float* e = E2 + (size_t)r * C;
                    float acc = 0.0f;
                    for (int j = 0; j < C; ++j) acc = fmaf(e[j], trw[c * C + j], acc);
                    float lv = fast_log2(acc) + tmax;
                    if (!(acc >= 0x1p-100f)) {
                        const double* x = X2 + (size_t)r * C;
                        float m = NEG;
                        for (int j = 0; j < C; ++j) m = fmaxf(m, (float)(x[j] - m2[r]) + tr2[c * C + j]);
                        float z = 0.0f;
                        for (int j = 0; j < C; ++j) z += fast_exp2((float)(x[j] - m2[r]) + tr2[c * C + j] - m);
                        lv = m + fast_log2(z);
                    }
                    out = m2[r] + (double)lv +
                          ((Pe ? (double)Pe[(size_t)(s - 1) * C + c] : 0.0) + Sb[(size_t)s * C + c] -
                           Sb[(size_t)L * C + c]) * LOG2E;
                }
                XB[(size_t)s * C + c] = out;
            }
        }
    }
}

// Label counts above 16: the two sums over labels of k_trans_step are small dense
// products per tile, [C x TM] x [TM x C] for the transition posteriors and
// [TM x C] x [C x C] per direction for the transition step, so they run register-blocked
// (4 x 4 outputs a thread, float4 operands from LDS, labels padded to C4 = ceil(C/4)*4
// with zeros) on the row exponentials E = 2^(X - row max):
//   partial[c', c] = 2^tr2[c', c] * sum_r 2^(m1[r] + m2[r] - log2 Z) E1[r, c'] E2[r, c]
// The row scale 2^(m1 + m2 - log2 Z) is at most about 2^(-min tr2) in exact arithmetic (a
// transition posterior is at most 1); a tile in which it, or 2^(max tr2), would leave the
// fp32 range (above 2^60) sums the exact per-term exponentials instead.  The transition
// step and its log-space replay are those of k_trans_step.

__global__ __launch_bounds__(256) void k_trans_step_wide(const TransStepArgs a) {
    extern __shared__ double lds[];
    const int C = a.C, T = a.T, TM = a.tile, C4 = c4_of(C);
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int L = abs(a.Leff[b]);
    const size_t rowC = (size_t)(T + 1) * C;
    double* X1 = lds;                                // [TM][C] forward messages (base 2)
    double* X2 = X1 + (size_t)TM * C;                // [TM][C] backward messages
    double* m1 = X2 + (size_t)TM * C;                // [TM] row maxima
    double* m2 = m1 + TM;
    float* sc = (float*)(m2 + TM);                   // [TM] 2^(m1 + m2 - log2 Z)
    float* E1 = sc + TM;                             // [TM][C4] 2^(X1 - m1), pad 0
    float* E2 = E1 + (size_t)TM * C4;                // [TM][C4]
    float* trw = E2 + (size_t)TM * C4;               // [C4][C4] 2^(tr2 - tmax), pad 0
    float* red = trw + (size_t)C4 * C4;              // [4] wavefront maxima
    int& exact_flag = *reinterpret_cast<int*>(red + 4);   // exact partials for this tile

    auto tr2_at = [&](int q) { return fmaxf((float)((double)a.trans[q] * LOG2E), NEG); };
    // tmax: block maximum of tr2
    float tm_loc = NEG;
    for (int q = tid; q < C * C; q += 256) tm_loc = fmaxf(tm_loc, tr2_at(q));
    for (int off = 32; off >= 1; off >>= 1) tm_loc = fmaxf(tm_loc, __shfl_xor(tm_loc, off, 64));
    if ((tid & 63) == 0) red[tid >> 6] = tm_loc;
    __syncthreads();
    const float tmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    for (int q = tid; q < C4 * C4; q += 256) {
        const int i = q / C4, j = q - i * C4;
        trw[q] = (i < C && j < C) ? fast_exp2(tr2_at(i * C + j) - tmax) : 0.0f;
    }

    double* XF = a.XF + (size_t)b * rowC;
    double* XB = a.XB + (size_t)b * rowC;
    const double* Sb = a.S + (size_t)b * rowC;
    const float* Ps = a.proj_start ? a.proj_start + (size_t)b * T * C : nullptr;
    const float* Pe = a.proj_end ? a.proj_end + (size_t)b * T * C : nullptr;
    const double logZ = a.logz[b];
    const double lz2 = logZ * LOG2E;
    const double* offF = a.off ? a.off + (size_t)b * a.nspans : nullptr;
    const double* offB = a.off ? a.off + ((size_t)a.B + b) * a.nspans : nullptr;
    auto oXF = [&](int s) { return offF ? offF[(s - 1) / a.delta] : 0.0; };
    auto oXB = [&](int s) { return offB ? offB[(L - s - 1) / a.delta] : 0.0; };
    double* part_trans = a.part_trans + ((size_t)b * a.ngroups + g) * C * C;
    const int NB4 = C4 / 4;

    const int tile_end = min(a.ntiles, (g + 1) * a.tpg);
    for (int tile = g * a.tpg; tile < tile_end; ++tile) {
        const int p0 = tile * TM;
        const bool first = tile == g * a.tpg;
        __syncthreads();   // the previous tile's LDS is read no more
        if (tid == 0) exact_flag = tmax > 60.0f;
        for (int q = tid; q < TM * C; q += 256) {
            const int r = q / C, c = q - r * C;
            const int s = p0 + r;
            const bool in = s >= 1 && s <= L - 1;
            X1[q] = in ? (XF[(size_t)s * C + c] + oXF(s)) * LOG2E : DNEG;
            X2[q] = in ? (XB[(size_t)s * C + c] + oXB(s)) * LOG2E : DNEG;
        }
        __syncthreads();
        for (int r = tid; r < 2 * TM; r += 256) {
            const double* x = (r < TM ? X1 : X2) + (size_t)(r % TM) * C;
            double m = DNEG;
            for (int c = 0; c < C; ++c) m = fmax(m, x[c]);
            (r < TM ? m1 : m2)[r % TM] = m;
        }
        __syncthreads();
        for (int r = tid; r < TM; r += 256) {
            const double e = m1[r] + m2[r] - lz2;
            if (e > 60.0) exact_flag = 1;
            sc[r] = fast_exp2((float)e);
        }
        for (int q = tid; q < 2 * TM * C4; q += 256) {
            const bool fw = q < TM * C4;
            const int qq = fw ? q : q - TM * C4;
            const int r = qq / C4, c = qq - r * C4;
            float e = 0.0f;
            if (c < C) e = fast_exp2((float)((fw ? X1 : X2)[(size_t)r * C + c] - (fw ? m1 : m2)[r]));
            (fw ? E1 : E2)[qq] = e;
        }
        __syncthreads();
        // transition partials, 4 x 4 blocks of (c', c)
        const bool exact = exact_flag;
        for (int q = tid; q < NB4 * NB4; q += 256) {
            const int i0 = (q / NB4) * 4, l0 = (q % NB4) * 4;
            float acc[4][4] = {};
            if (!exact) {
                for (int r = 0; r < TM; ++r) {
                    const float sr = sc[r];
                    const float4 x = *reinterpret_cast<const float4*>(E1 + (size_t)r * C4 + i0);
                    const float4 y = *reinterpret_cast<const float4*>(E2 + (size_t)r * C4 + l0);
                    const float xa[4] = {x.x * sr, x.y * sr, x.z * sr, x.w * sr};
                    const float ya[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int l = 0; l < 4; ++l) acc[i][l] = fmaf(xa[i], ya[l], acc[i][l]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int l = 0; l < 4; ++l) {
                    const int cp = i0 + i, c = l0 + l;
                    if (cp >= C || c >= C) continue;
                    const float tv = tr2_at(cp * C + c);
                    float v;
                    if (!exact) {
                        v = acc[i][l] * fast_exp2(tv);
                    } else {
                        v = 0.0f;
                        for (int r = 0; r < TM; ++r)
                            v += fast_exp2((float)(X1[(size_t)r * C + cp] + X2[(size_t)r * C + c] - lz2) + tv);
                    }
                    double* pt = part_trans + (size_t)cp * C + c;
                    *pt = first ? (double)v : *pt + (double)v;
                }
        }
        // the transition step, 4 rows x 4 labels a block per direction
        const int RB = TM / 4;
        for (int q = tid; q < 2 * RB * NB4; q += 256) {
            const bool fw = q < RB * NB4;
            const int qq = fw ? q : q - RB * NB4;
            const int r0 = (qq / NB4) * 4, l0 = (qq % NB4) * 4;
            const float* E = fw ? E1 : E2;
            float acc[4][4] = {};
            for (int j = 0; j < C4; j += 4) {
                float e[4][4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 v = *reinterpret_cast<const float4*>(E + (size_t)(r0 + i) * C4 + j);
                    e[i][0] = v.x; e[i][1] = v.y; e[i][2] = v.z; e[i][3] = v.w;
                }
                float w[4][4];   // w[jj][l]: weight of label j + jj into label l0 + l
                if (fw) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float4 v = *reinterpret_cast<const float4*>(trw + (size_t)(j + jj) * C4 + l0);
                        w[jj][0] = v.x; w[jj][1] = v.y; w[jj][2] = v.z; w[jj][3] = v.w;
                    }
                } else {
#pragma unroll
                    for (int l = 0; l < 4; ++l) {
                        const float4 v = *reinterpret_cast<const float4*>(trw + (size_t)(l0 + l) * C4 + j);
                        w[0][l] = v.x; w[1][l] = v.y; w[2][l] = v.z; w[3][l] = v.w;
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                        for (int l = 0; l < 4; ++l) acc[i][l] = fmaf(e[i][jj], w[jj][l], acc[i][l]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int l = 0; l < 4; ++l) {
                    const int r = r0 + i, c = l0 + l;
                    const int s = p0 + r;
                    if (c >= C || s > T) continue;
                    const float sum = acc[i][l];
                    double out;
                    if (fw) {
                        if (s == 0) out = ((Ps ? (double)Ps[c] : 0.0) + (offF ? offF[0] : 0.0) +
                                           Sb[(size_t)L * C + c] - logZ) * LOG2E;
                        else if (s > L - 1) out = DNEG;
                        else {
                            float lv = fast_log2(sum) + tmax;
                            if (!(sum >= 0x1p-100f)) {
                                const double* x = X1 + (size_t)r * C;
                                float m = NEG;
                                for (int jx = 0; jx < C; ++jx) m = fmaxf(m, (float)(x[jx] - m1[r]) + tr2_at(jx * C + c));
                                float z = 0.0f;
                                for (int jx = 0; jx < C; ++jx) z += fast_exp2((float)(x[jx] - m1[r]) + tr2_at(jx * C + c) - m);
                                lv = m + fast_log2(z);
                            }
                            out = m1[r] + (double)lv +
                                  ((Ps ? (double)Ps[(size_t)s * C + c] : 0.0) - Sb[(size_t)s * C + c] +
                                   Sb[(size_t)L * C + c] - logZ) * LOG2E;
                        }
                        XF[(size_t)s * C + c] = out;
                    } else {
                        if (s == L) out = ((Pe ? (double)Pe[(size_t)(L - 1) * C + c] : 0.0) +
                                           (offB ? offB[0] : 0.0)) * LOG2E;
                        else if (s < 1 || s > L) out = DNEG;
                        else {
                            float lv = fast_log2(sum) + tmax;
                            if (!(sum >= 0x1p-100f)) {
                                const double* x = X2 + (size_t)r * C;
                                float m = NEG;
                                for (int jx = 0; jx < C; ++jx) m = fmaxf(m, (float)(x[jx] - m2[r]) + tr2_at(c * C + jx));
                                float z = 0.0f;
                                for (int jx = 0; jx < C; ++jx) z += fast_exp2((float)(x[jx] - m2[r]) + tr2_at(c * C + jx) - m);
                                lv = m + fast_log2(z);
                            }
                            out = m2[r] + (double)lv +
                                  ((Pe ? (double)Pe[(size_t)(s - 1) * C + c] : 0.0) + Sb[(size_t)s * C + c] -
                                   Sb[(size_t)L * C + c]) * LOG2E;
                        }
                        XB[(size_t)s * C + c] = out;
                    }
                }
        }
    }
}

hipError_t launch_trans_step(const TransStepArgs& a, hipStream_t stream) {
    if (a.tpg < 1 || a.ngroups != (a.ntiles + a.tpg - 1) / a.tpg) return hipErrorInvalidValue;
    if (a.C > 16) {
        if (a.tile % 4 != 0) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_trans_step_wide, dim3(a.ngroups, a.B), dim3(256),
                           step_lds_wide(a.C, a.tile), stream, a);
        return hipGetLastError();
    }
    const dim3 grid(a.ngroups, a.B);
    const size_t lds = step_lds(a.C, a.tile);
#define STEP_CASE(n) \
    case n: hipLaunchKernelGGL(k_trans_step<n>, grid, dim3(256), lds, stream, a); break;
    switch (a.C) {
        STEP_CASE(1) STEP_CASE(2) STEP_CASE(3) STEP_CASE(4) STEP_CASE(5) STEP_CASE(6)
        STEP_CASE(7) STEP_CASE(8) STEP_CASE(9) STEP_CASE(10) STEP_CASE(11) STEP_CASE(12)
        STEP_CASE(13) STEP_CASE(14) STEP_CASE(15) STEP_CASE(16)
        default: hipLaunchKernelGGL(k_trans_step<0>, grid, dim3(256), lds, stream, a); break;
    }
#undef STEP_CASE
    return hipGetLastError();
}

// grid (ngroups, B, label groups), block 256: the tiles g*tpg .. (g+1)*tpg - 1 of sequence
// b in order, for the labels c0 .. c0+CL-1 of one label group (c0 = z * cg; the labels are
// independent here, and a group of at most 16 keeps the staged windows small enough for
// several workgroups a CU at large label counts).  Durations are taken in chunks [kc0, kc1] of at most KC: per chunk the starts
// [p0 - kc1, p0 + TM - 1 - kc0] and the ends [p0 + kc0, p0 + TM - 1 + kc1] are staged
// beside the tile's own starts and ends.  The duration partials of the group's tiles are
// summed in tile order (each lane owns the same entries in every tile).
// CLT > 0: the workgroup takes all CLT = C labels, known at compile time (the LDS strides
// and the row / label splits of the lane indexes fold into constants); CLT = 0: label
// groups of a.cg, the last one possibly shorter.
template <int CLT>
__global__ __launch_bounds__(256) void k_marginals(const MargArgs a) {
    extern __shared__ double lds[];
    const int C = a.C, K = a.K, T = a.T, TM = a.tile, KC = a.kchunk;
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int c0 = CLT ? 0 : blockIdx.z * a.cg;
    const int CL = CLT ? CLT : min(a.cg, C - c0);   // this workgroup's labels
    const int L = abs(a.Leff[b]);
    const size_t rowC = (size_t)(T + 1) * C;

    // LDS rows hold the group's CL labels
    double* AFt = lds;                               // [TM][CL]: starts p0 .. p0+TM-1
    double* ABt = AFt + (size_t)TM * CL;             // [TM][CL]: ends p0 .. p0+TM-1
    double* AFw = ABt + (size_t)TM * CL;             // [TM+KC][CL]: starts of the chunk's ends
    double* ABw = AFw + (size_t)(TM + KC) * CL;      // [TM+KC][CL]: ends of the chunk's starts
    double* Dst = ABw + (size_t)(TM + KC) * CL;      // [TM][CL] start mass
    double* Den = Dst + (size_t)TM * CL;             // [TM][CL] end mass
    double* csum = Den + (size_t)TM * CL;            // [256] prefix scratch
    float* dur2 = (float*)(csum + 256);              // [KC][CL]

    double* part_dur = a.part_dur + ((size_t)b * a.ngroups + g) * K * C;
    float* Dloc = a.Dloc + (size_t)b * T * C;
    const double* AF = a.AF + (size_t)b * rowC;
    const double* AB = a.AB + (size_t)b * rowC;
    const int tile_end = min(a.ntiles, (g + 1) * a.tpg);
    // q over [rows][CL]: row q / CL, global label c0 + q % CL
    for (int tile = g * a.tpg; tile < tile_end; ++tile) {
        const int p0 = tile * TM;
        const bool first = tile == g * a.tpg;    // stores the group's partials, later tiles add
        double* dn_tile = a.dn_tile + ((size_t)b * a.ntiles + tile) * C;
        if (p0 > L) {   // nothing of this sequence here
            for (int q = tid; q < CL; q += 256) dn_tile[c0 + q] = 0.0;
            for (int q = tid; q < TM * CL; q += 256) {
                const int r = q / CL;
                if (p0 + r < T) Dloc[(size_t)(p0 + r) * C + c0 + (q - r * CL)] = 0.0f;
            }
            if (first)
                for (int q = tid; q < K * CL; q += 256) {
                    const int k = q / CL;
                    part_dur[(size_t)k * C + c0 + (q - k * CL)] = 0.0;
                }
            continue;
        }
        // base 2; invalid starts / ends get DNEG so that their exponentials vanish
        auto af = [&](int s, int c) -> double {
            return (s >= 0 && s <= L - 1) ? AF[(size_t)s * C + c0 + c] : DNEG;
        };
        auto ab = [&](int u, int c) -> double {
            return (u >= 1 && u <= L) ? AB[(size_t)u * C + c0 + c] : DNEG;
        };

        for (int q = tid; q < TM * CL; q += 256) {
            const int r = q / CL, c = q - r * CL;
            const int s = p0 + r;
            AFt[q] = af(s, c);
            ABt[q] = ab(s, c);
            Dst[q] = 0.0;
            Den[q] = 0.0;
        }

        auto seg = [&](double v, float d) -> float { return fast_exp2((float)v + d); };

        for (int kc0 = 1; kc0 <= K; kc0 += KC) {
            const int kc1 = min(K, kc0 + KC - 1);
            const int nk = kc1 - kc0 + 1;
            __syncthreads();   // the previous chunk's windows are no longer read
            for (int q = tid; q < (TM + nk - 1) * CL; q += 256) {
                const int r = q / CL, c = q - r * CL;
                AFw[q] = af(p0 - kc1 + r, c);
                ABw[q] = ab(p0 + kc0 + r, c);
            }
            for (int q = tid; q < nk * CL; q += 256) {
                const int k = q / CL, c = q - k * CL;
                dur2[q] = fmaxf((float)((double)a.dur[(size_t)(kc0 - 1 + k) * C + c0 + c] * LOG2E), NEG);
            }
            __syncthreads();

            // ---- phase 1: per position, start and end mass of the chunk's segments (fp64
            // sums of the same per-segment values: they cancel exactly in mu's prefix)
            for (int q = tid; q < TM * CL; q += 256) {
                const int r = q / CL, c = q - r * CL;
                if (p0 + r > L) continue;
                double st = Dst[q], en = Den[q];
                const double a0 = AFt[q], b0 = ABt[q];
#pragma unroll 4
                for (int k = kc0; k <= kc1; ++k) {
                    const float d = dur2[(k - kc0) * CL + c];
                    st += (double)seg(a0 + ABw[(size_t)(r + k - kc0) * CL + c], d);   // [t, t+k)
                    en += (double)seg(AFw[(size_t)(r + kc1 - k) * CL + c] + b0, d);   // [t-k, t)
                }
                Dst[q] = st;
                Den[q] = en;
            }

            // ---- phase 2: duration partials, lanes over (k, c), segments starting in the
            // tile (an fp32 sum over the tile's rows, then fp64 across tiles)
            for (int q = tid; q < nk * CL; q += 256) {
                const int kk = q / CL, c = q - kk * CL;
                const float d = dur2[q];
                float acc = 0.0f;
#pragma unroll 4
                for (int r = 0; r < TM; ++r)
                    acc += seg(AFt[(size_t)r * CL + c] + ABw[(size_t)(r + kk) * CL + c], d);
                double* pd = part_dur + (size_t)(kc0 - 1 + kk) * C + c0 + c;
                *pd = first ? (double)acc : *pd + (double)acc;
            }
        }
        __syncthreads();

        // ---- raw boundary masses, then start mass - end mass per position
        if (a.pstart || a.pend)
            for (int q = tid; q < TM * CL; q += 256) {
                const int r = q / CL, c = c0 + (q - r * CL);
                const int t = p0 + r;
                if (a.pstart && t < L) a.pstart[((size_t)b * T + t) * C + c] = (float)Dst[q];
                if (a.pend && t >= 1 && t <= L) a.pend[((size_t)b * T + t - 1) * C + c] = (float)Den[q];
            }
        if (a.pbsum) {
            // one label group: the sum itself; several: this group's share, which
            // k_node_marginals adds up in group order
            float* out = a.cg < C ? a.pb_part + (size_t)blockIdx.z * a.B * T : a.pbsum;
            for (int r = tid; r < TM; r += 256) {
                const int t = p0 + r;
                if (t >= L) continue;
                double s = 0.0;
                for (int c = 0; c < CL; ++c) s += Dst[(size_t)r * CL + c];
                out[(size_t)b * T + t] = (float)s;
            }
        }
        __syncthreads();
        for (int q = tid; q < TM * CL; q += 256) Dst[q] -= Den[q];
        __syncthreads();
        // in-tile inclusive prefix per label: lanes over (label, row chunk), fixed order;
        // the last row's value is the tile total
        for (int cb = 0; cb < CL; cb += 256) {
            const int CW = min(256, CL - cb);
            const int R = 256 / CW;
            const int chunk = (TM + R - 1) / R;
            const int cw = tid % CW, r = tid / CW, c = cb + cw;
            const bool act = r < R;
            double acc = 0.0;
            if (act)
                for (int i = r * chunk; i < min(TM, (r + 1) * chunk); ++i) acc += Dst[(size_t)i * CL + c];
            csum[tid] = acc;
            __syncthreads();
            if (act) {
                double run = 0.0;
                for (int qq = 0; qq < r; ++qq) run += csum[qq * CW + cw];
                for (int i = r * chunk; i < min(TM, (r + 1) * chunk); ++i) {
                    run += Dst[(size_t)i * CL + c];
                    if (p0 + i < T) Dloc[(size_t)(p0 + i) * C + c0 + c] = (float)run;
                    if (i == TM - 1) dn_tile[c0 + c] = run;
                }
            }
            __syncthreads();
        }
    }
}

hipError_t launch_marginals(const MargArgs& a, hipStream_t stream) {
    if (a.cg < 1 || a.cg > a.C) return hipErrorInvalidValue;
    const int nlg = (a.C + a.cg - 1) / a.cg;
    if (nlg > 1 && a.pbsum && !a.pb_part) return hipErrorInvalidValue;
    const size_t lds = marg_lds(a.cg, a.tile, a.kchunk);
    if (a.tpg < 1 || a.ngroups != (a.ntiles + a.tpg - 1) / a.tpg) return hipErrorInvalidValue;
    const dim3 grid(a.ngroups, a.B, nlg);
#define MARG_CASE(n) \
    case n: hipLaunchKernelGGL(k_marginals<n>, grid, dim3(256), lds, stream, a); break;
    switch (nlg == 1 ? a.C : 0) {
        MARG_CASE(1) MARG_CASE(2) MARG_CASE(3) MARG_CASE(4) MARG_CASE(5) MARG_CASE(6)
        MARG_CASE(7) MARG_CASE(8) MARG_CASE(9) MARG_CASE(10) MARG_CASE(11) MARG_CASE(12)
        MARG_CASE(13) MARG_CASE(14) MARG_CASE(15) MARG_CASE(16)
        default: hipLaunchKernelGGL(k_marginals<0>, grid, dim3(256), lds, stream, a); break;
    }
#undef MARG_CASE
    return hipGetLastError();
}

int marg_tiles_per_group(int B, int ntiles, int C, int K) {
    // a group per tile while the partials stay within the budget (longer workgroups leave
    // the device's last pass over them mostly idle: four tiles a group cost 45 % more time
    // at B = 4, T = 10^5, K = 200), else the fewest tiles a group that meet it
    constexpr size_t BUDGET = (size_t)64 << 20;          // bytes of partials
    constexpr long long TARGET = 8192;                   // workgroups
    int tpg = (int)std::max<long long>(1, ((long long)B * ntiles + TARGET - 1) / TARGET);
    auto bytes = [&](int t) {
        return (size_t)B * ((ntiles + t - 1) / t) * (size_t)(8 * K + 8 * C) * C;
    };
    while (tpg < ntiles && bytes(tpg) > BUDGET) tpg *= 2;
    return std::min(tpg, std::max(ntiles, 1));
}

// grid (ntiles, B), block 256: mu over positions [p0, p0+TM) = the tile's offset (fp64
// prefix of the tile totals) + the in-tile prefix, normalised per position (one reciprocal
// of the raw sum per position); tile sums of mu and the tile's mean normaliser; the
// boundary outputs rescaled in place.  CT > 0: C = CT known at compile time.
template <int CT>
__global__ __launch_bounds__(256) void k_node_marginals(const float* Dloc,
                                                        const double* __restrict__ dn_off,
                                                        const int* __restrict__ Leff, int T, int Cr,
                                                        int TM, float* mu,
                                                        double* __restrict__ mu_tile,
                                                        double* __restrict__ z_tile,
                                                        const BoundaryOut bo) {
    extern __shared__ double lds[];
    const int C = CT ? CT : Cr;
    const int tile = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, ntiles = gridDim.x;
    const int L = abs(Leff[b]);
    const int p0 = tile * TM;
    double* v = lds;                       // [TM][C]
    double* zrow = v + (size_t)TM * C;     // [TM]
    double* rz = zrow + TM;                // [TM]: 1 / zrow
    const float* D = Dloc + (size_t)b * T * C;
    const int rows = max(0, min(TM, L - p0));   // positions p0 .. p0+rows-1 are < L
    const double* off = dn_off + ((size_t)b * ntiles + tile) * C;
    for (int q = tid; q < rows * C; q += 256) v[q] = off[q % C] + (double)D[(size_t)p0 * C + q];
    __syncthreads();
    for (int r = tid; r < rows; r += 256) {
        double z = 0.0;
        for (int c = 0; c < C; ++c) z += v[(size_t)r * C + c];
        zrow[r] = z;
        rz[r] = 1.0 / z;
    }
    __syncthreads();
    if (bo.node_mass)
        for (int r = tid; r < TM; r += 256) {
            const int t = p0 + r;
            if (t < T) bo.node_mass[(size_t)b * T + t] = r < rows ? (float)zrow[r] : 0.0f;
        }
    {
        // boundary probabilities and the projections' gradients: the raw start / end
        // masses over the same per-position normaliser (0 at padding)
        const double g = bo.grad_log_z ? (double)bo.grad_log_z[b] : 1.0;
        if (bo.boundary)
            for (int r = tid; r < TM; r += 256) {
                const int t = p0 + r;
                if (t >= T) continue;
                float* o = bo.boundary + (size_t)b * T + t;
                double raw = 0.0;
                if (r < rows) {
                    if (bo.pb_part)
                        for (int gq = 0; gq < bo.npb; ++gq) raw += (double)bo.pb_part[((size_t)gq * gridDim.y + b) * T + t];
                    else
                        raw = (double)*o;
                }
                *o = r < rows ? (float)(raw * rz[r]) : 0.0f;
            }
        if (bo.grad_proj_start || bo.grad_proj_end)
            for (int q = tid; q < TM * C; q += 256) {
                const int r = q / C;
                const int t = p0 + r;
                if (t >= T) continue;
                const size_t idx = (size_t)b * T * C + (size_t)p0 * C + q;
                const bool in = r < rows;
                if (bo.grad_proj_start)
                    bo.grad_proj_start[idx] =
                        in ? (float)(g * (double)bo.grad_proj_start[idx] * rz[r]) : 0.0f;
                if (bo.grad_proj_end)
                    bo.grad_proj_end[idx] =
                        in ? (float)(g * (double)bo.grad_proj_end[idx] * rz[r]) : 0.0f;
            }
    }
    float* mub = mu + (size_t)b * T * C;
    for (int q = tid; q < TM * C; q += 256) {
        const int r = q / C;
        const int t = p0 + r;
        if (t >= T) continue;
        float val = 0.0f;
        if (r < rows) {
            const double w = v[q] * rz[r];
            v[q] = w;
            val = (float)w;
        }
        mub[(size_t)t * C + (q - r * C)] = val;
    }
    __syncthreads();
    for (int c = tid; c < C; c += 256) {
        double s = 0.0;
        for (int r = 0; r < rows; ++r) s += v[(size_t)r * C + c];
        mu_tile[((size_t)b * ntiles + tile) * C + c] = s;
    }
    if (tid == 0) {
        double z = 0.0;
        for (int r = 0; r < rows; ++r) z += zrow[r];
        z_tile[(size_t)b * ntiles + tile] = rows > 0 ? z / rows : 1.0;
    }
}

hipError_t launch_node_marginals(const float* Dloc, const double* dn_off, const int* Leff, int B,
                                 int T, int C, int tile, int ntiles, float* mu, double* mu_tile,
                                 double* z_tile, const BoundaryOut& bo, hipStream_t stream) {
    const size_t lds = (size_t)8 * ((size_t)tile * C + 2 * tile);
    const dim3 grid(ntiles, B);
#define NODE_CASE(n)                                                                          \
    case n:                                                                                   \
        hipLaunchKernelGGL(k_node_marginals<n>, grid, dim3(256), lds, stream, Dloc, dn_off, Leff, \
                           T, C, tile, mu, mu_tile, z_tile, bo);                               \
        break;
    switch (C <= 16 ? C : 0) {
        NODE_CASE(1) NODE_CASE(2) NODE_CASE(3) NODE_CASE(4) NODE_CASE(5) NODE_CASE(6)
        NODE_CASE(7) NODE_CASE(8) NODE_CASE(9) NODE_CASE(10) NODE_CASE(11) NODE_CASE(12)
        NODE_CASE(13) NODE_CASE(14) NODE_CASE(15) NODE_CASE(16)
        default:
            hipLaunchKernelGGL(k_node_marginals<0>, grid, dim3(256), lds, stream, Dloc, dn_off,
                               Leff, T, C, tile, mu, mu_tile, z_tile, bo);
            break;
    }
#undef NODE_CASE
    return hipGetLastError();
}

// grid (ceil(T*C/256), B): grad_em = g * (mu - mean over the valid positions of mu).
// CT > 0: C = CT known at compile time.
template <int CT>
__global__ __launch_bounds__(256) void k_grad_em(const float* mu,
                                                 const double* __restrict__ mu_tot,
                                                 const int* __restrict__ Leff,
                                                 const float* __restrict__ grad_log_z, int T,
                                                 int Cr, float* grad_em) {
    const int C = CT ? CT : Cr;
    const int b = blockIdx.y;
    const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (size_t)T * C) return;
    const int L = abs(Leff[b]);
    const int t = (int)(q / C), c = (int)(q - (size_t)t * C);
    const size_t idx = (size_t)b * T * C + q;
    float out = 0.0f;
    if (t < L) {
        const double g = grad_log_z ? (double)grad_log_z[b] : 1.0;
        out = (float)(g * ((double)mu[idx] - mu_tot[(size_t)b * C + c] / (double)L));
    }
    grad_em[idx] = out;
}

hipError_t launch_grad_em(const float* mu, const double* mu_tot, const int* Leff,
                          const float* grad_log_z, int B, int T, int C, float* grad_em,
                          hipStream_t stream) {
    const size_t n = (size_t)T * C;
    const dim3 grid((unsigned)((n + 255) / 256), B);
#define GEM_CASE(n)                                                                            \
    case n:                                                                                    \
        hipLaunchKernelGGL(k_grad_em<n>, grid, dim3(256), 0, stream, mu, mu_tot, Leff, grad_log_z, \
                           T, C, grad_em);                                                      \
        break;
    switch (C <= 16 ? C : 0) {
        GEM_CASE(1) GEM_CASE(2) GEM_CASE(3) GEM_CASE(4) GEM_CASE(5) GEM_CASE(6)
        GEM_CASE(7) GEM_CASE(8) GEM_CASE(9) GEM_CASE(10) GEM_CASE(11) GEM_CASE(12)
        GEM_CASE(13) GEM_CASE(14) GEM_CASE(15) GEM_CASE(16)
        default:
            hipLaunchKernelGGL(k_grad_em<0>, grid, dim3(256), 0, stream, mu, mu_tot, Leff,
                               grad_log_z, T, C, grad_em);
            break;
    }
#undef GEM_CASE
    return hipGetLastError();
}

// one thread per output element of grad_dur [K*C] followed by grad_trans [C*C]
// grad_dur / grad_trans = sum over sequences b of g_b * sum over tile groups j of
// part[b][j] / z_j, z_j the mean per-position normaliser over the group's valid positions
// (it drifts by far less than 1e-6 across a group).  Pass 1: grid (ceil(n / 64),
// RP_SLICES / 4), block 256; lane (e, slice) sums the groups j = slice, slice + RP_SLICES,
// ... of every sequence into scratch[slice][e].  Pass 2: four wavefronts per 64 outputs
// add every fourth slice, then the four partials are added in order.  Fixed order throughout: bitwise reproducible.
constexpr int RP_SLICES = 128;

__global__ __launch_bounds__(256) void k_reduce_partials(const double* __restrict__ part_dur,
                                                         const double* __restrict__ part_trans,
                                                         const double* __restrict__ z_tile,
                                                         const int* __restrict__ Leff,
                                                         const float* __restrict__ grad_log_z,
                                                         int B, int C, int K, int TM, int ntiles,
                                                         int tpg, int ngroups,
                                                         double* __restrict__ scratch) {
    // weights g_b / z_j of the (sequence, group) pairs of this workgroup's four slices,
    // RP_W of them a pass, computed once and shared by the workgroup's 64 elements
    constexpr int RP_W = 256;
    __shared__ double wq[RP_W];
    const int n = K * C + C * C;
    const int e = blockIdx.x * 64 + (threadIdx.x & 63);
    const int sl4 = threadIdx.x >> 6;
    const int slice = blockIdx.y * 4 + sl4;
    const int nd = K * C;
    const bool isd = e < nd;
    const int ee = isd ? e : e - nd;
    const int stride = isd ? nd : C * C;
    const int npairs = B * ngroups;
    // pass m covers the pairs blockIdx.y * 4 + s + RP_SLICES * i, s < 4, i in
    // [m * RP_W / 4, (m + 1) * RP_W / 4): wq[s * RP_W / 4 + i - m * RP_W / 4]
    double total = 0.0;
    const int iters = (npairs + RP_SLICES - 1) / RP_SLICES;
    for (int i0 = 0; i0 < iters; i0 += RP_W / 4) {
        __syncthreads();   // the previous pass's weights are no longer read
        {
            const int s = threadIdx.x / (RP_W / 4), i = i0 + threadIdx.x % (RP_W / 4);
            const int q = blockIdx.y * 4 + s + RP_SLICES * i;
            double w = 0.0;
            if (q < npairs) {
                const int b = q / ngroups, j = q - b * ngroups;
                const int L = abs(Leff[b]);
                double zs = 0.0, ns = 0.0;
                for (int tl = j * tpg; tl < min(ntiles, (j + 1) * tpg); ++tl) {
                    const int rows = max(0, min(TM, L - tl * TM));
                    zs += (double)rows * z_tile[(size_t)b * ntiles + tl];
                    ns += (double)rows;
                }
                w = (grad_log_z ? (double)grad_log_z[b] : 1.0) / (ns > 0.0 ? zs / ns : 1.0);
            }
            wq[threadIdx.x] = w;
        }
        __syncthreads();
        if (e < n) {
            const int i1 = min(iters, i0 + RP_W / 4);
            // the pairs in order; the iterations are independent until the sum, so their
            // loads overlap
#pragma unroll 4
            for (int i = i0; i < i1; ++i) {
                const int q = slice + RP_SLICES * i;
                if (q >= npairs) break;
                const size_t at = (size_t)q * stride + ee;   // q = b * ngroups + j
                const double x = isd ? (double)part_dur[at] : part_trans[at];
                total += wq[sl4 * (RP_W / 4) + (i - i0)] * x;
            }
        }
    }
    if (e < n) scratch[(size_t)slice * n + e] = total;
}

// block 256 over 64 consecutive outputs: wavefront w adds the slices w, w + 4, ... of its
// lane's output, then lane 0..63 of wavefront 0 adds the four partials in order.
__global__ __launch_bounds__(256) void k_reduce_slices(const double* __restrict__ scratch, int C,
                                                       int K, float* __restrict__ grad_dur,
                                                       float* __restrict__ grad_trans) {
    __shared__ double part[4][64];
    const int n = K * C + C * C;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    double total = 0.0;
    if (e < n)
#pragma unroll 8
        for (int sl = w; sl < RP_SLICES; sl += 4) total += scratch[(size_t)sl * n + e];
    part[w][lane] = total;
    __syncthreads();
    if (w == 0 && e < n) {
        const double t = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
        if (e < K * C) grad_dur[e] = (float)t;
        else grad_trans[e - K * C] = (float)t;
    }
}

size_t reduce_scratch_doubles(int C, int K) { return (size_t)RP_SLICES * (K * C + C * C); }

hipError_t launch_reduce_partials(const double* part_dur, const double* part_trans,
                                  const double* z_tile, const int* Leff, const float* grad_log_z,
                                  int B, int C, int K, int tile, int ntiles, int tpg,
                                  double* scratch, float* grad_dur, float* grad_trans,
                                  hipStream_t stream) {
    const int n = K * C + C * C;
    const int ngroups = (ntiles + tpg - 1) / tpg;
    hipLaunchKernelGGL(k_reduce_partials, dim3((n + 63) / 64, RP_SLICES / 4), dim3(256), 0, stream,
                       part_dur, part_trans, z_tile, Leff, grad_log_z, B, C, K, tile, ntiles,
                       tpg, ngroups, scratch);
    hipLaunchKernelGGL(k_reduce_slices, dim3((n + 63) / 64), dim3(256), 0, stream, scratch, C, K,
                       grad_dur, grad_trans);
    return hipGetLastError();
}

__global__ void k_write_logz(const double* __restrict__ logz, int B, float* __restrict__ out) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) out[b] = (float)logz[b];
}

hipError_t launch_write_logz(const double* logz, int B, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(k_write_logz, dim3((B + 255) / 256), dim3(256), 0, stream, logz, B, out);
    return hipGetLastError();
}

}  // namespace semicrf
