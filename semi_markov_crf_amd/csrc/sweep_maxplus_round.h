// Max-plus (Viterbi) streaming sweep for small label counts (C <= 16), ROUND positions per
// workgroup barrier: the (max, +) form of k_lse_round (sweep_lse_round.h) with backpointers.
//
//  * chain wavefront (threads 0..63): lane c holds label c.  Per position p: the best
//    segment ending at p with label c over durations k = 1 .. DIRECT (register history of
//    the label's ring entries) and the bulk best over k >= 2*ROUND; then the transition
//    step over every label's value (DPP row broadcast), lowest-index argmax on ties
//    (durations before previous labels, k = 1 first).  Backpointer of (p, c):
//    k | c' << 16 (c' = best previous label of a segment of label c starting at p).
//  * bulk wavefronts (threads 64..): label rings in LDS, bulk max and its lowest k over
//    durations k >= 2*ROUND for the positions of the next round, ring insertion and
//    rebases one round late, S staging.
// Values are natural-log scores kept relative to a per-label fp64 base (moved every
// second round) and a common fp64 reference H that advances by integers.
#pragma once

#include "internal.h"
#include "ring.h"

namespace semicrf {

namespace {

// out[i] = v of lane i of this lane's 16-lane row, i < N (DPP row_newbcast, gfx90a+)
template <int N, int I = 0>
__device__ __forceinline__ void row_bcast_all_mp(float v, float* out) {
    if constexpr (I < N) {
        out[I] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                       0x150 + I, 0xF, 0xF, false));
        row_bcast_all_mp<N, I + 1>(v, out);
    }
}

__device__ __forceinline__ double nan_mp() { return __longlong_as_double(0x7ff8000000000000LL); }

}  // namespace

// G: bulk lanes per label (C <= 256/G); KPL: durations per bulk lane (k = 2*ROUND + j +
// i*G); MIR: mirrored ring.  Grid (B), block 64 + ceil(C*G/64)*64 threads.
template <int G, int KPL, bool MIR>
__global__ __launch_bounds__(320) void k_maxplus_round(const SweepArgs a, const int RS,
                                                      const int P, const int CH) {
    constexpr int M = ROUND;
    constexpr int CP = 256 / G;
    static_assert(CP <= 16, "the labels of the chain wavefront share one DPP row");
    constexpr int PF = (lse_chunk_max(G) + 1 + G - 1) / G;
    constexpr int KP = KPL > 0 ? KPL : 1;
    constexpr int HN = DIRECT + M;
    extern __shared__ double lds[];
    const int C = a.C, K = a.K, T = a.T;
    const int tid = threadIdx.x, NT = blockDim.x, NB = NT - 64;
    const bool chain = __builtin_amdgcn_readfirstlane(tid >> 6) == 0;
    const int bt = tid - 64;
    const int cb = chain ? C : bt / G;
    const int j = chain ? 0 : bt - cb * G;
    const bool bact = !chain && cb < C;
    const int cr = bact ? cb : C;
    const bool cact = chain && tid < C;
    const int cl = cact ? tid : 0;

    const int b = blockIdx.x;
    const int Lr = a.Leff[b];
    const bool bad = Lr < 0;
    const int L = bad ? -Lr : Lr;
    const int t0 = 0, t1 = L;
    const int RMASK = RS - 1;
    const int rowsN = (CH + 1) * C;

    double* Sbuf = lds;                                    // [2][CH+1][C]
    float* R = (float*)(Sbuf + 2 * rowsN);                 // [C+1][P]
    float* qsh = R + (C + 1) * P;                          // [2 rounds][M][max, k][CP]
    float* nsh = qsh + 2 * M * 2 * CP;                     // [2 rounds][M][CP] ring entries
    float* dlsh = nsh + 2 * M * CP;                        // [CP] rebase shift per label
    float* dummy = dlsh + CP;                              // [NT]
    float* Rrow = R + cr * P;

    const double* Sb = a.S + (size_t)b * (T + 1) * C;
    for (int q = tid; q < (C + 1) * P; q += NT) R[q] = NEG;

    // ---------------------------------------------------------------- constants
    auto durv = [&](int c, int k) -> float {
        return k <= K ? fmaxf(a.dur[(k - 1) * C + c], NEG) : NEG;
    };
    float dreg[KP];
#pragma unroll
    for (int i = 0; i < KPL; ++i) dreg[i] = bact ? durv(cb, 2 * M + j + i * G) : NEG;
    float dlog[DIRECT];
#pragma unroll
    for (int k = 0; k < DIRECT; ++k) dlog[k] = cact ? durv(cl, k + 1) : NEG;
    float treg[CP];
#pragma unroll
    for (int i = 0; i < CP; ++i) treg[i] = (cact && i < C) ? fmaxf(a.trans[i * C + cl], NEG) : NEG;
    __syncthreads();   // ring cleared

    // bulk best (k >= 2M) of the M positions p0 .. p0+M-1, published for round r
    auto bulk_round = [&](int r, int p0) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float best = NEG;
            int kb = INT_MAX;
            if constexpr (KPL > 0) {
                float v[KP];
                ring_load<G, KPL, MIR>(Rrow, p0 + m - 2 * M + 3, j, RS, v);
                best = group_argmax<G, KPL>(v, dreg, j, &kb);   // k = 3 + j + i*G here
                kb += 2 * M - 3;                                 // shift to k = 2M + j + i*G
            }
            float* slot = qsh + ((r & 1) * M + m) * 2 * CP;
            *(bact && j == 0 ? slot + cb : dummy + tid) = best;
            *(bact && j == 0 ? slot + CP + cb : dummy + tid) = __int_as_float(kb);
        }
    };

    // ---------------------------------------------------------------- start state
    if (bact && j == 0) ring_put<MIR>(Rrow, 0, RS, 0.0f);   // position 0: no transition into it
    float Rh[HN];
#pragma unroll
    for (int i = 0; i < HN; ++i) Rh[i] = NEG;
    Rh[DIRECT - 1] = 0.0f;
    double Bc = 0.0, H = 0.0;
    float Mref = 0.0f;

    double pf[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) pf[i] = 0.0;
    if (!chain) {
        for (int q = bt; q < rowsN; q += NB) {
            const int t = t0 + 1 + q / C;
            Sbuf[q] = (t <= t1) ? Sb[(size_t)(t0 + 1) * C + q] : 0.0;
        }
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int q = bt + i * NB;
            if (q < rowsN && t0 + 1 + CH + q / C <= t1) pf[i] = Sb[(size_t)(t0 + 1 + CH) * C + q];
        }
    }
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0);
    if (!chain) bulk_round(0, t0 + 1);
    __syncthreads();

    // ---------------------------------------------------------------- main loop
    double BH = Bc - H;
    float pdl = 0.0f;
    bool pend = false;
    const size_t outrow = (size_t)b * (T + 1);
    const int nrounds = (t1 - t0 + M - 1) / M;
    int tc = t0 + 1, nch = 0;
    for (int r = 0; r < nrounds; ++r) {
        const int rs = t0 + r * M;
        if (rs + 1 >= tc + CH) {
            tc += CH;
            ++nch;
        }
        const double* Srow = Sbuf + (nch & 1) * rowsN;
        const int row0 = rs + 1 - tc;
        if (chain) {
            float Q[M];
            int kQ[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float* slot = qsh + ((r & 1) * M + m) * 2 * CP;
                Q[m] = slot[cl];
                kQ[m] = __float_as_int(slot[CP + cl]);
            }
            if (pend) {
#pragma unroll
                for (int m = 0; m < M; ++m) Q[m] -= pdl;
                pend = false;
            }
            if ((r & 1) == 0 && r > 0) {
                const float ref = fmaxf(Mref, Rh[DIRECT - 1]);
                const float dl = cact && ref > NEG_HALF ? ref : 0.0f;
                Bc += (double)dl;
                BH += (double)dl;
                Mref -= dl;
#pragma unroll
                for (int i = 0; i < DIRECT; ++i) Rh[i] -= dl;
#pragma unroll
                for (int m = 0; m < M; ++m) Q[m] -= dl;
                *(cact ? dlsh + cl : dummy + tid) = dl;
                pdl = dl;
                pend = true;
            }
            const double H0 = H;
            float hb[M];
#pragma unroll
            for (int m = 0; m < M; ++m) hb[m] = (float)(Srow[(row0 + m) * C + cl] + BH);
            int eacc = 0;
            int ev[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int p = rs + 1 + m;
                // best segment of label cl ending at p: durations 1 .. DIRECT, then the bulk
                float best = Q[m];
                int kbest = kQ[m];
#pragma unroll
                for (int k = DIRECT; k >= 1; --k) {         // later k first: ties go to lower k
                    const float x = Rh[DIRECT - 1 + m + 1 - k] + dlog[k - 1];
                    if (x >= best) {
                        best = x;
                        kbest = k;
                    }
                }
                const float hp = hb[m] - (float)eacc;          // S(p) + B_c - H(p)
                const float u = cact ? hp + best : NEG;        // V(p, cl) - H(p)
                // transition step of p over every label's value
                float uv[CP];
                row_bcast_all_mp<CP>(u, uv);
                float mt = NEG, mu = NEG;
                int cbest = 0;
#pragma unroll
                for (int i = 0; i < CP; ++i) {
                    const float y = uv[i] + treg[i];
                    if (y > mt) {                               // strict: lowest c' on ties
                        mt = y;
                        cbest = i;
                    }
                    mu = fmaxf(mu, uv[i]);
                }
                const int e = mu > NEG_HALF ? (int)floorf(mu) : 0;
                Rh[DIRECT + m] = mt - hp;
                if (p <= t1 && cact)   // the label of position L + 1 is never read
                    a.bp[(outrow + p) * C + cl] = (uint32_t)kbest | ((uint32_t)cbest << 16);
                if (p == L) {
                    // final label: lowest argmax of V(L, c)
                    int cs = 0;
                    float vs = uv[0];
#pragma unroll
                    for (int i = 1; i < CP; ++i)
                        if (uv[i] > vs) {
                            vs = uv[i];
                            cs = i;
                        }
                    if (tid == 0) {
                        a.vscore[b] = bad ? nan_mp() : H0 + (double)eacc + (double)vs;
                        a.vcstar[b] = cs;
                    }
                }
                ev[m] = e;
                eacc += e;
            }
            int et = 0;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int p = rs + 1 + m;
                if (p > t1) break;
                et += ev[m];
                *(cact ? nsh + ((r & 1) * M + m) * CP + cl : dummy + tid) = Rh[DIRECT + m];
                if (Q[m] > NEG_HALF) Mref = Q[m];
            }
            H = H0 + (double)et;
            BH = Bc - H;
#pragma unroll
            for (int i = 0; i < DIRECT; ++i) Rh[i] = Rh[i + M];
        } else {
            if (rs + 1 == tc && tc + CH <= t1) {
                double* dst = Sbuf + ((nch + 1) & 1) * rowsN;
#pragma unroll
                for (int i = 0; i < PF; ++i) {
                    const int q = bt + i * NB;
                    if (q < rowsN) dst[q] = pf[i];
                }
#pragma unroll
                for (int i = 0; i < PF; ++i) {
                    const int q = bt + i * NB;
                    if (q < rowsN) pf[i] = (tc + 2 * CH + q / C <= t1) ? Sb[(size_t)(tc + 2 * CH) * C + q] : 0.0;
                }
            }
            // the chain rebased last round: move the live entries (positions rs-K-M+2 .. rs)
            if (r >= 3 && (r & 1) == 1) {
                const float dl = bact ? dlsh[cb] : 0.0f;
                constexpr int KR = KPL + 1;
                float v[KR];
#pragma unroll
                for (int i = 0; i < KR; ++i) v[i] = Rrow[(rs - j - i * G) & RMASK];
#pragma unroll
                for (int i = 0; i < KR; ++i) {
                    // slots outside the live window go to the spare row (read by idle lanes)
                    const int q = j + i * G;
                    const bool live = (q < K + M) & (rs - q >= 0);
                    ring_put<MIR>(live ? Rrow : R + C * P, rs - q, RS, v[i] - dl);
                }
            }
            // insert the chain's entries of round r-1
            if (r >= 1 && bact && j < M && rs - M + 1 + j <= t1)
                ring_put<MIR>(Rrow, rs - M + 1 + j, RS, nsh[(((r - 1) & 1) * M + j) * CP + cb]);
            bulk_round(r + 1, rs + M + 1);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ launch
template <int G, int KPL, bool MIR>
static hipError_t launch_maxplus_round_inst(const SweepArgs& a, const SweepCfg& cfg,
                                            hipStream_t stream) {
    if (cfg.NT > 320 || cfg.vit.CH > lse_chunk_max(G) || cfg.vit.CH % ROUND != 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_maxplus_round<G, KPL, MIR>), dim3(a.B), dim3(cfg.NT), cfg.vit.bytes,
                       stream, a, cfg.RS, cfg.vit.P, cfg.vit.CH);
    return hipGetLastError();
}

#define MAXPLUS_ROUND_KPL_CASES(G)                                               \
    switch (cfg.KPLr) {                                                          \
        case 0: return launch_maxplus_round_inst<G, 0, MIR>(a, cfg, stream);        \
        case 1: return launch_maxplus_round_inst<G, 1, MIR>(a, cfg, stream);        \
        case 2: return launch_maxplus_round_inst<G, 2, MIR>(a, cfg, stream);        \
        case 3: return launch_maxplus_round_inst<G, 3, MIR>(a, cfg, stream);        \
        case 4: return launch_maxplus_round_inst<G, 4, MIR>(a, cfg, stream);        \
        case 5: return launch_maxplus_round_inst<G, 5, MIR>(a, cfg, stream);        \
        case 6: return launch_maxplus_round_inst<G, 6, MIR>(a, cfg, stream);        \
        case 7: return launch_maxplus_round_inst<G, 7, MIR>(a, cfg, stream);        \
        case 8: return launch_maxplus_round_inst<G, 8, MIR>(a, cfg, stream);        \
        case 10: return launch_maxplus_round_inst<G, 10, MIR>(a, cfg, stream);      \
        case 12: return launch_maxplus_round_inst<G, 12, MIR>(a, cfg, stream);      \
        case 16: return launch_maxplus_round_inst<G, 16, MIR>(a, cfg, stream);      \
        case 24: return launch_maxplus_round_inst<G, 24, MIR>(a, cfg, stream);      \
        case 32: return launch_maxplus_round_inst<G, 32, MIR>(a, cfg, stream);      \
        default: return hipErrorInvalidValue;                                    \
    }

template <bool MIR>
hipError_t launch_maxplus_round_layout(const SweepCfg& cfg, const SweepArgs& a,
                                       hipStream_t stream) {
    if (cfg.G == 64) { MAXPLUS_ROUND_KPL_CASES(64) }
    if (cfg.G == 32) { MAXPLUS_ROUND_KPL_CASES(32) }
    if (cfg.G == 16) { MAXPLUS_ROUND_KPL_CASES(16) }
    return hipErrorInvalidValue;
}

#undef MAXPLUS_ROUND_KPL_CASES

}  // namespace semicrf
