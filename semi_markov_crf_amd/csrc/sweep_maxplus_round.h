// Max-plus (Viterbi) streaming sweep for small label counts (C <= 16), ROUND = 4 positions
// per workgroup barrier: the (max, +) form of k_lse_round (sweep_lse_round.h) with
// backpointers, on the same float4 ring blocks.
//
//  * chain wavefront (threads 0..63): lane c holds label c.  Per position p = (round
//    start) + 1 + m: the best segment of label c ending at p over durations k = 1 .. m+4
//    (registers: the previous round's block and this round's entries) and the bulk best
//    over the older ones; then the transition step of p over every label's value (DPP row
//    broadcast).  Ties go to the lowest index: durations before previous labels, k = 1
//    first.  Backpointer of (p, c): k | c' << 16 (c' = best previous label of a segment
//    of label c starting at p).  The chain writes its round's ring block itself.
//  * bulk wavefronts (threads 64..): lanes grouped G per label.  In round r they apply
//    the chain's rebase of round r-1 to the ring and form the bulk best (and its lowest
//    k) of each position of round r+1 over ring blocks of rounds <= r-1; they also stage
//    S, label-major.
// Values are natural-log scores relative to a per-label fp64 base (moved every second
// round) and a common fp64 reference H that advances by whole units once per round.
// Forward only: every checkpoint span at once from a burn-in (MODE_SPEC), then the repair
// of a failed seam (MODE_REPAIR); the backtrace follows the backpointers afterwards.
#pragma once

#include "internal.h"
#include "ring.h"

namespace semicrf {

namespace {

// out[i] = v of lane i of this lane's 16-lane row, i < N (DPP row_newbcast, gfx90a+; every
// lane has a source, so the bound control only lets the move fold into its consumer)
template <int N, int I = 0>
__device__ __forceinline__ void row_bcast_all_mp(float v, float* out) {
    if constexpr (I < N) {
        out[I] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                       0x150 + I, 0xF, 0xF, true));
        row_bcast_all_mp<N, I + 1>(v, out);
    }
}

__device__ __forceinline__ int slot_mp(int rho, int RMASK) { return (rho * ROUND) & RMASK; }
__device__ __forceinline__ float4 ld4_mp(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4_mp(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ float at4_mp(const float4& v, int d) {
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// max of n values (tree of v_max3)
template <int N>
__device__ __forceinline__ float max_tree(const float* x) {
    if constexpr (N == 1) return x[0];
    else if constexpr (N == 2) return fmaxf(x[0], x[1]);
    else {
        float y[(N + 2) / 3];
#pragma unroll
        for (int i = 0; i < (N + 2) / 3; ++i) {
            const float a0 = x[3 * i];
            const float a1 = 3 * i + 1 < N ? x[3 * i + 1] : a0;
            const float a2 = 3 * i + 2 < N ? x[3 * i + 2] : a0;
            y[i] = fmaxf(fmaxf(a0, a1), a2);
        }
        return max_tree<(N + 2) / 3>(y);
    }
}

// min of n values (tree of v_min3)
template <int N>
__device__ __forceinline__ int min_tree_i(const int* x) {
    if constexpr (N == 1) return x[0];
    else if constexpr (N == 2) return min(x[0], x[1]);
    else {
        int y[(N + 2) / 3];
#pragma unroll
        for (int i = 0; i < (N + 2) / 3; ++i) {
            const int a0 = x[3 * i];
            const int a1 = 3 * i + 1 < N ? x[3 * i + 1] : a0;
            const int a2 = 3 * i + 2 < N ? x[3 * i + 2] : a0;
            y[i] = min(min(a0, a1), a2);
        }
        return min_tree_i<(N + 2) / 3>(y);
    }
}

}  // namespace

// G: bulk lanes per label (C <= 256/G); BPL: ring blocks per bulk lane; CP: labels the
// chain broadcasts (>= C); PROJ: boundary projections present.  Grid (nspans, B) in
// MODE_SPEC, (B) in MODE_REPAIR; block 64 + ceil(C*G/64)*64 threads.
template <int G, int BPL, int CP, bool PROJ>
__global__ __launch_bounds__(512) void k_maxplus_round(const SweepArgs a, const int RS,
                                                      const int P, const int CH,
                                                      const float* __restrict__ proj_start,
                                                      const float* __restrict__ proj_end) {
    constexpr int M = ROUND;
    static_assert(M == 4, "ring blocks are float4");
    static_assert(CP <= 16, "the labels of the chain wavefront share one DPP row");
    static_assert(CP * G <= 512, "at most 7 bulk wavefronts beside the chain");
    constexpr int PF = (lse_chunk_max(G) + G - 1) / G;
    constexpr int BP = BPL > 0 ? BPL : 1;
    constexpr int KD = 2 * M - 1;
    constexpr int CP4 = (CP + 3) / 4 * 4;
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

    // MODE_SPEC: grid (nspans, B), every span of the forward sweep at once from a burn-in;
    // MODE_REPAIR: grid (B), the forward sweep again from the checkpoint at the first
    // failed seam.
    const bool spec = a.mode == MODE_SPEC;
    int b, span = 0;
    if (spec) {
        span = blockIdx.x; b = blockIdx.y;
    } else {
        b = blockIdx.x;
    }
    const int Lr = a.Leff[b];
    const int L = Lr < 0 ? -Lr : Lr;
    int t0 = 0, t1 = L, tout = 0;
    if (spec) {
        tout = span * a.delta;
        if (tout >= L) return;
        t1 = min(L, tout + a.delta);
        t0 = max(0, tout - a.warm);
    } else {
        span = a.first_bad[b];
        if (span >= a.nspans) return;
        tout = span * a.delta;
        if (tout >= L) return;
        t0 = tout;
    }
    const bool ckpt = spec && t1 < L;                   // checkpoint at the span's end
    const int hlo = (spec && span > 0) ? tout - K + 1 : INT_MAX;    // seam windows
    const int tlo = ckpt ? t1 - K + 1 : INT_MAX;
    const size_t winrow = ((size_t)b * a.nspans + span) * K;
    const size_t ckrow = (size_t)b * a.nspans;
    const int RMASK = RS - 1;
    const int bmax = (K + M - 1) / M;
    const int NR = bmax + 3;

    double* Sbuf = lds;                                    // [2][C][CH] label-major
    float* Pst = (float*)(Sbuf + 2 * C * CH);              // [2][end, start][C][CH] projections
    float* R = Pst + (PROJ ? 4 * C * CH : 0);              // [C+1][P]
    float* qsh = R + (C + 1) * P;                          // [2 rounds][CP][max, k][M]
    float* dlsh = qsh + 2 * CP * 2 * M;                    // [CP4] rebase shift per label
    float* sink = dlsh + CP4;                              // [8]
    float* nblk = sink + 8;                                // [4] NEG: blocks past K
    float* Rrow = R + cr * P;

    const double* Sb = a.S + (size_t)b * (T + 1) * C;
    // projections of position p: end side (segments ending at p) and start side
    // (segments starting at p); 0 without projections or outside [1, L] / [0, L-1]
    const float* PSb = proj_start ? proj_start + (size_t)b * T * C : nullptr;
    const float* PEb = proj_end ? proj_end + (size_t)b * T * C : nullptr;
    auto proj_e = [&](int p, int q) -> float {
        if constexpr (!PROJ) return 0.0f;
        return (PEb && p >= 1 && p <= L) ? PEb[(size_t)(p - 1) * C + q] : 0.0f;
    };
    auto proj_s = [&](int p, int q) -> float {
        if constexpr (!PROJ) return 0.0f;
        return (PSb && p >= 0 && p < L) ? PSb[(size_t)p * C + q] : 0.0f;
    };
    for (int q = tid; q < (C + 1) * P; q += NT) R[q] = NEG;
    for (int q = tid; q < 2 * CP * 2 * M; q += NT) qsh[q] = ((q / M) & 1) ? __int_as_float(INT_MAX) : NEG;
    if (tid < M) nblk[tid] = NEG;

    // ---------------------------------------------------------------- constants
    auto durv = [&](int c, int k) -> float {
        return (k >= 1 && k <= K) ? fmaxf(a.dur[(k - 1) * C + c], NEG) : NEG;
    };
    // bulk lanes: block i of lane j lies bb = 2 + j + i*G rounds back; its entry d enters
    // step m with duration k = 4*bb + m - d = 4*bb + t - 3, t = m - d + 3
    float Dc[BP][2 * M - 1];
#pragma unroll
    for (int i = 0; i < BPL; ++i)
#pragma unroll
        for (int t = 0; t < 2 * M - 1; ++t) Dc[i][t] = bact ? durv(cb, M * (2 + j + i * G) + t - 3) : NEG;
    float dlog[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) dlog[k] = cact ? durv(cl, k + 1) : NEG;
    float treg[CP];
#pragma unroll
    for (int i = 0; i < CP; ++i)
        treg[i] = (cact && i < C) ? fmaxf(a.trans[i * C + cl], NEG) : NEG;
    __syncthreads();   // ring cleared

    // bulk best (durations k >= m + 5) of the positions of round rr and its lowest k
    auto bulk_round = [&](int rr) {
        float Q[M];
        int kq[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            Q[m] = NEG;
            kq[m] = INT_MAX;
        }
        if constexpr (BPL > 0) {
            float4 v[BP];
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                const int bb = 2 + j + i * G;
                v[i] = ld4_mp(bb <= bmax ? Rrow + slot_mp(rr - bb, RMASK) : nblk);
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float x[BP * M];
#pragma unroll
                for (int i = 0; i < BPL; ++i)
#pragma unroll
                    for (int d = 0; d < M; ++d) x[i * M + d] = at4_mp(v[i], d) + Dc[i][m - d + 3];
                const float mx = group_reduce<G>(max_tree<BPL * M>(x), OpMax());
                int kk = INT_MAX;                           // candidates by decreasing k
#pragma unroll
                for (int i = BPL - 1; i >= 0; --i)
#pragma unroll
                    for (int d = 0; d < M; ++d)
                        if (x[i * M + d] == mx) kk = M * (2 + j + i * G) + m - d;
                Q[m] = mx;
                kq[m] = group_min_int<G>(kk);
            }
        }
        const bool wr = bact && j == 0;
        float* slot = qsh + ((rr & 1) * CP + cb) * 2 * M;
        st4_mp(wr ? slot : sink, make_float4(Q[0], Q[1], Q[2], Q[3]));
        st4_mp(wr ? slot + M : sink, make_float4(__int_as_float(kq[0]), __int_as_float(kq[1]),
                                                 __int_as_float(kq[2]), __int_as_float(kq[3])));
    };

    // ---------------------------------------------------------------- start state
    auto slot_of = [&](int pos) { return (pos - t0 - 1) & RMASK; };
    // chain history, i < M: the previous round's positions (round start) - 3 + i; i >= M:
    // this round's (ring entries A - B_c)
    float Rh[2 * M];
#pragma unroll
    for (int i = 0; i < 2 * M; ++i) Rh[i] = NEG;
    double Bc = 0.0, H = 0.0;
    float Mref = 0.0f;
    if (t0 == 0) {
        // position 0: no transition into it; the ring entry is its start-side projection
        if (bact && j == 0) Rrow[slot_of(0)] = fmaxf(proj_s(0, cb), NEG);
        Rh[M - 1] = cact ? fmaxf(proj_s(0, cl), NEG) : 0.0f;
    } else if (spec) {
        // burn-in start: every ring entry of positions t0-K+1 .. t0 equal
        if (bact)
            for (int q = j; q < K && t0 - q >= 0; q += G) Rrow[slot_of(t0 - q)] = 0.0f;
#pragma unroll
        for (int i = 0; i < M; ++i) {
            const int q = M - 1 - i;
            Rh[i] = (q < K && t0 - q >= 0) ? 0.0f : NEG;
        }
    } else {
        const size_t ck = ckrow + span;
        if (bact)
            for (int q = j; q < K; q += G) Rrow[slot_of(t0 - q)] = a.ck_ring[(ck * K + q) * C + cb];
        if (chain) {
            Bc = a.ck_base[ck * C + cl];
            Mref = a.ck_mprev[ck * C + cl];
            H = a.ck_href[ck];
#pragma unroll
            for (int i = 0; i < M; ++i) {
                const int q = M - 1 - i;
                Rh[i] = (q < K && t0 - q >= 0) ? a.ck_ring[(ck * K + q) * C + cl] : NEG;
            }
        }
    }
    if (cact && t0 == 0) {
        // seam window positions <= 0: position 0's value, nothing before it
        const double a0 = Bc + (double)Rh[M - 1];
        for (int p = hlo; p <= min(0, tout); ++p) a.head[(winrow + p - hlo) * C + cl] = p == 0 ? a0 : -1.0e300;
        for (int p = tlo; p <= min(0, t1); ++p) a.tail[(winrow + p - tlo) * C + cl] = p == 0 ? a0 : -1.0e300;
    }

    const int chunkN = CH * C;
    auto sidx = [&](int t, int q) -> size_t { return (size_t)t * C + q; };
    double pf[PF];
    float pfe[PF], pfs[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        pf[i] = 0.0;
        pfe[i] = pfs[i] = 0.0f;
    }
    if (!chain) {
        for (int q = bt; q < chunkN; q += NB) {
            const int row = q / C, l = q - row * C;
            const int t = t0 + 1 + row;
            const bool in = t <= t1;
            Sbuf[l * CH + row] = in ? Sb[sidx(t, l)] : 0.0;
            if constexpr (PROJ) {
                Pst[l * CH + row] = in ? proj_e(t, l) : 0.0f;
                Pst[C * CH + l * CH + row] = in ? proj_s(t, l) : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int q = bt + i * NB;
            if (q < chunkN) {
                const int row = q / C, l = q - row * C;
                const int t = t0 + 1 + CH + row;
                if (t <= t1) {
                    pf[i] = Sb[sidx(t, l)];
                    pfe[i] = proj_e(t, l);
                    pfs[i] = proj_s(t, l);
                }
            }
        }
    }
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0);
    if (!chain) bulk_round(0);
    __syncthreads();

    // bulk lanes: the chain rebased in round r-1: move the blocks of rounds <= r-2 (reads
    // first)
    auto rescale = [&](int r) {
        if (r >= 3 && (r & 1) == 1) {
            constexpr int BR = BPL + 1;
            const float dl = bact ? dlsh[cb] : 0.0f;
            float4 v[BR];
#pragma unroll
            for (int i = 0; i < BR; ++i) v[i] = ld4_mp(Rrow + slot_mp(r - 2 - j - i * G, RMASK));
#pragma unroll
            for (int i = 0; i < BR; ++i) {
                const int q = j + i * G;
                const int rho = r - 2 - q;
                // blocks outside the live window go to the spare row (read by idle lanes)
                const bool live = (q < NR) & (t0 + M * rho + M >= 0);
                float4 rv = v[i];
                rv.x -= dl;
                rv.y -= dl;
                rv.z -= dl;
                rv.w -= dl;
                st4_mp((live ? Rrow : R + C * P) + slot_mp(rho, RMASK), rv);
            }
        }
    };

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
        const double* Sch = Sbuf + (nch & 1) * chunkN;
        const int row0 = rs + 1 - tc;
        if (chain) {
            const float* slot = qsh + ((r & 1) * CP + cl) * 2 * M;
            const float4 q4 = ld4_mp(slot), k4 = ld4_mp(slot + M);
            float Q[M] = {q4.x, q4.y, q4.z, q4.w};
            const int kQ[M] = {__float_as_int(k4.x), __float_as_int(k4.y), __float_as_int(k4.z),
                               __float_as_int(k4.w)};
            if (pend) {
#pragma unroll
                for (int m = 0; m < M; ++m) Q[m] -= pdl;
                pend = false;
            }
            if ((r & 1) == 0 && r > 0) {
                const float ref = fmaxf(Mref, Rh[M - 1]);
                const float dl = cact && ref > NEG_HALF ? ref : 0.0f;
                Bc += (double)dl;
                BH += (double)dl;
                Mref -= dl;
#pragma unroll
                for (int i = 0; i < M; ++i) Rh[i] -= dl;
#pragma unroll
                for (int m = 0; m < M; ++m) Q[m] -= dl;
                *(cact ? dlsh + cl : sink + (tid & 7)) = dl;
                pdl = dl;
                pend = true;
            }
            const double H0 = H;
            float hbs[M], hbx[M];
            {
                const double2* sp = reinterpret_cast<const double2*>(Sch + cl * CH + row0);
                const double2 s01 = sp[0], s23 = sp[1];
                const double sv4[M] = {s01.x, s01.y, s23.x, s23.y};
                if constexpr (PROJ) {
                    const float* pp = Pst + (size_t)(nch & 1) * 2 * C * CH + cl * CH + row0;
                    const float4 pe4 = ld4_mp(pp), ps4 = ld4_mp(pp + C * CH);
                    const float pe[M] = {pe4.x, pe4.y, pe4.z, pe4.w};
                    const float ps[M] = {ps4.x, ps4.y, ps4.z, ps4.w};
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const double hm = sv4[m] + BH;       // S(p_m) + B_c - H0
                        hbs[m] = (float)(hm - (double)ps[m]); // start side
                        hbx[m] = cact ? (float)(hm + (double)pe[m]) : NEG;   // end side
                    }
                } else {
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        hbs[m] = (float)(sv4[m] + BH);       // S(p_m) + B_c - H0, both sides
                        hbx[m] = cact ? hbs[m] : NEG;
                    }
                }
            }
            // the round's last step inside the sweep sets the normaliser
            const int ml = min(M - 1, t1 - rs - 1);
            float me = NEG;
            float uu[M];
            uint32_t* bpp = a.bp + (outrow + rs + 1) * C + cl;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int p = rs + 1 + m;
                // best segment of label cl ending at p: durations 1 .. m+4 (entries past
                // them NEG), then the bulk
                float x[2 * M + 1];
#pragma unroll
                for (int k = 1; k <= 2 * M; ++k) x[k - 1] = k <= m + M ? Rh[M + m - k] + dlog[k - 1] : NEG;
                x[2 * M] = Q[m];
                const float best = max_tree<2 * M + 1>(x);
                // lowest duration attaining it: each direct one gives its k or a sentinel,
                // a min tree picks; the bulk's otherwise
                int kd[2 * M];
#pragma unroll
                for (int k = 1; k <= 2 * M; ++k) kd[k - 1] = (k <= m + M && x[k - 1] == best) ? k : INT_MAX;
                const int kmin = min_tree_i<2 * M>(kd);
                const int kbest = kmin != INT_MAX ? kmin : kQ[m];
                const float u = hbx[m] + best;                 // V(p, cl) - H0
                // transition step of p over every label's value, lowest c' on ties
                float uv[CP], y[CP];
                row_bcast_all_mp<CP>(u, uv);
#pragma unroll
                for (int i = 0; i < CP; ++i) y[i] = uv[i] + treg[i];
                const float mt = max_tree<CP>(y);
                int ci[CP];
#pragma unroll
                for (int i = 0; i < CP; ++i) ci[i] = y[i] == mt ? i : INT_MAX;
                const int cbest = min_tree_i<CP>(ci);
                Rh[M + m] = mt - hbs[m];
                if (p <= t1 && p > tout && cact)   // the label of position L + 1 is never read
                    bpp[m * C] = (uint32_t)kbest | ((uint32_t)cbest << 16);
                uu[m] = u;
                if (m == ml) {
                    float uw[CP];
                    row_bcast_all_mp<CP>(u, uw);
                    me = max_tree<CP>(uw);
                }
            }
            if (rs + M >= min(hlo, tlo) || rs + M >= L) {
                // seam windows (ring values, natural log, this sweep's frame) and the final
                // values V(L, c)
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const int p = rs + 1 + m;
                    if (cact && p <= t1) {
                        const double av = Bc + (double)Rh[M + m];
                        if (p >= hlo && p <= tout) a.head[(winrow + p - hlo) * C + cl] = av;
                        if (p >= tlo) a.tail[(winrow + p - tlo) * C + cl] = av;
                        if (p == L) a.vfin[(size_t)b * C + cl] = H0 + (double)uu[m];
                    }
                }
            }
            H = H0 + (me > NEG_HALF ? (double)floorf(me) : 0.0);
            BH = Bc - H;
            st4_mp(R + (cact ? cl : C) * P + slot_mp(r, RMASK),
                   make_float4(Rh[M], Rh[M + 1], Rh[M + 2], Rh[M + 3]));
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (rs + 1 + m <= t1 && Q[m] > NEG_HALF) Mref = Q[m];
            if (ckpt && rs < t1 && rs + M >= t1) {
                // checkpoint at the span's end (its ring is copied after the loop)
                const size_t ck = ckrow + t1 / a.delta;
                if (cact) {
                    a.ck_base[ck * C + cl] = Bc;
                    a.ck_mprev[ck * C + cl] = Mref;
                }
                if (tid == 0) a.ck_href[ck] = H0;
            }
#pragma unroll
            for (int i = 0; i < M; ++i) Rh[i] = Rh[i + M];
        } else {
            if (rs + 1 == tc && tc + CH <= t1) {
                double* dst = Sbuf + ((nch + 1) & 1) * chunkN;
                float* dp = Pst + (size_t)((nch + 1) & 1) * 2 * C * CH;
#pragma unroll
                for (int i = 0; i < PF; ++i) {
                    const int q = bt + i * NB;
                    if (q < chunkN) {
                        const int row = q / C, l = q - row * C;
                        dst[l * CH + row] = pf[i];
                        if constexpr (PROJ) {
                            dp[l * CH + row] = pfe[i];
                            dp[C * CH + l * CH + row] = pfs[i];
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < PF; ++i) {
                    const int q = bt + i * NB;
                    if (q < chunkN) {
                        const int rr = q / C, l = q - rr * C;
                        const int tt = tc + 2 * CH + rr;
                        const bool in = tt <= t1;
                        pf[i] = in ? Sb[sidx(tt, l)] : 0.0;
                        pfe[i] = in ? proj_e(tt, l) : 0.0f;
                        pfs[i] = in ? proj_s(tt, l) : 0.0f;
                    }
                }
            }
            rescale(r);
            bulk_round(r + 1);
        }
        __syncthreads();
    }
    if (ckpt) {
        // the ring at the span's end, once the last rebase has reached it
        if (!chain) rescale(nrounds);
        __syncthreads();
        if (bact) {
            const size_t ck = ckrow + t1 / a.delta;
            for (int qq = j; qq < K; qq += G) a.ck_ring[(ck * K + qq) * C + cb] = Rrow[slot_of(t1 - qq)];
        }
    }
}

// ------------------------------------------------------------------ launch
template <int G, int BPL, int CP, bool PROJ>
static hipError_t launch_maxplus_round_inst(const SweepLaunch& a, const SweepCfg& cfg,
                                            hipStream_t stream) {
    if (cfg.NT > 512 || cfg.NT < 64 + cfg.G * a.C || cfg.vit.CH > lse_chunk_max(G) || cfg.vit.CH % ROUND != 0 ||
        cfg.vit.P % 4 != 0 || cfg.RS % ROUND != 0)
        return hipErrorInvalidValue;
    const size_t bytes = maxplus_round_lds_bytes(a.C, CP, cfg.vit.P, cfg.vit.CH, PROJ);
    if (a.mode != MODE_SPEC && a.mode != MODE_REPAIR) return hipErrorInvalidValue;
    const dim3 grid = a.mode == MODE_SPEC ? dim3(a.nspans, a.B) : dim3(a.B);
    hipLaunchKernelGGL((k_maxplus_round<G, BPL, CP, PROJ>), grid, dim3(cfg.NT), bytes,
                       stream, static_cast<const SweepArgs&>(a), cfg.RS, cfg.vit.P, cfg.vit.CH,
                       a.proj_start, a.proj_end);
    return hipGetLastError();
}

#define MAXPLUS_ROUND_BPL_CASES(G, CP)                                         \
    switch (cfg.BPL) {                                                         \
        case 0: return launch_maxplus_round_inst<G, 0, CP, PROJ>(a, cfg, stream);       \
        case 1: return launch_maxplus_round_inst<G, 1, CP, PROJ>(a, cfg, stream);       \
        case 2: return launch_maxplus_round_inst<G, 2, CP, PROJ>(a, cfg, stream);       \
        case 3: return launch_maxplus_round_inst<G, 3, CP, PROJ>(a, cfg, stream);       \
        case 4: return launch_maxplus_round_inst<G, 4, CP, PROJ>(a, cfg, stream);       \
        case 5: return launch_maxplus_round_inst<G, 5, CP, PROJ>(a, cfg, stream);       \
        case 6: return launch_maxplus_round_inst<G, 6, CP, PROJ>(a, cfg, stream);       \
        case 7: return launch_maxplus_round_inst<G, 7, CP, PROJ>(a, cfg, stream);       \
        case 8: return launch_maxplus_round_inst<G, 8, CP, PROJ>(a, cfg, stream);       \
        default: return hipErrorInvalidValue;                                  \
    }

template <bool PROJ>
hipError_t launch_maxplus_round(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream) {
    if (cfg.G == 64 && cfg.CPr == 4) { MAXPLUS_ROUND_BPL_CASES(64, 4) }
    if (cfg.G == 64 && cfg.CPr == 6) { MAXPLUS_ROUND_BPL_CASES(64, 6) }
    if (cfg.G == 64 && cfg.CPr == 8) { MAXPLUS_ROUND_BPL_CASES(64, 8) }
    if (cfg.G == 32 && cfg.CPr == 6) { MAXPLUS_ROUND_BPL_CASES(32, 6) }
    if (cfg.G == 32 && cfg.CPr == 8) { MAXPLUS_ROUND_BPL_CASES(32, 8) }
    if (cfg.G == 16 && cfg.CPr == 12) { MAXPLUS_ROUND_BPL_CASES(16, 12) }
    if (cfg.G == 16 && cfg.CPr == 16) { MAXPLUS_ROUND_BPL_CASES(16, 16) }
    return hipErrorInvalidValue;
}

#undef MAXPLUS_ROUND_BPL_CASES

}  // namespace semicrf
