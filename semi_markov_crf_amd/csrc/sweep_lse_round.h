// Log-semiring streaming sweep for small label counts (C <= 16), ROUND = 4 positions per
// workgroup barrier.
//
// Same recurrence, base-2 linear-space arithmetic and checkpoints as k_lse
// (sweep_lse_kernel.h); the work is divided between wavefronts by role.
//
// Ring layout: the positions of round rho (rounds counted from the sweep start t0; round
// -1 ends at t0) fill one 16-byte block of a label's ring row, so every ring access of
// the hot loop is a float4.
//
//  * chain wavefront (threads 0..63): lane c holds label c.  The message of position
//    p = (round start) + 1 + m takes durations k = 1 .. m + 4 from registers (the
//    previous round's block and this round's entries) and the older ones from the bulk
//    sum; then the transition step of p: DPP row broadcasts of every label's message and
//    FMA trees.  The normaliser moves once per round.  Range checks of the linear sums
//    are combined; if any failed, the round is replayed exactly in log space.  At the end
//    of a round the chain writes its block of linear ring entries and, for the log ring,
//    each entry as a (linear value, log2 offset) pair to a staging area.
//  * bulk wavefronts (threads 64..): lanes grouped G per label.  In round r they turn the
//    staged entries of round r-1 into the log ring, apply the chain's rebase of round r-1
//    to the rings, copy checkpoint rings, and compute the bulk sums of round r+1
//    (durations k >= m + 5, i.e. ring blocks of rounds <= r-1): lane j takes blocks
//    b = 2 + j + i*G rounds back, 16 FMAs per block with per-lane coefficients.  They
//    also stage S, label-major.
// Per-label bases move at the start of every second round; the chain corrects the bulk
// sums that the bulk wavefronts formed from the ring before they rescaled it.
// Boundary projections (PROJ) split S into an end side S(p) + pe(p), which scales the
// messages of segments ending at p, and a start side S(p) - ps(p), which scales the ring
// entries of segments starting at p; the staged per-position factors carry both.
#pragma once

#include "sweep_lse_kernel.h"

namespace semicrf {

// out[i] = v of lane i of this lane's 16-lane row, i < N (DPP row_newbcast, gfx90a+; every
// lane has a source, so the bound control only lets the move fold into its consumer)
template <int N, int I = 0>
__device__ __forceinline__ void row_bcast_all(float v, float* out) {
    if constexpr (I < N) {
        out[I] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                       0x150 + I, 0xF, 0xF, true));
        row_bcast_all<N, I + 1>(v, out);
    }
}

// Sums of four values over an aligned group of G >= 16 lanes, transposed: lane j ends with
// the group sum of acc[sum_step(j)].  Two exchange steps leave one value per lane, then
// the lanes of equal j & 3 are added (row rotations, then the swaps across rows).
__device__ __forceinline__ int sum_step(int j) { return 2 * (j & 1) + ((j >> 1) & 1); }
template <int G>
__device__ __forceinline__ float group_sum4(const float* acc, int j) {
    static_assert(G >= 16 && G <= 64, "group size");
    const bool o1 = j & 1, o2 = j & 2;
    const float s0 = o1 ? acc[0] : acc[2], s1 = o1 ? acc[1] : acc[3];
    const float k0 = o1 ? acc[2] : acc[0], k1 = o1 ? acc[3] : acc[1];
    const float n0 = k0 + dpp_f<DPP_QUAD_1032>(s0), n1 = k1 + dpp_f<DPP_QUAD_1032>(s1);
    float v = (o2 ? n1 : n0) + dpp_f<DPP_QUAD_2301>(o2 ? n0 : n1);
    v += dpp_f<0x128>(v);                                  // row_ror:8
    v += dpp_f<0x124>(v);                                  // row_ror:4
    if constexpr (G >= 32) {
        const int iv = __builtin_bit_cast(int, v);
        auto p = __builtin_amdgcn_permlane16_swap(iv, iv, false, false);
        v = __builtin_bit_cast(float, (int)p[0]) + __builtin_bit_cast(float, (int)p[1]);
    }
    if constexpr (G >= 64) {
        const int iv = __builtin_bit_cast(int, v);
        auto p = __builtin_amdgcn_permlane32_swap(iv, iv, false, false);
        v = __builtin_bit_cast(float, (int)p[0]) + __builtin_bit_cast(float, (int)p[1]);
    }
    return v;
}

// 0 if every value is in [2^-60, 2^60] (positive, finite), else 1
template <int N>
__device__ __forceinline__ bool any_out_of_lin_range(const float* x) {
    uint32_t lo = __float_as_uint(x[0]), hi = lo;
#pragma unroll
    for (int i = 1; i < N; ++i) {
        lo = min(lo, __float_as_uint(x[i]));
        hi = max(hi, __float_as_uint(x[i]));
    }
    return (lo < 0x21800000u) | (hi > 0x5d800000u);       // 2^-60, 2^60 (sign bit: huge)
}

// first ring slot of round rho's block
__device__ __forceinline__ int round_slot(int rho, int RMASK) { return (rho * ROUND) & RMASK; }

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ float at4(const float4& v, int d) {
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// G: bulk lanes per label (C <= 256/G); BPL: ring blocks per bulk lane; CP: labels the
// chain broadcasts (>= C); LIN: linear ring and sums (else log-space bulk sums only);
// PROJ: boundary projections present (else the end and start sides coincide); XA: write
// the per-position outputs X; ND: directions per workgroup.  With ND = 2 (MODE_SPEC of both
// directions) the forward and the backward sweep of the same span share a workgroup: their
// positions, rounds and chunks coincide, so every branch stays wave-uniform; chain lane
// 16 d + c holds label c of direction d (one DPP row per direction), the bulk wavefronts
// of direction d follow those of direction d - 1, and each direction has its own LDS
// region.  Block: 64 + ND * ceil(C*G/64)*64 threads.
template <int G, int BPL, int CP, bool LIN, bool PROJ, bool XA, int ND>
__global__ __launch_bounds__(512) void k_lse_round(const SweepArgs a, const int RS,
                                                                   const int P, const int CH,
                                                                   const float* __restrict__ proj_start,
                                                                   const float* __restrict__ proj_end) {
    constexpr int M = ROUND;
    static_assert(M == 4, "ring blocks are float4");
    static_assert(CP <= 16, "the labels of the chain wavefront share one DPP row");
    static_assert(CP * G <= 512, "at most 7 bulk wavefronts beside the chain");
    static_assert(ND == 1 || ND == 2, "one or both directions");   // <= 512 threads either way
    constexpr int BP = BPL > 0 ? BPL : 1;
    constexpr int KD = 2 * M - 1;                              // chain durations, last step
    constexpr int CP4 = (CP + 3) / 4 * 4;
    extern __shared__ double lds[];
    const int C = a.C, K = a.K, T = a.T;
    const int tid = threadIdx.x, NT = blockDim.x;
    // the role is a property of the wavefront: a wave-uniform value, scalar branches
    const bool chain = __builtin_amdgcn_readfirstlane(tid >> 6) == 0;
    const int NTV = (NT - 64) / ND;                // bulk threads of a direction (waves)
    const int bdir = chain ? 0 : (tid - 64) / NTV;   // wave-uniform
    const int bt = chain ? 0 : tid - 64 - bdir * NTV;
    const int cb = chain ? C : bt / G;
    const int j = chain ? 0 : bt - cb * G;
    const bool bact = !chain && cb < C;
    const int cr = bact ? cb : C;                 // inactive lanes use the spare ring row C
    const int crow = chain ? (tid >> 4) : 0;      // chain lanes: DPP row = direction
    const bool crow_ok = chain && crow < ND;
    const bool cact = crow_ok && (tid & 15) < C;
    const int cl = cact ? (tid & 15) : 0;
    // the lane that writes a direction's scalars (checkpoint reference, replay flag, log Z)
    const bool clead = crow_ok && (tid & 15) == 0;
    // CP < 16: chain lane 15 of a row is no label; with unit transition weights from every
    // label its transition sum is the message total q of the step
    constexpr bool QLANE = CP < 16;
    const bool qlane = QLANE && crow_ok && (tid & 15) == 15;

    // MODE_SPEC: grid (nspans, B, ndir); MODE_REPAIR: grid (B, ndir)
    const bool spec = a.mode == MODE_SPEC;
    int b, span, dir;
    if (spec) {
        span = blockIdx.x; b = blockIdx.y;
        dir = ND == 1 ? (int)blockIdx.z : (chain ? min(crow, ND - 1) : bdir);
    } else {
        b = blockIdx.x; dir = blockIdx.y; span = 0;
    }
    const int Lr = a.Leff[b];
    const bool bad = Lr < 0;
    const int L = bad ? -Lr : Lr;
    // [tout, t1]: the positions this workgroup writes; t0: where its sweep starts (a
    // speculative span runs a burn-in from t0 = tout - warm, or exactly from 0)
    int t0 = 0, t1 = L, tout = 0;
    if (spec) {
        tout = span * a.delta;
        if (tout >= L) return;
        t1 = min(L, tout + a.delta);
        t0 = max(0, tout - a.warm);
    } else {
        span = a.first_bad[dir * a.B + b];
        if (span >= a.nspans) return;
        tout = span * a.delta;
        if (tout >= L) return;
        t0 = tout;
    }
    const int RMASK = RS - 1;
    // checkpoint at the end of a speculative span (the start of a repair)
    const bool ckpt = spec && t1 < L;
    // ring values of the windows the seam check compares (MODE_SPEC): head [hlo, tout] of
    // every span but the first, tail [tlo, t1] of every span but the last
    const int hlo = (spec && span > 0) ? tout - K + 1 : INT_MAX;
    const int tlo = (spec && t1 < L) ? t1 - K + 1 : INT_MAX;
    const size_t winrow = (((size_t)dir * a.B + b) * a.nspans + span) * K;
    const int bmax = (K + M - 1) / M;             // oldest block a bulk sum reaches
    const int NR = bmax + 3;                      // live blocks behind a round (rescale)

    // this lane's direction's LDS region (ND = 2: two regions of equal layout; ND = 1: the
    // only one, whichever direction the workgroup sweeps)
    const size_t region = lse_round_region_bytes(C, CP, P, CH, LIN, PROJ);
    const int rdir = ND == 1 ? 0 : dir;
    double* Sbuf = reinterpret_cast<double*>(reinterpret_cast<char*>(lds) + rdir * region);   // [2][C][CH] label-major
    double* SL = Sbuf + 2 * C * CH;                        // [C] (padded to 16 bytes)
    // per position p of a staged chunk, relative to S(p0), p0 the first position of its
    // round: ge = S(p) + pe(p) - S(p0) and gs = S(p) - ps(p) - S(p0), with pe / ps the
    // end-side / start-side projections (base 2): 2^ge, 2^-gs, ge, gs, pe  [2][5][C][CH];
    // without projections ge = gs = g: 2^g, 2^-g, g  [2][3][C][CH]
    constexpr int NPL = PROJ ? 5 : 3;
    float* Fst = (float*)(SL + (C + 1) / 2 * 2);
    float* R = Fst + 2 * NPL * C * CH;                     // [C+1][P] log ring
    float* E = R + (C + 1) * P;                            // [C+1][P] linear ring
    float* qsh = E + (LIN ? (C + 1) * P : 0);              // [2 rounds][CP][lin, log][M]
    float* nsh = qsh + 2 * CP * 2 * M;                     // [2 rounds][CP+1][s, offset][M]
    float* dlsh = nsh + 2 * (CP + 1) * 2 * M;              // [CP4] rebase shift per label
    float* dmsh = dlsh + CP4;                              // [CP4] dmax per label
    float* sink = dmsh + CP4;                              // [8] for non-writing lanes
    float* zblk = sink + 8;                                // [4] zeros: linear blocks past K
    float* nblk = zblk + 4;                                // [4] NEG: log blocks past K
    // per-position outputs of round r, written by the bulk lanes in round r+1: the message
    // sums (linear, or log2 when the round was replayed), the replay flag, the base B_c
    float* sgsh = nblk + 4;                                // [2 rounds][CP][M]
    int* rpsh = (int*)(sgsh + 2 * CP * M);                 // [2 rounds] (padded to 4)
    double* bcsh = (double*)(rpsh + 4);                    // [2 rounds][CP]
    float* Rrow = R + cr * P;
    float* Erow = E + cr * P;
    // a pointer of this lane's region moved to region d (initialisation covers both)
    auto in_region = [&](auto* ptr, int d) {
        return reinterpret_cast<decltype(ptr)>(reinterpret_cast<char*>(ptr) +
                                               (ptrdiff_t)(d - rdir) * (ptrdiff_t)region);
    };

    const double* Sb = a.S + (size_t)b * (T + 1) * C;
    for (int d = 0; d < ND; ++d)
        for (int q = tid; q < C; q += NT) in_region(SL, d)[q] = Sb[(size_t)L * C + q];
    // projections of sweep position p, base 2: end side (segments ending at p) and start
    // side (segments starting at p); 0 without projections or outside [1, L] / [0, L-1]
    const float* PSb = proj_start ? proj_start + (size_t)b * T * C : nullptr;
    const float* PEb = proj_end ? proj_end + (size_t)b * T * C : nullptr;
    // (the raw natural-log values, then their base-2 form: staging loads the raw values a
    // chunk ahead and converts them when it stores, so its loads are in flight together)
    auto proj_e_raw = [&](int p, int q) -> float {
        if constexpr (!PROJ) return 0.0f;
        const float* src = dir == 0 ? PEb : PSb;
        const int t = dir == 0 ? p - 1 : L - p;
        return (src && p >= 1 && p <= L) ? src[(size_t)t * C + q] : 0.0f;
    };
    auto proj_s_raw = [&](int p, int q) -> float {
        if constexpr (!PROJ) return 0.0f;
        const float* src = dir == 0 ? PSb : PEb;
        const int t = dir == 0 ? p : L - 1 - p;
        return (src && p >= 0 && p < L) ? src[(size_t)t * C + q] : 0.0f;
    };
    auto base2 = [](float raw) -> float { return (float)((double)raw * LOG2E); };
    auto proj_s = [&](int p, int q) -> float { return base2(proj_s_raw(p, q)); };
    for (int d = 0; d < ND; ++d) {
        for (int q = tid; q < (C + 1) * P; q += NT) {
            in_region(R, d)[q] = NEG;
            if constexpr (LIN) in_region(E, d)[q] = 0.0f;
        }
        for (int q = tid; q < 2 * CP * 2 * M; q += NT) in_region(qsh, d)[q] = ((q / M) & 1) ? NEG : 0.0f;
        if (tid < M) {
            in_region(zblk, d)[tid] = 0.0f;
            in_region(nblk, d)[tid] = NEG;
        }
    }

    // ---------------------------------------------------------------- constants, base 2
    auto durv = [&](int c, int k) -> float {
        return (k >= 1 && k <= K) ? fmaxf((float)((double)a.dur[(k - 1) * C + c] * LOG2E), NEG) : NEG;
    };
    // bulk lanes: block i of lane j lies bb = 2 + j + i*G rounds back; its entry d enters
    // the sum of step m with duration k = 4*bb + m - d = 4*bb + t - 3, t = m - d + 3
    float dmx = NEG;
    if (bact) {
        for (int k = 1; k <= KD; ++k) dmx = fmaxf(dmx, durv(cb, k));
#pragma unroll
        for (int i = 0; i < BPL; ++i)
#pragma unroll
            for (int t = 0; t < 2 * M - 1; ++t) dmx = fmaxf(dmx, durv(cb, M * (2 + j + i * G) + t - 3));
    }
    if (!chain) dmx = group_reduce<G>(dmx, OpMax());
    const float dmax_b = dmx > NEG_HALF ? dmx : 0.0f;
    float Dc[BP][2 * M - 1];                               // 2^(dur - dmax), 0 beyond K
#pragma unroll
    for (int i = 0; i < BPL; ++i)
#pragma unroll
        for (int t = 0; t < 2 * M - 1; ++t)
            Dc[i][t] = bact ? exp2_or_zero(durv(cb, M * (2 + j + i * G) + t - 3) - dmax_b) : 0.0f;
    if (bact && j == 0) dmsh[cb] = dmax_b;
    // chain lanes: durations k = 1 .. KD and the transitions into label cl
    float dlog[KD];
#pragma unroll
    for (int k = 0; k < KD; ++k) dlog[k] = cact ? durv(cl, k + 1) : NEG;
    float treg[CP], wreg[CP], zero[CP];
#pragma unroll
    for (int i = 0; i < CP; ++i) {
        float v = NEG;
        if (cact && i < C) {
            const float tv = dir == 0 ? a.trans[i * C + cl] : a.trans[cl * C + i];
            v = fmaxf((float)((double)tv * LOG2E), NEG);
        } else if (qlane && i < C) {
            v = 0.0f;
        }
        treg[i] = v;
        zero[i] = 0.0f;
    }
    // linear transitions 2^(trans - tmax) with one tmax over the whole matrix: both sweep
    // directions then multiply by bit-identical weights (a per-label tmax would round the
    // weights of the two directions differently, a bias that builds up over the sequence);
    // the q lane's unit weights keep tmax = 0
    float tmx = qlane ? 0.0f : NEG;
    if (cact)
        for (int q = 0; q < C * C; ++q) tmx = fmaxf(tmx, fmaxf((float)((double)a.trans[q] * LOG2E), NEG));
    const float tmax = tmx > NEG_HALF ? tmx : 0.0f;
#pragma unroll
    for (int i = 0; i < CP; ++i) wreg[i] = exp2_or_zero(treg[i] - tmax);
    __syncthreads();   // ring cleared, SL and dmax visible

    const float dmax = chain ? dmsh[cl] : dmax_b;
    float Dl[KD];                                          // 2^(dur - dmax), k = 1 .. KD
#pragma unroll
    for (int k = 0; k < KD; ++k) Dl[k] = exp2_or_zero(dlog[k] - dmax);

    // bulk sums of round rr (positions p0 .. p0+M-1): ring blocks of rounds <= rr-2
    auto bulk_round = [&](int rr, int p0) {
        const int mj = sum_step(j);                        // the step this lane publishes
        float ql = 0.0f, qg = NEG;
        if constexpr (BPL > 0) {
            bool ok = LIN;
            if constexpr (LIN) {
                float4 v[BP];
#pragma unroll
                for (int i = 0; i < BPL; ++i) {
                    const int bb = 2 + j + i * G;
                    v[i] = ld4(bb <= bmax ? Erow + round_slot(rr - bb, RMASK) : zblk);
                }
                float acc[M];
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    acc[m] = 0.0f;
#pragma unroll
                    for (int i = 0; i < BPL; ++i)
#pragma unroll
                        for (int d = 0; d < M; ++d) acc[m] = fmaf(at4(v[i], d), Dc[i][m - d + 3], acc[m]);
                }
                ql = group_sum4<G>(acc, j);
                qg = fast_log2(ql) + dmax_b;
                ok = in_lin_range(ql) | !bact | (p0 + mj > t1);
            }
            if (wave_any(!ok)) {
                // exact log-space sums (durations from global memory: a rare path)
                float4 w[BP];
#pragma unroll
                for (int i = 0; i < BPL; ++i) {
                    const int bb = 2 + j + i * G;
                    w[i] = ld4(bb <= bmax ? Rrow + round_slot(rr - bb, RMASK) : nblk);
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float x[BP * M], dd[BP * M];
#pragma unroll
                    for (int i = 0; i < BPL; ++i)
#pragma unroll
                        for (int d = 0; d < M; ++d) {
                            x[i * M + d] = at4(w[i], d);
                            dd[i * M + d] = bact ? durv(cb, M * (2 + j + i * G) + m - d) : NEG;
                        }
                    const float lg = group_lse<G, BPL * M>(x, dd);
                    if (m == mj && (!LIN || !(in_lin_range(ql) || !bact))) {
                        qg = lg;
                        ql = exp2_or_zero(lg - dmax_b);
                    }
                }
            }
        }
        const bool wr = bact && j < M;
        float* slot = qsh + ((rr & 1) * CP + cb) * 2 * M + mj;
        *(wr ? slot : sink + (tid & 7)) = ql;
        *(wr ? slot + M : sink + (tid & 7)) = qg;
    };

    // ---------------------------------------------------------------- state after trans(t0)
    const size_t ckrow = ((size_t)dir * a.B + b) * a.nspans;
    const size_t outrow = (size_t)b * (T + 1);
    double* Xout = dir == 0 ? a.XF : a.XB;
    auto slot_of = [&](int pos) { return (pos - t0 - 1) & RMASK; };
    double Bc = 0.0, H = 0.0;
    float Mref = 0.0f;
    // chain history, i < M: the previous round's positions (round start) - 3 + i; i >= M:
    // this round's.  Eh: linear ring entry; its log2 is log2(sH) + fH.
    float Eh[2 * M], sH[2 * M], fH[2 * M];
#pragma unroll
    for (int i = 0; i < 2 * M; ++i) {
        Eh[i] = 0.0f;
        sH[i] = 1.0f;
        fH[i] = NEG;
    }
    if (t0 == 0) {
        // position 0: no transition into it; the ring entry is its start-side projection
        if (bact && j == 0) {
            const float r0 = fmaxf(proj_s(0, cb), NEG);
            Rrow[slot_of(0)] = r0;
            if constexpr (LIN) Erow[slot_of(0)] = exp2_or_zero(r0);
        }
        const float r0 = cact ? fmaxf(proj_s(0, cl), NEG) : 0.0f;
        Eh[M - 1] = exp2_or_zero(r0);
        fH[M - 1] = r0;
    } else if (spec) {
        // burn-in start: every ring entry of positions t0-K+1 .. t0 equal (0 in log2, 1
        // linear), a positive state from which the sweep converges to the exact one up to
        // a constant; bases and normaliser 0
        if (bact)
            for (int q = j; q < K && t0 - q >= 0; q += G) {
                Rrow[slot_of(t0 - q)] = 0.0f;
                if constexpr (LIN) Erow[slot_of(t0 - q)] = 1.0f;
            }
        if (chain) {
#pragma unroll
            for (int i = 0; i < M; ++i) {
                const int q = M - 1 - i;                   // position t0 - q
                const bool in = q < K && t0 - q >= 0;
                fH[i] = in ? 0.0f : NEG;
                Eh[i] = in ? 1.0f : 0.0f;
            }
        }
    } else {
        const size_t ck = ckrow + span;
        if (bact)
            for (int q = j; q < K; q += G) {
                const float rv = a.ck_ring[(ck * K + q) * C + cb];
                Rrow[slot_of(t0 - q)] = rv;
                if constexpr (LIN) Erow[slot_of(t0 - q)] = exp2_or_zero(rv);
            }
        if (chain) {
            Bc = a.ck_base[ck * C + cl];
            Mref = a.ck_mprev[ck * C + cl];
            H = a.ck_href[ck];
#pragma unroll
            for (int i = 0; i < M; ++i) {
                const int q = M - 1 - i;                   // position t0 - q
                const float rv = (q < K && t0 - q >= 0) ? a.ck_ring[(ck * K + q) * C + cl] : NEG;
                fH[i] = rv;
                Eh[i] = exp2_or_zero(rv);
            }
        }
    }
    if (cact) {
        const double a0 = (Bc + (double)fH[M - 1]) * LN2;   // ring value of position t0
        if (t0 == 0) {
            // window positions <= 0: position 0's value, nothing before it
            for (int p = hlo; p <= min(0, tout); ++p)
                a.head[(winrow + p - hlo) * C + cl] = p == 0 ? a0 : -1.0e300;
            for (int p = tlo; p <= min(0, t1); ++p)
                a.tail[(winrow + p - tlo) * C + cl] = p == 0 ? a0 : -1.0e300;
        }
    }

    // ---------------------------------------------------------------- S staging (bulk lanes)
    const int chunkN = CH * C;
    auto sidx = [&](int t, int q) -> size_t { return (size_t)(dir == 0 ? t : L - t) * C + q; };
    auto spub = [&](double raw, int q) -> double {
        return dir == 0 ? raw * LOG2E : (SL[q] - raw) * LOG2E;
    };
    // bulk lane bt stages label sl's rows of round sq of a chunk (C*CH/4 <= C*G pairs)
    const bool stg = !chain && bt < C * (CH / M);
    const int sq = stg ? bt / C : 0;
    const int sl = stg ? bt - sq * C : 0;
    double pf[M];                                          // raw S of the chunk after next
    float pfe[M], pfs[M];                                  // and its raw projections
    auto stage_load = [&](int tcs) {
#pragma unroll
        for (int d = 0; d < M; ++d) {
            const int t = tcs + M * sq + d;
            const bool in = stg && t <= t1;
            pf[d] = in ? Sb[sidx(t, sl)] : 0.0;
            pfe[d] = in ? proj_e_raw(t, sl) : 0.0f;
            pfs[d] = in ? proj_s_raw(t, sl) : 0.0f;
        }
    };
    auto stage_store = [&](int buf) {
        if (!stg) return;
        double sv[M];
#pragma unroll
        for (int d = 0; d < M; ++d) sv[d] = spub(pf[d], sl);
        double2* dS = reinterpret_cast<double2*>(Sbuf + buf * chunkN + sl * CH + M * sq);
        dS[0] = make_double2(sv[0], sv[1]);
        dS[1] = make_double2(sv[2], sv[3]);
        float* f = Fst + (size_t)buf * NPL * C * CH + sl * CH + M * sq;
        if constexpr (PROJ) {
            // the scale factors from the fp64 exponents (exp2_d), the fp32 exponents for the
            // log-space path
            float ge[M], gs[M], pe2[M], fe[M], fs[M];
#pragma unroll
            for (int d = 0; d < M; ++d) {
                const double g = sv[d] - sv[0];
                const double pe = (double)pfe[d] * LOG2E, ps = (double)pfs[d] * LOG2E;
                pe2[d] = (float)pe;
                ge[d] = (float)(g + pe);
                gs[d] = (float)(g - ps);
                fe[d] = exp2_d(g + pe);
                fs[d] = exp2_d(ps - g);
            }
            st4(f, make_float4(fe[0], fe[1], fe[2], fe[3]));
            st4(f + C * CH, make_float4(fs[0], fs[1], fs[2], fs[3]));
            st4(f + 2 * C * CH, make_float4(ge[0], ge[1], ge[2], ge[3]));
            st4(f + 3 * C * CH, make_float4(gs[0], gs[1], gs[2], gs[3]));
            st4(f + 4 * C * CH, make_float4(pe2[0], pe2[1], pe2[2], pe2[3]));
        } else {
            // one side: ge = gs = g
            // the scale factors from the fp64 differences (exp2_d)
            float g[M];
#pragma unroll
            for (int d = 0; d < M; ++d) g[d] = (float)(sv[d] - sv[0]);
            st4(f, make_float4(1.0f, exp2_d(sv[1] - sv[0]), exp2_d(sv[2] - sv[0]),
                               exp2_d(sv[3] - sv[0])));
            st4(f + C * CH, make_float4(1.0f, exp2_d(sv[0] - sv[1]), exp2_d(sv[0] - sv[2]),
                                        exp2_d(sv[0] - sv[3])));
            st4(f + 2 * C * CH, make_float4(0.0f, g[1], g[2], g[3]));
        }
    };
    if (!chain) {
        stage_load(t0 + 1);
        stage_store(0);
        stage_load(t0 + 1 + CH);
    }
    __syncthreads();   // restored ring and chunk 0 visible
    __builtin_amdgcn_s_waitcnt(0);

    // bulk sums of round 0 (ring blocks of rounds <= -2)
    if (!chain) bulk_round(0, t0 + 1);
    __syncthreads();

    // bulk lanes at the start of round r (rs = its first position - 1): the log ring block
    // of round r-1 from the chain's staging, the chain's rebase of round r-1 applied to the
    // rings, the rings of the checkpoints the chain took in round r-1
    int next_ckb = ckpt ? t1 : INT_MAX;        // next checkpoint whose ring is to copy
    // Sprev: the staged S of round r-1's first position for this lane's label; Fprev: its
    // end-side projection plane (projections only)
    auto ring_round = [&](int r, int rs, const double* Sprev, const float* Fprev) {
        if (r >= 1 && bact && j < M) {
            const float* ns = nsh + (((r - 1) & 1) * (CP + 1) + cb) * 2 * M + j;
            const float rl = fast_log2(ns[0]) + ns[M];
            Rrow[round_slot(r - 1, RMASK) + j] = fmaxf(rl, NEG);
            // per-position outputs of round r-1 (position p = rs - M + 1 + j), natural log:
            // X on (tout, t1], A on [tout, t1); ring values of the seam windows
            const int p = rs - M + 1 + j;
            if (XA && p <= t1) {
                const double Bp = bcsh[((r - 1) & 1) * CP + cb];
                const double av = (Bp + (double)rl) * LN2;
                const size_t o = (outrow + (dir == 0 ? p : L - p)) * C + cb;
                if (a.write_xa && p > tout) {
                    const float sg = sgsh[(((r - 1) & 1) * CP + cb) * M + j];
                    const float sgl = rpsh[(r - 1) & 1] ? sg : fast_log2(sg) + dmax_b;
                    double Sp = Sprev[j];
                    if constexpr (PROJ) Sp += (double)Fprev[j];
                    Xout[o] = (Sp + Bp + (double)sgl) * LN2;
                }
                if (p >= hlo && p <= tout) a.head[(winrow + p - hlo) * C + cb] = av;
                if (p >= tlo) a.tail[(winrow + p - tlo) * C + cb] = av;
            }
        }
        // the chain rebased last round: move the blocks of rounds <= r-2 (reads first).
        // Linear entries are scaled by 2^-dl: one that underflowed is below 2^-126 and
        // negligible next to any linear sum the range checks accept (>= 2^-60); sums
        // that fail them are redone from the log ring.
        if (r >= 3 && (r & 1) == 1) {
            constexpr int BR = BPL + 1;               // covers NR = bmax + 3 <= BPL*G + G blocks
            const float dl = bact ? dlsh[cb] : 0.0f;
            const float sc = pow2_neg(dl);
            if constexpr (BR <= 3) {
                float4 v[BR], e[BR];
#pragma unroll
                for (int i = 0; i < BR; ++i) {
                    v[i] = ld4(Rrow + round_slot(r - 2 - j - i * G, RMASK));
                    if constexpr (LIN) e[i] = ld4(Erow + round_slot(r - 2 - j - i * G, RMASK));
                }
#pragma unroll
                for (int i = 0; i < BR; ++i) {
                    const int q = j + i * G;
                    const int rho = r - 2 - q;
                    // blocks outside the live window go to the spare row (read by idle lanes)
                    const bool live = (q < NR) & (t0 + M * rho + M >= 0);
                    const int sl = round_slot(rho, RMASK);
                    float4 rv = v[i];
                    rv.x -= dl;
                    rv.y -= dl;
                    rv.z -= dl;
                    rv.w -= dl;
                    st4((live ? Rrow : R + C * P) + sl, rv);
                    if constexpr (LIN)
                        st4((live ? Erow : E + C * P) + sl,
                            make_float4(e[i].x * sc, e[i].y * sc, e[i].z * sc, e[i].w * sc));
                }
            } else {
                // more blocks: batches of three (register pressure); each live block belongs
                // to one (lane, i), so the batches need no ordering among lanes
                constexpr int RB = 3;
#pragma unroll
                for (int i0 = 0; i0 < BR; i0 += RB) {
                    float4 v[RB], e[RB];
#pragma unroll
                    for (int ii = 0; ii < RB && i0 + ii < BR; ++ii) {
                        v[ii] = ld4(Rrow + round_slot(r - 2 - j - (i0 + ii) * G, RMASK));
                        if constexpr (LIN) e[ii] = ld4(Erow + round_slot(r - 2 - j - (i0 + ii) * G, RMASK));
                    }
#pragma unroll
                    for (int ii = 0; ii < RB && i0 + ii < BR; ++ii) {
                        const int q = j + (i0 + ii) * G;
                        const int rho = r - 2 - q;
                        const bool live = (q < NR) & (t0 + M * rho + M >= 0);
                        const int sl = round_slot(rho, RMASK);
                        float4 rv = v[ii];
                        rv.x -= dl;
                        rv.y -= dl;
                        rv.z -= dl;
                        rv.w -= dl;
                        st4((live ? Rrow : R + C * P) + sl, rv);
                        if constexpr (LIN)
                            st4((live ? Erow : E + C * P) + sl,
                                make_float4(e[ii].x * sc, e[ii].y * sc, e[ii].z * sc, e[ii].w * sc));
                    }
                }
            }
        }
        // checkpoint rings of the positions the chain checkpointed last round
        for (; next_ckb <= rs; next_ckb += a.delta) {
            const int pc = next_ckb;
            if (bact && pc < L) {
                const size_t ck = ckrow + pc / a.delta;
                for (int qq = j; qq < K; qq += G)
                    a.ck_ring[(ck * K + qq) * C + cb] = Rrow[slot_of(pc - qq)];
            }
        }
    };

    // ---------------------------------------------------------------- main loop
    double BH = Bc - H;                                   // B_c - H
    double lz = 0.0;
    int next_ck = ckpt ? t1 : INT_MAX;
    float pdl = 0.0f;          // chain: rebase of the last round, still to apply to the
    bool pend = false;         // bulk sums it reads this round
    const int nrounds = (t1 - t0 + M - 1) / M;
    int tc = t0 + 1, nch = 0;  // first position and index of the staged S chunk
    for (int r = 0; r < nrounds; ++r) {
        const int rs = t0 + r * M;                     // round covers positions rs+1 .. rs+M
        if (rs + 1 >= tc + CH) {
            tc += CH;
            ++nch;
        }
        const double* Sch = Sbuf + (nch & 1) * chunkN;
        const int row0 = rs + 1 - tc;                  // chunk row of position rs+1
        if (chain) {
            const float* slot = qsh + ((r & 1) * CP + cl) * 2 * M;
            const float4 ql4 = ld4(slot), qg4 = ld4(slot + M);
            float QL[M] = {ql4.x, ql4.y, ql4.z, ql4.w};
            float QG[M] = {qg4.x, qg4.y, qg4.z, qg4.w};
            if (pend) {                                // summed before the ring was rebased
                const float sc = pow2_neg(pdl);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    QL[m] *= sc;
                    QG[m] -= pdl;
                }
                pend = false;
            }
            if ((r & 1) == 0 && r > 0) {
                // ---- rebase: this label's values move to a new base
                const float rn = fmaxf(fast_log2(sH[M - 1]) + fH[M - 1], NEG);
                const float ref = fmaxf(Mref, rn);
                // a whole number of octaves: the linear values scale exactly
                const float dl = cact && ref > NEG_HALF ? floorf(ref) : 0.0f;
                const float sc = pow2_neg(dl);
                Bc += (double)dl;
                BH += (double)dl;
                Mref -= dl;
#pragma unroll
                for (int i = 0; i < M; ++i) {
                    fH[i] -= dl;
                    Eh[i] *= sc;
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    QL[m] *= sc;
                    QG[m] -= dl;
                }
                *(cact ? dlsh + cl : sink + (tid & 7)) = dl;
                pdl = dl;
                pend = true;
            }
            // ---- per-round constants (H fixed inside the round)
            const double H0 = H;
            float hbe[M], hbs[M], yv[M], fb[M], fo[M];
            if constexpr (!PROJ) {
                // S(p_m) + B_c - H0 from S(p_0) and the staged differences; the scales
                // 2^(hb + dmax) and 2^(tmax - hb) from one exp2 each and staged factors
                const float* f = Fst + (size_t)(nch & 1) * NPL * C * CH + cl * CH + row0;
                const float4 sg4 = ld4(f), is4 = ld4(f + C * CH), g4 = ld4(f + 2 * C * CH);
                const double hb64 = Sch[cl * CH + row0] + BH;
                const float hb0 = (float)hb64;
                const float y0 = cact ? exp2_d(hb64 + (double)dmax) : 0.0f;
                const float fo0 = tmax - hb0;
                const float f0 = exp2_d((double)tmax - hb64);
                const float gs[M] = {g4.x, g4.y, g4.z, g4.w};
                const float ss[M] = {sg4.x, sg4.y, sg4.z, sg4.w};
                const float is[M] = {is4.x, is4.y, is4.z, is4.w};
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    hbe[m] = hb0 + gs[m];
                    hbs[m] = hbe[m];
                    yv[m] = y0 * ss[m];                      // message scale
                    fo[m] = fo0 - gs[m];
                    fb[m] = f0 * is[m];                      // ring-entry scale
                }
            } else {
                // end side S(p_m) + pe + B_c - H0 and start side S(p_m) - ps + B_c - H0
                // from S(p_0) and the staged differences; the scales 2^(hbe + dmax) and
                // 2^(tmax - hbs) from one exp2 each and staged factors
                const float* f = Fst + (size_t)(nch & 1) * NPL * C * CH + cl * CH + row0;
                const float4 fe4 = ld4(f), fs4 = ld4(f + C * CH), ge4 = ld4(f + 2 * C * CH);
                const float4 gs4 = ld4(f + 3 * C * CH);
                const double hb64 = Sch[cl * CH + row0] + BH;
                const float hb0 = (float)hb64;
                const float y0 = cact ? exp2_d(hb64 + (double)dmax) : 0.0f;
                const float fo0 = tmax - hb0;
                const float f0 = exp2_d((double)tmax - hb64);
                const float ge[M] = {ge4.x, ge4.y, ge4.z, ge4.w};
                const float gs[M] = {gs4.x, gs4.y, gs4.z, gs4.w};
                const float fe[M] = {fe4.x, fe4.y, fe4.z, fe4.w};
                const float fs[M] = {fs4.x, fs4.y, fs4.z, fs4.w};
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    hbe[m] = hb0 + ge[m];
                    hbs[m] = hb0 + gs[m];
                    yv[m] = y0 * fe[m];                      // message scale
                    fo[m] = fo0 - gs[m];
                    fb[m] = f0 * fs[m];                      // ring-entry scale
                }
            }
            // ---- fast pass (linear space, no branches)
            float chk[3 * M];          // values the linear pass relies on
            float sig[M];              // combined message sum (linear) or its log2 (replay)
            float qv[M];               // message total of each step (log2 in a replay)
#pragma unroll
            for (int m = 0; m < M; ++m) qv[m] = 0.0f;
            // terms k = 2 .. m+4 of step m are formed ahead of its transition step, so only
            // one FMA waits for the newest ring entry
            float part = QL[0];
#pragma unroll
            for (int k = M; k >= 2; --k) part = fmaf(Eh[M - k], Dl[k - 1], part);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float sg = fmaf(Eh[M - 1 + m], Dl[0], part);
                sig[m] = sg;
                const float pn = sg * yv[m];
                if (m + 1 < M) {
                    float nx = QL[m + 1];
#pragma unroll
                    for (int k = m + 1 + M; k >= 2; --k) nx = fmaf(Eh[M + m + 1 - k], Dl[k - 1], nx);
                    part = nx;
                }
                // transition step of p: row broadcasts of every label's message (labels sit
                // in lanes 0..CP-1, one DPP row) and FMA trees
                float sv[CP], qa[CP];
                row_bcast_all<CP>(pn, qa);
#pragma unroll
                for (int i = 0; i < CP; ++i) sv[i] = qa[i] * wreg[i];
#pragma unroll
                for (int w = 1; w < CP; w *= 2)
#pragma unroll
                    for (int i = 0; i + w < CP; i += 2 * w) {
                        sv[i] += sv[i + w];
                        if constexpr (!QLANE) qa[i] += qa[i + w];
                    }
                const float s = sv[0];
                chk[3 * m] = cact ? sg : 1.0f;   // the q lane's sg is not a message
                chk[3 * m + 1] = s;
                if constexpr (QLANE) {
                    chk[3 * m + 2] = s;
                } else {
                    chk[3 * m + 2] = qa[0];
                    qv[m] = qa[0];
                }
                Eh[M + m] = s * fb[m];
                sH[M + m] = s;
                fH[M + m] = fo[m];
            }
            // label lanes only (lanes outside row 0 broadcast their own, empty row); a
            // round past the sweep end may replay for nothing
            const uint64_t row_lanes = ((1ull << C) - 1) | (QLANE ? (1ull << 15) : 0ull);
            const uint64_t lanes = ND == 1 ? row_lanes : row_lanes | (row_lanes << 16);
            bool replayed = false;
            if (__builtin_amdgcn_ballot_w64(any_out_of_lin_range<3 * M>(chk)) & lanes) {
                // ---- exact replay of the round in log space
                replayed = true;
                float Rl[2 * M];
#pragma unroll
                for (int i = 0; i < M; ++i) Rl[i] = fmaxf(fast_log2(sH[i]) + fH[i], NEG);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    // durations 1 .. m+4 from the history, then the bulk sum; unused: NEG
                    float x[2 * M + 1], xd[2 * M + 1];
#pragma unroll
                    for (int k = 1; k <= 2 * M; ++k) {
                        x[k - 1] = k <= m + M ? Rl[M + m - k] : NEG;
                        xd[k - 1] = k <= m + M ? dlog[k - 1] : 0.0f;
                    }
                    x[2 * M] = QG[m];
                    xd[2 * M] = 0.0f;
                    const float sigma = group_lse<1, 2 * M + 1>(x, xd);
                    sig[m] = sigma;
                    const float u = cact ? hbe[m] + sigma : NEG;
                    float uv[CP];
                    row_bcast_all<CP>(u, uv);
                    const float rn = group_lse<1, CP>(uv, treg) - hbs[m];
                    const float lq = group_lse<1, CP>(uv, zero);
                    Rl[M + m] = rn;
                    Eh[M + m] = exp2_or_zero(rn);
                    sH[M + m] = 1.0f;
                    fH[M + m] = rn;
                    qv[m] = lq;
                }
            }
            if constexpr (QLANE) {
                if (!replayed) {   // message totals: the q lane's transition sums
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        qv[m] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                    0, __builtin_bit_cast(int, sH[M + m]), 0x15F, 0xF, 0xF, true));
                }
            }
            {
                // the normaliser follows the round's last step; log Z when the round holds L
                float qe = qv[M - 1];
                if (rs + M >= t1) {
                    const int mL = L - rs - 1, ml = t1 - rs - 1;
                    float ql = qv[0];
#pragma unroll
                    for (int m = 1; m < M; ++m) {
                        if (m == mL) ql = qv[m];
                        if (m == ml) qe = qv[m];
                    }
                    if (mL >= 0 && mL < M) lz = H0 + (double)(replayed ? ql : fast_log2(ql));
                }
                int e;
                if (replayed) e = qe > NEG_HALF ? (int)floorf(qe) + 1 : 0;
                else e = __builtin_amdgcn_frexp_expf(qe);
                H = H0 + (double)e;
                BH = Bc - H;
            }
            // ---- publish the round: ring block, staging for the log ring, outputs, checkpoints
            if constexpr (LIN)
                st4(E + (cact ? cl : C) * P + round_slot(r, RMASK),
                    make_float4(Eh[M], Eh[M + 1], Eh[M + 2], Eh[M + 3]));
            {
                float* ns = nsh + ((r & 1) * (CP + 1) + (cact ? cl : CP)) * 2 * M;
                st4(ns, make_float4(sH[M], sH[M + 1], sH[M + 2], sH[M + 3]));
                st4(ns + M, make_float4(fH[M], fH[M + 1], fH[M + 2], fH[M + 3]));
            }
            if constexpr (XA) {
                // per-position outputs: staged here, written by the bulk lanes next round
                if (cact) {
                    st4(sgsh + ((r & 1) * CP + cl) * M, make_float4(sig[0], sig[1], sig[2], sig[3]));
                    bcsh[(r & 1) * CP + cl] = Bc;
                }
                if (clead) rpsh[r & 1] = replayed ? 1 : 0;
            } else if (a.write_xa) {
                // never taken (the launch picks XA when writing outputs); kept because the
                // register allocation of this instance is the faster one with it
                const float* fpe = Fst + (size_t)(nch & 1) * NPL * C * CH + 4 * C * CH + cl * CH + row0;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const int p = rs + 1 + m;
                    if (p <= t1 && cact) {
                        double Sp = Sch[cl * CH + row0 + m];
                        if constexpr (PROJ) Sp += (double)fpe[m];
                        const float sgl = replayed ? sig[m] : fast_log2(sig[m]) + dmax;
                        Xout[(outrow + (dir == 0 ? p : L - p)) * C + cl] = (Sp + Bc + (double)sgl) * LN2;
                    }
                }
            }
            if (next_ck <= rs + M) {
                // chain half of a checkpoint after the transition step of p; the ring half
                // is copied by the bulk lanes next round
                float mr = Mref;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const int p = rs + 1 + m;
                    if (p <= t1 && QG[m] > NEG_HALF) mr = QG[m];
                    if (p == next_ck) {
                        if (p < L) {
                            const size_t ck = ckrow + p / a.delta;
                            if (cact) {
                                a.ck_base[ck * C + cl] = Bc;
                                a.ck_mprev[ck * C + cl] = mr;
                            }
                            if (clead) a.ck_href[ck] = H0;
                        }
                        next_ck += a.delta;
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const bool use = (rs + 1 + m <= t1) & (QG[m] > NEG_HALF);
                Mref = use ? QG[m] : Mref;
            }
#pragma unroll
            for (int i = 0; i < M; ++i) {   // history for the next round
                Eh[i] = Eh[i + M];
                sH[i] = sH[i + M];
                fH[i] = fH[i + M];
            }
        } else {
            // ---- S staging: in the first round of a chunk publish the next one; with the
            // outputs, in the second (the first still writes those of the previous chunk's
            // last round)
            if (rs + 1 == tc + (XA ? M : 0) && tc + CH <= t1) {
                stage_store((nch + 1) & 1);
                stage_load(tc + 2 * CH);
            }
            if constexpr (XA) {
                // chunk row of round r-1's first position: this chunk, or the last row block
                // of the previous one
                const bool prevc = rs + 1 - M < tc;
                const int buf = (prevc ? nch - 1 : nch) & 1;
                const int rowp = rs + 1 - M - (prevc ? tc - CH : tc);
                ring_round(r, rs, Sbuf + buf * chunkN + cb * CH + rowp,
                           Fst + (size_t)buf * NPL * C * CH + (NPL - 1) * C * CH + cb * CH + rowp);
            } else {
                ring_round(r, rs, nullptr, nullptr);
            }
            // ---- bulk sums of round r+1 (ring blocks of rounds <= r-1)
            bulk_round(r + 1, rs + M + 1);
        }
        __syncthreads();
    }

    // checkpoints taken in the last round: their rings are copied here
    // checkpoints taken and outputs staged in the last round
    if constexpr (XA) {
        if (!chain && nrounds > 0) {
            const int rs = t0 + nrounds * M;
            const int tcl = t0 + 1 + ((nrounds - 1) * M) / CH * CH;   // chunk of the last round
            const int nchl = ((nrounds - 1) * M) / CH;
            const int rowp = rs + 1 - M - tcl;
            ring_round(nrounds, rs, Sbuf + (nchl & 1) * chunkN + cb * CH + rowp,
                       Fst + (size_t)(nchl & 1) * NPL * C * CH + (NPL - 1) * C * CH + cb * CH + rowp);
        }
    } else {
        if (ckpt && !chain) ring_round(nrounds, t0 + nrounds * M, nullptr, nullptr);
    }

    // ---------------------------------------------------------------- end of sequence
    if (t1 == L && clead) {
        if (spec) {
            a.lzloc[dir * a.B + b] = lz * LN2;           // the seam check adds the offsets
        } else {
            // a repaired sweep continues in the frame of the span before the failed seam
            const double base = a.off[((size_t)dir * a.B + b) * a.nspans + span - 1];
            (dir == 0 ? a.logz : a.logz_b)[b] = bad ? nan_d() : lz * LN2 + base;
        }
    }
}

// ------------------------------------------------------------------ launch
template <int G, int BPL, int CP, bool LIN, bool PROJ, bool XA, int ND>
static hipError_t launch_lse_round_inst(const SweepLaunch& a, dim3 grid, const SweepCfg& cfg,
                                        hipStream_t stream) {
    const int nt = 64 + ND * cfg.NTv;
    if (cfg.NT > 512 || cfg.NT != 64 + cfg.NTv || cfg.NTv % 64 != 0 || cfg.NT < 64 + cfg.G * a.C ||
        cfg.lse.CH > lse_chunk_max(G) || cfg.lse.CH % ROUND != 0 || cfg.lse.CH < 2 * ROUND ||
        cfg.lse.P % 4 != 0 || cfg.RS % ROUND != 0)
        return hipErrorInvalidValue;
    const size_t bytes = ND * lse_round_region_bytes(a.C, CP, cfg.lse.P, cfg.lse.CH, LIN, PROJ);
    hipLaunchKernelGGL((k_lse_round<G, BPL, CP, LIN, PROJ, XA, ND>), grid, dim3(nt), bytes, stream,
                       static_cast<const SweepArgs&>(a), cfg.RS, cfg.lse.P, cfg.lse.CH,
                       a.proj_start, a.proj_end);
    return hipGetLastError();
}

#define LSE_ROUND_BPL_ND(G, CP, B_)                                                            \
    return nd == 2 ? launch_lse_round_inst<G, B_, CP, LIN, PROJ, true, 2>(a, grid, cfg, stream) \
                   : launch_lse_round_inst<G, B_, CP, LIN, PROJ, true, 1>(a, grid, cfg, stream);
#define LSE_ROUND_BPL_CASES(G, CP)                                                   \
    switch (cfg.BPL) {                                                               \
        case 0: LSE_ROUND_BPL_ND(G, CP, 0)                                           \
        case 1: LSE_ROUND_BPL_ND(G, CP, 1)                                           \
        case 2: LSE_ROUND_BPL_ND(G, CP, 2)                                           \
        case 3: LSE_ROUND_BPL_ND(G, CP, 3)                                           \
        case 4: LSE_ROUND_BPL_ND(G, CP, 4)                                           \
        case 5: LSE_ROUND_BPL_ND(G, CP, 5)                                           \
        case 6: LSE_ROUND_BPL_ND(G, CP, 6)                                           \
        case 7: LSE_ROUND_BPL_ND(G, CP, 7)                                           \
        case 8: LSE_ROUND_BPL_ND(G, CP, 8)                                           \
        default: return hipErrorInvalidValue;                                        \
    }

// every shape of the round kernel with (LIN) or without the linear ring, with (PROJ) or
// without boundary projections
template <bool LIN, bool PROJ>
hipError_t launch_lse_round_layout(const SweepCfg& cfg, const SweepLaunch& a, int ndir,
                                   hipStream_t stream) {
    if (a.mode != MODE_SPEC && a.mode != MODE_REPAIR) return hipErrorInvalidValue;
    // both directions of a span in one workgroup where they fit (MODE_SPEC only: a repair
    // of each direction starts at its own failed seam)
    const bool fits = 64 + 2 * cfg.NTv <= 512 &&
                      2 * lse_round_region_bytes(a.C, cfg.CPr, cfg.lse.P, cfg.lse.CH, LIN, PROJ) <=
                          150 * 1024;
    const int nd = (a.mode == MODE_SPEC && ndir == 2 && fits) ? 2 : 1;
    const dim3 grid = a.mode == MODE_REPAIR ? dim3(a.B, ndir) : dim3(a.nspans, a.B, ndir / nd);
    if (cfg.G == 64 && cfg.CPr == 4) { LSE_ROUND_BPL_CASES(64, 4) }
    if (cfg.G == 64 && cfg.CPr == 6) { LSE_ROUND_BPL_CASES(64, 6) }
    if (cfg.G == 64 && cfg.CPr == 8) { LSE_ROUND_BPL_CASES(64, 8) }
    if (cfg.G == 32 && cfg.CPr == 6) { LSE_ROUND_BPL_CASES(32, 6) }
    if (cfg.G == 32 && cfg.CPr == 8) { LSE_ROUND_BPL_CASES(32, 8) }
    if (cfg.G == 16 && cfg.CPr == 12) { LSE_ROUND_BPL_CASES(16, 12) }
    if (cfg.G == 16 && cfg.CPr == 16) { LSE_ROUND_BPL_CASES(16, 16) }
    return hipErrorInvalidValue;
}

#undef LSE_ROUND_BPL_CASES
#undef LSE_ROUND_BPL_ND

}  // namespace semicrf
