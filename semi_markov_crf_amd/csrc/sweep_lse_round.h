// Log-semiring streaming sweep for small label counts (C <= 16), ROUND positions per
// workgroup barrier.
//
// Same recurrence, base-2 linear-space arithmetic and checkpoints as k_lse
// (sweep_lse_kernel.h); the work is divided between wavefronts by role, and the chain of
// positions runs ROUND steps between two workgroup barriers.
//
//  * chain wavefront (threads 0..63): lane c holds label c.  Per position p it forms the
//    message of p from its label's last DIRECT = 2*ROUND-1 ring entries (registers) and
//    the bulk sum of the older ones, then the transition step of p: every lane reads the
//    other labels' messages with v_readlane and sums them with FMA trees.  Messages never
//    leave the wavefront.  The range checks of the linear sums of a round are combined;
//    if any failed, the round is replayed exactly in log space (the replay rewrites
//    everything the fast pass stored).
//  * bulk wavefronts (threads 64..): lanes grouped G per label.  They own the label rings
//    in LDS; in round r they apply the chain's rebase of round r-1 to the ring, insert
//    the chain's ring entries of round r-1, copy checkpoint rings, and compute the bulk
//    sums (durations k >= 2*ROUND) of the positions of round r+1 -- these only need
//    entries up to the end of round r-1.  They also stage S.
// Per-label bases move at the start of every second round; the chain corrects the bulk
// sums that the bulk wavefronts formed from the ring before they rescaled it.
#pragma once

#include "sweep_lse_kernel.h"

namespace semicrf {

// out[i] = v of lane i of this lane's 16-lane row, i < N (DPP row_newbcast, gfx90a+)
template <int N, int I = 0>
__device__ __forceinline__ void row_bcast_all(float v, float* out) {
    if constexpr (I < N) {
        out[I] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                       0x150 + I, 0xF, 0xF, false));
        row_bcast_all<N, I + 1>(v, out);
    }
}

// G: bulk lanes per label (C <= 256/G); KPL: durations per bulk lane
// (k = 2*ROUND + j + i*G); LAY: ring layout bits.  Block: 64 + ceil(C*G/64)*64 threads.
template <int G, int KPL, int LAY>
__global__ __launch_bounds__(320) void k_lse_round(const SweepArgs a, const int RS, const int P,
                                                  const int CH) {
    constexpr int M = ROUND;
    constexpr int CP = 256 / G;                                // chain lanes in use (>= C)
    static_assert(CP <= 16, "the labels of the chain wavefront share one DPP row");
    constexpr int PF = (lse_chunk_max(G) + 1 + G - 1) / G;     // prefetched doubles per bulk lane
    constexpr int KP = KPL > 0 ? KPL : 1;
    constexpr int HN = DIRECT + M;                             // history + this round
    constexpr bool MIR = LAY & SWEEP_MIRRORED;
    constexpr bool LIN = LAY & SWEEP_LINEAR;
    extern __shared__ double lds[];
    const int C = a.C, K = a.K, T = a.T;
    const int tid = threadIdx.x, NT = blockDim.x, NB = NT - 64;
    // the role is a property of the wavefront: a wave-uniform value, scalar branches
    const bool chain = __builtin_amdgcn_readfirstlane(tid >> 6) == 0;
    const int bt = tid - 64;
    const int cb = chain ? C : bt / G;
    const int j = chain ? 0 : bt - cb * G;
    const bool bact = !chain && cb < C;
    const int cr = bact ? cb : C;                 // inactive lanes use the spare ring row C
    const bool cact = chain && tid < C;
    const int cl = cact ? tid : 0;

    int b, span, dir;
    if (a.mode == MODE_FULL) {
        b = blockIdx.x; dir = blockIdx.y; span = 0;
    } else {
        span = blockIdx.x; b = blockIdx.y; dir = blockIdx.z;
    }
    const int Lr = a.Leff[b];
    const bool bad = Lr < 0;
    const int L = bad ? -Lr : Lr;
    int t0 = 0, t1 = L;
    if (a.mode == MODE_SPAN) {
        t0 = span * a.delta;
        if (t0 >= L) return;
        t1 = min(L, t0 + a.delta);
    }
    const int RMASK = RS - 1;
    const int rowsN = (CH + 1) * C;
    const bool ckpt = a.mode == MODE_FULL && a.write_ckpt;

    double* Sbuf = lds;                                    // [2][CH+1][C]
    double* SL = Sbuf + 2 * rowsN;                         // [C]
    float* R = (float*)(SL + C);                           // [C+1][P]
    float* E = R + (C + 1) * P;                            // [C+1][P] (linear bulk only)
    float* qsh = E + (LIN ? (C + 1) * P : 0);              // [2 rounds][M][lin, log][CP]
    float* nsh = qsh + 2 * M * 2 * CP;                     // [2 rounds][M][R, E][CP]
    float* dlsh = nsh + 2 * M * 2 * CP;                    // [CP] rebase shift per label
    float* dmsh = dlsh + CP;                               // [CP] dmax per label
    float* dummy = dmsh + CP;                              // [NT] sink for non-writing lanes
    float* Rrow = R + cr * P;
    float* Erow = E + cr * P;

    const double* Sb = a.S + (size_t)b * (T + 1) * C;
    for (int q = tid; q < C; q += NT) SL[q] = Sb[(size_t)L * C + q];
    for (int q = tid; q < (C + 1) * P; q += NT) {
        R[q] = NEG;
        if constexpr (LIN) E[q] = 0.0f;
    }
    for (int q = tid; q < 2 * M * CP; q += NT) {
        qsh[(q / CP) * 2 * CP + q % CP] = 0.0f;
        qsh[(q / CP) * 2 * CP + CP + q % CP] = NEG;
    }

    // ---------------------------------------------------------------- constants, base 2
    auto durv = [&](int c, int k) -> float {
        return k <= K ? fmaxf((float)((double)a.dur[(k - 1) * C + c] * LOG2E), NEG) : NEG;
    };
    // bulk lanes: durations k = 2M + j + i*G of label cb, scaled by the label's largest
    float dreg[KP], dlin[KP];
    float dmx = NEG;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        dreg[i] = bact ? durv(cb, 2 * M + j + i * G) : NEG;
        dmx = fmaxf(dmx, dreg[i]);
    }
    if (bact)
        for (int k = 1; k < 2 * M; ++k) dmx = fmaxf(dmx, durv(cb, k));
    if (!chain) dmx = group_reduce<G>(dmx, OpMax());
    const float dmax_b = dmx > NEG_HALF ? dmx : 0.0f;
#pragma unroll
    for (int i = 0; i < KPL; ++i) dlin[i] = exp2_or_zero(dreg[i] - dmax_b);
    if (bact && j == 0) dmsh[cb] = dmax_b;
    // chain lanes: durations k = 1 .. DIRECT and the transitions into label cl
    float dlog[DIRECT];
#pragma unroll
    for (int k = 0; k < DIRECT; ++k) dlog[k] = cact ? durv(cl, k + 1) : NEG;
    float treg[CP], wreg[CP], zero[CP];
    float tmx = NEG;
#pragma unroll
    for (int i = 0; i < CP; ++i) {
        float v = NEG;
        if (cact && i < C) {
            const float tv = dir == 0 ? a.trans[i * C + cl] : a.trans[cl * C + i];
            v = fmaxf((float)((double)tv * LOG2E), NEG);
        }
        treg[i] = v;
        zero[i] = 0.0f;
        tmx = fmaxf(tmx, v);
    }
    const float tmax = tmx > NEG_HALF ? tmx : 0.0f;       // linear transitions: 2^(trans - tmax)
#pragma unroll
    for (int i = 0; i < CP; ++i) wreg[i] = exp2_or_zero(treg[i] - tmax);
    __syncthreads();   // ring cleared, SL and dmax visible

    const float dmax = chain ? dmsh[cl] : dmax_b;
    float Dl[DIRECT];                                      // 2^(dur - dmax), k = 1 .. DIRECT
#pragma unroll
    for (int k = 0; k < DIRECT; ++k) Dl[k] = exp2_or_zero(dlog[k] - dmax);

    auto publish_q = [&](int r, int m, float ql, float qg) {   // bulk sum, round r, step m
        float* slot = qsh + ((r & 1) * M + m) * 2 * CP;
        *(bact && j == 0 ? slot + cb : dummy + tid) = ql;
        *(bact && j == 0 ? slot + CP + cb : dummy + tid) = qg;
    };
    // the M bulk sums of round r (positions p0 .. p0+M-1) at once: loads, products, trees
    // and DPP reductions of the M sums interleave; one wavefront-uniform fallback
    auto bulk_round = [&](int r, int p0) {
        float ql[M], qg[M];
        if constexpr (KPL == 0) {
#pragma unroll
            for (int m = 0; m < M; ++m) publish_q(r, m, 0.0f, NEG);
        } else {
            bool ok = true;
            float v[M][KP];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                ql[m] = 0.0f;
                qg[m] = NEG;
            }
            if constexpr (LIN) {
#pragma unroll
                for (int m = 0; m < M; ++m) ring_load<G, KPL, MIR>(Erow, p0 + m - 2 * M + 3, j, RS, v[m]);
#pragma unroll
                for (int m = 0; m < M; ++m) {
#pragma unroll
                    for (int i = 0; i < KPL; ++i) v[m][i] *= dlin[i];
#pragma unroll
                    for (int w = 1; w < KPL; w *= 2)
#pragma unroll
                        for (int i = 0; i + w < KPL; i += 2 * w) v[m][i] += v[m][i + w];
                }
#pragma unroll
                for (int m = 0; m < M; ++m) ql[m] = group_reduce<G>(v[m][0], OpSum());
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    qg[m] = fast_log2(ql[m]) + dmax_b;
                    ok &= in_lin_range(ql[m]) | !bact | (p0 + m > t1);
                }
            } else {
                ok = false;
            }
            if (wave_any(!ok)) {
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float w[KP];
                    ring_load<G, KPL, MIR>(Rrow, p0 + m - 2 * M + 3, j, RS, w);
                    const float lg = group_lse<G, KPL>(w, dreg);
                    if (!LIN || !(in_lin_range(ql[m]) || !bact)) {
                        qg[m] = lg;
                        ql[m] = exp2_or_zero(lg - dmax_b);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < M; ++m) publish_q(r, m, ql[m], qg[m]);
        }
    };

    // ---------------------------------------------------------------- state after trans(t0)
    const size_t ckrow = ((size_t)dir * a.B + b) * a.nspans;
    const size_t outrow = (size_t)b * (T + 1);
    double* Xout = dir == 0 ? a.XF : a.XB;
    double* Aout = dir == 0 ? a.AF : a.AB;
    auto put_all = [&](int pos, float rv, float ev) {
        ring_put<MIR>(Rrow, pos, RS, rv);
        if constexpr (LIN) ring_put<MIR>(Erow, pos, RS, ev);
    };
    double Bc = 0.0, H = 0.0;
    float Mref = 0.0f;
    // chain history: Rh[i], Eh[i] = ring entry of position (round start) - (DIRECT-1) + i
    // for i < DIRECT; entries DIRECT .. DIRECT+M-1 are the positions of the round
    float Rh[HN], Eh[HN];
#pragma unroll
    for (int i = 0; i < HN; ++i) {
        Rh[i] = NEG;
        Eh[i] = 0.0f;
    }
    if (t0 == 0) {
        if (bact && j == 0) put_all(0, 0.0f, 1.0f);   // position 0: no transition into it
        Rh[DIRECT - 1] = 0.0f;
        Eh[DIRECT - 1] = 1.0f;
    } else {
        const size_t ck = ckrow + span;
        if (bact)
            for (int q = j; q < K; q += G) {
                const float rv = a.ck_ring[(ck * K + q) * C + cb];
                put_all(t0 - q, rv, exp2_or_zero(rv));
            }
        if (chain) {
            Bc = a.ck_base[ck * C + cl];
            Mref = a.ck_mprev[ck * C + cl];
            H = a.ck_href[ck];
#pragma unroll
            for (int i = 0; i < DIRECT; ++i) {
                const int q = DIRECT - 1 - i;           // position t0 - q
                const float rv = (q < K && t0 - q >= 0) ? a.ck_ring[(ck * K + q) * C + cl] : NEG;
                Rh[i] = rv;
                Eh[i] = exp2_or_zero(rv);
            }
        }
    }
    if (cact && a.write_xa)
        Aout[(outrow + (dir == 0 ? t0 : L - t0)) * C + cl] = (Bc + (double)Rh[DIRECT - 1]) * LN2;

    // ---------------------------------------------------------------- S staging (bulk lanes)
    auto sidx = [&](int t, int q) -> size_t { return (size_t)(dir == 0 ? t : L - t) * C + q; };
    auto spub = [&](double raw, int q) -> double {
        return dir == 0 ? raw * LOG2E : (SL[q] - raw) * LOG2E;
    };
    double pf[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) pf[i] = 0.0;
    if (!chain) {
        for (int q = bt; q < rowsN; q += NB) {
            const int row = q / C, l = q - row * C;
            const int t = t0 + 1 + row;
            Sbuf[q] = (t <= t1) ? spub(Sb[sidx(t, l)], l) : 0.0;
        }
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int q = bt + i * NB;
            if (q < rowsN) {
                const int row = q / C, l = q - row * C;
                const int t = t0 + 1 + CH + row;
                if (t <= t1) pf[i] = Sb[sidx(t, l)];
            }
        }
    }
    __syncthreads();   // restored ring and chunk 0 visible
    __builtin_amdgcn_s_waitcnt(0);

    // bulk sums of round 0 (positions t0+1 .. t0+M need entries <= t0)
    if (!chain) bulk_round(0, t0 + 1);
    __syncthreads();

    // bulk lanes at the start of round r (rs = its first position - 1): apply the chain's
    // rebase of round r-1 to the ring, insert the chain's entries of round r-1, copy the
    // rings of the checkpoints the chain took in round r-1
    int next_ckb = ckpt ? a.delta : INT_MAX;   // next checkpoint whose ring is to copy
    auto ring_round = [&](int r, int rs) {
        // the chain rebased last round: move the entries it wrote before that.  Live
        // entries are positions rs-K-M+2 .. rs; lane j takes rs - j - i*G, reads first
        if (r >= 3 && (r & 1) == 1) {
            const float dl = bact ? dlsh[cb] : 0.0f;
            constexpr int KR = KPL + 1;
            float v[KR];
#pragma unroll
            for (int i = 0; i < KR; ++i) v[i] = Rrow[(rs - j - i * G) & RMASK];
#pragma unroll
            for (int i = 0; i < KR; ++i) {
                // slots outside the live window go to the spare row (read by idle lanes only)
                const int q = j + i * G;
                const bool live = (q < K + M) & (rs - q >= 0);
                const float rv = v[i] - dl;
                ring_put<MIR>(live ? Rrow : R + C * P, rs - q, RS, rv);
                if constexpr (LIN) ring_put<MIR>(live ? Erow : E + C * P, rs - q, RS, exp2_or_zero(rv));
            }
        }
        // insert the chain's entries of round r-1 (positions rs-M+1 .. rs)
        if (r >= 1 && bact && j < M && rs - M + 1 + j <= t1) {
            const int pos = rs - M + 1 + j;
            const float* ns = nsh + (((r - 1) & 1) * M + j) * 2 * CP;
            put_all(pos, ns[cb], ns[CP + cb]);
        }
        // checkpoint rings of the positions the chain checkpointed last round
        for (; next_ckb <= rs; next_ckb += a.delta) {
            const int pc = next_ckb;
            if (bact && pc < L) {
                const size_t ck = ckrow + pc / a.delta;
                for (int qq = j; qq < K; qq += G)
                    a.ck_ring[(ck * K + qq) * C + cb] = Rrow[(pc - qq) & RMASK];
            }
        }
    };

    // ---------------------------------------------------------------- main loop
    double BH = Bc - H;                                   // B_c - H
    double lz = 0.0;
    int next_ck = ckpt ? a.delta : INT_MAX;
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
        const double* Srow = Sbuf + (nch & 1) * rowsN;
        const int row0 = rs + 1 - tc;                  // chunk row of position rs+1
        if (chain) {
            float QL[M], QG[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float* slot = qsh + ((r & 1) * M + m) * 2 * CP;
                QL[m] = slot[cl];
                QG[m] = slot[CP + cl];
            }
            if (pend) {                                // summed before the ring was rebased
                const float sc = fast_exp2(-pdl);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    QL[m] *= sc;
                    QG[m] -= pdl;
                }
                pend = false;
            }
            if ((r & 1) == 0 && r > 0) {
                // ---- rebase: this label's values move to a new base
                const float ref = fmaxf(Mref, Rh[DIRECT - 1]);
                const float dl = cact && ref > NEG_HALF ? ref : 0.0f;
                const float sc = fast_exp2(-dl);
                Bc += (double)dl;
                BH += (double)dl;
                Mref -= dl;
#pragma unroll
                for (int i = 0; i < DIRECT; ++i) {
                    Rh[i] -= dl;
                    Eh[i] *= sc;
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    QL[m] *= sc;
                    QG[m] -= dl;
                }
                *(cact ? dlsh + cl : dummy + tid) = dl;
                pdl = dl;
                pend = true;
            }
            // ---- per-round constants.  Inside the round H moves by integer exponents
            // only: H(p_m) = H0 + eacc_m with eacc_m the sum of the earlier steps' e, so
            // 2^(S(p_m) + B_c - H(p_m)) = 2^hb[m] * 2^-eacc_m exactly.
            const double H0 = H;
            float hb[M], yv[M], fb[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                hb[m] = (float)(Srow[(row0 + m) * C + cl] + BH);   // S(p_m) + B_c - H0
                yv[m] = fast_exp2(hb[m] + dmax);                  // message scale
                fb[m] = fast_exp2(tmax - hb[m]);                   // ring-entry scale
            }
            // ---- fast pass (linear space, no branches)
            bool ok = true;
            int ev[M];                 // normaliser exponent of each step
            float sig[M];              // combined message sum (linear) or its log2 (replay)
            float qv[M];               // message total of each step (log Z at p = L)
            int eacc = 0;
            // terms k >= 2 of the first message; each step forms the next one's ahead of
            // its transition step, so only one FMA waits for the newest ring entry
            float part = QL[0];
#pragma unroll
            for (int k = DIRECT; k >= 2; --k) part = fmaf(Eh[DIRECT - k], Dl[k - 1], part);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int p = rs + 1 + m;
                const float sg = fmaf(Eh[DIRECT - 1 + m], Dl[0], part);
                sig[m] = sg;
                const float pn = cact ? __builtin_amdgcn_ldexpf(sg * yv[m], -eacc) : 0.0f;
                if (m + 1 < M) {
                    float nx = QL[m + 1];
#pragma unroll
                    for (int k = DIRECT; k >= 2; --k) nx = fmaf(Eh[DIRECT + m + 1 - k], Dl[k - 1], nx);
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
                        qa[i] += qa[i + w];
                    }
                const float s = sv[0], q = qa[0];
                // label lanes only: lanes outside row 0 broadcast their own (empty) row
                ok &= (p > t1) | !cact | (in_lin_range(sg) & in_lin_range(s) & in_lin_range(q));
                const int e = __builtin_amdgcn_frexp_expf(q);          // q = m 2^e
                Eh[DIRECT + m] = __builtin_amdgcn_ldexpf(s * fb[m], eacc);
                Rh[DIRECT + m] = fast_log2(s) + (tmax - hb[m]) + (float)eacc;
                qv[m] = q;
                ev[m] = e;
                eacc += e;
            }
            bool replayed = false;
            if (wave_any(!ok)) {
                // ---- exact replay of the round in log space
                replayed = true;
                eacc = 0;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const int p = rs + 1 + m;
                    if (p > t1) break;
                    const float hp = hb[m] - (float)eacc;
                    float x[DIRECT + 1];
#pragma unroll
                    for (int k = 1; k <= DIRECT; ++k) x[k - 1] = Rh[DIRECT - 1 + m + 1 - k] + dlog[k - 1];
                    x[DIRECT] = QG[m];
                    float mx = x[0];
#pragma unroll
                    for (int k = 1; k <= DIRECT; ++k) mx = fmaxf(mx, x[k]);
                    float sm = 0.0f;
#pragma unroll
                    for (int k = 0; k <= DIRECT; ++k) sm += fast_exp2(x[k] - mx);
                    const float sigma = mx + fast_log2(sm);
                    sig[m] = sigma;
                    const float u = cact ? hp + sigma : NEG;
                    float uv[CP];
#pragma unroll
                    for (int i = 0; i < CP; ++i)
                        uv[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u), i));
                    const float rn = group_lse<1, CP>(uv, treg) - hp;
                    const float lq = group_lse<1, CP>(uv, zero);
                    const int e = lq > NEG_HALF ? (int)floorf(lq) + 1 : 0;
                    Rh[DIRECT + m] = rn;
                    Eh[DIRECT + m] = exp2_or_zero(rn);
                    qv[m] = lq;
                    ev[m] = e;
                    eacc += e;
                }
            }
            {
                const int mL = L - rs - 1;                 // log Z when the round holds L
                if (mL >= 0 && mL < M) {
                    int eb = 0;
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        if (m < mL) eb += ev[m];
                    float ql = qv[0];
#pragma unroll
                    for (int m = 1; m < M; ++m)
                        if (m == mL) ql = qv[m];
                    lz = H0 + (double)eb + (double)(replayed ? ql : fast_log2(ql));
                }
            }
            {
                int et = 0;                                // H moves by the steps taken
#pragma unroll
                for (int m = 0; m < M; ++m)
                    if (rs + 1 + m <= t1) et += ev[m];
                H = H0 + (double)et;
                BH = Bc - H;
            }
            // ---- publish the round: ring entries for the bulk lanes, outputs, checkpoints
            int ec = 0;                                    // steps taken so far this round
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int p = rs + 1 + m;
                if (p > t1) break;
                float* ns = nsh + ((r & 1) * M + m) * 2 * CP;
                *(cact ? ns + cl : dummy + tid) = Rh[DIRECT + m];
                *(cact ? ns + CP + cl : dummy + tid) = Eh[DIRECT + m];
                if (a.write_xa && cact) {
                    const double Sp = Srow[(row0 + m) * C + cl];
                    const float sgl = replayed ? sig[m] : fast_log2(sig[m]) + dmax;
                    Xout[(outrow + (dir == 0 ? p : L - p)) * C + cl] = (Sp + Bc + (double)sgl) * LN2;
                    if (p < t1)
                        Aout[(outrow + (dir == 0 ? p : L - p)) * C + cl] =
                            (Bc + (double)Rh[DIRECT + m]) * LN2;
                }
                ec += ev[m];                             // H after the transition step of p
                if (QG[m] > NEG_HALF) Mref = QG[m];
                if (p == next_ck) {
                    // chain half of the checkpoint after the transition step of p; the ring
                    // half is copied by the bulk lanes next round
                    if (p < L) {
                        const size_t ck = ckrow + p / a.delta;
                        if (cact) {
                            a.ck_base[ck * C + cl] = Bc;
                            a.ck_mprev[ck * C + cl] = Mref;
                        }
                        if (tid == 0) a.ck_href[ck] = H0 + (double)ec;
                    }
                    next_ck += a.delta;
                }
            }
#pragma unroll
            for (int i = 0; i < DIRECT; ++i) {   // history for the next round
                Rh[i] = Rh[i + M];
                Eh[i] = Eh[i + M];
            }
        } else {
            // ---- S staging: in the first round of a chunk publish the next one
            if (rs + 1 == tc && tc + CH <= t1) {
                double* dst = Sbuf + ((nch + 1) & 1) * rowsN;
#pragma unroll
                for (int i = 0; i < PF; ++i) {
                    const int q = bt + i * NB;
                    if (q < rowsN) dst[q] = spub(pf[i], q - (q / C) * C);
                }
#pragma unroll
                for (int i = 0; i < PF; ++i) {
                    const int q = bt + i * NB;
                    if (q < rowsN) {
                        const int rr = q / C, l = q - rr * C;
                        const int tt = tc + 2 * CH + rr;
                        pf[i] = (tt <= t1) ? Sb[sidx(tt, l)] : 0.0;
                    }
                }
            }
            ring_round(r, rs);
            // ---- bulk sums of round r+1 (entries <= rs suffice)
            bulk_round(r + 1, rs + M + 1);
        }
        __syncthreads();
    }

    // checkpoints taken in the last round: their rings are copied here
    if (ckpt && !chain) ring_round(nrounds, t0 + nrounds * M);

    // ---------------------------------------------------------------- end of sequence
    if (t1 == L && tid == 0) (dir == 0 ? a.logz : a.logz_b)[b] = bad ? nan_d() : lz * LN2;
}

// ------------------------------------------------------------------ launch
template <int G, int KPL, int LAY>
static hipError_t launch_lse_round_inst(const SweepArgs& a, dim3 grid, const SweepCfg& cfg,
                                        hipStream_t stream) {
    if (cfg.NT > 320 || cfg.lse.CH > lse_chunk_max(G) || cfg.lse.CH % ROUND != 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_lse_round<G, KPL, LAY>), grid, dim3(cfg.NT), cfg.lse.bytes, stream, a,
                       cfg.RS, cfg.lse.P, cfg.lse.CH);
    return hipGetLastError();
}

#define LSE_ROUND_KPL_CASES(G)                                                       \
    switch (cfg.KPLr) {                                                              \
        case 0: return launch_lse_round_inst<G, 0, LAY>(a, grid, cfg, stream);          \
        case 1: return launch_lse_round_inst<G, 1, LAY>(a, grid, cfg, stream);          \
        case 2: return launch_lse_round_inst<G, 2, LAY>(a, grid, cfg, stream);          \
        case 3: return launch_lse_round_inst<G, 3, LAY>(a, grid, cfg, stream);          \
        case 4: return launch_lse_round_inst<G, 4, LAY>(a, grid, cfg, stream);          \
        case 5: return launch_lse_round_inst<G, 5, LAY>(a, grid, cfg, stream);          \
        case 6: return launch_lse_round_inst<G, 6, LAY>(a, grid, cfg, stream);          \
        case 7: return launch_lse_round_inst<G, 7, LAY>(a, grid, cfg, stream);          \
        case 8: return launch_lse_round_inst<G, 8, LAY>(a, grid, cfg, stream);          \
        case 10: return launch_lse_round_inst<G, 10, LAY>(a, grid, cfg, stream);        \
        case 12: return launch_lse_round_inst<G, 12, LAY>(a, grid, cfg, stream);        \
        case 16: return launch_lse_round_inst<G, 16, LAY>(a, grid, cfg, stream);        \
        case 24: return launch_lse_round_inst<G, 24, LAY>(a, grid, cfg, stream);        \
        case 32: return launch_lse_round_inst<G, 32, LAY>(a, grid, cfg, stream);        \
        default: return hipErrorInvalidValue;                                        \
    }

template <int LAY>
hipError_t launch_lse_round_layout(const SweepCfg& cfg, const SweepArgs& a, int ndir,
                                   hipStream_t stream) {
    dim3 grid = a.mode == MODE_FULL ? dim3(a.B, ndir) : dim3(a.nspans, a.B, ndir);
    if (cfg.G == 64) { LSE_ROUND_KPL_CASES(64) }
    if (cfg.G == 32) { LSE_ROUND_KPL_CASES(32) }
    if (cfg.G == 16) { LSE_ROUND_KPL_CASES(16) }
    return hipErrorInvalidValue;
}

#undef LSE_ROUND_KPL_CASES

}  // namespace semicrf
