// Max-plus streaming sweep on gfx950 (Viterbi): the recurrence of the log-semiring sweep
// with LSE replaced by max, plus backpointers.
//
// Method ("Streaming Structured Inference with Flash-SemiCRF", gist.science EN explainer,
// "2. Methodology"; decoding is the (max, +) form of the same forward recursion).  In the
// factored form
//     abar[s, c]  = max_{c'} (V[s, c'] + trans[c', c])
//     V[t, c]     = S[t, c] + max_k (abar[t-k, c] - S[t-k, c] + dur[k-1, c])
// with abar[0, c] = 0.  The backpointer of (t, c) is the lowest k attaining the inner max
// and, for the segment start s = t - k, the lowest c' attaining abar[s, c]; packed as
// k | c' << 16 (c' stored at the start position s).
//
// Work layout as in the log-semiring sweep: one workgroup per checkpoint span (or per
// sequence for a repair), lanes in groups of G per label, the label's ring of A = abar - S (relative to a per-label fp64 base,
// moved every REBASE positions) in LDS, one barrier per position.  Iteration t runs
//   [B] transition step of position t-1: max over u(t-1)[c'] + T[c', c] (DPP) -> A[t-1, c]
//   [C] V(t): three-term max of the k = 1, 2 terms and the bulk value of t -> u(t) to LDS
//   [D] bulk value for position t+2: max over this label's ring (lane j owns k = 3+j+i*G)
// fp32 arithmetic on values kept small (u = V - H with a common fp64 reference H).
#pragma once

#include "internal.h"
#include "ring.h"

namespace semicrf {

namespace {

// Bulk value of position tq (terms k >= 3): max over the group and the lowest k attaining it.
template <int G, int KPL, bool MIR>
__device__ __forceinline__ float bulk_max(const float* Rrow, int tq, int j, int RS,
                                          const float* dreg, int* kbest) {
    if constexpr (KPL == 0) {
        *kbest = INT_MAX;
        return NEG;
    } else {
        float v[KPL];
        ring_load<G, KPL, MIR>(Rrow, tq, j, RS, v);
        return group_argmax<G, KPL>(v, dreg, j, kbest);
    }
}

}  // namespace

// G: lanes per label; KPL: durations k >= 3 per lane (k = 3 + j + i*G, i < KPL, covering
// k <= K + 1); CPL, GT: previous labels per lane and the lane count of the transition
// reduction (GT * CPL >= C, GT <= G); NTMAX: largest workgroup routed here.
// Natural-log units (max-plus needs no base change).
template <int G, int KPL, int CPL, int GT, int NTMAX, bool MIR>
__global__ __launch_bounds__(NTMAX) void k_maxplus(const SweepArgs a, const int RS, const int P,
                                                  const int CH,
                                                  const float* __restrict__ proj_start,
                                                  const float* __restrict__ proj_end) {
    constexpr int PF = (MAXPLUS_CHUNK_MAX + G - 1) / G;   // prefetched doubles per lane (NT >= C*G)
    constexpr int UP = GT * CPL;                   // padded u row (>= C)
    extern __shared__ double lds[];
    const int C = a.C, K = a.K, T = a.T;
    const int tid = threadIdx.x, NT = blockDim.x;
    const int c = tid / G;
    const int j = tid - c * G;
    const int jt = j & (GT - 1);             // every GT-subgroup repeats the transition step
    const bool act = c < C;
    const int cr = act ? c : C;              // inactive lanes use the spare LDS row C
    const int cc = act ? c : 0;

    // MODE_SPEC: grid (nspans, B), every span at once from a burn-in; MODE_REPAIR: grid
    // (B), from the checkpoint at the first failed seam to the end.
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
    const bool ckpt = spec && t1 < L;                    // checkpoint at the span's end
    const int hlo = (spec && span > 0) ? tout - K + 1 : INT_MAX;    // seam windows
    const int tlo = ckpt ? t1 - K + 1 : INT_MAX;
    const size_t winrow = ((size_t)b * a.nspans + span) * K;
    const size_t ckrow = (size_t)b * a.nspans;
    auto window = [&](int t, double av) {                // writer lanes
        if (t >= hlo && t <= tout) a.head[(winrow + t - hlo) * C + c] = av;
        if (t >= tlo && t <= t1) a.tail[(winrow + t - tlo) * C + c] = av;
    };
    const int RMASK = RS - 1;
    const int chunkN = CH * C;

    // end side S(t) + proj_end[t-1] and start side S(t) - proj_start[t]:
    // [2 chunks][2 sides][CH][C]
    double* Sbuf = lds;
    float* R = (float*)(Sbuf + 4 * chunkN);              // [C+1][P]
    float* u_sh = R + (C + 1) * P;                       // [2][UP]
    float* Rrow = R + cr * P;

    const double* Sb = a.S + (size_t)b * (T + 1) * C;
    const float* PSb = proj_start ? proj_start + (size_t)b * T * C : nullptr;
    const float* PEb = proj_end ? proj_end + (size_t)b * T * C : nullptr;
    // projections at position t (flat index q = t*C + l): 0 when absent or outside
    // [1, L] (end side) / [0, L-1] (start side)
    auto proj_e = [&](int t, size_t q) -> float {
        return (PEb && t >= 1 && t <= L) ? PEb[q - C] : 0.0f;
    };
    auto proj_s = [&](int t, size_t q) -> float { return (PSb && t < L) ? PSb[q] : 0.0f; };
    for (int q = tid; q < (C + 1) * P; q += NT) R[q] = NEG;
    for (int q = tid; q < 2 * UP; q += NT) u_sh[q] = NEG;

    // durations (k >= 3 per lane; k = 1, 2 group-uniform) and transitions
    auto durv = [&](int k) -> float {
        return (act && k <= K) ? fmaxf(a.dur[(k - 1) * C + c], NEG) : NEG;
    };
    float dreg[KPL > 0 ? KPL : 1];
#pragma unroll
    for (int i = 0; i < KPL; ++i) dreg[i] = durv(3 + j + i * G);
    const float d0 = durv(1), d1 = durv(2);
    float treg[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int cp = jt + i * GT;
        treg[i] = (act && cp < C) ? fmaxf(a.trans[cp * C + c], NEG) : NEG;
    }
    __syncthreads();   // ring and u cleared

    auto put = [&](int pos, float r) { ring_put<MIR>(Rrow, pos, RS, r); };

    double Bc = 0.0, H = 0.0;
    float Mref = 0.0f, Rn1 = NEG, Rn2 = NEG;
    if (t0 == 0) {
        // position 0: no transition into it; the ring entry is its start-side projection
        Rn1 = act ? fmaxf(proj_s(0, cc), NEG) : 0.0f;
        if (act && j == 0) put(0, Rn1);
        if (act && j == 0)
            for (int p = min(hlo, tlo); p <= 0; ++p) window(p, p == 0 ? (double)Rn1 : -1.0e300);
    } else if (spec) {
        // burn-in start: every ring entry of positions t0-K+1 .. t0 equal
        if (act)
            for (int q = j; q < K && t0 - q >= 0; q += G) put(t0 - q, 0.0f);
        Rn1 = 0.0f;
        Rn2 = (K >= 2 && t0 >= 1) ? 0.0f : NEG;
    } else {
        const size_t ck = ckrow + span;
        if (act)
            for (int q = j; q < K; q += G) put(t0 - q, a.ck_ring[(ck * K + q) * C + c]);
        Bc = a.ck_base[ck * C + cc];
        Mref = a.ck_mprev[ck * C + cc];
        H = a.ck_href[ck];
        Rn1 = a.ck_ring[(ck * K + 0) * C + cc];
        Rn2 = K >= 2 ? a.ck_ring[(ck * K + 1) * C + cc] : NEG;
    }
    __syncthreads();

    int kQa = 0, kQb = 0, kb_prev = 0;
    float Qa = bulk_max<G, KPL, MIR>(Rrow, t0 + 1, j, RS, dreg, &kQa);
    float Qb = bulk_max<G, KPL, MIR>(Rrow, t0 + 2, j, RS, dreg, &kQb);

    // ---------------------------------------------------------------- S staging
    for (int q = tid; q < chunkN; q += NT) {
        const int t = t0 + 1 + q / C;
        const size_t gq = (size_t)(t0 + 1) * C + q;
        const double sv = (t <= t1) ? Sb[gq] : 0.0;
        Sbuf[q] = (t <= t1) ? sv + (double)proj_e(t, gq) : 0.0;
        Sbuf[chunkN + q] = (t <= t1) ? sv - (double)proj_s(t, gq) : 0.0;
    }
    // the chunk after: values in registers, published CH positions later
    double pf[PF], pfs[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const int q = tid + i * NT;
        pf[i] = pfs[i] = 0.0;
        const int t = t0 + 1 + CH + q / C;
        if (q < chunkN && t <= t1) {
            const size_t gq = (size_t)(t0 + 1 + CH) * C + q;
            pf[i] = Sb[gq] + (double)proj_e(t, gq);
            pfs[i] = Sb[gq] - (double)proj_s(t, gq);
        }
    }
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0);   // nothing loaded before the loop is waited on inside it

    float h_prev = 0.0f;      // start side of the previous position, relative to H
    const size_t outrow = (size_t)b * (T + 1);

    // ---------------------------------------------------------------- main loop
    // the transition step [B] of position t-1, at iteration t (and once more after the loop
    // for a span's last position)
    auto transition = [&](int tp) {
        const float* us = u_sh + (tp & 1) * UP;
        float y[CPL], uv[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            uv[i] = us[jt + i * GT];
            y[i] = uv[i] + treg[i];
        }
        float mt = y[0], mu = uv[0];
#pragma unroll
        for (int i = 1; i < CPL; ++i) {
            mt = fmaxf(mt, y[i]);
            mu = fmaxf(mu, uv[i]);
        }
        mt = group_reduce<GT>(mt, OpMax());
        mu = group_reduce<GT>(mu, OpMax());
        int cb = INT_MAX;
#pragma unroll
        for (int i = CPL - 1; i >= 0; --i)
            if (y[i] == mt) cb = jt + i * GT;
        const int cbest = group_min_int<GT>(cb);
        const float Rnew = mt - h_prev;
        H += (double)mu;
        Rn2 = Rn1;
        Rn1 = Rnew;
        if (j == 0) {
            put(tp, Rnew);
            if (act && tp > tout)
                a.bp[(outrow + tp) * C + c] = (uint32_t)kb_prev | ((uint32_t)cbest << 16);
            if (act && tp >= min(hlo, tlo)) window(tp, Bc + (double)Rnew);
        }
    };
    for (int tc = t0 + 1, nch = 0; tc <= t1; tc += CH, ++nch) {
        const double* Srow = Sbuf + (nch & 1) * 2 * chunkN;   // end side; start side at +chunkN
        const int rows = min(CH, t1 - tc + 1);
        for (int row = 0; row < rows; ++row) {
            const int t = tc + row;
            if (t > t0 + 1) transition(t - 1);
            // ---- [C] V(t): k = 1, 2 from registers, k >= 3 from the bulk value
            const float e1 = Rn1 + d0, e2 = Rn2 + d1;
            const float sig = fmaxf(fmaxf(Qa, e1), e2);
            kb_prev = (e1 == sig) ? 1 : (e2 == sig) ? 2 : kQa;
            const float h = (float)(Srow[row * C + cc] + Bc - H);
            if (j == 0) u_sh[(t & 1) * UP + cr] = h + sig;
            h_prev = (float)(Srow[chunkN + row * C + cc] + Bc - H);

            // ---- [D] rebase, then the bulk value for position t+2
            if ((t & (REBASE - 1)) == 0) {
                const float ref = fmaxf(Mref, Rn1);
                const float dl = ref > NEG_HALF ? ref : 0.0f;
                Bc += (double)dl;
                Qb -= dl;
                Rn1 -= dl;
                Rn2 -= dl;
                h_prev += dl;
                if constexpr (KPL > 0) {
                    // every slot of positions t-1 .. t-KPL*G (the live window and older,
                    // dead, distinct slots): reads first, then writes
                    float v[KPL];
                    ring_load<G, KPL, MIR>(Rrow, t + 2, j, RS, v);
#pragma unroll
                    for (int i = 0; i < KPL; ++i) v[i] -= dl;
                    ring_store<G, KPL, MIR>(Rrow, t + 2, j, RS, v);
                }
            }
            int kQn = 0;
            const float Qn = bulk_max<G, KPL, MIR>(Rrow, t + 2, j, RS, dreg, &kQn);
            if (Qn > NEG_HALF) Mref = Qn;
            Qa = Qb;
            Qb = Qn;
            kQa = kQb;
            kQb = kQn;
            __syncthreads();
        }
        // ---- S staging: publish the next chunk, fetch the one after
        if (tc + CH <= t1) {
            double* dst = Sbuf + ((nch + 1) & 1) * 2 * chunkN;
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                const int q = tid + i * NT;
                if (q < chunkN) {
                    dst[q] = pf[i];
                    dst[chunkN + q] = pfs[i];
                }
            }
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                const int q = tid + i * NT;
                if (q < chunkN) {
                    const int tt = tc + 2 * CH + q / C;
                    const size_t gq = (size_t)(tc + 2 * CH) * C + q;
                    pf[i] = (tt <= t1) ? Sb[gq] + (double)proj_e(tt, gq) : 0.0;
                    pfs[i] = (tt <= t1) ? Sb[gq] - (double)proj_s(tt, gq) : 0.0;
                }
            }
            __syncthreads();
        }
    }

    if (t1 < L) {
        // a span's last position: its transition step (the previous-label field of its
        // backpointer, its ring entry, the tail window), then the checkpoint at it
        transition(t1);
        if (ckpt) {
            __syncthreads();                                // every label's ring entry of t1
            const size_t ck = ckrow + t1 / a.delta;
            if (act)
                for (int qq = j; qq < K; qq += G)
                    a.ck_ring[(ck * K + qq) * C + c] = Rrow[(t1 - qq) & RMASK];
            if (act && j == 0) {
                a.ck_base[ck * C + c] = Bc;
                a.ck_mprev[ck * C + c] = Mref;
            }
            if (tid == 0) a.ck_href[ck] = H;
        }
        return;
    }
    // ---------------------------------------------------------------- end of sequence
    const float* us = u_sh + (L & 1) * UP;
    if (act && j == 0) a.bp[(outrow + L) * C + c] = (uint32_t)kb_prev;
    // the values V(L, c) in this sweep's frame; the final label is chosen afterwards
    if (act && j == 0) a.vfin[(size_t)b * C + c] = H + (double)us[c];
}

// ------------------------------------------------------------------ launch
template <int G, int KPL, int CPL, int GT, int NTMAX, bool MIR>
static hipError_t launch_maxplus_inst(const SweepLaunch& a, const SweepCfg& cfg,
                                      hipStream_t stream) {
    if (cfg.NTv > NTMAX || cfg.vit.CH > MAXPLUS_CHUNK_MAX) return hipErrorInvalidValue;
    if (a.mode != MODE_SPEC && a.mode != MODE_REPAIR) return hipErrorInvalidValue;
    const dim3 grid = a.mode == MODE_SPEC ? dim3(a.nspans, a.B) : dim3(a.B);
    hipLaunchKernelGGL((k_maxplus<G, KPL, CPL, GT, NTMAX, MIR>), grid, dim3(cfg.NTv),
                       cfg.vit.bytes, stream, static_cast<const SweepArgs&>(a), cfg.RS,
                       cfg.vit.P, cfg.vit.CH, a.proj_start, a.proj_end);
    return hipGetLastError();
}

#define MAXPLUS_KPL_CASES(G, CPL, GT, NTMAX)                                         \
    switch (cfg.KPL) {                                                               \
        case 0: return launch_maxplus_inst<G, 0, CPL, GT, NTMAX, MIR>(a, cfg, stream);   \
        case 1: return launch_maxplus_inst<G, 1, CPL, GT, NTMAX, MIR>(a, cfg, stream);   \
        case 2: return launch_maxplus_inst<G, 2, CPL, GT, NTMAX, MIR>(a, cfg, stream);   \
        case 3: return launch_maxplus_inst<G, 3, CPL, GT, NTMAX, MIR>(a, cfg, stream);   \
        case 4: return launch_maxplus_inst<G, 4, CPL, GT, NTMAX, MIR>(a, cfg, stream);   \
        case 5: return launch_maxplus_inst<G, 5, CPL, GT, NTMAX, MIR>(a, cfg, stream);   \
        case 6: return launch_maxplus_inst<G, 6, CPL, GT, NTMAX, MIR>(a, cfg, stream);   \
        case 7: return launch_maxplus_inst<G, 7, CPL, GT, NTMAX, MIR>(a, cfg, stream);   \
        case 8: return launch_maxplus_inst<G, 8, CPL, GT, NTMAX, MIR>(a, cfg, stream);   \
        case 10: return launch_maxplus_inst<G, 10, CPL, GT, NTMAX, MIR>(a, cfg, stream); \
        case 12: return launch_maxplus_inst<G, 12, CPL, GT, NTMAX, MIR>(a, cfg, stream); \
        case 16: return launch_maxplus_inst<G, 16, CPL, GT, NTMAX, MIR>(a, cfg, stream); \
        case 24: return launch_maxplus_inst<G, 24, CPL, GT, NTMAX, MIR>(a, cfg, stream); \
        case 32: return launch_maxplus_inst<G, 32, CPL, GT, NTMAX, MIR>(a, cfg, stream); \
        default: return hipErrorInvalidValue;                                        \
    }

// every kernel shape of one ring layout (one translation unit per layout)
template <bool MIR>
hipError_t launch_maxplus_layout(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream) {
    // C <= 16 (G >= 16) runs the round kernel instead
    if (cfg.G == 8 && cfg.CPL == 4) { MAXPLUS_KPL_CASES(8, 4, 8, 256) }
    if (cfg.G == 8 && cfg.CPL == 8) { MAXPLUS_KPL_CASES(8, 8, 8, 512) }
    if (cfg.G == 4) { MAXPLUS_KPL_CASES(4, 32, 4, 512) }
    return hipErrorInvalidValue;
}

#undef MAXPLUS_KPL_CASES

}  // namespace semicrf
