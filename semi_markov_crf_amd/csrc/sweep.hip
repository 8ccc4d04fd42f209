// Streaming semi-CRF recurrence on gfx950: forward (alpha), backward (beta, run as a
// forward sweep over the mirrored sequence) and max-plus Viterbi.
//
// Method ("Streaming Structured Inference with Flash-SemiCRF", gist.science EN explainer,
// "2. Methodology"): segment potentials S[s+k,c] - S[s,c] + dur[k-1,c] + trans[c',c] are
// evaluated on the fly from the prefix sums; only a ring of the last K messages is kept
// ("Streaming Forward-Backward with Ring Buffers"); the ring and the cumulative
// normaliser are written out every delta positions and a later pass restarts from them
// ("Checkpointing").
//
// Factored recurrence.  The potential is a sum of a (start, length, label) term and a
// (previous label, label) term, so the log-sum over (k, c') splits exactly into
//     abar[s, c]  = LSE_{c'} (alpha[s, c'] + trans[c', c])              (C^2 per position)
//     alpha[t, c] = S[t, c] + LSE_{k} (abar[t-k, c] - S[t-k, c] + dur[k-1, c])   (K*C)
// with abar[0, c] = 0 (no transition into the first segment).  This evaluates the same
// K*C^2 edges per position with K*C + C^2 exponentials instead of K*C^2.  The ring holds
// A[s, c] = abar[s, c] - S[s, c].  The backward sweep is the same recurrence on the
// reversed sequence: S'[t] = S[L] - S[L-t], trans' = trans^T; its "alpha" is
// beta_bar[s, c] (all segmentations of [s, L) whose first segment has label c) and its
// "A" is beta[u, c] + S[u, c] - S[L, c].
//
// Work layout: one workgroup per (sequence, direction) for a full sweep, or per
// (checkpoint span, sequence, direction) for the recompute.  Lanes form groups of G per
// label c; lane j of group c owns durations k = j+1+i*G (i < KPL) and previous labels
// c' = j+i*G (i < CPL).  Each position takes two phases separated by workgroup barriers:
//   bulk:  the K-term log-sum-exp of group c (DPP max, exp2, DPP sum) -> u[c] in LDS
//   trans: the C-term log-sum-exp over u[c'] + trans[c', c] -> new ring entry A[t, c].
// Arithmetic is fp32 in base 2 on values kept small: ring entries are stored relative
// to an fp64 per-label base that is moved every REBASE positions, and S enters through
// the fp64 difference S[t, c] + base[c] - H, where H is a common fp64 reference that
// follows the running maximum.  Outputs are written in fp64, natural-log units.
#include <limits.h>

#include "common.h"
#include "internal.h"

namespace semicrf {

constexpr int REBASE = 8;      // rebase the ring every REBASE positions (global index)
constexpr int CHUNK = 64;      // positions of S staged per LDS chunk

__device__ __forceinline__ double nan_d() { return __longlong_as_double(0x7ff8000000000000LL); }

template <int G, int KPL, int CPL, bool VIT>
__global__ __launch_bounds__(1024) void k_sweep(const SweepArgs a, const int RS, const int RSP) {
    constexpr int PF = (CHUNK + G - 1) / G;   // prefetched doubles per lane (NT >= C*G)
    extern __shared__ double lds[];
    const int C = a.C, K = a.K, T = a.T;
    const int tid = threadIdx.x, NT = blockDim.x;
    const int c = tid / G;
    const int j = tid - c * G;
    const bool act = c < C;
    const int cc = act ? c : 0;

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
    const double scale = VIT ? 1.0 : LOG2E;
    const double inv_scale = VIT ? 1.0 : LN2;
    const int RMASK = RS - 1;
    const int chunkN = CHUNK * C;

    double* Sbuf = lds;                       // [2][CHUNK][C]
    double* SL = Sbuf + 2 * chunkN;           // [C]
    double* Hs = SL + C;                      // [2]
    float* ring = (float*)(Hs + 2);           // [C][RSP]
    float* u_sh = ring + C * RSP;             // [C]

    const double* Sb = a.S + (size_t)b * (T + 1) * C;
    for (int q = tid; q < C; q += NT) SL[q] = Sb[(size_t)L * C + q];

    // durations / transitions owned by this lane, scaled to base 2, -inf clamped
    float dreg[KPL], treg[CPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int k = j + 1 + i * G;
        dreg[i] = (act && k <= K) ? fmaxf((float)((double)a.dur[(k - 1) * C + c] * scale), NEG) : NEG;
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int cp = j + i * G;
        float v = NEG;
        if (act && cp < C) {
            const float tv = dir == 0 ? a.trans[cp * C + c] : a.trans[c * C + cp];
            v = fmaxf((float)((double)tv * scale), NEG);
        }
        treg[i] = v;
    }

    // ---------------------------------------------------------------- initial state
    const size_t ckrow = ((size_t)dir * a.B + b) * a.nspans;
    double Bc = 0.0, H = 0.0;
    float Mprev = 0.0f;
    double* Xout = dir == 0 ? a.XF : a.XB;
    double* Aout = dir == 0 ? a.AF : a.AB;
    // Every slot starts at NEG: lanes whose k exceeds K (masked by dur = NEG) still read
    // a slot each position, and must never see uninitialised LDS.
    for (int q = tid; q < C * RSP; q += NT) ring[q] = NEG;
    __syncthreads();
    if (t0 == 0) {
        if (act) {
#pragma unroll
            for (int i = 0; i < KPL; ++i) {
                const int k = j + 1 + i * G;
                if (k <= K) ring[c * RSP + ((1 - k) & RMASK)] = (k == 1) ? 0.0f : NEG;
            }
            if (a.write_xa && j == 0) Aout[((size_t)b * (T + 1) + (dir == 0 ? 0 : L)) * C + c] = 0.0;
        }
    } else {
        const size_t ck = ckrow + span;
        if (act) {
#pragma unroll
            for (int i = 0; i < KPL; ++i) {
                const int k = j + 1 + i * G;
                if (k <= K) ring[c * RSP + ((t0 + 1 - k) & RMASK)] = a.ck_ring[(ck * K + (k - 1)) * C + c];
            }
        }
        Bc = a.ck_base[ck * C + cc];
        Mprev = a.ck_mprev[ck * C + cc];
        H = a.ck_href[ck];
    }

    // ---------------------------------------------------------------- S staging
    auto sval = [&](int t, int q) -> double {
        return dir == 0 ? Sb[(size_t)t * C + q] * scale : (SL[q] - Sb[(size_t)(L - t) * C + q]) * scale;
    };
    __syncthreads();   // SL visible
    for (int q = tid; q < chunkN; q += NT) {
        const int row = q / C, l = q - row * C;
        const int t = t0 + 1 + row;
        Sbuf[q] = (t <= t1) ? sval(t, l) : 0.0;
    }
    double pf[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const int q = tid + i * NT;
        pf[i] = 0.0;
        if (q < chunkN) {
            const int row = q / C, l = q - row * C;
            const int t = t0 + 1 + CHUNK + row;
            if (t <= t1) pf[i] = sval(t, l);
        }
    }
    __syncthreads();

    int next_ck = (a.mode == MODE_FULL && a.write_ckpt) ? a.delta : INT_MAX;

    // ---------------------------------------------------------------- main loop
    for (int t = t0 + 1; t <= t1; ++t) {
        const int rel = t - t0 - 1;
        const int row = rel & (CHUNK - 1);
        const int nch = rel / CHUNK;
        const bool rebase = (t & (REBASE - 1)) == 0;
        const float dl = (Mprev > NEG_HALF) ? Mprev : 0.0f;

        // ---- bulk phase: sig[c] = LSE_k (ring[c][t-k] + dur[k-1][c])
        float x[KPL];
        float m = NEG;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const int k = j + 1 + i * G;
            const int sidx = cc * RSP + ((t - k) & RMASK);
            float r = ring[sidx];
            if (rebase) {
                r -= dl;
                if (act && k <= K) ring[sidx] = r;
            }
            x[i] = r + dreg[i];
            m = fmaxf(m, x[i]);
        }
        if (rebase) Bc += (double)dl;

        float sig;
        int kbest = 0;
        m = group_reduce<G>(m, OpMax());
        if constexpr (!VIT) {
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < KPL; ++i) s += fast_exp2(x[i] - m);
            s = group_reduce<G>(s, OpSum());
            sig = m + fast_log2(s);
        } else {
            int kk = INT_MAX;
#pragma unroll
            for (int i = 0; i < KPL; ++i)
                if (x[i] == m && kk == INT_MAX) kk = j + 1 + i * G;
            kbest = group_min_int<G>(kk);
            sig = m;
        }
        Mprev = m;

        const double g = Sbuf[(nch & 1) * chunkN + row * C + cc] + Bc;
        const float h = (float)(g - H);
        if (act && j == 0) {
            u_sh[c] = h + sig;
            if (a.write_xa) Xout[((size_t)b * (T + 1) + (dir == 0 ? t : L - t)) * C + c] = (g + (double)sig) * inv_scale;
        }
        __syncthreads();

        // ---- transition phase: A[t][c] = LSE_{c'} (u[c'] + T[c'][c]) - h
        float y[CPL];
        float mt = NEG;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int cp = j + i * G;
            y[i] = ((cp < C) ? u_sh[cp] : NEG) + treg[i];
            mt = fmaxf(mt, y[i]);
        }
        mt = group_reduce<G>(mt, OpMax());
        float Rn;
        int cbest = 0;
        if constexpr (!VIT) {
            float st = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) st += fast_exp2(y[i] - mt);
            st = group_reduce<G>(st, OpSum());
            Rn = mt + fast_log2(st) - h;
        } else {
            int cb = INT_MAX;
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                if (y[i] == mt && cb == INT_MAX) cb = j + i * G;
            cbest = group_min_int<G>(cb);
            Rn = mt - h;
        }
        if (act && j == 0) {
            ring[c * RSP + (t & RMASK)] = Rn;
            if (a.write_xa) Aout[((size_t)b * (T + 1) + (dir == 0 ? t : L - t)) * C + c] = (Bc + (double)Rn) * inv_scale;
            if constexpr (VIT) a.bp[((size_t)b * (T + 1) + t) * C + c] = (uint32_t)kbest | ((uint32_t)cbest << 16);
        }

        // ---- common reference for the next position; log Z / best score at t = L
        if (c == 0) {
            float mu = NEG;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int cp = j + i * G;
                if (cp < C) mu = fmaxf(mu, u_sh[cp]);
            }
            mu = group_reduce<G>(mu, OpMax());
            if (j == 0) Hs[0] = H + (double)mu;
            if (t == L) {
                if constexpr (!VIT) {
                    float s = 0.0f;
#pragma unroll
                    for (int i = 0; i < CPL; ++i) {
                        const int cp = j + i * G;
                        if (cp < C) s += fast_exp2(u_sh[cp] - mu);
                    }
                    s = group_reduce<G>(s, OpSum());
                    if (j == 0) {
                        const double lz = (H + (double)(mu + fast_log2(s))) * inv_scale;
                        (dir == 0 ? a.logz : a.logz_b)[b] = bad ? nan_d() : lz;
                    }
                } else {
                    int cb = INT_MAX;
#pragma unroll
                    for (int i = 0; i < CPL; ++i) {
                        const int cp = j + i * G;
                        if (cp < C && u_sh[cp] == mu && cb == INT_MAX) cb = cp;
                    }
                    cb = group_min_int<G>(cb);
                    if (j == 0) {
                        a.vscore[b] = bad ? nan_d() : H + (double)mu;
                        a.vcstar[b] = cb;
                    }
                }
            }
        }

        // ---- checkpoint: ring window for the next position, base, reference
        // (only where a later span starts, i.e. t < L; span index t / delta < nspans)
        if (t == next_ck && t < L) {
            const size_t ck = ckrow + t / a.delta;
            if (act) {
#pragma unroll
                for (int i = 0; i < KPL; ++i) {
                    const int k = j + 1 + i * G;
                    if (k <= K)
                        a.ck_ring[(ck * K + (k - 1)) * C + c] = (k == 1) ? Rn : ring[c * RSP + ((t + 1 - k) & RMASK)];
                }
                if (j == 0) {
                    a.ck_base[ck * C + c] = Bc;
                    a.ck_mprev[ck * C + c] = Mprev;
                }
            }
            if (tid == 0) a.ck_href[ck] = Hs[0];
            next_ck += a.delta;
        }

        // ---- S staging: publish the next chunk, fetch the one after
        if (row == CHUNK - 1) {
            double* dst = Sbuf + ((nch + 1) & 1) * chunkN;
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                const int q = tid + i * NT;
                if (q < chunkN) dst[q] = pf[i];
            }
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                const int q = tid + i * NT;
                if (q < chunkN) {
                    const int rr = q / C, l = q - rr * C;
                    const int tt = t0 + 1 + (nch + 2) * CHUNK + rr;
                    pf[i] = (tt <= t1) ? sval(tt, l) : 0.0;
                }
            }
        }
        __syncthreads();
        H = Hs[0];
    }
}

// ------------------------------------------------------------------ configuration
static int pow2_at_least(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

SweepCfg choose_sweep(int C, int K) {
    SweepCfg s{};
    s.ok = false;
    if (C < 1 || K < 1) return s;
    int G, CPL;
    if (C <= 16) { G = 64; CPL = 1; }
    else if (C <= 32) { G = 32; CPL = 1; }
    else if (C <= 64) { G = 16; CPL = 4; }
    else if (C <= 128) { G = 8; CPL = 16; }
    else return s;
    int KPL = pow2_at_least((K + G - 1) / G);
    if (KPL > 32) return s;
    s.G = G; s.KPL = KPL; s.CPL = CPL;
    s.NT = ((C * G + 63) / 64) * 64;
    s.RS = pow2_at_least(K + 1);
    if (s.RS < 2) s.RS = 2;
    s.RSP = s.RS + (G < 32 ? G : 0);
    s.CH = CHUNK;
    s.lds_bytes = (size_t)(2 * CHUNK * C + C + 2) * 8 + (size_t)(C * s.RSP + C) * 4;
    s.ok = s.NT <= 1024 && s.lds_bytes <= 160 * 1024;
    return s;
}

template <int G, int KPL, int CPL>
static hipError_t launch_inst(bool vit, const SweepArgs& a, dim3 grid, const SweepCfg& cfg,
                              hipStream_t stream) {
    if (vit)
        hipLaunchKernelGGL((k_sweep<G, KPL, CPL, true>), grid, dim3(cfg.NT), cfg.lds_bytes, stream, a,
                           cfg.RS, cfg.RSP);
    else
        hipLaunchKernelGGL((k_sweep<G, KPL, CPL, false>), grid, dim3(cfg.NT), cfg.lds_bytes, stream, a,
                           cfg.RS, cfg.RSP);
    return hipGetLastError();
}

#define SWEEP_KPL_CASES(G, CPL)                                                      \
    switch (cfg.KPL) {                                                               \
        case 1: return launch_inst<G, 1, CPL>(viterbi, a, grid, cfg, stream);       \
        case 2: return launch_inst<G, 2, CPL>(viterbi, a, grid, cfg, stream);       \
        case 4: return launch_inst<G, 4, CPL>(viterbi, a, grid, cfg, stream);       \
        case 8: return launch_inst<G, 8, CPL>(viterbi, a, grid, cfg, stream);       \
        case 16: return launch_inst<G, 16, CPL>(viterbi, a, grid, cfg, stream);     \
        case 32: return launch_inst<G, 32, CPL>(viterbi, a, grid, cfg, stream);     \
        default: return hipErrorInvalidValue;                                        \
    }

hipError_t launch_sweep(const SweepCfg& cfg, bool viterbi, const SweepArgs& a, int ndir,
                        hipStream_t stream) {
    dim3 grid = a.mode == MODE_FULL ? dim3(a.B, ndir) : dim3(a.nspans, a.B, ndir);
    if (cfg.G == 64 && cfg.CPL == 1) { SWEEP_KPL_CASES(64, 1) }
    if (cfg.G == 32 && cfg.CPL == 1) { SWEEP_KPL_CASES(32, 1) }
    if (cfg.G == 16 && cfg.CPL == 4) { SWEEP_KPL_CASES(16, 4) }
    if (cfg.G == 8 && cfg.CPL == 16) { SWEEP_KPL_CASES(8, 16) }
    return hipErrorInvalidValue;
}

}  // namespace semicrf
