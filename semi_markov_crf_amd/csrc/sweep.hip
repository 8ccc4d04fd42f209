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
// label c (a group never straddles a wavefront), so each label's ring is private to one
// wavefront and only u[c] = alpha[t, c] - H crosses groups, through a double-buffered LDS
// row and one workgroup barrier per position.  Iteration t runs
//   [B] transition step of position t-1: C-term log-sum-exp over u(t-1)[c'] + T[c', c]
//       (DPP reduction over the GT lanes that hold c') -> ring entry A[t-1, c]
//   [C] alpha(t): three-term log-sum-exp of the k = 1, 2 terms (registers) and the bulk
//       value of k >= 3 computed two iterations earlier -> u(t)[c] to LDS
//   [D] bulk value for position t+2: K-term log-sum-exp over this label's ring
//       (lane j owns k = 3+j+i*G; DPP max, exp2, DPP sum over G lanes)
// so the long K-term reduction is off the position-to-position dependency chain.
// Arithmetic is fp32 in base 2 on values kept small: ring entries are stored relative
// to an fp64 per-label base that is moved every REBASE positions, and S enters through
// the fp64 difference S[t, c] + base[c] - H, where H is a common fp64 reference that
// every group advances by max_c u(t-1)[c].  Outputs are fp64, natural-log units.
// A checkpoint holds the state right after the transition step of position j*delta:
// the last K ring entries, the label bases, H and the rebase reference.
#include <limits.h>

#include <algorithm>

#include "common.h"
#include "internal.h"

namespace semicrf {

constexpr int REBASE = 8;      // rebase the ring every REBASE positions (global index)
constexpr int CHUNK_MAX = 64;  // positions of S staged per LDS chunk (at most)
constexpr float LIN_LO = 0x1p-100f;   // linear-space bulk sums outside [LIN_LO, LIN_HI]
constexpr float LIN_HI = 0x1p+120f;   // are recomputed in log space

__device__ __forceinline__ double nan_d() { return __longlong_as_double(0x7ff8000000000000LL); }

// Ring of the last positions of one label.  Mirrored layout (when the LDS budget allows):
// position p lives in slots (p & RMASK) and (p & RMASK) + RS, so every window of up to RS
// consecutive positions is contiguous and lane j reads its KPL terms k = 3 + j + i*G of
// the bulk for position tq at compile-time offsets from one base address.  Plain layout:
// one copy, every read masked.  Lanes whose k exceeds K read some finite slot and
// weight it by dur = NEG (log space) or 0 (linear space).
template <int G, int KPL>
__device__ __forceinline__ int ring_slot(int tq, int j, int i, int RS, bool mir) {
    return mir ? ((tq - 3) & (RS - 1)) + RS - j - i * G : (tq - 3 - j - i * G) & (RS - 1);
}

template <int G, int KPL>
__device__ __forceinline__ void ring_load(const float* row, int tq, int j, int RS, bool mir,
                                          float* v) {
    if (mir) {
        const float* w = row + (((tq - 3) & (RS - 1)) + RS - j - (KPL - 1) * G);
#pragma unroll
        for (int i = 0; i < KPL; ++i) v[i] = w[(KPL - 1 - i) * G];
    } else {
        const int t3 = tq - 3 - j;
#pragma unroll
        for (int i = 0; i < KPL; ++i) v[i] = row[(t3 - i * G) & (RS - 1)];
    }
}

// Log-space bulk value: LSE (or max) over this lane's terms, group-reduced over G lanes.
template <int G, int KPL, bool VIT>
__device__ __forceinline__ float bulk_log(const float* r, const float* dreg, int j, int* kbest) {
    float x[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) x[i] = r[i] + dreg[i];
    float m = x[0];
#pragma unroll
    for (int i = 1; i < KPL; ++i) m = fmaxf(m, x[i]);
    m = group_reduce<G>(m, OpMax());
    if constexpr (VIT) {
        int kk = INT_MAX;
#pragma unroll
        for (int i = KPL - 1; i >= 0; --i)
            if (x[i] == m) kk = 3 + j + i * G;
        *kbest = group_min_int<G>(kk);
        return m;
    } else {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < KPL; ++i) s += fast_exp2(x[i] - m);
        s = group_reduce<G>(s, OpSum());
        return m + fast_log2(s);
    }
}

// Bulk value of position tq (terms k >= 3).  Log-sum-exp with the E ring (E = 2^R):
// linear-space dot product with 2^dur, one FMA per term and one sum reduction; when the
// sum leaves [LIN_LO, LIN_HI] (underflow, overflow, inf, NaN) the exact log-space form
// over the R ring is used instead.
template <int G, int KPL, bool VIT>
__device__ __forceinline__ float bulk_value(const float* Rrow, const float* Erow, int tq, int j,
                                            int RS, bool mir, bool lin, const float* dreg,
                                            const float* dlin, int* kbest) {
    if constexpr (KPL == 0) {
        *kbest = INT_MAX;
        return NEG;
    } else {
        float v[KPL];
        if constexpr (!VIT) {
            if (lin) {
                ring_load<G, KPL>(Erow, tq, j, RS, mir, v);
                float s = 0.0f;
#pragma unroll
                for (int i = 0; i < KPL; ++i) s = fmaf(v[i], dlin[i], s);
                s = group_reduce<G>(s, OpSum());
                if (s >= LIN_LO && s <= LIN_HI) return fast_log2(s);
            }
        }
        ring_load<G, KPL>(Rrow, tq, j, RS, mir, v);
        return bulk_log<G, KPL, VIT>(v, dreg, j, kbest);
    }
}

// Move every live slot this lane owns (k = 3 + j + i*G <= K + 1 for the bulk of tq, in
// both mirror copies) by -by; E follows as 2^R.
template <int G, int KPL, bool VIT>
__device__ __forceinline__ void rebase_ring(float* Rrow, float* Erow, int tq, int j, int RS,
                                            bool mir, bool lin, float by, int K) {
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        if (3 + j + i * G <= K + 1) {
            const int s0 = ring_slot<G, KPL>(tq, j, i, RS, mir);
            const float r = Rrow[s0] - by;
            Rrow[s0] = r;
            const int s1 = s0 >= RS ? s0 - RS : s0 + RS;
            if (mir) Rrow[s1] = r;
            if (!VIT && lin) {
                const float e = fast_exp2(r);
                Erow[s0] = e;
                if (mir) Erow[s1] = e;
            }
        }
    }
}

// G: lanes per label; KPL: durations k >= 3 per lane (k = 3 + j + i*G, i < KPL, covering
// k <= K + 1); CPL, GT: previous labels per lane and the lane count of the transition
// reduction (GT * CPL >= C, GT <= G); NTMAX: largest workgroup routed here.
template <int G, int KPL, int CPL, int GT, int NTMAX, bool VIT>
__global__ __launch_bounds__(NTMAX) void k_sweep(const SweepArgs a, const int RS, const int P,
                                                const int CH, const int layout) {
    constexpr int PF = (CHUNK_MAX + G - 1) / G;   // prefetched doubles per lane (NT >= C*G)
    constexpr int UP = GT * CPL;                   // padded u row (>= C)
    extern __shared__ double lds[];
    const int C = a.C, K = a.K, T = a.T;
    const int tid = threadIdx.x, NT = blockDim.x;
    const int c = tid / G;
    const int j = tid - c * G;
    const int jt = j & (GT - 1);             // every GT-subgroup repeats the transition step
    const bool act = c < C;
    const int cr = act ? c : C;              // inactive lanes use the spare LDS row C

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
    const int chunkN = CH * C;
    const bool mir = layout & SWEEP_MIRRORED;
    const bool lin = !VIT && (layout & SWEEP_LINEAR);

    double* Sbuf = lds;                                  // [2][CH][C]
    double* SL = Sbuf + 2 * chunkN;                      // [C]
    float* R = (float*)(SL + C);                         // [C+1][P]
    float* E = R + (C + 1) * P;                          // [C+1][P]   (linear space only)
    float* u_sh = E + (lin ? (C + 1) * P : 0);           // [2][UP]
    float* Rrow = R + cr * P;
    float* Erow = E + cr * P;

    const double* Sb = a.S + (size_t)b * (T + 1) * C;
    for (int q = tid; q < C; q += NT) SL[q] = Sb[(size_t)L * C + q];
    for (int q = tid; q < (C + 1) * P; q += NT) {
        R[q] = NEG;
        if (lin) E[q] = 0.0f;
    }
    for (int q = tid; q < 2 * UP; q += NT) u_sh[q] = NEG;

    // durations (k >= 3 per lane; k = 1, 2 group-uniform) and transitions, base 2
    auto durv = [&](int k) -> float {
        return (act && k <= K) ? fmaxf((float)((double)a.dur[(k - 1) * C + c] * scale), NEG) : NEG;
    };
    float dreg[KPL > 0 ? KPL : 1], dlin[KPL > 0 ? KPL : 1];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        dreg[i] = durv(3 + j + i * G);
        dlin[i] = dreg[i] > NEG_HALF ? fast_exp2(dreg[i]) : 0.0f;
    }
    const float d0 = durv(1), d1 = durv(2);
    float treg[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int cp = jt + i * GT;
        float v = NEG;
        if (act && cp < C) {
            const float tv = dir == 0 ? a.trans[cp * C + c] : a.trans[c * C + cp];
            v = fmaxf((float)((double)tv * scale), NEG);
        }
        treg[i] = v;
    }
    __syncthreads();   // ring and u cleared, SL visible

    auto put = [&](int pos, float r) {       // ring entry of position pos, both copies
        const int s0 = pos & RMASK;
        Rrow[s0] = r;
        if (mir) Rrow[s0 + RS] = r;
        if (lin) {
            const float e = fast_exp2(r);
            Erow[s0] = e;
            if (mir) Erow[s0 + RS] = e;
        }
    };

    // ---------------------------------------------------------------- state after trans(t0)
    const size_t ckrow = ((size_t)dir * a.B + b) * a.nspans;
    double Bc = 0.0, H = 0.0;
    float Mref = 0.0f, Rn1, Rn2;
    double* Xout = dir == 0 ? a.XF : a.XB;
    double* Aout = dir == 0 ? a.AF : a.AB;
    if (t0 == 0) {
        if (act && j == 0) put(0, 0.0f);        // position 0: no transition into it
        Rn1 = 0.0f;
        Rn2 = NEG;
    } else {
        const size_t ck = ckrow + span;
        if (act)
            for (int q = j; q < K; q += G) put(t0 - q, a.ck_ring[(ck * K + q) * C + c]);
        const int cc = act ? c : 0;
        Bc = a.ck_base[ck * C + cc];
        Mref = a.ck_mprev[ck * C + cc];
        H = a.ck_href[ck];
        Rn1 = a.ck_ring[(ck * K + 0) * C + cc];
        Rn2 = K >= 2 ? a.ck_ring[(ck * K + 1) * C + cc] : NEG;
    }
    if (act && j == 0 && a.write_xa)
        Aout[((size_t)b * (T + 1) + (dir == 0 ? t0 : L - t0)) * C + c] = (Bc + (double)Rn1) * inv_scale;
    __syncthreads();   // restored ring visible

    int kQa = 0, kQb = 0, kb_prev = 0;
    float Qa = bulk_value<G, KPL, VIT>(Rrow, Erow, t0 + 1, j, RS, mir, lin, dreg, dlin, &kQa);
    float Qb = bulk_value<G, KPL, VIT>(Rrow, Erow, t0 + 2, j, RS, mir, lin, dreg, dlin, &kQb);

    // ---------------------------------------------------------------- S staging
    auto sidx = [&](int t, int q) -> size_t { return (size_t)(dir == 0 ? t : L - t) * C + q; };
    auto spub = [&](double raw, int q) -> double {
        return dir == 0 ? raw * scale : (SL[q] - raw) * scale;
    };
    for (int q = tid; q < chunkN; q += NT) {
        const int row = q / C, l = q - row * C;
        const int t = t0 + 1 + row;
        Sbuf[q] = (t <= t1) ? spub(Sb[sidx(t, l)], l) : 0.0;
    }
    // the chunk after: raw values in registers, published CH positions later
    double pf[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const int q = tid + i * NT;
        pf[i] = 0.0;
        if (q < chunkN) {
            const int row = q / C, l = q - row * C;
            const int t = t0 + 1 + CH + row;
            if (t <= t1) pf[i] = Sb[sidx(t, l)];
        }
    }
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0);   // nothing loaded before the loop is waited on inside it

    int next_ck = (a.mode == MODE_FULL && a.write_ckpt) ? a.delta : INT_MAX;
    float h_prev = 0.0f;
    const size_t outrow = (size_t)b * (T + 1);

    // ---------------------------------------------------------------- main loop
    // iteration t: [B] transition step of position t-1 (needs every label's u(t-1));
    // [C] alpha(t) from the k = 1, 2 terms and the bulk value of t -> u(t);
    // [D] bulk value of position t+2 from this label's ring.  One barrier per position.
    for (int tc = t0 + 1, nch = 0; tc <= t1; tc += CH, ++nch) {
        const double* Srow = Sbuf + (nch & 1) * chunkN;
        const int rows = min(CH, t1 - tc + 1);
        for (int row = 0; row < rows; ++row) {
            const int t = tc + row;
            if (t > t0 + 1) {
                // ---- [B] A(t-1) = LSE_{c'} (u(t-1)[c'] + T[c'][c]) - h(t-1); H(t)
                const float* us = u_sh + ((t - 1) & 1) * UP;
                float y[CPL], uv[CPL];
                float mt, mu;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    uv[i] = us[jt + i * GT];
                    y[i] = uv[i] + treg[i];
                }
                mt = y[0];
                mu = uv[0];
#pragma unroll
                for (int i = 1; i < CPL; ++i) {
                    mt = fmaxf(mt, y[i]);
                    mu = fmaxf(mu, uv[i]);
                }
                mt = group_reduce<GT>(mt, OpMax());
                mu = group_reduce<GT>(mu, OpMax());
                float Rnew;
                int cbest = 0;
                if constexpr (!VIT) {
                    float st = 0.0f;
#pragma unroll
                    for (int i = 0; i < CPL; ++i) st += fast_exp2(y[i] - mt);
                    st = group_reduce<GT>(st, OpSum());
                    Rnew = mt + fast_log2(st) - h_prev;
                } else {
                    int cb = INT_MAX;
#pragma unroll
                    for (int i = CPL - 1; i >= 0; --i)
                        if (y[i] == mt) cb = jt + i * GT;
                    cbest = group_min_int<GT>(cb);
                    Rnew = mt - h_prev;
                }
                H += (double)mu;
                Rn2 = Rn1;
                Rn1 = Rnew;
                if (j == 0) {
                    put(t - 1, Rnew);
                    if (act && a.write_xa)
                        Aout[(outrow + (dir == 0 ? t - 1 : L - t + 1)) * C + c] =
                            (Bc + (double)Rnew) * inv_scale;
                    if constexpr (VIT) {
                        if (act) a.bp[(outrow + t - 1) * C + c] = (uint32_t)kb_prev | ((uint32_t)cbest << 16);
                    }
                }
                // ---- checkpoint: state after the transition step of position t-1
                if (t - 1 == next_ck) {
                    const size_t ck = ckrow + (t - 1) / a.delta;
                    if (act)
                        for (int q = j; q < K; q += G)
                            a.ck_ring[(ck * K + q) * C + c] = Rrow[(t - 1 - q) & RMASK];
                    if (act && j == 0) {
                        a.ck_base[ck * C + c] = Bc;
                        a.ck_mprev[ck * C + c] = Mref;
                    }
                    if (tid == 0) a.ck_href[ck] = H;
                    next_ck += a.delta;
                }
            }

            // ---- [C] alpha(t): k = 1, 2 from registers, k >= 3 from the bulk value
            const float e1 = Rn1 + d0, e2 = Rn2 + d1;
            const float m3 = fmaxf(fmaxf(Qa, e1), e2);
            float sig;
            if constexpr (!VIT) {
                sig = m3 + fast_log2(fast_exp2(Qa - m3) + fast_exp2(e1 - m3) + fast_exp2(e2 - m3));
            } else {
                sig = m3;
                kb_prev = (e1 == m3) ? 1 : (e2 == m3) ? 2 : kQa;
            }
            const double g = Srow[row * C + (act ? c : 0)] + Bc;
            const float h = (float)(g - H);
            if (j == 0) {
                u_sh[(t & 1) * UP + cr] = h + sig;
                if (act && a.write_xa)
                    Xout[(outrow + (dir == 0 ? t : L - t)) * C + c] = (g + (double)sig) * inv_scale;
            }
            h_prev = h;

            // ---- [D] rebase, then the bulk value for position t+2
            if ((t & (REBASE - 1)) == 0) {
                const float ref = fmaxf(Mref, Rn1);
                const float dl = ref > NEG_HALF ? ref : 0.0f;
                Bc += (double)dl;
                Qb -= dl;
                Rn1 -= dl;
                Rn2 -= dl;
                h_prev += dl;
                rebase_ring<G, KPL, VIT>(Rrow, Erow, t + 2, j, RS, mir, lin, dl, K);
            }
            int kQn = 0;
            const float Qn = bulk_value<G, KPL, VIT>(Rrow, Erow, t + 2, j, RS, mir, lin, dreg, dlin, &kQn);
            if (Qn > NEG_HALF) Mref = Qn;
            Qa = Qb;
            Qb = Qn;
            kQa = kQb;
            kQb = kQn;
            __syncthreads();
        }
        // ---- S staging: publish the next chunk, fetch the one after
        if (tc + CH <= t1) {
            double* dst = Sbuf + ((nch + 1) & 1) * chunkN;
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                const int q = tid + i * NT;
                if (q < chunkN) dst[q] = spub(pf[i], q - (q / C) * C);
            }
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                const int q = tid + i * NT;
                if (q < chunkN) {
                    const int rr = q / C, l = q - rr * C;
                    const int tt = tc + 2 * CH + rr;
                    pf[i] = (tt <= t1) ? Sb[sidx(tt, l)] : 0.0;
                }
            }
            __syncthreads();
        }
    }

    // ---------------------------------------------------------------- end of sequence
    if (t1 == L) {
        const float* us = u_sh + (L & 1) * UP;
        if constexpr (VIT) {
            if (act && j == 0) a.bp[(outrow + L) * C + c] = (uint32_t)kb_prev;
        }
        if (c == 0) {
            float mu = NEG;
#pragma unroll
            for (int i = 0; i < CPL; ++i) mu = fmaxf(mu, us[jt + i * GT]);
            mu = group_reduce<GT>(mu, OpMax());
            if constexpr (!VIT) {
                float s = 0.0f;
#pragma unroll
                for (int i = 0; i < CPL; ++i) s += fast_exp2(us[jt + i * GT] - mu);
                s = group_reduce<GT>(s, OpSum());
                if (j == 0) {
                    const double lz = (H + (double)(mu + fast_log2(s))) * inv_scale;
                    (dir == 0 ? a.logz : a.logz_b)[b] = bad ? nan_d() : lz;
                }
            } else {
                int cb = INT_MAX;
#pragma unroll
                for (int i = CPL - 1; i >= 0; --i)
                    if (us[jt + i * GT] == mu) cb = jt + i * GT;
                cb = group_min_int<GT>(cb);
                if (j == 0) {
                    a.vscore[b] = bad ? nan_d() : H + (double)mu;
                    a.vcstar[b] = cb;
                }
            }
        }
    }
}

// ------------------------------------------------------------------ configuration
static int pow2_at_least(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

static size_t sweep_lds(int C, int P, int CH, int UP, bool lin) {
    return (size_t)(2 * CH * C + C) * 8 + (size_t)((lin ? 2 : 1) * (C + 1) * P + 2 * UP) * 4;
}

// Largest S chunk (64 down to 8 positions) that keeps the workgroup's LDS under 150 KB.
static int fit_chunk(int C, int P, int UP, bool lin) {
    for (int ch = CHUNK_MAX; ch >= 8; ch >>= 1)
        if (sweep_lds(C, P, ch, UP, lin) <= 150 * 1024) return ch;
    return 0;
}

SweepCfg choose_sweep(int C, int K) {
    SweepCfg s{};
    s.ok = false;
    if (C < 1 || K < 1) return s;
    // lane groups: aim at <= 4 waves (one per SIMD) where the label count allows
    int G, CPL, GT;
    if (C <= 4) { G = 64; GT = 4; CPL = 1; }
    else if (C <= 8) { G = 32; GT = 8; CPL = 1; }
    else if (C <= 16) { G = 16; GT = 16; CPL = 1; }
    else if (C <= 32) { G = 8; GT = 8; CPL = 4; }
    else if (C <= 64) { G = 8; GT = 8; CPL = 8; }
    else if (C <= 128) { G = 4; GT = 4; CPL = 32; }
    else return s;
    // lanes cover k = 3 .. K+1: the bulk terms plus one more slot kept in the current base
    const int kpl = K > 1 ? (K - 1 + G - 1) / G : 0;
    static const int kInst[] = {0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16, 24, 32};
    int kmax = -1;
    for (int v : kInst)
        if (v >= kpl) { kmax = v; break; }
    if (kmax < 0) return s;
    s.G = G; s.KPL = kmax; s.CPL = CPL; s.GT = GT; s.kpl = kpl;
    s.NT = ((C * G + 63) / 64) * 64;
    // RS >= K + 2 live positions and >= the widest window a lane addresses (2 + KPL*G)
    s.RS = pow2_at_least(std::max(K + 2, 3 + kmax * G));
    const int pad = G < 32 ? G : 0;   // staggers the label rows over the LDS banks
    const int UP = GT * CPL;
    // layouts in order of preference while they fit: mirrored + linear, plain + linear,
    // plain + log-space only
    static const int pref[] = {SWEEP_MIRRORED | SWEEP_LINEAR, SWEEP_LINEAR, 0};
    for (int lay : pref) {
        const int P = ((lay & SWEEP_MIRRORED) ? 2 : 1) * s.RS + pad;
        const int ch = fit_chunk(C, P, UP, lay & SWEEP_LINEAR);
        if (ch == 0) continue;
        s.layout = lay; s.RSP = P; s.CH = ch;
        s.lds_bytes = sweep_lds(C, P, ch, UP, lay & SWEEP_LINEAR);
        // the max-plus sweep keeps no E ring
        s.lds_bytes_vit = sweep_lds(C, P, ch, UP, false);
        s.ok = s.NT <= 1024;
        return s;
    }
    return s;
}

template <int G, int KPL, int CPL, int GT, int NTMAX>
static hipError_t launch_inst(bool vit, const SweepArgs& a, dim3 grid, const SweepCfg& cfg,
                              hipStream_t stream) {
    if (cfg.NT > NTMAX) return hipErrorInvalidValue;
    if (vit)
        hipLaunchKernelGGL((k_sweep<G, KPL, CPL, GT, NTMAX, true>), grid, dim3(cfg.NT),
                           cfg.lds_bytes_vit, stream, a, cfg.RS, cfg.RSP, cfg.CH, cfg.layout);
    else
        hipLaunchKernelGGL((k_sweep<G, KPL, CPL, GT, NTMAX, false>), grid, dim3(cfg.NT),
                           cfg.lds_bytes, stream, a, cfg.RS, cfg.RSP, cfg.CH, cfg.layout);
    return hipGetLastError();
}

// NTMAX = G * (largest label count routed to the instance)
#define SWEEP_KPL_CASES(G, CPL, GT, NTMAX)                                                   \
    switch (cfg.KPL) {                                                                       \
        case 0: return launch_inst<G, 0, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);    \
        case 1: return launch_inst<G, 1, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);    \
        case 2: return launch_inst<G, 2, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);    \
        case 3: return launch_inst<G, 3, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);    \
        case 4: return launch_inst<G, 4, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);    \
        case 5: return launch_inst<G, 5, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);    \
        case 6: return launch_inst<G, 6, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);    \
        case 7: return launch_inst<G, 7, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);    \
        case 8: return launch_inst<G, 8, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);    \
        case 10: return launch_inst<G, 10, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);  \
        case 12: return launch_inst<G, 12, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);  \
        case 16: return launch_inst<G, 16, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);  \
        case 24: return launch_inst<G, 24, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);  \
        case 32: return launch_inst<G, 32, CPL, GT, NTMAX>(viterbi, a, grid, cfg, stream);  \
        default: return hipErrorInvalidValue;                                                \
    }

hipError_t launch_sweep(const SweepCfg& cfg, bool viterbi, const SweepArgs& a, int ndir,
                        hipStream_t stream) {
    dim3 grid = a.mode == MODE_FULL ? dim3(a.B, ndir) : dim3(a.nspans, a.B, ndir);
    if (cfg.G == 64) { SWEEP_KPL_CASES(64, 1, 4, 256) }
    if (cfg.G == 32) { SWEEP_KPL_CASES(32, 1, 8, 256) }
    if (cfg.G == 16) { SWEEP_KPL_CASES(16, 1, 16, 256) }
    if (cfg.G == 8 && cfg.CPL == 4) { SWEEP_KPL_CASES(8, 4, 8, 256) }
    if (cfg.G == 8 && cfg.CPL == 8) { SWEEP_KPL_CASES(8, 8, 8, 512) }
    if (cfg.G == 4) { SWEEP_KPL_CASES(4, 32, 4, 512) }
    return hipErrorInvalidValue;
}

}  // namespace semicrf
