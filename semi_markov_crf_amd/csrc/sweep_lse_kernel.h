// Log-semiring streaming sweep on gfx950: forward (alpha) and backward (beta, run as a
// forward sweep over the mirrored sequence), with checkpoints or per-position outputs.
//
// Method ("Streaming Structured Inference with Flash-SemiCRF", gist.science EN explainer,
// "2. Methodology"): segment potentials S[s+k,c] - S[s,c] + dur[k-1,c] + trans[c',c] are
// evaluated on the fly from the prefix sums; only a ring of the last K messages per label
// is kept ("Streaming Forward-Backward with Ring Buffers"); the ring and the cumulative
// normaliser are written out every delta positions and a later pass restarts from them
// ("Checkpointing").
//
// Factored recurrence (exact: the potential is a sum of a (start, length, label) term and
// a (previous label, label) term):
//     abar[s, c]  = LSE_{c'} (alpha[s, c'] + trans[c', c])                  (C^2 terms)
//     alpha[t, c] = S[t, c] + LSE_k (abar[t-k, c] - S[t-k, c] + dur[k-1, c])    (K*C terms)
// with abar[0, c] = 0 (no transition into the first segment).  The ring holds
// A[s, c] = abar[s, c] - S[s, c].  The backward sweep runs the same recurrence on the
// reversed sequence: S'[t] = S[L] - S[L-t], trans' = trans^T; its "alpha" is beta_bar[s, c]
// and its "A" is beta[u, c] + S[u, c] - S[L, c].
//
// Work layout: one workgroup per (sequence, direction), or per (checkpoint span, sequence,
// direction) for the recompute.  Lanes form groups of G per label; a group never straddles
// a wavefront, so each label's ring is private to one wavefront.  Only the per-label
// message of the newest position crosses groups, through a double-buffered LDS row and one
// workgroup barrier per position.
//
// Arithmetic: base 2, fp32, mostly in LINEAR space.  Every value is kept relative to a
// reference: ring entries R = A - B_c (per-label fp64 base B_c, moved every REBASE
// positions) with E = 2^R alongside; messages p[c] = 2^(alpha[t, c] - H) relative to a
// common fp64 reference H that all groups advance by the same power of two (the exponent
// of sum_c p).  The steps of position t are then
//   [C] combine   sig = E(t-1) 2^d0 + E(t-2) 2^d1 + Q(t)           (2 FMAs)
//       message   p(t) = sig * 2^(S[t] + B_c - H(t-1) + dmax) * 2^-e  (2 multiplies)
//   [D] bulk      Q(t+2) = sum_k E(t+2-k) 2^(dur[k-1] - dmax)      (one FMA per term)
//   [B] transition s = sum_c' p(t)[c'] 2^(trans[c', c] - tmax)      -> E(t), R(t)
// so the chain from one barrier to the next holds a handful of FMAs and one DPP sum, and
// the logarithms (R, the log-space copy of each message) are off it.  Every linear sum is
// range-checked: outside [LIN_LO, LIN_HI] (underflow, overflow, inf, NaN, forbidden
// transitions or durations) that step is recomputed exactly in log space from R and from
// the log-space messages, so the result never depends on the linear path being in range.
// Outputs are fp64, natural-log units.
#pragma once

#include "internal.h"
#include "ring.h"

namespace semicrf {

namespace {

constexpr float LIN_LO = 0x1p-60f;   // linear sums are trusted inside [LIN_LO, LIN_HI]:
constexpr float LIN_HI = 0x1p+60f;   // terms lost to fp32 underflow are then < 2^-66 of it

__device__ __forceinline__ double nan_d() { return __longlong_as_double(0x7ff8000000000000LL); }
// Range test on the bit pattern: false for 0, denormals, negatives, inf and NaN whatever
// the floating-point flags of the build.
__device__ __forceinline__ bool in_lin_range(float s) {
    constexpr uint32_t lo = __builtin_bit_cast(uint32_t, LIN_LO);
    constexpr uint32_t hi = __builtin_bit_cast(uint32_t, LIN_HI);
    return __float_as_uint(s) - lo <= hi - lo;
}
__device__ __forceinline__ float exp2_or_zero(float x) { return x > NEG_HALF ? fast_exp2(x) : 0.0f; }
// 2^x for an fp64 exponent, to about the accuracy of the hardware exp2 (a few 1e-8
// relative): the exponent is rounded to fp32 for exp2 and the part it dropped, x - fl(x),
// enters to first order, 2^(x - fl(x)) = 1 + (x - fl(x)) ln 2.  Rounding the exponent alone
// would cost up to half an ulp of |x|, about 1e-6 for |x| near 16, at every use.
__device__ __forceinline__ float exp2_d(double x) {
    const float xf = (float)x;
    const float lo = (float)(x - (double)xf);
    const float e = fast_exp2(xf);
    return fmaf(e, lo * 0.69314718f, e);
}
// 2^-n for a whole number n (a rebase shift), exactly (0 below the fp32 range)
__device__ __forceinline__ float pow2_neg(float n) {
    return __builtin_amdgcn_ldexpf(1.0f, -(int)fminf(fmaxf(n, -1.0e9f), 1.0e9f));
}
// true in every lane when any lane of the wavefront has `bad` set (a scalar branch)
__device__ __forceinline__ bool wave_any(bool bad) { return __builtin_amdgcn_ballot_w64(bad) != 0; }

}  // namespace

// G: lanes per label; KPL: durations k >= 3 per lane (k = 3 + j + i*G, i < KPL, covering
// k <= K + 1); CPL, GT: previous labels per lane and the lane count of the transition
// reduction (GT * CPL >= C, GT <= G); NTMAX: largest workgroup routed here.
//
// Loop iteration t (between the barriers that publish the messages of t and of t+1):
//   rebase (every REBASE positions)
//   [B] transition step of position t  ||  [D] bulk sum of position t+2
//   (one scalar branch: exact log-space redo of any of the three sums out of range)
//   ring entry of t, normaliser update, checkpoint
//   [C] message of position t+1 from E(t), E(t-1), bulk(t+1); publish
// LAY: ring layout bits (SWEEP_MIRRORED, SWEEP_LINEAR), fixed at compile time.
template <int G, int KPL, int CPL, int GT, int NTMAX, int LAY>
__global__ __launch_bounds__(NTMAX) void k_lse(const SweepArgs a, const int RS, const int P,
                                              const int CH,
                                              const float* __restrict__ proj_start,
                                              const float* __restrict__ proj_end) {
    constexpr int PF = (lse_chunk_max(G) + 1 + G - 1) / G;   // prefetched doubles per lane
    constexpr int UP = GT * CPL;                               // padded message row (>= C)
    constexpr int KP = KPL > 0 ? KPL : 1;
    extern __shared__ double lds[];
    const int C = a.C, K = a.K, T = a.T;
    const int tid = threadIdx.x, NT = blockDim.x;
    const int c = tid / G;
    const int j = tid - c * G;
    const int jt = j & (GT - 1);             // every GT-subgroup repeats the transition step
    const bool act = c < C;
    const int cr = act ? c : C;              // inactive lanes use the spare ring row C
    const int cc = act ? c : 0;
    const bool writer = act && j == 0;       // one lane per label publishes

    // MODE_SPEC: grid (nspans, B, ndir); MODE_REPAIR: grid (B, ndir)
    const bool spec = a.mode == MODE_SPEC;
    int b, span, dir;
    if (spec) {
        span = blockIdx.x; b = blockIdx.y; dir = blockIdx.z;
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
    // seam windows (MODE_SPEC): head [hlo, tout] of every span but the first, tail [tlo, t1]
    // of every span but the last
    const int hlo = (spec && span > 0) ? tout - K + 1 : INT_MAX;
    const int tlo = (spec && t1 < L) ? t1 - K + 1 : INT_MAX;
    const size_t winrow = (((size_t)dir * a.B + b) * a.nspans + span) * K;
    auto window = [&](int t, double av) {                 // writer lanes
        if (t >= hlo && t <= tout) a.head[(winrow + t - hlo) * C + c] = av;
        if (t >= tlo && t <= t1) a.tail[(winrow + t - tlo) * C + c] = av;
    };
    const int RMASK = RS - 1;
    const int rowsN = (CH + 1) * C;           // staged S values per chunk and side
    constexpr bool MIR = LAY & SWEEP_MIRRORED;
    constexpr bool LIN = LAY & SWEEP_LINEAR;

    // end side S(p) + pe(p) and start side S(p) - ps(p) (projections, base 2):
    // [2 chunks][2 sides][CH+1][C]
    double* Sbuf = lds;
    double* SL = Sbuf + 4 * rowsN;                        // [C]
    float* R = (float*)(SL + C);                          // [C+1][P]
    float* E = R + (C + 1) * P;                           // [C+1][P] (linear bulk only)
    float* p_sh = E + (LIN ? (C + 1) * P : 0);            // [2][UP] messages, linear
    float* u_sh = p_sh + 2 * UP;                          // [2][UP] messages, log2
    float* dummy = u_sh + 2 * UP;                         // [NT] sink for non-publishing lanes
    float* Rrow = R + cr * P;
    float* Erow = E + cr * P;

    const double* Sb = a.S + (size_t)b * (T + 1) * C;
    for (int q = tid; q < C; q += NT) SL[q] = Sb[(size_t)L * C + q];
    // projections of sweep position p, base 2: end side (segments ending at p) and start
    // side (segments starting at p); 0 without projections or outside [1, L] / [0, L-1]
    const float* PSb = proj_start ? proj_start + (size_t)b * T * C : nullptr;
    const float* PEb = proj_end ? proj_end + (size_t)b * T * C : nullptr;
    auto proj_e = [&](int p, int q) -> double {
        const float* src = dir == 0 ? PEb : PSb;
        const int t = dir == 0 ? p - 1 : L - p;
        return (src && p >= 1 && p <= L) ? (double)src[(size_t)t * C + q] * LOG2E : 0.0;
    };
    auto proj_s = [&](int p, int q) -> double {
        const float* src = dir == 0 ? PSb : PEb;
        const int t = dir == 0 ? p : L - 1 - p;
        return (src && p >= 0 && p < L) ? (double)src[(size_t)t * C + q] * LOG2E : 0.0;
    };
    for (int q = tid; q < (C + 1) * P; q += NT) {
        R[q] = NEG;
        if constexpr (LIN) E[q] = 0.0f;
    }
    for (int q = tid; q < 2 * UP; q += NT) {
        p_sh[q] = 0.0f;
        u_sh[q] = NEG;
    }

    // ---------------------------------------------------------------- constants, base 2
    auto durv = [&](int k) -> float {
        return (act && k <= K) ? fmaxf((float)((double)a.dur[(k - 1) * C + c] * LOG2E), NEG) : NEG;
    };
    float dreg[KP], dlin[KP];
    float dmx = NEG;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        dreg[i] = durv(3 + j + i * G);
        dmx = fmaxf(dmx, dreg[i]);
    }
    const float d0 = durv(1), d1 = durv(2);
    dmx = group_reduce<G>(fmaxf(dmx, fmaxf(d0, d1)), OpMax());
    const float dmax = dmx > NEG_HALF ? dmx : 0.0f;      // linear durations are 2^(dur - dmax)
#pragma unroll
    for (int i = 0; i < KPL; ++i) dlin[i] = exp2_or_zero(dreg[i] - dmax);
    const float D0 = exp2_or_zero(d0 - dmax), D1 = exp2_or_zero(d1 - dmax);

    float treg[CPL], wreg[CPL], zero[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int cp = jt + i * GT;
        float v = NEG;
        if (act && cp < C) {
            const float tv = dir == 0 ? a.trans[cp * C + c] : a.trans[c * C + cp];
            v = fmaxf((float)((double)tv * LOG2E), NEG);
        }
        treg[i] = v;
        zero[i] = 0.0f;
    }
    // linear transitions 2^(trans - tmax) with one tmax over the whole matrix, so that both
    // sweep directions multiply by bit-identical weights (block-wide max through the sink)
    float tmx = NEG;
    for (int q = tid; q < C * C; q += NT) tmx = fmaxf(tmx, fmaxf((float)((double)a.trans[q] * LOG2E), NEG));
    dummy[tid] = tmx;
    __syncthreads();
    for (int q = 0; q < NT; ++q) tmx = fmaxf(tmx, dummy[q]);
    __syncthreads();
    const float tmax = tmx > NEG_HALF ? tmx : 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) wreg[i] = exp2_or_zero(treg[i] - tmax);
    __syncthreads();   // ring and messages cleared, SL visible

    // bulk of position tq: linear sum (dlin weights) when in range, else exact log space
    auto bulk = [&](int tq, float& qlin, float& qlog) {
        qlin = 0.0f;
        qlog = NEG;
        if constexpr (KPL > 0) {
            float v[KP];
            bool ok = false;
            if constexpr (LIN) {
                ring_load<G, KPL, MIR>(Erow, tq, j, RS, v);
                float sm = 0.0f;
#pragma unroll
                for (int i = 0; i < KPL; ++i) sm = fmaf(v[i], dlin[i], sm);
                sm = group_reduce<G>(sm, OpSum());
                ok = in_lin_range(sm) || !act;
                qlin = sm;
                qlog = fast_log2(sm) + dmax;
            }
            if (wave_any(!ok)) {
                ring_load<G, KPL, MIR>(Rrow, tq, j, RS, v);
                const float lg = group_lse<G, KPL>(v, dreg);
                if (!ok) {
                    qlog = lg;
                    qlin = exp2_or_zero(lg - dmax);
                }
            }
        }
    };

    // ---------------------------------------------------------------- state after trans(t0)
    const size_t ckrow = ((size_t)dir * a.B + b) * a.nspans;
    const size_t outrow = (size_t)b * (T + 1);
    double* Xout = dir == 0 ? a.XF : a.XB;
    auto put_all = [&](int pos, float r) {   // every ring copy of one position
        ring_put<MIR>(Rrow, pos, RS, r);
        if constexpr (LIN) ring_put<MIR>(Erow, pos, RS, exp2_or_zero(r));
    };
    double Bc = 0.0, H = 0.0;
    float Mref = 0.0f, Rn1, Rn2;
    if (t0 == 0) {
        // position 0: no transition into it; the ring entry is its start-side projection
        Rn1 = act ? fmaxf((float)proj_s(0, c), NEG) : 0.0f;
        if (writer) put_all(0, Rn1);
        Rn2 = NEG;
    } else if (spec) {
        // burn-in start: every ring entry of positions t0-K+1 .. t0 equal (0 in log2)
        if (act)
            for (int q = j; q < K && t0 - q >= 0; q += G) put_all(t0 - q, 0.0f);
        Rn1 = 0.0f;
        Rn2 = (K >= 2 && t0 >= 1) ? 0.0f : NEG;
    } else {
        const size_t ck = ckrow + span;
        if (act)
            for (int q = j; q < K; q += G) put_all(t0 - q, a.ck_ring[(ck * K + q) * C + c]);
        Bc = a.ck_base[ck * C + cc];
        Mref = a.ck_mprev[ck * C + cc];
        H = a.ck_href[ck];
        Rn1 = a.ck_ring[(ck * K + 0) * C + cc];
        Rn2 = K >= 2 ? a.ck_ring[(ck * K + 1) * C + cc] : NEG;
    }
    if (writer && t0 == 0)   // window positions <= 0: position 0's value, nothing before it
        for (int p = min(hlo, tlo); p <= 0; ++p) window(p, p == 0 ? (Bc + (double)Rn1) * LN2 : -1.0e300);
    float En1 = exp2_or_zero(Rn1), En2 = exp2_or_zero(Rn2);

    // ---------------------------------------------------------------- S staging
    auto sidx = [&](int t, int q) -> size_t { return (size_t)(dir == 0 ? t : L - t) * C + q; };
    auto spub = [&](double raw, int q) -> double {
        return dir == 0 ? raw * LOG2E : (SL[q] - raw) * LOG2E;
    };
    // chunk n holds rows t = t0 + 1 + n*CH + r, r = 0..CH (the last row repeats the next
    // chunk's first, so position t+1 is always at hand)
    for (int q = tid; q < rowsN; q += NT) {
        const int row = q / C, l = q - row * C;
        const int t = t0 + 1 + row;
        const double sv = (t <= t1) ? spub(Sb[sidx(t, l)], l) : 0.0;
        Sbuf[q] = (t <= t1) ? sv + proj_e(t, l) : 0.0;
        Sbuf[rowsN + q] = (t <= t1) ? sv - proj_s(t, l) : 0.0;
    }
    double pf[PF];   // raw values of chunk n+1, fetched one chunk ahead
    float pfe[PF], pfs[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const int q = tid + i * NT;
        pf[i] = 0.0;
        pfe[i] = pfs[i] = 0.0f;
        if (q < rowsN) {
            const int row = q / C, l = q - row * C;
            const int t = t0 + 1 + CH + row;
            if (t <= t1) {
                pf[i] = Sb[sidx(t, l)];
                pfe[i] = (float)proj_e(t, l);
                pfs[i] = (float)proj_s(t, l);
            }
        }
    }
    __syncthreads();   // restored ring and chunk 0 visible
    __builtin_amdgcn_s_waitcnt(0);   // nothing loaded before the loop is waited on inside it

    // ---------------------------------------------------------------- message of t0+1
    float Qla, Qga;           // bulk of the next message's position (linear, log2)
    bulk(t0 + 1, Qla, Qga);
    double BH = Bc - H;       // B_c - H
    double Scur = Sbuf[rowsN + cc];   // start side of t0+1, base 2
    float rps = 1.0f;         // 2^-e of the last normaliser step
    auto publish = [&](int tn, double Sn, float z, float ql, float qg) {
        // message of position tn from E(tn-1) = En1, E(tn-2) = En2 and bulk (ql, qg);
        // z = 2^(S(tn) + B_c - H(tn-1) + dmax)
        const float hn = (float)(Sn + BH);                  // S(tn) + B_c - H(tn)
        const float sg = fmaf(En1, D0, fmaf(En2, D1, ql));
        const bool ok = in_lin_range(sg) || !act;
        float sigma = fast_log2(sg) + dmax;
        float p = sg * z * rps;
        if (wave_any(!ok)) {
            const float e1 = Rn1 + d0, e2 = Rn2 + d1;
            const float m3 = fmaxf(fmaxf(qg, e1), e2);
            const float lg =
                m3 + fast_log2(fast_exp2(qg - m3) + fast_exp2(e1 - m3) + fast_exp2(e2 - m3));
            if (!ok) {
                sigma = lg;
                p = fast_exp2(hn + lg);
            }
        }
        const int o = (tn & 1) * UP + c;
        *(writer ? p_sh + o : dummy + tid) = p;
        *(writer ? u_sh + o : dummy + tid) = hn + sigma;
        if (a.write_xa && writer && tn > tout)
            Xout[(outrow + (dir == 0 ? tn : L - tn)) * C + c] = (Sn + Bc + (double)sigma) * LN2;
    };
    publish(t0 + 1, Sbuf[cc], exp2_d(Sbuf[cc] + BH + (double)dmax), Qla, Qga);
    bulk(t0 + 2, Qla, Qga);
    double lz = 0.0;
    // checkpoint at the end of a speculative span (the start of a repair)
    const int ck_at = (spec && t1 < L) ? t1 : INT_MAX;
    __syncthreads();

    // ---------------------------------------------------------------- main loop
    for (int tc = t0 + 1, nch = 0; tc <= t1; tc += CH, ++nch) {
        const double* Srow = Sbuf + (nch & 1) * 2 * rowsN;   // end side; start side at +rowsN
        const int rows = min(CH, t1 - tc + 1);
        for (int row = 0; row < rows; ++row) {
            const int t = tc + row;
            if (row == 0 && tc + CH <= t1) {
                // publish chunk n+1 (its buffer was last read in chunk n-1), fetch n+2;
                // this position's barrier makes it visible
                double* dst = Sbuf + ((nch + 1) & 1) * 2 * rowsN;
#pragma unroll
                for (int i = 0; i < PF; ++i) {
                    const int q = tid + i * NT;
                    if (q < rowsN) {
                        const double sv = spub(pf[i], q - (q / C) * C);
                        dst[q] = sv + (double)pfe[i];
                        dst[rowsN + q] = sv - (double)pfs[i];
                    }
                }
#pragma unroll
                for (int i = 0; i < PF; ++i) {
                    const int q = tid + i * NT;
                    if (q < rowsN) {
                        const int rr = q / C, l = q - rr * C;
                        const int tt = tc + 2 * CH + rr;
                        const bool in = tt <= t1;
                        pf[i] = in ? Sb[sidx(tt, l)] : 0.0;
                        pfe[i] = in ? (float)proj_e(tt, l) : 0.0f;
                        pfs[i] = in ? (float)proj_s(tt, l) : 0.0f;
                    }
                }
            }
            // ---- rebase: move this label's values to a new base (every REBASE positions)
            if ((t & (REBASE - 1)) == 0) {
                const float ref = fmaxf(Mref, Rn1);
                // a whole number of octaves: the linear values scale exactly
                const float dl = ref > NEG_HALF ? floorf(ref) : 0.0f;
                const float sc = pow2_neg(dl);
                Bc += (double)dl;
                BH += (double)dl;
                Rn1 -= dl; Rn2 -= dl; Mref -= dl; Qga -= dl;
                En1 *= sc; En2 *= sc; Qla *= sc;
                if constexpr (KPL > 0) {
                    // every slot of positions t-1 .. t-KPL*G (all later bulks and
                    // checkpoints read inside it; the older ones are dead and distinct)
                    float v[KP];
                    ring_load<G, KPL, MIR>(Rrow, t + 2, j, RS, v);
#pragma unroll
                    for (int i = 0; i < KPL; ++i) v[i] -= dl;
                    ring_store<G, KPL, MIR>(Rrow, t + 2, j, RS, v);
                    if constexpr (LIN) {
#pragma unroll
                        for (int i = 0; i < KPL; ++i) v[i] = exp2_or_zero(v[i]);
                        ring_store<G, KPL, MIR>(Erow, t + 2, j, RS, v);
                    }
                }
            }
            const double Snx = Srow[(row + 1) * C + cc];      // end side of t+1
            const float h = (float)(Scur + BH);                 // start side of t + B_c - H(t)
            const float f = exp2_d((double)tmax - (Scur + BH)); // E(t) = s * f
            const float z = exp2_d(Snx + BH + (double)dmax);

            // ---- loads: bulk window of t+2 and the messages of t
            float bv[KP];
            if constexpr (KPL > 0) ring_load<G, KPL, MIR>(LIN ? Erow : Rrow, t + 2, j, RS, bv);
            float pv[CPL];
            {
                const float* pr = p_sh + (t & 1) * UP;
#pragma unroll
                for (int i = 0; i < CPL; ++i) pv[i] = pr[jt + i * GT];
            }
            // ---- [B] transition sums and [D] bulk sum, linear
            float s = 0.0f, q = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                s = fmaf(pv[i], wreg[i], s);
                q += pv[i];
            }
            float bs = 0.0f;
            if constexpr (LIN) {
#pragma unroll
                for (int i = 0; i < KPL; ++i) bs = fmaf(bv[i], dlin[i], bs);
                bs = group_reduce<G>(bs, OpSum());
            }
            s = group_reduce<GT>(s, OpSum());
            q = group_reduce<GT>(q, OpSum());
            const bool okS = in_lin_range(s) || !act;
            const bool okQ = in_lin_range(q);               // the same in every lane
            const bool okD = KPL == 0 || !act || (LIN && in_lin_range(bs));
            float Rnew = fast_log2(s) + tmax - h;
            float Enew = s * f;
            int e = __builtin_amdgcn_frexp_expf(q);          // q = m 2^e, m in [1/2, 1)
            float Qlc = bs, Qgc = KPL == 0 ? NEG : fast_log2(bs) + dmax;
            float lq = 0.0f;                                 // log2 q where it is needed
            if (wave_any(!(okS && okQ))) {
                // exact log-space transition step from the log-space messages
                float uv[CPL];
                const float* ur = u_sh + (t & 1) * UP;
#pragma unroll
                for (int i = 0; i < CPL; ++i) uv[i] = ur[jt + i * GT];
                const float ls = group_lse<GT, CPL>(uv, treg) - h;
                const float lqq = group_lse<GT, CPL>(uv, zero);
                if (!okS) {
                    Rnew = ls;
                    Enew = exp2_or_zero(ls);
                }
                if (!okQ) {
                    lq = lqq;
                    e = lqq > NEG_HALF ? (int)floorf(lqq) + 1 : 0;
                }
            }
            if constexpr (KPL > 0) {
                if (wave_any(!okD)) {
                    // exact log-space bulk from the R ring
                    ring_load<G, KPL, MIR>(Rrow, t + 2, j, RS, bv);
                    const float lg = group_lse<G, KPL>(bv, dreg);
                    if (!okD) {
                        Qgc = lg;
                        Qlc = exp2_or_zero(lg - dmax);
                    }
                }
            }
            if (t == L) lz = H + (double)(okQ ? fast_log2(q) : lq);   // log2 Z
            rps = __builtin_amdgcn_ldexpf(1.0f, -e);
            H += (double)e;
            BH -= (double)e;
            {
                const int s0 = t & RMASK;
                *(writer ? Rrow + s0 : dummy + tid) = Rnew;
                if constexpr (MIR) *(writer ? Rrow + s0 + RS : dummy + tid) = Rnew;
                if constexpr (LIN) {
                    *(writer ? Erow + s0 : dummy + tid) = Enew;
                    if constexpr (MIR) *(writer ? Erow + s0 + RS : dummy + tid) = Enew;
                }
            }
            if (writer && t >= min(hlo, tlo)) window(t, (Bc + (double)Rnew) * LN2);
            Rn2 = Rn1; En2 = En1;
            Rn1 = Rnew; En1 = Enew;
            if (Qgc > NEG_HALF) Mref = Qgc;
            // ---- checkpoint: state right after the transition step of position t
            if (t == ck_at) {
                const size_t ck = ckrow + t / a.delta;
                if (act)
                    for (int qq = j; qq < K; qq += G)
                        a.ck_ring[(ck * K + qq) * C + c] = Rrow[(t - qq) & RMASK];
                if (writer) {
                    a.ck_base[ck * C + c] = Bc;
                    a.ck_mprev[ck * C + c] = Mref;
                }
                if (tid == 0) a.ck_href[ck] = H;
            }
            // ---- [C] message of t+1
            if (t < t1) publish(t + 1, Snx, z, Qla, Qga);
            Scur = Srow[rowsN + (row + 1) * C + cc];            // start side of t+1
            Qla = Qlc;
            Qga = Qgc;
            __syncthreads();
        }
    }

    // ---------------------------------------------------------------- end of sequence
    if (t1 == L && tid == 0) {
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
template <int G, int KPL, int CPL, int GT, int NTMAX, int LAY>
static hipError_t launch_lse_inst(const SweepLaunch& a, dim3 grid, const SweepCfg& cfg,
                                  hipStream_t stream) {
    if (cfg.NT > NTMAX || cfg.lse.CH > lse_chunk_max(G)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_lse<G, KPL, CPL, GT, NTMAX, LAY>), grid, dim3(cfg.NT), cfg.lse.bytes,
                       stream, static_cast<const SweepArgs&>(a), cfg.RS, cfg.lse.P, cfg.lse.CH,
                       a.proj_start, a.proj_end);
    return hipGetLastError();
}

#define LSE_KPL_CASES(G, CPL, GT, NTMAX)                                                \
    switch (cfg.KPL) {                                                                  \
        case 0: return launch_lse_inst<G, 0, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream);   \
        case 1: return launch_lse_inst<G, 1, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream);   \
        case 2: return launch_lse_inst<G, 2, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream);   \
        case 3: return launch_lse_inst<G, 3, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream);   \
        case 4: return launch_lse_inst<G, 4, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream);   \
        case 5: return launch_lse_inst<G, 5, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream);   \
        case 6: return launch_lse_inst<G, 6, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream);   \
        case 7: return launch_lse_inst<G, 7, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream);   \
        case 8: return launch_lse_inst<G, 8, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream);   \
        case 10: return launch_lse_inst<G, 10, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream); \
        case 12: return launch_lse_inst<G, 12, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream); \
        case 16: return launch_lse_inst<G, 16, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream); \
        case 24: return launch_lse_inst<G, 24, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream); \
        case 32: return launch_lse_inst<G, 32, CPL, GT, NTMAX, LAY>(a, grid, cfg, stream); \
        default: return hipErrorInvalidValue;                                           \
    }

// every kernel shape of one ring layout for C > 16 (one translation unit per layout)
template <int LAY>
hipError_t launch_lse_layout(const SweepCfg& cfg, const SweepLaunch& a, int ndir,
                             hipStream_t stream) {
    if (a.mode != MODE_SPEC && a.mode != MODE_REPAIR) return hipErrorInvalidValue;
    const dim3 grid = a.mode == MODE_REPAIR ? dim3(a.B, ndir) : dim3(a.nspans, a.B, ndir);
    // C <= 16 (G >= 16) runs the split-role kernel instead
    if (cfg.G == 8 && cfg.CPL == 4) { LSE_KPL_CASES(8, 4, 8, 256) }
    if (cfg.G == 8 && cfg.CPL == 8) { LSE_KPL_CASES(8, 8, 8, 512) }
    if (cfg.G == 4) { LSE_KPL_CASES(4, 32, 4, 512) }
    return hipErrorInvalidValue;
}

#undef LSE_KPL_CASES

}  // namespace semicrf
