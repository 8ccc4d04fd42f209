// Streaming sweeps for long maximum durations (K up to 8193) on gfx950: the log-semiring
// sweep (forward and mirrored backward) and the max-plus sweep (Viterbi) in one template.
//
// Method ("Streaming Structured Inference with Flash-SemiCRF", gist.science EN explainer,
// "2. Methodology", and the genome-scale regime of "4. Results and Benchmarks", where the
// maximum duration reaches thousands of positions).  The factored recurrence
//     abar[s, c]  = (+)_{c'} (alpha[s, c'] + trans[c', c])
//     alpha[t, c] = S[t, c] + (+)_k (abar[t-k, c] - S[t-k, c] + dur[k-1, c])
// with (+) the log-sum-exp (log semiring) or max (max-plus), keeps per label a ring of
// A[s, c] = abar[s, c] - S[s, c] for the last K positions.  For large K the ring is the
// only large state: K*C floats per ring, 192 KB at K = 8000, C = 6, more than the LDS of
// a compute unit.  Where it fits, the ring sits in LDS; otherwise in a per-workgroup slice
// of global memory, read through the L2 cache (the pages' fused kernel keeps its ring in
// on-chip memory, which caps K there).
//
// Work layout: one workgroup per (checkpoint span, sequence, direction), as the other
// sweeps (burn-in, seam windows, end checkpoint, in-order repair).
//  * chain wavefront (threads 0..63): lane c holds label c.  At position t it combines
//    the bulk value of t (durations k >= 2, from the bulk wavefronts) with the k = 1 term
//    from its own register, forms alpha(t, c), runs the transition step over every label
//    (lane broadcasts) and writes the ring entry A(t, c).
//  * bulk wavefronts (threads 64..): G lanes per label (G <= 64, inside one wavefront).
//    At position t they form the bulk value of t+1 over the ring entries of positions
//    <= t-1: lane j owns durations k = 2 + j + i*G, i < KPL, with the duration weights in
//    registers (up to 128 per lane: 512 threads, two wavefronts per SIMD, 256 VGPRs).
//    One workgroup barrier per position.
// Log semiring: the bulk sum is linear in fp32 (E = 2^(A - B_c), weights 2^(dur - dmax)),
// range-checked per wavefront and, outside range, recomputed exactly in log space from the
// log ring; the chain works in log space throughout (a few exponentials per position).
// Max-plus: the bulk is a max with the lowest k on ties, the chain's k = 1 term wins ties.
// Values are fp32 relative to per-label fp64 bases B_c (moved every XK_REBASE positions)
// and a common fp64 reference H; outputs fp64, natural-log units.
#pragma once

#include "common.h"
#include "internal.h"

namespace semicrf {

namespace {

// Linear bulk sums are trusted inside [2^-60, 2^60]: a term lost to fp32 underflow (an
// entry or a weight below 2^-126, the weights relative to the label's largest duration
// score) is far under 2^-23 of such a sum, and nothing overflowed.  With a rebase every
// XK_REBASE positions the newest ring entries stay within that range unless the log
// partition function grows by more than about 60 / XK_REBASE octaves a position; outside
// it (inf and NaN included) the sum is redone exactly in log space.
constexpr float XK_LIN_LO = 0x1p-60f;
constexpr float XK_LIN_HI = 0x1p+60f;

__device__ __forceinline__ bool xk_in_range(float s) {
    constexpr uint32_t lo = __builtin_bit_cast(uint32_t, XK_LIN_LO);
    constexpr uint32_t hi = __builtin_bit_cast(uint32_t, XK_LIN_HI);
    return __float_as_uint(s) - lo <= hi - lo;
}

// some lane of the wavefront
__device__ __forceinline__ bool xk_wave_any(bool v) { return __builtin_amdgcn_ballot_w64(v) != 0; }

__device__ __forceinline__ double xk_nan() { return __longlong_as_double(0x7ff8000000000000LL); }

// 2^x, 0 for x <= -126 (NEG included); +inf past the fp32 range (a linear sum holding it
// fails the range check and is redone in log space)
__device__ __forceinline__ float xk_exp2(float x) { return x > -126.0f ? fast_exp2(x) : 0.0f; }

// log2(2^a + 2^b), NEG when both are NEG
__device__ __forceinline__ float xk_lse2(float a, float b) {
    const float m = fmaxf(a, b);
    if (m <= NEG_HALF) return NEG;
    return m + fast_log2(xk_exp2(a - m) + xk_exp2(b - m));
}

// exact 2^-n for a whole number n (the scale of a whole-octave rebase)
__device__ __forceinline__ float xk_pow2_neg(float n) {
    return __builtin_amdgcn_ldexpf(1.0f, -(int)n);
}

}  // namespace

// MAXP: max-plus (Viterbi) instead of the log semiring.  RM: where the rings live
// (XK_RING_LDS: plain rows in LDS; XK_RING_MIRRORED: the ring the bulk sums read, mirrored
// in LDS (every position in two slots RS apart, so a lane's window is contiguous and its
// reads take compile-time offsets), with the log ring of the log semiring in global
// memory; XK_RING_GLOBAL: plain rows in global memory).  G: bulk lanes per label (<= 64);
// KPLMAX: duration weights per lane (registers); NTMAX: the largest block.
// Block: 64 + ceil(C*G/64)*64 threads.  Grid: (nspans, B, ndir) in MODE_SPEC, (B, ndir) in
// MODE_REPAIR (ndir = 1 for max-plus).
template <bool MAXP, int RM, int G, int KPLMAX, int NTMAX>
__global__ __launch_bounds__(NTMAX) void k_sweep_xk(const SweepArgs a, const XkParams x,
                                                   const float* __restrict__ proj_start,
                                                   const float* __restrict__ proj_end) {
    static_assert(G <= 64, "a label's lanes share one wavefront");
    constexpr int U = XK_UNROLL;
    // ring reads of a bulk value in flight at once: the whole window of a lane when the
    // ring is in LDS and the window is short (one LDS round trip a position), else U
    constexpr int UB = (RM != XK_RING_GLOBAL && KPLMAX <= 32) ? KPLMAX : U;
    constexpr double SC = MAXP ? 1.0 : LOG2E;      // working units: natural (max) or base 2
    constexpr double OUT = MAXP ? 1.0 : LN2;       // back to natural-log units
    extern __shared__ double lds[];
    const int C = a.C, K = a.K, T = a.T;
    const int tid = threadIdx.x, NT = blockDim.x, NB = NT - 64;
    const bool chain = __builtin_amdgcn_readfirstlane(tid >> 6) == 0;
    const int bt = tid - 64;
    const int cb = chain ? C : bt / G;
    const int j = chain ? 0 : bt - cb * G;
    const bool bact = !chain && cb < C;
    const bool cact = chain && tid < C;
    const int cl = cact ? tid : 0;
    const int RS = x.RS, RMASK = RS - 1, CH = x.CH, kplr = x.kpl;

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
    const bool ckpt = spec && t1 < L;
    const int hlo = (spec && span > 0) ? tout - K + 1 : INT_MAX;    // seam windows
    const int tlo = ckpt ? t1 - K + 1 : INT_MAX;
    const size_t drow = (size_t)dir * a.B + b;   // (direction, sequence) row
    const size_t winrow = (drow * a.nspans + span) * K;
    const size_t ckrow = drow * a.nspans;
    auto window = [&](int t, int c, double av) {
        if (t >= hlo && t <= tout) a.head[(winrow + t - hlo) * C + c] = av;
        if (t >= tlo && t <= t1) a.tail[(winrow + t - tlo) * C + c] = av;
    };

    // ---------------------------------------------------------------- LDS
    // log ring R (both semirings) and linear ring E (log semiring): where they live, and
    // whether a row is mirrored
    constexpr bool RMIR = MAXP && RM == XK_RING_MIRRORED;
    constexpr bool EMIR = !MAXP && RM == XK_RING_MIRRORED;
    constexpr bool RGLB = RM == XK_RING_GLOBAL || (!MAXP && RM == XK_RING_MIRRORED);
    constexpr bool EGLB = !MAXP && RM == XK_RING_GLOBAL;
    constexpr int NGR = (RGLB ? 1 : 0) + (EGLB ? 1 : 0);   // rings in global memory
    static_assert(NGR == xk_global_rings(MAXP, RM), "the host sizes the global rings");
    // The chain stages every position's outputs in LDS (it issues no global memory
    // operation inside the loop); the bulk lanes write them out.  With plain global rings
    // the bulk sum of the next position reads the newest entry from global memory, so a
    // position's outputs are written one position later (history of 2 positions); else a
    // whole chunk of CH positions at the next chunk's first row (history of two chunks),
    // so that the lanes, whose global stores share the vector memory counter with their
    // loads, wait on stores once a chunk.
    constexpr bool FLUSH_FIRST = RM == XK_RING_GLOBAL;
    const int rowsN = CH * C;
    const int HD = FLUSH_FIRST ? 2 : 2 * CH;              // history depth (positions)
    double* Sbuf = lds;                                   // [2 chunks][end, start][CH][C]
    double* SL = Sbuf + 4 * rowsN;                        // [C]
    double* hA = SL + C;                                  // [HD][C] A (working units)
    double* hX = hA + HD * C;                             // [HD][C] X (log semiring)
    float* trl = (float*)(hX + (MAXP ? 0 : HD * C));      // [C][C]: trl[c' * C + c]
    float* part = trl + C * C;                            // [2][C][2] bulk values
    float* dlsh = part + 4 * C;                           // [C] rebase shift
    float* hR = dlsh + C;                                 // [HD][C] ring entry
    uint32_t* hB = (uint32_t*)(hR + HD * C);              // [HD][C] backpointer (max-plus)
    // history row of position p >= t0 + 1
    auto hrow = [&](int p) { return FLUSH_FIRST ? (p & 1) : (p - t0 - 1) % HD; };
    // log semiring: [C][NE] each label's total base shift (whole octaves) in force at the
    // epochs of XK_REBASE positions, by epoch mod NE.  A log ring entry keeps the base of
    // its epoch (only the linear ring is moved at a rebase); the table takes it to any
    // later base.
    const int NE = MAXP ? 0 : x.NE, NEM = NE - 1;
    int* cumt = (int*)(hB + (MAXP ? HD * C : 0));
    float* ringl = (float*)(cumt + (MAXP ? 0 : C * NE));  // the rings held in LDS
    // rings: base and row pitch; a repair reuses its span's global slice
    const int RP = RMIR ? 2 * RS : RS, EP = EMIR ? 2 * RS : RS;
    float* gslice = x.ring ? x.ring + (drow * a.nspans + span) * (size_t)NGR * C * RS : nullptr;
    float* Rbase = RGLB ? gslice : ringl;
    float* Ebase = EGLB ? gslice + (RGLB ? (size_t)C * RS : 0) : RGLB ? ringl : ringl + (size_t)C * RP;
    const int crow = bact ? cb : 0;
    float* Rrow = Rbase + (size_t)crow * RP;
    float* Erow = Ebase + (size_t)crow * EP;
    auto slot = [&](int p) { return p & RMASK; };
    // ring entries of position p of label c (every copy)
    auto putR = [&](int c, int p, float v) {
        float* row = Rbase + (size_t)c * RP;
        row[slot(p)] = v;
        if constexpr (RMIR) row[slot(p) + RS] = v;
    };
    auto putE = [&](int c, int p, float v) {
        float* row = Ebase + (size_t)c * EP;
        row[slot(p)] = v;
        if constexpr (EMIR) row[slot(p) + RS] = v;
    };

    const double* Sb = a.S + (size_t)b * (T + 1) * C;
    for (int q = tid; q < C; q += NT) SL[q] = Sb[(size_t)L * C + q];
    const float* PSb = proj_start ? proj_start + (size_t)b * T * C : nullptr;
    const float* PEb = proj_end ? proj_end + (size_t)b * T * C : nullptr;
    // projections of sweep position p in working units: end side (segments ending at p)
    // and start side (segments starting at p); 0 without projections or outside the
    // sequence.  The mirrored direction swaps their roles.
    auto proj_e = [&](int p, int q) -> double {
        const float* src = dir == 0 ? PEb : PSb;
        const int t = dir == 0 ? p - 1 : L - p;
        return (src && p >= 1 && p <= L) ? (double)src[(size_t)t * C + q] * SC : 0.0;
    };
    auto proj_s = [&](int p, int q) -> double {
        const float* src = dir == 0 ? PSb : PEb;
        const int t = dir == 0 ? p : L - 1 - p;
        return (src && p >= 0 && p < L) ? (double)src[(size_t)t * C + q] * SC : 0.0;
    };
    // transitions into each label (transposed for the mirrored direction)
    for (int q = tid; q < C * C; q += NT) {
        const int cp = q / C, c = q - cp * C;
        const float tv = dir == 0 ? a.trans[cp * C + c] : a.trans[c * C + cp];
        trl[q] = fmaxf((float)((double)tv * SC), NEG);
    }
    // rings: every slot cleared (log NEG, linear 0)
    for (size_t q = tid; q < (size_t)C * RP; q += NT) Rbase[q] = NEG;
    if constexpr (!MAXP)
        for (size_t q = tid; q < (size_t)C * EP; q += NT) Ebase[q] = 0.0f;
    if constexpr (!MAXP)
        for (int q = tid; q < C * NE; q += NT) cumt[q] = 0;   // positions <= t0: base 0
    auto epoch = [&](int p) { return (p >> XK_LOG_REBASE) & NEM; };

    // ---------------------------------------------------------------- durations
    auto durv = [&](int c, int k) -> float {
        return (k >= 1 && k <= K) ? fmaxf((float)((double)a.dur[(k - 1) * C + c] * SC), NEG) : NEG;
    };
    // bulk lanes: weights of durations k = 2 + j + i*G (linear, relative to the label's
    // largest duration score dmax, or log for max-plus); NEG / 0 past K
    float Dw[KPLMAX];
    float dmx = NEG;
#pragma unroll
    for (int i = 0; i < KPLMAX; ++i) {
        Dw[i] = (bact && i < kplr) ? durv(cb, 2 + j + i * G) : NEG;
        dmx = fmaxf(dmx, Dw[i]);
    }
    if (!chain) dmx = group_reduce<G>(dmx, OpMax());
    const float dmax = dmx > NEG_HALF ? dmx : 0.0f;
    if constexpr (!MAXP) {
#pragma unroll
        for (int i = 0; i < KPLMAX; ++i) Dw[i] = xk_exp2(Dw[i] - dmax);
    }
    const float d1 = cact ? durv(cl, 1) : NEG;            // chain: the k = 1 term
    // chain: the transitions into this lane's label in registers (C <= CT = 8), so the
    // transition step is an unrolled run of lane broadcasts and adds; larger C reads them
    // from LDS
    constexpr int CT = G == 64 ? 8 : 0;
    float trv[CT > 0 ? CT : 1];
    __syncthreads();   // ring cleared (the start state below overwrites slots other
                       // threads cleared) and trl visible
    if constexpr (CT > 0) {
#pragma unroll
        for (int i = 0; i < CT; ++i) trv[i] = (cact && i < C) ? trl[i * C + cl] : NEG;
    }

    // ---------------------------------------------------------------- start state
    double Bc = 0.0, H = 0.0;
    float Rn1 = NEG;                                      // chain: A(t-1) - B_c
    float Mref = 0.0f;                                    // chain: last bulk value (rebase)
    if (t0 == 0) {
        // position 0: no transition into it; its ring entry is its start-side projection
        if (bact && j == 0) {
            const float r0 = fmaxf((float)proj_s(0, cb), NEG);
            putR(cb, 0, r0);
            if constexpr (!MAXP) putE(cb, 0, xk_exp2(r0));
        }
        Rn1 = cact ? fmaxf((float)proj_s(0, cl), NEG) : NEG;
    } else if (spec) {
        // burn-in start: every ring entry of positions t0-K+1 .. t0 equal (0)
        if (bact)
            for (int q = j; q < K && t0 - q >= 0; q += G) {
                putR(cb, t0 - q, 0.0f);
                if constexpr (!MAXP) putE(cb, t0 - q, 1.0f);
            }
        Rn1 = cact ? 0.0f : NEG;
    } else {
        const size_t ck = ckrow + span;
        if (bact)
            for (int q = j; q < K && t0 - q >= 0; q += G) {
                const float rv = a.ck_ring[(ck * K + q) * C + cb];
                putR(cb, t0 - q, rv);
                if constexpr (!MAXP) putE(cb, t0 - q, xk_exp2(rv));
            }
        if (chain) {
            Bc = a.ck_base[ck * C + cl];
            H = a.ck_href[ck];
            Mref = a.ck_mprev[ck * C + cl];
            Rn1 = cact ? a.ck_ring[(ck * K + 0) * C + cl] : NEG;
        }
    }
    const size_t outrow = (size_t)b * (T + 1);
    double* Xout = dir == 0 ? a.XF : a.XB;
    if (cact) {
        const double a0 = (Bc + (double)Rn1) * OUT;
        if (t0 == 0)   // window positions <= 0: position 0's value, nothing before it
            for (int p = min(hlo, tlo); p <= 0; ++p) window(p, cl, p == 0 ? a0 : -1.0e300);
    }
    // the staged outputs of position p, label c (bulk lanes of label c, so that a label's
    // global ring entries are written and read back by one wavefront): X, A, backpointer,
    // seam windows, and the ring entries held in global memory (the LDS ones come from the
    // chain)
    auto emit = [&](int p, int c) {
        const int h = hrow(p) * C + c;
        const double av = hA[h];
        const size_t o = (outrow + (dir == 0 ? p : L - p)) * C + c;
        if constexpr (MAXP) {
            if (p > tout) a.bp[(outrow + p) * C + c] = hB[h];
        } else if (a.write_xa) {
            if (p > tout) Xout[o] = hX[h] * OUT;
        }
        if (p >= min(hlo, tlo)) window(p, c, av * OUT);
        if constexpr (RGLB) putR(c, p, hR[h]);
        if constexpr (EGLB) putE(c, p, xk_exp2(hR[h]));
    };
    // one position (FLUSH_FIRST), or positions p0 .. p1 (a chunk)
    auto flush = [&](int p0, int p1) {
        if (!bact) return;
        if constexpr (FLUSH_FIRST) {
            if (j == 0) emit(p0, cb);
        } else {
            for (int p = p0 + j; p <= p1; p += G) emit(p, cb);
        }
    };

    // ---------------------------------------------------------------- S staging
    // chunk n holds rows t = t0 + 1 + n*CH + r, r < CH: end side S(t) + pe(t) and start
    // side S(t) - ps(t), working units; staged by the bulk lanes a chunk ahead
    auto sidx = [&](int t, int q) -> size_t { return (size_t)(dir == 0 ? t : L - t) * C + q; };
    auto spub = [&](double raw, int q) -> double { return dir == 0 ? raw * SC : (SL[q] - raw) * SC; };
    __syncthreads();                                      // SL visible
    const int pfn = (rowsN + NB - 1) / NB;                // staged values per bulk lane
    if (!chain)
        for (int q = bt; q < rowsN; q += NB) {
            const int row = q / C, l = q - row * C;
            const int t = t0 + 1 + row;
            const bool in = t <= t1;
            const double sv = in ? spub(Sb[sidx(t, l)], l) : 0.0;
            Sbuf[q] = in ? sv + proj_e(t, l) : 0.0;
            Sbuf[rowsN + q] = in ? sv - proj_s(t, l) : 0.0;
        }
    // the next chunk, loaded and stored at once (at most XK_PF values per lane): no global
    // load stays in flight across positions, so the lanes never wait on their own output
    // stores (they share the vector memory counter) except at the chunk's first row
    const float* PEd = dir == 0 ? PEb : PSb;              // end-side projection source
    const float* PSd = dir == 0 ? PSb : PEb;              // start-side projection source
    auto stage = [&](int tcs, int buf) {
        double pf[XK_PF];
        float pfe[XK_PF], pfs[XK_PF];
#pragma unroll
        for (int i = 0; i < XK_PF; ++i) {
            const int q = bt + i * NB;
            const int row = q / C, l = q - row * C;
            const int t = tcs + row;
            const bool in = !chain && i < pfn && q < rowsN && t <= t1;
            const int te = dir == 0 ? t - 1 : L - t;       // end side: valid for 1 <= t <= L
            const int ts = dir == 0 ? t : L - 1 - t;       // start side: valid for t <= L-1
            pf[i] = in ? Sb[sidx(t, l)] : 0.0;
            pfe[i] = (in && PEd && t >= 1) ? PEd[(size_t)te * C + l] : 0.0f;
            pfs[i] = (in && PSd && t < L) ? PSd[(size_t)ts * C + l] : 0.0f;
        }
        double* dst = Sbuf + buf * 2 * rowsN;
#pragma unroll
        for (int i = 0; i < XK_PF; ++i) {
            const int q = bt + i * NB;
            if (!chain && i < pfn && q < rowsN) {
                const double sv = spub(pf[i], q - (q / C) * C);
                dst[q] = sv + (double)pfe[i] * SC;
                dst[rowsN + q] = sv - (double)pfs[i] * SC;
            }
        }
    };
    __syncthreads();                                      // ring, chunk 0 visible

    // ---------------------------------------------------------------- bulk value
    // of position tq over durations k >= 2 (ring entries of positions <= tq - 2): log value
    // (both semirings) and, for max-plus, the lowest k attaining it; written to
    // part[tq & 1][label]
    auto bulk = [&](int tq) {
        const int p0 = tq - 2 - j;                        // position of k = 2 + j (i = 0)
        // ring value of position p0 - i*G of the ring the sums read: on a mirrored row the
        // lane's window is one contiguous stretch below slot(p0) + RS (RS >= (KPLMAX-1)*G,
        // checked on the host), read at compile-time offsets from its lowest slot
        int lo = slot(p0) + RS - (KPLMAX - 1) * G;
        // opaque to the compiler, so the offsets stay positive (the LDS offset field is
        // unsigned) instead of being rewritten from the top of the window
        asm volatile("" : "+v"(lo));
        auto bulk_at = [&](const float* row, int i) -> float {
            if constexpr (RM == XK_RING_MIRRORED) return row[lo + (KPLMAX - 1 - i) * G];
            else return row[slot(p0 - i * G)];
        };
        float qv = NEG;
        int kq = INT_MAX;
        if constexpr (MAXP) {
            float best = NEG;
            int kb = INT_MAX;
#pragma unroll
            for (int i0 = 0; i0 < KPLMAX; i0 += UB) {
                if (i0 < kplr) {
                    float v[UB];
#pragma unroll
                    for (int u = 0; u < UB; ++u) v[u] = bulk_at(Rrow, i0 + u);
#pragma unroll
                    for (int u = 0; u < UB; ++u) {
                        const float y = v[u] + Dw[i0 + u];
                        if (y > best) {                   // ascending k: the lowest wins ties
                            best = y;
                            kb = 2 + j + (i0 + u) * G;
                        }
                    }
                }
            }
            qv = group_reduce<G>(best, OpMax());
            kq = group_min_int<G>(best == qv && qv > NEG_HALF ? kb : INT_MAX);
        } else {
            float acc = 0.0f;
#pragma unroll
            for (int i0 = 0; i0 < KPLMAX; i0 += UB) {
                if (i0 < kplr) {
                    float v[UB];
#pragma unroll
                    for (int u = 0; u < UB; ++u) v[u] = bulk_at(Erow, i0 + u);
#pragma unroll
                    for (int u = 0; u < UB; ++u) acc = fmaf(v[u], Dw[i0 + u], acc);
                }
            }
            acc = group_reduce<G>(acc, OpSum());
            const bool ok = xk_in_range(acc) || !bact;   // per label group
            qv = fast_log2(acc) + dmax;
            if (xk_wave_any(!ok)) {
                // exact log-space sum (log ring, each entry taken from the base of its
                // epoch to that of the linear ring, the one of position tq - 2; the
                // duration scores from global memory)
                const int* cum = cumt + crow * NE;
                const int cnow = cum[epoch(tq - 2)];
                // positions of the chunk of tq - 1 and the one before it are only staged
                const int hlo_pos = t0 + 1 + max(0, (tq - 2 - t0) / CH - 1) * CH;
                float m = NEG, s = 0.0f;
                for (int i0 = 0; i0 < kplr; i0 += U) {
                    {
                        float y[U];
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            const int k = 2 + j + (i0 + u) * G;
                            const int p = p0 - (i0 + u) * G;
                            float rv;
                            if constexpr (RGLB && !FLUSH_FIRST)   // chunks not yet written
                                rv = p >= hlo_pos ? hR[hrow(p) * C + crow] : Rrow[slot(p)];
                            else
                                rv = Rrow[slot(p)];
                            y[u] = rv - (float)(cnow - cum[epoch(p)]) + (bact ? durv(cb, k) : NEG);
                        }
                        float mc = y[0];
#pragma unroll
                        for (int u = 1; u < U; ++u) mc = fmaxf(mc, y[u]);
                        const float mn = fmaxf(m, mc);
                        if (mn > NEG_HALF) {
                            s *= xk_exp2(m - mn);
#pragma unroll
                            for (int u = 0; u < U; ++u) s += xk_exp2(y[u] - mn);
                            m = mn;
                        }
                    }
                }
                const float gm = group_reduce<G>(m, OpMax());
                float sg = gm > NEG_HALF ? s * xk_exp2(m - gm) : 0.0f;
                sg = group_reduce<G>(sg, OpSum());
                const float lg = gm > NEG_HALF ? gm + fast_log2(sg) : NEG;
                if (!ok) qv = lg;
            }
        }
        if (bact && j == 0) {
            float* pp = part + ((tq & 1) * C + cb) * 2;
            pp[0] = qv;
            pp[1] = __int_as_float(kq);
        }
    };
    // bulk lanes, one position after a rebase at position tr: the live entries of
    // positions tr-K+1 .. tr-1 this lane reads for the bulk of tr + 2 move to the new base
    // (the entry of tr was written in it; older ones are never weighted again, and the
    // ring holds RS >= K + 2 positions, so every live slot is moved exactly once).  The
    // ring the bulk sums read moves: the log ring of max-plus, the linear ring of the log
    // semiring (its log ring keeps its epochs' bases).
    auto rebase_ring = [&](int tq) {
        const int trb = tq - 2;                           // the chain's rebase positions
        if (!bact || (trb & (XK_REBASE - 1)) != 0 || trb <= t0 || trb >= t1) return;
        const int p0 = tq - 2 - j;
        for (int i0 = 0; i0 < kplr; i0 += UB) {
            // a chunk's loads (the whole window when it is short) and the shift first, then
            // its stores (each slot belongs to one lane): one LDS round trip
            float v[UB];
#pragma unroll
            for (int u = 0; u < UB; ++u) v[u] = (MAXP ? Rrow : Erow)[slot(p0 - (i0 + u) * G)];
            const float dl = dlsh[cb];
            const float sc = MAXP ? 1.0f : xk_pow2_neg(dl);
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const int p = p0 - (i0 + u) * G;
                if (p <= trb - 1 && p >= trb - K + 1) {
                    if constexpr (MAXP) putR(cb, p, v[u] - dl);
                    else putE(cb, p, v[u] * sc);
                }
            }
        }
    };
    if (bact) bulk(t0 + 1);
    __syncthreads();

    // ---------------------------------------------------------------- main loop
    double lz = 0.0;
    float pdl = 0.0f;
    bool pend = false;
    int ocum = 0;                                         // chain: total shift (octaves)
    for (int tc = t0 + 1, nch = 0; tc <= t1; tc += CH, ++nch) {
        const double* Sch = Sbuf + (nch & 1) * 2 * rowsN;
        const int rows = min(CH, t1 - tc + 1);
        for (int row = 0; row < rows; ++row) {
            const int t = tc + row;
            if (chain) {
                // ---- bulk value of t (and its lowest k for max-plus)
                const float* pp = part + ((t & 1) * C + cl) * 2;
                float Q = pp[0];
                const int kQ = __float_as_int(pp[1]);
                if (pend) {                               // summed before the last rebase
                    Q -= pdl;
                    pend = false;
                }
                // ---- rebase: this label's values move to a new base (never at the span's
                // end, so that the ring is in one base when the checkpoint copies it)
                if ((t & (XK_REBASE - 1)) == 0 && t < t1) {
                    const float ref = fmaxf(Mref, Rn1);
                    float dl = cact && ref > NEG_HALF ? ref : 0.0f;
                    if constexpr (!MAXP) dl = floorf(dl);  // whole octaves: exact linear scale
                    Bc += (double)dl;
                    Rn1 -= dl;
                    Mref -= dl;
                    Q -= dl;
                    if (cact) dlsh[cl] = dl;
                    pdl = dl;
                    pend = true;
                    if constexpr (!MAXP) ocum += (int)dl;
                }
                // the shift in force from here to the next epoch (none at the span's end)
                if constexpr (!MAXP)
                    if ((t & (XK_REBASE - 1)) == 0 && cact) cumt[cl * NE + epoch(t)] = ocum;
                // ---- alpha(t): the k = 1 term and the bulk
                const double Se = Sch[row * C + cl];                  // end side of t
                const double Ss = Sch[rowsN + row * C + cl];          // start side of t
                const float e1 = Rn1 + d1;
                float sig;
                int kb = 1;
                if constexpr (MAXP) {
                    sig = fmaxf(e1, Q);
                    kb = (e1 >= Q) ? 1 : kQ;
                } else {
                    sig = xk_lse2(e1, Q);
                }
                const float u = cact ? (float)(Se + Bc - H) + sig : NEG;  // alpha(t) - H
                const int hr = (FLUSH_FIRST ? (t & 1) : (nch & 1) * CH + row) * C + cl;
                if (!MAXP && cact) hX[hr] = Se + Bc + (double)sig;
                // ---- transition step of t over every label's alpha (lane broadcasts; the
                // lowest c' on ties)
                float mu = NEG;                                        // max_c' u(c')
                float mt = NEG;                                        // max_c' u + trans
                int cbest = 0;
                float abar;                                            // abar(t) - H
                float zs = 0.0f;                                       // sum_c' 2^(u - mu)
                if constexpr (CT > 0) {
                    float uv[CT], y[CT];
#pragma unroll
                    for (int i = 0; i < CT; ++i) {
                        uv[i] = i < C ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u), i)) : NEG;
                        y[i] = uv[i] + trv[i];
                        mu = fmaxf(mu, uv[i]);
                        if (y[i] > mt) {
                            mt = y[i];
                            cbest = i;
                        }
                    }
                    abar = mt;
                    if constexpr (!MAXP) {
                        if (mt > NEG_HALF) {
                            float s = 0.0f;
#pragma unroll
                            for (int i = 0; i < CT; ++i) s += xk_exp2(y[i] - mt);
                            abar = mt + fast_log2(s);
                        }
                        if (t == L && mu > NEG_HALF)
#pragma unroll
                            for (int i = 0; i < CT; ++i) zs += xk_exp2(uv[i] - mu);
                    }
                } else {
#pragma unroll 8
                    for (int cp = 0; cp < C; ++cp) {
                        const float uv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u), cp));
                        const float y = uv + trl[cp * C + cl];
                        mu = fmaxf(mu, uv);
                        if (y > mt) {
                            mt = y;
                            cbest = cp;
                        }
                    }
                    abar = mt;
                    if constexpr (!MAXP) {
                        if (mt > NEG_HALF) {
                            float s = 0.0f;
#pragma unroll 8
                            for (int cp = 0; cp < C; ++cp) {
                                const float uv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u), cp));
                                s += xk_exp2(uv + trl[cp * C + cl] - mt);
                            }
                            abar = mt + fast_log2(s);
                        }
                        if (t == L && mu > NEG_HALF)
                            for (int cp = 0; cp < C; ++cp) {
                                const float uv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u), cp));
                                zs += xk_exp2(uv - mu);
                            }
                    }
                }
                if constexpr (!MAXP) {
                    if (t == L && mu > NEG_HALF) lz = H + (double)mu + (double)fast_log2(zs);   // log2 Z
                } else {
                    if (t == L && cact) a.vfin[(size_t)b * C + cl] = H + (double)u;
                }
                const float Rnew = cact ? fmaxf(abar - (float)(Ss + Bc - H), NEG) : NEG;
                if (mu > NEG_HALF) H += (double)mu;
                if (cact) {
                    // outputs of t, staged; the ring entry goes straight to an LDS ring
                    if constexpr (MAXP)
                        hB[hr] = (uint32_t)kb | (t < L ? ((uint32_t)cbest << 16) : 0u);
                    hA[hr] = Bc + (double)Rnew;
                    hR[hr] = Rnew;
                    if constexpr (!RGLB) putR(cl, t, Rnew);
                    if constexpr (!MAXP && !EGLB) putE(cl, t, xk_exp2(Rnew));
                }
                Rn1 = Rnew;
                if (Q > NEG_HALF) Mref = Q;
            } else {
                // ---- S staging (the next chunk, into the buffer the chain left at the last
                // barrier), the rebase of the ring, the bulk value of t+1, and the staged
                // outputs: of t-1 before the bulk value (plain global rings), or of the
                // previous chunk after it, at a chunk's first row
                if constexpr (FLUSH_FIRST)
                    if (t - 1 > t0) flush(t - 1, t - 1);
                if (row == 0 && tc + CH <= t1) stage(tc + CH, (nch + 1) & 1);
                rebase_ring(t + 1);
                if (t + 1 <= t1 && bact) bulk(t + 1);
                if constexpr (!FLUSH_FIRST)
                    if (row == 0 && nch > 0) flush(tc - CH, tc - 1);
            }
            __syncthreads();
        }
    }
    if constexpr (FLUSH_FIRST) flush(t1, t1);
    else flush(t0 + 1 + (t1 - t0 - 1) / CH * CH, t1);    // the last chunk
    __syncthreads();                                      // the ring entry of t1 (global form)

    // ---------------------------------------------------------------- span end
    if (ckpt) {
        // the ring in its final base (no rebase at t1; the one before it was applied
        // during t1) and the chain's state: the checkpoint a repair restarts from
        const size_t ck = ckrow + t1 / a.delta;
        if (bact) {
            if constexpr (MAXP) {
                for (int q = j; q < K; q += G) a.ck_ring[(ck * K + q) * C + cb] = Rrow[slot(t1 - q)];
            } else {
                // log ring entries in the final base
                const int* cum = cumt + cb * NE;
                const int cnow = cum[epoch(t1)];
                for (int q = j; q < K; q += G)
                    a.ck_ring[(ck * K + q) * C + cb] =
                        Rrow[slot(t1 - q)] - (float)(cnow - cum[epoch(t1 - q)]);
            }
        }
        if (cact) {
            a.ck_base[ck * C + cl] = Bc;
            a.ck_mprev[ck * C + cl] = Mref;
        }
        if (tid == 0) a.ck_href[ck] = H;
    }
    if constexpr (!MAXP) {
        if (t1 == L && tid == 0) {
            if (spec) {
                a.lzloc[dir * a.B + b] = lz * LN2;       // the seam check adds the offsets
            } else {
                // a repaired sweep continues in the frame of the span before the failed seam
                const double base = a.off[drow * a.nspans + span - 1];
                (dir == 0 ? a.logz : a.logz_b)[b] = bad ? xk_nan() : lz * LN2 + base;
            }
        }
    }
}

}  // namespace semicrf
