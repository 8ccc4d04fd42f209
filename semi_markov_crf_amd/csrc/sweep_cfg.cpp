// Host-side shape selection for the sweep kernels: lane grouping, ring size and the LDS
// layout that fits the 160 KB of a gfx950 compute unit.
#include <algorithm>

#include "internal.h"

namespace semicrf {

namespace {

constexpr size_t LDS_BUDGET = 150 * 1024;   // leaves room for the compiler's own LDS use

int pow2_at_least(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// The ring sweeps with every duration weight in registers (short and moderate K).
SweepCfg choose_ring_sweeps(int C, int K) {
    SweepCfg s{};
    s.ok = false;
    if (C < 1 || K < 1) return s;
    // lane groups: aim at <= 4 waves (one per SIMD) where the label count allows
    int G, CPL, GT;
    // a lane covers at most 32 durations (8 ring blocks of ROUND positions in the round
    // kernels), so 32 lanes per label reach K = 1025; above it up to 7 labels take 64
    // lanes each (7 bulk waves beside the chain)
    if (C <= 4) { G = 64; GT = 4; CPL = 1; }
    else if (C <= 7 && K > 32 * 32 + 1) { G = 64; GT = 8; CPL = 1; }
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
    s.NTv = ((C * G + 63) / 64) * 64;
    // C <= 16: a chain wavefront in front of the label groups (round kernels)
    s.split = G >= 16;
    s.NT = s.split ? 64 + s.NTv : s.NTv;
    // RS >= K + 2 live positions and >= the widest window a lane addresses (2 + KPL*G)
    s.RS = pow2_at_least(std::max(K + 2, 3 + kmax * G));
    s.BPL = 0;
    s.CPr = 0;
    if (G >= 16) {
        // round kernels: ring blocks of ROUND positions; a bulk sum reaches back bmax
        // blocks, the ring holds those plus the rounds in flight
        const int bmax = (K + ROUND - 1) / ROUND;
        s.BPL = (std::max(bmax - 1, 0) + G - 1) / G;
        if (s.BPL > 8) return s;
        s.CPr = C <= 4 ? 4 : C <= 6 ? 6 : C <= 8 ? 8 : C <= 12 ? 12 : 16;
        s.RS = pow2_at_least(ROUND * (bmax + 5));
    }
    const int pad = G < 32 ? G : 0;   // staggers the label rows over the LDS banks
    const int UP = GT * CPL;
    auto pitch = [&](int layout) { return ((layout & SWEEP_MIRRORED) ? 2 : 1) * s.RS + pad; };

    // log-semiring sweep: mirrored + linear, plain + linear, plain + log-space only; the
    // round kernel keeps one copy of each ring (float4 blocks), rows 16 bytes apart in bank
    for (int lay : {int(SWEEP_MIRRORED | SWEEP_LINEAR), int(SWEEP_LINEAR), 0}) {
        if (s.split && (lay & SWEEP_MIRRORED)) continue;
        const int P = s.split ? s.RS + 4 : pitch(lay);
        // the round kernel needs two rounds per chunk (it restages one round late)
        for (int ch = lse_chunk_max(G); ch >= (s.split ? 2 * ROUND : 4) && s.lse.bytes == 0;
             ch >>= 1) {
            // sized for the projection instances, the larger of the two
            const size_t n = s.split ? lse_round_lds_bytes(C, s.CPr, P, ch, lay & SWEEP_LINEAR, true)
                                     : lse_lds_bytes(C, s.NT, UP, P, ch, lay & SWEEP_LINEAR);
            if (n <= LDS_BUDGET) s.lse = SweepLds{lay, P, ch, n};
        }
        if (s.lse.bytes) break;
    }
    // max-plus sweep: mirrored, then plain (the round kernel: one copy, float4 blocks)
    for (int lay : {int(SWEEP_MIRRORED), 0}) {
        if (s.split && (lay & SWEEP_MIRRORED)) continue;
        const int P = s.split ? s.RS + 4 : pitch(lay);
        for (int ch = s.split ? lse_chunk_max(G) : MAXPLUS_CHUNK_MAX; ch >= 4 && s.vit.bytes == 0; ch >>= 1) {
            const size_t n = s.split ? maxplus_round_lds_bytes(C, s.CPr, P, ch, true)
                                     : maxplus_lds_bytes(C, UP, P, ch);
            if (n <= LDS_BUDGET) s.vit = SweepLds{lay, P, ch, n};
        }
        if (s.vit.bytes) break;
    }
    s.ok = s.NT <= 1024 && s.NTv <= 1024 && s.lse.bytes > 0 && s.vit.bytes > 0;
    return s;
}

}  // namespace

XkCfg choose_xk(int C, int K, bool maxp) {
    XkCfg x{};
    x.ok = false;
    if (C < 1 || K < 2) return x;
    // lanes per label and duration weights per lane: a whole wavefront per label with 128
    // weights (512 threads, 256 VGPRs a lane) up to 7 labels, else 64 weights (at most 576
    // threads, 168 VGPRs a lane)
    const int G = C <= 7 ? 64 : C <= 16 ? 32 : C <= 64 ? 8 : 0;
    if (G == 0) return x;
    int kpl = (K - 1 + G - 1) / G;                       // durations k = 2 .. K
    kpl = (kpl + XK_UNROLL - 1) / XK_UNROLL * XK_UNROLL;
    // the instance's register capacity: 32 or 128 weights at G = 64, else 64
    const int kplmax = G == 64 ? (kpl <= 32 ? 32 : 128) : 64;
    if (kpl > kplmax) return x;
    x.G = G;
    x.kplmax = kplmax;
    x.kpl = kpl;
    x.NT = 64 + (C * G + 63) / 64 * 64;
    x.RS = pow2_at_least(K + 2);
    const int NB = x.NT - 64;
    // S chunk: every bulk lane stages at most XK_PF values of it
    x.CH = std::min(64, XK_PF * NB / C);
    if (x.CH < 1) return x;
    // log semiring: a table of each label's total base shift per epoch of XK_REBASE
    // positions, covering more than the K + 2 positions a ring holds
    x.NE = maxp ? 0 : pow2_at_least((K + 2 + 3 * XK_REBASE - 1) / XK_REBASE);
    // S chunks, S(L) and the output history (fp64); transitions, bulk values, rebase
    // shifts, the output history and the shift table (32-bit).  The history holds two
    // chunks of positions, or two positions when the rings are in global memory.
    auto base = [&](int HD) {
        return (size_t)8 * (4 * x.CH * C + C + (maxp ? 1 : 2) * (size_t)HD * C) +
               (size_t)4 * (C * C + 4 * C + C + (maxp ? 2 : 1) * (size_t)HD * C + (size_t)C * x.NE);
    };
    // rings: the one the bulk sums read mirrored in LDS (its log twin, for the log
    // semiring, in global memory) when the window addressing allows it and it fits, else
    // every ring plain in LDS, else every ring in global memory
    const size_t row = (size_t)4 * C * x.RS;
    const bool mir_ok = (size_t)(kplmax - 1) * G <= (size_t)x.RS;
    const size_t bch = base(2 * x.CH);
    if (mir_ok && bch + 2 * row <= LDS_BUDGET) {
        x.ring = XK_RING_MIRRORED;
        x.lds = bch + 2 * row;
    } else if (bch + (maxp ? 1 : 2) * row <= LDS_BUDGET) {
        x.ring = XK_RING_LDS;
        x.lds = bch + (maxp ? 1 : 2) * row;
    } else {
        x.ring = XK_RING_GLOBAL;
        x.lds = base(2);
    }
    x.ok = x.lds <= LDS_BUDGET;
    return x;
}

size_t xk_ring_floats(const XkCfg& xc, int C, int workgroups, bool maxp) {
    if (!xc.ok) return 0;
    return (size_t)workgroups * xk_global_rings(maxp, xc.ring) * C * xc.RS;
}

SweepCfg choose_sweep(int C, int K) {
    SweepCfg s = choose_ring_sweeps(C, K);
    s.xk = false;
    if (K >= XK_FROM || !s.ok) {
        // long durations: the duration weights no longer fit the lanes' registers
        s.xk_lse = choose_xk(C, K, false);
        s.xk_vit = choose_xk(C, K, true);
        if (s.xk_lse.ok && s.xk_vit.ok) {
            s.xk = true;
            s.ok = true;
        }
    }
    return s;
}

// A span's state converges to the exact one (up to a constant) within about 1.25 K
// positions on every workload tried; the seam compares the K positions before the span, so
// the burn-in is 3 K (at least 64 positions for small K).
int spec_warm(int K) { return std::max(3 * K, 64); }

hipError_t launch_lse(const SweepCfg& cfg, const SweepLaunch& a, int ndir, hipStream_t stream) {
    if (cfg.xk) return launch_xk_lse(cfg.xk_lse, a, ndir, stream);
    switch (cfg.lse.layout) {
        case SWEEP_MIRRORED | SWEEP_LINEAR: return launch_lse_mirror(cfg, a, ndir, stream);
        case SWEEP_LINEAR: return launch_lse_plain(cfg, a, ndir, stream);
        case 0: return launch_lse_log(cfg, a, ndir, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_maxplus(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream) {
    if (cfg.xk) return launch_xk_maxplus(cfg.xk_vit, a, stream);
    switch (cfg.vit.layout) {
        case SWEEP_MIRRORED: return launch_maxplus_mirror(cfg, a, stream);
        case 0: return launch_maxplus_plain(cfg, a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace semicrf
