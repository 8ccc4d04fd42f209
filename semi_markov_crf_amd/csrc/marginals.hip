// Posterior marginals and gradients of log Z on gfx950.
//
// From the per-position forward / backward quantities written by the span recompute
//   XF[s,c] = alpha[s,c]        AF[s,c] = abar[s,c] - S[s,c] + P_start[s,c]
//   XB[s,c] = beta_bar[s,c]     AB[u,c] = beta[u,c] + S[u,c] + P_end[u-1,c] - S[L,c]
// (the boundary projections P_start / P_end are zero when absent) the posterior of one
// segment [s, s+k) of label c is
//   p(s,k,c) = exp(AF[s,c] + AB[s+k,c] + S[L,c] + dur[k-1,c] - logZ)
// and that of a transition c' -> c at s is exp(XF[s,c'] + trans[c',c] + XB[s,c] - logZ).
// Their sums are the gradients of log Z with respect to dur and trans, and the
// position marginal mu[t,c] (the probability that t lies in a segment of label c) is the
// mass of the segments covering t.  The pages validate exactly these quantities
// ("Streaming Structured Inference with Flash-SemiCRF", gist.science EN explainer,
// "4. Results and Benchmarks": marginals sum to 1, exact gradients).
//
// mu is formed as a prefix sum over positions of (start mass - end mass), where both
// masses are sums of the same per-segment values, so each segment's contribution
// cancels exactly once it has ended.  mu is then divided by its sum over labels at each
// position (1 in exact arithmetic).  This per-position normalisation removes the slow
// drift between the forward and backward sweeps' rounding over 10^5..10^6 positions;
// the dur / trans partial sums of a tile are divided by the tile's mean normaliser.
// The start and end masses at each position, divided by the same per-position
// normaliser, are the gradients with respect to the projections; their sum over labels
// at t is the probability that a segment boundary (a segment start) lies at t (the pages
// check that these boundary probabilities are valid at genome scale, "4. Results and
// Benchmarks").
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace semicrf {

// LDS of k_marginals for tile TM and duration chunk KC: the tile's own start / end values,
// the two shifted windows of a chunk, XF / XB, start / end mass accumulators (fp64), the
// chunk's durations and the transitions (fp32).
static size_t marg_lds(int C, int TM, int KC) {
    return (size_t)8 * C * (8 * TM + 2 * KC) + (size_t)4 * ((size_t)KC * C + (size_t)C * C);
}

// Tile and duration chunk.  First choice: the largest tile of at least max(32, K/4)
// positions (the per-tile duration partials, K*C doubles, then take at most as much memory
// as the four per-position input arrays) whose LDS, with a chunk of at least min(K, 64) durations, lets
// three workgroups share a CU (12 wavefronts to hide the latency of the exponentials and
// the fp64 sums).  Otherwise the largest tile that fits one workgroup per CU with such a
// chunk; the smallest tile takes any chunk.
static void marg_shape(int C, int K, int* tm, int* kc) {
    auto chunks = [&](int t, int min_kc, size_t budget) {
        if (K <= 512 && marg_lds(C, t, K) <= budget) return K;
        for (int k = 512; k >= min_kc; k >>= 1)
            if (k < K && marg_lds(C, t, k) <= budget) return k;
        return 0;
    };
    int tmin = 32;
    while (tmin < 512 && 4 * tmin < K) tmin *= 2;
    for (int t = 512; t >= tmin; t >>= 1) {
        const int k = chunks(t, std::min(K, 64), 52 * 1024);
        if (k > 0) {
            *tm = t;
            *kc = k;
            return;
        }
    }
    for (int t = 512; t >= 8; t >>= 1) {
        const int k = chunks(t, t > 8 ? std::min(K, 64) : 1, 150 * 1024);
        if (k > 0) {
            *tm = t;
            *kc = k;
            return;
        }
    }
    *tm = 8;
    *kc = 1;
}

int marg_tile(int C, int K) {
    int tm, kc;
    marg_shape(C, K, &tm, &kc);
    return tm;
}

int marg_kchunk(int C, int K) {
    int tm, kc;
    marg_shape(C, K, &tm, &kc);
    return kc;
}

constexpr double DNEG = -1.0e300;

// grid (ngroups, B), block 256: the tiles g*tpg .. (g+1)*tpg - 1 of sequence b in order.
// Durations are taken in chunks [kc0, kc1] of at most KC: per chunk the starts
// [p0 - kc1, p0 + TM - 1 - kc0] and the ends [p0 + kc0, p0 + TM - 1 + kc1] are staged
// beside the tile's own starts and ends.  The duration and transition partials of the
// group's tiles are summed in tile order (each lane owns the same entries in every tile).
__global__ __launch_bounds__(256) void k_marginals(const MargArgs a) {
    extern __shared__ double lds[];
    const int C = a.C, K = a.K, T = a.T, TM = a.tile, KC = a.kchunk;
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int L = abs(a.Leff[b]);
    const size_t rowC = (size_t)(T + 1) * C;

    double* AFt = lds;                               // [TM][C]: starts p0 .. p0+TM-1
    double* ABt = AFt + (size_t)TM * C;              // [TM][C]: ends p0 .. p0+TM-1
    double* AFw = ABt + (size_t)TM * C;              // [TM+KC][C]: starts of the chunk's ends
    double* ABw = AFw + (size_t)(TM + KC) * C;       // [TM+KC][C]: ends of the chunk's starts
    double* XFs = ABw + (size_t)(TM + KC) * C;       // [TM][C]
    double* XBs = XFs + (size_t)TM * C;              // [TM][C]
    double* Dst = XBs + (size_t)TM * C;              // [TM][C] start mass
    double* Den = Dst + (size_t)TM * C;              // [TM][C] end mass
    float* dur2 = (float*)(Den + (size_t)TM * C);    // [KC][C]
    float* tr2 = dur2 + (size_t)KC * C;              // [C][C]

    double* part_dur = a.part_dur + ((size_t)b * a.ngroups + g) * K * C;
    double* part_trans = a.part_trans + ((size_t)b * a.ngroups + g) * C * C;
    double* Dn = a.Dn + (size_t)b * rowC;
    for (int q = tid; q < C * C; q += 256) tr2[q] = fmaxf((float)((double)a.trans[q] * LOG2E), NEG);
    const int tile_end = min(a.ntiles, (g + 1) * a.tpg);
    for (int tile = g * a.tpg; tile < tile_end; ++tile) {
        const int p0 = tile * TM;
        const bool first = tile == g * a.tpg;    // stores the group's partials, later tiles add
        double* dn_tile = a.dn_tile + ((size_t)b * a.ntiles + tile) * C;
        if (p0 > L) {   // nothing of this sequence here
            for (int q = tid; q < C; q += 256) dn_tile[q] = 0.0;
            for (int q = tid; q < TM * C; q += 256)
                if (p0 + q / C <= T) Dn[(size_t)p0 * C + q] = 0.0;
            if (first) {
                for (int q = tid; q < K * C; q += 256) part_dur[q] = 0.0;
                for (int q = tid; q < C * C; q += 256) part_trans[q] = 0.0;
            }
            continue;
        }
        const double logZ = a.logz[b];
        const double* Sb = a.S + (size_t)b * rowC;
        const double* XF = a.XF + (size_t)b * rowC;
        const double* AF = a.AF + (size_t)b * rowC;
        const double* XB = a.XB + (size_t)b * rowC;
        const double* AB = a.AB + (size_t)b * rowC;
        // frame offsets of the spans that wrote each value (0 without speculative spans):
        // forward X / A of position s from span floor((s-1)/delta) / floor(s/delta), backward
        // ones of s from the mirrored position L - s
        const double* offF = a.off ? a.off + (size_t)b * a.nspans : nullptr;
        const double* offB = a.off ? a.off + ((size_t)a.B + b) * a.nspans : nullptr;
        auto oAF = [&](int s) { return offF ? offF[s / a.delta] : 0.0; };
        auto oXF = [&](int s) { return offF ? offF[(s - 1) / a.delta] : 0.0; };
        auto oAB = [&](int u) { return offB ? offB[(L - u) / a.delta] : 0.0; };
        auto oXB = [&](int s) { return offB ? offB[(L - s - 1) / a.delta] : 0.0; };
        // staged in base 2 (times log2 e); invalid starts / ends get DNEG so that their
        // exponentials vanish
        auto af = [&](int s, int c) -> double {
            return (s >= 0 && s <= L - 1)
                       ? (AF[(size_t)s * C + c] + oAF(s) + Sb[(size_t)L * C + c] - logZ) * LOG2E
                       : DNEG;
        };
        auto ab = [&](int u, int c) -> double {
            return (u >= 1 && u <= L) ? (AB[(size_t)u * C + c] + oAB(u)) * LOG2E : DNEG;
        };

        for (int q = tid; q < TM * C; q += 256) {
            const int r = q / C, c = q - r * C;
            const int s = p0 + r;
            AFt[q] = af(s, c);
            ABt[q] = ab(s, c);
            XFs[q] = (s >= 1 && s <= L - 1) ? (XF[(size_t)s * C + c] + oXF(s)) * LOG2E : DNEG;
            XBs[q] = (s >= 1 && s <= L - 1) ? (XB[(size_t)s * C + c] + oXB(s) - logZ) * LOG2E
                                            : DNEG;
            Dst[q] = 0.0;
            Den[q] = 0.0;
        }

        auto seg = [&](double v, float d) -> float { return fast_exp2((float)v + d); };

        for (int kc0 = 1; kc0 <= K; kc0 += KC) {
            const int kc1 = min(K, kc0 + KC - 1);
            const int nk = kc1 - kc0 + 1;
            __syncthreads();   // the previous chunk's windows are no longer read
            for (int q = tid; q < (TM + nk - 1) * C; q += 256) {
                const int r = q / C, c = q - r * C;
                AFw[q] = af(p0 - kc1 + r, c);
                ABw[q] = ab(p0 + kc0 + r, c);
            }
            for (int q = tid; q < nk * C; q += 256)
                dur2[q] = fmaxf((float)((double)a.dur[(size_t)(kc0 - 1) * C + q] * LOG2E), NEG);
            __syncthreads();

            // ---- phase 1: per position, start and end mass of the chunk's segments
            for (int q = tid; q < TM * C; q += 256) {
                const int r = q / C, c = q - r * C;
                if (p0 + r > L) continue;
                double st = Dst[q], en = Den[q];
                const double a0 = AFt[q], b0 = ABt[q];
#pragma unroll 4
                for (int k = kc0; k <= kc1; ++k) {
                    const float d = dur2[(k - kc0) * C + c];
                    st += (double)seg(a0 + ABw[(size_t)(r + k - kc0) * C + c], d);   // [t, t+k)
                    en += (double)seg(AFw[(size_t)(r + kc1 - k) * C + c] + b0, d);   // [t-k, t)
                }
                Dst[q] = st;
                Den[q] = en;
            }

            // ---- phase 2: duration partials, lanes over (k, c), segments starting in the tile
            for (int q = tid; q < nk * C; q += 256) {
                const int kk = q / C, c = q - kk * C;
                const float d = dur2[q];
                double acc = 0.0;
#pragma unroll 4
                for (int r = 0; r < TM; ++r)
                    acc += (double)seg(AFt[(size_t)r * C + c] + ABw[(size_t)(r + kk) * C + c], d);
                double* pd = part_dur + (size_t)(kc0 - 1) * C + q;
            *pd = first ? acc : *pd + acc;
            }
        }
        __syncthreads();

        // ---- start mass - end mass per position, the tile's sums, boundary masses
        for (int q = tid; q < TM * C; q += 256) {
            const int r = q / C, c = q - r * C;
            const int t = p0 + r;
            const double st = Dst[q], en = Den[q];
            const double d = st - en;
            Dst[q] = d;
            if (t <= T) Dn[(size_t)t * C + c] = d;
            if (a.pstart && t < L) a.pstart[((size_t)b * T + t) * C + c] = (float)st;
            if (a.pend && t >= 1 && t <= L) a.pend[((size_t)b * T + t - 1) * C + c] = (float)en;
        }
        __syncthreads();
        for (int c = tid; c < C; c += 256) {
            double s = 0.0;
            for (int r = 0; r < TM; ++r) s += Dst[(size_t)r * C + c];
            dn_tile[c] = s;
        }

        // ---- phase 3: transition partials, lanes over (c', c)
        for (int q = tid; q < C * C; q += 256) {
            const int cp = q / C, c = q - cp * C;
            const float tv = tr2[q];
            double acc = 0.0;
            for (int r = 0; r < TM; ++r) {
                const double v = XFs[(size_t)r * C + cp] + XBs[(size_t)r * C + c];
                acc += (double)fast_exp2((float)v + tv);
            }
            part_trans[q] = first ? acc : part_trans[q] + acc;
        }
        __syncthreads();   // the tile's LDS is read no more
    }
}

hipError_t launch_marginals(const MargArgs& a, hipStream_t stream) {
    const size_t lds = marg_lds(a.C, a.tile, a.kchunk);
    if (a.tpg < 1 || a.ngroups != (a.ntiles + a.tpg - 1) / a.tpg) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_marginals, dim3(a.ngroups, a.B), dim3(256), lds, stream, a);
    return hipGetLastError();
}

int marg_tiles_per_group(int B, int ntiles, int C, int K) {
    // a group per tile while the partials stay within the budget (longer workgroups leave
    // the device's last pass over them mostly idle: four tiles a group cost 45 % more time
    // at B = 4, T = 10^5, K = 200), else the fewest tiles a group that meet it
    constexpr size_t BUDGET = (size_t)64 << 20;          // bytes of partials
    constexpr long long TARGET = 8192;                   // workgroups
    int tpg = (int)std::max<long long>(1, ((long long)B * ntiles + TARGET - 1) / TARGET);
    auto bytes = [&](int t) {
        return (size_t)B * ((ntiles + t - 1) / t) * (size_t)(K + C) * C * sizeof(double);
    };
    while (tpg < ntiles && bytes(tpg) > BUDGET) tpg *= 2;
    return std::min(tpg, std::max(ntiles, 1));
}

// grid (ntiles, B), block 256: mu over positions [p0, p0+TM) of the prefix sum of Dn,
// normalised per position; tile sums of mu and the tile's mean normaliser.
__global__ __launch_bounds__(256) void k_node_marginals(const double* __restrict__ Dn,
                                                        const double* __restrict__ dn_off,
                                                        const int* __restrict__ Leff, int T, int C,
                                                        int TM, float* __restrict__ mu,
                                                        double* __restrict__ mu_tile,
                                                        double* __restrict__ z_tile,
                                                        const BoundaryOut bo) {
    extern __shared__ double lds[];
    const int tile = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, ntiles = gridDim.x;
    const int L = abs(Leff[b]);
    const int p0 = tile * TM;
    double* v = lds;                       // [TM][C]
    double* csum = v + (size_t)TM * C;     // [256]
    double* zrow = csum + 256;             // [TM]
    const double* D = Dn + (size_t)b * (T + 1) * C;
    const int rows = max(0, min(TM, L - p0));   // positions p0 .. p0+rows-1 are < L
    for (int q = tid; q < rows * C; q += 256) v[q] = D[(size_t)p0 * C + q];
    __syncthreads();
    const double* off = dn_off + ((size_t)b * ntiles + tile) * C;
    for (int c0 = 0; c0 < C; c0 += 256) {
        const int CW = min(256, C - c0);
        const int R = 256 / CW;
        const int chunk = (rows + R - 1) / R;
        const int cw = tid % CW, r = tid / CW, c = c0 + cw;
        const bool act = r < R;
        double acc = 0.0;
        if (act)
            for (int i = r * chunk; i < min(rows, (r + 1) * chunk); ++i) acc += v[(size_t)i * C + c];
        csum[tid] = acc;
        __syncthreads();
        if (act) {
            double run = off[c];
            for (int qq = 0; qq < r; ++qq) run += csum[qq * CW + cw];
            for (int i = r * chunk; i < min(rows, (r + 1) * chunk); ++i) {
                run += v[(size_t)i * C + c];
                v[(size_t)i * C + c] = run;
            }
        }
        __syncthreads();
    }
    for (int r = tid; r < rows; r += 256) {
        double z = 0.0;
        for (int c = 0; c < C; ++c) z += v[(size_t)r * C + c];
        zrow[r] = z;
    }
    __syncthreads();
    if (bo.node_mass)
        for (int r = tid; r < TM; r += 256) {
            const int t = p0 + r;
            if (t < T) bo.node_mass[(size_t)b * T + t] = r < rows ? (float)zrow[r] : 0.0f;
        }
    if (bo.pstart) {
        // boundary probabilities and the projections' gradients: the raw start / end
        // masses over the same per-position normaliser (0 at padding)
        const size_t base = (size_t)b * T * C;
        const double g = bo.grad_log_z ? (double)bo.grad_log_z[b] : 1.0;
        for (int r = tid; r < TM; r += 256) {
            const int t = p0 + r;
            if (t >= T || !bo.boundary) continue;
            double s = 0.0;
            if (r < rows)
                for (int c = 0; c < C; ++c) s += (double)bo.pstart[base + (size_t)t * C + c];
            bo.boundary[(size_t)b * T + t] = r < rows ? (float)(s / zrow[r]) : 0.0f;
        }
        for (int q = tid; q < TM * C; q += 256) {
            const int r = q / C;
            const int t = p0 + r;
            if (t >= T) continue;
            const size_t idx = base + (size_t)p0 * C + q;
            const bool in = r < rows;
            if (bo.grad_proj_start)
                bo.grad_proj_start[idx] = in ? (float)(g * (double)bo.pstart[idx] / zrow[r]) : 0.0f;
            if (bo.grad_proj_end)
                bo.grad_proj_end[idx] = in ? (float)(g * (double)bo.pend[idx] / zrow[r]) : 0.0f;
        }
    }
    float* mub = mu + (size_t)b * T * C;
    for (int q = tid; q < TM * C; q += 256) {
        const int r = q / C;
        const int t = p0 + r;
        if (t >= T) continue;
        float val = 0.0f;
        if (r < rows) {
            const double w = v[q] / zrow[r];
            v[q] = w;
            val = (float)w;
        }
        mub[(size_t)t * C + (q - r * C)] = val;
    }
    __syncthreads();
    for (int c = tid; c < C; c += 256) {
        double s = 0.0;
        for (int r = 0; r < rows; ++r) s += v[(size_t)r * C + c];
        mu_tile[((size_t)b * ntiles + tile) * C + c] = s;
    }
    if (tid == 0) {
        double z = 0.0;
        for (int r = 0; r < rows; ++r) z += zrow[r];
        z_tile[(size_t)b * ntiles + tile] = rows > 0 ? z / rows : 1.0;
    }
}

hipError_t launch_node_marginals(const double* Dn, const double* dn_off, const int* Leff, int B,
                                 int T, int C, int tile, int ntiles, float* mu, double* mu_tile,
                                 double* z_tile, const BoundaryOut& bo, hipStream_t stream) {
    const size_t lds = (size_t)8 * ((size_t)tile * C + 256 + tile);
    hipLaunchKernelGGL(k_node_marginals, dim3(ntiles, B), dim3(256), lds, stream, Dn, dn_off, Leff,
                       T, C, tile, mu, mu_tile, z_tile, bo);
    return hipGetLastError();
}

// grid (ceil(T*C/256), B): grad_em = g * (mu - mean over the valid positions of mu)
__global__ __launch_bounds__(256) void k_grad_em(const float* __restrict__ mu,
                                                 const double* __restrict__ mu_tot,
                                                 const int* __restrict__ Leff,
                                                 const float* __restrict__ grad_log_z, int T,
                                                 int C, float* __restrict__ grad_em) {
    const int b = blockIdx.y;
    const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (size_t)T * C) return;
    const int L = abs(Leff[b]);
    const int t = (int)(q / C), c = (int)(q - (size_t)t * C);
    const size_t idx = (size_t)b * T * C + q;
    float out = 0.0f;
    if (t < L) {
        const double g = grad_log_z ? (double)grad_log_z[b] : 1.0;
        out = (float)(g * ((double)mu[idx] - mu_tot[(size_t)b * C + c] / (double)L));
    }
    grad_em[idx] = out;
}

hipError_t launch_grad_em(const float* mu, const double* mu_tot, const int* Leff,
                          const float* grad_log_z, int B, int T, int C, float* grad_em,
                          hipStream_t stream) {
    const size_t n = (size_t)T * C;
    hipLaunchKernelGGL(k_grad_em, dim3((unsigned)((n + 255) / 256), B), dim3(256), 0, stream, mu,
                       mu_tot, Leff, grad_log_z, T, C, grad_em);
    return hipGetLastError();
}

// one thread per output element of grad_dur [K*C] followed by grad_trans [C*C]
// grad_dur / grad_trans = sum over sequences b of g_b * sum over tile groups j of
// part[b][j] / z_j, z_j the mean per-position normaliser over the group's valid positions
// (it drifts by far less than 1e-6 across a group).  Pass 1: grid (ceil(n / 64),
// RP_SLICES / 4), block 256; lane (e, slice) sums the groups j = slice, slice + RP_SLICES,
// ... of every sequence into scratch[slice][e].  Pass 2: one lane per output adds the
// slices in order.  Fixed order throughout: bitwise reproducible.
constexpr int RP_SLICES = 128;

__global__ __launch_bounds__(256) void k_reduce_partials(const double* __restrict__ part_dur,
                                                         const double* __restrict__ part_trans,
                                                         const double* __restrict__ z_tile,
                                                         const int* __restrict__ Leff,
                                                         const float* __restrict__ grad_log_z,
                                                         int B, int C, int K, int TM, int ntiles,
                                                         int tpg, int ngroups,
                                                         double* __restrict__ scratch) {
    const int n = K * C + C * C;
    const int e = blockIdx.x * 64 + (threadIdx.x & 63);
    const int slice = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (e >= n) return;
    const int nd = K * C;
    const bool isd = e < nd;
    const int ee = isd ? e : e - nd;
    const int stride = isd ? nd : C * C;
    const double* src = isd ? part_dur : part_trans;
    double total = 0.0;
    for (int b = 0; b < B; ++b) {
        const int L = abs(Leff[b]);
        double s = 0.0;
        for (int j = slice; j < ngroups; j += RP_SLICES) {
            double zs = 0.0, ns = 0.0;
            for (int tl = j * tpg; tl < min(ntiles, (j + 1) * tpg); ++tl) {
                const int rows = max(0, min(TM, L - tl * TM));
                zs += (double)rows * z_tile[(size_t)b * ntiles + tl];
                ns += (double)rows;
            }
            s += src[((size_t)b * ngroups + j) * stride + ee] / (ns > 0.0 ? zs / ns : 1.0);
        }
        total += (grad_log_z ? (double)grad_log_z[b] : 1.0) * s;
    }
    scratch[(size_t)slice * n + e] = total;
}

__global__ __launch_bounds__(256) void k_reduce_slices(const double* __restrict__ scratch, int C,
                                                       int K, float* __restrict__ grad_dur,
                                                       float* __restrict__ grad_trans) {
    const int n = K * C + C * C;
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    double total = 0.0;
    for (int sl = 0; sl < RP_SLICES; ++sl) total += scratch[(size_t)sl * n + e];
    if (e < K * C) grad_dur[e] = (float)total;
    else grad_trans[e - K * C] = (float)total;
}

size_t reduce_scratch_doubles(int C, int K) { return (size_t)RP_SLICES * (K * C + C * C); }

hipError_t launch_reduce_partials(const double* part_dur, const double* part_trans,
                                  const double* z_tile, const int* Leff, const float* grad_log_z,
                                  int B, int C, int K, int tile, int ntiles, int tpg,
                                  double* scratch, float* grad_dur, float* grad_trans,
                                  hipStream_t stream) {
    const int n = K * C + C * C;
    const int ngroups = (ntiles + tpg - 1) / tpg;
    hipLaunchKernelGGL(k_reduce_partials, dim3((n + 63) / 64, RP_SLICES / 4), dim3(256), 0, stream,
                       part_dur, part_trans, z_tile, Leff, grad_log_z, B, C, K, tile, ntiles,
                       tpg, ngroups, scratch);
    hipLaunchKernelGGL(k_reduce_slices, dim3((n + 255) / 256), dim3(256), 0, stream, scratch, C, K,
                       grad_dur, grad_trans);
    return hipGetLastError();
}

__global__ void k_write_logz(const double* __restrict__ logz, int B, float* __restrict__ out) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) out[b] = (float)logz[b];
}

hipError_t launch_write_logz(const double* logz, int B, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(k_write_logz, dim3((B + 255) / 256), dim3(256), 0, stream, logz, B, out);
    return hipGetLastError();
}

}  // namespace semicrf
