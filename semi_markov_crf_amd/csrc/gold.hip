// Training loss of gold segmentations on gfx950: nll[b] = log Z_b - score_b(y*), and
// the gold half of its gradients.
//
// The score of a segmentation sums, over its segments [s, e) of label c, the potential
// S[e,c] - S[s,c] + dur[e-s-1, c] (+ the boundary projections P_start[s,c] + P_end[e-1,c])
// and, between consecutive segments, trans[c', c] -- the same centred, additive potential
// as log Z ("Streaming Structured Inference with Flash-SemiCRF", gist.science EN
// explainer, "2. Methodology").  nll is the negative
// log-probability of y*, the training loss of the pages' convergence check ("4. Results
// and Benchmarks"); its gradient is the posterior expectation of the features (the
// gradients of log Z, from the backward pass) minus the features of y*.
//
//   k_gold_zero      clear the per-sequence counters
//   k_gold_segments  grid (ceil(T/256), B): a lane per position; a lane at a segment
//                    start walks to the segment's end, checks it (length <= K, one
//                    label), adds its score to a fixed-order block sum and its feature
//                    counts to integer counters (atomics on integers: exact, any order)
//   k_gold_finish    grid (B): fixed-order sum of the block sums; nll = log Z - score,
//                    NaN and the status flag for an invalid length or segmentation
//   k_gold_params    grad_dur / grad_trans -= sum_b g_b * counts (fixed order over b)
//   k_gold_em        grad_em[b,t,c] -= g_b * (1[y*_t = c] - n_c / L)  (the centring);
//                    grad_proj_start / grad_proj_end -= g_b * the gold segments'
//                    start / last-position indicators
// A sequence whose gold segmentation is invalid keeps only its log Z half of the
// gradients.
#include "common.h"
#include "internal.h"

namespace semicrf {

namespace {
constexpr int GT = 256;    // positions per block of k_gold_segments
}

int gold_blocks(int T) { return (T + GT - 1) / GT; }

// counters per sequence: [K*C] segment lengths, [C*C] transitions, [C] labelled
// positions, [1] invalid flag
__global__ void k_gold_zero(int* __restrict__ cnt, int n) {
    const int q = blockIdx.x * 256 + threadIdx.x;
    if (q < n) cnt[q] = 0;
}

__global__ __launch_bounds__(GT) void k_gold_segments(const GoldArgs g) {
    __shared__ double red[GT / 64];
    const int b = blockIdx.y, tid = threadIdx.x;
    const int t = blockIdx.x * GT + tid;
    const int C = g.C, K = g.K, T = g.T;
    const int L = abs(g.Leff[b]);
    const int ncnt = K * C + C * C + C + 1;
    int* cnt = g.cnt + (size_t)b * ncnt;
    const int32_t* lab = g.labels + (size_t)b * T;
    const uint8_t* st = g.seg_start + (size_t)b * T;
    const double* S = g.S + (size_t)b * (T + 1) * C;
    double v = 0.0;
    if (t < L) {
        const int c = lab[t];
        bool bad = (c < 0) | (c >= C) | (t == 0 && st[0] == 0);
        if (!bad && (t == 0 || st[t])) {
            // this segment's end: the next start, or L; longer than K is invalid
            int e = t + 1;
            while (e < L && !st[e] && e - t <= K) {
                bad |= lab[e] != c;
                ++e;
            }
            const int k = e - t;
            bad |= k > K;
            if (!bad) {
                v = S[(size_t)e * C + c] - S[(size_t)t * C + c] + (double)g.dur[(k - 1) * C + c];
                if (g.proj_start) v += (double)g.proj_start[((size_t)b * T + t) * C + c];
                if (g.proj_end) v += (double)g.proj_end[((size_t)b * T + e - 1) * C + c];
                atomicAdd(cnt + (k - 1) * C + c, 1);
                atomicAdd(cnt + K * C + C * C + c, k);
                if (t > 0) {
                    const int cp = lab[t - 1];
                    if (cp >= 0 && cp < C) {
                        v += (double)g.trans[cp * C + c];
                        atomicAdd(cnt + K * C + cp * C + c, 1);
                    }
                }
            }
        }
        if (bad) atomicOr(cnt + ncnt - 1, 1);
    }
    // fixed-order block sum of the segment scores
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    if (tid == 0) {
        double s = 0.0;
        for (int w = 0; w < GT / 64; ++w) s += red[w];
        g.part[(size_t)b * gridDim.x + blockIdx.x] = s;
    }
}

// grid (B), block 256
__global__ __launch_bounds__(256) void k_gold_finish(const GoldArgs g, int nblk) {
    __shared__ double scratch[16];
    const int b = blockIdx.x;
    double s = 0.0;
    for (int j = threadIdx.x; j < nblk; j += 256) s += g.part[(size_t)b * nblk + j];
    s = block_sum_double(s, scratch);
    if (threadIdx.x == 0) {
        const int ncnt = g.K * g.C + g.C * g.C + g.C + 1;
        const bool bad = g.Leff[b] < 0 || g.cnt[(size_t)b * ncnt + ncnt - 1] != 0;
        g.nll[b] = bad ? __int_as_float(0x7fc00000) : (float)(g.logz[b] - s);
        if (bad) g.status[0] = 1;
    }
}

// grid (ceil((K*C + C*C) / 256)), block 256
__global__ __launch_bounds__(256) void k_gold_params(const GoldArgs g) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int nd = g.K * g.C, n = nd + g.C * g.C;
    if (e >= n) return;
    const int ncnt = n + g.C + 1;
    double s = 0.0;
    for (int b = 0; b < g.B; ++b) {
        const int* cnt = g.cnt + (size_t)b * ncnt;
        if (cnt[ncnt - 1]) continue;   // invalid gold segmentation: no gold counts
        s += (g.grad_nll ? (double)g.grad_nll[b] : 1.0) * (double)cnt[e];
    }
    float* out = e < nd ? g.grad_dur + e : g.grad_trans + (e - nd);
    *out = (float)((double)*out - s);
}

// grid (ceil(T*C / 256), B), block 256
__global__ __launch_bounds__(256) void k_gold_em(const GoldArgs g) {
    const int b = blockIdx.y;
    const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
    const int C = g.C, T = g.T;
    if (q >= (size_t)T * C) return;
    const int t = (int)(q / C), c = (int)(q - (size_t)t * C);
    const int L = abs(g.Leff[b]);
    if (t >= L) return;
    const int ncnt = g.K * C + C * C + C + 1;
    const int* cnt = g.cnt + (size_t)b * ncnt;
    if (cnt[ncnt - 1]) return;   // invalid gold segmentation: no gold counts
    const double gb = g.grad_nll ? (double)g.grad_nll[b] : 1.0;
    const bool lab = g.labels[(size_t)b * T + t] == c;
    const double ind = lab ? 1.0 : 0.0;
    const double mean = (double)cnt[g.K * C + C * C + c] / (double)L;
    const size_t idx = ((size_t)b * T + t) * C + c;
    float* out = g.grad_em + idx;
    *out = (float)((double)*out - gb * (ind - mean));
    const uint8_t* st = g.seg_start + (size_t)b * T;
    if (g.grad_proj_start && lab && (t == 0 || st[t]))
        g.grad_proj_start[idx] = (float)((double)g.grad_proj_start[idx] - gb);
    if (g.grad_proj_end && lab && (t + 1 == L || st[t + 1]))
        g.grad_proj_end[idx] = (float)((double)g.grad_proj_end[idx] - gb);
}

hipError_t launch_gold(const GoldArgs& g, hipStream_t stream) {
    const int ncnt = g.K * g.C + g.C * g.C + g.C + 1;
    const int nz = g.B * ncnt;
    const int nblk = gold_blocks(g.T);
    hipLaunchKernelGGL(k_gold_zero, dim3((nz + 255) / 256), dim3(256), 0, stream, g.cnt, nz);
    hipLaunchKernelGGL(k_gold_segments, dim3(nblk, g.B), dim3(GT), 0, stream, g);
    hipLaunchKernelGGL(k_gold_finish, dim3(g.B), dim3(256), 0, stream, g, nblk);
    const int np = g.K * g.C + g.C * g.C;
    hipLaunchKernelGGL(k_gold_params, dim3((np + 255) / 256), dim3(256), 0, stream, g);
    const size_t tc = (size_t)g.T * g.C;
    hipLaunchKernelGGL(k_gold_em, dim3((unsigned)((tc + 255) / 256), g.B), dim3(256), 0, stream, g);
    return hipGetLastError();
}

}  // namespace semicrf
