// Viterbi backtrace on gfx950.
//
// The max-plus sweep (sweep.hip, VIT instantiation) stores per position t and label c
// the best duration k of a segment of label c ending at t (low 16 bits) and the best
// previous label for a segment of label c starting at t (high 16 bits), with ties
// resolved to the lowest index.  Walking them from (L, c*) recovers the best
// segmentation: segment [t-k, t) has label c, and the label before it is the
// previous-label field stored at position t-k.
#include "common.h"
#include "internal.h"

namespace semicrf {

// grid (B), block 256.  seg_ws: [B][2*T] int32 scratch for (start, label) pairs.
__global__ __launch_bounds__(256) void k_backtrace(const uint32_t* __restrict__ bp,
                                                   const double* __restrict__ vscore,
                                                   const int* __restrict__ vcstar,
                                                   const int* __restrict__ Leff, int T, int C,
                                                   int32_t* __restrict__ seg_ws,
                                                   float* __restrict__ best_score,
                                                   int32_t* __restrict__ labels,
                                                   uint8_t* __restrict__ seg_start) {
    __shared__ int nseg;
    const int b = blockIdx.x, tid = threadIdx.x;
    const int L = abs(Leff[b]);
    int32_t* ws = seg_ws + (size_t)b * 2 * T;
    const uint32_t* bpb = bp + (size_t)b * (T + 1) * C;
    if (tid == 0) {
        int t = L, c = min(max(vcstar[b], 0), C - 1), n = 0;
        while (t > 0) {
            const uint32_t w = bpb[(size_t)t * C + c];
            const int k = (int)(w & 0xFFFFu);
            const int s = t - k;
            ws[2 * n] = s;
            ws[2 * n + 1] = c;
            ++n;
            if (s <= 0 || k < 1) break;
            c = min((int)(bpb[(size_t)s * C + c] >> 16), C - 1);
            t = s;
        }
        nseg = n;
        best_score[b] = (float)vscore[b];
    }
    __syncthreads();
    const int n = nseg;
    int32_t* lab = labels + (size_t)b * T;
    uint8_t* ss = seg_start + (size_t)b * T;
    // segments were recorded from the end: segment i covers [ws[2i], end_i) with
    // end_0 = L and end_i = start of segment i-1
    for (int i = tid; i < n; i += 256) {
        const int s = ws[2 * i];
        const int c = ws[2 * i + 1];
        const int e = (i == 0) ? L : ws[2 * (i - 1)];
        for (int t = max(s, 0); t < e; ++t) {
            lab[t] = c;
            ss[t] = (t == s) ? 1 : 0;
        }
    }
    for (int t = L + tid; t < T; t += 256) {
        lab[t] = -1;
        ss[t] = 0;
    }
}

hipError_t launch_backtrace(const uint32_t* bp, const double* vscore, const int* vcstar,
                            const int* Leff, int B, int T, int C, int32_t* seg_ws,
                            float* best_score, int32_t* labels, uint8_t* seg_start,
                            hipStream_t stream) {
    hipLaunchKernelGGL(k_backtrace, dim3(B), dim3(256), 0, stream, bp, vscore, vcstar, Leff, T, C,
                       seg_ws, best_score, labels, seg_start);
    return hipGetLastError();
}

}  // namespace semicrf
