// Viterbi backtrace on gfx950, parallel over chunks of positions.
//
// The max-plus sweep stores per position t and label c the best duration k of a segment
// of label c ending at t (low 16 bits) and the best previous label for a segment of
// label c starting at t (high 16 bits), ties resolved to the lowest index.  A node
// (t, c) is "a segment of label c ends at t"; its successor is (t - k, c') with c' the
// previous-label field at t - k, until t - k = 0.  The best segmentation is the chain of
// successors of (L, c*).
//
// The chain has one node per segment and can be as long as the sequence, so it is not
// walked in one lane.  Positions are cut into chunks of W (> K) from the end of the
// sequence: chunk j holds ends t in [lo_j, hi_j) with hi_j = L + 1 - j*W.  Since a
// segment is at most K long, the chain enters chunk j at an end t in the top K positions
// [hi_j - K, hi_j): K*C possible entry nodes, numbered e = (hi_j - 1 - t)*C + c.
//   1. k_bt_transfer (all chunks at once): for every entry node of chunk j, walk inside
//      the chunk (backpointers staged in LDS) to the entry node of chunk j+1 it leads to.
//   2. k_bt_compose (one lane per sequence): chain the chunk tables from (L, c*).
//   3. k_bt_fill (all chunks at once): walk each chunk from its actual entry node and
//      write the labels and segment starts of the segments ending inside it.
#include "common.h"
#include "internal.h"

namespace semicrf {

namespace {

constexpr int BT_THREADS = 256;

// rows [base, hi) of one sequence's backpointers into LDS (row t at tile[(t - base) * C])
__device__ __forceinline__ void stage_rows(uint32_t* tile, const uint32_t* bpb, int base, int hi,
                                           int C) {
    const int cnt = (hi - base) * C;
    const uint32_t* src = bpb + (size_t)base * C;
    for (int q = threadIdx.x; q < cnt; q += BT_THREADS) tile[q] = src[q];
}

}  // namespace

// grid (nch, B), block BT_THREADS, dynamic LDS (W + K) * C * 4 bytes.
// tr: [B][nch][K*C], the entry node of chunk j+1 reached from each entry node of chunk j,
// or -1 when the chain ends inside chunk j (or the entry is not a valid end).
__global__ __launch_bounds__(BT_THREADS) void k_bt_transfer(const uint32_t* __restrict__ bp,
                                                           const int* __restrict__ Leff, int T,
                                                           int C, int K, int W, int nch,
                                                           int32_t* __restrict__ tr) {
    extern __shared__ uint32_t tile[];
    const int j = blockIdx.x, b = blockIdx.y;
    const int L = abs(Leff[b]);
    const int KC = K * C;
    int32_t* trj = tr + ((size_t)b * nch + j) * KC;
    const int hi = L + 1 - j * W;
    if (hi <= 0) {
        for (int e = threadIdx.x; e < KC; e += BT_THREADS) trj[e] = -1;
        return;
    }
    const int lo = max(0, hi - W);
    const int base = max(0, lo - K);
    stage_rows(tile, bp + (size_t)b * (T + 1) * C, base, hi, C);
    __syncthreads();
    for (int e = threadIdx.x; e < KC; e += BT_THREADS) {
        const int r = e / C;
        int t = hi - 1 - r, c = e - r * C;
        int out = -1;
        if (t >= lo && t >= 1) {
            while (true) {
                const int k = (int)(tile[(t - base) * C + c] & 0xFFFFu);
                const int s = t - k;
                if (s <= 0 || k < 1 || k > K) break;        // chain ends (or corrupt entry)
                const int cp = min((int)(tile[(s - base) * C + c] >> 16), C - 1);
                if (s < lo) {                                // leaves the chunk
                    out = (lo - 1 - s) * C + cp;
                    break;
                }
                t = s;
                c = cp;
            }
        }
        trj[e] = out;
    }
}

// grid (B), block 64: ent[b][j] = entry node of chunk j on the best chain (-1 past its end)
__global__ __launch_bounds__(64) void k_bt_compose(const int32_t* __restrict__ tr,
                                                  const double* __restrict__ vscore,
                                                  const int* __restrict__ vcstar, int C, int K,
                                                  int nch, int32_t* __restrict__ ent,
                                                  float* __restrict__ best_score) {
    const int b = blockIdx.x;
    if (threadIdx.x != 0) return;
    const size_t KC = (size_t)K * C;
    int e = min(max(vcstar[b], 0), C - 1);   // (L, c*): r = 0
    for (int j = 0; j < nch; ++j) {
        ent[(size_t)b * nch + j] = e;
        if (e >= 0) e = tr[((size_t)b * nch + j) * KC + e];
    }
    best_score[b] = (float)vscore[b];
}

// grid (nch, B), block BT_THREADS, dynamic LDS (W + K) * C * 4 + 3 * W * 4 bytes.
__global__ __launch_bounds__(BT_THREADS) void k_bt_fill(const uint32_t* __restrict__ bp,
                                                       const int* __restrict__ Leff,
                                                       const int32_t* __restrict__ ent, int T,
                                                       int C, int K, int W, int nch,
                                                       int32_t* __restrict__ labels,
                                                       uint8_t* __restrict__ seg_start) {
    extern __shared__ uint32_t tile[];
    __shared__ int s_nseg;
    const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int L = abs(Leff[b]);
    int32_t* lab = labels + (size_t)b * T;
    uint8_t* ss = seg_start + (size_t)b * T;
    if (j == 0)
        for (int u = L + tid; u < T; u += BT_THREADS) {
            lab[u] = -1;
            ss[u] = 0;
        }
    const int hi = L + 1 - j * W;
    if (hi <= 0) return;
    const int lo = max(0, hi - W);
    const int base = max(0, lo - K);
    int* segs = (int*)(tile + (size_t)(hi - base) * C);     // [W][3]: start, end, label
    const int e = ent[(size_t)b * nch + j];
    if (e < 0) return;                                       // chain ended before this chunk
    stage_rows(tile, bp + (size_t)b * (T + 1) * C, base, hi, C);
    __syncthreads();
    if (tid == 0) {
        const int r = e / C;
        int t = hi - 1 - r, c = e - r * C, n = 0;
        while (t >= 1 && n < W) {
            const int k = (int)(tile[(t - base) * C + c] & 0xFFFFu);
            const int s = t - k;
            segs[3 * n] = max(s, 0);
            segs[3 * n + 1] = t;
            segs[3 * n + 2] = c;
            ++n;
            if (s <= 0 || k < 1 || k > K || s < lo) break;   // the next chunk starts at s
            c = min((int)(tile[(s - base) * C + c] >> 16), C - 1);
            t = s;
        }
        s_nseg = n;
    }
    __syncthreads();
    const int n = s_nseg;
    for (int i = tid; i < n; i += BT_THREADS) {
        const int s = segs[3 * i], t = segs[3 * i + 1], c = segs[3 * i + 2];
        for (int u = s; u < t; ++u) {
            lab[u] = c;
            ss[u] = (u == s) ? 1 : 0;
        }
    }
}

int backtrace_chunk(int C, int K) {
    // W > K (a segment never skips a chunk), LDS of the fill kernel within budget
    return max(K + 1, min(max(1024, 2 * K), 20480 / max(C, 1) - K));
}

int backtrace_chunks(int T, int C, int K) {
    const int W = backtrace_chunk(C, K);
    return (T + 1 + W - 1) / W;
}

hipError_t launch_backtrace(const uint32_t* bp, const double* vscore, const int* vcstar,
                            const int* Leff, int B, int T, int C, int K, int32_t* tr,
                            int32_t* ent, float* best_score, int32_t* labels,
                            uint8_t* seg_start, hipStream_t stream) {
    const int W = backtrace_chunk(C, K);
    const int nch = backtrace_chunks(T, C, K);
    const size_t lds_t = (size_t)(W + K) * C * sizeof(uint32_t);
    const size_t lds_f = lds_t + (size_t)3 * W * sizeof(int);
    if (lds_f > 150 * 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_bt_transfer, dim3(nch, B), dim3(BT_THREADS), lds_t, stream, bp, Leff, T,
                       C, K, W, nch, tr);
    hipLaunchKernelGGL(k_bt_compose, dim3(B), dim3(64), 0, stream, tr, vscore, vcstar, C, K, nch,
                       ent, best_score);
    hipLaunchKernelGGL(k_bt_fill, dim3(nch, B), dim3(BT_THREADS), lds_f, stream, bp, Leff, ent, T,
                       C, K, W, nch, labels, seg_start);
    return hipGetLastError();
}

}  // namespace semicrf
