// Viterbi end and backtrace on gfx950, the backtrace parallel over chunks of positions.
//
// The max-plus sweep stores per position t and label c the best duration k of a segment
// of label c ending at t (low 16 bits) and the best previous label for a segment of
// label c starting at t (high 16 bits), ties resolved to the lowest index.  A node
// (t, c) is "a segment of label c ends at t"; its successor is (t - k, c') with c' the
// previous-label field at t - k, until t - k = 0.  The chain starts at (L, c*), c* the
// best final label.
//
// A chain has one node per segment and can be as long as the sequence, so it is not
// walked in one lane.  Positions are cut into chunks of W (> K) from the end L: chunk j
// holds ends t in [lo_j, hi_j) with hi_j = L + 1 - j*W.  Since a segment is at most K
// long, the chain enters chunk j at an end t in the top K positions [hi_j - K, hi_j):
// K*C possible entry nodes, numbered e = (hi_j - 1 - t)*C + c.
//   1. k_bt_transfer (all chunks at once): for every entry node of chunk j, the entry
//      node of chunk j+1 its chain reaches (pointer jumping inside the chunk).
//   2. k_bt_compose (one lane per sequence): chain the chunk tables from (L, c*).
//   3. k_bt_fill (all chunks at once): walk each chunk from its actual entry node and
//      write the labels and segment starts of the segments ending inside it.
// The per-chunk tables live in LDS; where a chunk's do not fit (large K) they live in a
// global scratch instead, read and written the same way.
#include "common.h"
#include "internal.h"

namespace semicrf {

namespace {

constexpr int BT_THREADS = 256;
constexpr size_t BT_LDS_MAX = 150 * 1024;

}  // namespace

// one thread per sequence: the best final label over the values V(L, c) of the span that
// holds L (lowest on ties) and the best score in the exact frame (that span's offset);
// vend[b] = {L, c*}
__global__ void k_vit_final(const double* __restrict__ vfin, const double* __restrict__ off,
                            const int* __restrict__ Leff, int B, int C, int delta, int nspans,
                            int* __restrict__ vend, float* __restrict__ best_score) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int L = abs(Leff[b]);
    const int n = (L + delta - 1) / delta;
    double best = -INFINITY;
    int bc = 0;
    for (int c = 0; c < C; ++c) {
        const double v = vfin[(size_t)b * C + c];
        if (v > best) {
            best = v;
            bc = c;
        }
    }
    vend[2 * b] = L;
    vend[2 * b + 1] = bc;
    best_score[b] = Leff[b] < 0 ? __int_as_float(0x7fc00000)
                                : (float)(best + off[(size_t)b * nspans + max(n - 1, 0)]);
}

hipError_t launch_vit_final(const double* vfin, const double* off, const int* Leff, int B,
                            int C, int delta, int nspans, int* vend, float* best_score,
                            hipStream_t stream) {
    hipLaunchKernelGGL(k_vit_final, dim3((B + 255) / 256), dim3(256), 0, stream, vfin, off, Leff,
                       B, C, delta, nspans, vend, best_score);
    return hipGetLastError();
}

// grid (nch, B), block BT_THREADS.  nxt: [W * C] in LDS (GLB false) or the chunk's slice
// of the global scratch gnxt [B][nch][W * C] (GLB true).
// tr: [B][nch][K*C], the entry node of chunk j+1 reached from each entry node of chunk j,
// or -1 when the chain ends inside chunk j (or the entry is not a valid end).
// Every node (t, c) of the chunk first points at its successor (t - k, c') when that lies
// in the chunk, else holds where the chain goes next: the entry node of chunk j+1, or the
// end of the chain.  ceil(log2 W) rounds of pointer jumping (n -> next[next[n]]) then take
// every node to where its chain leaves the chunk.  The rounds update in place: any value
// a lane reads is a node further along the same chain, so the result is the same and the
// distance covered at least doubles per round.
template <bool GLB>
__global__ __launch_bounds__(BT_THREADS) void k_bt_transfer(const uint32_t* __restrict__ bp,
                                                           const int* __restrict__ vend, int B,
                                                           int T, int C, int K, int W, int nch,
                                                           int32_t* __restrict__ tr,
                                                           int* __restrict__ gnxt) {
    extern __shared__ int lnxt[];                        // node n = (t - lo) * C + c
    const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    int* nxt = GLB ? gnxt + ((size_t)b * nch + j) * W * C : lnxt;
    const int E = vend[2 * b];
    const int KC = K * C;
    int32_t* trj = tr + ((size_t)b * nch + j) * KC;
    const int hi = E + 1 - j * W;
    if (hi <= 0) {
        for (int e = tid; e < KC; e += BT_THREADS) trj[e] = -1;
        return;
    }
    const int lo = max(0, hi - W);
    const int rows = hi - lo;                            // <= W
    const uint32_t* bpb = bp + (size_t)b * (T + 1) * C;
    // successors: >= 0 a node of the chunk; -1 the chain ends; -(x + 2) it enters chunk
    // j+1 at entry node x
    for (int n = tid; n < rows * C; n += BT_THREADS) {
        const int t = lo + n / C, c = n - (n / C) * C;
        int v = -1;
        if (t >= 1) {
            const int k = (int)(bpb[(size_t)t * C + c] & 0xFFFFu);
            const int s = t - k;
            if (s > 0 && k >= 1 && k <= K) {
                const int cp = min((int)(bpb[(size_t)s * C + c] >> 16), C - 1);
                v = s >= lo ? (s - lo) * C + cp : -((lo - 1 - s) * C + cp + 2);
            }
        }
        nxt[n] = v;
    }
    __syncthreads();
    for (int span = 1; span < rows; span *= 2) {
        for (int n = tid; n < rows * C; n += BT_THREADS) {
            const int v = nxt[n];
            if (v >= 0) nxt[n] = nxt[v];
        }
        __syncthreads();
    }
    for (int e = tid; e < KC; e += BT_THREADS) {
        const int r = e / C;
        const int t = hi - 1 - r, c = e - r * C;
        int out = -1;
        if (t >= lo && t >= 1) {
            const int v = nxt[(t - lo) * C + c];
            out = v <= -2 ? -v - 2 : -1;
        }
        trj[e] = out;
    }
}

// grid (B), block 64: ent[b][j] = entry node of chunk j on the chain (-1 past its end)
__global__ __launch_bounds__(64) void k_bt_compose(const int32_t* __restrict__ tr,
                                                  const int* __restrict__ vend, int B, int C,
                                                  int K, int nch, int32_t* __restrict__ ent) {
    const int b = blockIdx.x;
    if (threadIdx.x != 0) return;
    const size_t KC = (size_t)K * C;
    const size_t row = (size_t)b * nch;
    int e = min(max(vend[2 * b + 1], 0), C - 1);         // (L, c*): r = 0
    for (int j = 0; j < nch; ++j) {
        ent[row + j] = e;
        if (e >= 0) e = tr[(row + j) * KC + e];
    }
}

// grid (nch, B), block BT_THREADS.  GLB false: the chunk's backpointer rows [lo - K, hi)
// staged in LDS and its segment list [W][3] beside them; GLB true: the rows read from
// global memory and the segment list in the chunk's slice of gseg [B][nch][3 W].
template <bool GLB>
__global__ __launch_bounds__(BT_THREADS) void k_bt_fill(const uint32_t* __restrict__ bp,
                                                       const int* __restrict__ vend,
                                                       const int32_t* __restrict__ ent, int B,
                                                       int T, int C, int K, int W, int nch,
                                                       int* __restrict__ gseg,
                                                       int32_t* __restrict__ labels,
                                                       uint8_t* __restrict__ seg_start) {
    extern __shared__ uint32_t lds_rows[];
    __shared__ int s_nseg;
    const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int E = vend[2 * b], L = E;
    int32_t* lab = labels + (size_t)b * T;
    uint8_t* ss = seg_start + (size_t)b * T;
    if (j == 0)
        for (int u = L + tid; u < T; u += BT_THREADS) {
            lab[u] = -1;
            ss[u] = 0;
        }
    const int hi = E + 1 - j * W;
    if (hi <= 0) return;
    const int lo = max(0, hi - W);
    const int base = max(0, lo - K);
    const int e = ent[(size_t)b * nch + j];
    if (e < 0) return;                                       // chain ended before this chunk
    const uint32_t* bpb = bp + (size_t)b * (T + 1) * C;
    const uint32_t* tile;                                    // row t at tile[(t - base) * C]
    int* segs;                                               // [W][3]: start, end, label
    if constexpr (GLB) {
        tile = bpb + (size_t)base * C;
        segs = gseg + ((size_t)b * nch + j) * 3 * W;
    } else {
        const int cnt = (hi - base) * C;
        for (int q = tid; q < cnt; q += BT_THREADS) lds_rows[q] = bpb[(size_t)base * C + q];
        tile = lds_rows;
        segs = (int*)(lds_rows + (size_t)(hi - base) * C);
        __syncthreads();
    }
    if (tid == 0) {
        const int r = e / C;
        int t = hi - 1 - r, c = e - r * C, n = 0;
        while (t >= 1 && n < W) {
            const int k = (int)(tile[(size_t)(t - base) * C + c] & 0xFFFFu);
            const int s = t - k;
            segs[3 * n] = max(s, 0);
            segs[3 * n + 1] = t;
            segs[3 * n + 2] = c;
            ++n;
            if (s <= 0 || k < 1 || k > K || s < lo) break;   // the next chunk starts at s
            c = min((int)(tile[(size_t)(s - base) * C + c] >> 16), C - 1);
            t = s;
        }
        s_nseg = n;
    }
    __syncthreads();
    const int n = s_nseg;
    if (n == 0) return;
    // the chunk's segments cover [segs[n-1].start, segs[0].end) without gaps, in
    // decreasing order: one lane per position finds its segment by bisection
    const int u0 = segs[3 * (n - 1)], u1 = segs[1];
    for (int u = u0 + tid; u < u1; u += BT_THREADS) {
        int a = 0, z = n - 1;                            // segs[a].start > u >= segs[z].start
        while (a < z) {
            const int m = (a + z) >> 1;
            if (segs[3 * m] <= u) z = m;
            else a = m + 1;
        }
        lab[u] = segs[3 * a + 2];
        ss[u] = (u == segs[3 * a]) ? 1 : 0;
    }
}

int backtrace_chunk(int T, int C, int K) {
    // The fill walks a chunk's chain one segment at a time (up to W steps, short decoded
    // segments make it that long) and the compose walks the chunks one after another
    // ((T + 1) / W steps of about 1.4x a walk step): W ~ 1.2 sqrt(T) balances them.  W > K
    // (a segment never skips a chunk); the LDS form needs (W + K) C + 3 W words.
    const int w = max(64, (int)ceil(1.2 * sqrt((double)T + 1.0)));
    return max(K + 1, min(w, 20480 / max(C, 1) - K));
}

int backtrace_chunks(int T, int C, int K) {
    const int W = backtrace_chunk(T, C, K);
    return (T + 1 + W - 1) / W;
}

bool backtrace_global(int T, int C, int K) {
    const size_t W = (size_t)backtrace_chunk(T, C, K);
    const size_t lds_t = W * C * sizeof(int);
    const size_t lds_f = (W + K) * C * sizeof(uint32_t) + 3 * W * sizeof(int);
    return lds_t > BT_LDS_MAX || lds_f > BT_LDS_MAX;
}

size_t backtrace_scratch_ints(int B, int T, int C, int K) {
    if (!backtrace_global(T, C, K)) return 0;
    const size_t W = (size_t)backtrace_chunk(T, C, K);
    return (size_t)B * backtrace_chunks(T, C, K) * (W * C + 3 * W);
}

hipError_t launch_backtrace(const uint32_t* bp, const int* vend, int B, int T, int C, int K,
                            int32_t* tr, int32_t* ent, int* gscratch, int32_t* labels,
                            uint8_t* seg_start, hipStream_t stream) {
    const int W = backtrace_chunk(T, C, K);
    const int nch = backtrace_chunks(T, C, K);
    if (backtrace_global(T, C, K)) {
        if (!gscratch) return hipErrorInvalidValue;
        int* gnxt = gscratch;
        int* gseg = gscratch + (size_t)B * nch * W * C;
        hipLaunchKernelGGL(k_bt_transfer<true>, dim3(nch, B), dim3(BT_THREADS), 0, stream, bp,
                           vend, B, T, C, K, W, nch, tr, gnxt);
        hipLaunchKernelGGL(k_bt_compose, dim3(B), dim3(64), 0, stream, tr, vend, B, C, K, nch, ent);
        hipLaunchKernelGGL(k_bt_fill<true>, dim3(nch, B), dim3(BT_THREADS), 0, stream, bp, vend,
                           ent, B, T, C, K, W, nch, gseg, labels, seg_start);
    } else {
        const size_t lds_t = (size_t)W * C * sizeof(int);
        const size_t lds_f = (size_t)(W + K) * C * sizeof(uint32_t) + (size_t)3 * W * sizeof(int);
        hipLaunchKernelGGL(k_bt_transfer<false>, dim3(nch, B), dim3(BT_THREADS), lds_t, stream,
                           bp, vend, B, T, C, K, W, nch, tr, nullptr);
        hipLaunchKernelGGL(k_bt_compose, dim3(B), dim3(64), 0, stream, tr, vend, B, C, K, nch, ent);
        hipLaunchKernelGGL(k_bt_fill<false>, dim3(nch, B), dim3(BT_THREADS), lds_f, stream, bp,
                           vend, ent, B, T, C, K, W, nch, nullptr, labels, seg_start);
    }
    return hipGetLastError();
}

}  // namespace semicrf
