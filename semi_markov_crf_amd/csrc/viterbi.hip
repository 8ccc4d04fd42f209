// Viterbi combine and backtrace on gfx950, the backtrace parallel over chunks of positions.
//
// The max-plus sweep stores per position t and label c the best duration k of a segment
// of label c ending at t (low 16 bits) and the best previous label for a segment of
// label c starting at t (high 16 bits), ties resolved to the lowest index.  A node
// (t, c) is "a segment of label c ends at t"; its successor is (t - k, c') with c' the
// previous-label field at t - k, until t - k = 0.
//
// With the two-direction sweep (C <= 16) the best segmentation is split at a boundary
// t* of the meeting window: part 0 is the chain of forward backpointers from (t*, c_left)
// and part 1 the chain of the mirrored sequence's backpointers from (L - t*, c_right),
// whose segments map back to [t*, L).  The one-direction sweep gives t* = L and an empty
// part 1.
//
// A chain has one node per segment and can be as long as the sequence, so it is not
// walked in one lane.  Positions are cut into chunks of W (> K) from the chain's end E:
// chunk j holds ends t in [lo_j, hi_j) with hi_j = E + 1 - j*W.  Since a segment is at
// most K long, the chain enters chunk j at an end t in the top K positions
// [hi_j - K, hi_j): K*C possible entry nodes, numbered e = (hi_j - 1 - t)*C + c.
//   1. k_bt_transfer (all chunks at once): for every entry node of chunk j, walk inside
//      the chunk (backpointers staged in LDS) to the entry node of chunk j+1 it leads to.
//   2. k_bt_compose (one lane per chain): chain the chunk tables from (E, c0).
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

// chain end E and start label of part `part` of sequence b; split[b] = {t*, c_left,
// c_right, L}
__device__ __forceinline__ void part_of(const int* split, int b, int part, int* E, int* c0) {
    const int* sp = split + 4 * b;
    *E = part == 0 ? sp[0] : sp[3] - sp[0];
    *c0 = part == 0 ? sp[1] : sp[2];
}

}  // namespace

// grid (B), block 256: split[b] and best_score[b] from the meeting window (bidir) or from
// the one-direction sweep's end (t* = L).  The window candidates are t in [lo, mm], c, c'
// with V(t, c) + trans[c][c'] + W(t, c') for 0 < t < L, W(0, c') at t = 0 and V(L, c) at
// t = L; the largest wins, the lowest (t, c, c') on ties.
__global__ __launch_bounds__(256) void k_vit_combine(const double* __restrict__ vwin,
                                                    const float* __restrict__ trans,
                                                    const int* __restrict__ Leff, int B, int C,
                                                    int K, int bidir,
                                                    const double* __restrict__ vscore,
                                                    const int* __restrict__ vcstar,
                                                    int* __restrict__ split,
                                                    float* __restrict__ best_score) {
    __shared__ double sv[256];
    __shared__ int si[256];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int Lr = Leff[b];
    const int L = abs(Lr);
    if (!bidir) {
        if (tid == 0) {
            split[4 * b] = L;
            split[4 * b + 1] = min(max(vcstar[b], 0), C - 1);
            split[4 * b + 2] = 0;
            split[4 * b + 3] = L;
            best_score[b] = (float)vscore[b];
        }
        return;
    }
    const int mm = min(L, (L + K - 1) / 2);
    const int lo = max(0, mm - K + 1);
    const int n = (mm - lo + 1) * C * C;
    const double* V = vwin + (size_t)b * K * C;
    const double* Wv = vwin + ((size_t)B + b) * K * C;
    double best = -INFINITY;
    int bi = INT_MAX;
    for (int q = tid; q < n; q += 256) {                 // ascending: first maximum kept
        const int i = q / (C * C), r = q - i * C * C;
        const int c = r / C, c2 = r - c * C;
        const int t = lo + i;
        double v;
        if (t == 0) {
            if (c != 0) continue;
            v = Wv[i * C + c2];
        } else if (t == L) {
            if (c2 != 0) continue;
            v = V[i * C + c];
        } else {
            v = V[i * C + c] + (double)trans[c * C + c2] + Wv[i * C + c2];
        }
        if (v > best) {
            best = v;
            bi = q;
        }
    }
    sv[tid] = best;
    si[tid] = bi;
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
        if (tid < st) {
            const double o = sv[tid + st];
            const int oi = si[tid + st];
            if (o > sv[tid] || (o == sv[tid] && oi < si[tid])) {
                sv[tid] = o;
                si[tid] = oi;
            }
        }
        __syncthreads();
    }
    if (tid == 0) {
        const int q = si[0] == INT_MAX ? 0 : si[0];      // no finite candidate: any split
        const int i = q / (C * C), r = q - i * C * C;
        split[4 * b] = lo + i;
        split[4 * b + 1] = r / C;
        split[4 * b + 2] = r - (r / C) * C;
        split[4 * b + 3] = L;
        best_score[b] = Lr < 0 ? __int_as_float(0x7fc00000) : (float)sv[0];
    }
}

// one thread per sequence: the best final label of the forward decode over speculative
// spans (lowest on ties) and its score in the exact frame (the last span's offset)
__global__ void k_vit_final(const double* __restrict__ vfin, const double* __restrict__ off,
                            const int* __restrict__ Leff, int B, int C, int delta, int nspans,
                            double* __restrict__ vscore, int* __restrict__ vcstar) {
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
    vscore[b] = Leff[b] < 0 ? __longlong_as_double(0x7ff8000000000000LL)
                            : best + off[(size_t)b * nspans + max(n - 1, 0)];
    vcstar[b] = bc;
}

hipError_t launch_vit_final(const double* vfin, const double* off, const int* Leff, int B,
                            int C, int delta, int nspans, double* vscore, int* vcstar,
                            hipStream_t stream) {
    hipLaunchKernelGGL(k_vit_final, dim3((B + 255) / 256), dim3(256), 0, stream, vfin, off, Leff,
                       B, C, delta, nspans, vscore, vcstar);
    return hipGetLastError();
}

// grid (nch, B, 2 parts), block BT_THREADS, dynamic LDS W * C * 4 bytes.
// tr: [2][B][nch][K*C], the entry node of chunk j+1 reached from each entry node of chunk
// j, or -1 when the chain ends inside chunk j (or the entry is not a valid end).
// Every node (t, c) of the chunk first points at its successor (t - k, c') when that lies
// in the chunk, else holds where the chain goes next: the entry node of chunk j+1, or the
// end of the chain.  ceil(log2 W) rounds of pointer jumping (n -> next[next[n]]) then take
// every node to where its chain leaves the chunk.  The rounds update in place: any value
// a lane reads is a node further along the same chain, so the result is the same and the
// distance covered at least doubles per round.
__global__ __launch_bounds__(BT_THREADS) void k_bt_transfer(const uint32_t* __restrict__ bp,
                                                           const int* __restrict__ split, int B,
                                                           int T, int C, int K, int W, int nch,
                                                           int32_t* __restrict__ tr) {
    extern __shared__ int nxt[];                         // [W * C]: node n = (t - lo) * C + c
    const int j = blockIdx.x, b = blockIdx.y, part = blockIdx.z, tid = threadIdx.x;
    int E, c0;
    part_of(split, b, part, &E, &c0);
    const int KC = K * C;
    int32_t* trj = tr + (((size_t)part * B + b) * nch + j) * KC;
    const int hi = E + 1 - j * W;
    if (hi <= 0) {
        for (int e = tid; e < KC; e += BT_THREADS) trj[e] = -1;
        return;
    }
    const int lo = max(0, hi - W);
    const int rows = hi - lo;                            // <= W
    const uint32_t* bpb = bp + ((size_t)part * B + b) * (T + 1) * C;
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

// grid (B, 2 parts), block 64: ent[part][b][j] = entry node of chunk j on the chain (-1
// past its end)
__global__ __launch_bounds__(64) void k_bt_compose(const int32_t* __restrict__ tr,
                                                  const int* __restrict__ split, int B, int C,
                                                  int K, int nch, int32_t* __restrict__ ent) {
    const int b = blockIdx.x, part = blockIdx.y;
    if (threadIdx.x != 0) return;
    int E, c0;
    part_of(split, b, part, &E, &c0);
    const size_t KC = (size_t)K * C;
    const size_t row = ((size_t)part * B + b) * nch;
    int e = min(max(c0, 0), C - 1);          // (E, c0): r = 0
    for (int j = 0; j < nch; ++j) {
        ent[row + j] = e;
        if (e >= 0) e = tr[(row + j) * KC + e];
    }
}

// grid (nch, B, 2 parts), block BT_THREADS, dynamic LDS (W + K) * C * 4 + 3 * W * 4 bytes.
// Part 1 walks the mirrored sequence: its segment [s, t) covers original [L - t, L - s).
__global__ __launch_bounds__(BT_THREADS) void k_bt_fill(const uint32_t* __restrict__ bp,
                                                       const int* __restrict__ split,
                                                       const int32_t* __restrict__ ent, int B,
                                                       int T, int C, int K, int W, int nch,
                                                       int32_t* __restrict__ labels,
                                                       uint8_t* __restrict__ seg_start) {
    extern __shared__ uint32_t tile[];
    __shared__ int s_nseg;
    const int j = blockIdx.x, b = blockIdx.y, part = blockIdx.z, tid = threadIdx.x;
    int E, c0;
    part_of(split, b, part, &E, &c0);
    const int L = split[4 * b + 3];
    int32_t* lab = labels + (size_t)b * T;
    uint8_t* ss = seg_start + (size_t)b * T;
    if (j == 0 && part == 0)
        for (int u = L + tid; u < T; u += BT_THREADS) {
            lab[u] = -1;
            ss[u] = 0;
        }
    const int hi = E + 1 - j * W;
    if (hi <= 0) return;
    const int lo = max(0, hi - W);
    const int base = max(0, lo - K);
    int* segs = (int*)(tile + (size_t)(hi - base) * C);     // [W][3]: start, end, label
    const int e = ent[((size_t)part * B + b) * nch + j];
    if (e < 0) return;                                       // chain ended before this chunk
    stage_rows(tile, bp + ((size_t)part * B + b) * (T + 1) * C, base, hi, C);
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
        const int s = segs[3 * a], c = segs[3 * a + 2];
        if (part == 0) {
            lab[u] = c;
            ss[u] = (u == s) ? 1 : 0;
        } else {
            // part 1 walks the mirrored sequence: [s, t) covers original [L - t, L - s)
            const int t = segs[3 * a + 1];
            lab[L - 1 - u] = c;
            ss[L - 1 - u] = (L - 1 - u == L - t) ? 1 : 0;
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

hipError_t launch_vit_combine(const double* vwin, const float* trans, const int* Leff, int B,
                              int C, int K, bool bidir, const double* vscore, const int* vcstar,
                              int* split, float* best_score, hipStream_t stream) {
    hipLaunchKernelGGL(k_vit_combine, dim3(B), dim3(256), 0, stream, vwin, trans, Leff, B, C, K,
                       bidir ? 1 : 0, vscore, vcstar, split, best_score);
    return hipGetLastError();
}

hipError_t launch_backtrace(const uint32_t* bp, const int* split, int B, int T, int C, int K,
                            int32_t* tr, int32_t* ent, int32_t* labels, uint8_t* seg_start,
                            hipStream_t stream) {
    const int W = backtrace_chunk(C, K);
    const int nch = backtrace_chunks(T, C, K);
    const size_t lds_t = (size_t)W * C * sizeof(int);
    const size_t lds_f = (size_t)(W + K) * C * sizeof(uint32_t) + (size_t)3 * W * sizeof(int);
    if (lds_f > 150 * 1024 || lds_t > 150 * 1024) return hipErrorInvalidValue;
    // the decode ends at (L, final label) in one direction: part 1 is empty
    const int parts = 1;
    hipLaunchKernelGGL(k_bt_transfer, dim3(nch, B, parts), dim3(BT_THREADS), lds_t, stream, bp,
                       split, B, T, C, K, W, nch, tr);
    hipLaunchKernelGGL(k_bt_compose, dim3(B, parts), dim3(64), 0, stream, tr, split, B, C, K, nch,
                       ent);
    hipLaunchKernelGGL(k_bt_fill, dim3(nch, B, parts), dim3(BT_THREADS), lds_f, stream, bp, split,
                       ent, B, T, C, K, W, nch, labels, seg_start);
    return hipGetLastError();
}

}  // namespace semicrf
