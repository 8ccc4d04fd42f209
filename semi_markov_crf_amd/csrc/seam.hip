// Seam check of the speculative checkpoint spans on gfx950.
//
// The streamed recurrences of the pages ("Streaming Structured Inference with
// Flash-SemiCRF", gist.science EN explainer, "2. Methodology": ring buffers of the last K
// messages, checkpoints every delta positions) are sequential in the position.  Here every
// span of a sequence is swept at once: span j > 0 starts `warm` positions before its first
// position from a ring in which every entry is equal, instead of waiting for the checkpoint
// the previous span would leave.  The recurrence is linear and positive in linear space
// (the log-semiring sums), so the state it carries forgets where it started: after the
// burn-in the span's ring values equal the exact ones plus one constant per span, to within
// rounding.  This kernel proves it span by span.
//
// For the seam at t0 = j * delta it compares, at the K positions t0-K+1 .. t0 and every
// label, the ring values of span j-1 (tail, its own frame) with those span j reached in its
// burn-in (head, its frame): d = tail - head.  If every finite entry of one agrees with the
// other's finiteness and max d - min d <= 2 * tol, the two states are the same up to the
// constant c_j = (max d + min d) / 2 with every entry within tol of it; since every later
// value of span j is a log-sum of the ring state with positive weights, it is within tol of
// the value the sequential sweep would have reached from span j-1's state, plus c_j.  The
// frame offsets off[j] = off[j-1] + c_j (off[0] = 0: span 0 starts exactly at position 0)
// then put every span in the exact frame, and log Z = (last span's own log Z) + off[last].
// The first seam that fails stops the chain: the spans from there on are swept again in
// order (MODE_REPAIR) from the checkpoint span j-1 left at its end, in span j-1's frame.
//
// k_seam_stats reduces every seam's window at once; k_seam then walks the seams of each
// sequence and direction in order.  Per (sequence, direction) it also records the sum and
// maximum of the accepted half-ranges (a bound on the error the speculation adds, in
// natural-log units) and the first failed seam.
#include "common.h"
#include "internal.h"

namespace semicrf {

// grid (nspans - 1, B, ndir), block 256: the statistics of seam j = blockIdx.x + 1 of one
// sequence and direction: max and min of d = tail - head over the finite entries (both
// finite), and whether the two sides disagree on finiteness anywhere.  Fixed reduction
// order (lanes, then the four wavefronts in order): bitwise reproducible.
__global__ __launch_bounds__(256) void k_seam_stats(const SeamArgs s) {
    __shared__ double wmax[4], wmin[4];
    __shared__ int wmis[4];
    const int j = blockIdx.x + 1, b = blockIdx.y, dir = blockIdx.z, tid = threadIdx.x;
    const int L = abs(s.Leff[b]);
    const int n = (L + s.delta - 1) / s.delta;                    // spans that hold positions
    if (j >= n) return;
    const size_t row = (size_t)dir * s.B + b;
    const int KC = s.K * s.C;
    const double* tl = s.tail + (row * s.nspans + j - 1) * KC;
    const double* hd = s.head + (row * s.nspans + j) * KC;
    double lmax = -1.0e300, lmin = 1.0e300;
    int mis = 0;
    for (int q = tid; q < KC; q += 256) {
        const double tv = tl[q], hv = hd[q];
        const bool vt = tv > -1.0e29, vh = hv > -1.0e29;
        if (vt != vh) {
            mis = 1;
        } else if (vt) {
            const double d = tv - hv;
            lmax = fmax(lmax, d);
            lmin = fmin(lmin, d);
        }
    }
    for (int o = 32; o >= 1; o >>= 1) {
        lmax = fmax(lmax, __shfl_xor(lmax, o, 64));
        lmin = fmin(lmin, __shfl_xor(lmin, o, 64));
        mis |= __shfl_xor(mis, o, 64);
    }
    if ((tid & 63) == 0) {
        wmax[tid >> 6] = lmax;
        wmin[tid >> 6] = lmin;
        wmis[tid >> 6] = mis;
    }
    __syncthreads();
    if (tid == 0) {
        double gmax = wmax[0], gmin = wmin[0];
        int gm = wmis[0];
        for (int w = 1; w < 4; ++w) {
            gmax = fmax(gmax, wmax[w]);
            gmin = fmin(gmin, wmin[w]);
            gm |= wmis[w];
        }
        double* st = s.stats + (row * s.nspans + j) * 3;
        st[0] = gmax;
        st[1] = gmin;
        st[2] = (double)gm;
    }
}

// grid (B, ndir), one wavefront: the seams of one sequence and direction in order.  If
// every finite entry of one side agrees with the other's finiteness and max d - min d <= 2 tol,
// the spans' states are the same up to c_j = (max d + min d) / 2; the frame offsets chain
// the c_j; the first seam that fails stops the chain.
__global__ __launch_bounds__(64) void k_seam(const SeamArgs s) {
    const int b = blockIdx.x, dir = blockIdx.y, lane = threadIdx.x;
    const int Lr = s.Leff[b];
    const bool bad = Lr < 0;
    const int L = bad ? -Lr : Lr;
    const int n = (L + s.delta - 1) / s.delta;                    // spans that hold positions
    const size_t row = (size_t)dir * s.B + b;
    double* off = s.off + row * s.nspans;
    // the seams 1 .. n-1, 64 at a time, one a lane: the first one not accepted stops the
    // chain; the frame offsets are the prefix sums of the accepted constants (a fixed-order
    // wavefront scan), the bound the sum and maximum of their tau
    double cur = 0.0, sum = 0.0, mx = 0.0;                         // the same in every lane
    int fb = s.nspans;
    if (lane == 0) off[0] = 0.0;
    for (int j0 = 1; j0 < n; j0 += 64) {
        const int j = j0 + lane;
        const bool in = j < n;
        double c = 0.0, tau = 0.0;
        bool ok = true;
        if (in) {
            const double* st = s.stats + (row * s.nspans + j) * 3;
            const double gmax = st[0], gmin = st[1];
            const bool any = gmax >= gmin;                         // some finite entry
            tau = any ? 0.5 * (gmax - gmin) : 0.0;
            ok = st[2] == 0.0 && tau <= s.tol;
            c = any ? 0.5 * (gmax + gmin) : 0.0;
        }
        const unsigned long long badm = __ballot(in && !ok);
        const int first = badm ? __builtin_ctzll(badm) : 64;     // first seam not accepted
        const bool acc = in && lane < first;
        double v = acc ? c : 0.0;                                  // inclusive scan
        for (int d = 1; d < 64; d <<= 1) {
            const double u = __shfl_up(v, d, 64);
            if (lane >= d) v += u;
        }
        if (acc) off[j] = cur + v;
        double ts = acc ? tau : 0.0, tm = ts;
        for (int d = 32; d >= 1; d >>= 1) {
            ts += __shfl_xor(ts, d, 64);
            tm = fmax(tm, __shfl_xor(tm, d, 64));
        }
        cur += __shfl(v, 63, 64);
        sum += ts;
        mx = fmax(mx, tm);
        if (badm) {
            fb = j0 + first;
            break;
        }
    }
    // a repaired sweep continues in the frame of span fb-1
    for (int j = fb + lane; j < n; j += 64) off[j] = cur;
    if (lane != 0) return;
    s.first_bad[row] = fb;
    if (fb >= s.nspans) {
        const double lz = bad ? __longlong_as_double(0x7ff8000000000000LL) : s.lzloc[row] + cur;
        (dir == 0 ? s.logz : s.logz_b)[b] = lz;
    }
    double* dg = s.diag + row * 4;
    dg[0] = sum;
    dg[1] = mx;
    dg[2] = fb < s.nspans ? (double)fb : -1.0;
    dg[3] = (double)(n > 0 ? n - 1 : 0);
}

hipError_t launch_seam(const SeamArgs& s, int ndir, hipStream_t stream) {
    if (s.nspans > 1)
        hipLaunchKernelGGL(k_seam_stats, dim3(s.nspans - 1, s.B, ndir), dim3(256), 0, stream, s);
    hipLaunchKernelGGL(k_seam, dim3(s.B, ndir), dim3(64), 0, stream, s);
    return hipGetLastError();
}

}  // namespace semicrf

namespace semicrf {

// per sequence: the sum of the accepted half-ranges over the directions' seams, and the
// number of directions swept again from a failed seam
__global__ void k_seam_report(const double* __restrict__ diag, int B, int ndir,
                              float* __restrict__ bound, int* __restrict__ repairs) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    double s = 0.0;
    int r = 0;
    for (int d = 0; d < ndir; ++d) {
        const double* dg = diag + ((size_t)d * B + b) * 4;
        s += dg[0];
        r += dg[2] >= 0.0 ? 1 : 0;
    }
    if (bound) bound[b] = (float)s;
    if (repairs) repairs[b] = r;
}

hipError_t launch_seam_report(const double* diag, int B, int ndir, float* bound, int* repairs,
                              hipStream_t stream) {
    if (!bound && !repairs) return hipSuccess;
    hipLaunchKernelGGL(k_seam_report, dim3((B + 255) / 256), dim3(256), 0, stream, diag, B, ndir,
                       bound, repairs);
    return hipGetLastError();
}

}  // namespace semicrf
