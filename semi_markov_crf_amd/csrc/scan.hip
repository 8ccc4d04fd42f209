// Centring and prefix-sum kernels (gfx950).
//
// S[b, 0, c] = 0 and S[b, t, c] = sum_{u < t} (em[b, u, c] - nu[b, c]) for t <= L_b, with
// nu[b, c] the mean of em[b, :L_b, c] ("Streaming Structured Inference with Flash-SemiCRF",
// gist.science EN explainer, "2. Methodology": "Emission Baseline Centering" and
// "On-the-Fly Edge Computation via Prefix Sums").  Positions t > L_b repeat S[b, L_b].
//
// Three streaming passes, all HBM bound, with fp64 accumulation:
//   1. per-tile column sums of the valid emissions,
//   2. an exclusive scan of the tile sums per sequence (also gives nu),
//   3. the in-tile centred prefix sum.
// For C <= 8 (tile 1024 rows) passes 1 and 3 give each lane four consecutive rows, so a
// wavefront's loads and stores cover one contiguous stretch of the tile; every load of a
// lane is issued before the first is used, and the tile's prefix comes from a wavefront
// scan of the lanes' row sums (DPP row shifts and row broadcasts, fp64) plus one LDS
// exchange between the four wavefronts.  Larger C keeps the column-per-thread kernels,
// which stage the tile through LDS.
#include "common.h"
#include "internal.h"

namespace semicrf {

int scan_tile(int C) {
    int ts = 1024;
    while (ts > 32 && ts * C > 8192) ts >>= 1;
    return ts;
}

// grid (ntiles, B), block 256
__global__ __launch_bounds__(256) void k_em_tile_sums(const float* __restrict__ em,
                                                      const int32_t* __restrict__ lengths,
                                                      int T, int C, int TS,
                                                      double* __restrict__ tile_sums,
                                                      int* __restrict__ Leff) {
    __shared__ double part[256];
    const int tile = blockIdx.x, b = blockIdx.y, ntiles = gridDim.x;
    const int Lraw = lengths[b];
    const bool bad = Lraw < 1 || Lraw > T;
    const int L = min(max(Lraw, 1), T);
    if (tile == 0 && threadIdx.x == 0) Leff[b] = bad ? -L : L;   // negated: length was invalid
    const int t0 = tile * TS;
    const int t1 = min(t0 + TS, L);
    const float* e = em + (size_t)b * T * C;
    for (int c0 = 0; c0 < C; c0 += 256) {
        const int CW = min(256, C - c0);
        const int R = 256 / CW;
        const int tid = threadIdx.x;
        const int cw = tid % CW, r = tid / CW;
        double acc = 0.0;
        if (r < R)
            for (int t = t0 + r; t < t1; t += R) acc += (double)e[(size_t)t * C + c0 + cw];
        part[tid] = acc;
        __syncthreads();
        if (tid < CW) {
            double s = 0.0;
            for (int i = 0; i < R; ++i) s += part[i * CW + tid];
            tile_sums[((size_t)b * ntiles + tile) * C + c0 + tid] = s;
        }
        __syncthreads();
    }
}

// grid (C, B), block 256: one workgroup per (label, sequence).  Exclusive prefix (or
// suffix) over the n tiles of one column: thread i sums the tiles at ordinal positions
// [i*per, (i+1)*per) of the scan order (ascending tile index, or descending when reverse)
// in order; a fixed-order scan of those 256 sums (Hillis-Steele within each wavefront,
// then the four wavefront totals) gives each thread its offset, and it writes the
// offsets of its tiles in order.  Every addition happens in the same order on every
// call, so results are reproducible bit for bit.
__global__ __launch_bounds__(256) void k_tile_scan(const double* __restrict__ tile_sums, int n,
                                                  int C, int reverse,
                                                  double* __restrict__ offsets,
                                                  double* __restrict__ totals) {
    __shared__ double wsum[4];
    const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int per = (n + 255) / 256;
    const double* in = tile_sums + (size_t)b * n * C;
    auto idx = [&](int o) { return (size_t)(reverse ? n - 1 - o : o) * C + c; };
    double s = 0.0;
    for (int i = 0; i < per; ++i) {
        const int o = tid * per + i;
        if (o < n) s += in[idx(o)];
    }
    double v = s;   // inclusive scan within the wavefront
    for (int d = 1; d < 64; d <<= 1) {
        const double u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    if (lane == 63) wsum[w] = v;
    double excl = __shfl_up(v, 1, 64);
    if (lane == 0) excl = 0.0;
    __syncthreads();
    double base = 0.0;
    for (int i = 0; i < w; ++i) base += wsum[i];
    double run = base + excl;
    if (offsets)
        for (int i = 0; i < per; ++i) {
            const int o = tid * per + i;
            if (o < n) {
                offsets[(size_t)b * n * C + idx(o)] = run;
                run += in[idx(o)];
            }
        }
    if (totals && tid == 255) totals[(size_t)b * C + c] = base + v;
}

// grid (ntiles, B), block 256, dynamic LDS = TS*C*4 + TS*C*8 + 256*8 bytes.
__global__ __launch_bounds__(256) void k_prefix(const float* __restrict__ em,
                                                const int* __restrict__ Leff, int B, int T, int C,
                                                int TS, const double* __restrict__ tile_off,
                                                const double* __restrict__ totals,
                                                double* __restrict__ S, int* __restrict__ status) {
    extern __shared__ double lds[];
    const int tile = blockIdx.x, b = blockIdx.y, ntiles = gridDim.x;
    const int L = abs(Leff[b]);
    const int t0 = tile * TS;
    const int rows = min(TS, T - t0);           // emission rows of this tile
    if (tile == 0 && b == 0 && threadIdx.x == 0) {
        int flag = 0;
        for (int i = 0; i < B; ++i) flag |= Leff[i] < 0;
        status[0] = flag;
    }
    double* out = lds;                          // [TS][C] doubles
    double* csum = out + (size_t)TS * C;        // [256]
    float* in = (float*)(csum + 256);           // [TS][C] floats
    const float* e = em + ((size_t)b * T + t0) * C;
    const int tid = threadIdx.x;
    for (int i = tid; i < rows * C; i += 256) in[i] = e[i];
    __syncthreads();
    const double* off = tile_off + ((size_t)b * ntiles + tile) * C;
    const double* tot = totals + (size_t)b * C;
    const int nvalid_before = min(t0, L);
    for (int c0 = 0; c0 < C; c0 += 256) {
        const int CW = min(256, C - c0);
        const int R = 256 / CW;
        const int chunk = (rows + R - 1) / R;
        const int cw = tid % CW, r = tid / CW, c = c0 + cw;
        const bool act = r < R;
        const double nu = tot[c] / (double)L;
        double acc = 0.0;
        if (act)
            for (int i = r * chunk; i < min(rows, (r + 1) * chunk); ++i)
                if (t0 + i < L) acc += (double)in[i * C + c] - nu;
        csum[tid] = acc;
        __syncthreads();
        if (act) {
            double run = off[c] - nu * (double)nvalid_before;
            for (int q = 0; q < r; ++q) run += csum[q * CW + cw];
            for (int i = r * chunk; i < min(rows, (r + 1) * chunk); ++i) {
                if (t0 + i < L) run += (double)in[i * C + c] - nu;
                out[i * C + c] = run;
            }
        }
        __syncthreads();
    }
    double* Sb = S + (size_t)b * (T + 1) * C;
    for (int i = tid; i < rows * C; i += 256) Sb[(size_t)(t0 + 1) * C + i] = out[i];
    if (tile == 0)
        for (int c = tid; c < C; c += 256) Sb[c] = 0.0;
}

// ---------------------------------------------------------------- C <= 8: rows per lane
constexpr int SCAN_ROWS = 4;   // consecutive rows per lane; 256 lanes x 4 = the 1024-row tile

// one 32-bit half of a double moved by a DPP control; lanes without a source (or outside
// row_mask) read 0
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_d(double v) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWMASK, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWMASK, 0xF, false);
    return __hiloint2double(hi, lo);
}

// inclusive sum over the 64 lanes of a wavefront, in lane order: shifts by 1, 2, 4, 8
// inside each row of 16 lanes, then the last lane of row 0 / 2 into rows 1 / 3, then the
// last lane of row 1 into rows 2 and 3
__device__ __forceinline__ double wave_inclusive_sum(double x) {
    x += dpp_d<0x111, 0xF>(x);
    x += dpp_d<0x112, 0xF>(x);
    x += dpp_d<0x114, 0xF>(x);
    x += dpp_d<0x118, 0xF>(x);
    x += dpp_d<0x142, 0xA>(x);
    x += dpp_d<0x143, 0xC>(x);
    return x;
}

__device__ __forceinline__ double lane63(double v) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 63),
                            __builtin_amdgcn_readlane(__double2loint(v), 63));
}

// the lane's rows t0 + 4*tid + i of sequence b, C = CC floats each (0 past T)
template <int CC>
__device__ __forceinline__ void load_rows(const float* __restrict__ em, int b, int T, int tr,
                                          float (&v)[SCAN_ROWS][CC]) {
    const float* e = em + ((size_t)b * T + tr) * CC;
    if (tr + SCAN_ROWS <= T) {
#pragma unroll
        for (int i = 0; i < SCAN_ROWS; ++i)
#pragma unroll
            for (int c = 0; c < CC; ++c) v[i][c] = e[i * CC + c];
    } else {
#pragma unroll
        for (int i = 0; i < SCAN_ROWS; ++i)
#pragma unroll
            for (int c = 0; c < CC; ++c) v[i][c] = tr + i < T ? e[i * CC + c] : 0.0f;
    }
}

// grid (ntiles, B), block 256, tile 1024 rows
template <int CC>
__global__ __launch_bounds__(256) void k_em_tile_sums_rows(const float* __restrict__ em,
                                                           const int32_t* __restrict__ lengths,
                                                           int T, double* __restrict__ tile_sums,
                                                           int* __restrict__ Leff) {
    __shared__ double wsum[4][CC];
    const int tile = blockIdx.x, b = blockIdx.y, ntiles = gridDim.x, tid = threadIdx.x;
    const int Lraw = lengths[b];
    const bool bad = Lraw < 1 || Lraw > T;
    const int L = min(max(Lraw, 1), T);
    if (tile == 0 && tid == 0) Leff[b] = bad ? -L : L;   // negated: length was invalid
    const int tr = tile * 1024 + SCAN_ROWS * tid;
    float v[SCAN_ROWS][CC];
    load_rows<CC>(em, b, T, tr, v);
#pragma unroll
    for (int c = 0; c < CC; ++c) {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < SCAN_ROWS; ++i) s += tr + i < L ? (double)v[i][c] : 0.0;
        s = lane63(wave_inclusive_sum(s));
        if ((tid & 63) == 0) wsum[tid >> 6][c] = s;
    }
    __syncthreads();
    if (tid < CC)
        tile_sums[((size_t)b * ntiles + tile) * CC + tid] =
            ((wsum[0][tid] + wsum[1][tid]) + wsum[2][tid]) + wsum[3][tid];
}

// grid (ntiles, B), block 256, tile 1024 rows
template <int CC>
__global__ __launch_bounds__(256) void k_prefix_rows(const float* __restrict__ em,
                                                     const int* __restrict__ Leff, int B, int T,
                                                     const double* __restrict__ tile_off,
                                                     const double* __restrict__ totals,
                                                     double* __restrict__ S,
                                                     int* __restrict__ status) {
    __shared__ double wsum[4][CC];
    extern __shared__ double stage[];   // [256][SCAN_ROWS * CC + 1]
    const int tile = blockIdx.x, b = blockIdx.y, ntiles = gridDim.x, tid = threadIdx.x;
    const int w = tid >> 6;
    const int L = abs(Leff[b]);
    const int t0 = tile * 1024;
    if (tile == 0 && b == 0 && tid == 0) {
        int flag = 0;
        for (int i = 0; i < B; ++i) flag |= Leff[i] < 0;
        status[0] = flag;
    }
    const int tr = t0 + SCAN_ROWS * tid;
    float v[SCAN_ROWS][CC];
    load_rows<CC>(em, b, T, tr, v);
    const double* off = tile_off + ((size_t)b * ntiles + tile) * CC;
    const double* tot = totals + (size_t)b * CC;
    double x[SCAN_ROWS][CC], excl[CC];
#pragma unroll
    for (int c = 0; c < CC; ++c) {
        const double nu = tot[c] / (double)L;
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < SCAN_ROWS; ++i) {
            x[i][c] = tr + i < L ? (double)v[i][c] - nu : 0.0;
            s += x[i][c];
        }
        const double incl = wave_inclusive_sum(s);
        excl[c] = incl - s;
        if ((tid & 63) == 63) wsum[w][c] = incl;
    }
    __syncthreads();
    double* Sb = S + (size_t)b * (T + 1) * CC;
#pragma unroll
    for (int c = 0; c < CC; ++c) {
        const double nu = tot[c] / (double)L;
        double run = off[c] - nu * (double)min(t0, L);
        for (int q = 0; q < w; ++q) run += wsum[q][c];
        excl[c] += run;
    }
    // the tile's rows t0+1 .. t0+1024 go out through LDS, so that each store instruction
    // writes 64 consecutive doubles instead of one double every 4*CC: lane blocks of
    // 4*CC values one double apart (odd stride: no bank conflicts on the writes)
    constexpr int LB = SCAN_ROWS * CC + 1;
    double* st = stage + (size_t)tid * LB;
#pragma unroll
    for (int i = 0; i < SCAN_ROWS; ++i)
#pragma unroll
        for (int c = 0; c < CC; ++c) {
            excl[c] += x[i][c];
            st[i * CC + c] = excl[c];
        }
    __syncthreads();
    const int nout = min(1024, T - t0) * CC;   // rows t0+1 .. min(t0+1024, T)
    double* dst = Sb + (size_t)(t0 + 1) * CC;
    for (int e = tid; e < nout; e += 256) {
        const int lane = e / (SCAN_ROWS * CC);
        dst[e] = stage[(size_t)lane * LB + (e - lane * SCAN_ROWS * CC)];
    }
    if (tile == 0 && tid < CC) Sb[tid] = 0.0;
}

hipError_t launch_em_tile_sums(const float* em, const int32_t* lengths, int B, int T, int C,
                               double* tile_sums, int* Leff, hipStream_t stream) {
    const int TS = scan_tile(C);
    const int nt = (T + TS - 1) / TS;
#define SEMICRF_ROWS_CASE(CC)                                                                  \
    case CC:                                                                                   \
        hipLaunchKernelGGL(k_em_tile_sums_rows<CC>, dim3(nt, B), dim3(256), 0, stream, em,     \
                           lengths, T, tile_sums, Leff);                                       \
        return hipGetLastError();
    if (TS == 1024) switch (C) {
            SEMICRF_ROWS_CASE(1) SEMICRF_ROWS_CASE(2) SEMICRF_ROWS_CASE(3) SEMICRF_ROWS_CASE(4)
            SEMICRF_ROWS_CASE(5) SEMICRF_ROWS_CASE(6) SEMICRF_ROWS_CASE(7) SEMICRF_ROWS_CASE(8)
            default: break;
        }
#undef SEMICRF_ROWS_CASE
    hipLaunchKernelGGL(k_em_tile_sums, dim3(nt, B), dim3(256), 0, stream, em, lengths, T, C, TS,
                       tile_sums, Leff);
    return hipGetLastError();
}

hipError_t launch_tile_scan(const double* tile_sums, int B, int n, int C, bool reverse,
                            double* offsets, double* totals, hipStream_t stream) {
    if (B < 1 || C < 1) return hipSuccess;
    hipLaunchKernelGGL(k_tile_scan, dim3(C, B), dim3(256), 0, stream, tile_sums, n, C,
                       reverse ? 1 : 0, offsets, totals);
    return hipGetLastError();
}

hipError_t launch_prefix(const float* em, const int* Leff, int B, int T, int C,
                         const double* tile_offsets, const double* totals, double* S, int* status,
                         hipStream_t stream) {
    const int TS = scan_tile(C);
    const int nt = (T + TS - 1) / TS;
#define SEMICRF_ROWS_CASE(CC)                                                                  \
    case CC:                                                                                   \
        hipLaunchKernelGGL(k_prefix_rows<CC>, dim3(nt, B), dim3(256),                        \
                           (size_t)256 * (4 * (CC) + 1) * 8, stream, em, Leff, B,            \
                           T, tile_offsets, totals, S, status);                                \
        return hipGetLastError();
    if (TS == 1024) switch (C) {
            SEMICRF_ROWS_CASE(1) SEMICRF_ROWS_CASE(2) SEMICRF_ROWS_CASE(3) SEMICRF_ROWS_CASE(4)
            SEMICRF_ROWS_CASE(5) SEMICRF_ROWS_CASE(6) SEMICRF_ROWS_CASE(7) SEMICRF_ROWS_CASE(8)
            default: break;
        }
#undef SEMICRF_ROWS_CASE
    const size_t lds = (size_t)TS * C * 8 + 256 * 8 + (size_t)TS * C * 4;
    hipLaunchKernelGGL(k_prefix, dim3(nt, B), dim3(256), lds, stream, em, Leff, B, T, C, TS,
                       tile_offsets, totals, S, status);
    return hipGetLastError();
}

}  // namespace semicrf
