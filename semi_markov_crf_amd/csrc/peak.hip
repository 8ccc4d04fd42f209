// Peak issue rates of the gfx950 vector ALU, measured: the denominators of the sweeps'
// roofline (bench.py).  Built into libsemicrf_peak.so, apart from the library.
//
// Each kernel keeps every SIMD full (1024 workgroups of 256 lanes, 8 independent
// dependency chains per lane so that latency never limits issue) and counts operations
// per lane:
//   fma  : v_fma_f32, a = a * x + y
//   exp2 : v_exp_f32, a = 2^(-a) (bounded in (0, 1])
//   mix  : one v_exp_f32 and one v_fma_f32 per step, to see whether the two co-issue
// The rate is operations per second over the whole chip (lane operations), timed with
// HIP events around `reps` launches after one warm-up launch.
#include <hip/hip_runtime.h>

namespace {

constexpr int BLOCKS = 1024, THREADS = 256, CHAINS = 8;

__global__ __launch_bounds__(THREADS) void k_peak_fma(int iters, float x, float y, float* out) {
    float a[CHAINS];
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) a[i] = (float)(threadIdx.x + i) * 1e-3f;
    for (int n = 0; n < iters; ++n) {
#pragma unroll
        for (int i = 0; i < CHAINS; ++i) a[i] = fmaf(a[i], x, y);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) s += a[i];
    out[(size_t)blockIdx.x * THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(THREADS) void k_peak_exp2(int iters, float* out) {
    float a[CHAINS];
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) a[i] = (float)(threadIdx.x + i) * 1e-3f;
    for (int n = 0; n < iters; ++n) {
#pragma unroll
        for (int i = 0; i < CHAINS; ++i) a[i] = __builtin_amdgcn_exp2f(-a[i]);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) s += a[i];
    out[(size_t)blockIdx.x * THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(THREADS) void k_peak_mix(int iters, float x, float y, float* out) {
    float a[CHAINS], b[CHAINS];
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) {
        a[i] = (float)(threadIdx.x + i) * 1e-3f;
        b[i] = a[i];
    }
    for (int n = 0; n < iters; ++n) {
#pragma unroll
        for (int i = 0; i < CHAINS; ++i) {
            a[i] = __builtin_amdgcn_exp2f(-a[i]);
            b[i] = fmaf(b[i], x, y);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) s += a[i] + b[i];
    out[(size_t)blockIdx.x * THREADS + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// out[0] = v_fma_f32 lane operations / s, out[1] = v_exp_f32 lane operations / s,
// out[2] = (v_exp_f32 + v_fma_f32) lane operations / s when interleaved.
// 0 on success, 1 on a HIP error.
int semicrf_peak_rates(int iters, int reps, double* out) {
    if (iters < 1 || reps < 1 || !out) return 1;
    float* buf = nullptr;
    if (hipMalloc(&buf, sizeof(float) * BLOCKS * THREADS) != hipSuccess) return 1;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
    const double lanes = (double)BLOCKS * THREADS * CHAINS * iters;
    int rc = 0;
    for (int which = 0; which < 3 && !rc; ++which) {
        auto launch = [&]() {
            if (which == 0)
                hipLaunchKernelGGL(k_peak_fma, dim3(BLOCKS), dim3(THREADS), 0, 0, iters, 0.999f,
                                   1e-3f, buf);
            else if (which == 1)
                hipLaunchKernelGGL(k_peak_exp2, dim3(BLOCKS), dim3(THREADS), 0, 0, iters, buf);
            else
                hipLaunchKernelGGL(k_peak_mix, dim3(BLOCKS), dim3(THREADS), 0, 0, iters, 0.999f,
                                   1e-3f, buf);
        };
        launch();
        if (hipDeviceSynchronize() != hipSuccess) { rc = 1; break; }
        hipEventRecord(e0, 0);
        for (int r = 0; r < reps; ++r) launch();
        hipEventRecord(e1, 0);
        if (hipEventSynchronize(e1) != hipSuccess) { rc = 1; break; }
        float ms = 0.0f;
        hipEventElapsedTime(&ms, e0, e1);
        out[which] = lanes * reps * (which == 2 ? 2.0 : 1.0) / (ms * 1e-3);
    }
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    hipFree(buf);
    return rc;
}

}  // extern "C"
