// Long-duration max-plus sweep (sweep_xk.h), forward only: the instances and their launcher.
#include "sweep_xk.h"

namespace semicrf {

namespace {

template <bool GRING, int G, int KPLMAX, int NTMAX>
hipError_t launch_inst(const XkCfg& xc, const SweepLaunch& a, int ndir, hipStream_t stream) {
    if (GRING && !a.xk_ring) return hipErrorInvalidValue;
    if (xc.NT > NTMAX || xc.NT < 64 + a.C * G || xc.kpl > KPLMAX || xc.kpl % XK_UNROLL != 0 ||
        (xc.RS & (xc.RS - 1)) != 0 || xc.RS < a.K + 2 || xc.CH * a.C > XK_PF * (xc.NT - 64))
        return hipErrorInvalidValue;
    if (a.mode != MODE_SPEC && a.mode != MODE_REPAIR) return hipErrorInvalidValue;
    const dim3 grid = a.mode == MODE_REPAIR ? dim3(a.B, ndir) : dim3(a.nspans, a.B, ndir);
    const XkParams p{GRING ? a.xk_ring : nullptr, xc.RS, xc.CH, xc.kpl};
    hipLaunchKernelGGL((k_sweep_xk<true, GRING, G, KPLMAX, NTMAX>), grid, dim3(xc.NT), xc.lds, stream,
                       static_cast<const SweepArgs&>(a), p, a.proj_start, a.proj_end);
    return hipGetLastError();
}

template <bool GRING>
hipError_t launch_ring(const XkCfg& xc, const SweepLaunch& a, int ndir, hipStream_t stream) {
    switch (xc.G) {
        case 64: return launch_inst<GRING, 64, 128, 512>(xc, a, ndir, stream);
        case 32: return launch_inst<GRING, 32, 64, 576>(xc, a, ndir, stream);
        case 8: return launch_inst<GRING, 8, 64, 576>(xc, a, ndir, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_xk_maxplus(const XkCfg& xc, const SweepLaunch& a, hipStream_t stream) {
    if (!xc.ok) return hipErrorInvalidValue;
    return xc.gring ? launch_ring<true>(xc, a, 1, stream) : launch_ring<false>(xc, a, 1, stream);
}

}  // namespace semicrf
