// Long-duration max-plus sweep (sweep_xk.h), forward only: the instances and their launcher.
#include "sweep_xk.h"

namespace semicrf {

namespace {

template <int RM, int G, int KPLMAX, int NTMAX>
hipError_t launch_inst(const XkCfg& xc, const SweepLaunch& a, int ndir, hipStream_t stream) {
    if (xk_ring_floats(xc, a.C, 1, true) > 0 && !a.xk_ring) return hipErrorInvalidValue;
    if (xc.NT > NTMAX || xc.NT < 64 + a.C * G || xc.kpl > KPLMAX || xc.kpl % XK_UNROLL != 0 ||
        (RM == XK_RING_MIRRORED && (KPLMAX - 1) * G > xc.RS) ||
        (xc.RS & (xc.RS - 1)) != 0 || xc.RS < a.K + 2 || xc.CH * a.C > XK_PF * (xc.NT - 64))
        return hipErrorInvalidValue;
    if (a.mode != MODE_SPEC && a.mode != MODE_REPAIR) return hipErrorInvalidValue;
    const dim3 grid = a.mode == MODE_REPAIR ? dim3(a.B, ndir) : dim3(a.nspans, a.B, ndir);
    const XkParams p{a.xk_ring, xc.RS, xc.CH, xc.kpl, xc.NE};
    hipLaunchKernelGGL((k_sweep_xk<true, RM, G, KPLMAX, NTMAX>), grid, dim3(xc.NT), xc.lds, stream,
                       static_cast<const SweepArgs&>(a), p, a.proj_start, a.proj_end);
    return hipGetLastError();
}

template <int RM>
hipError_t launch_ring(const XkCfg& xc, const SweepLaunch& a, int ndir, hipStream_t stream) {
    switch (xc.G) {
        case 64:   // 32 duration weights a lane up to K = 2049, else 128
            if (xc.kplmax == 32) return launch_inst<RM, 64, 32, 512>(xc, a, ndir, stream);
            if constexpr (RM != XK_RING_MIRRORED)   // the host keeps these windows in plain rows
                return launch_inst<RM, 64, 128, 512>(xc, a, ndir, stream);
            return hipErrorInvalidValue;
        case 32: return launch_inst<RM, 32, 64, 576>(xc, a, ndir, stream);
        case 8: return launch_inst<RM, 8, 64, 576>(xc, a, ndir, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_xk_maxplus(const XkCfg& xc, const SweepLaunch& a, hipStream_t stream) {
    if (!xc.ok) return hipErrorInvalidValue;
    switch (xc.ring) {
        case XK_RING_LDS: return launch_ring<XK_RING_LDS>(xc, a, 1, stream);
        case XK_RING_MIRRORED: return launch_ring<XK_RING_MIRRORED>(xc, a, 1, stream);
        case XK_RING_GLOBAL: return launch_ring<XK_RING_GLOBAL>(xc, a, 1, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace semicrf
