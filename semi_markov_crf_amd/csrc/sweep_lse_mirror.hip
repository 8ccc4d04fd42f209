// Log-semiring sweep kernels for one ring layout (mirror); the kernel itself is in
// sweep_lse_kernel.h.  One translation unit per layout keeps the builds parallel.
#include "sweep_lse_kernel.h"

namespace semicrf {

hipError_t launch_lse_mirror(const SweepCfg& cfg, const SweepLaunch& a, int ndir, hipStream_t stream) {
    if (cfg.split) return hipErrorInvalidValue;   // the round kernel keeps one ring copy
    return launch_lse_layout<SWEEP_MIRRORED|SWEEP_LINEAR>(cfg, a, ndir, stream);
}

}  // namespace semicrf
