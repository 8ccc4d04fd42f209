// Log-semiring sweep kernels for one ring layout (plain); the kernel itself is in
// sweep_lse_kernel.h.  One translation unit per layout keeps the builds parallel.
#include "sweep_lse_kernel.h"
#include "sweep_lse_round.h"

namespace semicrf {

hipError_t launch_lse_plain(const SweepCfg& cfg, const SweepLaunch& a, int ndir, hipStream_t stream) {
    if (cfg.split)
        return (a.proj_start || a.proj_end) ? launch_lse_round_proj(cfg, a, ndir, true, stream)
                                            : launch_lse_round_layout<true, false>(cfg, a, ndir, stream);
    return launch_lse_layout<SWEEP_LINEAR>(cfg, a, ndir, stream);
}

}  // namespace semicrf
