// Round kernel (C <= 16) with boundary projections and the log-space ring only.
#include "sweep_lse_round.h"

namespace semicrf {

hipError_t launch_lse_round_proj_log(const SweepCfg& cfg, const SweepLaunch& a, int ndir,
                                     hipStream_t stream) {
    return launch_lse_round_layout<false, true>(cfg, a, ndir, stream);
}

}  // namespace semicrf
