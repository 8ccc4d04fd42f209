// Round kernels (C <= 16) with boundary projections: the log-semiring sweep with the
// linear ring (the log-space-only one is in sweep_round_proj_log.hip) and the max-plus
// sweep.  Translation units of their own keep the builds parallel; without projections
// the other units' instances run.
#include "sweep_lse_round.h"
#include "sweep_maxplus_round.h"

namespace semicrf {

hipError_t launch_lse_round_proj_log(const SweepCfg& cfg, const SweepLaunch& a, int ndir,
                                     hipStream_t stream);

hipError_t launch_lse_round_proj(const SweepCfg& cfg, const SweepLaunch& a, int ndir, bool lin,
                                 hipStream_t stream) {
    return lin ? launch_lse_round_layout<true, true>(cfg, a, ndir, stream)
               : launch_lse_round_proj_log(cfg, a, ndir, stream);
}

hipError_t launch_maxplus_round_proj(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream) {
    return launch_maxplus_round<true>(cfg, a, stream);
}

}  // namespace semicrf
