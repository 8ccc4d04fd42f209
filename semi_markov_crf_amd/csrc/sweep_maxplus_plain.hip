// Max-plus (Viterbi) sweep kernels for one ring layout (plain); the kernel itself is in
// sweep_maxplus_kernel.h.  One translation unit per layout keeps the builds parallel.
#include "sweep_maxplus_kernel.h"
#include "sweep_maxplus_round.h"

namespace semicrf {

hipError_t launch_maxplus_plain(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream) {
    if (cfg.split)
        return (a.proj_start || a.proj_end) ? launch_maxplus_round_proj(cfg, a, stream)
                                            : launch_maxplus_round<false>(cfg, a, stream);
    return launch_maxplus_layout<false>(cfg, a, stream);
}

}  // namespace semicrf
