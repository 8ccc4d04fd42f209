// Max-plus (Viterbi) sweep kernels for one ring layout (mirror); the kernel itself is in
// sweep_maxplus_kernel.h.  One translation unit per layout keeps the builds parallel.
#include "sweep_maxplus_kernel.h"

namespace semicrf {

hipError_t launch_maxplus_mirror(const SweepCfg& cfg, const SweepLaunch& a, hipStream_t stream) {
    if (cfg.split) return hipErrorInvalidValue;   // the round kernel keeps one ring copy
    return launch_maxplus_layout<true>(cfg, a, stream);
}

}  // namespace semicrf
