// Fused guided step, fp32 storage instantiations.
#include "bcg_step_impl.h"

namespace bcg {
hipError_t launch_step_f32(const StepParams& p, bool vec, bool heun, bool inpaint, int block,
                           hipStream_t s) {
    return launch_step<float>(p, vec, heun, inpaint, block, s);
}
}  // namespace bcg
