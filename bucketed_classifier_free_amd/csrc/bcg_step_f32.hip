// Fused guided step, fp32 storage, ordinary loads/stores.
#include "bcg_step_impl.h"

namespace bcg {
hipError_t launch_step_f32(const StepParams& p, bool vec, bool heun, bool inpaint, int block,
                           hipStream_t s) {
    return launch_step<float, KeepTune, true>(p, vec, heun, inpaint, block, s);
}
}  // namespace bcg
