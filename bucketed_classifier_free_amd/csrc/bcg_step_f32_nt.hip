// Fused guided step, fp32 storage, nontemporal loads/stores (128-bit path).
#include "bcg_step_impl.h"

namespace bcg {
hipError_t launch_step_f32_stream(const StepParams& p, bool heun, bool inpaint, int block,
                                  hipStream_t s) {
    return launch_step<float, StreamTune, false>(p, true, heun, inpaint, block, s);
}
}  // namespace bcg
