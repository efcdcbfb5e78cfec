// Fused guided step, fp32 storage, continuous batching (slots holding queued requests).
#include "bcg_step_impl.h"

namespace bcg {
hipError_t launch_step_f32_queue(const StepParams& p, bool heun, bool inpaint, int block, hipStream_t s) {
    return launch_step_queue<float>(p, heun, inpaint, block, s);
}
}  // namespace bcg
