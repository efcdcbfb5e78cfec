// Fused guided step, bf16 storage, continuous batching (slots holding queued requests).
#include "bcg_step_impl.h"

namespace bcg {
hipError_t launch_step_bf16_queue(const StepParams& p, bool heun, bool inpaint, int block, hipStream_t s) {
    return launch_step_queue<bf16_t>(p, heun, inpaint, block, s);
}
}  // namespace bcg
