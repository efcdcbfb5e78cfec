// Fused guided step, bf16 storage instantiations (fp32 arithmetic).
#include "bcg_step_impl.h"

namespace bcg {
hipError_t launch_step_bf16(const StepParams& p, bool vec, bool heun, bool inpaint, int block,
                            hipStream_t s) {
    return launch_step<bf16_t>(p, vec, heun, inpaint, block, s);
}
}  // namespace bcg
