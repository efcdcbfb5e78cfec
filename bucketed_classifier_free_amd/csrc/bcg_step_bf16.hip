// Fused guided step, bf16 storage (fp32 arithmetic), ordinary loads/stores.
#include "bcg_step_impl.h"

namespace bcg {
hipError_t launch_step_bf16(const StepParams& p, bool vec, bool heun, bool inpaint, int block,
                            hipStream_t s) {
    return launch_step<bf16_t, KeepTune, true>(p, vec, heun, inpaint, block, s);
}
}  // namespace bcg
