// Fused guided step, bf16 storage, nontemporal loads/stores (128-bit path).
#include "bcg_step_impl.h"

namespace bcg {
hipError_t launch_step_bf16_stream(const StepParams& p, bool heun, bool inpaint, int block,
                                   hipStream_t s) {
    return launch_step<bf16_t, StreamTune, false>(p, true, heun, inpaint, block, s);
}
}  // namespace bcg
