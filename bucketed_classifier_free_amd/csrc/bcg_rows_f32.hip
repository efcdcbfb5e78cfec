// Materialised-branch step kernels, f32 storage.
#include "bcg_rows_impl.h"

namespace bcg {
hipError_t launch_rows_f32(const RowsParams& p, bool vec, bool inpaint, bool nt, int block, hipStream_t s) {
    return launch_rows<float>(p, vec, inpaint, nt, block, s);
}
}  // namespace bcg
