// Materialised-branch step kernels, bf16 storage.
#include "bcg_rows_impl.h"

namespace bcg {
hipError_t launch_rows_bf16(const RowsParams& p, bool vec, bool inpaint, bool nt, int block, hipStream_t s) {
    return launch_rows<bf16_t>(p, vec, inpaint, nt, block, s);
}
}  // namespace bcg
