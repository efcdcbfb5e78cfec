// Host-side helpers shared by the launching translation units of libbcg:
// pointer checks, status conversion and the launch shape of the streaming
// step kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bcg_common.h"

namespace bcg {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t elem_size(int dtype) { return dtype == BCG_BF16 ? 2 : 4; }

// Two byte ranges overlap without being the same range.
inline bool partial_overlap(const void* a, const void* b, size_t bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    if (x == y) return false;
    return x < y + bytes && y < x + bytes;
}

// Two byte ranges share any byte (the same range included).
inline bool any_overlap(const void* a, size_t abytes, const void* b, size_t bbytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bbytes && y < x + abytes;
}

inline int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(BCG_EHIP, "%s: %s", what, hipGetErrorString(e));
    return BCG_OK;
}

// Launch shape of the streaming step kernels: workgroups of `block` lanes,
// each lane taking `vpt` vectors.  One vector per lane: a large batch is
// several rounds of workgroups, which the hardware dispatcher hands to CUs as
// earlier ones retire, so CUs whose waves run ahead take more of the work
// and the launch ends without a long tail (a single resident round of
// longer workgroups leaves the waves that lose arbitration finishing last).
// Small batches shrink the workgroup so the grid still spreads over the
// CUs; only grids beyond 2^22 workgroups give lanes more vectors.
struct LaunchShape {
    int block, vpt;
};
inline LaunchShape pick_shape(int64_t samples, int64_t nvec) {
    constexpr int64_t kResident = 256 * 4;
    int bs = 256, vpt = 1;
    auto blocks = [&](int b, int v) { return samples * ((nvec + (int64_t)b * v - 1) / ((int64_t)b * v)); };
    while (bs > 64 && blocks(bs, vpt) < kResident) bs /= 2;
    while (vpt < 64 && blocks(bs, vpt) > ((int64_t)1 << 22)) vpt *= 2;
    return {bs, vpt};
}

}  // namespace bcg
