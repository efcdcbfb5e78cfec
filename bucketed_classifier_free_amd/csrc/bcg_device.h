// Device-side building blocks of libbcg for gfx950: storage loads/stores,
// the per-pixel region weights and the launch parameter block of the fused
// guided step.  Included by the .hip translation units only.
//
// Arithmetic contract (all .hip files are compiled with -ffp-contract=off and
// HIP's default correctly rounded fp32 division): every expression below is
// evaluated as the fp32 operations written, in the order written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bcg.h"

namespace bcg {

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- storage

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even; gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ bf16_t to_bf16(float a) { return __builtin_bit_cast(bf16_t, (__bf16)a); }

// V consecutive elements of storage type T as fp32.  V * sizeof(T) is 16
// bytes on the vector path (one 128-bit access per lane) or one element.
template <typename T, int V> struct Io;

template <> struct Io<float, 1> {
    __device__ static __forceinline__ void load(const float* p, float (&v)[1]) { v[0] = *p; }
    __device__ static __forceinline__ void store(float* p, const float (&v)[1]) { *p = v[0]; }
};
template <> struct Io<float, 4> {
    __device__ static __forceinline__ void load(const float* p, float (&v)[4]) {
        const float4 q = *reinterpret_cast<const float4*>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    __device__ static __forceinline__ void store(float* p, const float (&v)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};
template <> struct Io<float, 8> {
    __device__ static __forceinline__ void load(const float* p, float (&v)[8]) {
        const float4 q0 = reinterpret_cast<const float4*>(p)[0];
        const float4 q1 = reinterpret_cast<const float4*>(p)[1];
        v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
        v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
    }
};
template <> struct Io<bf16_t, 1> {
    __device__ static __forceinline__ void load(const bf16_t* p, float (&v)[1]) {
        v[0] = __uint_as_float(uint32_t(*p) << 16);
    }
    __device__ static __forceinline__ void store(bf16_t* p, const float (&v)[1]) { *p = to_bf16(v[0]); }
};
template <> struct Io<bf16_t, 8> {
    __device__ static __forceinline__ void load(const bf16_t* p, float (&v)[8]) {
        const uint4 q = *reinterpret_cast<const uint4*>(p);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
    __device__ static __forceinline__ void store(bf16_t* p, const float (&v)[8]) {
        uint4 q;
        q.x = pack_bf16x2(v[0], v[1]); q.y = pack_bf16x2(v[2], v[3]);
        q.z = pack_bf16x2(v[4], v[5]); q.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<uint4*>(p) = q;
    }
};

template <typename T> struct VecWidth { static constexpr int value = 16 / sizeof(T); };

// ---------------------------------------------------------------- regions

// One region of one sample, as the weights need it.
struct RegionDesc {
    int y0, h, x0, w;
    float strength;
};

// Feathered box weight of one pixel ("calc_cond_batch()": mask and
// feathering).  Linear ramp of F pixels on every edge, separable:
//   n_y = min(dy+1, F) * min(h-dy, F), n_x likewise (0 outside the box),
//   f = float(n_y*n_x) * (1/F^4)  (exact: n_y*n_x <= F^4 <= 2^24),
//   weight = strength * f.
__device__ __forceinline__ float region_weight(const RegionDesc& r, int y, int x, int F,
                                               float inv_f4) {
    const int dy = y - r.y0, dx = x - r.x0;
    if (dy < 0 || dy >= r.h || dx < 0 || dx >= r.w) return 0.0f;
    const int ny = min(dy + 1, F) * min(r.h - dy, F);
    const int nx = min(dx + 1, F) * min(r.w - dx, F);
    const float f = float(ny * nx) * inv_f4;
    return r.strength * f;
}

// ---------------------------------------------------------------- step

// Launch parameter block of the fused guided step (device pointers).
struct StepParams {
    int n, C, H, W, R;            // R: stride of the region arrays
    int feather;                  // >= 1 (0 is passed as 1: no ramp)
    float inv_f4;                 // 1 / feather^4
    int n_active, num_sigmas;
    int64_t HW;
    int nvec;                     // vectors of V pixels per sample
    int tiles;                    // blocks per sample
    int mask_stride;              // HW if per-sample mask, else 0
    float s2;
    const void* x;
    void* x_out;
    const float* sigmas;
    const int32_t* order;
    const int32_t* step_idx;
    const float* scale;
    const int32_t* uncond_row;
    const float* mu_uncond;
    const float* mu_cond;
    const int32_t* region_count;
    const int32_t* region_box;
    const float* region_strength;
    const float* mu_region;
    const void* x_orig;
    const float* mask;
};

// Per-launch launchers, one per storage dtype (bcg_step_f32.hip,
// bcg_step_bf16.hip).  `vec` selects the 128-bit path.
hipError_t launch_step_f32(const StepParams& p, bool vec, bool heun, bool inpaint, int block,
                           hipStream_t s);
hipError_t launch_step_bf16(const StepParams& p, bool vec, bool heun, bool inpaint, int block,
                            hipStream_t s);

}  // namespace bcg
