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

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Global load/store, optionally with the nontemporal (streaming) hint.
template <bool NT, typename V>
__device__ __forceinline__ V ld(const V* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT, typename V>
__device__ __forceinline__ void st(V* p, V v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// V consecutive elements of storage type T: one raw access (16 bytes on the
// vector path, one element otherwise), unpacked to / packed from fp32.
template <typename T, int V> struct Io;

template <> struct Io<float, 1> {
    typedef float Raw;
    template <bool NT = false> __device__ static __forceinline__ Raw load_raw(const float* p) { return ld<NT>(p); }
    __device__ static __forceinline__ void unpack(const Raw& r, float (&v)[1]) { v[0] = r; }
    __device__ static __forceinline__ void load(const float* p, float (&v)[1]) { v[0] = *p; }
    template <bool NT = false> __device__ static __forceinline__ void store(float* p, const float (&v)[1]) { st<NT>(p, v[0]); }
};
template <> struct Io<float, 4> {
    typedef f32x4_t Raw;
    template <bool NT = false> __device__ static __forceinline__ Raw load_raw(const float* p) {
        return ld<NT>(reinterpret_cast<const f32x4_t*>(p));
    }
    __device__ static __forceinline__ void unpack(const Raw& r, float (&v)[4]) {
        v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    }
    __device__ static __forceinline__ void load(const float* p, float (&v)[4]) { unpack(load_raw(p), v); }
    __device__ static __forceinline__ Raw pack(const float (&v)[4]) { return f32x4_t{v[0], v[1], v[2], v[3]}; }
    template <bool NT = false> __device__ static __forceinline__ void store(float* p, const float (&v)[4]) {
        const f32x4_t q = {v[0], v[1], v[2], v[3]};
        st<NT>(reinterpret_cast<f32x4_t*>(p), q);
    }
};
template <> struct Io<float, 8> {  // the fp32 mask of a bf16 lane
    __device__ static __forceinline__ void load(const float* p, float (&v)[8]) {
        const f32x4_t q0 = reinterpret_cast<const f32x4_t*>(p)[0];
        const f32x4_t q1 = reinterpret_cast<const f32x4_t*>(p)[1];
        v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
        v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
    }
};
template <> struct Io<bf16_t, 1> {
    typedef bf16_t Raw;
    template <bool NT = false> __device__ static __forceinline__ Raw load_raw(const bf16_t* p) { return ld<NT>(p); }
    __device__ static __forceinline__ void unpack(const Raw& r, float (&v)[1]) { v[0] = __uint_as_float(uint32_t(r) << 16); }
    __device__ static __forceinline__ void load(const bf16_t* p, float (&v)[1]) { unpack(*p, v); }
    template <bool NT = false> __device__ static __forceinline__ void store(bf16_t* p, const float (&v)[1]) { st<NT>(p, to_bf16(v[0])); }
};
template <> struct Io<bf16_t, 8> {
    typedef u32x4_t Raw;
    template <bool NT = false> __device__ static __forceinline__ Raw load_raw(const bf16_t* p) {
        return ld<NT>(reinterpret_cast<const u32x4_t*>(p));
    }
    __device__ static __forceinline__ void unpack(const Raw& q, float (&v)[8]) {
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
    __device__ static __forceinline__ void load(const bf16_t* p, float (&v)[8]) { unpack(load_raw(p), v); }
    // round to nearest even
    __device__ static __forceinline__ Raw pack(const float (&v)[8]) {
        return u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7])};
    }
    template <bool NT = false> __device__ static __forceinline__ void store(bf16_t* p, const float (&v)[8]) {
        const u32x4_t q = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                           pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
        st<NT>(reinterpret_cast<u32x4_t*>(p), q);
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
    int vpt;                      // vectors per lane (blockDim apart)
    int rows_aligned;             // W % V == 0: a lane's V pixels share a row
    int identity;                 // every sample active: workgroup j takes sample j
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
    // Device-built plan (dplan = 1): step_idx holds this step's indices and
    // the sample's bucket, scale and uncond decision are derived in the
    // kernel; workgroup plan_block (if >= 0) writes the full plan and the
    // step advance.
    int dplan;
    int t_end;                    // samples with t outside [0, t_end) are skipped
    int steps, nb, wrap;
    int plan_block;
    const float* bucket_cfg;
    const float* bucket_cfg_end;  // NULL: constant within a bucket
    const float* cfg_override;
    const int32_t* covered;
    int32_t* step_out;
    int32_t* plan_bucket_id;
    float* plan_scale;
    int32_t* plan_uncond_row;
    int32_t* plan_cond_row;
    int32_t* plan_order;
    int32_t* plan_bucket_count;
    int32_t* plan_bucket_offset;
    int32_t* plan_uncond_offset;
    int32_t* plan_totals;
    const double* region_range;   // [n][R][2] validity ranges, or NULL (always valid)
    int range_steps;              // trajectory length for the ranges
    const uint16_t* covered_sets; // device plans with ranges: coverage of every region subset
    const float* record_in;       // [n][4] (sigma, sigma', scale, flags) per sample, or NULL
    float* record_out;            // plan workgroup: the records of the next step's indices
    // Norm statistics inside the step (NULL: none): the first lane of each
    // group of stats_group lanes (one latent row) writes the sums of its
    // row norms of C, U and pred to slot (sample, tile, group), 3 floats.
    float* stats_part;
    int stats_group;
    // Continuous batching (queue_len > 0): x and x_out hold n slots, and every
    // other per-sample table (means, regions, override, coverage, x_orig,
    // mask, noise) is indexed by request, queue_len of them.  A slot's record
    // carries its request (flags >> 8) and whether the request joins at this
    // step (flags bit 6: its state is built from its noise before the step).
    // The plan workgroup refills the slots whose request takes its last step
    // with the next queued requests (slot order), for the next step.
    int queue_len;
    int queue_ring;               // request ids modulo queue_len (an endless queue)
    const float* noise;           // [queue_len, C, H, W] fp32
    const int32_t* slot_req;      // [n] request of each slot at this step
    int32_t* slot_req_out;        // [n] ... at the next step
    const int32_t* queue_in;      // [1] next request of the queue
    int32_t* queue_out;           // [1]
    // Joins dispatched first: the grid starts with join_front groups of
    // `tiles` workgroups; group q takes slot join_in[q] (-1: none), whose
    // record carries flag bit 7 so the slot's own workgroups leave it.  The
    // plan workgroup lists the next step's first join_front joins in join_out.
    int join_front;
    const int32_t* join_in;       // [join_front]
    int32_t* join_out;            // [join_front]
};

// Launch parameter block of the materialised-branch step (device pointers).
struct RowsParams {
    int n, C, n_active, num_sigmas, rows;
    int phase;                    // BCG_PHASE_*
    int nvec, tiles, vpt;
    int identity;                 // every sample active: workgroup j takes sample j
    int mask_stride;              // HW if per-sample mask, else 0
    int64_t HW;
    const void* x;
    void* x_out;
    float* d;
    const void* x_tilde;
    const void* pred;
    const float* sigmas;
    const int32_t* order;
    const int32_t* step_idx;
    const float* scale;
    const int32_t* uncond_row;
    const int32_t* cond_row;
    const void* x_orig;
    const float* mask;
    // Workgroup plan_block (if >= 0), the last of the grid, builds the device
    // plan `plan` describes (another step's, typically the next) alongside the
    // update, as a one-workgroup plan launch would.
    int plan_block;
    StepParams plan;
};

// Launchers of the materialised-branch step (bcg_rows_*.hip).
hipError_t launch_rows_f32(const RowsParams& p, bool vec, bool inpaint, bool nt, int block, hipStream_t s);
hipError_t launch_rows_bf16(const RowsParams& p, bool vec, bool inpaint, bool nt, int block, hipStream_t s);

// Launchers, one per storage dtype and cache behaviour (bcg_step_*.hip).
// `vec` selects the 128-bit path; the streaming launchers take only it.
hipError_t launch_step_f32(const StepParams& p, bool vec, bool heun, bool inpaint, int block,
                           hipStream_t s);
hipError_t launch_step_bf16(const StepParams& p, bool vec, bool heun, bool inpaint, int block,
                            hipStream_t s);
hipError_t launch_step_f32_stream(const StepParams& p, bool heun, bool inpaint, int block,
                                  hipStream_t s);
hipError_t launch_step_bf16_stream(const StepParams& p, bool heun, bool inpaint, int block,
                                   hipStream_t s);
// Continuous batching (p.queue_len > 0), 16-byte vector path only (bcg_step_*_queue.hip).
hipError_t launch_step_f32_queue(const StepParams& p, bool heun, bool inpaint, int block, hipStream_t s);
hipError_t launch_step_bf16_queue(const StepParams& p, bool heun, bool inpaint, int block, hipStream_t s);

}  // namespace bcg
