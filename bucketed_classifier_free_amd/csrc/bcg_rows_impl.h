// The guided update from materialised branch predictions (one pass per call).
//
// What one launch computes, per active sample i (SGLang BCG write-up, section
// 3: the [uncond (compacted) | cond] batch layout and the per-bucket split
// and combine; ComfyUI guide "12 · Samplers, schedulers and CFG": "core of
// CFG", "the cfg = 1 optimisation", "inpaint and mask", "one step may call the
// model more than steps times"):
//   P = C (scale 1, no uncond row read) or fma(w, C - U, U) with C, U the
//   model's rows cond_row[i], uncond_row[i]; inpaint P = fma(m, P, (1-m) xo);
//   Euler x' = fma(x - P, q, x) (P on a last step);
//   Heun first call  d = (x - P)/sigma -> d, x~ = fma(h, d, x) (P on a last step);
//   Heun second call x~ = fma(h, d, x), d' = (x~ - P)/sigma',
//                    x' = fma(d + d', hh, x) (x~ copied on a last step).
// Layout and streaming as the fused inline step: workgroup = sample x tile of
// 16-byte vectors, lanes take vpt vectors blockDim apart and walk the channel
// planes (from a start channel rotated per workgroup) with the next three
// channels' loads in flight; per-sample modes (scale 1,
// last step) are uniform branches outside the channel loop.  With a device
// plan to build (guided_step_rows_dplan), one extra workgroup, the last of the
// grid, builds it while the others stream.
#pragma once

#include <atomic>
#include "bcg_device.h"
#include "bcg_plan_dev.h"

namespace bcg {

// fp32 slope vectors of V pixels.
template <int V> struct DVec;
template <> struct DVec<1> {
    typedef float Raw;
    template <bool NT> __device__ static __forceinline__ Raw load(const float* p) { return ld<NT>(p); }
    __device__ static __forceinline__ void unpack(const Raw& r, float (&v)[1]) { v[0] = r; }
    template <bool NT> __device__ static __forceinline__ void store(float* p, const float (&v)[1]) { st<NT>(p, v[0]); }
};
template <> struct DVec<4> {
    typedef f32x4_t Raw;
    template <bool NT> __device__ static __forceinline__ Raw load(const float* p) {
        return ld<NT>(reinterpret_cast<const f32x4_t*>(p));
    }
    __device__ static __forceinline__ void unpack(const Raw& r, float (&v)[4]) {
        v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    }
    template <bool NT> __device__ static __forceinline__ void store(float* p, const float (&v)[4]) {
        const f32x4_t q = {v[0], v[1], v[2], v[3]};
        st<NT>(reinterpret_cast<f32x4_t*>(p), q);
    }
};
template <> struct DVec<8> {
    struct Raw {
        f32x4_t a, b;
    };
    template <bool NT> __device__ static __forceinline__ Raw load(const float* p) {
        const f32x4_t* q = reinterpret_cast<const f32x4_t*>(p);
        return Raw{ld<NT>(q), ld<NT>(q + 1)};
    }
    __device__ static __forceinline__ void unpack(const Raw& r, float (&v)[8]) {
        v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
        v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
    }
    template <bool NT> __device__ static __forceinline__ void store(float* p, const float (&v)[8]) {
        f32x4_t* q = reinterpret_cast<f32x4_t*>(p);
        const f32x4_t a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
        st<NT>(q, a);
        st<NT>(q + 1, b);
    }
};

struct RowsScalars {
    float w, q, is, isn, h, hh;
};

// What a mode reads per element.
template <int PHASE, bool ONE, bool FIN, bool INP>
struct RowsMode {
    static constexpr bool copy = PHASE == BCG_PHASE_HEUN_CORRECT && FIN;  // x' = x~
    static constexpr bool need_x = !FIN;
    static constexpr bool need_c = !copy;
    static constexpr bool need_u = !copy && !ONE;
    static constexpr bool need_o = !copy && INP;
    static constexpr bool need_d = PHASE == BCG_PHASE_HEUN_CORRECT && !FIN;
    static constexpr bool write_d = PHASE == BCG_PHASE_HEUN_PREDICT && !FIN;
};

// The raw vectors of one channel.
template <typename T, int V, typename M>
struct RowsStage {
    typename Io<T, V>::Raw x, c, u, o, t;
    typename DVec<V>::Raw d;
};

template <typename T, int V, typename M, bool NT>
__device__ __forceinline__ void rows_load(RowsStage<T, V, M>& sg, const RowsParams& p, int64_t xoff,
                                          int64_t coff, int64_t uoff) {
    if constexpr (M::need_x) sg.x = Io<T, V>::template load_raw<NT>(static_cast<const T*>(p.x) + xoff);
    if constexpr (M::need_c) sg.c = Io<T, V>::template load_raw<NT>(static_cast<const T*>(p.pred) + coff);
    if constexpr (M::need_u) sg.u = Io<T, V>::template load_raw<NT>(static_cast<const T*>(p.pred) + uoff);
    if constexpr (M::need_o) sg.o = Io<T, V>::template load_raw<NT>(static_cast<const T*>(p.x_orig) + xoff);
    if constexpr (M::need_d) sg.d = DVec<V>::template load<NT>(p.d + xoff);
    if constexpr (M::copy) sg.t = Io<T, V>::template load_raw<NT>(static_cast<const T*>(p.x_tilde) + xoff);
}

template <typename T, int V, int PHASE, typename M, bool NT>
__device__ __forceinline__ void rows_compute(const RowsStage<T, V, M>& sg, const RowsParams& p,
                                             const RowsScalars& s, const float (&m)[V],
                                             const float (&om)[V], int64_t xoff) {
    float out[V];
    if constexpr (M::copy) {
        Io<T, V>::unpack(sg.t, out);
    } else {
        float x[V], c[V], u[V], o[V], d[V], dn[V];
        if constexpr (M::need_x) Io<T, V>::unpack(sg.x, x);
        Io<T, V>::unpack(sg.c, c);
        if constexpr (M::need_u) Io<T, V>::unpack(sg.u, u);
        if constexpr (M::need_o) Io<T, V>::unpack(sg.o, o);
        if constexpr (M::need_d) DVec<V>::unpack(sg.d, d);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float pred;
            if constexpr (M::need_u) pred = __builtin_fmaf(s.w, c[e] - u[e], u[e]);
            else pred = c[e];
            if constexpr (M::need_o) pred = __builtin_fmaf(m[e], pred, om[e] * o[e]);
            if constexpr (!M::need_x) {
                out[e] = pred;
            } else if constexpr (PHASE == BCG_PHASE_EULER) {
                out[e] = __builtin_fmaf(x[e] - pred, s.q, x[e]);
            } else if constexpr (PHASE == BCG_PHASE_HEUN_PREDICT) {
                dn[e] = (x[e] - pred) * s.is;
                out[e] = __builtin_fmaf(s.h, dn[e], x[e]);
            } else {
                const float xt = __builtin_fmaf(s.h, d[e], x[e]);
                const float d2 = (xt - pred) * s.isn;
                out[e] = __builtin_fmaf(d[e] + d2, s.hh, x[e]);
            }
        }
        if constexpr (M::write_d) DVec<V>::template store<NT>(p.d + xoff, dn);
    }
    Io<T, V>::template store<NT>(static_cast<T*>(p.x_out) + xoff, out);
}

template <typename T, int V, int PHASE, bool INP, bool NT, bool ONE, bool FIN>
__device__ __forceinline__ void rows_sample(const RowsParams& p, const RowsScalars& s, int i, int cr,
                                            int ur, int vi0, int rot) {
    typedef RowsMode<PHASE, ONE, FIN, INP> M;
    const int C = p.C;
    const int64_t HW = p.HW;
    for (int v = 0; v < p.vpt; ++v) {
        const int vi = vi0 + v * (int)blockDim.x;
        if (vi >= p.nvec) return;
        const int64_t p0 = (int64_t)vi * V;
        const int64_t xb = (int64_t)i * C * HW + p0;
        const int64_t cb = (int64_t)cr * C * HW + p0;
        const int64_t ub = (int64_t)ur * C * HW + p0;
        float m[V], om[V];
        if constexpr (M::need_o) {
            Io<float, V>::load(p.mask + (int64_t)i * p.mask_stride + p0, m);
#pragma unroll
            for (int e = 0; e < V; ++e) om[e] = 1.0f - m[e];
        }
        // walk position c is channel (c + rot) mod C
        auto plane = [&](int c) { return (int64_t)(c + rot >= C ? c + rot - C : c + rot) * HW; };
        // a ring of K single-channel stages: K - 1 channels' loads in flight
        // while one is computed (channel c lives in slot c mod K)
        constexpr int K = 4;
        RowsStage<T, V, M> st[K];
#pragma unroll
        for (int k = 0; k < K - 1; ++k) {
            if (k < C) {
                const int64_t o = plane(k);
                rows_load<T, V, M, NT>(st[k], p, xb + o, cb + o, ub + o);
            }
        }
        bool done = false;
        for (int c0 = 0; !done; c0 += K) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int c = c0 + k;
                if (c + K - 1 < C) {  // into the slot of channel c - 1, already computed
                    const int64_t o = plane(c + K - 1);
                    rows_load<T, V, M, NT>(st[(k + K - 1) % K], p, xb + o, cb + o, ub + o);
                }
                rows_compute<T, V, PHASE, M, NT>(st[k], p, s, m, om, xb + plane(c));
                if (c + 1 >= C) {
                    done = true;
                    break;
                }
            }
        }
    }
}

constexpr int kRowsPlanInts = 4 * BCG_MAX_DEVICE_BUCKETS;  // the plan workgroup's LDS

// Dynamic LDS of a rows launch of `blocks` workgroups of `block` lanes: the
// plan workgroup's counters when there is one, and, for the streaming
// (nontemporal) variants when the grid is at least two rounds at 3 waves per
// SIMD, an allocation that lets a CU hold no more workgroups than 3 waves per
// SIMD (12 per CU) need.  With the 59-109 VGPRs
// of these variants a CU would otherwise hold up to 8 waves per SIMD, and the
// large shape's grid would be one resident round that ends on the waves that
// lose arbitration: 94.7 us per step at 3 waves per SIMD against 96.7 at 8.
// (The in-place batch, ordinary loads and partly cache-resident, measured
// 93.0 us at 8 and 94.8 at 3: the cache-keep variants are not capped.)
inline hipError_t rows_lds_bytes(int64_t blocks, int block, bool plan, bool nt, size_t& bytes) {
    bytes = plan ? kRowsPlanInts * sizeof(int) : 0;
    const int waves_per_wg = (block + 63) / 64;
    const int wg_per_cu = 12 / waves_per_wg > 0 ? 12 / waves_per_wg : 1;
    // CUs and LDS per CU of the current device, looked up once per device
    // (concurrent first lookups store the same values; LDS is published first)
    constexpr int kDevices = 64;
    static std::atomic<int> cus_of[kDevices], lds_of[kDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = dev >= 0 && dev < kDevices ? cus_of[dev].load(std::memory_order_acquire) : 0;
    int lds_cu = cus > 0 ? lds_of[dev].load(std::memory_order_relaxed) : 0;
    if (cus == 0) {
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < kDevices) {
            lds_of[dev].store(lds_cu, std::memory_order_relaxed);
            cus_of[dev].store(cus, std::memory_order_release);
        }
    }
    if (nt && blocks >= (int64_t)2 * wg_per_cu * cus && lds_cu > 0) {
        // the largest allocation (in 1 KiB units) of which wg_per_cu fit and one more does not
        const size_t cap = (size_t)(lds_cu / (wg_per_cu + 1) / 1024 + 1) * 1024;
        if (cap * wg_per_cu <= (size_t)lds_cu && cap > bytes) bytes = cap;
    }
    return hipSuccess;
}

template <typename T, int V, int PHASE, bool INP, bool NT>
__global__ __launch_bounds__(256) void rows_kernel(const RowsParams p) {
    // Dynamic LDS: the plan workgroup's counters, and for large grids the
    // allocation that holds a CU to 3 waves per SIMD (rows_lds_bytes).
    extern __shared__ int rows_lds[];
    if ((int)blockIdx.x == p.plan_block) {
        plan_workgroup(p.plan, rows_lds, kRowsPlanInts);
        return;
    }
    const int j = blockIdx.x / p.tiles;
    const int tile = blockIdx.x - j * p.tiles;
    if (j >= p.n_active) return;
    const int i = p.identity ? j : p.order[j];
    if (i < 0 || i >= p.n) return;
    const int t = p.step_idx[i];
    if (t < 0 || t + 1 >= p.num_sigmas) return;
    const int cr = p.cond_row[i];
    if (cr < 0 || cr >= p.rows) return;
    RowsScalars s;
    s.w = p.scale[i];
    const bool one = s.w == 1.0f;
    const int ur = one ? 0 : p.uncond_row[i];
    if (ur < 0 || ur >= p.rows) return;
    const float sig = p.sigmas[t];
    const float sgn = p.sigmas[t + 1];
    const bool fin = sgn == 0.0f;
    s.q = (sgn - sig) / sig;
    s.h = sgn - sig;
    s.is = 1.0f / sig;
    s.isn = 1.0f / sgn;
    s.hh = s.h * 0.5f;
    const int vi0 = tile * (int)blockDim.x * p.vpt + (int)threadIdx.x;
    // the workgroup's walk starts at channel 7*blockIdx mod C (as the fused
    // step's; 97.1 us per step on the large shape against 98.8 with 5), so the
    // workgroups in flight spread their requests over the channel planes
    const int rot = (int)((7u * blockIdx.x) % (unsigned)p.C);
    if (one) {
        if (fin) rows_sample<T, V, PHASE, INP, NT, true, true>(p, s, i, cr, ur, vi0, rot);
        else rows_sample<T, V, PHASE, INP, NT, true, false>(p, s, i, cr, ur, vi0, rot);
    } else {
        if (fin) rows_sample<T, V, PHASE, INP, NT, false, true>(p, s, i, cr, ur, vi0, rot);
        else rows_sample<T, V, PHASE, INP, NT, false, false>(p, s, i, cr, ur, vi0, rot);
    }
}

template <typename T, int V, bool INP, bool NT>
hipError_t launch_rows_v(const RowsParams& p, int block, hipStream_t st) {
    const int64_t blocks = (int64_t)p.n_active * p.tiles + (p.plan_block >= 0 ? 1 : 0);
    const dim3 grid((unsigned)blocks), blk((unsigned)block);
    size_t lds = 0;
    const hipError_t e = rows_lds_bytes(blocks, block, p.plan_block >= 0, NT, lds);
    if (e != hipSuccess) return e;
    switch (p.phase) {
        case BCG_PHASE_EULER: hipLaunchKernelGGL((rows_kernel<T, V, BCG_PHASE_EULER, INP, NT>), grid, blk, lds, st, p); break;
        case BCG_PHASE_HEUN_PREDICT: hipLaunchKernelGGL((rows_kernel<T, V, BCG_PHASE_HEUN_PREDICT, INP, NT>), grid, blk, lds, st, p); break;
        default: hipLaunchKernelGGL((rows_kernel<T, V, BCG_PHASE_HEUN_CORRECT, INP, NT>), grid, blk, lds, st, p); break;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_rows(const RowsParams& p, bool vec, bool inp, bool nt, int block, hipStream_t st) {
    if (p.n_active == 0) return hipSuccess;
    constexpr int VV = VecWidth<T>::value;
    if (vec) {
        if (inp) return nt ? launch_rows_v<T, VV, true, true>(p, block, st) : launch_rows_v<T, VV, true, false>(p, block, st);
        return nt ? launch_rows_v<T, VV, false, true>(p, block, st) : launch_rows_v<T, VV, false, false>(p, block, st);
    }
    return inp ? launch_rows_v<T, 1, true, false>(p, block, st) : launch_rows_v<T, 1, false, false>(p, block, st);
}

}  // namespace bcg
