// The fused guided step kernel (one pass over the latent per sampler step).
//
// What one launch computes, per active sample i (ComfyUI guide "12 ·
// Samplers, schedulers and CFG": "core of CFG", "the cfg = 1 optimisation",
// "calc_cond_batch()", "inpaint and mask"; SGLang BCG write-up sections 3 and
// 4: per-sample scales over a mixed-bucket batch, fp32 guidance over
// half-precision storage):
//   branch predictions of the closed-form stand-in denoiser, the regional
//   cond accumulated by feathered strength weights and normalised, the CFG
//   combine with the sample's bucket scale, the inpaint blend, and the Euler
//   or Heun update, then a rounded store.
//
// Design for gfx950 (bandwidth-bound, no contraction => no MFMA):
//   * one workgroup = one sample x a tile of `blockDim` 128-bit pixel vectors;
//     per-sample scalars come from uniform loads, per-channel branch offsets
//     b_k[c] = sigma^2 mu_k[c] / (s2 + sigma^2) are computed once per
//     workgroup into LDS and read back as broadcasts;
//   * each lane owns V consecutive pixels (16 bytes of storage) and computes
//     their region weights, coverage, mask and normalisers once, then walks
//     the C channels (stride H*W), 4 channels of loads in flight at a time;
//   * every element is read once and written once (in place allowed);
//   * per-sample modes (scale == 1, last step, sample without regions) are
//     uniform branches taken outside the channel loop.
// Evaluation order (fp32, contraction off), identical for every path:
//   ax = a*x; u = ax + bu; c = ax + bc  |  c = sum_r wh_r*(ax + br_r)
//   pred = u + w*(c - u) | u + weff*(c - u) | c | (sel ? c : u)
//   pred = m*pred + (1-m)*xo;  Euler x' = x + (x - pred)*q
//   Heun d = (x - pred)*is; xt = x + h*d; d2 = (xt - pred(xt))*isn;
//        x' = x + (d + d2)*hh;  last step x' = pred.
#pragma once

#include "bcg_device.h"

namespace bcg {

constexpr int kBranches = 2 + BCG_MAX_REGIONS;   // uncond, cond, regions
constexpr int kSet = kBranches * BCG_MAX_CHANNELS;  // one sigma's coefficients

// Per-sample scalars of one step.
struct StepScalars {
    float a, a2;      // s2/(s2 + sigma^2) at sigma and sigma'
    float w;          // guidance scale
    float q;          // Euler: (sigma' - sigma)/sigma
    float h, is, isn, hh;  // Heun: sigma' - sigma, 1/sigma, 1/sigma', h*0.5
};

// Per-lane, per-pixel state (V pixels).
template <int V, int NR>
struct LaneState {
    float wh[NR > 0 ? NR : 1][V];  // normalised region weights
    float weff[V];                  // scale where covered, else 0
    bool sel[V];                    // scale-1 path: take c (else u)
    float m[V], om[V];              // inpaint mask and 1 - mask
};

template <int V, int NR, int NRB, bool INP, bool ONE>
__device__ __forceinline__ float guided_pred(const LaneState<V, NR>& L, int e, float x, float xo,
                                             float a, float w, float bu, float bc,
                                             const float (&br)[NRB > 0 ? NRB : 1]) {
    const float ax = a * x;
    const float u = ax + bu;
    float c;
    if constexpr (NRB == 0) {
        c = ax + bc;
    } else {
        c = L.wh[0][e] * (ax + br[0]);
#pragma unroll
        for (int r = 1; r < NRB; ++r) c = c + L.wh[r][e] * (ax + br[r]);
    }
    float pred;
    if constexpr (!ONE) {
        if constexpr (NRB == 0) pred = u + w * (c - u);
        else pred = u + L.weff[e] * (c - u);
    } else {
        if constexpr (NRB == 0) pred = c;
        else pred = L.sel[e] ? c : u;
    }
    if constexpr (INP) pred = L.m[e] * pred + L.om[e] * xo;
    return pred;
}

template <typename T, int V, int NR, int NRB, bool INP, bool HEUN, bool ONE, bool FINAL>
__device__ __forceinline__ void update_vec(const LaneState<V, NR>& L, const StepScalars& s,
                                           const float* __restrict__ coef, int c,
                                           const float (&xv)[V], const float (&ov)[V],
                                           float (&out)[V]) {
    const float bu = coef[c];
    const float bc = coef[BCG_MAX_CHANNELS + c];
    float br[NRB > 0 ? NRB : 1];
#pragma unroll
    for (int r = 0; r < NRB; ++r) br[r] = coef[(2 + r) * BCG_MAX_CHANNELS + c];
    float bu2 = 0.f, bc2 = 0.f;
    float br2[NRB > 0 ? NRB : 1];
    if constexpr (HEUN && !FINAL) {
        bu2 = coef[kSet + c];
        bc2 = coef[kSet + BCG_MAX_CHANNELS + c];
#pragma unroll
        for (int r = 0; r < NRB; ++r) br2[r] = coef[kSet + (2 + r) * BCG_MAX_CHANNELS + c];
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const float x = xv[e];
        const float pb = guided_pred<V, NR, NRB, INP, ONE>(L, e, x, ov[e], s.a, s.w, bu, bc, br);
        if constexpr (FINAL) {
            out[e] = pb;
        } else if constexpr (!HEUN) {
            out[e] = x + (x - pb) * s.q;
        } else {
            const float d = (x - pb) * s.is;
            const float xt = x + s.h * d;
            const float pb2 = guided_pred<V, NR, NRB, INP, ONE>(L, e, xt, ov[e], s.a2, s.w, bu2, bc2, br2);
            const float d2 = (xt - pb2) * s.isn;
            out[e] = x + (d + d2) * s.hh;
        }
    }
}

template <typename T, int V, int NR, int NRB, bool INP, bool HEUN, bool ONE, bool FINAL>
__device__ __forceinline__ void channel_loop(const LaneState<V, NR>& L, const StepScalars& s,
                                             const float* __restrict__ coef, const T* xs, T* xd,
                                             const T* xo, int C, int64_t HW) {
    constexpr int U = 4;  // channels of loads in flight per lane
    int c = 0;
    for (; c + U <= C; c += U) {
        float xv[U][V], ov[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            Io<T, V>::load(xs + (c + u) * HW, xv[u]);
            if constexpr (INP) Io<T, V>::load(xo + (c + u) * HW, ov[u]);
            else {
#pragma unroll
                for (int e = 0; e < V; ++e) ov[u][e] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float out[V];
            update_vec<T, V, NR, NRB, INP, HEUN, ONE, FINAL>(L, s, coef, c + u, xv[u], ov[u], out);
            Io<T, V>::store(xd + (c + u) * HW, out);
        }
    }
    for (; c < C; ++c) {
        float xv[V], ov[V], out[V];
        Io<T, V>::load(xs + c * HW, xv);
        if constexpr (INP) Io<T, V>::load(xo + c * HW, ov);
        else {
#pragma unroll
            for (int e = 0; e < V; ++e) ov[e] = 0.f;
        }
        update_vec<T, V, NR, NRB, INP, HEUN, ONE, FINAL>(L, s, coef, c, xv, ov, out);
        Io<T, V>::store(xd + c * HW, out);
    }
}

template <typename T, int V, int NR, int NRB, bool INP, bool HEUN>
__device__ __forceinline__ void dispatch_modes(bool one, bool fin, const LaneState<V, NR>& L,
                                               const StepScalars& s, const float* coef,
                                               const T* xs, T* xd, const T* xo, int C, int64_t HW) {
    if (one) {
        if (fin) channel_loop<T, V, NR, NRB, INP, HEUN, true, true>(L, s, coef, xs, xd, xo, C, HW);
        else channel_loop<T, V, NR, NRB, INP, HEUN, true, false>(L, s, coef, xs, xd, xo, C, HW);
    } else {
        if (fin) channel_loop<T, V, NR, NRB, INP, HEUN, false, true>(L, s, coef, xs, xd, xo, C, HW);
        else channel_loop<T, V, NR, NRB, INP, HEUN, false, false>(L, s, coef, xs, xd, xo, C, HW);
    }
}

// NR: regions evaluated per pixel (>= the sample's count; extra regions are
// zero-weight padding).  V: pixels per lane (16 bytes, or 1 for shapes whose
// H*W is not a multiple of the vector).
template <typename T, int V, int NR, bool INP, bool HEUN>
__global__ __launch_bounds__(256) void guided_step_kernel(const StepParams p) {
    __shared__ float coef[2 * kSet];
    const int j = blockIdx.x / p.tiles;
    const int tile = blockIdx.x - j * p.tiles;
    if (j >= p.n_active) return;
    const int i = p.order[j];
    if (i < 0 || i >= p.n) return;
    const int t = p.step_idx[i];
    if (t < 0 || t + 1 >= p.num_sigmas) return;

    const float sig = p.sigmas[t];
    const float sgn = p.sigmas[t + 1];
    const float w = p.scale[i];
    const bool keep_u = p.uncond_row[i] >= 0;
    int cnt = 0;
    if constexpr (NR > 0) {
        cnt = p.region_count[i];
        cnt = cnt < 0 ? 0 : cnt;
        cnt = cnt > p.R ? p.R : cnt;
        cnt = cnt > NR ? NR : cnt;
    }
    const int C = p.C;
    const float s2 = p.s2;
    const float v = sig * sig;
    const float den = s2 + v;
    const float v2 = sgn * sgn;
    const float den2 = s2 + v2;

    // Branch offsets b_k[c] = (sigma^2 mu_k[c]) / (s2 + sigma^2) into LDS.
    for (int k = threadIdx.x; k < C; k += blockDim.x) {
        const float mu_u = p.mu_uncond[(int64_t)i * C + k];
        const float mu_c = p.mu_cond[(int64_t)i * C + k];
        coef[k] = (v * mu_u) / den;
        coef[BCG_MAX_CHANNELS + k] = (v * mu_c) / den;
        if constexpr (HEUN) {
            coef[kSet + k] = (v2 * mu_u) / den2;
            coef[kSet + BCG_MAX_CHANNELS + k] = (v2 * mu_c) / den2;
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float mu_r = r < cnt ? p.mu_region[((int64_t)i * p.R + r) * C + k] : 0.0f;
            coef[(2 + r) * BCG_MAX_CHANNELS + k] = (v * mu_r) / den;
            if constexpr (HEUN) coef[kSet + (2 + r) * BCG_MAX_CHANNELS + k] = (v2 * mu_r) / den2;
        }
    }
    __syncthreads();

    const int vi = tile * (int)blockDim.x + (int)threadIdx.x;
    if (vi >= p.nvec) return;
    const int64_t p0 = (int64_t)vi * V;

    StepScalars s;
    s.a = s2 / den;
    s.a2 = s2 / den2;
    s.w = w;
    s.q = (sgn - sig) / sig;
    s.h = sgn - sig;
    s.is = 1.0f / sig;
    s.isn = 1.0f / sgn;
    s.hh = s.h * 0.5f;

    LaneState<V, NR> L;
    if constexpr (NR > 0) {
        RegionDesc rd[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            if (r < cnt) {
                const int32_t* b = p.region_box + ((int64_t)i * p.R + r) * 4;
                rd[r].y0 = b[0];
                rd[r].h = b[1] - b[0];
                rd[r].x0 = b[2];
                rd[r].w = b[3] - b[2];
                rd[r].strength = p.region_strength[(int64_t)i * p.R + r];
            } else {
                rd[r].y0 = rd[r].x0 = 0;
                rd[r].h = rd[r].w = 0;
                rd[r].strength = 0.0f;
            }
        }
        int y = (int)(p0 / p.W);
        int xx = (int)(p0 - (int64_t)y * p.W);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            float ws[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) ws[r] = region_weight(rd[r], y, xx, p.feather, p.inv_f4);
            float wsum = ws[0];
#pragma unroll
            for (int r = 1; r < NR; ++r) wsum = wsum + ws[r];
            const bool cv = wsum > 0.0f;
            const float iw = cv ? 1.0f / wsum : 0.0f;
#pragma unroll
            for (int r = 0; r < NR; ++r) L.wh[r][e] = ws[r] * iw;
            L.weff[e] = cv ? w : 0.0f;
            L.sel[e] = keep_u ? cv : true;
            if (++xx == p.W) { xx = 0; ++y; }
        }
    }
    if constexpr (INP) {
        Io<float, V>::load(p.mask + (int64_t)i * p.mask_stride + p0, L.m);
#pragma unroll
        for (int e = 0; e < V; ++e) L.om[e] = 1.0f - L.m[e];
    }

    const int64_t base = (int64_t)i * C * p.HW + p0;
    const T* xs = static_cast<const T*>(p.x) + base;
    T* xd = static_cast<T*>(p.x_out) + base;
    const T* xo = INP ? static_cast<const T*>(p.x_orig) + base : nullptr;
    const bool one = (w == 1.0f);
    const bool fin = (sgn == 0.0f);
    if (NR > 0 && cnt > 0)
        dispatch_modes<T, V, NR, NR, INP, HEUN>(one, fin, L, s, coef, xs, xd, xo, C, p.HW);
    else
        dispatch_modes<T, V, NR, 0, INP, HEUN>(one, fin, L, s, coef, xs, xd, xo, C, p.HW);
}

template <typename T, int V, int NR>
hipError_t launch_nr(const StepParams& p, bool heun, bool inp, int block, hipStream_t st) {
    const dim3 grid((unsigned)((int64_t)p.n_active * p.tiles)), blk((unsigned)block);
    if (heun) {
        if (inp) hipLaunchKernelGGL((guided_step_kernel<T, V, NR, true, true>), grid, blk, 0, st, p);
        else hipLaunchKernelGGL((guided_step_kernel<T, V, NR, false, true>), grid, blk, 0, st, p);
    } else {
        if (inp) hipLaunchKernelGGL((guided_step_kernel<T, V, NR, true, false>), grid, blk, 0, st, p);
        else hipLaunchKernelGGL((guided_step_kernel<T, V, NR, false, false>), grid, blk, 0, st, p);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_step(const StepParams& p, bool vec, bool heun, bool inp, int block, hipStream_t st) {
    if (p.n_active == 0) return hipSuccess;
    constexpr int VV = VecWidth<T>::value;
    if (!vec) {
        // Scalar path for shapes the 128-bit path cannot take; regions run
        // with the maximum count (extra regions are zero-weight padding).
        if (p.R > 0) return launch_nr<T, 1, BCG_MAX_REGIONS>(p, heun, inp, block, st);
        return launch_nr<T, 1, 0>(p, heun, inp, block, st);
    }
    switch (p.R) {
        case 0: return launch_nr<T, VV, 0>(p, heun, inp, block, st);
        case 1: return launch_nr<T, VV, 1>(p, heun, inp, block, st);
        case 2: return launch_nr<T, VV, 2>(p, heun, inp, block, st);
        case 3: return launch_nr<T, VV, 3>(p, heun, inp, block, st);
        default: return launch_nr<T, VV, 4>(p, heun, inp, block, st);
    }
}

}  // namespace bcg
