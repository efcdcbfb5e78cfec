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
//     per-sample scalars come from uniform (scalar) loads, the per-channel
//     tables of the update (below) are computed once per workgroup into LDS
//     and read back as broadcasts;
//   * each lane owns V consecutive pixels (16 bytes of storage) and computes
//     their region weights, coverage, mask and normalisers once, then walks
//     the C channels (stride H*W);
//   * the first two stages (2U channels) are requested before the pixel and
//     coefficient set-up (the LDS barrier waits on LDS traffic only), and the
//     channel walk is software-pipelined: the loads of channels c+U.. are in
//     flight while channels c.. are computed and stored;
//   * every element is read once and written once (in place allowed);
//   * per-sample modes (scale == 1, last step, sample without regions) are
//     uniform branches taken outside the channel loop.
// Evaluation order (fp32; contraction off, so the only fused operations are
// the explicit fma(a, b, c) = a*b + c rounded once).  The stand-in denoiser
// is affine in x, so every branch, the CFG combine, the inpaint blend and
// both of Heun's evaluations fold into x' = K x + B: K per sample (per pixel
// when inpainting), B from per-channel tables and per-pixel region weights:
//   per sample:  a = s2/den, b1 = v/den (v = sigma^2, den = s2 + v);
//     last step  g = 1, K = a;  Euler q = (sigma'-sigma)/sigma, g = -q,
//     K = fma(q, b1, 1);  Heun e1 = b1/sigma, e2 = b2/sigma',
//     K = fma(hh, fma(e2, fma(h, e1, 1), e1), 1), c1 = (-hh/sigma) fma(h, e2, 1),
//     c2 = -hh/sigma'
//   per channel: bu = v mu_u/den; without regions one offset
//     P = fma(w, v (mu_c - mu_u)/den, bu) (v mu_c/den at scale 1); with
//     regions t0 = bu, t_r = v (mu_r - mu_u)/den (also when the uncond is
//     skipped: where no region has weight the cond is the uncond); tables
//     g*t, or fma(c1, t, c2*t') for Heun (t' at sigma')
//   per pixel:   om_r = (covered ? w : 0) * wh_r (normalised region weights)
//   per element: B = T0, B = fma(om_r, T_r, B);  x' = fma(K, x, B)
//   inpaint:     x' = fma(k, x, fma(l1, B1, [fma(l2, B2,] lo*xo)) with the
//                per-pixel k, l1, l2, lo of the mask, B1/B2 unscaled chains.
#pragma once

#include "bcg_device.h"
#include "bcg_plan_dev.h"

namespace bcg {

constexpr int kBranches = 2 + BCG_MAX_REGIONS;      // uncond, cond, regions
constexpr int kSet = kBranches * BCG_MAX_CHANNELS;  // one sigma's coefficients
constexpr int kPlanLds = 4 * 2 * kSet;              // ints of the coefficient LDS

// Compile-time tuning of the streaming loop (the stage width U is chosen per
// kernel variant at launch, see stage_width).
template <int U_, bool NT_, bool PF_ = false, bool FULL_ = false, bool STATS_ = false, bool QUEUE_ = false>
struct Tune {
    static constexpr int U = U_;        // channels per pipeline stage
    static constexpr bool NT = NT_;     // nontemporal (streaming) loads and stores
    static constexpr bool PF = PF_;     // next pass's head stage requested during this pass
    static constexpr bool FULL = FULL_; // C is a multiple of 2U: every stage is full
    static constexpr bool STATS = STATS_;  // norm statistics of the first evaluation
    static constexpr bool QUEUE = QUEUE_;  // continuous batching: slots hold requests
};
template <typename TN>
using QueueOf = Tune<TN::U, TN::NT, TN::PF, TN::FULL, false, true>;
typedef Tune<2, false, false, false, true> StatsTune;  // ordinary loads/stores, with the statistics
typedef Tune<2, false> KeepTune;    // ordinary loads/stores (BCG_CACHE_KEEP)
typedef Tune<2, true> StreamTune;   // nontemporal loads/stores (BCG_CACHE_STREAM)
typedef KeepTune DefaultTune;

// Per-sample scalars of one step.
struct StepScalars {
    float a, a2;           // s2/(s2 + sigma^2) at sigma and sigma'
    float w;               // guidance scale
    float q;               // Euler: (sigma' - sigma)/sigma
    float h, is, isn, hh;  // Heun: sigma' - sigma, 1/sigma, 1/sigma', h*0.5
    float g;               // Euler and last step: the tables' factor (-q, or 1)
    float K;               // x' = K x + B
    float c1, c2;          // Heun: the tables' weights at sigma and sigma'
};

// Per-lane, per-pixel state (V pixels).
template <int V, int NR>
struct LaneState {
    float wh[NR > 0 ? NR : 1][V];  // normalised region weights
    float weff[V];                  // scale where covered, else 0
    bool sel[V];                    // scale-1 path: take c (else u) (statistics)
    bool cov[V];                    // some region has weight
    float m[V], om[V];              // inpaint mask and 1 - mask
    float wr[NR > 0 ? NR : 1][V];  // folded: weff * wh_r
    float k[V], l1[V], l2[V], lo[V];  // folded inpaint: x' = fma(k, x, fma(l1, B1, [fma(l2, B2,] lo*xo))
};

// Norm statistics of one lane: sums of squares of C, U and pred over the
// lane's pixels of the current channel (sq), and the running sums of the row
// norms of its lane group (tot; every lane of a group holds the same values).
struct LaneStats {
    float sq[3];
    float tot[3];
};

// The norm statistics of one element: the branch predictions U and C and
// their combine (before the inpaint blend), each as its own sequence --
// u = fma(a, x, bu); c = fma(a, x, bc), or c = wh_0*fma(a, x, br_0),
// c = fma(wh_r, fma(a, x, br_r), c); pred = fma(w, c - u, u) or
// fma(weff, c - u, u), c (sel ? c : u) at scale 1 -- added to the lane's
// sums of squares (C is U where no region has weight).
template <int V, int NR, int NRB, bool ONE>
__device__ __forceinline__ void stats_element(const LaneState<V, NR>& L, int e, float x, float a, float w,
                                              float bu, float bc, const float (&br)[NRB > 0 ? NRB : 1],
                                              LaneStats* st) {
    const float u = __builtin_fmaf(a, x, bu);
    float c;
    if constexpr (NRB == 0) {
        c = __builtin_fmaf(a, x, bc);
    } else {
        c = L.wh[0][e] * __builtin_fmaf(a, x, br[0]);
#pragma unroll
        for (int r = 1; r < NRB; ++r) c = __builtin_fmaf(L.wh[r][e], __builtin_fmaf(a, x, br[r]), c);
    }
    float pred;
    if constexpr (!ONE) {
        if constexpr (NRB == 0) pred = __builtin_fmaf(w, c - u, u);
        else pred = __builtin_fmaf(L.weff[e], c - u, u);
    } else {
        if constexpr (NRB == 0) pred = c;
        else pred = L.sel[e] ? c : u;
    }
    const float cs = (NRB == 0 || L.cov[e]) ? c : u;
    st->sq[0] = __builtin_fmaf(cs, cs, st->sq[0]);
    st->sq[1] = __builtin_fmaf(u, u, st->sq[1]);
    st->sq[2] = __builtin_fmaf(pred, pred, st->sq[2]);
}

// One channel's V elements: x' = K x + B, B = T0 + sum_r om_r T_r from the
// channel's tables (coef: slot 0 and slots 1.. of the regions; the inpaint
// blend of Heun's step keeps the chains at sigma and sigma' apart, the second
// at kSet; the statistics' branch offsets at 2 kSet).
template <int V, int NR, int NRB, bool INP, bool HEUN, bool ONE, bool FINAL, bool ST = false>
__device__ __forceinline__ void update_vec(const LaneState<V, NR>& L, const StepScalars& s,
                                           const float* __restrict__ coef, int c,
                                           const float (&xv)[V], const float (&ov)[V],
                                           float (&out)[V], LaneStats* st = nullptr) {
    constexpr bool TWO = INP && HEUN && !FINAL;
    constexpr int NB = NRB > 0 ? NRB : 1;
    const float t0 = coef[c];
    float tr[NB];
#pragma unroll
    for (int r = 0; r < NRB; ++r) tr[r] = coef[(1 + r) * BCG_MAX_CHANNELS + c];
    float t0b = 0.0f, trb[NB];
    if constexpr (TWO) {
        t0b = coef[kSet + c];
#pragma unroll
        for (int r = 0; r < NRB; ++r) trb[r] = coef[kSet + (1 + r) * BCG_MAX_CHANNELS + c];
    }
    float bu = 0.0f, bc = 0.0f, br[NB];
    if constexpr (ST) {
        bu = coef[2 * kSet + c];
        bc = coef[2 * kSet + BCG_MAX_CHANNELS + c];
#pragma unroll
        for (int r = 0; r < NRB; ++r) br[r] = coef[2 * kSet + (2 + r) * BCG_MAX_CHANNELS + c];
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const float x = xv[e];
        if constexpr (ST) stats_element<V, NR, NRB, ONE>(L, e, x, s.a, s.w, bu, bc, br, st);
        float B = t0;
#pragma unroll
        for (int r = 0; r < NRB; ++r) B = __builtin_fmaf(L.wr[r][e], tr[r], B);
        if constexpr (!INP) {
            out[e] = __builtin_fmaf(s.K, x, B);
        } else if constexpr (TWO) {
            float B2 = t0b;
#pragma unroll
            for (int r = 0; r < NRB; ++r) B2 = __builtin_fmaf(L.wr[r][e], trb[r], B2);
            out[e] = __builtin_fmaf(L.k[e], x, __builtin_fmaf(L.l1[e], B, __builtin_fmaf(L.l2[e], B2, L.lo[e] * ov[e])));
        } else {
            out[e] = __builtin_fmaf(L.k[e], x, __builtin_fmaf(L.l1[e], B, L.lo[e] * ov[e]));
        }
    }
}

// One pipeline stage: the raw vectors of U consecutive channels (x and, when
// inpainting, the original latent).
template <typename T, int V, int U, bool INP>
struct Stage {
    typename Io<T, V>::Raw x[U];
    typename Io<T, V>::Raw o[INP ? U : 1];
};

// Channel visited at walk position c (0 <= c < C) by a workgroup whose walk
// starts at channel rot (0 <= rot < C).
__device__ __forceinline__ int walk_channel(int c, int rot, int C) {
    const int r = c + rot;
    return r >= C ? r - C : r;
}

// Elements from a sample's start to channel plane c: c < 64 and H*W <= 2^30
// (both checked at launch), so one 32 x 32 -> 64-bit product.
__device__ __forceinline__ int64_t plane_offset(int c, int64_t HW) {
    return (int64_t)((uint64_t)(uint32_t)c * (uint64_t)(uint32_t)HW);
}

template <typename T, int V, typename TN, bool INP>
__device__ __forceinline__ void load_stage(Stage<T, V, TN::U, INP>& sg, const T* xs, const T* xo,
                                           int c0, int rot, int C, int64_t HW) {
#pragma unroll
    for (int u = 0; u < TN::U; ++u) {
        if (TN::FULL || c0 + u < C) {
            const int64_t off = plane_offset(walk_channel(c0 + u, rot, C), HW);
            sg.x[u] = Io<T, V>::template load_raw<TN::NT>(xs + off);
            if constexpr (INP) sg.o[u] = Io<T, V>::template load_raw<TN::NT>(xo + off);
        }
    }
}

// The row norms of one channel for the statistics: the lanes of a latent row
// (a group of `group` lanes, a power of two) add their sums of squares in a
// fixed butterfly, and each lane adds the square roots to its running sums.
__device__ __forceinline__ void stats_rows(LaneStats& st, int group) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        float v = st.sq[q];
        for (int o = group >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
        st.tot[q] += sqrtf(v);
        st.sq[q] = 0.0f;
    }
}

template <typename T, int V, typename TN, int NR, int NRB, bool INP, bool HEUN, bool ONE, bool FINAL>
__device__ __forceinline__ void compute_stage(const Stage<T, V, TN::U, INP>& sg, const LaneState<V, NR>& L,
                                              const StepScalars& s, const float* __restrict__ coef,
                                              T* xd, int c0, int rot, int C, int64_t HW, LaneStats* st,
                                              int group) {
#pragma unroll
    for (int u = 0; u < TN::U; ++u) {
        if (TN::FULL || c0 + u < C) {
            const int c = walk_channel(c0 + u, rot, C);
            float xv[V], ov[V], out[V];
            Io<T, V>::unpack(sg.x[u], xv);
            if constexpr (INP) Io<T, V>::unpack(sg.o[u], ov);
            else {
#pragma unroll
                for (int e = 0; e < V; ++e) ov[e] = 0.f;
            }
            update_vec<V, NR, NRB, INP, HEUN, ONE, FINAL, TN::STATS>(L, s, coef, c, xv, ov, out, st);
            Io<T, V>::template store<TN::NT>(xd + plane_offset(c, HW), out);
            if constexpr (TN::STATS) stats_rows(*st, group);
        }
    }
}

// The channel walk, two stages in flight (ping-pong): stage `a` arrives
// holding channels [0, U) already requested, and stage `b` channels [U, 2U)
// when b_ready.  When the lane has a next pass
// (nxs != nullptr), its head stage is requested into whichever buffer frees up
// during this pass's last stage, so the walk does not drain between passes;
// the return value says where it went (true: `b`, false: `a`).
template <typename T, int V, typename TN, int NR, int NRB, bool INP, bool HEUN, bool ONE, bool FINAL>
__device__ __forceinline__ bool channel_loop(Stage<T, V, TN::U, INP>& a, Stage<T, V, TN::U, INP>& b,
                                             const LaneState<V, NR>& L, const StepScalars& s,
                                             const float* __restrict__ coef, const T* xs, T* xd, const T* xo,
                                             const T* nxs, const T* nxo, int rot, int C, int64_t HW,
                                             bool b_ready, LaneStats* st, int group) {
    constexpr int U = TN::U;
    for (int c0 = 0;; c0 += 2 * U) {
        if (c0 + U < C) {
            if (c0 > 0 || !b_ready) load_stage<T, V, TN, INP>(b, xs, xo, c0 + U, rot, C, HW);
        }
        else if (nxs) load_stage<T, V, TN, INP>(b, nxs, nxo, 0, rot, C, HW);
        compute_stage<T, V, TN, NR, NRB, INP, HEUN, ONE, FINAL>(a, L, s, coef, xd, c0, rot, C, HW, st, group);
        if (c0 + U >= C) return true;
        if (c0 + 2 * U < C) load_stage<T, V, TN, INP>(a, xs, xo, c0 + 2 * U, rot, C, HW);
        else if (nxs) load_stage<T, V, TN, INP>(a, nxs, nxo, 0, rot, C, HW);
        compute_stage<T, V, TN, NR, NRB, INP, HEUN, ONE, FINAL>(b, L, s, coef, xd, c0 + U, rot, C, HW, st, group);
        if (c0 + 2 * U >= C) return false;
    }
}

// Per-sample constants a lane needs to set up its pixels.
template <int NR>
struct SampleRegions {
    RegionDesc rd[NR > 0 ? NR : 1];
    int cnt;
};

// Normalised weights, coverage flag and guided-scale of one pixel from its
// region weights ws (sum, one correctly rounded reciprocal, products).
template <int V, int NR, int NRB>
__device__ __forceinline__ void finish_pixel(LaneState<V, NR>& L, int e, const float (&ws)[NRB], float w,
                                             bool keep_u) {
    float wsum = ws[0];
#pragma unroll
    for (int r = 1; r < NRB; ++r) wsum = wsum + ws[r];
    const bool cv = wsum > 0.0f;
    const float iw = cv ? 1.0f / wsum : 0.0f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) L.wh[r][e] = ws[r] * iw;
    L.weff[e] = cv ? w : 0.0f;
    L.sel[e] = keep_u ? cv : true;
    L.cov[e] = cv;
}

// Region weights, coverage and mask of the V pixels starting at p0.  When
// the lane's pixels share a row, the feather's row factor is the lane's and
// each pixel adds its column factor: n = n_y * n_x with both factors products
// of two clamped distances (at most F^2 <= 4096, so 24-bit multiplies are
// exact), the same integer region_weight forms, converted and scaled alike.
template <int V, int NR, int NRB, bool INP>
__device__ __forceinline__ void setup_lane(LaneState<V, NR>& L, const SampleRegions<NR>& sr,
                                           const StepParams& p, int i, int64_t p0, float w,
                                           bool keep_u) {
    if constexpr (NRB > 0) {
        const int F = p.feather;
        const float inv_f4 = p.inv_f4;
        const int y = (int)(p0 / p.W);
        const int xx = (int)(p0 - (int64_t)y * p.W);
        if (p.rows_aligned != 0) {
            unsigned ny[NRB];  // feather factors of the lane's row
            int dx0[NRB];      // column of the lane's first pixel inside each box
#pragma unroll
            for (int r = 0; r < NRB; ++r) {
                const int dy = y - sr.rd[r].y0;
                const unsigned f = __umul24((unsigned)min(dy + 1, F), (unsigned)min(sr.rd[r].h - dy, F));
                ny[r] = (unsigned)dy < (unsigned)sr.rd[r].h ? f : 0u;
                dx0[r] = xx - sr.rd[r].x0;
            }
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float ws[NRB];
#pragma unroll
                for (int r = 0; r < NRB; ++r) {
                    const int dx = dx0[r] + e;
                    const unsigned fx = __umul24((unsigned)min(dx + 1, F), (unsigned)min(sr.rd[r].w - dx, F));
                    const unsigned nx = (unsigned)dx < (unsigned)sr.rd[r].w ? fx : 0u;
                    const float f = float(__umul24(ny[r], nx)) * inv_f4;
                    ws[r] = sr.rd[r].strength * f;
                }
                finish_pixel<V, NR, NRB>(L, e, ws, w, keep_u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float ws[NRB];
#pragma unroll
                for (int r = 0; r < NRB; ++r) {
                    const int px = xx + e;  // walk the row, wrapping to the next
                    ws[r] = region_weight(sr.rd[r], y + px / p.W, px - (px / p.W) * p.W, F, inv_f4);
                }
                finish_pixel<V, NR, NRB>(L, e, ws, w, keep_u);
            }
        }
    }
    if constexpr (INP) {
        Io<float, V>::load(p.mask + (int64_t)i * p.mask_stride + p0, L.m);
#pragma unroll
        for (int e = 0; e < V; ++e) L.om[e] = 1.0f - L.m[e];
    }
}

// The per-pixel factors of the folded update: the region weights times the
// pixel's guidance (om_r = weff * wh_r), and with inpainting the mask's
// coefficients:
//   last   k = m a, l1 = g m, lo = g (1 - m)
//   Euler  k = fma(q, fma(-m, a, 1), 1), l1 = g m, lo = g (1 - m)
//   Heun   A = fma(-m, a, 1) at sigma and sigma', f = A/sigma, f' = A'/sigma',
//          G = fma(h, f', 1), k = fma(hh, fma(f', fma(h, f, 1), f), 1),
//          l1 = ((-hh/sigma) G) m, l2 = (-hh/sigma') m, lo = (-hh fma(1/sigma, G, 1/sigma')) (1 - m)
// (each "/sigma" a product with the correctly rounded reciprocal).
template <int V, int NR, int NRB, bool INP, bool HEUN, bool FINAL>
__device__ __forceinline__ void fold_lane(LaneState<V, NR>& L, const StepScalars& s) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
#pragma unroll
        for (int r = 0; r < NRB; ++r) L.wr[r][e] = L.weff[e] * L.wh[r][e];
        if constexpr (INP) {
            const float m = L.m[e], om = L.om[e];
            const float al = s.a;
            if constexpr (FINAL) {
                L.k[e] = m * al;
                L.l1[e] = s.g * m;
                L.lo[e] = s.g * om;
            } else if constexpr (!HEUN) {
                L.k[e] = __builtin_fmaf(s.q, __builtin_fmaf(-m, al, 1.0f), 1.0f);
                L.l1[e] = s.g * m;
                L.lo[e] = s.g * om;
            } else {
                const float f1 = s.is * __builtin_fmaf(-m, al, 1.0f);
                const float f2 = s.isn * __builtin_fmaf(-m, s.a2, 1.0f);
                const float G = __builtin_fmaf(s.h, f2, 1.0f);
                const float nh = -s.hh;
                L.k[e] = __builtin_fmaf(s.hh, __builtin_fmaf(f2, __builtin_fmaf(s.h, f1, 1.0f), f1), 1.0f);
                L.l1[e] = ((nh * s.is) * G) * m;
                L.l2[e] = (nh * s.isn) * m;
                L.lo[e] = (nh * __builtin_fmaf(s.is, G, s.isn)) * om;
            }
        }
    }
}

// A lane's vectors vi0, vi0 + blockDim, ... (p.vpt of them) of one sample.
template <typename T, int V, typename TN, int NR, int NRB, bool INP, bool HEUN, bool ONE, bool FINAL>
__device__ __forceinline__ void run_lane(Stage<T, V, TN::U, INP>& a, Stage<T, V, TN::U, INP>& b,
                                         LaneState<V, NR>& L, const SampleRegions<NR>& sr,
                                         const StepParams& p, const StepScalars& s,
                                         const float* __restrict__ coef, int i, int ri, int vi0, int rot,
                                         bool keep_u, LaneStats* st) {
    const int C = p.C;
    const int64_t sbase = (int64_t)i * C * p.HW;   // the slot's state
    const int64_t rbase = (int64_t)ri * C * p.HW;  // its request's original latent
    for (int v = 0; v < p.vpt; ++v) {
        const int vi = vi0 + v * (int)blockDim.x;
        if (vi >= p.nvec) return;
        const int64_t p0 = (int64_t)vi * V;
        const T* xs = static_cast<const T*>(p.x) + sbase + p0;
        T* xd = static_cast<T*>(p.x_out) + sbase + p0;
        const T* xo = INP ? static_cast<const T*>(p.x_orig) + rbase + p0 : nullptr;
        // the next pass's pixels (its head stage is requested during this pass)
        const int nvi = vi + (int)blockDim.x;
        const bool more = TN::PF && v + 1 < p.vpt && nvi < p.nvec;
        const int64_t np0 = (int64_t)nvi * V;
        const T* nxs = more ? static_cast<const T*>(p.x) + sbase + np0 : nullptr;
        const T* nxo = (more && INP) ? static_cast<const T*>(p.x_orig) + rbase + np0 : nullptr;
        if (v > 0) {
            if (!TN::PF) load_stage<T, V, TN, INP>(a, xs, xo, 0, rot, C, p.HW);  // else requested during the last pass
            setup_lane<V, NR, NRB, INP>(L, sr, p, ri, p0, s.w, keep_u);
        }
        fold_lane<V, NR, NRB, INP, HEUN, FINAL>(L, s);
        const bool in_b = channel_loop<T, V, TN, NR, NRB, INP, HEUN, ONE, FINAL>(a, b, L, s, coef, xs, xd, xo,
                                                                                  nxs, nxo, rot, C, p.HW, v == 0,
                                                                                  st, p.stats_group);
        if (more && in_b) a = b;
    }
}

// A request joining at this step (continuous batching): its state is built
// from its noise at the step's sigma -- noise * sigma, plus its original
// latent when inpainting (one fused multiply-add), stored in the storage
// dtype -- and stepped at once; the slot's previous contents are not read.
// The walk is pipelined like the slot's own (two stages, the next one's loads
// in flight during a compute), a stage holding UJ channels of fp32 noise: half
// the stage width for bf16 storage, so the noise takes the registers the
// state's stages take.
template <typename T, int V, typename TN, bool INP>
struct JoinStage {
    static constexpr int UJ = sizeof(T) == 2 ? (TN::U > 1 ? TN::U / 2 : 1) : TN::U;
    f32x4_t nz[UJ][V / 4];
    typename Io<T, V>::Raw o[INP ? UJ : 1];
};

template <typename T, int V, typename TN, bool INP>
__device__ __forceinline__ void join_load(JoinStage<T, V, TN, INP>& sg, const StepParams& p, int64_t rbase,
                                          int64_t p0, int c0, int rot) {
    constexpr int UJ = JoinStage<T, V, TN, INP>::UJ;
#pragma unroll
    for (int u = 0; u < UJ; ++u) {
        if (c0 + u < p.C) {
            const int64_t ro = rbase + plane_offset(walk_channel(c0 + u, rot, p.C), p.HW) + p0;
#pragma unroll
            for (int q = 0; q < V / 4; ++q)
                sg.nz[u][q] = ld<TN::NT>(reinterpret_cast<const f32x4_t*>(p.noise + ro) + q);
            if constexpr (INP) sg.o[u] = Io<T, V>::template load_raw<TN::NT>(static_cast<const T*>(p.x_orig) + ro);
        }
    }
}

template <typename T, int V, typename TN, int NR, int NRB, bool INP, bool HEUN, bool ONE, bool FINAL>
__device__ __forceinline__ void join_compute(const JoinStage<T, V, TN, INP>& sg, const LaneState<V, NR>& L,
                                             const StepScalars& s, const float* __restrict__ coef,
                                             const StepParams& p, T* xd, int c0, int rot, float sig) {
    constexpr int UJ = JoinStage<T, V, TN, INP>::UJ;
#pragma unroll
    for (int u = 0; u < UJ; ++u) {
        if (c0 + u < p.C) {
            const int c = walk_channel(c0 + u, rot, p.C);
            float ov[V], xv[V], out[V];
            if constexpr (INP) Io<T, V>::unpack(sg.o[u], ov);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float nz = sg.nz[u][e / 4][e % 4];
                if constexpr (!INP) ov[e] = 0.0f;
                xv[e] = INP ? __builtin_fmaf(nz, sig, ov[e]) : nz * sig;
            }
            Io<T, V>::unpack(Io<T, V>::pack(xv), xv);  // the stored state
            update_vec<V, NR, NRB, INP, HEUN, ONE, FINAL>(L, s, coef, c, xv, ov, out);
            Io<T, V>::template store<TN::NT>(xd + plane_offset(c, p.HW), out);
        }
    }
}

template <typename T, int V, typename TN, int NR, int NRB, bool INP, bool HEUN, bool ONE, bool FINAL>
__device__ __forceinline__ void join_lane(LaneState<V, NR>& L, const SampleRegions<NR>& sr, const StepParams& p,
                                          const StepScalars& s, const float* __restrict__ coef, int i, int ri,
                                          int vi0, int rot, bool keep_u, float sig) {
    typedef JoinStage<T, V, TN, INP> JS;
    constexpr int UJ = JS::UJ;
    const int C = p.C;
    const int64_t rbase = (int64_t)ri * C * p.HW;
    for (int v = 0; v < p.vpt; ++v) {
        const int vi = vi0 + v * (int)blockDim.x;
        if (vi >= p.nvec) return;
        const int64_t p0 = (int64_t)vi * V;
        T* xd = static_cast<T*>(p.x_out) + (int64_t)i * C * p.HW + p0;
        JS a, b;
        join_load<T, V, TN, INP>(a, p, rbase, p0, 0, rot);
        if (UJ < C) join_load<T, V, TN, INP>(b, p, rbase, p0, UJ, rot);
        if (v > 0) setup_lane<V, NR, NRB, INP>(L, sr, p, ri, p0, s.w, keep_u);
        fold_lane<V, NR, NRB, INP, HEUN, FINAL>(L, s);
        for (int c0 = 0;; c0 += 2 * UJ) {
            join_compute<T, V, TN, NR, NRB, INP, HEUN, ONE, FINAL>(a, L, s, coef, p, xd, c0, rot, sig);
            if (c0 + UJ >= C) break;
            if (c0 + 2 * UJ < C) join_load<T, V, TN, INP>(a, p, rbase, p0, c0 + 2 * UJ, rot);
            join_compute<T, V, TN, NR, NRB, INP, HEUN, ONE, FINAL>(b, L, s, coef, p, xd, c0 + UJ, rot, sig);
            if (c0 + 2 * UJ >= C) break;
            if (c0 + 3 * UJ < C) join_load<T, V, TN, INP>(b, p, rbase, p0, c0 + 3 * UJ, rot);
        }
    }
}

// After the first two stages are requested: the first pass's pixel set-up
// (it overlaps the latent loads), then the branch offsets into this wavefront's
// own LDS slice (lane k computes channel k's; no workgroup barrier), then the
// channel walks.
template <typename T, int V, typename TN, int NR, int NRB, bool INP, bool HEUN>
__device__ __forceinline__ void run_sample(Stage<T, V, TN::U, INP>& a, Stage<T, V, TN::U, INP>& b, bool lane_ok,
                                           const SampleRegions<NR>& sr, const StepParams& p,
                                           StepScalars s, float* coef, int i, int ri, bool join, int vi0,
                                           int rot, bool keep_u, float sig, float sgn, float mu_u, float mu_c,
                                           const float (&mu_r)[NR > 0 ? NR : 1]) {
    LaneState<V, NR> L;
    if (lane_ok) setup_lane<V, NR, NRB, INP>(L, sr, p, ri, (int64_t)vi0 * V, s.w, keep_u);

    const int C = p.C;
    const float s2 = p.s2;
    const float v = sig * sig;
    const float den = s2 + v;
    const float v2 = sgn * sgn;
    const float den2 = s2 + v2;
    const bool one = (s.w == 1.0f);
    const bool fin = (sgn == 0.0f);
    const bool two = HEUN && !fin;  // Heun's second evaluation takes part
    // the sample's scalars of the folded update
    s.a = s2 / den;
    s.a2 = s2 / den2;
    const float b1 = v / den;
    s.h = sgn - sig;
    s.q = s.h / sig;
    s.is = 1.0f / sig;
    s.isn = 1.0f / sgn;
    s.hh = s.h * 0.5f;
    s.c1 = 0.0f;
    s.c2 = 0.0f;
    if (!two) {
        s.g = fin ? 1.0f : -s.q;
        s.K = fin ? s.a : __builtin_fmaf(s.q, b1, 1.0f);
    } else {
        const float e1 = b1 * s.is, e2 = (v2 / den2) * s.isn, nh = -s.hh;
        s.g = 1.0f;
        s.K = __builtin_fmaf(s.hh, __builtin_fmaf(e2, __builtin_fmaf(s.h, e1, 1.0f), e1), 1.0f);
        s.c1 = (nh * s.is) * __builtin_fmaf(s.h, e2, 1.0f);
        s.c2 = nh * s.isn;
    }
    // Channel k's tables (lane k): the offsets at sigma (and sigma'), folded
    // with the step's weights unless the inpaint blend needs them apart.
    const int k = (int)threadIdx.x & 63;
    if (k < C) {
        constexpr int NB = NRB > 0 ? NRB : 1;
        float t0, tr[NB], t0b = 0.0f, trb[NB];
        const float bu = (v * mu_u) / den;
        if constexpr (NRB == 0) {
            t0 = one ? (v * mu_c) / den : __builtin_fmaf(s.w, (v * (mu_c - mu_u)) / den, bu);
        } else {
            t0 = bu;
#pragma unroll
            for (int r = 0; r < NRB; ++r) tr[r] = (v * (mu_r[r] - mu_u)) / den;
        }
        if (two) {
            const float bub = (v2 * mu_u) / den2;
            if constexpr (NRB == 0) {
                t0b = one ? (v2 * mu_c) / den2 : __builtin_fmaf(s.w, (v2 * (mu_c - mu_u)) / den2, bub);
            } else {
                t0b = bub;
#pragma unroll
                for (int r = 0; r < NRB; ++r) trb[r] = (v2 * (mu_r[r] - mu_u)) / den2;
            }
        }
        if constexpr (!INP) {
            if (two) {
                coef[k] = __builtin_fmaf(s.c1, t0, s.c2 * t0b);
#pragma unroll
                for (int r = 0; r < NRB; ++r)
                    coef[(1 + r) * BCG_MAX_CHANNELS + k] = __builtin_fmaf(s.c1, tr[r], s.c2 * trb[r]);
            } else {
                coef[k] = s.g * t0;
#pragma unroll
                for (int r = 0; r < NRB; ++r) coef[(1 + r) * BCG_MAX_CHANNELS + k] = s.g * tr[r];
            }
        } else {
            coef[k] = t0;
#pragma unroll
            for (int r = 0; r < NRB; ++r) coef[(1 + r) * BCG_MAX_CHANNELS + k] = tr[r];
            if (two) {
                coef[kSet + k] = t0b;
#pragma unroll
                for (int r = 0; r < NRB; ++r) coef[kSet + (1 + r) * BCG_MAX_CHANNELS + k] = trb[r];
            }
        }
        if constexpr (TN::STATS) {  // the branch offsets of the statistics
            coef[2 * kSet + k] = bu;
            coef[2 * kSet + BCG_MAX_CHANNELS + k] = (v * mu_c) / den;
#pragma unroll
            for (int r = 0; r < NRB; ++r) coef[2 * kSet + (2 + r) * BCG_MAX_CHANNELS + k] = (v * mu_r[r]) / den;
        }
    }
    // LDS writes of this wavefront become visible to all its lanes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (!lane_ok) return;

    LaneStats st = {{0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f}};
    if constexpr (TN::QUEUE) {
        if (join) {
            if (one) {
                if (fin) join_lane<T, V, TN, NR, NRB, INP, HEUN, true, true>(L, sr, p, s, coef, i, ri, vi0, rot, keep_u, sig);
                else join_lane<T, V, TN, NR, NRB, INP, HEUN, true, false>(L, sr, p, s, coef, i, ri, vi0, rot, keep_u, sig);
            } else {
                if (fin) join_lane<T, V, TN, NR, NRB, INP, HEUN, false, true>(L, sr, p, s, coef, i, ri, vi0, rot, keep_u, sig);
                else join_lane<T, V, TN, NR, NRB, INP, HEUN, false, false>(L, sr, p, s, coef, i, ri, vi0, rot, keep_u, sig);
            }
            return;
        }
    }
    if (one) {
        if (fin) run_lane<T, V, TN, NR, NRB, INP, HEUN, true, true>(a, b, L, sr, p, s, coef, i, ri, vi0, rot, keep_u, &st);
        else run_lane<T, V, TN, NR, NRB, INP, HEUN, true, false>(a, b, L, sr, p, s, coef, i, ri, vi0, rot, keep_u, &st);
    } else {
        if (fin) run_lane<T, V, TN, NR, NRB, INP, HEUN, false, true>(a, b, L, sr, p, s, coef, i, ri, vi0, rot, keep_u, &st);
        else run_lane<T, V, TN, NR, NRB, INP, HEUN, false, false>(a, b, L, sr, p, s, coef, i, ri, vi0, rot, keep_u, &st);
    }
    if constexpr (TN::STATS) {
        // the first lane of each row group writes the group's sums of row
        // norms: slot (sample, tile, group) of the partials
        const int g = (int)threadIdx.x / p.stats_group;
        if ((int)threadIdx.x == g * p.stats_group) {
            const int tile = (int)blockIdx.x - (int)(blockIdx.x / p.tiles) * p.tiles;
            const int64_t slot = ((int64_t)i * p.tiles + tile) * ((int)blockDim.x / p.stats_group) + g;
            float* o = p.stats_part + slot * 3;
            o[0] = st.tot[0];
            o[1] = keep_u ? st.tot[1] : 0.0f;
            o[2] = st.tot[2];
        }
    }
}

// NR: regions evaluated per pixel (>= the sample's count; extra regions are
// zero-weight padding).  V: pixels per lane (16 bytes, or 1 for shapes whose
// H*W is not a multiple of the vector).  Each workgroup covers blockDim * vpt
// vectors of one sample (vpt per lane, blockDim apart); its wavefronts do not
// synchronise with each other.  When every sample is active the workgroup
// index maps to the sample directly (the processing order is immaterial), so
// the first latent loads wait on no other load.  With a device-built plan the
// grid covers every sample (inactive ones exit at once) and one more
// workgroup, the last, builds the step's full plan alongside the streaming.
template <typename T, int V, int NR, bool INP, bool HEUN, typename TN = DefaultTune>
__global__ __launch_bounds__(256) void guided_step_kernel(const StepParams p) {
    __shared__ union {
        float coef[4][(TN::STATS ? 3 : 2) * kSet];  // one slice per wavefront
        int plan[kPlanLds];                    // the plan workgroup's counters
    } sh;
    if ((int)blockIdx.x == p.plan_block) {
        plan_workgroup(p, sh.plan, kPlanLds);
        return;
    }
    float* coef = sh.coef[threadIdx.x >> 6];
    // Continuous batching puts join_front groups of workgroups first, each
    // taking a slot whose request joins now (the plan lists them).
    int jb = (int)blockIdx.x;
    bool front = false;
    if constexpr (TN::QUEUE) {
        const int nf = p.join_front * p.tiles;
        if (jb < nf) {
            const int fslot = p.join_in[jb / p.tiles];
            if (fslot < 0 || fslot >= p.n) return;
            front = true;
            jb = fslot * p.tiles + (jb - (jb / p.tiles) * p.tiles);
        } else {
            jb -= nf;
        }
    }
    const int j = jb / p.tiles;
    const int tile = jb - j * p.tiles;
    if (j >= p.n_active) return;
    const int i = p.identity ? j : p.order[j];
    if (i < 0 || i >= p.n) return;
    const int C = p.C;
    const int vi0 = tile * (int)blockDim.x * p.vpt + (int)threadIdx.x;
    const bool lane_ok = vi0 < p.nvec;

    // The workgroup's channel walk starts at channel 7*blockIdx mod C, so the
    // workgroups in flight spread their requests over the channel planes
    // instead of all reading one plane's rows at a time.  (Workgroup b runs on
    // XCD b mod 8; the multiplier sets which planes the XCDs stream together:
    // on the 16-channel large workload 7 and 9 measured fastest, 5 and 3 0.6 us
    // slower per launch, 1 and 15 1.2-2.5 us slower.)
    const int rot = (int)((7u * blockIdx.x) % (unsigned)C);
    Stage<T, V, TN::U, INP> a, b;
    const int64_t p0 = (int64_t)vi0 * V;
    const T* xs0 = static_cast<const T*>(p.x) + (int64_t)i * C * p.HW + p0;

    // Continuous batching: the slot's record names its request, whose tables
    // the step reads, and says whether the request joins now.  Without
    // inpainting the slot's first stages are requested before the record is
    // consulted (they are in bounds whatever it says, and unused when the
    // request joins).
    int ri = i;
    bool join = false;
    float4 qrec;
    if constexpr (TN::QUEUE) {
        qrec = reinterpret_cast<const float4*>(p.record_in)[i];
        if constexpr (!INP) {
            if (lane_ok && !front) {
                load_stage<T, V, TN, INP>(a, xs0, nullptr, 0, rot, C, p.HW);
                if (TN::U < C) load_stage<T, V, TN, INP>(b, xs0, nullptr, TN::U, rot, C, p.HW);
            }
        }
        const uint32_t fl = __float_as_uint(qrec.w);
        if (!(fl & 1u)) return;
        if (((fl & 128u) != 0) != front) return;  // a front join: left to (or taken by) the front groups
        ri = (int)(fl >> 8);
        join = (fl & 64u) != 0;
    }

    // Channel k's means (lane k), the region tables and the first two stages
    // of the latent's walk, all requested before anything waits: every region slot below NR
    // is read (the slot index clamped to the table's R), and the sample's
    // count only selects among them afterwards.
    const int k = (int)threadIdx.x & 63;
    const int kk = k < C ? k : 0;
    const float mu_u = p.mu_uncond[(int64_t)ri * C + kk];
    const float mu_c = p.mu_cond[(int64_t)ri * C + kk];
    int cnt = 0;
    float mu_r[NR > 0 ? NR : 1];
    int4 box[NR > 0 ? NR : 1];
    float str[NR > 0 ? NR : 1];
    if constexpr (NR > 0) {
        cnt = p.region_count[ri];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int64_t slot = (int64_t)ri * p.R + (r < p.R ? r : p.R - 1);
            const int32_t* b = p.region_box + slot * 4;
            box[r] = make_int4(b[0], b[1], b[2], b[3]);
            str[r] = p.region_strength[slot];
            mu_r[r] = p.mu_region[slot * C + kk];
        }
    }
    if (lane_ok && !join && !(TN::QUEUE && !INP)) {
        const T* xo0 = INP ? static_cast<const T*>(p.x_orig) + (int64_t)ri * C * p.HW + p0 : nullptr;
        load_stage<T, V, TN, INP>(a, xs0, xo0, 0, rot, C, p.HW);
        if (TN::U < C) load_stage<T, V, TN, INP>(b, xs0, xo0, TN::U, rot, C, p.HW);
    }
    if constexpr (NR > 0) {
        cnt = cnt < 0 ? 0 : cnt;
        cnt = cnt > p.R ? p.R : cnt;
        cnt = cnt > NR ? NR : cnt;
#pragma unroll
        for (int r = 0; r < NR; ++r) mu_r[r] = r < cnt ? mu_r[r] : 0.0f;
    }
    // The sample's step: from its record when given (one load that waits for
    // nothing else), else derived from its step index.
    StepScalars s;
    float sig, sgn;
    bool keep_u;
    unsigned valid = 0xfu;  // regions taking part in this step
    if (p.record_in) {
        float4 r;
        if constexpr (TN::QUEUE) r = qrec;
        else r = reinterpret_cast<const float4*>(p.record_in)[i];
        const uint32_t fl = __float_as_uint(r.w);
        if (!(fl & 1u)) return;
        sig = r.x;
        sgn = r.y;
        s.w = r.z;
        keep_u = (fl & 2u) != 0;
        valid = (fl >> 2) & 0xfu;
    } else {
        const int t = p.step_idx[i];
        if (t < 0 || t >= p.t_end) return;
        sig = p.sigmas[t];
        sgn = p.sigmas[t + 1];
        if (p.dplan) {
            int b;
            dplan_sample(p, i, t, b, s.w, keep_u, &valid);
        } else {
            s.w = p.scale[i];
            keep_u = p.uncond_row[i] >= 0;
            if (NR > 0 && p.region_range) valid = region_mask(p, i, t);
        }
    }
    SampleRegions<NR> sr;
    sr.cnt = cnt;
    if constexpr (NR > 0) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            if (r < cnt) {
                sr.rd[r].y0 = box[r].x;
                sr.rd[r].h = box[r].y - box[r].x;
                sr.rd[r].x0 = box[r].z;
                sr.rd[r].w = box[r].w - box[r].z;
                sr.rd[r].strength = ((valid >> r) & 1u) ? str[r] : 0.0f;
            } else {
                sr.rd[r].y0 = sr.rd[r].x0 = 0;
                sr.rd[r].h = sr.rd[r].w = 0;
                sr.rd[r].strength = 0.0f;
            }
        }
    }
    if (NR > 0 && cnt > 0)
        run_sample<T, V, TN, NR, NR, INP, HEUN>(a, b, lane_ok, sr, p, s, coef, i, ri, join, vi0, rot, keep_u, sig, sgn,
                                                mu_u, mu_c, mu_r);
    else
        run_sample<T, V, TN, NR, 0, INP, HEUN>(a, b, lane_ok, sr, p, s, coef, i, ri, join, vi0, rot, keep_u, sig, sgn,
                                               mu_u, mu_c, mu_r);
}

// Pipeline shape of a kernel variant: channels per stage (4 puts more latent
// loads in flight per lane than 2) and whether a lane's next pass has its head
// stage requested during the current pass (only lanes with more than one
// vector have a next pass).  Both pay only where a lane waits on HBM with few
// bytes in flight: on the nontemporal (streaming) variants.  There, from the
// register counts of every variant under this toolchain: fp32 takes
// (4, prefetch) at 4 waves per SIMD, except 4 regions under Heun (2, prefetch);
// bf16 takes (4, prefetch) up to 2 regions (3 or 4 waves per SIMD), and width 2
// with 3 or 4 regions (prefetch except 3 regions under Heun, where it would
// cost a wave).  Measured on the large 2-region bf16 workload (one vector per
// lane, several rounds of workgroups): (4, prefetch) 50.2 us per launch at 3
// waves per SIMD against 50.9 at (2, prefetch) and 51.0 at (4, none), both at
// 4.  Inpaint variants stay at (2, none): width 4 reaches the 256-register
// ceiling, and the prefetch, which costs them 8 registers, has no measurement
// in their favour.  The cache-keep variants, whose batch is partly held by the
// last-level cache, keep (2, none).  Only the speed depends on the choice:
// every variant computes the same values in the same order.
template <typename T, int NR, bool INP, bool HEUN, bool NT>
constexpr int stage_width() {
    if (!NT || INP) return 2;
    if (sizeof(T) == 4) return (NR == 4 && HEUN) ? 2 : 4;
    return NR <= 2 ? 4 : 2;
}
template <typename T, int NR, bool INP, bool HEUN, bool NT>
constexpr bool stage_prefetch() {
    if (!NT || INP) return false;
    return sizeof(T) == 4 || !(NR == 3 && HEUN);
}

template <typename T, int NR, bool INP, bool HEUN, bool NT>
using StageTune = Tune<stage_width<T, NR, INP, HEUN, NT>(), NT, stage_prefetch<T, NR, INP, HEUN, NT>()>;

// One variant at its pipeline shape.  The table's shape needs channels to
// overlap: a latent of at most 4 channels, or with fewer than two of the
// table's stages per pass, runs at (2, none).  On the 4-channel workloads
// (f32 and bf16, Euler and Heun, with and without inpaint) that shape measured
// at least as fast as any other (Heun bf16: 5.68 us per launch against 5.77
// at (2, prefetch) and 6.05 at (4, prefetch)); the 16-channel large workload
// gains from the table.  When C is a multiple of two stages every stage is
// full, and the variant without per-channel bounds checks is taken (its loads
// and stores are then not each behind a branch): 46.4 us per launch on the
// large workload against 47.8 with the checks.
template <typename T, int V, int NR, bool INP, bool HEUN, bool NT>
void launch_variant(const StepParams& p, dim3 grid, dim3 blk, hipStream_t st) {
    typedef StageTune<T, NR, INP, HEUN, NT> Wide;
    typedef Tune<Wide::U, NT, Wide::PF, true> WideFull;
    typedef Tune<2, NT, false> Narrow;
    if constexpr (!NT && V > 1) {  // the statistics: ordinary loads and stores, two-channel stages
        if (p.stats_part) {
            hipLaunchKernelGGL((guided_step_kernel<T, V, NR, INP, HEUN, StatsTune>), grid, blk, 0, st, p);
            return;
        }
    }
    if (p.C > 4 && p.C % (2 * Wide::U) == 0)
        hipLaunchKernelGGL((guided_step_kernel<T, V, NR, INP, HEUN, WideFull>), grid, blk, 0, st, p);
    else if (p.C > 4 && p.C >= 2 * Wide::U)
        hipLaunchKernelGGL((guided_step_kernel<T, V, NR, INP, HEUN, Wide>), grid, blk, 0, st, p);
    else
        hipLaunchKernelGGL((guided_step_kernel<T, V, NR, INP, HEUN, Narrow>), grid, blk, 0, st, p);
}

// Continuous batching: the streaming variants whose slots hold requests (the
// full-stage shape where C allows it, else two-channel stages).
template <typename T, int V, int NR, bool INP, bool HEUN>
void launch_queue_variant(const StepParams& p, dim3 grid, dim3 blk, hipStream_t st) {
    typedef StageTune<T, NR, INP, HEUN, true> Wide;
    typedef Tune<Wide::U, true, Wide::PF, true> WideFull;
    typedef Tune<2, true, false> Narrow;
    if (p.C > 4 && p.C % (2 * Wide::U) == 0)
        hipLaunchKernelGGL((guided_step_kernel<T, V, NR, INP, HEUN, QueueOf<WideFull>>), grid, blk, 0, st, p);
    else
        hipLaunchKernelGGL((guided_step_kernel<T, V, NR, INP, HEUN, QueueOf<Narrow>>), grid, blk, 0, st, p);
}

template <typename T, int NR>
hipError_t launch_queue_nr(const StepParams& p, bool heun, bool inp, int block, hipStream_t st) {
    constexpr int V = VecWidth<T>::value;
    const dim3 grid((unsigned)((int64_t)(p.join_front + p.n_active) * p.tiles + (p.plan_block >= 0 ? 1 : 0))),
        blk((unsigned)block);
    if (heun) {
        if (inp) launch_queue_variant<T, V, NR, true, true>(p, grid, blk, st);
        else launch_queue_variant<T, V, NR, false, true>(p, grid, blk, st);
    } else {
        if (inp) launch_queue_variant<T, V, NR, true, false>(p, grid, blk, st);
        else launch_queue_variant<T, V, NR, false, false>(p, grid, blk, st);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_step_queue(const StepParams& p, bool heun, bool inp, int block, hipStream_t st) {
    if (p.n_active == 0) return hipSuccess;
    switch (p.R) {
        case 0: return launch_queue_nr<T, 0>(p, heun, inp, block, st);
        case 1: return launch_queue_nr<T, 1>(p, heun, inp, block, st);
        case 2: return launch_queue_nr<T, 2>(p, heun, inp, block, st);
        case 3: return launch_queue_nr<T, 3>(p, heun, inp, block, st);
        default: return launch_queue_nr<T, 4>(p, heun, inp, block, st);
    }
}

template <typename T, int V, int NR, typename TN = DefaultTune>
hipError_t launch_nr(const StepParams& p, bool heun, bool inp, int block, hipStream_t st) {
    const dim3 grid((unsigned)((int64_t)p.n_active * p.tiles + (p.plan_block >= 0 ? 1 : 0))),
        blk((unsigned)block);
    if (heun) {
        if (inp) launch_variant<T, V, NR, true, true, TN::NT>(p, grid, blk, st);
        else launch_variant<T, V, NR, false, true, TN::NT>(p, grid, blk, st);
    } else {
        if (inp) launch_variant<T, V, NR, true, false, TN::NT>(p, grid, blk, st);
        else launch_variant<T, V, NR, false, false, TN::NT>(p, grid, blk, st);
    }
    return hipGetLastError();
}

// Launch of one storage type and tuning.  The scalar path (shapes the 128-bit
// path cannot take) is instantiated only where SCALAR is set.
template <typename T, typename TN, bool SCALAR>
hipError_t launch_step(const StepParams& p, bool vec, bool heun, bool inp, int block, hipStream_t st) {
    if (p.n_active == 0) return hipSuccess;
    constexpr int VV = VecWidth<T>::value;
    if (!vec) {
        if constexpr (SCALAR) {
            // regions run with the maximum count (extra regions are zero-weight padding)
            if (p.R > 0) return launch_nr<T, 1, BCG_MAX_REGIONS, TN>(p, heun, inp, block, st);
            return launch_nr<T, 1, 0, TN>(p, heun, inp, block, st);
        } else {
            return hipErrorInvalidValue;
        }
    }
    switch (p.R) {
        case 0: return launch_nr<T, VV, 0, TN>(p, heun, inp, block, st);
        case 1: return launch_nr<T, VV, 1, TN>(p, heun, inp, block, st);
        case 2: return launch_nr<T, VV, 2, TN>(p, heun, inp, block, st);
        case 3: return launch_nr<T, VV, 3, TN>(p, heun, inp, block, st);
        default: return launch_nr<T, VV, 4, TN>(p, heun, inp, block, st);
    }
}

}  // namespace bcg
