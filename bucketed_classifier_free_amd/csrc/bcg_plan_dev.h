// The bucket plan of one step built on the GPU (SGLang BCG write-up, section
// 2: bucket assignment; section 3: BucketPlan, per-bucket offsets and the
// [uncond | cond] layout; ComfyUI guide "12 · Samplers, schedulers and CFG",
// "the cfg = 1 optimisation").  Same definition as the host plan build:
//   bucket = min(floor(t * nb / steps), nb - 1)       exact integer arithmetic
//   scale  = override if given and not NaN, else bucket_cfg[bucket] (or the
//            within-bucket interpolation towards bucket_cfg_end[bucket])
//   uncond kept unless scale == 1 and the sample's conds cover the frame
//   order  = active samples stably sorted by (bucket, sample)
// Included by the .hip translation units only.
#pragma once

#include "bcg_device.h"

namespace bcg {

// Regions of sample i taking part in step t (ComfyUI guide, "calc_cond_batch()":
// the current timestep must be valid for a cond): start <= t/steps < end in
// double; every region without ranges.
__device__ __forceinline__ unsigned region_mask(const StepParams& p, int i, int t) {
    int k = p.region_count ? p.region_count[i] : p.R;
    k = k < 0 ? 0 : (k > p.R ? p.R : k);
    if (!p.region_range) return (1u << k) - 1u;
    const double prog = double(t) / double(p.range_steps);
    unsigned v = 0;
    for (int r = 0; r < k; ++r) {
        const double* rg = p.region_range + ((int64_t)i * p.R + r) * 2;
        if (rg[0] <= prog && prog < rg[1]) v |= 1u << r;
    }
    return v;
}

// Bucket, scale and uncond decision of sample i at an active step t (i
// indexes the per-sample tables: the slot's request under continuous batching).
// t * nb < 2^20 * 2^10 fits 32 bits (both limits are checked on the host).
__device__ __forceinline__ void dplan_sample(const StepParams& p, int i, int t, int& b, float& w,
                                             bool& need_u, unsigned* valid = nullptr) {
    b = (int)(((uint32_t)t * (uint32_t)p.nb) / (uint32_t)p.steps);
    b = b < p.nb - 1 ? b : p.nb - 1;
    w = p.bucket_cfg[b];
    if (p.bucket_cfg_end) {  // within-bucket interpolation, in double as on the host
        const double f = double((int)((uint32_t)t * (uint32_t)p.nb - (uint32_t)b * (uint32_t)p.steps)) /
                         double(p.steps);
        const double lo = w, hi = p.bucket_cfg_end[b];
        w = float(lo + (hi - lo) * f);
    }
    if (p.cfg_override) {
        const float o = p.cfg_override[i];
        if (o == o) w = o;  // NaN = no override
    }
    bool cov = p.covered ? p.covered[i] != 0 : true;
    if (p.region_range) {
        const unsigned v = region_mask(p, i, t);
        cov = ((p.covered_sets[i] >> v) & 1u) != 0;
        if (valid) *valid = v;
    } else if (valid) {
        *valid = 0xfu;
    }
    need_u = !(w == 1.0f && cov);
}

// The sample record of request r at step t of its trajectory (0 <= t < steps):
// sigma, sigma', scale, flags = active | keep-uncond << 1 | valid regions << 2
// | joins << 6 | r << 8 (the request under continuous batching).
__device__ __forceinline__ float4 step_record(const StepParams& p, int r, int t, bool join) {
    int b;
    float w;
    bool need;
    unsigned v;
    dplan_sample(p, r, t, b, w, need, &v);
    uint32_t fl = (need ? 3u : 1u) | ((v & 0xfu) << 2);
    if (p.queue_len > 0) fl |= (join ? 64u : 0u) | ((uint32_t)r << 8);
    return float4{p.sigmas[t], p.sigmas[t + 1], w, __uint_as_float(fl)};
}

// Continuous batching: the slots that take a new request at the next step
// (empty, or holding a request that takes its last step now) get the next
// queued requests, in slot order, by one wavefront (`lane` 0..63): a ballot
// per 64 slots and the popcount of the lanes below give each candidate its
// place in the queue; the next 64 slots' indices are requested while the
// current ones are placed.  Each refilled slot's next step index is 0, its
// record joins; a slot left without a request gets index -1 and an all-zero
// record.
__device__ __forceinline__ void refill_slots(const StepParams& p, int lane) {
    const int n = p.n;
    const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int Q = p.queue_len;
    const int nxt = *p.queue_in;
    int run = 0;
    int t_n = lane < n ? p.step_idx[lane] : 0, r_n = lane < n ? p.slot_req[lane] : 0;
    for (int s0 = 0; s0 < n; s0 += 64) {
        const int s = s0 + lane;
        const int t = t_n, rq = r_n;
        if (s + 64 < n) {
            t_n = p.step_idx[s + 64];
            r_n = p.slot_req[s + 64];
        }
        const bool cand = s < n && !(rq >= 0 && t >= 0 && t + 1 < p.steps);
        const unsigned long long bal = __ballot(cand);
        if (cand) {
            const int rank = run + __popcll(bal & below);  // this step's joins, in slot order
            const int q = nxt + rank;
            const int r = p.queue_ring ? q % Q : (q < Q ? q : -1);
            p.step_out[s] = r >= 0 ? 0 : -1;
            p.slot_req_out[s] = r;
            float4 rec = float4{0.0f, 0.0f, 0.0f, 0.0f};
            if (r >= 0) {
                rec = step_record(p, r, 0, true);
                if (rank < p.join_front) {  // joins the front workgroups take
                    p.join_out[rank] = s;
                    rec.w = __uint_as_float(__float_as_uint(rec.w) | 128u);
                }
            }
            reinterpret_cast<float4*>(p.record_out)[s] = rec;
        }
        run += __popcll(bal);
    }
    const int joins = p.queue_ring ? run : min(run, max(Q - nxt, 0));
    for (int q = joins + lane; q < p.join_front; q += 64) p.join_out[q] = -1;
    if (lane == 0) *p.queue_out = p.queue_ring ? (nxt + run) % Q : min(nxt + run, Q);
}

// The step index after this step: t + 1, modulo steps once non-negative
// when wrapping (a finished slot restarts at step 0).
__device__ __forceinline__ int dplan_next(const StepParams& p, int t) {
    if (t == 0x7fffffff) return t;
    const int nt = t + 1;
    return (p.wrap && nt >= 0) ? nt % p.steps : nt;
}

// The full plan and the step advance, by one workgroup (blockDim >= 64,
// a multiple of 64).  `sh` holds lds_ints >= 2 * nb ints of LDS; when
// n <= lds_ints - 2 * nb it also keeps each sample's bucket and flags from
// pass 1 for pass 3 (otherwise pass 3 derives them again).
//   pass 1 (all lanes): per sample, bucket/scale (or the inactive markers)
//     and the step advance (with the next step's sample record); per-bucket counts of the cond and uncond halves
//     by LDS atomics;
//   pass 2 (wavefront 0): exclusive prefix sums of the counts, 64 buckets at
//     a time, which become the running write cursors of each bucket;
//   pass 3 (wavefront 0): samples in index order, 64 at a time; each lane
//     finds the lanes of its own bucket with one ballot per bit of the bucket
//     id, and the lanes of one bucket take consecutive slots in lane order
//     (popcount of the lanes below), so the order within a bucket is the
//     sample order; the bucket's lowest lane then advances its cursors.
__device__ __forceinline__ void plan_workgroup(const StepParams& p, int* sh, int lds_ints) {
    const int n = p.n, nb = p.nb;
    const int tid = (int)threadIdx.x, T = (int)blockDim.x;
    const bool full = p.plan_bucket_id != nullptr;
    int* cnt = sh;
    int* ucnt = sh + nb;
    int* info = sh + 2 * nb;  // bucket | need_u << 16 | active << 17
    const bool keep = n <= lds_ints - 2 * nb;
    if (full)
        for (int b = tid; b < nb; b += T) {
            cnt[b] = 0;
            ucnt[b] = 0;
        }
    __syncthreads();
    const bool queue = p.queue_len > 0;
    for (int i = tid; i < n; i += T) {
        const int t = p.step_idx[i];
        const int ri = queue ? p.slot_req[i] : i;  // the sample's tables
        if (queue) {  // a slot that keeps its request: its next step and record
            if (ri >= 0 && t >= 0 && t + 1 < p.steps) {
                p.step_out[i] = t + 1;
                p.slot_req_out[i] = ri;
                reinterpret_cast<float4*>(p.record_out)[i] = step_record(p, ri, t + 1, false);
            }
        } else if (p.step_out) {
            p.step_out[i] = dplan_next(p, t);
        }
        if (p.record_out && !queue) {  // the next step's record (all zero when inactive)
            const int nt = dplan_next(p, t);
            float4 r = {0.0f, 0.0f, 0.0f, 0.0f};
            if (nt >= 0 && nt < p.steps && nt + 1 < p.num_sigmas) {
                int b2;
                float w2;
                bool need2;
                unsigned v2;
                dplan_sample(p, i, nt, b2, w2, need2, &v2);
                r = float4{p.sigmas[nt], p.sigmas[nt + 1], w2,
                           __uint_as_float((need2 ? 3u : 1u) | ((v2 & 0xfu) << 2))};
            }
            reinterpret_cast<float4*>(p.record_out)[i] = r;
        }
        if (!full) continue;
        int v = 0;
        if (ri >= 0 && t >= 0 && t < p.steps) {
            int b;
            float w;
            bool need_u;
            dplan_sample(p, ri, t, b, w, need_u);
            p.plan_bucket_id[i] = b;
            p.plan_scale[i] = w;
            atomicAdd(&cnt[b], 1);
            if (need_u) atomicAdd(&ucnt[b], 1);
            v = b | (need_u ? 1 << 16 : 0) | 1 << 17;
        } else {
            p.plan_bucket_id[i] = -1;
            p.plan_scale[i] = 0.0f;
            p.plan_uncond_row[i] = -1;
            p.plan_cond_row[i] = -1;
        }
        if (keep) info[i] = v;
    }
    if (!full && !queue) return;
    __syncthreads();
    // the refills (of slots no line above writes): by wavefront 1 while
    // wavefront 0 orders, or by wavefront 0 afterwards in a 64-lane workgroup
    const bool refill_w1 = queue && blockDim.x >= 128;
    if (refill_w1 && tid >= 64 && tid < 128) {
        refill_slots(p, tid - 64);
        return;
    }
    if (tid >= 64) return;
    if (full) {

        int run = 0, urun = 0;
        for (int b0 = 0; b0 < nb; b0 += 64) {
            const int b = b0 + tid;
            const int c = b < nb ? cnt[b] : 0;
            const int u = b < nb ? ucnt[b] : 0;
            int ic = c, iu = u;  // inclusive scans over the 64 lanes
    #pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int xc = __shfl_up(ic, o, 64);
                const int xu = __shfl_up(iu, o, 64);
                if (tid >= o) {
                    ic += xc;
                    iu += xu;
                }
            }
            if (b < nb) {
                p.plan_bucket_count[b] = c;
                p.plan_bucket_offset[b] = run + ic - c;
                p.plan_uncond_offset[b] = urun + iu - u;
                cnt[b] = run + ic - c;
                ucnt[b] = urun + iu - u;
            }
            run += __shfl(ic, 63, 64);
            urun += __shfl(iu, 63, 64);
        }
        if (tid == 0) {
            p.plan_bucket_offset[nb] = run;
            p.plan_uncond_offset[nb] = urun;
            p.plan_totals[0] = run;
            p.plan_totals[1] = urun;
        }

        const int m = urun;  // rows of the uncond half
        const unsigned long long below = tid == 0 ? 0ull : (~0ull >> (64 - tid));
        const int kbits = nb > 1 ? 32 - __clz(nb - 1) : 0;  // bits of a bucket id
        for (int i0 = 0; i0 < n; i0 += 64) {
            const int i = i0 + tid;
            bool act = false, need_u = false;
            int b = 0;
            if (i < n) {
                if (keep) {
                    const int v = info[i];
                    act = (v >> 17) & 1;
                    need_u = (v >> 16) & 1;
                    b = v & 0xffff;
                } else {
                    const int t = p.step_idx[i];
                    const int ri = queue ? p.slot_req[i] : i;
                    act = ri >= 0 && t >= 0 && t < p.steps;
                    float w;
                    if (act) dplan_sample(p, ri, t, b, w, need_u);
                }
            }
            // Lanes holding the same bucket, one ballot per bit of the id.
            unsigned long long same = __ballot(act);
            for (int k = 0; k < kbits; ++k) {
                const bool bit = (b >> k) & 1;
                const unsigned long long ones = __ballot(act && bit);
                same &= bit ? ones : ~ones;
            }
            const unsigned long long needs = same & __ballot(act && need_u);
            if (act) {
                const int cbase = cnt[b], ubase = ucnt[b];
                const int pos = cbase + __popcll(same & below);
                p.plan_order[pos] = i;
                p.plan_cond_row[i] = m + pos;
                p.plan_uncond_row[i] = need_u ? ubase + __popcll(needs & below) : -1;
                if ((same & below) == 0) {  // the bucket's first lane advances its cursors
                    cnt[b] = cbase + __popcll(same);
                    ucnt[b] = ubase + __popcll(needs);
                }
            }
        }
        for (int j = run + tid; j < n; j += 64) p.plan_order[j] = -1;
    }
    if (queue && !refill_w1) refill_slots(p, tid);
}

}  // namespace bcg
