// Host half of libbcg: error state, sigma schedule, bucket table and the
// per-step bucket plan.  Pure C++ (no HIP calls), O(n) per step.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "bcg_common.h"

namespace bcg {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = '\0'; }

}  // namespace bcg

using bcg::fail;

extern "C" const char* bcg_last_error(void) { return bcg::g_err; }

extern "C" int bcg_abi_version(void) { return 9; }

// "12 · Samplers, schedulers and CFG", sections "sigma sequence" and
// "denoise below 1": the schedule runs from high to low noise and ends at 0;
// for denoise < 1 a longer base schedule is built and its tail kept.  The base
// length is the smallest N with N*denoise >= steps, computed as ceil(steps /
// denoise) in double.
extern "C" int sigma_schedule(int kind, double sigma_max, double sigma_min, int steps,
                              double denoise, float* sigmas, int* base_steps) {
    bcg::clear_error();
    if (kind != BCG_SCHED_LOGLINEAR) return fail(BCG_EINVAL, "sigma_schedule: unknown kind %d", kind);
    if (!(std::isfinite(sigma_max) && std::isfinite(sigma_min) && sigma_min > 0.0 &&
          sigma_max > sigma_min))
        return fail(BCG_EINVAL, "sigma_schedule: need sigma_max > sigma_min > 0 (got %g, %g)",
                    sigma_max, sigma_min);
    if (steps < 1 || steps > 100000) return fail(BCG_EINVAL, "sigma_schedule: steps %d out of range", steps);
    if (!(denoise > 0.0 && denoise <= 1.0))
        return fail(BCG_EINVAL, "sigma_schedule: denoise %g not in (0, 1]", denoise);
    if (!sigmas) return fail(BCG_EINVAL, "sigma_schedule: sigmas is NULL");
    double nb = denoise >= 1.0 ? double(steps) : std::ceil(double(steps) / denoise);
    if (nb > 1e7) return fail(BCG_EINVAL, "sigma_schedule: base schedule too long (%g)", nb);
    const int N = int(nb);
    const double la = std::log(sigma_max), lb = std::log(sigma_min);
    // Point i of the base schedule (i in [0, N]); index N is the terminal 0.
    auto point = [&](int i) -> double {
        if (i == N) return 0.0;
        if (i == 0) return sigma_max;
        if (i == N - 1) return sigma_min;
        return std::exp(la + (lb - la) * (double(i) / double(N - 1)));
    };
    for (int k = 0; k <= steps; ++k) sigmas[k] = float(point(N - steps + k));
    if (base_steps) *base_steps = N;
    return BCG_OK;
}

// SGLang BCG write-up, section 2 (a continuous curve cut into buckets,
// constant per bucket) and section 5 (linear decay and front-high shapes).
namespace {

int check_curve(int curve, double p0, double p1, double p2, int num_buckets, const char* who) {
    if (num_buckets < 1 || num_buckets > BCG_MAX_BUCKETS)
        return fail(BCG_EINVAL, "%s: num_buckets %d out of range", who, num_buckets);
    if (!(std::isfinite(p0) && std::isfinite(p1) && std::isfinite(p2)))
        return fail(BCG_EINVAL, "%s: non-finite curve parameter", who);
    if (curve < BCG_CURVE_CONST || curve > BCG_CURVE_MID_PEAK)
        return fail(BCG_EINVAL, "%s: unknown curve %d", who, curve);
    if (curve == BCG_CURVE_MID_PEAK && !(p2 > 0.0 && p2 < 1.0))
        return fail(BCG_EINVAL, "%s: mid-peak position %g not in (0, 1)", who, p2);
    return BCG_OK;
}

// [B] section 5's curve shapes at progress u (double).
double curve_at(int curve, double p0, double p1, double p2, double u) {
    if (curve == BCG_CURVE_LINEAR) return p0 + (p1 - p0) * u;
    if (curve == BCG_CURVE_FRONT_HIGH) return u < p2 ? p0 : p1;
    if (curve == BCG_CURVE_MID_PEAK) return p0 + (p1 - p0) * (u <= p2 ? u / p2 : (1.0 - u) / (1.0 - p2));
    return p0;
}

}  // namespace

extern "C" int bucket_table(int curve, double p0, double p1, double p2, int num_buckets,
                            float* table) {
    bcg::clear_error();
    const int rc = check_curve(curve, p0, p1, p2, num_buckets, "bucket_table");
    if (rc) return rc;
    if (!table) return fail(BCG_EINVAL, "bucket_table: table is NULL");
    for (int b = 0; b < num_buckets; ++b) {
        const double u = num_buckets == 1 ? 0.0 : double(b) / double(num_buckets - 1);
        table[b] = float(curve_at(curve, p0, p1, p2, u));
    }
    return BCG_OK;
}

extern "C" int bucket_bounds(int curve, double p0, double p1, double p2, int num_buckets,
                             float* lo, float* hi) {
    bcg::clear_error();
    const int rc = check_curve(curve, p0, p1, p2, num_buckets, "bucket_bounds");
    if (rc) return rc;
    if (!lo || !hi) return fail(BCG_EINVAL, "bucket_bounds: NULL output");
    for (int b = 0; b < num_buckets; ++b) {
        lo[b] = float(curve_at(curve, p0, p1, p2, double(b) / double(num_buckets)));
        hi[b] = float(curve_at(curve, p0, p1, p2, double(b + 1) / double(num_buckets)));
    }
    return BCG_OK;
}

extern "C" int sigma_crop(const float* sigmas, int num_sigmas, int start_step, int last_step,
                          int force_full_denoise, float* out, int* count) {
    bcg::clear_error();
    if (!sigmas || !out || !count) return fail(BCG_EINVAL, "sigma_crop: NULL argument");
    if (num_sigmas < 1) return fail(BCG_EINVAL, "sigma_crop: num_sigmas %d < 1", num_sigmas);
    const int end = num_sigmas - 1;
    const int last = (last_step < 0 || last_step > end) ? end : last_step;
    if (start_step < 0 || start_step > last)
        return fail(BCG_EINVAL, "sigma_crop: start_step %d not in [0, %d]", start_step, last);
    const int m = last - start_step + 1;
    for (int k = 0; k < m; ++k) out[k] = sigmas[start_step + k];
    if (force_full_denoise && out[m - 1] != 0.0f) out[m - 1] = 0.0f;
    *count = m;
    return BCG_OK;
}

namespace {

// The integer nearest to the exact product f * n, a tie going to the larger
// integer.  f is a finite double with |f| <= 1e6 (checked by the caller) and
// 0 < n < 2^31.  f = M * 2^-k with M the 53-bit integer significand, so
// f * n = P * 2^-k with P = M * n exact in 128 bits, and the nearest integer
// with ties upward is floor((P + 2^(k-1)) / 2^k), an arithmetic shift.
long long nearest_up(double f, int n) {
    if (f == 0.0) return 0;
    int e = 0;
    const double m = std::frexp(f, &e);                 // f = m * 2^e, 0.5 <= |m| < 1
    const long long M = (long long)std::ldexp(m, 53);   // exact: |M| < 2^53
    const __int128 P = (__int128)M * n;                 // exact: |P| < 2^84
    const int k = 53 - e;                               // f * n = P * 2^-k
    if (k <= 0) return (long long)(P << -k);            // an integer already (|f*n| <= 1e6 * 2^31)
    if (k > 100) return 0;                              // |f * n| < 2^84 * 2^-101 < 1/2
    return (long long)((P + ((__int128)1 << (k - 1))) >> k);
}

// "calc_cond_batch()": area fractions become latent slices.  Each coordinate
// is the integer nearest to the exact product of its fraction and the extent
// (ties to the larger integer); the side is clamped so the box keeps at least
// one pixel and the offset so the box stays inside.
void area_slice(const double* f, int H, int W, int32_t* box) {
    const double fy = f[0], fx = f[1], fh = f[2], fw = f[3];
    long long h = std::min<long long>(std::max<long long>(nearest_up(fh, H), 1), H);
    long long w = std::min<long long>(std::max<long long>(nearest_up(fw, W), 1), W);
    long long y0 = std::min<long long>(std::max<long long>(nearest_up(fy, H), 0), H - h);
    long long x0 = std::min<long long>(std::max<long long>(nearest_up(fx, W), 0), W - w);
    box[0] = int32_t(y0);
    box[1] = int32_t(y0 + h);
    box[2] = int32_t(x0);
    box[3] = int32_t(x0 + w);
}

// Sorted distinct values of a small array, in place; returns the count.
int sort_unique(int* v, int m) {
    std::sort(v, v + m);
    return int(std::unique(v, v + m) - v);
}

// True when the union of the boxes covers [0,H) x [0,W).  Coordinate
// compression over the box edges: every elementary cell is tested.
bool covers(const int32_t (*boxes)[4], int k, int H, int W) {
    if (k == 0) return false;
    int ys[2 * BCG_MAX_REGIONS + 2] = {0, H}, xs[2 * BCG_MAX_REGIONS + 2] = {0, W};
    int ny = 2, nx = 2;
    for (int r = 0; r < k; ++r) {
        ys[ny++] = boxes[r][0]; ys[ny++] = boxes[r][1];
        xs[nx++] = boxes[r][2]; xs[nx++] = boxes[r][3];
    }
    ny = sort_unique(ys, ny);
    nx = sort_unique(xs, nx);
    for (int a = 0; a + 1 < ny; ++a)
        for (int b = 0; b + 1 < nx; ++b) {
            const int cy = ys[a], cx = xs[b];  // cell [ys[a], ys[a+1]) x [xs[b], xs[b+1])
            if (cy < 0 || cy >= H || cx < 0 || cx >= W) continue;
            bool hit = false;
            for (int r = 0; r < k && !hit; ++r)
                hit = boxes[r][0] <= cy && cy < boxes[r][1] && boxes[r][2] <= cx && cx < boxes[r][3];
            if (!hit) return false;
        }
    return true;
}

}  // namespace

// SGLang BCG write-up, section 2 (assign_bucket), section 3 (BucketPlan with
// per-sample (bucket, scale) and per-bucket offsets; the [uncond | cond]
// layout), section 4 stage 3 (the plan is built in the scheduler, before the
// launch); "12 · Samplers...", "the cfg = 1 optimisation".
extern "C" int bcg_plan_build(const bcg_plan_in* in, bcg_plan_out* out) {
    bcg::clear_error();
    if (!in || !out) return fail(BCG_EINVAL, "bcg_plan_build: NULL argument");
    const int n = in->n, steps = in->steps, nb = in->num_buckets, R = in->max_regions;
    if (n < 0 || n > (1 << 24)) return fail(BCG_ESHAPE, "bcg_plan_build: n %d out of range", n);
    if (steps < 1) return fail(BCG_EINVAL, "bcg_plan_build: steps %d < 1", steps);
    if (nb < 1 || nb > BCG_MAX_BUCKETS) return fail(BCG_EINVAL, "bcg_plan_build: num_buckets %d out of range", nb);
    if (R < 0 || R > BCG_MAX_REGIONS) return fail(BCG_EINVAL, "bcg_plan_build: max_regions %d out of range", R);
    if (in->C < 1 || in->H < 1 || in->W < 1) return fail(BCG_ESHAPE, "bcg_plan_build: bad C/H/W");
    if (!in->bucket_cfg || (n > 0 && !in->step_idx))
        return fail(BCG_EINVAL, "bcg_plan_build: bucket_cfg/step_idx is NULL");
    if (!out->bucket_id || !out->scale || !out->uncond_row || !out->cond_row || !out->order ||
        !out->bucket_count || !out->bucket_offset || !out->uncond_offset)
        return fail(BCG_EINVAL, "bcg_plan_build: NULL output array");
    const bool regions = R > 0 && in->region_count && !in->covered && !in->covered_sets;
    if (regions && (!in->region_frac || !in->region_strength))
        return fail(BCG_EINVAL, "bcg_plan_build: region_count given without region_frac/strength");
    const bool ranged = R > 0 && in->region_range;
    if (ranged && !regions && !in->covered_sets)
        return fail(BCG_EINVAL, "bcg_plan_build: validity ranges need the region arrays or covered_sets");
    for (int i = 0; ranged && i < n; ++i)
        for (int q = 0; q < 2 * R; ++q)
            if (std::isnan(in->region_range[size_t(i) * R * 2 + q]))
                return fail(BCG_EINVAL, "bcg_plan_build: region_range of sample %d is NaN", i);
    for (int b = 0; b < nb; ++b) {
        if (!std::isfinite(in->bucket_cfg[b])) return fail(BCG_EINVAL, "bcg_plan_build: bucket_cfg[%d] not finite", b);
        if (in->bucket_cfg_end && !std::isfinite(in->bucket_cfg_end[b]))
            return fail(BCG_EINVAL, "bcg_plan_build: bucket_cfg_end[%d] not finite", b);
    }
    for (int i = 0; i < n; ++i) {
        if (in->cfg_override) {
            const float o = in->cfg_override[i];
            if (std::isinf(o)) return fail(BCG_EINVAL, "bcg_plan_build: cfg_override[%d] infinite", i);
        }
        if (regions) {
            const int k = in->region_count[i];
            if (k < 0 || k > R) return fail(BCG_EINVAL, "bcg_plan_build: region_count[%d] = %d not in [0, %d]", i, k, R);
            for (int r = 0; r < k; ++r) {
                const float s = in->region_strength[i * R + r];
                if (!(s == 0.0f || (s >= 1e-30f && s <= 1e30f)))
                    return fail(BCG_EINVAL, "bcg_plan_build: region_strength[%d][%d] = %g not 0 or in [1e-30, 1e30]", i, r, double(s));
                const double* f = in->region_frac + (size_t(i) * R + r) * 4;
                for (int q = 0; q < 4; ++q)
                    if (!std::isfinite(f[q]) || std::fabs(f[q]) > 1e6)
                        return fail(BCG_EINVAL, "bcg_plan_build: region_frac[%d][%d] not finite", i, r);
            }
        }
    }

    // Region boxes, crop offsets and per-sample coverage (unless given): of all
    // regions, and of every subset of them (bit s of sets: the live regions in
    // mask s cover the frame; a sample without regions is covered by any).
    std::vector<char> covered(size_t(n), 1);
    std::vector<uint16_t> sets(size_t(n), 0xffff);
    if (in->covered)
        for (int i = 0; i < n; ++i) covered[i] = in->covered[i] != 0;
    if (in->covered_sets)
        for (int i = 0; i < n; ++i) {
            sets[i] = in->covered_sets[i];
            const int k = in->region_count ? std::max(0, std::min(in->region_count[i], R)) : R;
            if (!in->covered) covered[i] = (sets[i] >> ((1u << k) - 1u)) & 1u;
        }
    int64_t off = 0;
    for (int i = 0; regions && i < n; ++i) {
        const int k = in->region_count[i];
        int32_t boxes[BCG_MAX_REGIONS][4] = {};
        int32_t live[BCG_MAX_REGIONS][4] = {};
        int nlive = 0;
        for (int r = 0; r < R; ++r) {
            if (r < k) {
                area_slice(in->region_frac + (size_t(i) * R + r) * 4, in->H, in->W, boxes[r]);
                if (in->region_strength[i * R + r] > 0.0f) {
                    std::memcpy(live[nlive++], boxes[r], sizeof boxes[r]);
                }
            }
            if (out->region_box) std::memcpy(out->region_box + (size_t(i) * R + r) * 4, boxes[r], sizeof boxes[r]);
            if (out->region_off) out->region_off[size_t(i) * R + r] = off;
            if (r < k) off += int64_t(in->C) * (boxes[r][1] - boxes[r][0]) * (boxes[r][3] - boxes[r][2]);
        }
        if (k > 0) {
            covered[i] = covers(live, nlive, in->H, in->W);
            uint16_t bits = 0;
            for (unsigned s = 0; s < (1u << R); ++s) {
                int32_t sub[BCG_MAX_REGIONS][4];
                int m = 0;
                for (int r = 0; r < k; ++r)
                    if (((s >> r) & 1u) && in->region_strength[i * R + r] > 0.0f)
                        std::memcpy(sub[m++], boxes[r], sizeof boxes[r]);
                if (covers(sub, m, in->H, in->W)) bits = uint16_t(bits | (1u << s));
            }
            sets[i] = bits;
        }
    }
    if (regions && out->region_off && R > 0) out->region_off[size_t(n) * R] = off;
    if (out->covered_out)
        for (int i = 0; i < n; ++i) out->covered_out[i] = covered[i] ? 1 : 0;
    if (out->covered_sets_out)
        for (int i = 0; i < n; ++i) out->covered_sets_out[i] = sets[i];

    // Buckets, scales and the skip decision.
    std::vector<char> need_u(size_t(n), 0);
    int n_act = 0;
    for (int b = 0; b < nb; ++b) out->bucket_count[b] = 0;
    for (int i = 0; i < n; ++i) {
        const long long t = in->step_idx[i];
        out->uncond_row[i] = -1;
        out->cond_row[i] = -1;
        if (out->region_valid) out->region_valid[i] = 0;
        if (t < 0 || t >= steps) {
            out->bucket_id[i] = -1;
            out->scale[i] = 0.0f;
            continue;
        }
        // Regions taking part in this step ("calc_cond_batch()": valid timestep).
        const int k = in->region_count ? std::max(0, std::min(in->region_count[i], R)) : R;
        unsigned v = k > 0 ? (1u << k) - 1u : 0u;
        if (ranged) {
            const double prog = double(t) / double(steps);
            v = 0;
            for (int r = 0; r < k; ++r) {
                const double* rg = in->region_range + (size_t(i) * R + r) * 2;
                if (rg[0] <= prog && prog < rg[1]) v |= 1u << r;
            }
        }
        if (out->region_valid) out->region_valid[i] = int32_t(v);
        const bool cov = ranged ? ((sets[i] >> v) & 1u) != 0 : covered[i] != 0;
        const int b = int(std::min<long long>(t * nb / steps, nb - 1));
        out->bucket_id[i] = b;
        float w = in->bucket_cfg[b];
        if (in->bucket_cfg_end) {  // within-bucket interpolation
            const double f = double(t * nb - (long long)b * steps) / double(steps);
            const double lo = in->bucket_cfg[b], hi = in->bucket_cfg_end[b];
            w = float(lo + (hi - lo) * f);
        }
        if (in->cfg_override && !std::isnan(in->cfg_override[i])) w = in->cfg_override[i];
        out->scale[i] = w;
        need_u[i] = !(w == 1.0f && cov);
        out->bucket_count[b] += 1;
        ++n_act;
    }
    // Stable counting sort by bucket: order = active samples by (bucket, i).
    std::vector<int> ucount(size_t(nb), 0);
    out->bucket_offset[0] = 0;
    for (int b = 0; b < nb; ++b) out->bucket_offset[b + 1] = out->bucket_offset[b] + out->bucket_count[b];
    for (int i = 0; i < n; ++i)
        if (out->bucket_id[i] >= 0 && need_u[i]) ucount[out->bucket_id[i]] += 1;
    out->uncond_offset[0] = 0;
    for (int b = 0; b < nb; ++b) out->uncond_offset[b + 1] = out->uncond_offset[b] + ucount[b];
    const int m = out->uncond_offset[nb];
    std::vector<int> cpos(out->bucket_offset, out->bucket_offset + nb);
    std::vector<int> upos(out->uncond_offset, out->uncond_offset + nb);
    for (int i = 0; i < n; ++i) {
        const int b = out->bucket_id[i];
        if (b < 0) continue;
        const int p = cpos[b]++;
        out->order[p] = i;
        out->cond_row[i] = m + p;
        if (need_u[i]) out->uncond_row[i] = upos[b]++;
    }
    for (int j = n_act; j < n; ++j) out->order[j] = -1;
    out->n_active = n_act;
    out->n_uncond = m;
    return BCG_OK;
}

extern "C" int bcg_plan_records(int n, int steps, const int32_t* step_idx, const float* scale,
                                const int32_t* uncond_row, const int32_t* region_valid,
                                const float* sigmas, int num_sigmas, float* records) {
    bcg::clear_error();
    if (n < 0 || steps < 1 || num_sigmas < 1) return fail(BCG_EINVAL, "bcg_plan_records: bad sizes");
    if (n > 0 && (!step_idx || !scale || !uncond_row || !sigmas || !records))
        return fail(BCG_EINVAL, "bcg_plan_records: NULL argument");
    for (int i = 0; i < n; ++i) {
        float* r = records + 4 * size_t(i);
        const int t = step_idx[i];
        if (t >= 0 && t < steps && t + 1 < num_sigmas) {
            const uint32_t valid = region_valid ? uint32_t(region_valid[i]) & 0xfu : 0xfu;
            const uint32_t fl = (uncond_row[i] >= 0 ? 3u : 1u) | (valid << 2);
            r[0] = sigmas[t];
            r[1] = sigmas[t + 1];
            r[2] = scale[i];
            std::memcpy(&r[3], &fl, sizeof fl);
        } else {
            r[0] = r[1] = r[2] = r[3] = 0.0f;
        }
    }
    return BCG_OK;
}
