// Device half of libbcg's C ABI: argument checks and launches of the fused
// guided step, its optional norm statistics, the latent initialiser and the
// standalone regional accumulation and mask blend kernels.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "bcg_common.h"
#include "bcg_device.h"
#include "bcg_plan_dev.h"
#include "bcg_launch.h"

using bcg::fail;

namespace bcg {
namespace {

// ------------------------------------------------------------ norm stats

// Wave-level reduction over the 64 lanes, fixed butterfly order.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// One wavefront per latent row (sample j, channel c, row y): the L2 norm over
// W of the cond prediction C, the uncond prediction U and the guided pred at
// the step's first evaluation point.  Same per-element arithmetic as the step.
template <typename T>
__global__ __launch_bounds__(256) void stats_rows_kernel(const StepParams p, float* rows) {
    const int64_t CH = (int64_t)p.C * p.H;
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (g >= (int64_t)p.n_active * CH) return;
    const int j = (int)(g / CH);
    const int rem = (int)(g - (int64_t)j * CH);
    const int c = rem / p.H, y = rem - (rem / p.H) * p.H;
    float* out = rows + g * 3;
    const int i = p.order[j];
    int t = -1;
    if (i >= 0 && i < p.n) t = p.step_idx[i];
    if (i < 0 || i >= p.n || t < 0 || t + 1 >= p.num_sigmas) {
        if (lane == 0) { out[0] = 0.f; out[1] = 0.f; out[2] = 0.f; }
        return;
    }
    const float sig = p.sigmas[t];
    const float w = p.scale[i];
    const bool keep_u = p.uncond_row[i] >= 0;
    int cnt = p.R > 0 ? p.region_count[i] : 0;
    cnt = std::max(0, std::min(cnt, std::min(p.R, BCG_MAX_REGIONS)));
    const unsigned valid = (cnt > 0 && p.region_range) ? region_mask(p, i, t) : 0xfu;
    const float s2 = p.s2;
    const float v = sig * sig;
    const float den = s2 + v;
    const float a = s2 / den;
    const float bu = (v * p.mu_uncond[(int64_t)i * p.C + c]) / den;
    const float bc = (v * p.mu_cond[(int64_t)i * p.C + c]) / den;
    float br[BCG_MAX_REGIONS];
    RegionDesc rd[BCG_MAX_REGIONS];
    for (int r = 0; r < BCG_MAX_REGIONS; ++r) {
        br[r] = 0.f;
        rd[r] = RegionDesc{0, 0, 0, 0, 0.f};
        if (r < cnt) {
            br[r] = (v * p.mu_region[((int64_t)i * p.R + r) * p.C + c]) / den;
            const int32_t* b = p.region_box + ((int64_t)i * p.R + r) * 4;
            rd[r] = RegionDesc{b[0], b[1] - b[0], b[2], b[3] - b[2],
                               ((valid >> r) & 1u) ? p.region_strength[(int64_t)i * p.R + r] : 0.0f};
        }
    }
    const T* xs = static_cast<const T*>(p.x) + ((int64_t)i * p.C + c) * p.HW + (int64_t)y * p.W;
    float sc = 0.f, su = 0.f, sp = 0.f;
    for (int x = lane; x < p.W; x += 64) {
        float xv[1];
        Io<T, 1>::load(xs + x, xv);
        const float xx = xv[0];
        const float u = __builtin_fmaf(a, xx, bu);
        float cc, pred;
        if (cnt == 0) {
            cc = __builtin_fmaf(a, xx, bc);
            pred = (w == 1.0f) ? cc : __builtin_fmaf(w, cc - u, u);
        } else {
            float ws[BCG_MAX_REGIONS];
            float wsum = 0.f;
            for (int r = 0; r < cnt; ++r) {
                ws[r] = region_weight(rd[r], y, x, p.feather, p.inv_f4);
                wsum = r == 0 ? ws[0] : wsum + ws[r];
            }
            const bool cv = wsum > 0.0f;
            const float iw = cv ? 1.0f / wsum : 0.0f;
            cc = (ws[0] * iw) * __builtin_fmaf(a, xx, br[0]);
            for (int r = 1; r < cnt; ++r) cc = __builtin_fmaf(ws[r] * iw, __builtin_fmaf(a, xx, br[r]), cc);
            if (w == 1.0f) pred = (keep_u ? cv : true) ? cc : u;
            else pred = __builtin_fmaf(cv ? w : 0.0f, cc - u, u);
            if (!cv) cc = u;  // the cond prediction where no region has weight
        }
        sc += cc * cc;
        su += u * u;
        sp += pred * pred;
    }
    sc = wave_sum(sc);
    su = wave_sum(su);
    sp = wave_sum(sp);
    if (lane == 0) {
        out[0] = sqrtf(sc);
        out[1] = keep_u ? sqrtf(su) : 0.f;
        out[2] = sqrtf(sp);
    }
}

// Mean of the row norms per sample: one workgroup per active sample, fixed
// strided partial sums then a fixed-order tree in LDS (deterministic).
__global__ __launch_bounds__(256) void stats_final_kernel(const StepParams p, const float* rows,
                                                          float* stats) {
    __shared__ float part[3][256];
    const int j = blockIdx.x;
    const int64_t CH = (int64_t)p.C * p.H;
    const float* r0 = rows + (int64_t)j * CH * 3;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f;
    for (int64_t g = threadIdx.x; g < CH; g += 256) {
        a0 += r0[g * 3 + 0];
        a1 += r0[g * 3 + 1];
        a2 += r0[g * 3 + 2];
    }
    part[0][threadIdx.x] = a0;
    part[1][threadIdx.x] = a1;
    part[2][threadIdx.x] = a2;
    __syncthreads();
    for (int s = 128; s >= 1; s >>= 1) {
        if ((int)threadIdx.x < s) {
            part[0][threadIdx.x] += part[0][threadIdx.x + s];
            part[1][threadIdx.x] += part[1][threadIdx.x + s];
            part[2][threadIdx.x] += part[2][threadIdx.x + s];
        }
        __syncthreads();
    }
    const int i = p.order[j];
    if (threadIdx.x < 3 && i >= 0 && i < p.n) stats[(int64_t)i * 3 + threadIdx.x] = part[threadIdx.x][0] / float(CH);
}

// Means of the row norms per sample from the step's own partials (p.stats_part):
// one workgroup per sample the step's grid covers; a sample the step skipped
// (inactive) is not written.  Slot (tile, group) of a sample holds the sums of
// the row norms of one lane group; slots whose group has no row are never
// written and are skipped.  Fixed strided sums, then a fixed-order tree.
__global__ __launch_bounds__(256) void stats_slots_final_kernel(const StepParams p, int block, float* stats) {
    __shared__ float part[3][256];
    const int j = blockIdx.x;
    const int i = p.identity ? j : p.order[j];
    if (i < 0 || i >= p.n) return;
    bool active;
    if (p.record_in) {
        active = (__float_as_uint(p.record_in[(int64_t)i * 4 + 3]) & 1u) != 0;
    } else {
        const int t = p.step_idx[i];
        active = t >= 0 && t < p.t_end;
    }
    if (!active) return;
    const int gpw = block / p.stats_group;  // lane groups per workgroup
    const int nslot = p.tiles * gpw;
    const float* s0 = p.stats_part + (int64_t)i * nslot * 3;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f;
    for (int q = threadIdx.x; q < nslot; q += 256) {
        const int tile = q / gpw, g = q - (q / gpw) * gpw;
        if ((int64_t)tile * block * p.vpt + (int64_t)g * p.stats_group >= p.nvec) continue;
        a0 += s0[q * 3 + 0];
        a1 += s0[q * 3 + 1];
        a2 += s0[q * 3 + 2];
    }
    part[0][threadIdx.x] = a0;
    part[1][threadIdx.x] = a1;
    part[2][threadIdx.x] = a2;
    __syncthreads();
    for (int s = 128; s >= 1; s >>= 1) {
        if ((int)threadIdx.x < s) {
            part[0][threadIdx.x] += part[0][threadIdx.x + s];
            part[1][threadIdx.x] += part[1][threadIdx.x + s];
            part[2][threadIdx.x] += part[2][threadIdx.x + s];
        }
        __syncthreads();
    }
    if (threadIdx.x < 3) stats[(int64_t)i * 3 + threadIdx.x] = part[threadIdx.x][0] / float((int64_t)p.C * p.H);
}

// ------------------------------------------------------------ latent init

template <typename T, int V>
__global__ __launch_bounds__(256) void latent_init_kernel(int n, int C, int64_t HW, const float* noise,
                                                          const T* latent, const float* sigmas,
                                                          int num_sigmas, const int32_t* step_idx,
                                                          T* out) {
    const int64_t nv = HW / V;
    const int64_t per = (int64_t)C * nv;
    const int64_t total = (int64_t)n * per;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int i = (int)(k / per);
        const int t = step_idx[i];
        if (t < 0 || t >= num_sigmas) continue;
        const float sg = sigmas[t];
        const int64_t e0 = k * V;
        float nz[V], lt[V], o[V];
        Io<float, V>::load(noise + e0, nz);
        if (latent) Io<T, V>::load(latent + e0, lt);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            o[e] = latent ? __builtin_fmaf(nz[e], sg, lt[e]) : nz[e] * sg;
        }
        Io<T, V>::store(out + e0, o);
    }
}

// ------------------------------------------------------------ mask blend

template <typename T, int V>
__global__ __launch_bounds__(256) void mask_blend_kernel(int n, int C, int64_t HW, const T* a,
                                                         const T* b, const float* mask,
                                                         int64_t mask_stride, T* out) {
    const int64_t nv = HW / V;
    const int64_t total = (int64_t)n * C * nv;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t ic = k / nv;
        const int64_t pv = k - ic * nv;
        const int64_t i = ic / C;
        const int64_t e0 = k * V;
        float av[V], bv[V], m[V], o[V];
        Io<T, V>::load(a + e0, av);
        Io<T, V>::load(b + e0, bv);
        Io<float, V>::load(mask + i * mask_stride + pv * V, m);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float om = 1.0f - m[e];
            o[e] = __builtin_fmaf(m[e], av[e], om * bv[e]);
        }
        Io<T, V>::store(out + e0, o);
    }
}

// ------------------------------------------------------------ area accumulate

// Gather form: one lane per output pixel walks the regions that contain it.
__global__ __launch_bounds__(256) void area_accumulate_kernel(
    int n, int C, int H, int W, int F, float inv_f4, int R, const float* pred, int64_t pred_elems,
    const int64_t* region_off, const int32_t* region_count, const int32_t* region_box,
    const float* region_strength, const float* fallback, float* cond_out, float* wsum_out,
    int tiles) {
    const int i = blockIdx.x / tiles;
    const int tile = blockIdx.x - i * tiles;
    if (i >= n) return;
    const int64_t HW = (int64_t)H * W;
    const int64_t p = (int64_t)tile * blockDim.x + threadIdx.x;
    if (p >= HW) return;
    const int y = (int)(p / W), x = (int)(p - (int64_t)(p / W) * W);
    int cnt = region_count[i];
    cnt = std::max(0, std::min(cnt, std::min(R, BCG_MAX_REGIONS)));
    RegionDesc rd[BCG_MAX_REGIONS];
    int64_t off[BCG_MAX_REGIONS];
    bool ok[BCG_MAX_REGIONS];
    float ws[BCG_MAX_REGIONS];
    float wsum = 0.f;
    for (int r = 0; r < BCG_MAX_REGIONS; ++r) {
        ok[r] = false;
        ws[r] = 0.f;
        if (r >= cnt) continue;
        const int32_t* b = region_box + ((int64_t)i * R + r) * 4;
        const int y0 = b[0], y1 = b[1], x0 = b[2], x1 = b[3];
        const int64_t o = region_off[(int64_t)i * R + r];
        const int64_t o_next = region_off[(int64_t)i * R + r + 1];
        const int64_t sz = (int64_t)C * (y1 - y0) * (x1 - x0);
        ok[r] = 0 <= y0 && y0 < y1 && y1 <= H && 0 <= x0 && x0 < x1 && x1 <= W && o >= 0 &&
                o + sz <= pred_elems && o + sz <= o_next;
        if (!ok[r]) continue;
        rd[r] = RegionDesc{y0, y1 - y0, x0, x1 - x0, region_strength[(int64_t)i * R + r]};
        off[r] = o;
        ws[r] = region_weight(rd[r], y, x, F, inv_f4);
        wsum = r == 0 ? ws[0] : wsum + ws[r];
    }
    const bool cv = wsum > 0.0f;
    const float iw = cv ? 1.0f / wsum : 0.0f;
    float wh[BCG_MAX_REGIONS];
    bool in[BCG_MAX_REGIONS];
    for (int r = 0; r < BCG_MAX_REGIONS; ++r) {
        wh[r] = ws[r] * iw;
        in[r] = ok[r] && y >= rd[r].y0 && y < rd[r].y0 + rd[r].h && x >= rd[r].x0 &&
                x < rd[r].x0 + rd[r].w;
    }
    for (int c = 0; c < C; ++c) {
        float acc = 0.f;
        bool started = false;
        for (int r = 0; r < cnt; ++r) {
            if (!in[r]) continue;
            const float v = pred[off[r] + ((int64_t)c * rd[r].h + (y - rd[r].y0)) * rd[r].w + (x - rd[r].x0)];
            acc = started ? __builtin_fmaf(wh[r], v, acc) : wh[r] * v;
            started = true;
        }
        const int64_t q = ((int64_t)i * C + c) * HW + p;
        cond_out[q] = cv ? acc : (fallback ? fallback[q] : 0.0f);
    }
    if (wsum_out) wsum_out[(int64_t)i * HW + p] = wsum;
}

int grid_for(int64_t work, int block) {
    const int64_t g = (work + block - 1) / block;
    return (int)std::max<int64_t>(1, std::min<int64_t>(g, 1 << 20));
}

// ------------------------------------------------------------ device plan

__global__ __launch_bounds__(256) void plan_kernel(const StepParams p) {
    constexpr int kInts = 4 * BCG_MAX_DEVICE_BUCKETS;
    __shared__ int sh[kInts];
    plan_workgroup(p, sh, kInts);
}

// Checks a device plan for n samples; `step` says whether it drives a step.
int check_dplan(const bcg_device_plan* d, int n, bool step, const char* who) {
    if (!d) return fail(BCG_EINVAL, "%s: plan is NULL", who);
    if (d->steps < 1 || d->steps > BCG_MAX_DEVICE_STEPS)
        return fail(BCG_EINVAL, "%s: steps %d not in [1, %d]", who, d->steps, BCG_MAX_DEVICE_STEPS);
    if (d->num_buckets < 1 || d->num_buckets > BCG_MAX_DEVICE_BUCKETS)
        return fail(BCG_EINVAL, "%s: num_buckets %d not in [1, %d]", who, d->num_buckets, BCG_MAX_DEVICE_BUCKETS);
    if (d->wrap != 0 && d->wrap != 1) return fail(BCG_EINVAL, "%s: wrap must be 0 or 1", who);
    if (n == 0) return BCG_OK;
    if (!d->bucket_cfg || !d->step_in) return fail(BCG_EINVAL, "%s: bucket_cfg/step_in is NULL", who);
    const void* outs[] = {d->bucket_id, d->scale, d->uncond_row, d->cond_row, d->order,
                          d->bucket_count, d->bucket_offset, d->uncond_offset, d->totals};
    int given = 0;
    for (const void* o : outs) given += o != nullptr;
    if (given != 0 && given != 9) return fail(BCG_EINVAL, "%s: plan outputs must be all given or all NULL", who);
    if (!step && given == 0 && !d->step_out && !d->record_out)
        return fail(BCG_EINVAL, "%s: nothing to write", who);
    if (d->step_out) {
        const size_t bytes = (size_t)n * sizeof(int32_t);
        const uintptr_t a = reinterpret_cast<uintptr_t>(d->step_in), b = reinterpret_cast<uintptr_t>(d->step_out);
        if (a < b + bytes && b < a + bytes) return fail(BCG_EINVAL, "%s: step_out overlaps step_in", who);
    }
    if (d->record_out && !step && (!d->sigmas || d->num_sigmas < 1))
        return fail(BCG_EINVAL, "%s: record_out needs the schedule (sigmas, num_sigmas)", who);
    if (d->record_in && !step) return fail(BCG_EINVAL, "%s: record_in is read by a step only", who);
    if (d->record_in && d->record_out &&
        any_overlap(d->record_in, (size_t)n * 16, d->record_out, (size_t)n * 16))
        return fail(BCG_EINVAL, "%s: record_out overlaps record_in", who);
    if (d->queue_len < 0 || d->queue_len >= (1 << 24))
        return fail(BCG_EINVAL, "%s: queue_len %d not in [0, 2^24)", who, d->queue_len);
    if (d->queue_len > 0) {
        if (!step) return fail(BCG_EINVAL, "%s: continuous batching runs inside guided_step_dplan", who);
        if (d->queue_ring != 0 && d->queue_ring != 1) return fail(BCG_EINVAL, "%s: queue_ring must be 0 or 1", who);
        if (d->wrap) return fail(BCG_EINVAL, "%s: continuous batching replaces wrap (set it to 0)", who);
        if (d->queue_len < n) return fail(BCG_EINVAL, "%s: queue_len %d < n %d slots", who, d->queue_len, n);
        if (!d->noise || !d->slot_req_in || !d->slot_req_out || !d->queue_in || !d->queue_out ||
            !d->record_in || !d->record_out || !d->step_out)
            return fail(BCG_EINVAL, "%s: continuous batching needs noise, slot_req_in/out, queue_in/out, "
                        "record_in/out and step_out", who);
        const size_t in4 = (size_t)n * 4;
        if (any_overlap(d->slot_req_in, in4, d->slot_req_out, in4) || any_overlap(d->queue_in, 4, d->queue_out, 4))
            return fail(BCG_EINVAL, "%s: slot_req_out / queue_out overlap their inputs", who);
        if (d->join_front < 0 || d->join_front > n)
            return fail(BCG_EINVAL, "%s: join_front %d not in [0, n]", who, d->join_front);
        if (d->join_front > 0) {
            const size_t j4 = (size_t)d->join_front * 4;
            if (!d->join_in || !d->join_out) return fail(BCG_EINVAL, "%s: join_front needs join_in and join_out", who);
            if (any_overlap(d->join_in, j4, d->join_out, j4))
                return fail(BCG_EINVAL, "%s: join_out overlaps join_in", who);
        }
    } else if (d->slot_req_in || d->slot_req_out || d->queue_in || d->queue_out || d->noise || d->join_front ||
               d->join_in || d->join_out) {
        return fail(BCG_EINVAL, "%s: queue arrays given with queue_len = 0", who);
    }
    return BCG_OK;
}

void fill_dplan(StepParams& p, const bcg_device_plan* d) {
    p.dplan = 1;
    p.steps = d->steps;
    p.nb = d->num_buckets;
    p.wrap = d->wrap;
    p.bucket_cfg = d->bucket_cfg;
    p.bucket_cfg_end = d->bucket_cfg_end;
    p.cfg_override = d->cfg_override;
    p.covered = d->covered;
    p.step_idx = d->step_in;
    p.step_out = d->step_out;
    p.plan_bucket_id = d->bucket_id;
    p.plan_scale = d->scale;
    p.plan_uncond_row = d->uncond_row;
    p.plan_cond_row = d->cond_row;
    p.plan_order = d->order;
    p.plan_bucket_count = d->bucket_count;
    p.plan_bucket_offset = d->bucket_offset;
    p.plan_uncond_offset = d->uncond_offset;
    p.plan_totals = d->totals;
    p.record_in = d->record_in;
    p.record_out = d->record_out;
    p.region_range = d->region_range;
    p.range_steps = d->steps;
    p.covered_sets = d->covered_sets;
    p.queue_len = d->queue_len;
    p.queue_ring = d->queue_ring;
    p.noise = d->noise;
    p.slot_req = d->slot_req_in;
    p.slot_req_out = d->slot_req_out;
    p.queue_in = d->queue_in;
    p.queue_out = d->queue_out;
    p.join_front = d->queue_len > 0 ? d->join_front : 0;
    p.join_in = d->join_in;
    p.join_out = d->join_out;
}

}  // namespace
}  // namespace bcg

using namespace bcg;

// Stats workspace: the row norms of the two-pass form ([n][C][H][3]) or the
// step's own partials ([n][tiles][groups][3]: a row per lane group, fewer
// than H + 256 slots a sample with the last tile's unused groups).
extern "C" size_t guided_step_workspace_size(int n, int C, int H, int W, int dtype) {
    (void)W;
    (void)dtype;
    if (n <= 0 || C <= 0 || H <= 0) return 0;
    return (size_t)n * (size_t)std::max<int64_t>((int64_t)C * H, (int64_t)H + 256) * 3 * sizeof(float);
}

namespace {

int hip_status_of(hipError_t e, const char* who, const char* what) {
    if (e != hipSuccess) return fail(BCG_EHIP, "%s: %s: %s", who, what, hipGetErrorString(e));
    return BCG_OK;
}

// guided_step with the host plan (d == NULL) or a device-built one (d).
int step_impl(const bcg_step_args* a, const bcg_device_plan* d, void* stream, const char* who,
              bool static_ws = false) {
    if (!a) return fail(BCG_EINVAL, "%s: args is NULL", who);
    if (a->n < 0 || a->C < 1 || a->C > BCG_MAX_CHANNELS || a->H < 1 || a->W < 1)
        return fail(BCG_ESHAPE, "%s: bad shape n=%d C=%d H=%d W=%d (C must be in [1, %d])", who,
                    a->n, a->C, a->H, a->W, BCG_MAX_CHANNELS);
    const int64_t HW = (int64_t)a->H * a->W;
    if (HW > (int64_t(1) << 30)) return fail(BCG_ESHAPE, "%s: H*W too large", who);
    if (a->dtype != BCG_F32 && a->dtype != BCG_BF16) return fail(BCG_EDTYPE, "%s: unknown dtype %d", who, a->dtype);
    if (a->sampler != BCG_EULER && a->sampler != BCG_HEUN)
        return fail(BCG_EINVAL, "%s: unknown sampler %d", who, a->sampler);
    if (a->max_regions < 0 || a->max_regions > BCG_MAX_REGIONS)
        return fail(BCG_EINVAL, "%s: max_regions %d not in [0, %d]", who, a->max_regions, BCG_MAX_REGIONS);
    if (a->feather < 0 || a->feather > BCG_MAX_FEATHER)
        return fail(BCG_EINVAL, "%s: feather %d out of range", who, a->feather);
    if (!d && (a->n_active < 0 || a->n_active > a->n))
        return fail(BCG_EINVAL, "%s: n_active %d not in [0, n]", who, a->n_active);
    if (a->num_sigmas < 2) return fail(BCG_EINVAL, "%s: num_sigmas %d < 2", who, a->num_sigmas);
    if (!(a->s2 > 0.0f) || !std::isfinite(a->s2)) return fail(BCG_EINVAL, "%s: s2 must be finite and > 0", who);
    if (a->mask_per_sample != 0 && a->mask_per_sample != 1)
        return fail(BCG_EINVAL, "%s: mask_per_sample must be 0 or 1", who);
    if (a->cache_hint != BCG_CACHE_KEEP && a->cache_hint != BCG_CACHE_STREAM)
        return fail(BCG_EINVAL, "%s: unknown cache_hint %d", who, a->cache_hint);
    if (a->launch_vpt < 0 || a->launch_vpt > 64)
        return fail(BCG_EINVAL, "%s: launch_vpt %d not in [0, 64]", who, a->launch_vpt);
    if (d) {
        const int rc = check_dplan(d, a->n, true, who);
        if (rc) return rc;
        if (a->order || a->step_idx || a->scale || a->uncond_row)
            return fail(BCG_EINVAL, "%s: order/step_idx/scale/uncond_row come from the device plan and must be NULL", who);
        if (a->num_sigmas < d->steps + 1)
            return fail(BCG_EINVAL, "%s: num_sigmas %d < steps + 1 = %d", who, a->num_sigmas, d->steps + 1);
        if (a->max_regions > 0 && a->region_count && !d->covered && !(d->region_range && d->covered_sets))
            return fail(BCG_EINVAL, "%s: a step with regions needs the coverage flags", who);
        if (d->region_range && (!d->covered_sets || d->max_regions != a->max_regions))
            return fail(BCG_EINVAL, "%s: validity ranges need covered_sets and max_regions = R", who);
        if (a->region_range && a->region_range != d->region_range)
            return fail(BCG_EINVAL, "%s: give the validity ranges in the device plan", who);
        if ((d->record_in || d->record_out) && (!aligned16(d->record_in) || !aligned16(d->record_out)))
            return fail(BCG_EINVAL, "%s: records must be 16-byte aligned", who);
    }
    if (!d && a->max_regions > 0 && a->region_range && a->steps < 1)
        return fail(BCG_EINVAL, "%s: validity ranges need steps >= 1", who);
    const int n_run = d ? a->n : a->n_active;  // samples the grid covers
    if (n_run == 0) return BCG_OK;
    if (!a->x || !a->x_out || !a->sigmas || !a->mu_uncond || !a->mu_cond ||
        (!d && (!a->order || !a->step_idx || !a->scale || !a->uncond_row)))
        return fail(BCG_EINVAL, "%s: NULL device pointer", who);
    if (a->max_regions > 0 && (!a->region_count || !a->region_box || !a->region_strength || !a->mu_region))
        return fail(BCG_EINVAL, "%s: max_regions > 0 needs region_count/box/strength/mu_region", who);
    if ((a->x_orig == nullptr) != (a->mask == nullptr))
        return fail(BCG_EINVAL, "%s: x_orig and mask must be given together", who);
    const size_t bytes = (size_t)a->n * a->C * HW * elem_size(a->dtype);
    if (partial_overlap(a->x, a->x_out, bytes)) return fail(BCG_EINVAL, "%s: x and x_out partially overlap", who);
    if (d && (d->step_out || d->bucket_id || d->record_out)) {
        // The plan's workgroup runs alongside the step: nothing it writes may
        // be read or written by the step, nor may it read the step's output.
        struct Span {
            const void* p;
            size_t bytes;
        };
        const size_t in4 = (size_t)a->n * 4, nb4 = (size_t)(d->num_buckets + 1) * 4;
        const size_t cfg4 = (size_t)d->num_buckets * 4;
        // per-sample tables: one entry per request under continuous batching
        const size_t nt = d->queue_len > 0 ? (size_t)d->queue_len : (size_t)a->n;
        const size_t t4 = nt * 4;
        const size_t R = (size_t)a->max_regions, nC4 = t4 * a->C;
        const size_t mbytes = a->mask ? (a->mask_per_sample ? nt : 1) * HW * 4 : 0;
        const size_t obytes = nt * a->C * HW * elem_size(a->dtype);
        const Span writes[] = {{d->bucket_id, in4},     {d->scale, in4},          {d->uncond_row, in4},
                               {d->cond_row, in4},      {d->order, in4},          {d->bucket_count, nb4},
                               {d->bucket_offset, nb4}, {d->uncond_offset, nb4},  {d->totals, 8},
                               {d->step_out, in4},      {d->record_out, in4 * 4},
                               {d->slot_req_out, d->queue_len ? in4 : 0}, {d->queue_out, d->queue_len ? 4u : 0u},
                               {d->join_out, d->queue_len ? (size_t)d->join_front * 4 : 0}};
        const Span step_uses[] = {{a->x, bytes},       // [0], [1]: the state; inputs from [2] on
                                  {a->x_out, bytes},
                                  {a->x_orig, a->x_orig ? obytes : 0},
                                  {a->mask, mbytes},
                                  {a->sigmas, (size_t)a->num_sigmas * 4},
                                  {a->mu_uncond, nC4},
                                  {a->mu_cond, nC4},
                                  {a->region_count, R ? t4 : 0},
                                  {a->region_box, t4 * R * 4},
                                  {a->region_strength, t4 * R},
                                  {a->mu_region, nC4 * R},
                                  {d->record_in, d->record_in ? in4 * 4 : 0},
                                  {d->step_in, in4},
                                  {d->bucket_cfg, cfg4},
                                  {d->bucket_cfg_end, d->bucket_cfg_end ? cfg4 : 0},
                                  {d->cfg_override, d->cfg_override ? t4 : 0},
                                  {d->covered, d->covered ? t4 : 0},
                                  {d->covered_sets, d->covered_sets ? nt * 2 : 0},
                                  {d->region_range, d->region_range ? t4 * 4 * R : 0},
                                  {d->noise, d->noise ? nt * a->C * HW * 4 : 0},
                                  {d->slot_req_in, d->slot_req_in ? in4 : 0},
                                  {d->queue_in, d->queue_in ? 4u : 0u},
                                  {d->join_in, d->queue_len ? (size_t)d->join_front * 4 : 0}};
        for (const Span& w : writes)
            for (const Span& r : step_uses)
                if (w.p && r.p && r.bytes && any_overlap(w.p, w.bytes, r.p, r.bytes))
                    return fail(BCG_EINVAL, "%s: the plan's outputs overlap arrays the step reads or writes", who);
        // every input of the step and of its plan but x itself (x_out may be x) vs the output
        for (size_t q = 2; q < sizeof(step_uses) / sizeof(step_uses[0]); ++q) {
            const Span& r = step_uses[q];
            if (r.p && r.bytes && any_overlap(r.p, r.bytes, a->x_out, bytes))
                return fail(BCG_EINVAL, "%s: an input of the step or its plan overlaps x_out", who);
        }
    }
    const bool inpaint = a->x_orig != nullptr;
    const int VV = a->dtype == BCG_BF16 ? 8 : 4;
    const bool vec = HW % VV == 0 && aligned16(a->x) && aligned16(a->x_out) &&
                     (!inpaint || (aligned16(a->x_orig) && aligned16(a->mask)));
    // Statistics inside the step when a latent row is a power-of-two group of
    // at most 64 lanes (W a multiple of the vector, W / vector a power of
    // two); otherwise (host plans only) two extra kernels read x again.
    if (d && d->queue_len > 0) {
        if (!vec)
            return fail(BCG_EINVAL, "%s: continuous batching needs the 16-byte vector path (H*W a multiple of %d, "
                        "16-byte aligned arrays)", who, VV);
        if (a->stats) return fail(BCG_EINVAL, "%s: stats are not available with continuous batching", who);
        if (!aligned16(d->noise)) return fail(BCG_EINVAL, "%s: noise must be 16-byte aligned", who);
    }
    const int row_lanes = vec && a->W % VV == 0 ? a->W / VV : 0;
    const bool fused_stats = a->stats && row_lanes >= 1 && row_lanes <= 64 && (row_lanes & (row_lanes - 1)) == 0;
    if (a->stats) {
        if (d && !fused_stats)
            return fail(BCG_EINVAL, "%s: stats with a device plan need W to be a power-of-two multiple (at most 64) "
                        "of the %d-pixel vector, and 16-byte aligned arrays", who, VV);
        const size_t need = guided_step_workspace_size(d ? a->n : a->n_active, a->C, a->H, a->W, a->dtype);
        if (!a->workspace || (!static_ws && a->workspace_bytes < need))
            return fail(BCG_EINVAL, "%s: stats need a workspace of %zu bytes", who, need);
    }

    StepParams p{};
    p.n = a->n; p.C = a->C; p.H = a->H; p.W = a->W; p.R = a->max_regions;
    p.feather = std::max(a->feather, 1);
    p.inv_f4 = 1.0f / float(p.feather * p.feather * p.feather * p.feather);
    p.n_active = n_run;
    p.num_sigmas = a->num_sigmas;
    p.HW = HW;
    p.nvec = (int)(vec ? HW / VV : HW);
    p.rows_aligned = vec ? (a->W % VV == 0) : 1;
    p.identity = n_run == a->n ? 1 : 0;
    p.mask_stride = a->mask_per_sample ? (int)HW : 0;
    p.s2 = a->s2;
    p.x = a->x; p.x_out = a->x_out; p.sigmas = a->sigmas; p.order = a->order;
    p.step_idx = a->step_idx; p.scale = a->scale; p.uncond_row = a->uncond_row;
    p.mu_uncond = a->mu_uncond; p.mu_cond = a->mu_cond; p.region_count = a->region_count;
    p.region_box = a->region_box; p.region_strength = a->region_strength; p.mu_region = a->mu_region;
    p.x_orig = a->x_orig; p.mask = a->mask;
    p.t_end = a->num_sigmas - 1;
    p.plan_block = -1;
    p.region_range = a->max_regions > 0 ? a->region_range : nullptr;
    p.range_steps = a->steps;
    if (d) {
        fill_dplan(p, d);
        p.t_end = d->steps;
    }
    const LaunchShape shape = a->launch_vpt > 0 ? LaunchShape{256, a->launch_vpt} : pick_shape(p.n_active, p.nvec);
    const int block = shape.block;
    p.vpt = shape.vpt;
    p.tiles = (int)(((int64_t)p.nvec + (int64_t)block * p.vpt - 1) / ((int64_t)block * p.vpt));
    if ((int64_t)p.n_active * p.tiles >= INT32_MAX) return fail(BCG_ESHAPE, "%s: grid too large", who);
    if (fused_stats) {
        const size_t need = (size_t)a->n * p.tiles * (block / row_lanes) * 3 * sizeof(float);
        if (a->workspace_bytes < need) {
            if (static_ws)
                return fail(BCG_EINVAL, "%s: the statistics of %d samples at this shape need %zu bytes, more than "
                            "the library's static scratch of %zu bytes", who, a->n, need, a->workspace_bytes);
            return fail(BCG_EINVAL, "%s: stats need a workspace of %zu bytes", who, need);
        }
        p.stats_part = static_cast<float*>(a->workspace);
        p.stats_group = row_lanes;
    }
    const int64_t lead = p.join_front;
    if ((lead + p.n_active) * p.tiles >= INT32_MAX) return fail(BCG_ESHAPE, "%s: grid too large", who);
    if (d && (d->step_out || d->bucket_id || d->record_out))
        p.plan_block = (int)((lead + p.n_active) * p.tiles);
    hipStream_t st = static_cast<hipStream_t>(stream);

    if (a->stats && !fused_stats) {
        float* rows = static_cast<float*>(a->workspace);
        const int64_t nrows = (int64_t)p.n_active * p.C * p.H;
        const int g = (int)((nrows + 3) / 4);
        if (a->dtype == BCG_BF16) hipLaunchKernelGGL(stats_rows_kernel<bf16_t>, dim3(g), dim3(256), 0, st, p, rows);
        else hipLaunchKernelGGL(stats_rows_kernel<float>, dim3(g), dim3(256), 0, st, p, rows);
        int rc = hip_status_of(hipGetLastError(), who, "stats launch");
        if (rc) return rc;
        hipLaunchKernelGGL(stats_final_kernel, dim3(p.n_active), dim3(256), 0, st, p, rows, a->stats);
        rc = hip_status_of(hipGetLastError(), who, "stats launch");
        if (rc) return rc;
    }
    const bool heun = a->sampler == BCG_HEUN;
    hipError_t e;
    const bool queue = d && d->queue_len > 0;  // continuous batching runs on the streaming variants
    if (queue)
        e = a->dtype == BCG_BF16 ? launch_step_bf16_queue(p, heun, inpaint, block, st)
                                 : launch_step_f32_queue(p, heun, inpaint, block, st);
    else if (vec && a->cache_hint == BCG_CACHE_STREAM && !fused_stats)  // the statistics run on the keep variants
        e = a->dtype == BCG_BF16 ? launch_step_bf16_stream(p, heun, inpaint, block, st)
                                 : launch_step_f32_stream(p, heun, inpaint, block, st);
    else
        e = a->dtype == BCG_BF16 ? launch_step_bf16(p, vec, heun, inpaint, block, st)
                                 : launch_step_f32(p, vec, heun, inpaint, block, st);
    int rc = hip_status_of(e, who, "launch");
    if (rc || !fused_stats) return rc;
    hipLaunchKernelGGL(stats_slots_final_kernel, dim3(p.n_active), dim3(256), 0, st, p, block, a->stats);
    return hip_status_of(hipGetLastError(), who, "stats launch");
}

}  // namespace

extern "C" int guided_step(const bcg_step_args* a, void* stream) {
    bcg::clear_error();
    return step_impl(a, nullptr, stream, "guided_step");
}

extern "C" int guided_step_dplan(const bcg_step_args* a, const bcg_device_plan* d, void* stream) {
    bcg::clear_error();
    if (!d) return fail(BCG_EINVAL, "guided_step_dplan: plan is NULL");
    return step_impl(a, d, stream, "guided_step_dplan");
}

// The statistics' partials of guided_step_dplan_static: one array per GPU, part
// of the library's code object (no allocation call), held until the process ends.
static __device__ __align__(256) float scratch[BCG_STATIC_SCRATCH_BYTES / sizeof(float)];

namespace {

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept; the host-side name is only a stand-in
// and is never passed to a kernel.
int scratch_address(float** out, const char* who) {
    constexpr int kDevices = 64;
    static std::mutex mu;
    static float* addr[kDevices] = {};
    int dev = 0;
    int rc = hip_status_of(hipGetDevice(&dev), who, "hipGetDevice");
    if (rc) return rc;
    if (dev < 0 || dev >= kDevices) return fail(BCG_EINVAL, "%s: device %d beyond %d", who, dev, kDevices);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* ptr = nullptr;
        rc = hip_status_of(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), who, "hipGetSymbolAddress(scratch)");
        if (rc) return rc;
        if (!ptr) return fail(BCG_EHIP, "%s: no device address for the static scratch", who);
        addr[dev] = static_cast<float*>(ptr);
    }
    *out = addr[dev];
    return BCG_OK;
}

}  // namespace

extern "C" int guided_step_dplan_static(const bcg_step_args* a, const bcg_device_plan* d, void* stream) {
    bcg::clear_error();
    const char* who = "guided_step_dplan_static";
    if (!a) return fail(BCG_EINVAL, "%s: args is NULL", who);
    if (!d) return fail(BCG_EINVAL, "%s: plan is NULL", who);
    if (a->workspace || a->workspace_bytes)
        return fail(BCG_EINVAL, "%s: workspace must be NULL (the library's static scratch is used)", who);
    if (!a->stats) return step_impl(a, d, stream, who);
    float* ptr = nullptr;
    const int rc = scratch_address(&ptr, who);
    if (rc) return rc;
    bcg_step_args b = *a;
    b.workspace = ptr;
    b.workspace_bytes = BCG_STATIC_SCRATCH_BYTES;
    return step_impl(&b, d, stream, who, true);
}

// Parameters of a plan built on its own (no step in the same workgroup).
static StepParams plan_only_params(int n, const bcg_device_plan* d) {
    StepParams p{};
    p.n = n;
    fill_dplan(p, d);
    p.t_end = d->steps;
    p.plan_block = 0;
    p.R = d->max_regions;
    p.region_count = d->region_count;
    p.sigmas = d->sigmas;
    p.num_sigmas = d->num_sigmas;
    return p;
}

extern "C" int bcg_plan_device(int n, const bcg_device_plan* d, void* stream) {
    bcg::clear_error();
    if (n < 0 || n > (1 << 24)) return fail(BCG_ESHAPE, "bcg_plan_device: n %d out of range", n);
    const int rc = check_dplan(d, n, false, "bcg_plan_device");
    if (rc) return rc;
    if (n == 0) return BCG_OK;
    const StepParams p = plan_only_params(n, d);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream), p);
    return hip_status(hipGetLastError(), "bcg_plan_device: launch");
}

// A rows call, validated, with its launch shape (launch is false when there
// is no sample to update).
struct RowsLaunch {
    RowsParams p;
    bool vec, inpaint, nt, launch;
    int block;
    int dtype;
};

static int rows_prepare(const bcg_rows_args* a, const char* who, RowsLaunch& L) {
    if (!a) return fail(BCG_EINVAL, "%s: args is NULL", who);
    if (a->n < 0 || a->C < 1 || a->H < 1 || a->W < 1)
        return fail(BCG_ESHAPE, "%s: bad shape n=%d C=%d H=%d W=%d", who, a->n, a->C, a->H, a->W);
    const int64_t HW = (int64_t)a->H * a->W;
    if (HW > (int64_t(1) << 30) || (int64_t)a->C * HW > (int64_t(1) << 36))
        return fail(BCG_ESHAPE, "%s: C*H*W too large", who);
    if (a->dtype != BCG_F32 && a->dtype != BCG_BF16) return fail(BCG_EDTYPE, "%s: unknown dtype %d", who, a->dtype);
    if (a->phase != BCG_PHASE_EULER && a->phase != BCG_PHASE_HEUN_PREDICT && a->phase != BCG_PHASE_HEUN_CORRECT)
        return fail(BCG_EINVAL, "%s: unknown phase %d", who, a->phase);
    if (a->n_active < 0 || a->n_active > a->n) return fail(BCG_EINVAL, "%s: n_active %d not in [0, n]", who, a->n_active);
    if (a->num_sigmas < 2) return fail(BCG_EINVAL, "%s: num_sigmas %d < 2", who, a->num_sigmas);
    if (a->rows < 0) return fail(BCG_EINVAL, "%s: rows %d < 0", who, a->rows);
    if (a->mask_per_sample != 0 && a->mask_per_sample != 1)
        return fail(BCG_EINVAL, "%s: mask_per_sample must be 0 or 1", who);
    if (a->cache_hint != BCG_CACHE_KEEP && a->cache_hint != BCG_CACHE_STREAM)
        return fail(BCG_EINVAL, "%s: unknown cache_hint %d", who, a->cache_hint);
    if (a->launch_vpt < 0 || a->launch_vpt > 64)
        return fail(BCG_EINVAL, "%s: launch_vpt %d not in [0, 64]", who, a->launch_vpt);
    L.launch = a->n_active > 0;
    L.dtype = a->dtype;
    if (!L.launch) return BCG_OK;
    if (!a->x || !a->x_out || !a->pred || !a->sigmas || !a->order || !a->step_idx || !a->scale ||
        !a->uncond_row || !a->cond_row)
        return fail(BCG_EINVAL, "%s: NULL device pointer", who);
    const bool heun = a->phase != BCG_PHASE_EULER;
    if (heun && !a->d) return fail(BCG_EINVAL, "%s: Heun phases need d", who);
    if (a->phase == BCG_PHASE_HEUN_CORRECT && !a->x_tilde) return fail(BCG_EINVAL, "%s: the corrector needs x_tilde", who);
    if ((a->x_orig == nullptr) != (a->mask == nullptr))
        return fail(BCG_EINVAL, "%s: x_orig and mask must be given together", who);
    const size_t es = elem_size(a->dtype);
    const size_t bytes = (size_t)a->n * a->C * HW * es;
    const size_t pbytes = (size_t)a->rows * a->C * HW * es;
    if (partial_overlap(a->x, a->x_out, bytes)) return fail(BCG_EINVAL, "%s: x and x_out partially overlap", who);
    if (any_overlap(a->pred, pbytes, a->x_out, bytes)) return fail(BCG_EINVAL, "%s: pred overlaps x_out", who);
    if (heun && any_overlap(a->d, (size_t)a->n * a->C * HW * 4, a->x_out, bytes))
        return fail(BCG_EINVAL, "%s: d overlaps x_out", who);
    if (a->x_tilde && a->phase == BCG_PHASE_HEUN_CORRECT && partial_overlap(a->x_tilde, a->x_out, bytes))
        return fail(BCG_EINVAL, "%s: x_tilde and x_out partially overlap", who);
    const bool inpaint = a->x_orig != nullptr;
    const int VV = a->dtype == BCG_BF16 ? 8 : 4;
    const bool vec = HW % VV == 0 && aligned16(a->x) && aligned16(a->x_out) && aligned16(a->pred) &&
                     (!inpaint || (aligned16(a->x_orig) && aligned16(a->mask))) && (!heun || aligned16(a->d)) &&
                     (a->phase != BCG_PHASE_HEUN_CORRECT || aligned16(a->x_tilde));
    RowsParams& p = L.p;
    p = RowsParams{};
    p.plan_block = -1;
    p.n = a->n; p.C = a->C; p.n_active = a->n_active; p.num_sigmas = a->num_sigmas; p.rows = a->rows;
    p.phase = a->phase;
    p.HW = HW;
    p.nvec = (int)(vec ? HW / VV : HW);
    p.identity = a->n_active == a->n ? 1 : 0;
    p.mask_stride = a->mask_per_sample ? (int)HW : 0;
    p.x = a->x; p.x_out = a->x_out; p.d = heun ? a->d : nullptr;
    p.x_tilde = a->phase == BCG_PHASE_HEUN_CORRECT ? a->x_tilde : nullptr;
    p.pred = a->pred; p.sigmas = a->sigmas; p.order = a->order; p.step_idx = a->step_idx;
    p.scale = a->scale; p.uncond_row = a->uncond_row; p.cond_row = a->cond_row;
    p.x_orig = a->x_orig; p.mask = a->mask;
    const LaunchShape shape = a->launch_vpt > 0 ? LaunchShape{256, a->launch_vpt} : pick_shape(p.n_active, p.nvec);
    p.vpt = shape.vpt;
    p.tiles = (int)(((int64_t)p.nvec + (int64_t)shape.block * p.vpt - 1) / ((int64_t)shape.block * p.vpt));
    if ((int64_t)p.n_active * p.tiles >= INT32_MAX - 1) return fail(BCG_ESHAPE, "%s: grid too large", who);
    L.vec = vec;
    L.inpaint = inpaint;
    L.nt = a->cache_hint == BCG_CACHE_STREAM;
    L.block = shape.block;
    return BCG_OK;
}

static int rows_launch(const RowsLaunch& L, void* stream, const char* who) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = L.dtype == BCG_BF16 ? launch_rows_bf16(L.p, L.vec, L.inpaint, L.nt, L.block, st)
                                             : launch_rows_f32(L.p, L.vec, L.inpaint, L.nt, L.block, st);
    return hip_status(e, who);
}

extern "C" int guided_step_rows(const bcg_rows_args* a, void* stream) {
    bcg::clear_error();
    RowsLaunch L;
    const int rc = rows_prepare(a, "guided_step_rows", L);
    if (rc || !L.launch) return rc;
    return rows_launch(L, stream, "guided_step_rows: launch");
}

extern "C" int guided_step_rows_dplan(const bcg_rows_args* a, const bcg_device_plan* d, void* stream) {
    bcg::clear_error();
    const char* who = "guided_step_rows_dplan";
    RowsLaunch L;
    int rc = rows_prepare(a, who, L);
    if (rc) return rc;
    const int n = a->n;
    rc = check_dplan(d, n, false, who);
    if (rc) return rc;
    if (n == 0) return BCG_OK;
    // The plan's workgroup runs alongside the update: nothing it writes may
    // be read or written by the update, nor may it read the update's outputs.
    const size_t es = elem_size(a->dtype);
    const size_t xbytes = (size_t)a->n * a->C * a->H * a->W * es;
    const size_t dbytes = a->d ? (size_t)a->n * a->C * a->H * a->W * 4 : 0;
    const size_t in4 = (size_t)n * 4, nb4 = (size_t)(d->num_buckets + 1) * 4;
    struct Span {
        const void* p;
        size_t bytes;
    };
    const Span writes[] = {{d->bucket_id, in4},    {d->scale, in4},         {d->uncond_row, in4},
                           {d->cond_row, in4},     {d->order, in4},         {d->bucket_count, nb4},
                           {d->bucket_offset, nb4}, {d->uncond_offset, nb4}, {d->totals, 8},
                           {d->step_out, in4},     {d->record_out, in4 * 4}};
    const Span upd_reads[] = {{a->order, (size_t)a->n_active * 4}, {a->step_idx, in4}, {a->scale, in4},
                              {a->uncond_row, in4}, {a->cond_row, in4}, {a->sigmas, (size_t)a->num_sigmas * 4},
                              {a->x_out, xbytes}, {a->d, dbytes}};
    for (const Span& w : writes)
        for (const Span& r : upd_reads)
            if (w.p && r.p && r.bytes && any_overlap(w.p, w.bytes, r.p, r.bytes))
                return fail(BCG_EINVAL, "%s: the plan's outputs overlap arrays of the update", who);
    const Span plan_reads[] = {{d->step_in, in4}, {d->bucket_cfg, nb4}, {d->cfg_override, d->cfg_override ? in4 : 0},
                               {d->covered, d->covered ? in4 : 0}};
    for (const Span& r : plan_reads)
        if (r.p && r.bytes && (any_overlap(r.p, r.bytes, a->x_out, xbytes) ||
                               (dbytes && any_overlap(r.p, r.bytes, a->d, dbytes))))
            return fail(BCG_EINVAL, "%s: the plan's inputs overlap the update's outputs", who);
    if (!L.launch) {  // nothing to update: the plan alone
        const StepParams p = plan_only_params(n, d);
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream), p);
        return hip_status(hipGetLastError(), "guided_step_rows_dplan: launch");
    }
    L.p.plan = plan_only_params(n, d);
    L.p.plan_block = (int)((int64_t)L.p.n_active * L.p.tiles);
    return rows_launch(L, stream, "guided_step_rows_dplan: launch");
}

extern "C" int latent_init(int n, int C, int H, int W, int dtype, const float* noise, const void* latent,
                           const float* sigmas, int num_sigmas, const int32_t* step_idx, void* x_out,
                           void* stream) {
    bcg::clear_error();
    if (n < 0 || C < 1 || H < 1 || W < 1) return fail(BCG_ESHAPE, "latent_init: bad shape");
    if (dtype != BCG_F32 && dtype != BCG_BF16) return fail(BCG_EDTYPE, "latent_init: unknown dtype %d", dtype);
    if (num_sigmas < 1) return fail(BCG_EINVAL, "latent_init: num_sigmas < 1");
    if (n == 0) return BCG_OK;
    if (!noise || !sigmas || !step_idx || !x_out) return fail(BCG_EINVAL, "latent_init: NULL device pointer");
    const int64_t HW = (int64_t)H * W;
    const int64_t total = (int64_t)n * C * HW;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool vec = HW % 8 == 0 && aligned16(noise) && aligned16(x_out) && (!latent || aligned16(latent));
    const int block = 256;
    if (dtype == BCG_BF16) {
        const bf16_t* lt = static_cast<const bf16_t*>(latent);
        bf16_t* o = static_cast<bf16_t*>(x_out);
        if (vec) hipLaunchKernelGGL((latent_init_kernel<bf16_t, 8>), dim3(grid_for(total / 8, block)), dim3(block), 0, st, n, C, HW, noise, lt, sigmas, num_sigmas, step_idx, o);
        else hipLaunchKernelGGL((latent_init_kernel<bf16_t, 1>), dim3(grid_for(total, block)), dim3(block), 0, st, n, C, HW, noise, lt, sigmas, num_sigmas, step_idx, o);
    } else {
        const float* lt = static_cast<const float*>(latent);
        float* o = static_cast<float*>(x_out);
        if (vec) hipLaunchKernelGGL((latent_init_kernel<float, 4>), dim3(grid_for(total / 4, block)), dim3(block), 0, st, n, C, HW, noise, lt, sigmas, num_sigmas, step_idx, o);
        else hipLaunchKernelGGL((latent_init_kernel<float, 1>), dim3(grid_for(total, block)), dim3(block), 0, st, n, C, HW, noise, lt, sigmas, num_sigmas, step_idx, o);
    }
    return hip_status(hipGetLastError(), "latent_init: launch");
}

extern "C" int mask_blend(int n, int C, int H, int W, int dtype, const void* a, const void* b,
                          const float* mask, int mask_per_sample, void* out, void* stream) {
    bcg::clear_error();
    if (n < 0 || C < 1 || H < 1 || W < 1) return fail(BCG_ESHAPE, "mask_blend: bad shape");
    if (dtype != BCG_F32 && dtype != BCG_BF16) return fail(BCG_EDTYPE, "mask_blend: unknown dtype %d", dtype);
    if (mask_per_sample != 0 && mask_per_sample != 1) return fail(BCG_EINVAL, "mask_blend: mask_per_sample must be 0 or 1");
    if (n == 0) return BCG_OK;
    if (!a || !b || !mask || !out) return fail(BCG_EINVAL, "mask_blend: NULL device pointer");
    const int64_t HW = (int64_t)H * W;
    const int64_t total = (int64_t)n * C * HW;
    const size_t bytes = (size_t)total * elem_size(dtype);
    if (partial_overlap(a, out, bytes) || partial_overlap(b, out, bytes))
        return fail(BCG_EINVAL, "mask_blend: out partially overlaps an input");
    const int64_t ms = mask_per_sample ? HW : 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int block = 256;
    if (dtype == BCG_BF16) {
        const bool vec = HW % 8 == 0 && aligned16(a) && aligned16(b) && aligned16(mask) && aligned16(out);
        auto A = static_cast<const bf16_t*>(a); auto B = static_cast<const bf16_t*>(b); auto O = static_cast<bf16_t*>(out);
        if (vec) hipLaunchKernelGGL((mask_blend_kernel<bf16_t, 8>), dim3(grid_for(total / 8, block)), dim3(block), 0, st, n, C, HW, A, B, mask, ms, O);
        else hipLaunchKernelGGL((mask_blend_kernel<bf16_t, 1>), dim3(grid_for(total, block)), dim3(block), 0, st, n, C, HW, A, B, mask, ms, O);
    } else {
        const bool vec = HW % 4 == 0 && aligned16(a) && aligned16(b) && aligned16(mask) && aligned16(out);
        auto A = static_cast<const float*>(a); auto B = static_cast<const float*>(b); auto O = static_cast<float*>(out);
        if (vec) hipLaunchKernelGGL((mask_blend_kernel<float, 4>), dim3(grid_for(total / 4, block)), dim3(block), 0, st, n, C, HW, A, B, mask, ms, O);
        else hipLaunchKernelGGL((mask_blend_kernel<float, 1>), dim3(grid_for(total, block)), dim3(block), 0, st, n, C, HW, A, B, mask, ms, O);
    }
    return hip_status(hipGetLastError(), "mask_blend: launch");
}

extern "C" int area_accumulate(int n, int C, int H, int W, int feather, int max_regions,
                               const float* region_pred, int64_t pred_elems, const int64_t* region_off,
                               const int32_t* region_count, const int32_t* region_box,
                               const float* region_strength, const float* fallback, float* cond_out,
                               float* wsum_out, void* stream) {
    bcg::clear_error();
    if (n < 0 || C < 1 || H < 1 || W < 1) return fail(BCG_ESHAPE, "area_accumulate: bad shape");
    if (max_regions < 1 || max_regions > BCG_MAX_REGIONS)
        return fail(BCG_EINVAL, "area_accumulate: max_regions %d not in [1, %d]", max_regions, BCG_MAX_REGIONS);
    if (feather < 0 || feather > BCG_MAX_FEATHER) return fail(BCG_EINVAL, "area_accumulate: feather out of range");
    if (pred_elems < 0) return fail(BCG_EINVAL, "area_accumulate: pred_elems < 0");
    if (n == 0) return BCG_OK;
    if (!region_pred || !region_off || !region_count || !region_box || !region_strength || !cond_out)
        return fail(BCG_EINVAL, "area_accumulate: NULL device pointer");
    const int64_t HW = (int64_t)H * W;
    if (HW > (int64_t(1) << 30)) return fail(BCG_ESHAPE, "area_accumulate: H*W too large");
    const int F = std::max(feather, 1);
    const float inv_f4 = 1.0f / float(F * F * F * F);
    const int block = 256;
    const int tiles = (int)((HW + block - 1) / block);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(area_accumulate_kernel, dim3((unsigned)((int64_t)n * tiles)), dim3(block), 0, st, n, C, H, W,
                       F, inv_f4, max_regions, region_pred, pred_elems, region_off, region_count, region_box,
                       region_strength, fallback, cond_out, wsum_out, tiles);
    return hip_status(hipGetLastError(), "area_accumulate: launch");
}
