// Native sampler loop: per-step plan build, staging, upload and launch with no
// interpreter in between (the loop is launch-rate bound only by this code).
#include <hip/hip_runtime.h>

#include <cstring>
#include <vector>

#include "bcg_common.h"

using bcg::fail;

struct bcg_loop {
    bcg_loop_desc d;
    std::vector<hipEvent_t> row_ev;   // one per staging row: its last upload
    std::vector<char> row_used;
    std::vector<hipEvent_t> t_ev;     // timing pairs, grown on demand
    // host scratch of the plan outputs that do not go to the device
    std::vector<int32_t> bucket_id, cond_row, bucket_count, bucket_offset, uncond_offset;
    std::vector<int32_t> region_box;
    std::vector<int64_t> region_off;
};

namespace {

int hip_ok(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(BCG_EHIP, "%s: %s", what, hipGetErrorString(e));
    return BCG_OK;
}

}  // namespace

extern "C" int bcg_loop_create(const bcg_loop_desc* desc, bcg_loop** out) {
    bcg::clear_error();
    if (!desc || !out) return fail(BCG_EINVAL, "bcg_loop_create: NULL argument");
    const int n = desc->plan.n, R = desc->plan.max_regions, nb = desc->plan.num_buckets;
    if (n < 0 || nb < 1 || nb > BCG_MAX_BUCKETS || R < 0 || R > BCG_MAX_REGIONS)
        return fail(BCG_EINVAL, "bcg_loop_create: bad plan sizes");
    if (desc->rows < 1) return fail(BCG_EINVAL, "bcg_loop_create: rows < 1");
    if (n > 0 && (!desc->start || !desc->host_slab || !desc->dev_slab))
        return fail(BCG_EINVAL, "bcg_loop_create: NULL start/staging pointer");
    if (desc->step.n != n) return fail(BCG_ESHAPE, "bcg_loop_create: step.n != plan.n");
    if (desc->step.max_regions != R) return fail(BCG_EINVAL, "bcg_loop_create: step/plan max_regions differ");
    if (desc->replicas < 1 || (desc->replicas > 1 && desc->replica_stride <= 0))
        return fail(BCG_EINVAL, "bcg_loop_create: replicas must be >= 1 with a positive stride");
    auto* L = new bcg_loop();
    L->d = *desc;
    L->row_ev.assign(size_t(desc->rows), nullptr);
    L->row_used.assign(size_t(desc->rows), 0);
    for (auto& e : L->row_ev) {
        const hipError_t rc = hipEventCreateWithFlags(&e, hipEventDisableTiming);
        if (rc != hipSuccess) {
            bcg_loop_destroy(L);
            return hip_ok(rc, "bcg_loop_create: hipEventCreate");
        }
    }
    L->bucket_id.resize(size_t(n));
    L->cond_row.resize(size_t(n));
    L->bucket_count.resize(size_t(nb));
    L->bucket_offset.resize(size_t(nb) + 1);
    L->uncond_offset.resize(size_t(nb) + 1);
    L->region_box.resize(size_t(n) * R * 4 + 1);
    L->region_off.resize(size_t(n) * R + 1);
    *out = L;
    return BCG_OK;
}

extern "C" int bcg_loop_destroy(bcg_loop* L) {
    if (!L) return BCG_OK;
    for (auto e : L->row_ev)
        if (e) (void)hipEventDestroy(e);
    for (auto e : L->t_ev)
        if (e) (void)hipEventDestroy(e);
    delete L;
    return BCG_OK;
}

extern "C" int bcg_loop_run(bcg_loop* L, int k0, int count, void* stream, float* kernel_ms) {
    bcg::clear_error();
    if (!L) return fail(BCG_EINVAL, "bcg_loop_run: NULL loop");
    if (count < 0 || k0 < 0) return fail(BCG_EINVAL, "bcg_loop_run: negative k0/count");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bcg_loop_desc& d = L->d;
    const int n = d.plan.n, steps = d.plan.steps;
    if (kernel_ms) {
        while (L->t_ev.size() < size_t(2 * count)) {
            hipEvent_t e;
            int rc = hip_ok(hipEventCreate(&e), "bcg_loop_run: hipEventCreate");
            if (rc) return rc;
            L->t_ev.push_back(e);
        }
        *kernel_ms = 0.0f;
    }
    for (int j = 0; j < count; ++j) {
        const int k = k0 + j;
        const int row = k % d.rows;
        if (L->row_used[size_t(row)]) {
            int rc = hip_ok(hipEventSynchronize(L->row_ev[size_t(row)]), "bcg_loop_run: row wait");
            if (rc) return rc;
        }
        int32_t* h = d.host_slab + size_t(row) * 4 * n;
        int32_t* dv = d.dev_slab + size_t(row) * 4 * n;
        for (int i = 0; i < n; ++i) {
            long long t = (long long)d.start[i] + k;
            if (d.wrap) t %= steps;
            h[i] = int32_t(t);
        }
        bcg_plan_in pin = d.plan;
        pin.step_idx = h;
        bcg_plan_out po{};
        po.bucket_id = L->bucket_id.data();
        po.scale = reinterpret_cast<float*>(h + n);
        po.uncond_row = h + 2 * n;
        po.cond_row = L->cond_row.data();
        po.order = h + 3 * n;
        po.bucket_count = L->bucket_count.data();
        po.bucket_offset = L->bucket_offset.data();
        po.uncond_offset = L->uncond_offset.data();
        po.region_box = d.plan.max_regions > 0 ? L->region_box.data() : nullptr;
        po.region_off = d.plan.max_regions > 0 ? L->region_off.data() : nullptr;
        int rc = bcg_plan_build(&pin, &po);
        if (rc) return rc;
        rc = hip_ok(hipMemcpyAsync(dv, h, sizeof(int32_t) * 4 * size_t(n), hipMemcpyHostToDevice, st),
                    "bcg_loop_run: plan upload");
        if (rc) return rc;
        rc = hip_ok(hipEventRecord(L->row_ev[size_t(row)], st), "bcg_loop_run: event record");
        if (rc) return rc;
        L->row_used[size_t(row)] = 1;
        bcg_step_args a = d.step;
        if (d.replicas > 1) {
            const int64_t off = int64_t(k % d.replicas) * d.replica_stride;
            a.x = static_cast<const char*>(a.x) + off;
            a.x_out = static_cast<char*>(a.x_out) + off;
        }
        a.step_idx = dv;
        a.scale = reinterpret_cast<const float*>(dv + n);
        a.uncond_row = dv + 2 * n;
        a.order = dv + 3 * n;
        a.n_active = po.n_active;
        if (kernel_ms) {
            rc = hip_ok(hipEventRecord(L->t_ev[size_t(2 * j)], st), "bcg_loop_run: event record");
            if (rc) return rc;
        }
        rc = guided_step(&a, stream);
        if (rc) return rc;
        if (kernel_ms) {
            rc = hip_ok(hipEventRecord(L->t_ev[size_t(2 * j + 1)], st), "bcg_loop_run: event record");
            if (rc) return rc;
        }
    }
    if (kernel_ms && count > 0) {
        int rc = hip_ok(hipEventSynchronize(L->t_ev[size_t(2 * count - 1)]), "bcg_loop_run: timing wait");
        if (rc) return rc;
        double total = 0.0;
        for (int j = 0; j < count; ++j) {
            float ms = 0.0f;
            rc = hip_ok(hipEventElapsedTime(&ms, L->t_ev[size_t(2 * j)], L->t_ev[size_t(2 * j + 1)]),
                        "bcg_loop_run: elapsed");
            if (rc) return rc;
            total += ms;
        }
        *kernel_ms = float(total);
    }
    return BCG_OK;
}
