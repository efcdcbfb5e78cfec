// Native sampler loop: per-step plan build, staging, upload and launch with no
// interpreter in between.  Plan uploads run on a copy stream of the loop's own
// (default priority) so they overlap the previous step's kernel; the compute
// stream waits on the upload's event, and an upload into a device row waits
// for the kernel that last read that row.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "bcg_common.h"

using bcg::fail;

struct bcg_loop {
    bcg_loop_desc d;
    hipStream_t copy = nullptr;       // plan uploads
    std::vector<hipEvent_t> row_ev;   // per staging row: its last upload done
    std::vector<hipEvent_t> use_ev;   // per staging row: the last kernel reading it done
    std::vector<char> row_used;
    std::vector<hipEvent_t> t_ev;     // timing pairs, grown on demand
    // host scratch of the plan outputs that do not go to the device
    std::vector<int32_t> bucket_id, cond_row, bucket_count, bucket_offset, uncond_offset;
    std::vector<int32_t> region_box;
    std::vector<int64_t> region_off;
    std::vector<uint8_t> covered;     // per-sample coverage, computed once
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
    if (desc->timing_every < 1) return fail(BCG_EINVAL, "bcg_loop_create: timing_every must be >= 1");
    if (desc->upload_batch < 1 || desc->upload_batch > 64 || desc->rows % desc->upload_batch != 0)
        return fail(BCG_EINVAL, "bcg_loop_create: upload_batch %d must be in [1, 64] and divide rows %d",
                    desc->upload_batch, desc->rows);
    auto* L = new bcg_loop();
    L->d = *desc;
    L->row_ev.assign(size_t(desc->rows), nullptr);
    L->use_ev.assign(size_t(desc->rows), nullptr);
    L->row_used.assign(size_t(desc->rows), 0);
    hipError_t rc = hipStreamCreateWithFlags(&L->copy, hipStreamNonBlocking);
    for (size_t r = 0; rc == hipSuccess && r < L->row_ev.size(); ++r) {
        rc = hipEventCreateWithFlags(&L->row_ev[r], hipEventDisableTiming);
        if (rc == hipSuccess) rc = hipEventCreateWithFlags(&L->use_ev[r], hipEventDisableTiming);
    }
    if (rc != hipSuccess) {
        bcg_loop_destroy(L);
        return hip_ok(rc, "bcg_loop_create: stream/event creation");
    }
    L->bucket_id.resize(size_t(n));
    L->cond_row.resize(size_t(n));
    L->bucket_count.resize(size_t(nb));
    L->bucket_offset.resize(size_t(nb) + 1);
    L->uncond_offset.resize(size_t(nb) + 1);
    L->region_box.resize(size_t(n) * R * 4 + 1);
    L->region_off.resize(size_t(n) * R + 1);
    L->covered.assign(size_t(n) + 1, 1);
    // Boxes and coverage depend on the conds only: derive the coverage flags
    // once, so each step's plan is the O(n) bucket work alone.
    if (R > 0 && desc->plan.region_count && !desc->plan.covered && n > 0) {
        const size_t nn = size_t(n);
        std::vector<int32_t> t0(nn, 0), sc(nn), ur(nn), ord(nn);
        std::vector<float> scale(nn);
        bcg_plan_in pin = desc->plan;
        pin.step_idx = t0.data();
        bcg_plan_out po{};
        po.bucket_id = sc.data();
        po.scale = scale.data();
        po.uncond_row = ur.data();
        po.cond_row = L->cond_row.data();
        po.order = ord.data();
        po.bucket_count = L->bucket_count.data();
        po.bucket_offset = L->bucket_offset.data();
        po.uncond_offset = L->uncond_offset.data();
        po.covered_out = L->covered.data();
        const int rc2 = bcg_plan_build(&pin, &po);
        if (rc2) {
            bcg_loop_destroy(L);
            return rc2;
        }
        L->d.plan.covered = L->covered.data();
    }
    *out = L;
    return BCG_OK;
}

extern "C" int bcg_loop_destroy(bcg_loop* L) {
    if (!L) return BCG_OK;
    if (L->copy) (void)hipStreamSynchronize(L->copy);
    for (auto e : L->row_ev)
        if (e) (void)hipEventDestroy(e);
    for (auto e : L->use_ev)
        if (e) (void)hipEventDestroy(e);
    if (L->copy) (void)hipStreamDestroy(L->copy);
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
    const int n = d.plan.n, steps = d.plan.steps, P = d.upload_batch;
    hipStream_t up = d.async_upload ? L->copy : st;
    const int every = d.timing_every;
    const int n_timed = (count + every - 1) / every;
    if (kernel_ms) {
        while (L->t_ev.size() < size_t(2 * n_timed)) {
            hipEvent_t e;
            int rc = hip_ok(hipEventCreate(&e), "bcg_loop_run: hipEventCreate");
            if (rc) return rc;
            L->t_ev.push_back(e);
        }
        *kernel_ms = 0.0f;
    }
    const size_t row_elems = 4 * size_t(n);
    int j = 0;
    while (j < count) {
        // One chunk: launches k .. k+m-1, all inside one aligned group of P rows.
        const int k = k0 + j;
        const int row0 = k % d.rows;
        const int m = std::min(count - j, P - (row0 % P));
        const int g = row0 / P;  // upload group (rows g*P .. g*P+P-1)
        if (L->row_used[size_t(g)]) {
            // the host rows are free once the group's previous copy is done; the
            // device rows once the last launch that read them is done
            int rc = hip_ok(hipEventSynchronize(L->row_ev[size_t(g)]), "bcg_loop_run: row wait");
            if (rc) return rc;
            if (d.async_upload) {
                rc = hip_ok(hipStreamWaitEvent(up, L->use_ev[size_t(g)], 0), "bcg_loop_run: row reuse wait");
                if (rc) return rc;
            }
        }
        int n_active[64];
        int32_t* h0 = d.host_slab + size_t(row0) * row_elems;
        int32_t* dv0 = d.dev_slab + size_t(row0) * row_elems;
        for (int q = 0; q < m; ++q) {
            int32_t* h = h0 + size_t(q) * row_elems;
            for (int i = 0; i < n; ++i) {
                long long t = (long long)d.start[i] + (k + q);
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
            const int rc = bcg_plan_build(&pin, &po);
            if (rc) return rc;
            n_active[q] = po.n_active;
        }
        int rc = hip_ok(hipMemcpyAsync(dv0, h0, sizeof(int32_t) * row_elems * size_t(m),
                                       hipMemcpyHostToDevice, up), "bcg_loop_run: plan upload");
        if (rc) return rc;
        rc = hip_ok(hipEventRecord(L->row_ev[size_t(g)], up), "bcg_loop_run: event record");
        if (rc) return rc;
        if (d.async_upload) {
            rc = hip_ok(hipStreamWaitEvent(st, L->row_ev[size_t(g)], 0), "bcg_loop_run: upload wait");
            if (rc) return rc;
        }
        L->row_used[size_t(g)] = 1;
        for (int q = 0; q < m; ++q, ++j) {
            const int kk = k + q;
            const int32_t* dv = dv0 + size_t(q) * row_elems;
            bcg_step_args a = d.step;
            if (d.replicas > 1) {
                const int64_t off = int64_t(kk % d.replicas) * d.replica_stride;
                a.x = static_cast<const char*>(a.x) + off;
                a.x_out = static_cast<char*>(a.x_out) + off;
            }
            a.step_idx = dv;
            a.scale = reinterpret_cast<const float*>(dv + n);
            a.uncond_row = dv + 2 * n;
            a.order = dv + 3 * n;
            a.n_active = n_active[q];
            const bool timed = kernel_ms && j % every == 0;
            if (timed) {
                rc = hip_ok(hipEventRecord(L->t_ev[size_t(2 * (j / every))], st), "bcg_loop_run: event record");
                if (rc) return rc;
            }
            rc = guided_step(&a, stream);
            if (rc) return rc;
            if (timed) {
                rc = hip_ok(hipEventRecord(L->t_ev[size_t(2 * (j / every) + 1)], st), "bcg_loop_run: event record");
                if (rc) return rc;
            }
        }
        if (d.async_upload) {
            rc = hip_ok(hipEventRecord(L->use_ev[size_t(g)], st), "bcg_loop_run: event record");
            if (rc) return rc;
        }
    }
    if (kernel_ms && count > 0) {
        int rc = hip_ok(hipEventSynchronize(L->t_ev[size_t(2 * n_timed - 1)]), "bcg_loop_run: timing wait");
        if (rc) return rc;
        double total = 0.0;
        for (int q = 0; q < n_timed; ++q) {
            float ms = 0.0f;
            rc = hip_ok(hipEventElapsedTime(&ms, L->t_ev[size_t(2 * q)], L->t_ev[size_t(2 * q + 1)]),
                        "bcg_loop_run: elapsed");
            if (rc) return rc;
            total += ms;
        }
        *kernel_ms = float(total / n_timed);
    }
    return BCG_OK;
}
