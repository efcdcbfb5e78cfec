// Native sampler loop with no interpreter in between launches.
//   Host plans: per-step plan build, staging and upload, then the launch.
//   Plan uploads run on the compute stream, or on a copy stream of the loop's
//   own (default priority) where the compute stream waits on the upload's
//   event and an upload into a device row waits for the kernel that last
//   read that row.
//   Device plans: one guided_step_dplan per launch, which builds the plan
//   and advances the step indices on the device; optionally replays of a
//   captured graph of G launches.
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
    hipEvent_t t_ev[2] = {nullptr, nullptr};  // the pair bracketing a timed run
    int32_t last_replayed = 0;        // launches of the last run inside graph replays
    int32_t last_direct = 0;          // launches of the last run launched directly
    // host scratch of the plan outputs that do not go to the device
    std::vector<int32_t> bucket_id, cond_row, bucket_count, bucket_offset, uncond_offset;
    std::vector<int32_t> region_box;
    std::vector<int64_t> region_off;
    std::vector<uint8_t> covered;     // per-sample coverage, computed once
    std::vector<uint16_t> sets;       // coverage of every region subset (validity ranges)
    // device plans
    int64_t k_next = 0;               // launches done since the last restart
    std::vector<int32_t> t0;          // initial step indices (from start)
    std::vector<float> rec0;          // their sample records (with dev_records)
    std::vector<int32_t> q0;          // continuous batching: slot s holds request s, next = n
    // graph g replays launches k .. k+G-1 for any k = g (mod 2*replicas): one
    // per phase of the buffer pattern, so a replay can start at any launch
    std::vector<hipGraph_t> graph;
    std::vector<hipGraphExec_t> graph_exec;
};

namespace {

int hip_ok(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(BCG_EHIP, "%s: %s", what, hipGetErrorString(e));
    return BCG_OK;
}

// Validates the device-plan launch template without launching anything.
int check_dplan(bcg_loop* L, const char* who) {
    bcg_step_args a = L->d.step;
    a.order = nullptr;
    a.step_idx = nullptr;
    a.scale = nullptr;
    a.uncond_row = nullptr;
    const bcg_device_plan& d = L->d.dplan;
    if (d.steps < 1 || d.steps > BCG_MAX_DEVICE_STEPS || d.num_buckets > BCG_MAX_DEVICE_BUCKETS)
        return fail(BCG_EINVAL, "%s: device plans need steps <= %d and num_buckets <= %d", who,
                    BCG_MAX_DEVICE_STEPS, BCG_MAX_DEVICE_BUCKETS);
    if (a.num_sigmas < d.steps + 1) return fail(BCG_EINVAL, "%s: num_sigmas < steps + 1", who);
    if (a.stats) return fail(BCG_EINVAL, "%s: stats need host plans", who);
    if (a.n > 0 && !d.bucket_cfg) return fail(BCG_EINVAL, "%s: dplan.bucket_cfg is NULL", who);
    if (a.max_regions > 0 && a.region_count && !d.covered && !(d.region_range && d.covered_sets))
        return fail(BCG_EINVAL, "%s: a step with regions needs dplan.covered (or covered_sets with ranges)", who);
    return BCG_OK;
}

// Writes the initial step indices (and sigma pairs) into buffer 0 of every
// replica, in order on `st` (the sources are the loop's own host copies,
// which never change).
int reset_steps(bcg_loop* L, hipStream_t st) {
    const int n = L->d.plan.n;
    for (int r = 0; r < L->d.replicas && n > 0; ++r) {
        int rc = hip_ok(hipMemcpyAsync(L->d.dev_steps + size_t(2 * r) * n, L->t0.data(),
                                       sizeof(int32_t) * size_t(n), hipMemcpyHostToDevice, st),
                        "bcg_loop: step index upload");
        if (rc) return rc;
        if (L->d.dev_records) {
            rc = hip_ok(hipMemcpyAsync(L->d.dev_records + size_t(2 * r) * n * 4, L->rec0.data(),
                                       sizeof(float) * 4 * size_t(n), hipMemcpyHostToDevice, st),
                        "bcg_loop: record upload");
            if (rc) return rc;
        }
        if (L->d.queue_len > 0) {
            const size_t qn = size_t(n) + 1 + size_t(L->d.join_front);
            rc = hip_ok(hipMemcpyAsync(L->d.dev_queue + size_t(2 * r) * qn, L->q0.data(), sizeof(int32_t) * qn,
                                       hipMemcpyHostToDevice, st),
                        "bcg_loop: queue upload");
            if (rc) return rc;
        }
    }
    L->k_next = 0;
    return BCG_OK;
}

// Launch k of a device-plan loop (replica k mod R, its own launch k / R).
int launch_dplan(bcg_loop* L, int64_t k, hipStream_t st) {
    const bcg_loop_desc& d = L->d;
    const int n = d.plan.n;
    const int64_t r = k % d.replicas, m = k / d.replicas;
    bcg_step_args a = d.step;
    if (d.replicas > 1) {
        a.x = static_cast<const char*>(a.x) + r * d.replica_stride;
        a.x_out = static_cast<char*>(a.x_out) + r * d.replica_stride;
    }
    a.order = nullptr;
    a.step_idx = nullptr;
    a.scale = nullptr;
    a.uncond_row = nullptr;
    bcg_device_plan dp = d.dplan;
    dp.step_in = d.dev_steps + size_t(2 * r + (m & 1)) * n;
    dp.step_out = d.dev_steps + size_t(2 * r + ((m + 1) & 1)) * n;
    if (d.dev_records) {
        dp.record_in = d.dev_records + size_t(2 * r + (m & 1)) * n * 4;
        dp.record_out = d.dev_records + size_t(2 * r + ((m + 1) & 1)) * n * 4;
    } else {
        dp.record_in = nullptr;
        dp.record_out = nullptr;
    }
    if (d.queue_len > 0) {
        const size_t qn = size_t(n) + 1 + size_t(d.join_front);
        int32_t* qi = d.dev_queue + size_t(2 * r + (m & 1)) * qn;
        int32_t* qo = d.dev_queue + size_t(2 * r + ((m + 1) & 1)) * qn;
        dp.queue_len = d.queue_len;
        dp.queue_ring = d.queue_ring;
        dp.noise = d.noise;
        dp.slot_req_in = qi;
        dp.slot_req_out = qo;
        dp.queue_in = qi + n;
        dp.queue_out = qo + n;
        dp.join_front = d.join_front;
        dp.join_in = d.join_front > 0 ? qi + n + 1 : nullptr;
        dp.join_out = d.join_front > 0 ? qo + n + 1 : nullptr;
    }
    return guided_step_dplan(&a, &dp, st);
}

// Captures, for each phase g of the buffer pattern (period 2*replicas),
// launches g .. g+G-1 into a graph on the loop's own stream; nothing runs
// until one is launched.  A launch's buffers depend on k only through
// k mod (2*replicas), so graph g replays launches k .. k+G-1 of any
// k = g (mod 2*replicas).
int build_graphs(bcg_loop* L) {
    const int G = L->d.graph_launches;
    const int period = 2 * L->d.replicas;
    L->graph.assign(size_t(period), nullptr);
    L->graph_exec.assign(size_t(period), nullptr);
    for (int ph = 0; ph < period; ++ph) {
        int rc = hip_ok(hipStreamBeginCapture(L->copy, hipStreamCaptureModeThreadLocal), "bcg_loop: begin capture");
        if (rc) return rc;
        int rc_launch = BCG_OK;
        for (int k = ph; k < ph + G && rc_launch == BCG_OK; ++k) rc_launch = launch_dplan(L, k, L->copy);
        hipGraph_t g = nullptr;
        rc = hip_ok(hipStreamEndCapture(L->copy, &g), "bcg_loop: end capture");
        if (rc_launch || rc) {
            if (g) (void)hipGraphDestroy(g);
            return rc_launch ? rc_launch : rc;
        }
        L->graph[size_t(ph)] = g;
        rc = hip_ok(hipGraphInstantiate(&L->graph_exec[size_t(ph)], g, nullptr, nullptr, 0),
                    "bcg_loop: graph instantiate");
        if (rc) {
            L->graph_exec[size_t(ph)] = nullptr;
            return rc;
        }
        // the graph's first replay then needs no upload of its own
        rc = hip_ok(hipGraphUpload(L->graph_exec[size_t(ph)], L->copy), "bcg_loop: graph upload");
        if (rc) return rc;
    }
    return hip_ok(hipStreamSynchronize(L->copy), "bcg_loop: graph upload");
}

// bcg_loop_run with device plans.
int run_device(bcg_loop* L, int k0, int count, hipStream_t st) {
    const bcg_loop_desc& d = L->d;
    int rc = BCG_OK;
    if (k0 == 0 && L->k_next != 0) {
        rc = reset_steps(L, st);
        if (rc) return rc;
    } else if (k0 != L->k_next) {
        return fail(BCG_EINVAL, "bcg_loop_run: device plans continue at launch %lld (or restart at 0), not %d",
                    (long long)L->k_next, k0);
    }
    const int G = d.graph_launches;
    const int64_t period = 2 * int64_t(d.replicas);
    int64_t k = k0;
    int j = 0;
    while (j < count) {
        const bool replay = !L->graph_exec.empty() && G > 0 && count - j >= G;
        const int span = replay ? G : 1;
        if (replay) {
            rc = hip_ok(hipGraphLaunch(L->graph_exec[size_t(k % period)], st), "bcg_loop_run: graph launch");
        } else {
            rc = launch_dplan(L, k, st);
        }
        if (rc) return rc;
        (replay ? L->last_replayed : L->last_direct) += span;
        k += span;
        j += span;
        L->k_next = k;
    }
    return BCG_OK;
}

// bcg_loop_run with host plans.
int run_host(bcg_loop* L, int k0, int count, hipStream_t st) {
    const bcg_loop_desc& d = L->d;
    const int n = d.plan.n, steps = d.plan.steps, P = d.upload_batch;
    hipStream_t up = d.async_upload ? L->copy : st;
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
                long long t = (long long)d.start[i] + (k + q) / d.replicas;
                if (d.wrap && t >= 0) t %= steps;
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
            rc = guided_step(&a, st);
            if (rc) return rc;
            ++L->last_direct;
        }
        if (d.async_upload) {
            rc = hip_ok(hipEventRecord(L->use_ev[size_t(g)], st), "bcg_loop_run: event record");
            if (rc) return rc;
        }
    }
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
    if (n > 0 && (!desc->start || (!desc->device_plan && (!desc->host_slab || !desc->dev_slab))))
        return fail(BCG_EINVAL, "bcg_loop_create: NULL start/staging pointer");
    if (desc->step.n != n) return fail(BCG_ESHAPE, "bcg_loop_create: step.n != plan.n");
    if (desc->step.max_regions != R) return fail(BCG_EINVAL, "bcg_loop_create: step/plan max_regions differ");
    if (desc->replicas < 1 || (desc->replicas > 1 && desc->replica_stride <= 0))
        return fail(BCG_EINVAL, "bcg_loop_create: replicas must be >= 1 with a positive stride");
    if (desc->device_plan != 0 && desc->device_plan != 1)
        return fail(BCG_EINVAL, "bcg_loop_create: device_plan must be 0 or 1");
    if (!desc->device_plan &&
        (desc->upload_batch < 1 || desc->upload_batch > 64 || desc->rows % desc->upload_batch != 0))
        return fail(BCG_EINVAL, "bcg_loop_create: upload_batch %d must be in [1, 64] and divide rows %d",
                    desc->upload_batch, desc->rows);
    if (desc->queue_len != 0) {
        if (!desc->device_plan || !desc->dev_records || !desc->dev_queue || !desc->noise)
            return fail(BCG_EINVAL, "bcg_loop_create: continuous batching needs device plans, dev_records, "
                        "dev_queue and noise");
        if (desc->queue_len < n || desc->wrap)
            return fail(BCG_EINVAL, "bcg_loop_create: continuous batching needs queue_len >= n and wrap = 0");
        if (desc->join_front < 0 || desc->join_front > n)
            return fail(BCG_EINVAL, "bcg_loop_create: join_front %d not in [0, n]", desc->join_front);
        for (int i = 0; i < n; ++i)
            if (desc->start[i] < 0 || desc->start[i] >= desc->plan.steps)
                return fail(BCG_EINVAL, "bcg_loop_create: start[%d] = %d not in [0, steps) (continuous batching)",
                            i, desc->start[i]);
    }
    if (desc->device_plan) {
        if (n > 0 && !desc->dev_steps) return fail(BCG_EINVAL, "bcg_loop_create: dev_steps is NULL");
        if (desc->graph_launches < 0 || desc->graph_launches > 4096)
            return fail(BCG_EINVAL, "bcg_loop_create: graph_launches %d not in [0, 4096]", desc->graph_launches);
    } else if (desc->graph_launches != 0) {
        return fail(BCG_EINVAL, "bcg_loop_create: graph_launches needs device plans");
    }
    auto* L = new bcg_loop();
    L->d = *desc;
    L->row_ev.assign(size_t(desc->rows), nullptr);
    L->use_ev.assign(size_t(desc->rows), nullptr);
    L->row_used.assign(size_t(desc->rows), 0);
    hipError_t rc = hipStreamCreateWithFlags(&L->copy, hipStreamNonBlocking);
    for (int q = 0; q < 2 && rc == hipSuccess; ++q) rc = hipEventCreate(&L->t_ev[q]);
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
    L->sets.assign(size_t(n) + 1, 0xffff);
    if (R > 0 && desc->plan.region_count && !desc->plan.covered && !desc->plan.covered_sets && n > 0) {
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
        po.covered_sets_out = L->sets.data();
        const int rc2 = bcg_plan_build(&pin, &po);
        if (rc2) {
            bcg_loop_destroy(L);
            return rc2;
        }
        if (desc->plan.region_range) L->d.plan.covered_sets = L->sets.data();
        else L->d.plan.covered = L->covered.data();
    }
    if (desc->device_plan) {
        bcg_device_plan& dp = L->d.dplan;
        dp.steps = desc->plan.steps;
        dp.num_buckets = desc->plan.num_buckets;
        dp.wrap = desc->wrap ? 1 : 0;
        L->t0.resize(size_t(n));
        for (int i = 0; i < n; ++i) {
            long long t = desc->start[i];
            if (desc->wrap && t >= 0) t %= desc->plan.steps;
            L->t0[size_t(i)] = int32_t(t);
        }
        if (desc->dev_records && n > 0) {  // the records of t0: host plan + schedule
            const int ns = desc->step.num_sigmas;
            if (ns < 1 || !desc->step.sigmas) {
                bcg_loop_destroy(L);
                return fail(BCG_EINVAL, "bcg_loop_create: dev_records needs step.sigmas");
            }
            const size_t nsz = size_t(ns);
            std::vector<float> sg(nsz);
            int rc3 = hip_ok(hipMemcpy(sg.data(), desc->step.sigmas, sizeof(float) * size_t(ns),
                                       hipMemcpyDeviceToHost), "bcg_loop_create: schedule read");
            if (rc3) {
                bcg_loop_destroy(L);
                return rc3;
            }
            std::vector<int32_t> bid(size_t(n) + 1), ur(size_t(n) + 1), cr(size_t(n) + 1), ord(size_t(n) + 1);
            std::vector<float> scl(size_t(n) + 1);
            std::vector<int32_t> rv(size_t(n) + 1);
            bcg_plan_in pin = L->d.plan;
            pin.step_idx = L->t0.data();
            bcg_plan_out po{};
            po.bucket_id = bid.data();
            po.scale = scl.data();
            po.uncond_row = ur.data();
            po.cond_row = cr.data();
            po.order = ord.data();
            po.bucket_count = L->bucket_count.data();
            po.bucket_offset = L->bucket_offset.data();
            po.uncond_offset = L->uncond_offset.data();
            po.region_valid = rv.data();
            L->rec0.assign(4 * size_t(n), 0.0f);
            rc3 = bcg_plan_build(&pin, &po);
            if (rc3 == BCG_OK)
                rc3 = bcg_plan_records(n, desc->plan.steps, L->t0.data(), scl.data(), ur.data(),
                                       L->d.plan.region_range ? rv.data() : nullptr, sg.data(), ns,
                                       L->rec0.data());
            if (rc3) {
                bcg_loop_destroy(L);
                return rc3;
            }
            if (desc->queue_len > 0) {  // every slot's first request joins at the first launch
                const int J = desc->join_front;
                L->q0.assign(size_t(n) + 1 + size_t(J), -1);
                for (int i = 0; i < n; ++i) {
                    L->q0[size_t(i)] = i;
                    uint32_t fl;
                    std::memcpy(&fl, &L->rec0[size_t(i) * 4 + 3], 4);
                    fl |= 64u | (uint32_t(i) << 8) | (i < J ? 128u : 0u);  // the first J go to the front groups
                    std::memcpy(&L->rec0[size_t(i) * 4 + 3], &fl, 4);
                }
                L->q0[size_t(n)] = n;
                for (int q = 0; q < J; ++q) L->q0[size_t(n) + 1 + size_t(q)] = q;
            }
        }
        // Check the launch template once with the first launch's pointers.
        dp.step_in = desc->dev_steps;
        dp.step_out = desc->dev_steps + n;
        int rc2 = check_dplan(L, "bcg_loop_create");
        if (rc2 == BCG_OK) rc2 = reset_steps(L, nullptr);
        if (rc2 == BCG_OK) rc2 = hip_ok(hipStreamSynchronize(nullptr), "bcg_loop_create: step index upload");
        if (rc2 == BCG_OK && desc->graph_launches > 0 && n > 0) rc2 = build_graphs(L);
        if (rc2) {
            bcg_loop_destroy(L);
            return rc2;
        }
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
    for (auto e : L->graph_exec)
        if (e) (void)hipGraphExecDestroy(e);
    for (auto g : L->graph)
        if (g) (void)hipGraphDestroy(g);
    delete L;
    return BCG_OK;
}

extern "C" int bcg_loop_run(bcg_loop* L, int k0, int count, void* stream, float* kernel_ms) {
    bcg::clear_error();
    if (!L) return fail(BCG_EINVAL, "bcg_loop_run: NULL loop");
    if (count < 0 || k0 < 0) return fail(BCG_EINVAL, "bcg_loop_run: negative k0/count");
    hipStream_t st = static_cast<hipStream_t>(stream);
    L->last_replayed = L->last_direct = 0;
    int rc = BCG_OK;
    if (kernel_ms) {
        *kernel_ms = 0.0f;
        rc = hip_ok(hipEventRecord(L->t_ev[0], st), "bcg_loop_run: event record");
        if (rc) return rc;
    }
    rc = L->d.device_plan ? run_device(L, k0, count, st) : run_host(L, k0, count, st);
    if (rc || !kernel_ms) return rc;
    rc = hip_ok(hipEventRecord(L->t_ev[1], st), "bcg_loop_run: event record");
    if (rc == BCG_OK) rc = hip_ok(hipEventSynchronize(L->t_ev[1]), "bcg_loop_run: timing wait");
    float ms = 0.0f;
    if (rc == BCG_OK) rc = hip_ok(hipEventElapsedTime(&ms, L->t_ev[0], L->t_ev[1]), "bcg_loop_run: elapsed");
    if (rc == BCG_OK && count > 0) *kernel_ms = ms / float(count);
    return rc;
}

extern "C" int bcg_loop_last_run(const bcg_loop* L, int32_t* replayed, int32_t* direct) {
    bcg::clear_error();
    if (!L) return fail(BCG_EINVAL, "bcg_loop_last_run: NULL loop");
    if (replayed) *replayed = L->last_replayed;
    if (direct) *direct = L->last_direct;
    return BCG_OK;
}
