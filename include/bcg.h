/*
 * bcg.h -- C ABI of libbcg: the per-step guided denoising update of a
 * diffusion sampler with bucketed classifier-free guidance (BCG), for AMD
 * Instinct MI355X (gfx950).
 *
 * Sources of the operations (page title and section):
 *   [S] "12 · Samplers, schedulers and CFG" (ComfyUI guide, sampling chapter):
 *       "sigma sequence", "denoise below 1", "core of CFG", "the cfg = 1
 *       optimisation", "calc_cond_batch()", "inpaint and mask",
 *       "data shapes of one sampling step".
 *   [B] SGLang diffusion BCG write-up (zwxr.cn news 258547): section 2 "BCG
 *       core mechanism" (bucket assignment), section 3 "bucket construction
 *       under tensor parallelism" (BucketPlan, per-bucket offsets, split and
 *       combine, the [uncond_0..uncond_n | cond_0..cond_n] layout), section 4
 *       "debug chain" (plan built in the scheduler before launch, guidance in
 *       fp32 for half-precision storage, norm logging), section 5 (guidance
 *       curve shapes).
 *   [P] "10 · ModelPatcher and weight views" (ComfyUI guide, model-patcher
 *       chapter): "patches record format", "how a weight is patched",
 *       "strength_model and strength_patch", "offset patch".
 *
 * Conventions (all entry points):
 *   - Every function returns an int status: BCG_OK (0) or a negative code.
 *     bcg_last_error() returns a thread-local message for the last failure.
 *   - Arguments are validated before anything is launched; a failed call has
 *     no side effects.  A HIP launch failure is reported as BCG_EHIP.
 *   - The library never allocates, frees, moves or casts caller memory.
 *     "host" arrays are ordinary CPU memory; "device" arrays are GPU memory
 *     (e.g. torch tensor storage), contiguous, row-major as stated.
 *   - Device work is asynchronous on the caller's stream (a hipStream_t,
 *     passed as void*; NULL is the null stream).  Nothing synchronises.
 *   - Latents are [n, C, H, W] contiguous in the storage dtype (BCG_F32 or
 *     BCG_BF16); all arithmetic is fp32, stores round to nearest even.
 */
#ifndef BCG_H
#define BCG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { BCG_OK = 0, BCG_EINVAL = -1, BCG_ESHAPE = -2, BCG_EDTYPE = -3, BCG_EHIP = -4 };
enum { BCG_F32 = 0, BCG_BF16 = 1 };
enum { BCG_EULER = 0, BCG_HEUN = 1 };
enum { BCG_SCHED_LOGLINEAR = 0 };
enum { BCG_CURVE_CONST = 0, BCG_CURVE_LINEAR = 1, BCG_CURVE_FRONT_HIGH = 2, BCG_CURVE_MID_PEAK = 3 };
/* Cache behaviour of the latent streams of guided_step:
 *   BCG_CACHE_KEEP    ordinary loads/stores: the state is expected back soon
 *                     (one batch advanced in place; the 256 MB last-level cache
 *                     can hold it between steps)
 *   BCG_CACHE_STREAM  nontemporal loads/stores: the state will not be read
 *                     again before the caches turn over (several batches served
 *                     round-robin, each larger than the cache) */
enum { BCG_CACHE_KEEP = 0, BCG_CACHE_STREAM = 1 };
/* Calls of a step whose branch outputs come from a model (guided_step_rows). */
enum { BCG_PHASE_EULER = 0, BCG_PHASE_HEUN_PREDICT = 1, BCG_PHASE_HEUN_CORRECT = 2 };

#define BCG_MAX_REGIONS 4    /* regional conds per sample */
#define BCG_MAX_CHANNELS 64  /* latent channels */
#define BCG_MAX_FEATHER 64   /* feather width in latent pixels */
#define BCG_MAX_BUCKETS 4096
#define BCG_MAX_DEVICE_BUCKETS 1024  /* buckets of a device-built plan */
#define BCG_MAX_DEVICE_STEPS (1 << 20)  /* trajectory length of a device-built plan */
#define BCG_MAX_PATCHES 8    /* patches of one weight_patch call */

/* Patch kinds and weight rounding (weight_patch). */
enum { BCG_PATCH_DIFF = 0, BCG_PATCH_LOWRANK = 1 };
enum { BCG_ROUND_NEAREST = 0, BCG_ROUND_STOCHASTIC = 1 };

/* Thread-local message describing the last failed call ("" if none). */
const char* bcg_last_error(void);

/* ABI version of this header (incremented on any layout change). */
int bcg_abi_version(void);

/*
 * sigma_schedule -- [S] "sigma sequence", "denoise below 1".
 * Descending noise levels for `steps` sampler steps.  A base schedule of
 * N = ceil(steps/denoise) points (N = steps when denoise >= 1) evenly spaced
 * in log(sigma) from sigma_max down to sigma_min (endpoints exact), then a
 * terminal 0; the last steps+1 values are written.
 *   kind        BCG_SCHED_LOGLINEAR
 *   sigma_max > sigma_min > 0, steps in [1, 100000], denoise in (0, 1]
 *   sigmas      host float[steps+1], out
 *   base_steps  host int*, out (N), may be NULL
 * Errors: BCG_EINVAL for any argument out of range.
 */
int sigma_schedule(int kind, double sigma_max, double sigma_min, int steps,
                   double denoise, float* sigmas, int* base_steps);

/*
 * sigma_crop -- [S] "denoise below 1" (start_step and last_step crop the
 * sequence further, for staged sampling) and "force_full_denoise" (a cropped
 * sequence that does not end at 0 gets 0 as its last sigma, so the output is
 * fully denoised).  out = sigmas[start_step .. last], last = last_step, or
 * the last index when last_step < 0 or beyond it; with force_full_denoise a
 * nonzero out[count-1] becomes 0.  The cropped sequence is a schedule of
 * count-1 steps (count = 1: nothing to run).
 *   sigmas  host float[num_sigmas], num_sigmas >= 1
 *   out     host float[num_sigmas] (room for the whole sequence), not aliasing sigmas
 *   count   host int*, out
 * Errors: BCG_EINVAL (NULL pointer, num_sigmas < 1, start_step outside
 * [0, last]).
 */
int sigma_crop(const float* sigmas, int num_sigmas, int start_step, int last_step,
               int force_full_denoise, float* out, int* count);

/*
 * bucket_table -- [B] sections 2 and 5.  Guidance scale per bucket from a
 * continuous curve sampled at u = b/(num_buckets-1) (u = 0 for one bucket):
 *   BCG_CURVE_CONST       p0
 *   BCG_CURVE_LINEAR      p0 + (p1 - p0) u
 *   BCG_CURVE_FRONT_HIGH  p0 if u < p2 else p1
 *   BCG_CURVE_MID_PEAK    p0 at both ends, p1 at u = p2 (0 < p2 < 1), linear
 *                         in between: p0 + (p1 - p0) u/p2 for u <= p2, else
 *                         p0 + (p1 - p0) (1 - u)/(1 - p2)
 * Evaluated in double, stored as float.  table: host float[num_buckets], out.
 * Errors: BCG_EINVAL (unknown curve, num_buckets out of [1, BCG_MAX_BUCKETS],
 * non-finite value, mid-peak position outside (0, 1)).
 */
int bucket_table(int curve, double p0, double p1, double p2, int num_buckets,
                 float* table);

/*
 * bucket_bounds -- [B] section 2: the curve is cut at the bucket boundaries
 * and, within a bucket, held constant or linearly interpolated.  Bucket b
 * covers progress [b/num_buckets, (b+1)/num_buckets) (the bucket_id rule),
 * so lo[b] = curve(b/num_buckets) and hi[b] = curve((b+1)/num_buckets) (curves
 * as bucket_table; double, stored as float).  Passed to a plan as bucket_cfg
 * (lo) and bucket_cfg_end (hi), they give the within-bucket interpolation.
 * Errors: as bucket_table.
 */
int bucket_bounds(int curve, double p0, double p1, double p2, int num_buckets,
                  float* lo, float* hi);

/*
 * bcg_plan_build -- [B] section 2 (assign_bucket), section 3 (BucketPlan:
 * per-sample bucket and scale, per-bucket offsets; the [uncond | cond]
 * layout), section 4 stage 3 (the plan is built before launch and is
 * immutable during the step); [S] "the cfg = 1 optimisation", and
 * "calc_cond_batch()" (area fractions -> latent slices).
 *
 * All arrays are host memory.  For every sample i with 0 <= step_idx[i] < steps
 * (active):
 *   bucket_id[i] = min(floor(step_idx[i]*num_buckets/steps), num_buckets-1)
 *                  (exact integer arithmetic)
 *   scale[i]     = cfg_override[i] if given and not NaN, else bucket_cfg[bucket],
 *                  or, with bucket_cfg_end, the within-bucket interpolation
 *                  float(lo + (hi - lo) * f) in double, lo = bucket_cfg[b],
 *                  hi = bucket_cfg_end[b], f = (t*num_buckets - b*steps)/steps
 *   the uncond branch is skipped iff scale[i] == 1.0f and the sample's conds
 *   cover every latent pixel (no regions, or the boxes with strength > 0
 *   cover the frame); otherwise it is kept (uncovered pixels use it).
 *   Validity ranges ([S] "calc_cond_batch()": each cond entry is checked for
 *   the current timestep): with region_range, region r of sample i takes part
 *   in step t iff start <= t/steps < end (double); region_valid[i] gets the
 *   bit mask of those regions and coverage is that of the valid ones (a
 *   sample with regions but none valid is not covered).
 * Layout: cond rows are the active samples stably ordered by (bucket, i) and
 * follow the uncond half; the uncond half is the same order without skipped
 * samples.  order[0..n_active) lists the active samples in that order.
 * Inactive samples: bucket_id = -1, scale = 0, rows = -1.
 * Region boxes (half-open y0,y1,x0,x1) from fractions (fy,fx,fh,fw):
 *   h = clamp(floor(fh*H + 0.5), 1, H); y0 = clamp(floor(fy*H + 0.5), 0, H-h);
 *   same for x.  region_off[i*R + r] is the element offset of region r's
 *   packed [C,h,w] crop (size 0 for r >= region_count[i]); region_off[n*R] is
 *   the total.  Boxes and coverage depend only on the conds, not on the step:
 *   a sampler computes them once (covered_out) and passes them back as
 *   `covered` on every step, which leaves only the O(n) bucket work per step.
 */
typedef struct {
    int32_t n;                       /* samples, >= 0 */
    int32_t steps;                   /* trajectory length, >= 1 */
    int32_t num_buckets;             /* [1, BCG_MAX_BUCKETS] */
    int32_t C, H, W;                 /* latent shape (for region slices) */
    int32_t max_regions;             /* R in [0, BCG_MAX_REGIONS], array stride */
    const float* bucket_cfg;         /* [num_buckets] */
    const int32_t* step_idx;         /* [n] t_i; outside [0, steps) = inactive */
    const float* cfg_override;       /* [n] or NULL; NaN = none; else finite */
    const int32_t* region_count;     /* [n] in [0, R], or NULL (all 0) */
    const double* region_frac;       /* [n][R][4] (fy,fx,fh,fw), or NULL if R == 0 */
    const float* region_strength;    /* [n][R]: 0 or in [1e-30, 1e30], or NULL if R == 0 */
    const uint8_t* covered;          /* [n] or NULL: precomputed coverage flags (1 = the
                                        sample's conds cover the frame), e.g. from an
                                        earlier call's covered_out; when given, region
                                        arrays are not read and region outputs not written */
    const float* bucket_cfg_end;     /* [num_buckets] or NULL: bucket-end scales for the
                                        within-bucket interpolation (bucket_bounds) */
    const double* region_range;      /* [n][R][2] (start, end) progress or NULL (always valid) */
    const uint16_t* covered_sets;    /* [n] or NULL: precomputed coverage of every subset of
                                        regions (bit s: the regions in bit mask s cover the
                                        frame), e.g. an earlier call's covered_sets_out; needed
                                        with region_range when the region arrays are not read */
} bcg_plan_in;

typedef struct {
    int32_t* bucket_id;              /* [n] */
    float* scale;                    /* [n] */
    int32_t* uncond_row;             /* [n] row in the uncond half, -1 = skipped/inactive */
    int32_t* cond_row;               /* [n] row of the full batch (n_uncond + pos), -1 = inactive */
    int32_t* order;                  /* [n] first n_active entries valid */
    int32_t* bucket_count;           /* [num_buckets] active samples per bucket */
    int32_t* bucket_offset;          /* [num_buckets+1] exclusive prefix, cond half */
    int32_t* uncond_offset;          /* [num_buckets+1] exclusive prefix, uncond half */
    int32_t* region_box;             /* [n][R][4] or NULL */
    int64_t* region_off;             /* [n*R+1] or NULL */
    uint8_t* covered_out;            /* [n] or NULL: coverage flags of all regions */
    int32_t n_active;                /* out */
    int32_t n_uncond;                /* out */
    uint16_t* covered_sets_out;      /* [n] or NULL: coverage of every subset of regions */
    int32_t* region_valid;           /* [n] or NULL: regions taking part in this step (bits) */
} bcg_plan_out;

int bcg_plan_build(const bcg_plan_in* in, bcg_plan_out* out);

/*
 * guided_step -- one sampler step of the guided update, fused in one pass
 * over the latent.  [S] "core of CFG", "the cfg = 1 optimisation",
 * "calc_cond_batch()", "inpaint and mask"; [B] section 3 (per-sample scales
 * over a mixed-bucket batch), section 4 (fp32 guidance for bf16 storage).
 *
 * For each sample i = order[j], j < n_active, with t = step_idx[i],
 * sigma = sigmas[t], sigma' = sigmas[t+1], w = scale[i]:
 *   branch predictions (closed-form stand-in denoiser, Gaussian data
 *     N(mu_k, s2)):  D_k(x) = (s2*x + sigma^2*mu_k[c]) / (s2 + sigma^2)
 *   U = D_uncond; C = D_cond, or with regions
 *     C = sum_r w_r(p) D_r / sum_r w_r(p), w_r = strength_r * feather_r(p),
 *     and C = U where no region has weight
 *   pred = C if w == 1, else U + w (C - U)   (U not evaluated if uncond_row[i] < 0)
 *   inpaint: pred = m pred + (1 - m) x_orig
 *   Euler: x' = x + (sigma' - sigma)(x - pred)/sigma;  Heun adds a second
 *   evaluation at the Euler point and averages the slopes; x' = pred when
 *   sigma' = 0.
 * The evaluation order is a fixed sequence of fp32 operations, with fused
 * multiply-adds (one rounding) at fixed places; stores round to the storage
 * dtype.
 *
 * x_out may equal x (in place); otherwise the two must not overlap.  Samples
 * not in order[0..n_active) are neither read nor written.  Entries of order
 * outside [0, n), and samples whose t or t+1 falls outside [0, num_sigmas),
 * are skipped on the device.  Feather: linear ramp of `feather` pixels on
 * each box edge (weight (d+1)/F ... 1), separable in y and x.
 * Stats (optional): stats[i][0..2] = mean over (c, row) of the L2 norm over W
 * of C, U (0 if skipped) and pred (before the inpaint blend), from the first
 * evaluation ([B] section 4 stage 2: norms logged around the guidance); needs
 * a device workspace of guided_step_workspace_size() bytes.  When W is a
 * power-of-two multiple (at most 64) of the 16-byte vector and the arrays are
 * 16-byte aligned, the step computes them itself: the lanes of a latent row
 * sum their squares in a fixed butterfly, each row group writes the sums of
 * its row norms to the workspace, and a second small kernel adds a sample's
 * groups in a fixed order (the step then runs with ordinary loads and stores
 * whatever cache_hint says).  Other shapes take two kernels that read x again
 * before the step.
 * Errors: BCG_ESHAPE (sizes), BCG_EDTYPE (dtype), BCG_EINVAL (NULL pointer,
 * sampler, R > 0 without region arrays, inpaint arrays half given, stats
 * without workspace or with too small a workspace), BCG_EHIP.
 */
typedef struct {
    int32_t n, C, H, W;              /* n >= 0, C in [1, 64], H, W >= 1 */
    int32_t dtype;                   /* BCG_F32 | BCG_BF16: x, x_out, x_orig */
    int32_t sampler;                 /* BCG_EULER | BCG_HEUN */
    int32_t max_regions;             /* R in [0, BCG_MAX_REGIONS]; 0 = no regions */
    int32_t feather;                 /* [0, BCG_MAX_FEATHER] */
    int32_t n_active;                /* entries of order[] to process, [0, n] */
    int32_t num_sigmas;              /* length of sigmas */
    int32_t mask_per_sample;         /* 1: mask [n,1,H,W]; 0: [1,1,H,W] */
    int32_t cache_hint;              /* BCG_CACHE_KEEP | BCG_CACHE_STREAM */
    float s2;                        /* stand-in data variance, > 0 */
    const void* x;                   /* device [n,C,H,W] */
    void* x_out;                     /* device [n,C,H,W] */
    const float* sigmas;             /* device [num_sigmas] */
    const int32_t* order;            /* device [n_active] sample ids */
    const int32_t* step_idx;         /* device [n] */
    const float* scale;              /* device [n] */
    const int32_t* uncond_row;       /* device [n]; < 0 = uncond branch skipped */
    const float* mu_uncond;          /* device [n][C] */
    const float* mu_cond;            /* device [n][C] (samples with 0 regions) */
    const int32_t* region_count;     /* device [n] or NULL when R == 0 */
    const int32_t* region_box;       /* device [n][R][4] y0,y1,x0,x1 */
    const float* region_strength;    /* device [n][R] */
    const float* mu_region;          /* device [n][R][C] */
    const void* x_orig;              /* device [n,C,H,W] or NULL (no inpaint) */
    const float* mask;               /* device mask or NULL (with x_orig) */
    float* stats;                    /* device [n][3] or NULL */
    void* workspace;                 /* device scratch for stats, or NULL */
    size_t workspace_bytes;
    const double* region_range;      /* device [n][R][2] (start, end) progress or NULL: region r
                                        takes part iff start <= t/steps < end (as the plan) */
    int32_t steps;                   /* trajectory length, with region_range */
    int32_t launch_vpt;              /* 0: launch shape chosen by the library; k in [1, 64]:
                                        workgroups of 256 lanes, each lane taking k pixel
                                        vectors (the shape only: results are identical) */
} bcg_step_args;

int guided_step(const bcg_step_args* args, void* stream);

/* Bytes of device workspace guided_step needs for stats at this shape. */
size_t guided_step_workspace_size(int n, int C, int H, int W, int dtype);

/*
 * Device-built plans -- [B] section 2 (assign_bucket), section 3 (BucketPlan
 * and the [uncond | cond] layout) and section 4 stage 3 (the plan of a step
 * is fixed before that step's guidance runs), computed on the GPU from
 * per-sample step indices held in device memory, so a step loop needs no
 * host work and no upload per step (and can be captured in a graph).
 *
 * The plan is the one bcg_plan_build defines, bit for bit: for a sample with
 * 0 <= t < steps, bucket = min(floor(t*num_buckets/steps), num_buckets-1),
 * scale = cfg_override (if given and not NaN) else bucket_cfg[bucket] (or the
 * within-bucket interpolation towards bucket_cfg_end[bucket]), uncond
 * skipped iff scale == 1.0f and covered; stable (bucket, i) order; offsets,
 * rows and totals as in bcg_plan_out.  Coverage is not recomputed on the
 * device: pass the flags bcg_plan_build returned in covered_out (they depend
 * on the conds only).  Region boxes likewise come from bcg_plan_build.
 *
 * Step advance: if step_out is given, step_out[i] = t + 1, reduced modulo
 * steps when wrap is set and t + 1 >= 0 (a sample with a negative index has
 * not joined yet; with wrap, a sample that finished restarts at step 0:
 * continuous batching with every slot refilled).  step_out must not overlap
 * step_in; a loop alternates two buffers.
 *
 * Sample records (four floats per sample): (sigma, sigma', scale, flags) of
 * the sample's step t, with sigma = sigmas[t], sigma' = sigmas[t+1], scale as
 * above and flags the bit pattern of the fourth float: bit 0 = active
 * (0 <= t < steps), bit 1 = uncond branch kept, bits 2..5 = the regions
 * valid at t (all of them without validity ranges); an inactive sample's record
 * is all zero bits.  A step that reads its records needs no load that waits
 * on another (its plan wrote them one launch earlier); they must describe
 * step_in.  bcg_plan_records builds them on the host for a first step.
 *
 * Continuous batching (queue_len > 0; [B] section 3: one batch carries
 * samples of several buckets, section 4 stage 3: the scheduler builds every
 * step's plan): the n samples are slots, each holding a request of a queue of
 * queue_len.  slot_req_in[s] is the request of slot s (-1: empty), step_in[s]
 * its step; every per-sample table (cfg_override, covered, region_range,
 * covered_sets, region_count, and the step's mu / region / x_orig / mask
 * arrays) and `noise` are indexed by request, so a request's regions take
 * part over its own validity ranges of its own progress.
 * The plan (rows, order, ...) is over slots.  For the next step the plan
 * workgroup writes step_out, slot_req_out, record_out and queue_out: a slot
 * whose request takes its last step now (t = steps - 1), and an empty slot,
 * takes the next queued request (freed slots in slot order, requests in
 * queue order from *queue_in), which joins at step 0; with queue_ring the
 * request ids run modulo queue_len (the pool is served over and over), else a
 * slot left without a request gets step -1, request -1 and an all-zero
 * record.  Records then also carry bit 6 = the request joins at this step
 * and bits 8..31 = the request; a joining request's state is built inside
 * guided_step_dplan from noise[r] * sigma (+ the stored x_orig[r] when
 * inpainting, one fused multiply-add), rounded to the storage dtype, then
 * stepped; the slot's previous contents are not read.  Requires records in
 * and out, step_out, the 16-byte vector path and no stats; wrap must be 0.  bcg_plan_records (OR'ing in the join bit and the
 * request) gives the first step's records.
 *
 * The device arrays are not validated (a host plan build validates the same
 * tables): bucket_cfg finite, cfg_override finite or NaN.
 */
typedef struct {
    int32_t steps;                   /* trajectory length, [1, BCG_MAX_DEVICE_STEPS] */
    int32_t num_buckets;             /* [1, BCG_MAX_DEVICE_BUCKETS] */
    int32_t wrap;                    /* 0 | 1, see above */
    const float* bucket_cfg;         /* device [num_buckets] */
    const float* cfg_override;       /* device [n] or NULL; NaN = none */
    const int32_t* covered;          /* device [n] coverage flags, or NULL = all covered
                                        (required when the step has regions) */
    const int32_t* step_in;          /* device [n] t_i of this step */
    int32_t* step_out;               /* device [n] or NULL: the next step's t_i */
    /* the full plan of this step, device arrays, all given or all NULL: */
    int32_t* bucket_id;              /* [n] */
    float* scale;                    /* [n] */
    int32_t* uncond_row;             /* [n] */
    int32_t* cond_row;               /* [n] */
    int32_t* order;                  /* [n] (-1 past n_active) */
    int32_t* bucket_count;           /* [num_buckets] */
    int32_t* bucket_offset;          /* [num_buckets+1] */
    int32_t* uncond_offset;          /* [num_buckets+1] */
    int32_t* totals;                 /* [2]: n_active, n_uncond */
    const float* bucket_cfg_end;     /* device [num_buckets] or NULL (no interpolation) */
    const float* record_in;          /* device [n][4] or NULL: this step's sample records, see
                                        below; guided_step_dplan reads them instead of deriving
                                        sigma, sigma', scale and the uncond decision from step_in */
    float* record_out;               /* device [n][4] or NULL: the records of the next step's
                                        indices (the next step's record_in); needs sigmas */
    const float* sigmas;             /* device [num_sigmas]: the schedule, for record_out
                                        (guided_step_dplan uses its own args->sigmas) */
    int32_t num_sigmas;
    const double* region_range;      /* device [n][R][2] or NULL: validity ranges, as the host
                                        plan (with them covered_sets replaces covered) */
    const uint16_t* covered_sets;    /* device [n]: bcg_plan_build's covered_sets_out */
    const int32_t* region_count;     /* device [n] (with region_range; guided_step_dplan uses
                                        args->region_count) */
    int32_t max_regions;             /* R, the stride of region_range */
    /* continuous batching (see above): */
    int32_t queue_len;               /* 0: off; else the requests of the queue, < 2^24 */
    int32_t queue_ring;              /* 0 | 1: request ids modulo queue_len */
    const float* noise;              /* device fp32 [queue_len, C, H, W] */
    const int32_t* slot_req_in;      /* device [n] request of each slot at this step */
    int32_t* slot_req_out;           /* device [n] ... at the next step */
    const int32_t* queue_in;         /* device [1] next queued request */
    int32_t* queue_out;              /* device [1] ... after this step's refills */
    int32_t join_front;              /* J in [0, n]: the launch starts with J groups of
                                        workgroups that take this step's first J joins,
                                        listed in join_in (-1: none), before the slots' own
                                        (a joining request's step reads its fp32 noise, so it
                                        runs first rather than at the end of the grid); the
                                        plan lists the next step's in join_out, and flags
                                        those records with bit 7 */
    const int32_t* join_in;          /* device [J] */
    int32_t* join_out;               /* device [J] */
} bcg_device_plan;

/*
 * bcg_plan_records -- sample records (see above) of step indices step_idx from
 * a host plan of the same indices (bcg_plan_build's scale, uncond_row and
 * region_valid, which may be NULL: every region valid) and the schedule; all
 * host arrays, records [n][4] out.  Active means
 * 0 <= t < steps and t + 1 < num_sigmas.
 * Errors: BCG_EINVAL (NULL pointer, n < 0, steps < 1, num_sigmas < 1).
 */
int bcg_plan_records(int n, int steps, const int32_t* step_idx, const float* scale,
                     const int32_t* uncond_row, const int32_t* region_valid,
                     const float* sigmas, int num_sigmas, float* records);

/*
 * bcg_plan_device -- the plan of one step for n samples, built by one
 * workgroup on `stream` (and the step advance).  Needs the plan outputs or
 * step_out (or both).
 * Errors: BCG_EINVAL (sizes out of range, NULL table/step_in, outputs half
 * given, nothing to write, step_out overlapping step_in), BCG_EHIP.
 */
int bcg_plan_device(int n, const bcg_device_plan* plan, void* stream);

/*
 * guided_step_dplan -- guided_step whose per-sample step index, scale and
 * uncond decision come from a device-built plan, in the same launch: every
 * sample with 0 <= step_in[i] < steps is advanced (the others are neither
 * read nor written), and one extra workgroup of the launch writes the full
 * plan (if requested) and step_out.  Results are bit-identical to
 * guided_step with the host plan of the same step indices.
 * args: as guided_step, except order, step_idx, scale and uncond_row must be
 * NULL and n_active is ignored; num_sigmas must be >= steps + 1; with regions
 * (max_regions > 0), plan->covered is required.  Stats (optional, as
 * guided_step's) are computed inside the step, which needs W to be a
 * power-of-two multiple, at most 64, of the 16-byte vector (4 fp32 or 8 bf16
 * pixels) and 16-byte aligned arrays (else BCG_EINVAL).
 * Errors: as guided_step and bcg_plan_device.
 */
int guided_step_dplan(const bcg_step_args* args, const bcg_device_plan* plan, void* stream);

/*
 * guided_step_dplan_static -- guided_step_dplan for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): args->workspace must be NULL and
 * workspace_bytes 0, and the statistics' partials (when args->stats is given)
 * go to a scratch array of the library's own, BCG_STATIC_SCRATCH_BYTES on each
 * GPU, part of the library's code object and held until the process ends; no
 * allocation or free is made.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams) race.  Every partial a
 * call reads is written earlier in the same call, so nothing needs clearing
 * between calls.  Results are bit-identical to guided_step_dplan with a
 * workspace.
 * Errors: as guided_step_dplan; BCG_EINVAL when a workspace is given or the
 * partials of this call (n * tiles * row groups * 12 bytes, at most
 * guided_step_workspace_size) exceed BCG_STATIC_SCRATCH_BYTES.
 */
#define BCG_STATIC_SCRATCH_BYTES (4u << 20)
int guided_step_dplan_static(const bcg_step_args* args, const bcg_device_plan* plan, void* stream);

/*
 * guided_step_rows -- the guided update when the branch predictions are
 * materialised by a model: [B] section 3 (the [uncond_0..uncond_m |
 * cond_0..cond_n] batch layout and its per-bucket split and combine, with the
 * uncond half compacted to the samples that need it), [S] "core of CFG",
 * "the cfg = 1 optimisation", "inpaint and mask", "one step may call the
 * model more than steps times" (Heun evaluates the model twice per step).
 *
 * pred holds one model evaluation in the plan's layout: sample i's cond
 * prediction is row cond_row[i], its uncond prediction row uncond_row[i]
 * (bcg_plan_build gives both).  The cond row is the final cond (regional
 * conds accumulated into it beforehand, e.g. by area_accumulate with the
 * uncond prediction as fallback).  For i = order[j], j < n_active,
 * t = step_idx[i], sigma = sigmas[t], sigma' = sigmas[t+1], w = scale[i]:
 *   P = C if w == 1 (no uncond row is read), else U + w (C - U); inpaint:
 *   P = m P + (1 - m) x_orig
 *   BCG_PHASE_EULER: x_out = x + (sigma' - sigma)(x - P)/sigma; P if sigma' = 0
 *   BCG_PHASE_HEUN_PREDICT: d = (x - P)/sigma (fp32, to `d`), x_out = x~ =
 *     x + (sigma' - sigma) d, the point the model is evaluated at next; on a
 *     last step (sigma' = 0) x_out = P and d is not written
 *   BCG_PHASE_HEUN_CORRECT (pred evaluated at x~, sigma'): x~ = x + h d is
 *     recomputed in fp32 from `d`, d' = (x~ - P)/sigma', x_out = x + h (d + d')/2;
 *     on a last step x_out = x_tilde (the predictor's output)
 * The fp32 evaluation order has fused multiply-adds at fixed places (as
 * guided_step); stores round to the storage dtype.
 * Samples whose rows are missing (cond_row outside [0, rows), or w != 1 with
 * uncond_row outside [0, rows)), or whose t or t+1 falls outside
 * [0, num_sigmas), are neither read nor written.  x_out may equal x; d,
 * pred, x_tilde must not overlap x_out.
 * Errors: BCG_ESHAPE, BCG_EDTYPE, BCG_EINVAL (NULL pointer, unknown phase,
 * d missing for Heun, x_tilde missing for the corrector, inpaint arrays half
 * given, overlaps), BCG_EHIP.
 */
typedef struct {
    int32_t n, C, H, W;              /* n >= 0, C >= 1, H, W >= 1 */
    int32_t dtype;                   /* BCG_F32 | BCG_BF16: x, x_out, x_tilde, pred, x_orig */
    int32_t phase;                   /* BCG_PHASE_* */
    int32_t n_active;                /* entries of order[] to process, [0, n] */
    int32_t num_sigmas;              /* length of sigmas */
    int32_t rows;                    /* rows of pred (n_uncond + n_active of the plan) */
    int32_t mask_per_sample;         /* 1: mask [n,1,H,W]; 0: [1,1,H,W] */
    int32_t cache_hint;              /* BCG_CACHE_KEEP | BCG_CACHE_STREAM */
    const void* x;                   /* device [n,C,H,W], the state at sigma */
    void* x_out;                     /* device [n,C,H,W] */
    float* d;                        /* device fp32 [n,C,H,W] (Heun phases), else NULL */
    const void* x_tilde;             /* device [n,C,H,W] (corrector), else NULL */
    const void* pred;                /* device [rows,C,H,W] */
    const float* sigmas;             /* device [num_sigmas] */
    const int32_t* order;            /* device [n_active] */
    const int32_t* step_idx;         /* device [n] */
    const float* scale;              /* device [n] */
    const int32_t* uncond_row;       /* device [n] */
    const int32_t* cond_row;         /* device [n] */
    const void* x_orig;              /* device [n,C,H,W] or NULL (no inpaint) */
    const float* mask;               /* device mask or NULL (with x_orig) */
    int32_t launch_vpt;              /* 0: launch shape chosen by the library; k in [1, 64]:
                                        workgroups of 256 lanes, k pixel vectors per lane */
} bcg_rows_args;

int guided_step_rows(const bcg_rows_args* args, void* stream);

/*
 * guided_step_rows_dplan -- guided_step_rows, and in the same launch the
 * device plan `plan` describes for the same n samples, exactly as
 * bcg_plan_device(args->n, plan) builds it (one extra workgroup of the launch
 * builds it while the others update).  With a model in the loop the plan of
 * step k+1 is due before the model's step-(k+1) forward, which comes after
 * the update of step k: building it in that update's launch ([B] section 3's
 * per-step BucketPlan, here on the device; [S] "calc_cond_batch()" batches the
 * model's rows by that plan) takes its own launch off the step.
 * The two run concurrently, so the plan's outputs (plan table, step_out,
 * record_out) must overlap neither the update's plan arrays (order, step_idx,
 * scale, uncond_row, cond_row), its sigmas, nor x_out or d, and the plan's
 * step_in and tables must not overlap x_out or d; both are checked before the
 * launch.  With n_active == 0 only the plan is built.
 * Errors: as guided_step_rows and bcg_plan_device; BCG_EINVAL for the
 * overlaps above.
 */
int guided_step_rows_dplan(const bcg_rows_args* args, const bcg_device_plan* plan, void* stream);

/*
 * latent_init -- [S] "deterministic noise", "disable_noise": the sampler
 * starts from the latent plus noise at the sample's first sigma,
 *   x_out[i] = latent[i] + noise[i] * sigmas[step_idx[i]]   (fp32, rounded on store)
 * latent (storage dtype) may be NULL (zero).  noise is device fp32
 * [n,C,H,W] (drawn on the host by the caller).  Samples whose step_idx is
 * outside [0, num_sigmas) are not written.
 */
int latent_init(int n, int C, int H, int W, int dtype, const float* noise,
                const void* latent, const float* sigmas, int num_sigmas,
                const int32_t* step_idx, void* x_out, void* stream);

/*
 * area_accumulate -- [S] "calc_cond_batch()": region outputs are accumulated
 * into the full latent by strength and mask and overlaps are normalised by
 * the weight sum.  Gather form (one writer per output element, no atomics).
 *   region_pred  device fp32, packed crops: region r of sample i is [C,h,w]
 *                at region_pred + region_off[i*R + r] (h, w from its box)
 *   cond_out[i,c,y,x] = sum_r wh_r(y,x) * crop_r[c, y-y0_r, x-x0_r], with
 *                wh_r = w_r / sum_r w_r over regions containing the pixel, or
 *                fallback[i,c,y,x] (0 if fallback is NULL) where the sum is 0
 *   wsum_out[i,y,x] = sum_r w_r(y,x)  (optional)
 * Per-pixel weights are the guided_step ones.  Boxes whose crop does not fit
 * between consecutive region_off entries, or past pred_elems, are skipped.
 */
int area_accumulate(int n, int C, int H, int W, int feather, int max_regions,
                    const float* region_pred, int64_t pred_elems,
                    const int64_t* region_off, const int32_t* region_count,
                    const int32_t* region_box, const float* region_strength,
                    const float* fallback, float* cond_out, float* wsum_out,
                    void* stream);

/*
 * mask_blend -- [S] "inpaint and mask": out = m*a + (1 - m)*b with the mask
 * broadcast over channels (mask [n,1,H,W] if mask_per_sample, else
 * [1,1,H,W]); a, b, out in the storage dtype, out may alias a or b.
 */
int mask_blend(int n, int C, int H, int W, int dtype, const void* a, const void* b,
               const float* mask, int mask_per_sample, void* out, void* stream);

/*
 * weight_patch -- one weight with its patches applied: [P] "patches record
 * format" (a patch entry: strength_patch, the patch value, strength_model,
 * an optional offset), "strength_model and strength_patch" (W' =
 * strength_model W + strength_patch dW, dW a low-rank pair or a direct
 * diff), "offset patch" (a patch on a slice of the tensor), "how a weight is
 * patched" (every patch of the weight overlaid in a compute precision, then
 * written back by stochastic rounding or a cast).
 *
 * w and out are device [rows, cols], row-major, in w_dtype and out_dtype.
 * Patch q covers weight rows [offset_q, offset_q + rows_q).  Per element, in
 * fp32 and in patch order:
 *   a = w;  for q covering the row:  a = fma(sp_q, d_q, sm_q * a)
 * with d_q = diff_q[row - offset_q, col] (BCG_PATCH_DIFF), or
 * sum_k up_q[row - offset_q, k] down_q[k, col] (BCG_PATCH_LOWRANK: bf16
 * factors, exact products summed in fp32 on the matrix cores, in an order
 * the kernel chooses).  The store: out = a (BCG_F32), or bf16 of a, by
 * nearest even (BCG_ROUND_NEAREST), or stochastically (BCG_ROUND_STOCHASTIC):
 * 16 random bits r_e are added to a's fp32 bit pattern and the high 16 bits
 * kept (rounds away from zero with probability equal to the dropped
 * fraction; NaN and infinities round to nearest).  r_e of the element with
 * flat index e = row * cols + col is the 16-bit half (e mod 2, low half
 * first) of word (e mod 8) / 2 of Philox4x32-10 (Salmon et al., SC 2011)
 * at counter (low, high word of e / 8, 0, 0) and key (low, high word of
 * seed): a given seed rounds a given element the same way however the
 * weight is tiled or launched.
 *
 * out may equal w (same dtype), in place; it must not otherwise overlap w or
 * any patch tensor.  patches is a host array, read during the call only.
 * Errors: BCG_ESHAPE (rows or cols negative, a patch outside the weight,
 * rank < 1), BCG_EDTYPE (dtype not BCG_F32/BCG_BF16, low-rank factors not
 * bf16), BCG_EINVAL (NULL pointer, num_patches outside [0,
 * BCG_MAX_PATCHES], unknown kind or rounding, overlaps), BCG_EHIP.
 */
typedef struct {
    int32_t kind;                    /* BCG_PATCH_DIFF | BCG_PATCH_LOWRANK */
    int32_t offset;                  /* first weight row covered, >= 0 */
    int32_t rows;                    /* rows covered, >= 0, offset + rows <= weight rows */
    int32_t rank;                    /* low-rank r >= 1 (ignored for a diff) */
    int32_t dtype;                   /* diff: BCG_F32 | BCG_BF16; low-rank: BCG_BF16 */
    float strength_patch;            /* sp */
    float strength_model;            /* sm */
    int32_t reserved;                /* 0 */
    const void* diff;                /* device [rows, cols] (diff), else NULL */
    const void* up;                  /* device bf16 [rows, rank] (low-rank), else NULL */
    const void* down;                /* device bf16 [rank, cols] (low-rank), else NULL */
} bcg_patch;

typedef struct {
    int32_t rows, cols;              /* >= 0 */
    int32_t w_dtype, out_dtype;      /* BCG_F32 | BCG_BF16 */
    int32_t num_patches;             /* [0, BCG_MAX_PATCHES] */
    int32_t rounding;                /* BCG_ROUND_* (bf16 out; ignored for f32) */
    uint64_t seed;                   /* key of the stochastic rounding */
    const void* w;                   /* device [rows, cols] */
    void* out;                       /* device [rows, cols] */
    const bcg_patch* patches;        /* host [num_patches] (NULL if none) */
} bcg_weight_args;

int weight_patch(const bcg_weight_args* args, void* stream);

/*
 * bcg_loop_* -- the sampler loop's per-step work in native code, for
 * launches k = k0 .. k0+count-1.  Launch k advances replica r = k mod
 * replicas (several independent batches served round-robin; 1 by default)
 * by one step of its own trajectory: t_i = start[i] + floor(k / replicas),
 * reduced modulo steps when wrap is set and t_i >= 0 (steady-state continuous
 * batching: a finished slot restarts at step 0).
 *
 * Host plans (device_plan = 0): the bucket plan of each launch is built on
 * the host (bcg_plan_build) straight into pinned staging row k mod rows,
 * copied to the device row (hipMemcpyAsync, P rows per copy) and one
 * guided_step is launched with that row.  Every plan is built before its
 * launch is queued; batching only merges the copies (a plan depends on the
 * step index, never on the state).  [B] section 4 stage 3: the plan is built
 * by the scheduler before the launch and is immutable while the step runs.
 * A staging row is rewritten only after its previous copy has completed.
 * Row layout (4n int32): [step_idx | scale (float bits) | uncond_row | order].
 *
 * Device plans (device_plan = 1): each launch is one guided_step_dplan that
 * builds the step's plan on the device (into dplan's plan outputs, if given)
 * and advances the replica's step indices in dev_steps (two buffers per
 * replica, alternating; with dev_records, the sample records of those
 * indices too, which the next launch reads instead of deriving them); no
 * host work or copy per launch.  The indices (and records) are written from
 * `start` at bcg_loop_create and again whenever a run starts at k0 = 0;
 * otherwise k0 must continue the previous run.  With graph_launches
 * G > 0, every run of G launches is the replay of a HIP graph: at
 * bcg_loop_create one graph per phase of the buffer pattern (launches
 * g .. g+G-1, g < 2*replicas) is captured on a stream of the loop's own, so
 * a replay can start at any launch; launches left over (fewer than G) are
 * launched directly.
 *
 * The descriptor is copied at create time; the arrays it points to (host plan
 * inputs, staging rows, dev_steps, every device array of `step` and `dplan`)
 * are owned by the caller and must outlive the loop.  step.order / step_idx /
 * scale / uncond_row / n_active are ignored (filled per launch); with
 * replicas > 1, step.x and step.x_out are offset by r * replica_stride bytes.
 * If kernel_ms is not NULL, one pair of HIP events on `stream` brackets the
 * whole run (the first recorded before its first launch, the second after
 * its last), bcg_loop_run waits for the second, and *kernel_ms receives the
 * elapsed time divided by count: the mean time per launch, gaps between
 * launches included.  bcg_loop_last_run reports how many launches of the
 * last run were graph replays and how many were launched directly.
 * Errors: as bcg_plan_build, guided_step and guided_step_dplan; BCG_EHIP.
 */
typedef struct {
    bcg_plan_in plan;                /* plan.step_idx is ignored */
    const int32_t* start;            /* host [n] start step of each sample */
    int32_t wrap;                    /* 1: t reduced modulo steps once >= 0 */
    int32_t rows;                    /* staging rows, >= 1 (host plans) */
    int32_t* host_slab;              /* pinned host [rows][4n] (host plans) */
    int32_t* dev_slab;               /* device [rows][4n] (host plans) */
    int32_t replicas;                /* >= 1 independent states of the batch */
    int64_t replica_stride;          /* bytes between replicas of x and x_out */
    int32_t upload_batch;            /* P in [1, 64]: plans of P consecutive launches are
                                        built, then uploaded with one copy; rows must
                                        be a multiple of P (host plans) */
    int32_t async_upload;            /* 1: uploads on the loop's own copy stream,
                                        overlapping earlier launches; 0: on `stream` */
    bcg_step_args step;              /* launch template (replica 0) */
    int32_t device_plan;             /* 0: host plans; 1: device plans */
    int32_t graph_launches;          /* device plans: G in [0, 4096], see above */
    int32_t* dev_steps;              /* device plans: device [replicas][2][n] */
    bcg_device_plan dplan;           /* device plans: template (steps, num_buckets and
                                        wrap are taken from plan/wrap; step_in and
                                        step_out are set per launch) */
    float* dev_records;              /* device plans: device [replicas][2][n][4] or NULL: the
                                        sample records that go with dev_steps (each launch
                                        reads one buffer and its plan writes the other) */
    /* continuous batching (device plans with records; see bcg_device_plan): the n samples
       are slots, slot s starts with request s at step start[s] (in [0, steps)) and joins at
       the first launch (its state is built there from its noise; x need not be initialised);
       freed slots take the next queued requests.  The per-sample arrays of `plan`, `step`
       and `dplan` hold queue_len requests (dplan.covered for every request when the step
       has regions); wrap must be 0. */
    int32_t queue_len;               /* 0: off; else the requests of the queue (>= n) */
    int32_t queue_ring;              /* 0 | 1: request ids modulo queue_len */
    const float* noise;              /* device fp32 [queue_len, C, H, W] */
    int32_t* dev_queue;              /* device [replicas][2][n + 1 + join_front]: the slots'
                                        requests, the next queued request and the list of
                                        joins dispatched first (alternating like dev_steps) */
    int32_t join_front;              /* J in [0, n], see bcg_device_plan */
} bcg_loop_desc;

typedef struct bcg_loop bcg_loop;

int bcg_loop_create(const bcg_loop_desc* desc, bcg_loop** out);
int bcg_loop_run(bcg_loop* loop, int k0, int count, void* stream, float* kernel_ms);
/* Launches of the last bcg_loop_run inside graph replays (*replayed) and
 * launched directly (*direct); either pointer may be NULL. */
int bcg_loop_last_run(const bcg_loop* loop, int32_t* replayed, int32_t* direct);
int bcg_loop_destroy(bcg_loop* loop);

#ifdef __cplusplus
}
#endif
#endif /* BCG_H */
