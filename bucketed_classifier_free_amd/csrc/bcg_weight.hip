// weight_patch: a weight with its diff and low-rank patches applied, written
// back with nearest or stochastic rounding (ComfyUI guide "10 · ModelPatcher
// and weight views": "patches record format", "strength_model and
// strength_patch", "offset patch", "how a weight is patched").
//
// One fused, HBM-bound kernel.  A workgroup owns a 64 x 128 tile of the
// weight; each lane holds four 8-element row vectors of it in fp32 registers
// (16-byte accesses, consecutive lanes on consecutive addresses), applies the
// patches in order and stores the result once.  A diff patch streams its
// slice of the diff through the same lane layout.  A low-rank patch's delta
// tile is a genuine contraction (up [64, r] x down [r, 128]) and runs on the
// matrix cores: `down` is staged 32 k-rows at a time into LDS transposed
// (k contiguous per column, the B-operand layout of v_mfma_f32_32x32x16_bf16),
// `up` is read straight from global memory in the A-operand layout, each wave
// accumulates two 32x32 fp32 sub-tiles, and the tile goes through LDS once to
// reach the streaming layout.  The stochastic rounding bits come from
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011), one call per 8 consecutive elements.
#include "bcg_device.h"
#include "bcg_launch.h"

namespace bcg {
namespace {

constexpr int TR = 64;       // tile rows
constexpr int TC = 128;      // tile columns
constexpr int NT = 256;      // lanes per workgroup
constexpr int KC = 32;       // rows of `down` staged per chunk
constexpr int KP = KC + 8;   // LDS row of the transposed chunk, in bf16 (80 bytes)
constexpr int DP = TC + 4;   // LDS row of the delta tile, in fp32 (528 bytes)
constexpr int VPL = TR * TC / 8 / NT;  // 8-element vectors per lane (4)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct PatchDev {
    int kind, offset, rows, rank, dtype, upvec;
    float sp, sm;
    const void* diff;
    const bf16_t* up;
    const bf16_t* down;
};

struct WeightParams {
    int rows, cols;
    int ctiles;       // column tiles
    int np;           // patches
    int stochastic;   // bf16 out: 1 = stochastic rounding
    int vec;          // cols % 8 == 0 and every streamed array 16-byte aligned
    uint32_t key0, key1;
    const void* w;
    void* out;
    PatchDev p[BCG_MAX_PATCHES];
};

// ---------------------------------------------------------------- Philox4x32-10

__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                              uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
}

// The 16 random bits of element e (all 8 of a call when e % 8 == 0 is used
// by the vector path through random8).
__device__ __forceinline__ uint32_t random16(const WeightParams& p, uint64_t e) {
    const uint64_t b = e >> 3;
    uint32_t c0 = (uint32_t)b, c1 = (uint32_t)(b >> 32), c2 = 0, c3 = 0;
    philox4x32_10(c0, c1, c2, c3, p.key0, p.key1);
    const int wsel = (int)((e & 7) >> 1);
    const uint32_t w = wsel == 0 ? c0 : wsel == 1 ? c1 : wsel == 2 ? c2 : c3;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

__device__ __forceinline__ void random8(const WeightParams& p, uint64_t e8, uint32_t (&r)[8]) {
    const uint64_t b = e8 >> 3;
    uint32_t c0 = (uint32_t)b, c1 = (uint32_t)(b >> 32), c2 = 0, c3 = 0;
    philox4x32_10(c0, c1, c2, c3, p.key0, p.key1);
    r[0] = c0 & 0xffffu; r[1] = c0 >> 16; r[2] = c1 & 0xffffu; r[3] = c1 >> 16;
    r[4] = c2 & 0xffffu; r[5] = c2 >> 16; r[6] = c3 & 0xffffu; r[7] = c3 >> 16;
}

// fp32 -> bf16 by adding 16 random bits to the bit pattern and truncating;
// NaN and infinities take the nearest-even conversion.
__device__ __forceinline__ uint32_t sr_bf16(float x, uint32_t r16) {
    const uint32_t b = __float_as_uint(x);
    if ((b & 0x7f800000u) == 0x7f800000u) return to_bf16(x);
    return (b + r16) >> 16;
}

// ---------------------------------------------------------------- element access

template <typename T>
__device__ __forceinline__ void load8(const T* base, int64_t off, int n, bool vec, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* base, int64_t off, int n, bool vec, float (&v)[8]) {
    if (vec) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(base + off);
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(base + off + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = e < n ? base[off + e] : 0.0f;
    }
}

template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* base, int64_t off, int n, bool vec, float (&v)[8]) {
    if (vec) {
        const u32x4_t q = *reinterpret_cast<const u32x4_t*>(base + off);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = e < n ? __uint_as_float((uint32_t)base[off + e] << 16) : 0.0f;
    }
}

// The 8 values at flat index e of the output (on the element path only the
// first min(n, 8) of them: n counts the columns left in the row).
template <typename TO>
__device__ __forceinline__ void store8(const WeightParams& p, TO* out, int64_t e, int n, bool vec,
                                       const float (&v)[8]) {
    if constexpr (sizeof(TO) == 4) {
        if (vec) {
            *reinterpret_cast<f32x4_t*>(out + e) = f32x4_t{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<f32x4_t*>(out + e + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (i < n) out[e + i] = v[i];
        }
    } else if (p.stochastic) {
        if (vec) {
            uint32_t r[8];
            random8(p, (uint64_t)e, r);
            u32x4_t q;
            q.x = sr_bf16(v[0], r[0]) | (sr_bf16(v[1], r[1]) << 16);
            q.y = sr_bf16(v[2], r[2]) | (sr_bf16(v[3], r[3]) << 16);
            q.z = sr_bf16(v[4], r[4]) | (sr_bf16(v[5], r[5]) << 16);
            q.w = sr_bf16(v[6], r[6]) | (sr_bf16(v[7], r[7]) << 16);
            *reinterpret_cast<u32x4_t*>(out + e) = q;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (i < n) out[e + i] = (bf16_t)sr_bf16(v[i], random16(p, (uint64_t)(e + i)));
        }
    } else {
        if (vec) {
            const u32x4_t q = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                               pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
            *reinterpret_cast<u32x4_t*>(out + e) = q;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (i < n) out[e + i] = to_bf16(v[i]);
        }
    }
}

// ---------------------------------------------------------------- low-rank delta tile

struct LowRankLds {
    bf16_t b[TC * KP];     // down chunk, transposed: b[col * KP + k]
    float d[TR * DP];      // delta tile, d[row * DP + col]
};

// The low-rank delta of patch q over the tile at (r0, c0) into s.d (fp32;
// rows outside the patch and columns outside the weight hold 0).  Called by
// the whole workgroup (contains barriers); ends with a barrier after the
// tile is written.
__device__ __forceinline__ void lowrank_tile(const WeightParams& p, const PatchDev& q, int r0, int c0,
                                             LowRankLds& s) {
    const int t = (int)threadIdx.x, l = t & 63, wave = t >> 6;
    const int wr = (wave & 1) * 32, wc = (wave >> 1) * 64;
    const int hi = l >> 5, lo = l & 31;
    // A operand: weight row r0 + wr + lo, i.e. patch row pr.
    const int pr = r0 + wr + lo - q.offset;
    const bool arow = pr >= 0 && pr < q.rows;
    const bf16_t* urow = q.up + (int64_t)(arow ? pr : 0) * q.rank;
    f32x16_t acc0 = {}, acc1 = {};
    for (int kc = 0; kc < q.rank; kc += KC) {
        __syncthreads();  // the previous chunk's B reads are done
#pragma unroll
        for (int j = 0; j < (KC * TC / 8) / NT; ++j) {
            const int v = t + j * NT;
            const int kr = v >> 4, cv = (v & 15) * 8;
            const int k = kc + kr, col = c0 + cv;
            float x[8];
            if (k < q.rank && col < p.cols) {
                load8<bf16_t>(q.down, (int64_t)k * p.cols + col, p.cols - col, p.vec != 0, x);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) s.b[(cv + e) * KP + kr] = (bf16_t)(__float_as_uint(x[e]) >> 16);
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KC; kk += 16) {
            const int k = kc + kk + 8 * hi;  // this lane's 8 k of the step
            if (kc + kk >= q.rank) break;    // uniform
            bf16x8_t a;
            if (arow && q.upvec && k < q.rank) {
                a = *reinterpret_cast<const bf16x8_t*>(urow + k);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    a[e] = (arow && k + e < q.rank) ? __builtin_bit_cast(__bf16, urow[k + e])
                                                    : __builtin_bit_cast(__bf16, (bf16_t)0);
            }
            const int kb = kk + 8 * hi;
            const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(&s.b[(wc + lo) * KP + kb]);
            const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(&s.b[(wc + 32 + lo) * KP + kb]);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc1, 0, 0, 0);
        }
    }
    // D[m][n] of a 32x32 MFMA: lane n + 32 * ((m / 4) % 2), register (m % 4) + 4 * (m / 8).
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int m = 8 * (v >> 2) + 4 * hi + (v & 3);
        s.d[(wr + m) * DP + wc + lo] = acc0[v];
        s.d[(wr + m) * DP + wc + 32 + lo] = acc1[v];
    }
    __syncthreads();
}

// ---------------------------------------------------------------- the kernel

template <typename TW, typename TO, bool LR>
__global__ __launch_bounds__(NT) void weight_patch_kernel(WeightParams p) {
    const int64_t tile = blockIdx.x;
    const int r0 = (int)(tile / p.ctiles) * TR, c0 = (int)(tile % p.ctiles) * TC;
    const int t = (int)threadIdx.x;
    const bool vec = p.vec != 0;

    // Lane vectors: j-th at tile row (t + 256 j) / 16, columns 8 * ((t + 256 j) % 16) .. +7.
    float a[VPL][8];
    int row[VPL];
    const int cl = c0 + (t & 15) * 8;
    const int ncol = p.cols - cl;  // elements of the lane's vectors inside the weight (<= 0: none)
    const TW* w = static_cast<const TW*>(p.w);
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        row[j] = r0 + ((t + j * NT) >> 4);
        if (row[j] < p.rows && ncol > 0) load8<TW>(w, (int64_t)row[j] * p.cols + cl, ncol, vec, a[j]);
    }

    extern __shared__ __align__(16) unsigned char lds_raw[];
    for (int q = 0; q < p.np; ++q) {
        const PatchDev& pq = p.p[q];
        if (pq.rows <= 0 || r0 >= pq.offset + pq.rows || r0 + TR <= pq.offset) continue;  // uniform
        if (pq.kind == BCG_PATCH_DIFF) {
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                const int pr = row[j] - pq.offset;
                if (pr < 0 || pr >= pq.rows || ncol <= 0) continue;
                float d[8];
                const int64_t off = (int64_t)pr * p.cols + cl;
                if (pq.dtype == BCG_BF16) load8<bf16_t>(static_cast<const bf16_t*>(pq.diff), off, ncol, vec, d);
                else load8<float>(static_cast<const float*>(pq.diff), off, ncol, vec, d);
#pragma unroll
                for (int e = 0; e < 8; ++e) a[j][e] = fmaf(pq.sp, d[e], pq.sm * a[j][e]);
            }
        } else if constexpr (LR) {
            LowRankLds& s = *reinterpret_cast<LowRankLds*>(lds_raw);
            lowrank_tile(p, pq, r0, c0, s);
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                const int pr = row[j] - pq.offset;
                if (pr < 0 || pr >= pq.rows || ncol <= 0) continue;
                const float* dr = &s.d[((t + j * NT) >> 4) * DP + (t & 15) * 8];
                const f32x4_t x = *reinterpret_cast<const f32x4_t*>(dr);
                const f32x4_t y = *reinterpret_cast<const f32x4_t*>(dr + 4);
                const float d[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) a[j][e] = fmaf(pq.sp, d[e], pq.sm * a[j][e]);
            }
        }
    }

    TO* out = static_cast<TO*>(p.out);
#pragma unroll
    for (int j = 0; j < VPL; ++j)
        if (row[j] < p.rows && ncol > 0) store8<TO>(p, out, (int64_t)row[j] * p.cols + cl, ncol, vec, a[j]);
}

template <typename TW, typename TO>
hipError_t launch(const WeightParams& p, bool lr, int64_t tiles, hipStream_t s) {
    if (lr) {
        hipLaunchKernelGGL((weight_patch_kernel<TW, TO, true>), dim3((unsigned)tiles), dim3(NT),
                           sizeof(LowRankLds), s, p);
    } else {
        hipLaunchKernelGGL((weight_patch_kernel<TW, TO, false>), dim3((unsigned)tiles), dim3(NT), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace bcg

using namespace bcg;

extern "C" int weight_patch(const bcg_weight_args* a, void* stream) {
    clear_error();
    const char* who = "weight_patch";
    if (!a) return fail(BCG_EINVAL, "%s: args is NULL", who);
    if (a->rows < 0 || a->cols < 0) return fail(BCG_ESHAPE, "%s: bad shape %d x %d", who, a->rows, a->cols);
    if ((a->w_dtype != BCG_F32 && a->w_dtype != BCG_BF16) || (a->out_dtype != BCG_F32 && a->out_dtype != BCG_BF16))
        return fail(BCG_EDTYPE, "%s: unknown dtype (w %d, out %d)", who, a->w_dtype, a->out_dtype);
    if (a->num_patches < 0 || a->num_patches > BCG_MAX_PATCHES)
        return fail(BCG_EINVAL, "%s: num_patches %d not in [0, %d]", who, a->num_patches, BCG_MAX_PATCHES);
    if (a->num_patches > 0 && !a->patches) return fail(BCG_EINVAL, "%s: patches is NULL", who);
    if (a->rounding != BCG_ROUND_NEAREST && a->rounding != BCG_ROUND_STOCHASTIC)
        return fail(BCG_EINVAL, "%s: unknown rounding %d", who, a->rounding);
    const int64_t elems = (int64_t)a->rows * a->cols;
    const size_t wbytes = (size_t)elems * elem_size(a->w_dtype), obytes = (size_t)elems * elem_size(a->out_dtype);
    bool lr = false;
    for (int q = 0; q < a->num_patches; ++q) {
        const bcg_patch& pq = a->patches[q];
        if (pq.kind != BCG_PATCH_DIFF && pq.kind != BCG_PATCH_LOWRANK)
            return fail(BCG_EINVAL, "%s: patch %d: unknown kind %d", who, q, pq.kind);
        if (pq.offset < 0 || pq.rows < 0 || (int64_t)pq.offset + pq.rows > a->rows)
            return fail(BCG_ESHAPE, "%s: patch %d: rows [%d, %d) outside the weight's %d", who, q, pq.offset,
                        pq.offset + pq.rows, a->rows);
        if (pq.kind == BCG_PATCH_DIFF) {
            if (pq.dtype != BCG_F32 && pq.dtype != BCG_BF16) return fail(BCG_EDTYPE, "%s: patch %d: diff dtype %d", who, q, pq.dtype);
        } else {
            if (pq.dtype != BCG_BF16) return fail(BCG_EDTYPE, "%s: patch %d: low-rank factors must be bf16", who, q);
            if (pq.rank < 1 || pq.rank > (1 << 16)) return fail(BCG_ESHAPE, "%s: patch %d: rank %d not in [1, 65536]", who, q, pq.rank);
            lr = lr || (pq.rows > 0 && elems > 0);
        }
    }
    if (elems == 0) return BCG_OK;
    if (!a->w || !a->out) return fail(BCG_EINVAL, "%s: NULL device pointer", who);
    const bool same = a->w == a->out && a->w_dtype == a->out_dtype;
    if (!same && any_overlap(a->w, wbytes, a->out, obytes)) return fail(BCG_EINVAL, "%s: w and out overlap", who);
    WeightParams p{};
    p.rows = a->rows;
    p.cols = a->cols;
    p.np = a->num_patches;
    p.stochastic = a->out_dtype == BCG_BF16 && a->rounding == BCG_ROUND_STOCHASTIC;
    p.key0 = (uint32_t)a->seed;
    p.key1 = (uint32_t)(a->seed >> 32);
    p.w = a->w;
    p.out = a->out;
    bool vec = a->cols % 8 == 0 && aligned16(a->w) && aligned16(a->out);
    for (int q = 0; q < a->num_patches; ++q) {
        const bcg_patch& pq = a->patches[q];
        PatchDev& d = p.p[q];
        d.kind = pq.kind; d.offset = pq.offset; d.rows = pq.rows; d.dtype = pq.dtype;
        d.sp = pq.strength_patch; d.sm = pq.strength_model;
        if (pq.rows == 0) continue;
        if (pq.kind == BCG_PATCH_DIFF) {
            if (!pq.diff) return fail(BCG_EINVAL, "%s: patch %d: diff is NULL", who, q);
            const size_t db = (size_t)pq.rows * a->cols * elem_size(pq.dtype);
            if (any_overlap(pq.diff, db, a->out, obytes)) return fail(BCG_EINVAL, "%s: patch %d overlaps out", who, q);
            d.diff = pq.diff;
            vec = vec && aligned16(pq.diff);
        } else {
            if (!pq.up || !pq.down) return fail(BCG_EINVAL, "%s: patch %d: up or down is NULL", who, q);
            const size_t ub = (size_t)pq.rows * pq.rank * 2, db = (size_t)pq.rank * a->cols * 2;
            if (any_overlap(pq.up, ub, a->out, obytes) || any_overlap(pq.down, db, a->out, obytes))
                return fail(BCG_EINVAL, "%s: patch %d overlaps out", who, q);
            d.rank = pq.rank;
            d.up = static_cast<const bf16_t*>(pq.up);
            d.down = static_cast<const bf16_t*>(pq.down);
            d.upvec = pq.rank % 8 == 0 && aligned16(pq.up);
            vec = vec && aligned16(pq.down);
        }
    }
    p.vec = vec;
    const int64_t rtiles = ((int64_t)a->rows + TR - 1) / TR, ctiles = ((int64_t)a->cols + TC - 1) / TC;
    if (rtiles * ctiles > INT32_MAX) return fail(BCG_ESHAPE, "%s: weight too large", who);
    p.ctiles = (int)ctiles;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (a->w_dtype == BCG_BF16)
        e = a->out_dtype == BCG_BF16 ? launch<bf16_t, bf16_t>(p, lr, rtiles * ctiles, st)
                                     : launch<bf16_t, float>(p, lr, rtiles * ctiles, st);
    else
        e = a->out_dtype == BCG_BF16 ? launch<float, bf16_t>(p, lr, rtiles * ctiles, st)
                                     : launch<float, float>(p, lr, rtiles * ctiles, st);
    return hip_status(e, "weight_patch: launch");
}
