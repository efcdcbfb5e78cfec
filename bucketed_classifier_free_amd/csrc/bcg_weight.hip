// weight_patch: a weight with its diff and low-rank patches applied, written
// back with nearest or stochastic rounding (ComfyUI guide "10 · ModelPatcher
// and weight views": "patches record format", "strength_model and
// strength_patch", "offset patch", "how a weight is patched").
//
// Every kernel applies the patches of a weight in order (a = fma(sp, d,
// sm * a) per element in fp32 registers), loads and stores each weight
// element once, and rounds on the store.
//
//   patch_stream_kernel  (no low-rank patch): the weight as a flat sequence
//     of 8-element row vectors (16-byte accesses, consecutive lanes on
//     consecutive addresses), a grid of about one resident round (no partly
//     filled last round) sweeping it front to back; with one diff over every
//     row (patch_stream1_kernel) each lane's next vectors are requested
//     before the current ones are combined.
//   patch_lowrank_strip_kernel (low-rank patches, padded ranks summing to at
//     most 128): the deltas are genuine contractions and run on the matrix
//     cores as the transposed product dW^T = down^T up^T
//     (v_mfma_f32_32x32x16_bf16), with the columns of each 32 x 32 sub-tile
//     relabelled so that a lane's 16 accumulators are 16 consecutive weight
//     columns of one weight row, and combined straight from the accumulators.
//     A workgroup keeps one 128-column strip of `down` in LDS (transposed
//     once) and walks its row tiles with four independent waves (the kernel
//     comment below has the details).
//   patch_lowrank_wide_kernel (bf16 weight and output, every low-rank patch
//     over every row, ranks multiples of 16, rows a multiple of 128): the
//     strip kernel with 128-row tiles, each wave taking 32 rows of both of
//     the strip's 64-column halves in turn, so each `up` fragment it loads
//     serves 128 columns.
//   patch_lowrank_unit_kernel (the same conditions, rows and columns
//     multiples of 384 in a multiple of 256 units): one 12-wave workgroup per
//     CU and 384 x 384 unit, each wave's `up` fragments serving 384 columns.
//   patch_lowrank_kernel (larger ranks): 64 x 128 tiles; the factors of the
//     low-rank patches meeting the tile are concatenated along k and staged
//     per tile, up to 128 k-rows per round, by direct global-to-LDS loads;
//     `up` goes in k-contiguous (16-byte fragment reads, XOR-swizzled against
//     bank conflicts), `down` row-major (the transposed fragment is gathered
//     2 bytes at a time, with padding that keeps the two lane halves on
//     different banks); the weight passes through a padded LDS tile between
//     the streaming layout and the MFMA layout.
//
// The stochastic rounding bits come from Philox4x32-10 (Salmon, Moraes, Dror
// and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), one call
// per 8 consecutive elements.
#include <atomic>

#include "bcg_device.h"
#include "bcg_launch.h"

namespace bcg {
namespace {

constexpr int TR = 64;        // low-rank tile rows
constexpr int TC = 128;       // low-rank tile columns
constexpr int NT = 256;       // lanes per workgroup

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Loads of `up` through pointers read out of LDS (the step table): the
// compiler cannot tell where such a pointer points and would emit flat
// accesses, which also count against the LDS counter, so that each wait for a
// step descriptor in LDS would wait for the `up` loads before it as well.
// These name the global address space.
typedef __attribute__((address_space(1))) const bf16x8_t gbf16x8_t;
typedef __attribute__((address_space(1))) const bf16_t gbf16_t;
__device__ __forceinline__ bf16x8_t ld_up8(const bf16_t* q) { return *(gbf16x8_t*)q; }
__device__ __forceinline__ bf16_t ld_up1(const bf16_t* q) { return *(gbf16_t*)q; }

struct PatchDev {
    int kind, offset, rows, rank, dtype, upvec;
    float sp, sm;
    const void* diff;
    const bf16_t* up;
    const bf16_t* down;
};

// One 16-row k-step of the concatenated low-rank factors (strip kernel).
struct __attribute__((aligned(8))) StepDesc {
    const bf16_t* up;  // `up` of the step's patch, advanced to the step's first k-column
    int q;             // patch index
    int sk;            // first k-row of the step inside the patch
    int rank;          // the patch's rank
    int off, rows;     // weight rows the patch covers
    int flags;         // bit 0: `up` loads 16 bytes at a time; bit 1: last k-step of the patch
    float sp, sm;      // the patch's strengths
};

struct WeightParams {
    int rows, cols;
    int ctiles;       // column tiles (low-rank kernel)
    int np;           // patches
    int stochastic;   // bf16 out: 1 = stochastic rounding
    int vec;          // cols % 8 == 0 and every streamed array 16-byte aligned
    int kalloc;       // k-rows of one staging round (low-rank kernel)
    int rtiles;       // 64-row tiles (strip kernel)
    int grows;        // row-tile groups per column strip (strip kernel)
    int kt_all;       // concatenated padded rank of every low-rank patch (strip kernel)
    int steps;        // 16-row k-steps of that concatenation (strip kernel)
    StepDesc sd[8];   // the k-steps (strip kernel)
    int sm1;          // every low-rank patch has strength_model 1 (strip kernel)
    int onediff;      // one diff patch over every row, vector path (stream kernel)
    int nodiff;       // no diff patch with rows (strip kernel)
    int full;         // every low-rank patch covers every row, ranks multiples of 16 with 16-byte `up` rows, rows a multiple of 64
    int wide;         // full, ranks up to 64 and rows a multiple of 128: the 128-row tiles
    int unit;         // wide, rows and columns multiples of 384 in a multiple of 256 units: the unit kernel
    int nvr;          // 8-element vectors per row (stream kernel)
    int vpt;          // vectors per lane (stream kernel)
    uint32_t nvec;    // vectors of the weight (stream kernel)
    uint32_t key0, key1;
    const void* w;
    void* out;
    PatchDev p[BCG_MAX_PATCHES];
};

// ---------------------------------------------------------------- Philox4x32-10

// a ^ b ^ c in one instruction (v_bitop3_b32 with truth table 0x96).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, (unsigned char)0x96);
}

__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                              uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        // one 32 x 32 -> 64-bit product each (v_mad_u64_u32), not a low and a high multiply
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0), n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
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
    if (vec) {  // streamed once: nontemporal
        const f32x4_t a = ld<true>(reinterpret_cast<const f32x4_t*>(base + off));
        const f32x4_t b = ld<true>(reinterpret_cast<const f32x4_t*>(base + off + 4));
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = e < n ? base[off + e] : 0.0f;
    }
}

template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* base, int64_t off, int n, bool vec, float (&v)[8]) {
    if (vec) {  // streamed once: nontemporal
        const u32x4_t q = ld<true>(reinterpret_cast<const u32x4_t*>(base + off));
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
            st<true>(reinterpret_cast<f32x4_t*>(out + e), f32x4_t{v[0], v[1], v[2], v[3]});
            st<true>(reinterpret_cast<f32x4_t*>(out + e + 4), f32x4_t{v[4], v[5], v[6], v[7]});
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
            st<true>(reinterpret_cast<u32x4_t*>(out + e), q);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (i < n) out[e + i] = (bf16_t)sr_bf16(v[i], random16(p, (uint64_t)(e + i)));
        }
    } else {
        if (vec) {
            const u32x4_t q = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                               pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
            st<true>(reinterpret_cast<u32x4_t*>(out + e), q);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (i < n) out[e + i] = to_bf16(v[i]);
        }
    }
}

// ---------------------------------------------------------------- patches in order

// Diff patch q on a lane vector: weight row `row`, columns c .. c+7 (n of them inside).
template <typename TA>
__device__ __forceinline__ void apply_diff(const WeightParams& p, const PatchDev& q, int row, int c, int n,
                                           bool vec, float (&a)[8]) {
    const int pr = row - q.offset;
    if (pr < 0 || pr >= q.rows || n <= 0) return;
    float d[8];
    load8<TA>(static_cast<const TA*>(q.diff), (int64_t)pr * p.cols + c, n, vec, d);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = fmaf(q.sp, d[e], q.sm * a[e]);
}

__device__ __forceinline__ void apply_diff_any(const WeightParams& p, const PatchDev& q, int row, int c, int n,
                                               bool vec, float (&a)[8]) {
    if (q.dtype == BCG_BF16) apply_diff<bf16_t>(p, q, row, c, n, vec, a);
    else apply_diff<float>(p, q, row, c, n, vec, a);
}

// ---------------------------------------------------------------- stream kernel

template <typename TW, typename TO>
__global__ __launch_bounds__(NT) void patch_stream_kernel(WeightParams p) {
    const bool vec = p.vec != 0;
    const TW* w = static_cast<const TW*>(p.w);
    TO* out = static_cast<TO*>(p.out);
    // round i covers vectors [i * grid * 256, (i + 1) * grid * 256): the whole grid
    // sweeps the weight front to back together (better DRAM page locality than
    // a contiguous share per workgroup)
    for (int i = 0; i < p.vpt; ++i) {
        const uint32_t v = ((uint32_t)i * gridDim.x + blockIdx.x) * NT + threadIdx.x;
        if (v >= p.nvec) break;
        const uint32_t row = v / (uint32_t)p.nvr;
        const int c = (int)(v - row * (uint32_t)p.nvr) * 8;
        const int n = p.cols - c;
        const int64_t e = (int64_t)row * p.cols + c;
        float a[8];
        load8<TW>(w, e, n, vec, a);
        for (int q = 0; q < p.np; ++q) apply_diff_any(p, p.p[q], (int)row, c, n, vec, a);
        store8<TO>(p, out, e, n, vec, a);
    }
}

// ---------------------------------------------------------------- low-rank kernel

constexpr int KMAX = 128;  // concatenated k-rows staged per round (at most)

__device__ __forceinline__ bool hits_tile(const PatchDev& q, int r0) {
    return q.rows > 0 && r0 < q.offset + q.rows && r0 + TR > q.offset;
}

__host__ __device__ __forceinline__ int padded_rank(int rank) { return (rank + 15) & ~15; }

// `down` area of a round: k-rows of 256 bytes (128 bf16 columns), 4 per KiB
// block, 128 bytes of padding after every second block so that rows kl and
// kl + 8 (read together by the two lane halves) sit on different LDS banks.
__device__ __forceinline__ int sb_blk(int g) { return g * 1024 + (g >> 1) * 128; }
__device__ __forceinline__ int sb_off(int kl) { return sb_blk(kl >> 2) + (kl & 3) * 256; }
__host__ __device__ __forceinline__ int sb_bytes(int k) { return (k / 4) * 1024 + (k / 8) * 128; }

// `up` area of a round: per patch piece of kp k-rows, C = kp / 8 chunks of
// 16 bytes per tile row; chunk c of row n in slot n C + (c ^ swz(n)), a
// swizzle (for power-of-two C) that puts 16 consecutive rows at one chunk on
// 16 different 4-bank groups.
__device__ __forceinline__ int su_swz(int n, int C) {
    if (C & (C - 1)) return 0;
    return (C >= 16 ? n : n / (16 / C)) & (C - 1);
}
__device__ __forceinline__ int su_slot(int n, int c, int C) { return n * C + (c ^ su_swz(n, C)); }

// 8 consecutive elements of storage type T in their raw form.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> { u32x4_t v; };
template <> struct Raw8<float> { f32x4_t a, b; };

template <bool STREAM = false>  // STREAM: nontemporal (read or written once)
__device__ __forceinline__ Raw8<bf16_t> raw_load(const bf16_t* base, int64_t off, int n, bool vec) {
    Raw8<bf16_t> r;
    if (vec) {
        r.v = ld<STREAM>(reinterpret_cast<const u32x4_t*>(base + off));
    } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = e < n ? base[off + e] : 0u;
        r.v = u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
    }
    return r;
}
template <bool STREAM = false>  // STREAM: nontemporal (read or written once)
__device__ __forceinline__ Raw8<float> raw_load(const float* base, int64_t off, int n, bool vec) {
    Raw8<float> r;
    if (vec) {
        r.a = ld<STREAM>(reinterpret_cast<const f32x4_t*>(base + off));
        r.b = ld<STREAM>(reinterpret_cast<const f32x4_t*>(base + off + 4));
    } else {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = e < n ? base[off + e] : 0.0f;
        r.a = f32x4_t{x[0], x[1], x[2], x[3]};
        r.b = f32x4_t{x[4], x[5], x[6], x[7]};
    }
    return r;
}
template <bool STREAM = false>  // STREAM: nontemporal (read or written once)
__device__ __forceinline__ void raw_store(bf16_t* base, int64_t off, int n, bool vec, const Raw8<bf16_t>& r) {
    if (vec) {
        st<STREAM>(reinterpret_cast<u32x4_t*>(base + off), r.v);
    } else {
        const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < n) base[off + e] = (bf16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
}
template <bool STREAM = false>  // STREAM: nontemporal (read or written once)
__device__ __forceinline__ void raw_store(float* base, int64_t off, int n, bool vec, const Raw8<float>& r) {
    if (vec) {
        st<STREAM>(reinterpret_cast<f32x4_t*>(base + off), r.a);
        st<STREAM>(reinterpret_cast<f32x4_t*>(base + off + 4), r.b);
    } else {
        const float x[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < n) base[off + e] = x[e];
    }
}
__device__ __forceinline__ void raw_lds_st(unsigned char* q, const Raw8<bf16_t>& r) {
    *reinterpret_cast<u32x4_t*>(q) = r.v;
}
__device__ __forceinline__ void raw_lds_st(unsigned char* q, const Raw8<float>& r) {
    *reinterpret_cast<f32x4_t*>(q) = r.a;
    *reinterpret_cast<f32x4_t*>(q + 16) = r.b;
}
template <typename T> __device__ __forceinline__ Raw8<T> raw_lds_ld(const unsigned char* q);
template <> __device__ __forceinline__ Raw8<bf16_t> raw_lds_ld<bf16_t>(const unsigned char* q) {
    return Raw8<bf16_t>{*reinterpret_cast<const u32x4_t*>(q)};
}
template <> __device__ __forceinline__ Raw8<float> raw_lds_ld<float>(const unsigned char* q) {
    return Raw8<float>{*reinterpret_cast<const f32x4_t*>(q), *reinterpret_cast<const f32x4_t*>(q + 16)};
}
__device__ __forceinline__ void raw_unpack(const Raw8<bf16_t>& r, float (&v)[8]) {
    v[0] = bf16_lo(r.v.x); v[1] = bf16_hi(r.v.x); v[2] = bf16_lo(r.v.y); v[3] = bf16_hi(r.v.y);
    v[4] = bf16_lo(r.v.z); v[5] = bf16_hi(r.v.z); v[6] = bf16_lo(r.v.w); v[7] = bf16_hi(r.v.w);
}
__device__ __forceinline__ void raw_unpack(const Raw8<float>& r, float (&v)[8]) {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
}
// The stored form of the values v of flat elements e .. e + 7 (n inside the row).
template <typename TO> __device__ __forceinline__ Raw8<TO> raw_pack(const WeightParams& p, const float (&v)[8],
                                                                    int64_t e, int n, bool vec);
template <> __device__ __forceinline__ Raw8<float> raw_pack<float>(const WeightParams&, const float (&v)[8],
                                                                   int64_t, int, bool) {
    return Raw8<float>{f32x4_t{v[0], v[1], v[2], v[3]}, f32x4_t{v[4], v[5], v[6], v[7]}};
}
template <> __device__ __forceinline__ Raw8<bf16_t> raw_pack<bf16_t>(const WeightParams& p, const float (&v)[8],
                                                                     int64_t e, int n, bool vec) {
    Raw8<bf16_t> r;
    if (!p.stochastic) {
        r.v = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7])};
        return r;
    }
    uint32_t rb[8];
    if (vec) {
        random8(p, (uint64_t)e, rb);
        // Adding the random bits and keeping the high halves is the rounding for
        // every value but NaN (an infinity keeps its code: the bits stay below
        // the exponent); two results per word by one byte permute, and the
        // lanes with a NaN redo their vector below.
        uint32_t q[4];
        bool nan = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t s0 = __float_as_uint(v[2 * i]) + rb[2 * i];
            const uint32_t s1 = __float_as_uint(v[2 * i + 1]) + rb[2 * i + 1];
            q[i] = __builtin_amdgcn_perm(s1, s0, 0x07060302u);
            nan = nan || v[2 * i] != v[2 * i] || v[2 * i + 1] != v[2 * i + 1];
        }
        if (__builtin_expect(!nan, 1)) {
            r.v = u32x4_t{q[0], q[1], q[2], q[3]};
            return r;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) rb[i] = i < n ? random16(p, (uint64_t)(e + i)) : 0u;
    }
    r.v = u32x4_t{sr_bf16(v[0], rb[0]) | sr_bf16(v[1], rb[1]) << 16, sr_bf16(v[2], rb[2]) | sr_bf16(v[3], rb[3]) << 16,
                  sr_bf16(v[4], rb[4]) | sr_bf16(v[5], rb[5]) << 16, sr_bf16(v[6], rb[6]) | sr_bf16(v[7], rb[7]) << 16};
    return r;
}

// ---------------------------------------------------------------- stream kernel, one full diff

// One diff patch over every row on the 8-element vector path (the flat index
// of vector v's first element is 8 v): the grid sweeps the weight as the
// stream kernel does, and each lane requests its next round's weight and
// diff vectors before this round's arithmetic.
template <typename TW, typename TO, typename TD>
__global__ __launch_bounds__(NT) void patch_stream1_kernel(WeightParams p) {
    const TW* w = static_cast<const TW*>(p.w);
    const TD* d = static_cast<const TD*>(p.p[0].diff);
    TO* out = static_cast<TO*>(p.out);
    const float sp = p.p[0].sp, sm = p.p[0].sm;
    const uint32_t step = gridDim.x * NT;
    uint32_t v = blockIdx.x * NT + threadIdx.x;
    if (v >= p.nvec) return;
    Raw8<TW> wc = raw_load<true>(w, (int64_t)v * 8, 8, true);
    Raw8<TD> dc = raw_load<true>(d, (int64_t)v * 8, 8, true);
    for (;;) {
        const bool more = p.nvec > step && v < p.nvec - step;  // the next round's vector v + step exists
        const uint32_t nv = more ? v + step : v;
        const Raw8<TW> wn = raw_load<true>(w, (int64_t)nv * 8, 8, true);
        const Raw8<TD> dn = raw_load<true>(d, (int64_t)nv * 8, 8, true);
        float a[8], b[8];
        raw_unpack(wc, a);
        raw_unpack(dc, b);
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = fmaf(sp, b[k], sm * a[k]);
        store8<TO>(p, out, (int64_t)v * 8, 8, true, a);
        if (!more) break;
        v = nv;
        wc = wn;
        dc = dn;
    }
}

// Stage concatenated k-rows [kf0, kf0 + kalloc) of the low-rank patches
// meeting the tile at (r0, c0) into the round areas sb (`down`) and su
// (`up`): the patches are walked in order with uniform (scalar) control, each
// patch's piece split into 1 KiB direct global-to-LDS loads dealt round-robin
// to the 4 waves.  Zeros where a row is past a patch's rank, a tile row
// outside the patch or a column outside the weight (and wherever the vector
// path does not apply, the same slots are filled by ordinary loads).
__device__ __forceinline__ void stage_round(const WeightParams& p, int r0, int c0, int kf0, int kalloc,
                                            unsigned char* sb, unsigned char* su, bool vec) {
    const int w = (int)(threadIdx.x >> 6), L = (int)(threadIdx.x & 63);
    int kbase = 0, di = 0, ui = 0;
    for (int q = 0; q < p.np; ++q) {
        const PatchDev& d = p.p[q];
        if (d.kind != BCG_PATCH_LOWRANK || !hits_tile(d, r0)) continue;
        const int rp = padded_rank(d.rank);
        const int lo_k = max(kbase, kf0), hi_k = min(kbase + rp, kf0 + kalloc);
        kbase += rp;
        if (lo_k >= hi_k) continue;
        const int kq0 = lo_k - (kbase - rp);  // first k-row of the piece inside the patch
        // down: (hi_k - lo_k) / 4 blocks of 4 k-rows x 128 columns
        for (int i = 0; i < (hi_k - lo_k) / 4; ++i, ++di) {
            if ((di & 3) != w) continue;
            unsigned char* dst = sb + sb_blk((lo_k - kf0) / 4 + i);
            const int k = kq0 + 4 * i + (L >> 4), col = c0 + 8 * (L & 15);
            const bool ok = k < d.rank && col < p.cols;
            const bf16_t* src = d.down + (int64_t)k * p.cols + col;
            if (ok && vec) {
                __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
            } else {
                Raw8<bf16_t> r{u32x4_t{0u, 0u, 0u, 0u}};
                if (ok) r = raw_load(src, 0, p.cols - col, false);
                raw_lds_st(dst + L * 16, r);
            }
        }
        // up: 64 tile rows x C chunks, C 1 KiB loads
        const int C = (hi_k - lo_k) / 8;
        unsigned char* region = su + (lo_k - kf0) * TR * 2;
        for (int i = 0; i < C; ++i, ++ui) {
            if ((ui & 3) != w) continue;
            const int sl = 64 * i + L, n = sl / C;
            const int c = (sl % C) ^ su_swz(n, C);
            const int k = kq0 + 8 * c, pr = r0 + n - d.offset;
            const bool ok = k < d.rank && pr >= 0 && pr < d.rows;
            const bf16_t* src = d.up + (int64_t)pr * d.rank + k;
            unsigned char* dst = region + i * 1024;
            if (ok && d.upvec) {
                __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
            } else {
                Raw8<bf16_t> r{u32x4_t{0u, 0u, 0u, 0u}};
                if (ok) r = raw_load(src, 0, d.rank - k, false);
                raw_lds_st(dst + L * 16, r);
            }
        }
    }
}

// Sub-tile s of a wave: D^T[m][n] with n the weight row (lane % 32) and m
// relabelled to weight column 4 (m / 8) + m % 4 + 32 ((m / 4) % 2) + 16 s of
// the wave's 64 columns.  Accumulator v of a 32x32 MFMA sits at m = 8 (v / 4)
// + 4 (lane / 32) + v % 4, i.e. at column v + 16 s + 32 (lane / 32): lane
// vector 2 s + v / 8, element v % 8.
__device__ __forceinline__ int sub_col(int lo, int s) {
    return 4 * (lo >> 3) + (lo & 3) + 32 * ((lo >> 2) & 1) + 16 * s;
}

// Slot of strip column c in the transposed `down` area of the strip kernels:
// each group of 8 columns is rotated by its index (c + c / 8 modulo 8 inside
// the group).  The row pitch is an odd number of 16-byte units (kt_all + 8
// for a concatenated rank that is a multiple of 16), so slots that differ
// modulo 8 lie on different banks of a 128-byte bank cycle.  The fragment
// reads of 8 consecutive lanes (columns a .. a + 3 and a + 32 .. a + 35,
// sub_col) then take 8 distinct residues, and so do the staging stores of 8
// consecutive lanes (column j of 8 consecutive groups).
__device__ __forceinline__ int dslot(int c) { return (c & ~7) | ((c + (c >> 3)) & 7); }

// down^T of the strip into LDS, k-step s covering concatenated k-rows 16 s ..
// 16 s + 15, and slot dslot(c) holding column c's k-values contiguously (pitch
// kp).  Each lane takes an 8 x 8 block (8 k-rows of one patch, 8 columns):
// eight 16-byte row loads (the lanes of one k-row on NCOL contiguous columns), a
// transposition in registers (each dword two bfloat16 of one column from two
// rows) and eight 16-byte stores, one per column.  Rows past the rank and
// columns past the weight stage as zeros.
template <int NCOL = TC, int NTH = NT>  // strip columns, lanes of the workgroup
__device__ __forceinline__ void stage_down(const WeightParams& p, bf16_t* sdt, int kp, int c0, bool vec) {
    constexpr int NG = NCOL / 8;  // 8-column groups (a multiple of 8: 8 consecutive lanes take 8 consecutive groups)
    static_assert(NG % 8 == 0, "strip width");
    for (int u = (int)threadIdx.x; u < 2 * NG * p.steps; u += NTH) {
        const int g = u % NG, kb = (u / NG) & 1, s = u / (2 * NG);
        const StepDesc& sd = p.sd[s];
        const PatchDev& d = p.p[sd.q];
        const int col = c0 + 8 * g, k0 = sd.sk + 8 * kb;
        u32x4_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (k0 + i < d.rank && col < p.cols) v[i] = raw_load(d.down, (int64_t)(k0 + i) * p.cols + col, p.cols - col, vec).v;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;  // the high or the low halves
            const u32x4_t f = {__builtin_amdgcn_perm(v[1][j >> 1], v[0][j >> 1], sel),
                               __builtin_amdgcn_perm(v[3][j >> 1], v[2][j >> 1], sel),
                               __builtin_amdgcn_perm(v[5][j >> 1], v[4][j >> 1], sel),
                               __builtin_amdgcn_perm(v[7][j >> 1], v[6][j >> 1], sel)};
            *reinterpret_cast<u32x4_t*>(sdt + dslot(8 * g + j) * kp + 16 * s + 8 * kb) = f;
        }
    }
}

// Dynamic LDS: [transposition tile: 64 rows x trow bytes][down area: sb_bytes(kalloc)][up area: 64 x kalloc x 2].
template <typename TW, typename TO>
__global__ __launch_bounds__(NT) void patch_lowrank_kernel(WeightParams p) {
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int ES = sizeof(TW) > sizeof(TO) ? sizeof(TW) : sizeof(TO);
    constexpr int TROW = TC * ES + 16;
    unsigned char* st = lds;
    unsigned char* sb = lds + TR * TROW;
    unsigned char* su = sb + sb_bytes(p.kalloc);
    const int tile = (int)blockIdx.x;
    const int r0 = (tile / p.ctiles) * TR, c0 = (tile % p.ctiles) * TC;
    const int t = (int)threadIdx.x, l = t & 63, wave = t >> 6;
    const int hi = l >> 5, lo = l & 31;
    const int wr = 32 * (wave & 1), wc = 64 * (wave >> 1);
    const bool vec = p.vec != 0;

    // Streaming layout: vector j of lane t at tile row t / 16 + 16 j, columns 8 (t % 16) .. +7.
    const int scol = (t & 15) * 8, sn = p.cols - (c0 + scol);
    Raw8<TW> wraw[4];
    const TW* w = static_cast<const TW*>(p.w);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = r0 + (t >> 4) + 16 * j;
        if (row < p.rows && sn > 0) wraw[j] = raw_load(w, (int64_t)row * p.cols + c0 + scol, sn, vec);
        else wraw[j] = raw_load(w, 0, 0, false);  // zeros, nothing read
    }
    int kt = 0;  // concatenated k-rows of the tile
    for (int q = 0; q < p.np; ++q)
        if (p.p[q].kind == BCG_PATCH_LOWRANK && hits_tile(p.p[q], r0)) kt += padded_rank(p.p[q].rank);
    if (kt > 0) stage_round(p, r0, c0, 0, p.kalloc, sb, su, vec);
#pragma unroll
    for (int j = 0; j < 4; ++j) raw_lds_st(st + ((t >> 4) + 16 * j) * TROW + scol * sizeof(TW), wraw[j]);
    __builtin_amdgcn_s_waitcnt(0);  // the staged factors have landed
    __syncthreads();

    // MFMA layout: this lane holds weight row `row`, columns cl .. cl + 31 (vector j at cl + 8 j).
    const int row = r0 + wr + lo, cl = c0 + wc + 32 * hi;
    const bool rin = row < p.rows;
    float a[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        raw_unpack(raw_lds_ld<TW>(st + (wr + lo) * TROW + (wc + 32 * hi + 8 * j) * sizeof(TW)), a[j]);

    int kbase = 0, kf0 = 0;
    const int colw0 = wc + sub_col(lo, 0), colw1 = wc + sub_col(lo, 1);
    for (int q = 0; q < p.np; ++q) {
        const PatchDev& d = p.p[q];
        if (d.kind == BCG_PATCH_DIFF) {
            if (d.rows > 0 && rin)
#pragma unroll
                for (int j = 0; j < 4; ++j) apply_diff_any(p, d, row, cl + 8 * j, p.cols - (cl + 8 * j), vec, a[j]);
            continue;
        }
        if (!hits_tile(d, r0)) continue;
        f32x16_t acc0 = {}, acc1 = {};
        const int rp = padded_rank(d.rank);
        for (int k0 = 0; k0 < rp; k0 += 16) {
            const int kf = kbase + k0;
            if (kf >= kf0 + p.kalloc) {  // the next round (more k-rows than one round holds)
                __syncthreads();
                kf0 += p.kalloc;
                stage_round(p, r0, c0, kf0, p.kalloc, sb, su, vec);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
            const int lo_k = max(kbase, kf0);
            const int C = (min(kbase + rp, kf0 + p.kalloc) - lo_k) / 8;
            const unsigned char* region = su + (lo_k - kf0) * TR * 2;
            const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(
                region + su_slot(wr + lo, (kf - lo_k) / 8 + hi, C) * 16);
            const int kl = kf - kf0 + 8 * hi;
            bf16x8_t a0, a1;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const unsigned char* rowp = sb + sb_off(kl + i);
                a0[i] = *reinterpret_cast<const __bf16*>(rowp + colw0 * 2);
                a1[i] = *reinterpret_cast<const __bf16*>(rowp + colw1 * 2);
            }
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc1, 0, 0, 0);
        }
        kbase += rp;
        const int pr = row - d.offset;
        if (rin && pr >= 0 && pr < d.rows) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                a[v >> 3][v & 7] = fmaf(d.sp, acc0[v], d.sm * a[v >> 3][v & 7]);
                a[2 + (v >> 3)][v & 7] = fmaf(d.sp, acc1[v], d.sm * a[2 + (v >> 3)][v & 7]);
            }
        }
    }

    // Round to the stored form in the MFMA layout, back through LDS to the streaming layout.
    __syncthreads();  // every lane has read its weight values out of the tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = cl + 8 * j;
        const Raw8<TO> r = raw_pack<TO>(p, a[j], (int64_t)row * p.cols + c, p.cols - c, vec);
        raw_lds_st(st + (wr + lo) * TROW + (wc + 32 * hi + 8 * j) * sizeof(TO), r);
    }
    __syncthreads();
    TO* out = static_cast<TO*>(p.out);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int srow = r0 + (t >> 4) + 16 * j;
        if (srow < p.rows && sn > 0)
            raw_store(out, (int64_t)srow * p.cols + c0 + scol, sn, vec,
                      raw_lds_ld<TO>(st + ((t >> 4) + 16 * j) * TROW + scol * sizeof(TO)));
    }
}

// ---------------------------------------------------------------- strip kernel

constexpr int PSTEPS = 8;  // k-steps of 16 rows: concatenated padded rank <= 128

// One workgroup per (column strip of 128, row-tile group): the strip's
// `down` rows of every low-rank patch are staged once, transposed (k
// contiguous per column: each MFMA A fragment is one 16-byte LDS read), and
// stay in LDS, read-only, while the workgroup walks its row tiles rt =
// group, group + grows, ...  After that staging the four waves run
// independently (no workgroup barrier): wave w owns the 32 x 64 quarter
// (rows 32 (w % 2), columns 64 (w / 2)) of every tile, moves it between
// global memory and registers in a streaming layout (8 rows x 128 bytes per
// instruction) and turns it to and from the MFMA layout through its own LDS
// region; the next tile's quarter is loaded before this tile's arithmetic and
// the tile's `up` fragments (global memory to registers) land while its
// quarter is transposed.  Specialisations: SM1 (every strength_model is 1:
// no product by it), DIFF = false (no diff patch: no diff walks between the
// low-rank patches), FULL (every low-rank patch covers every row, ranks are
// multiples of 16 with 16-byte `up` rows and the rows a multiple of 64: no
// per-tile or per-lane coverage tests).  Each patch's first k-step starts
// its accumulators from an inline zero.
// Dynamic LDS: [4 wave regions: 32 rows x wrow bytes][down^T: 128 columns x (kt_all + 8) bf16].
template <typename TW, typename TO, bool VEC, bool SM1, bool DIFF = true, bool FULL = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(3, 3))) void patch_lowrank_strip_kernel(WeightParams p) {
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int ES = sizeof(TW) > sizeof(TO) ? sizeof(TW) : sizeof(TO);
    constexpr int WROW = 64 * ES + 16;
    const int t = (int)threadIdx.x, l = t & 63, wave = t >> 6;
    const int hi = l >> 5, lo = l & 31;
    const int wr = 32 * (wave & 1), wc = 64 * (wave >> 1);
    unsigned char* rg = lds + wave * 32 * WROW;  // this wave's region
    bf16_t* sdt = reinterpret_cast<bf16_t*>(lds + 4 * 32 * WROW);
    const int kp = p.kt_all + 8;
    const int ct = (int)blockIdx.x % p.ctiles, gr = (int)blockIdx.x / p.ctiles;
    const int c0 = ct * TC;
    constexpr bool vec = VEC;  // 8-element accesses (the element path is its own instantiation)

    __shared__ StepDesc sdl[PSTEPS];
    if (t == 0) {
#pragma unroll
        for (int s = 0; s < PSTEPS; ++s) sdl[s] = p.sd[s];
    }
    stage_down(p, sdt, kp, c0, vec);
    __syncthreads();  // the only workgroup barrier: down^T and the step table are in place

    // Streaming layout of the wave's quarter: vector j of lane l at quarter row l / 8 + 8 j, columns 8 (l % 8) .. +7.
    const int qc = c0 + wc + 8 * (l & 7), qn = p.cols - qc;
    const TW* w = static_cast<const TW*>(p.w);
    TO* out = static_cast<TO*>(p.out);
    // The next tile's quarter of the weight and its `up` fragments, loaded one
    // tile ahead of the arithmetic.
    Raw8<TW> wn[4];
    bf16x8_t bn[PSTEPS];  // this tile's `up` fragments
    auto load_next_w = [&](int rt) __attribute__((always_inline)) {
        const int r0 = rt * TR;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = r0 + wr + (l >> 3) + 8 * j;
            if (row < p.rows && qn > 0) wn[j] = raw_load<true>(w, (int64_t)row * p.cols + qc, qn, vec);
            else wn[j] = raw_load(w, 0, 0, false);
        }
    };
    auto load_next_up = [&](int rt) __attribute__((always_inline)) {
        const int r0 = rt * TR;
        const int row = r0 + wr + lo;
#pragma unroll
        for (int s = 0; s < PSTEPS; ++s) {
            bn[s] = bf16x8_t{};
            if (s >= p.steps) continue;
            const StepDesc sd = sdl[s];
            const int pr = row - sd.off, k = 8 * hi, rem = sd.rank - sd.sk;
            if (!FULL && (r0 >= sd.off + sd.rows || r0 + TR <= sd.off || pr < 0 || pr >= sd.rows || k >= rem)) continue;
            const bf16_t* src = sd.up + (int64_t)pr * sd.rank + k;
            if (sd.flags & 1) {
                bn[s] = ld_up8(src);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    bn[s][e] = __builtin_bit_cast(__bf16, (bf16_t)(k + e < rem ? ld_up1(src + e) : 0));
            }
        }
    };
    if (gr < p.rtiles) load_next_w(gr);
    const int colw0 = wc + sub_col(lo, 0), colw1 = wc + sub_col(lo, 1);

    for (int rt = gr; rt < p.rtiles; rt += p.grows) {
        const int r0 = rt * TR;
        const int row = r0 + wr + lo, cl = c0 + wc + 32 * hi;
        const bool rin = row < p.rows;
        const bool more = rt + p.grows < p.rtiles;
        load_next_up(rt);  // this tile's fragments: they land while the quarter is transposed
        // to the MFMA layout through the wave's region (LDS accesses of one wave
        // are in order), then the next tile's quarter into the freed registers
#pragma unroll
        for (int j = 0; j < 4; ++j) raw_lds_st(rg + ((l >> 3) + 8 * j) * WROW + 8 * (l & 7) * sizeof(TW), wn[j]);
        if (more) load_next_w(rt + p.grows);
        __builtin_amdgcn_wave_barrier();
        float a[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) raw_unpack(raw_lds_ld<TW>(rg + lo * WROW + (32 * hi + 8 * j) * sizeof(TW)), a[j]);

        // patches in order: k-steps of the low-rank ones, diffs in between
        int qn_ = 0;
        f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
        for (int s = 0; s < PSTEPS; ++s) {
            if (s >= p.steps) break;
            const StepDesc sd = sdl[s];
            if (sd.sk == 0) {
                if constexpr (DIFF) for (; qn_ < sd.q; ++qn_) {
                    const PatchDev& f = p.p[qn_];
                    if (f.kind == BCG_PATCH_DIFF && f.rows > 0 && rin)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            apply_diff_any(p, f, row, cl + 8 * j, p.cols - (cl + 8 * j), vec, a[j]);
                }
            }
            const bool hit = FULL || (r0 < sd.off + sd.rows && r0 + TR > sd.off);
            if (hit) {
                const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(sdt + dslot(colw0) * kp + 16 * s + 8 * hi);
                const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(sdt + dslot(colw1) * kp + 16 * s + 8 * hi);
                if (sd.sk == 0) {  // a patch's first k-step starts from zero (an inline operand)
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bn[s], f32x16_t{}, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bn[s], f32x16_t{}, 0, 0, 0);
                } else {
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bn[s], acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bn[s], acc1, 0, 0, 0);
                }
            }
            if (sd.flags & 2) {  // the patch's last k-step
                const int pr = row - sd.off;
                if (FULL || (hit && rin && pr >= 0 && pr < sd.rows)) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        if constexpr (SM1) {  // every strength_model is 1: 1 * a is a
                            a[v >> 3][v & 7] = fmaf(sd.sp, acc0[v], a[v >> 3][v & 7]);
                            a[2 + (v >> 3)][v & 7] = fmaf(sd.sp, acc1[v], a[2 + (v >> 3)][v & 7]);
                        } else {
                            a[v >> 3][v & 7] = fmaf(sd.sp, acc0[v], sd.sm * a[v >> 3][v & 7]);
                            a[2 + (v >> 3)][v & 7] = fmaf(sd.sp, acc1[v], sd.sm * a[2 + (v >> 3)][v & 7]);
                        }
                    }
                }
                qn_ = sd.q + 1;
            }
        }
        if constexpr (DIFF) for (; qn_ < p.np; ++qn_) {
            const PatchDev& f = p.p[qn_];
            if (f.kind == BCG_PATCH_DIFF && f.rows > 0 && rin)
#pragma unroll
                for (int j = 0; j < 4; ++j) apply_diff_any(p, f, row, cl + 8 * j, p.cols - (cl + 8 * j), vec, a[j]);
        }

        // stored form in the MFMA layout, back to the streaming layout through the region
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = cl + 8 * j;
            const Raw8<TO> r = raw_pack<TO>(p, a[j], (int64_t)row * p.cols + c, p.cols - c, vec);
            raw_lds_st(rg + lo * WROW + (32 * hi + 8 * j) * sizeof(TO), r);
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int srow = r0 + wr + (l >> 3) + 8 * j;
            if (srow < p.rows && qn > 0)
                raw_store<true>(out, (int64_t)srow * p.cols + qc, qn, vec,
                          raw_lds_ld<TO>(rg + ((l >> 3) + 8 * j) * WROW + 8 * (l & 7) * sizeof(TO)));
        }
        __builtin_amdgcn_wave_barrier();
    }
}


// The full-cover case (every patch low-rank over every row, ranks multiples of
// 16 up to 64, rows a multiple of 128) with 128-row tiles: wave w owns rows
// 32 w of the tile and walks its two 64-column halves through its LDS region
// in turn, so each `up` fragment it loads serves both halves (half the `up`
// traffic of the 64-row tiles, where two waves load the same rows).
template <typename TW, typename TO, bool SM1>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(3, 3))) void patch_lowrank_wide_kernel(WeightParams p) {
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int ES = sizeof(TW) > sizeof(TO) ? sizeof(TW) : sizeof(TO);
    constexpr int WROW = 64 * ES + 16;
    constexpr int TRW = 128;  // tile rows
    const int t = (int)threadIdx.x, l = t & 63, wave = t >> 6;
    const int hi = l >> 5, lo = l & 31;
    const int wr = 32 * wave;
    unsigned char* rg = lds + wave * 32 * WROW;  // this wave's region
    bf16_t* sdt = reinterpret_cast<bf16_t*>(lds + 4 * 32 * WROW);
    const int kp = p.kt_all + 8;
    const int ct = (int)blockIdx.x % p.ctiles, gr = (int)blockIdx.x / p.ctiles;
    const int c0 = ct * TC;
    const int nrt = p.rows / TRW;

    __shared__ StepDesc sdl[PSTEPS];
    if (t == 0) {
#pragma unroll
        for (int s = 0; s < PSTEPS; ++s) sdl[s] = p.sd[s];
    }

    const TW* w = static_cast<const TW*>(p.w);
    TO* out = static_cast<TO*>(p.out);
    Raw8<TW> wn[4];
    bf16x8_t bn[PSTEPS];
    // the quarter (32 rows x 64 columns, half h of the strip) of tile rt, streaming layout
    auto load_w = [&](int rt, int h) __attribute__((always_inline)) {
        const int qc = c0 + 64 * h + 8 * (l & 7), qn = p.cols - qc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = rt * TRW + wr + (l >> 3) + 8 * j;
            if (qn > 0) wn[j] = raw_load<true>(w, (int64_t)row * p.cols + qc, qn, true);
            else wn[j] = raw_load(w, 0, 0, false);
        }
    };
    // Every fragment load is issued on every path, so that the waits for the
    // weight loads before them need not wait for these; past the table every
    // lane reads the first fragment of the first step (one cache line; never
    // used).
    auto load_up = [&](int rt) __attribute__((always_inline)) {
        const int row = rt * TRW + wr + lo;
#pragma unroll
        for (int s = 0; s < PSTEPS; ++s) {
            const StepDesc& sd = sdl[s < p.steps ? s : 0];
            bn[s] = ld_up8(s < p.steps ? sd.up + (int64_t)(row - sd.off) * sd.rank + 8 * hi : sd.up);
        }
    };
    if (gr < nrt) load_w(gr, 0);  // in flight while down^T is staged
    stage_down(p, sdt, kp, c0, true);
    __syncthreads();  // the only workgroup barrier: down^T and the step table are in place

    for (int rt = gr; rt < nrt; rt += p.grows) {
        const int row = rt * TRW + wr + lo;
        load_up(rt);  // serves both halves
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int wc = 64 * h, cl = c0 + wc + 32 * hi;
            const int qc = c0 + wc + 8 * (l & 7), qn = p.cols - qc;
#pragma unroll
            for (int j = 0; j < 4; ++j) raw_lds_st(rg + ((l >> 3) + 8 * j) * WROW + 8 * (l & 7) * sizeof(TW), wn[j]);
            if (h == 0) load_w(rt, 1);
            else if (rt + p.grows < nrt) load_w(rt + p.grows, 0);
            __builtin_amdgcn_wave_barrier();
            float a[4][8];
#pragma unroll
            for (int j = 0; j < 4; ++j) raw_unpack(raw_lds_ld<TW>(rg + lo * WROW + (32 * hi + 8 * j) * sizeof(TW)), a[j]);
            const int colw0 = wc + sub_col(lo, 0), colw1 = wc + sub_col(lo, 1);
            f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
            for (int s = 0; s < PSTEPS; ++s) {
                if (s >= p.steps) break;
                const StepDesc sd = sdl[s];
                const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(sdt + dslot(colw0) * kp + 16 * s + 8 * hi);
                const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(sdt + dslot(colw1) * kp + 16 * s + 8 * hi);
                if (sd.sk == 0) {
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bn[s], f32x16_t{}, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bn[s], f32x16_t{}, 0, 0, 0);
                } else {
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bn[s], acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bn[s], acc1, 0, 0, 0);
                }
                if (sd.flags & 2) {  // the patch's last k-step
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        if constexpr (SM1) {
                            a[v >> 3][v & 7] = fmaf(sd.sp, acc0[v], a[v >> 3][v & 7]);
                            a[2 + (v >> 3)][v & 7] = fmaf(sd.sp, acc1[v], a[2 + (v >> 3)][v & 7]);
                        } else {
                            a[v >> 3][v & 7] = fmaf(sd.sp, acc0[v], sd.sm * a[v >> 3][v & 7]);
                            a[2 + (v >> 3)][v & 7] = fmaf(sd.sp, acc1[v], sd.sm * a[2 + (v >> 3)][v & 7]);
                        }
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = cl + 8 * j;
                const Raw8<TO> r = raw_pack<TO>(p, a[j], (int64_t)row * p.cols + c, p.cols - c, true);
                raw_lds_st(rg + lo * WROW + (32 * hi + 8 * j) * sizeof(TO), r);
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int srow = rt * TRW + wr + (l >> 3) + 8 * j;
                if (qn > 0)
                    raw_store<true>(out, (int64_t)srow * p.cols + qc, qn, true,
                                    raw_lds_ld<TO>(rg + ((l >> 3) + 8 * j) * WROW + 8 * (l & 7) * sizeof(TO)));
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}


// The unit kernel: bf16 weight and output, every low-rank patch over every
// row (ranks multiples of 16), one workgroup of 12 waves per CU (3 per SIMD)
// and per unit of UR = 384 rows x UC = 384 columns.  down^T of the unit's
// columns is staged once; wave w owns rows 32 w of the unit, loads their `up`
// fragments once and walks the unit's six 64-column quarters (from a
// staggered start) through its LDS region, so each fragment serves 384
// columns (three times the wide kernel's 128) and its rows are read by a
// third as many workgroups.  Units are
// numbered row block first: workgroup b runs on XCD b % 8, so with a multiple
// of 8 row blocks each row block's `up` rows are read on one XCD.
constexpr int UW = 12;       // waves per workgroup
constexpr int UNT = 64 * UW; // lanes per workgroup
constexpr int UR = 32 * UW;  // unit rows
constexpr int UQ = 6;        // 64-column quarters per unit
constexpr int UC = 64 * UQ;  // unit columns

inline size_t unit_lds_bytes(int kt_all) {
    return (size_t)UW * 32 * (64 * 2 + 16) + (size_t)UC * (kt_all + 8) * 2;
}

template <bool SM1>
__global__ __launch_bounds__(UNT) __attribute__((amdgpu_waves_per_eu(3, 3))) void patch_lowrank_unit_kernel(WeightParams p) {
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int WROW = 64 * 2 + 16;
    const int t = (int)threadIdx.x, l = t & 63, wave = t >> 6;
    const int hi = l >> 5, lo = l & 31;
    unsigned char* rg = lds + wave * 32 * WROW;  // this wave's region
    bf16_t* sdt = reinterpret_cast<bf16_t*>(lds + UW * 32 * WROW);
    const int kp = p.kt_all + 8;
    const int nrb = p.rows / UR;
    const int rb = (int)blockIdx.x % nrb, cs = (int)blockIdx.x / nrb;
    const int c0 = cs * UC, r0 = rb * UR + 32 * wave;  // the unit's first column, the wave's first row

    __shared__ StepDesc sdl[PSTEPS];
    if (t == 0) {
#pragma unroll
        for (int s = 0; s < PSTEPS; ++s) sdl[s] = p.sd[s];
    }
    const bf16_t* w = static_cast<const bf16_t*>(p.w);
    bf16_t* out = static_cast<bf16_t*>(p.out);
    Raw8<bf16_t> wn[4];
    bf16x8_t bn[PSTEPS];
    // The wave walks the unit's quarters starting at (strip + wave) mod 6, so
    // that the waves of a CU, and the units of a row block, stream different
    // columns at a time (measured 1.0 us faster than every wave in column
    // order, 0.6 us faster than one start per workgroup at strip mod 6).
    auto qof = [&](int h) { return (h + cs + wave) % UQ; };
    // step h of the walk: its quarter of the wave's rows, streaming layout
    auto load_w = [&](int h) __attribute__((always_inline)) {
        const int qc = c0 + 64 * qof(h) + 8 * (l & 7);
#pragma unroll
        for (int j = 0; j < 4; ++j) wn[j] = raw_load<true>(w, (int64_t)(r0 + (l >> 3) + 8 * j) * p.cols + qc, 8, true);
    };
    load_w(0);  // in flight while down^T is staged
    stage_down<UC, UNT>(p, sdt, kp, c0, true);
    __syncthreads();  // the only workgroup barrier: down^T and the step table are in place
    {
        // every fragment load on every path; past the table every lane reads
        // the first fragment of the first step (never used)
        const int row = r0 + lo;
#pragma unroll
        for (int s = 0; s < PSTEPS; ++s) {
            const StepDesc& sd = sdl[s < p.steps ? s : 0];
            bn[s] = ld_up8(s < p.steps ? sd.up + (int64_t)(row - sd.off) * sd.rank + 8 * hi : sd.up);
        }
    }
    const int row = r0 + lo;
#pragma unroll
    for (int h = 0; h < UQ; ++h) {
        const int wc = 64 * qof(h), cl = c0 + wc + 32 * hi;
        const int qc = c0 + wc + 8 * (l & 7);
#pragma unroll
        for (int j = 0; j < 4; ++j) raw_lds_st(rg + ((l >> 3) + 8 * j) * WROW + 8 * (l & 7) * 2, wn[j]);
        if (h + 1 < UQ) load_w(h + 1);
        __builtin_amdgcn_wave_barrier();
        float a[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) raw_unpack(raw_lds_ld<bf16_t>(rg + lo * WROW + (32 * hi + 8 * j) * 2), a[j]);
        const int colw0 = wc + sub_col(lo, 0), colw1 = wc + sub_col(lo, 1);
        f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
        for (int s = 0; s < PSTEPS; ++s) {
            if (s >= p.steps) break;
            const StepDesc sd = sdl[s];
            const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(sdt + dslot(colw0) * kp + 16 * s + 8 * hi);
            const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(sdt + dslot(colw1) * kp + 16 * s + 8 * hi);
            if (sd.sk == 0) {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bn[s], f32x16_t{}, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bn[s], f32x16_t{}, 0, 0, 0);
            } else {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bn[s], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bn[s], acc1, 0, 0, 0);
            }
            if (sd.flags & 2) {  // the patch's last k-step
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    if constexpr (SM1) {
                        a[v >> 3][v & 7] = fmaf(sd.sp, acc0[v], a[v >> 3][v & 7]);
                        a[2 + (v >> 3)][v & 7] = fmaf(sd.sp, acc1[v], a[2 + (v >> 3)][v & 7]);
                    } else {
                        a[v >> 3][v & 7] = fmaf(sd.sp, acc0[v], sd.sm * a[v >> 3][v & 7]);
                        a[2 + (v >> 3)][v & 7] = fmaf(sd.sp, acc1[v], sd.sm * a[2 + (v >> 3)][v & 7]);
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = cl + 8 * j;
            const Raw8<bf16_t> r = raw_pack<bf16_t>(p, a[j], (int64_t)row * p.cols + c, 8, true);
            raw_lds_st(rg + lo * WROW + (32 * hi + 8 * j) * 2, r);
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < 4; ++j)
            raw_store<true>(out, (int64_t)(r0 + (l >> 3) + 8 * j) * p.cols + qc, 8, true,
                            raw_lds_ld<bf16_t>(rg + ((l >> 3) + 8 * j) * WROW + 8 * (l & 7) * 2));
        __builtin_amdgcn_wave_barrier();
    }
}

inline size_t strip_lds_bytes(int es, int kt_all) {
    return (size_t)4 * 32 * (64 * es + 16) + (size_t)TC * (kt_all + 8) * 2;
}

// LDS bytes of the low-rank kernel for kalloc staged k-rows.
inline size_t lowrank_lds_bytes(int es, int kalloc) {
    return (size_t)TR * (TC * es + 16) + sb_bytes(kalloc) + (size_t)TR * kalloc * 2;
}

enum { K_STREAM = 0, K_TILE = 1, K_STRIP = 2 };

// Raise a kernel's dynamic-LDS limit above the default 64 KiB (gfx950 has 160
// KiB per CU), once per kernel and device: `done` holds one bit per device.
inline hipError_t lds_limit(const void* fn, size_t bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

template <typename TW, typename TO>
hipError_t launch(const WeightParams& p, int kind, unsigned blocks, hipStream_t s) {
    constexpr int ES = sizeof(TW) > sizeof(TO) ? sizeof(TW) : sizeof(TO);
    if (kind == K_TILE) {
        static std::atomic<uint64_t> done{0};
        const hipError_t attr = lds_limit(reinterpret_cast<const void*>(&patch_lowrank_kernel<TW, TO>),
                                          lowrank_lds_bytes(ES, KMAX), done);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL((patch_lowrank_kernel<TW, TO>), dim3(blocks), dim3(NT),
                           lowrank_lds_bytes(ES, p.kalloc), s, p);
    } else if (kind == K_STRIP) {
        static std::atomic<uint64_t> done[3] = {{0}, {0}, {0}};
        const size_t lmax = strip_lds_bytes(ES, 16 * PSTEPS), lds = strip_lds_bytes(ES, p.kt_all);
        if (!p.vec) {
            const hipError_t e = lds_limit(
                reinterpret_cast<const void*>(&patch_lowrank_strip_kernel<TW, TO, false, false>), lmax, done[0]);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((patch_lowrank_strip_kernel<TW, TO, false, false>), dim3(blocks), dim3(NT), lds, s, p);
        } else if (sizeof(TW) == 2 && sizeof(TO) == 2 && p.nodiff && p.full && p.wide && p.unit) {  // bf16 in and out
            static std::atomic<uint64_t> done6[2] = {{0}, {0}};
            const size_t umax = unit_lds_bytes(16 * PSTEPS), ulds = unit_lds_bytes(p.kt_all);
            const void* fn = p.sm1 ? reinterpret_cast<const void*>(&patch_lowrank_unit_kernel<true>)
                                   : reinterpret_cast<const void*>(&patch_lowrank_unit_kernel<false>);
            const hipError_t e = lds_limit(fn, umax, done6[p.sm1 ? 0 : 1]);
            if (e != hipSuccess) return e;
            if (p.sm1) hipLaunchKernelGGL((patch_lowrank_unit_kernel<true>), dim3(blocks), dim3(UNT), ulds, s, p);
            else hipLaunchKernelGGL((patch_lowrank_unit_kernel<false>), dim3(blocks), dim3(UNT), ulds, s, p);
        } else if (sizeof(TW) == 2 && sizeof(TO) == 2 && p.nodiff && p.full && p.wide) {  // bf16 in and out
            static std::atomic<uint64_t> done5[2] = {{0}, {0}};
            if (p.sm1) {
                const hipError_t e = lds_limit(reinterpret_cast<const void*>(&patch_lowrank_wide_kernel<TW, TO, true>), lmax, done5[0]);
                if (e != hipSuccess) return e;
                hipLaunchKernelGGL((patch_lowrank_wide_kernel<TW, TO, true>), dim3(blocks), dim3(NT), lds, s, p);
            } else {
                const hipError_t e = lds_limit(reinterpret_cast<const void*>(&patch_lowrank_wide_kernel<TW, TO, false>), lmax, done5[1]);
                if (e != hipSuccess) return e;
                hipLaunchKernelGGL((patch_lowrank_wide_kernel<TW, TO, false>), dim3(blocks), dim3(NT), lds, s, p);
            }
        } else if (p.sm1 && p.nodiff && p.full) {
            static std::atomic<uint64_t> done4{0};
            const hipError_t e = lds_limit(
                reinterpret_cast<const void*>(&patch_lowrank_strip_kernel<TW, TO, true, true, false, true>), lmax, done4);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((patch_lowrank_strip_kernel<TW, TO, true, true, false, true>), dim3(blocks), dim3(NT), lds, s, p);
        } else if (p.sm1 && p.nodiff) {
            static std::atomic<uint64_t> done3{0};
            const hipError_t e = lds_limit(
                reinterpret_cast<const void*>(&patch_lowrank_strip_kernel<TW, TO, true, true, false>), lmax, done3);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((patch_lowrank_strip_kernel<TW, TO, true, true, false>), dim3(blocks), dim3(NT), lds, s, p);
        } else if (p.sm1) {
            const hipError_t e = lds_limit(
                reinterpret_cast<const void*>(&patch_lowrank_strip_kernel<TW, TO, true, true>), lmax, done[1]);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((patch_lowrank_strip_kernel<TW, TO, true, true>), dim3(blocks), dim3(NT), lds, s, p);
        } else {
            const hipError_t e = lds_limit(
                reinterpret_cast<const void*>(&patch_lowrank_strip_kernel<TW, TO, true, false>), lmax, done[2]);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((patch_lowrank_strip_kernel<TW, TO, true, false>), dim3(blocks), dim3(NT), lds, s, p);
        }
    } else if (p.onediff) {
        if (p.p[0].dtype == BCG_BF16)
            hipLaunchKernelGGL((patch_stream1_kernel<TW, TO, bf16_t>), dim3(blocks), dim3(NT), 0, s, p);
        else
            hipLaunchKernelGGL((patch_stream1_kernel<TW, TO, float>), dim3(blocks), dim3(NT), 0, s, p);
    } else {
        hipLaunchKernelGGL((patch_stream_kernel<TW, TO>), dim3(blocks), dim3(NT), 0, s, p);
    }
    return hipGetLastError();
}

// The largest concatenated (padded) rank over the 64-row tiles: the set of
// low-rank patches meeting a tile only changes at tiles holding a patch's
// first or last row, so those tiles and the ones after them cover every case.
int max_tile_k(const bcg_weight_args* a) {
    const int64_t rtiles = ((int64_t)a->rows + TR - 1) / TR;
    int best = 0;
    for (int q = 0; q < a->num_patches; ++q) {
        const bcg_patch& e = a->patches[q];
        if (e.kind != BCG_PATCH_LOWRANK || e.rows <= 0) continue;
        const int64_t cand[4] = {e.offset / TR, e.offset / TR + 1, ((int64_t)e.offset + e.rows - 1) / TR,
                                 ((int64_t)e.offset + e.rows - 1) / TR + 1};
        for (int64_t tr : cand) {
            if (tr >= rtiles) continue;
            const int64_t r0 = tr * TR;
            int k = 0;
            for (int u = 0; u < a->num_patches; ++u) {
                const bcg_patch& f = a->patches[u];
                if (f.kind == BCG_PATCH_LOWRANK && f.rows > 0 && r0 < (int64_t)f.offset + f.rows && r0 + TR > f.offset)
                    k += padded_rank(f.rank);
            }
            best = k > best ? k : best;
        }
    }
    return best;
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
    hipStream_t st = static_cast<hipStream_t>(stream);
    int64_t blocks;
    int kind = K_STREAM;
    if (lr) {
        const int64_t rtiles = ((int64_t)a->rows + TR - 1) / TR, ctiles = ((int64_t)a->cols + TC - 1) / TC;
        if (rtiles * ctiles > INT32_MAX) return fail(BCG_ESHAPE, "%s: weight too large", who);
        p.ctiles = (int)ctiles;
        p.rtiles = (int)rtiles;
        int kt_all = 0;
        for (int q = 0; q < a->num_patches; ++q)
            if (a->patches[q].kind == BCG_PATCH_LOWRANK && a->patches[q].rows > 0) kt_all += padded_rank(a->patches[q].rank);
        if (kt_all <= 16 * PSTEPS) {
            // the strip kernel: k-step table, one resident round (3 workgroups per CU on 256 CUs)
            kind = K_STRIP;
            p.kt_all = kt_all;
            p.steps = 0;
            p.sm1 = 1;
            p.nodiff = 1;
            for (int q = 0; q < a->num_patches; ++q)
                if (a->patches[q].kind == BCG_PATCH_DIFF && a->patches[q].rows > 0) p.nodiff = 0;
            p.full = a->rows % TR == 0;
            for (int q = 0; q < a->num_patches; ++q) {
                const bcg_patch& e = a->patches[q];
                if (e.kind == BCG_PATCH_LOWRANK && e.rows > 0 &&
                    (e.offset != 0 || e.rows != a->rows || e.rank % 16 != 0 || !aligned16(e.up)))
                    p.full = 0;
            }
            p.wide = p.full && a->rows % 128 == 0 && p.vec;
            const int64_t units = (int64_t)(a->rows / UR) * (a->cols / UC);
            p.unit = p.wide && a->rows % UR == 0 && a->cols % UC == 0 && units % 256 == 0;
            for (int q = 0; q < a->num_patches; ++q) {
                const bcg_patch& e = a->patches[q];
                if (e.kind != BCG_PATCH_LOWRANK || e.rows <= 0) continue;
                if (e.strength_model != 1.0f) p.sm1 = 0;
                for (int k = 0; k < padded_rank(e.rank); k += 16, ++p.steps) {
                    StepDesc& sd = p.sd[p.steps];
                    sd.up = static_cast<const bf16_t*>(e.up) + k;
                    sd.q = q;
                    sd.sk = k;
                    sd.rank = e.rank;
                    sd.off = e.offset;
                    sd.rows = e.rows;
                    sd.flags = (e.rank % 8 == 0 && aligned16(e.up) ? 1 : 0) | (k + 16 >= padded_rank(e.rank) ? 2 : 0);
                    sd.sp = e.strength_patch;
                    sd.sm = e.strength_model;
                }
            }
            constexpr int64_t kResident = 256 * 3;
            int64_t g = kResident / ctiles;
            g = g < 1 ? 1 : (g > rtiles ? rtiles : g);
            p.grows = (int)g;
            blocks = p.unit ? units : ctiles * g;
        } else {
            kind = K_TILE;
            blocks = rtiles * ctiles;
            const int kmax = max_tile_k(a);
            p.kalloc = kmax < KMAX ? (kmax > 16 ? kmax : 16) : KMAX;
        }
    } else {
        // about one resident round: 8 workgroups of 256 lanes per CU on 256 CUs
        constexpr int64_t kResident = 256 * 8;
        p.nvr = (a->cols + 7) / 8;
        const int64_t nvec = (int64_t)a->rows * p.nvr;
        if (nvec >= INT32_MAX) return fail(BCG_ESHAPE, "%s: weight too large", who);
        p.nvec = (uint32_t)nvec;
        p.vpt = (int)((nvec + kResident * NT - 1) / (kResident * NT));
        p.onediff = vec && a->num_patches == 1 && a->patches[0].kind == BCG_PATCH_DIFF &&
                    a->patches[0].offset == 0 && a->patches[0].rows == a->rows;
        blocks = (nvec + (int64_t)NT * p.vpt - 1) / ((int64_t)NT * p.vpt);
    }
    hipError_t e;
    if (a->w_dtype == BCG_BF16)
        e = a->out_dtype == BCG_BF16 ? launch<bf16_t, bf16_t>(p, kind, (unsigned)blocks, st)
                                     : launch<bf16_t, float>(p, kind, (unsigned)blocks, st);
    else
        e = a->out_dtype == BCG_BF16 ? launch<float, bf16_t>(p, kind, (unsigned)blocks, st)
                                     : launch<float, float>(p, kind, (unsigned)blocks, st);
    return hip_status(e, "weight_patch: launch");
}
