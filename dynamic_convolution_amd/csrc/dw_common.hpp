// dw_common.hpp -- device helpers shared by the gfx950 depthwise kernels:
// element types and their fp32 conversions, division by launch constants,
// and the coalesced global->LDS copy of a contiguous element range.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <algorithm>

namespace dw {

// ---------------------------------------------------------------- element types
// bfloat16 kept as raw bits; conversions below follow the format's definition
// (the upper 16 bits of an IEEE binary32).
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__half v) { return __half2float(v); }
__device__ __forceinline__ float to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v.bits) << 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ __half from_f32<__half>(float v) {
    return __float2half_rn(v);  // v_cvt_f16_f32: round to nearest even
}
// Round to nearest, ties to even (the hardware conversion, v_cvt_pk_bf16_f32
// on gfx950): overflow rounds to +-inf, a NaN stays a quiet NaN.
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
    bf16_t r;
    r.bits = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    return r;
}

// Two fp32 values rounded to nearest even into one word of 16-bit elements
// (element 0 in the low half): one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32.
typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<bf16_t>(float lo, float hi) {
    const f32x2_v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}
template <> __device__ __forceinline__ uint32_t pack2<__half>(float lo, float hi) {
    const f32x2_v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_v));
}

// Elements per 16-byte vector.
template <typename T> struct Vec { static constexpr int N = 16 / sizeof(T); };

// ---------------------------------------------------------------- division
// floor(u / d) for 0 <= u <= umax, 1 <= d.  When umax * d < 2^32 one mul_hi
// with m = ceil(2^32 / d) is exact: u*m/2^32 = u/d + u*e/2^32 with 0 <= e < 1,
// and u*e/2^32 < 1/d cannot move the floor.  Otherwise a plain division.
struct FastDiv {
    uint32_t d;
    uint32_t m;     // 0: use plain division
};

static inline FastDiv make_fastdiv(uint32_t d, uint64_t umax) {
    FastDiv f;
    f.d = d;
    f.m = (d > 1 && (umax + 1) * d < (1ull << 32))
              ? static_cast<uint32_t>(((1ull << 32) + d - 1) / d) : 0u;
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t u, FastDiv f) {
    return f.m ? __umulhi(u, f.m) : (f.d == 1 ? u : u / f.d);
}

// ---------------------------------------------------------------- global -> LDS
// Copies elements [gbeg, gend) of `src` into LDS.  The copy is done in 16-byte
// vectors aligned in global memory (src must be 16-byte aligned), so element e
// lands at lds[e - (gbeg rounded down to a vector)]; the return value is the
// LDS index of element gbeg.  Partially covered end vectors are read one
// element at a time so nothing outside [gbeg, gend) is touched.  Each thread
// issues up to kCopyBatch loads before its LDS stores, to keep several
// 16-byte requests per lane in flight.
constexpr int kCopyBatch = 4;

template <typename T>
__device__ __forceinline__ int lds_copy_range(T *lds, const T *__restrict__ src, int64_t gbeg,
                                              int64_t gend, int tid, int nthreads) {
    constexpr int VE = Vec<T>::N;
    const int64_t base = gbeg & ~static_cast<int64_t>(VE - 1);
    const int nvec = static_cast<int>((gend - base + VE - 1) / VE);
    for (int v0 = tid; v0 < nvec; v0 += nthreads * kCopyBatch) {
        uint4 r[kCopyBatch];
#pragma unroll
        for (int u = 0; u < kCopyBatch; ++u) r[u] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kCopyBatch; ++u) {
            const int v = v0 + u * nthreads;
            const int64_t e0 = base + static_cast<int64_t>(v) * VE;
            if (v < nvec && e0 >= gbeg && e0 + VE <= gend) r[u] = *reinterpret_cast<const uint4 *>(src + e0);
        }
#pragma unroll
        for (int u = 0; u < kCopyBatch; ++u) {
            const int v = v0 + u * nthreads;
            if (v >= nvec) continue;
            const int64_t e0 = base + static_cast<int64_t>(v) * VE;
            if (e0 >= gbeg && e0 + VE <= gend) {
                *reinterpret_cast<uint4 *>(lds + v * VE) = r[u];
            } else {
#pragma unroll
                for (int k = 0; k < VE; ++k) {
                    const int64_t e = e0 + k;
                    lds[v * VE + k] = (e >= gbeg && e < gend) ? src[e] : T{};
                }
            }
        }
    }
    return static_cast<int>(gbeg - base);
}

// Element-wise fallback for sources that are not 16-byte aligned.
template <typename T>
__device__ __forceinline__ int lds_copy_range_scalar(T *lds, const T *__restrict__ src,
                                                     int64_t gbeg, int64_t gend, int tid,
                                                     int nthreads) {
    const int cnt = static_cast<int>(gend - gbeg);
    for (int e = tid; e < cnt; e += nthreads) lds[e] = src[gbeg + e];
    return 0;
}

// LDS slots a copied range of `cnt` elements occupies (vector rounding on both ends).
template <typename T> __host__ __device__ constexpr int lds_slots(int cnt) {
    return ((cnt + 2 * Vec<T>::N - 1) / Vec<T>::N + 1) * Vec<T>::N;
}

// ---------------------------------------------------------------- band planning
// A workgroup either stages G whole input planes (full = 1, one band) or a
// band of BH output rows of a single plane.  full_bytes(G) and band_bytes(BH)
// give the LDS each option needs.  The plan keeps LDS within `pref` bytes
// (or `cap` when even a one-row band needs more), gives each workgroup about
// `target_items` thread items when the problem allows, and splits planes into
// bands when there are too few planes to give the grid `target_wg` groups.
struct BandPlan {
    int G, BH, nbands, full, lds_bytes, grid;
};

template <class FullBytes, class BandBytes>
static inline bool plan_bands(int nplanes, int out_rows, int NS, int pref, int cap, int target_wg,
                              int target_items, FullBytes full_bytes, BandBytes band_bytes,
                              BandPlan &bp) {
    const int64_t items_pp = static_cast<int64_t>(out_rows) * NS;
    const int nb_par = std::max(1, (target_wg + nplanes - 1) / nplanes);
    if (nb_par == 1 && full_bytes(1) <= pref) {
        int G = 1;
        const int64_t want = std::max<int64_t>(1, (target_items + items_pp - 1) / items_pp);
        while (G < want && G < nplanes / target_wg && full_bytes(G + 1) <= pref) ++G;
        bp.G = G;
        bp.BH = out_rows;
        bp.nbands = 1;
        bp.full = 1;
        bp.lds_bytes = static_cast<int>(full_bytes(G));
        bp.grid = (nplanes + G - 1) / G;
        return true;
    }
    const int lim = band_bytes(1) <= pref ? pref : cap;
    if (band_bytes(1) > lim) return false;
    int lo = 1, hi = out_rows;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (band_bytes(mid) <= lim) lo = mid; else hi = mid - 1;
    }
    const int bh_min = std::max(1, (target_items / 4 + NS - 1) / NS);
    const int bh_par = (out_rows + nb_par - 1) / nb_par;
    int BH = std::min(lo, std::max(bh_par, bh_min));
    BH = std::max(1, std::min(BH, out_rows));
    const int nbands = (out_rows + BH - 1) / BH;
    BH = (out_rows + nbands - 1) / nbands;
    bp.G = 1;
    bp.BH = BH;
    bp.nbands = nbands;
    bp.full = 0;
    bp.lds_bytes = static_cast<int>(band_bytes(BH));
    bp.grid = nplanes * nbands;
    return true;
}

// floor(a / b) and ceil(a / b) for b > 0 and any sign of a.
__host__ __device__ __forceinline__ int floordiv(int a, int b) {
    return a >= 0 ? a / b : -((-a + b - 1) / b);
}
__host__ __device__ __forceinline__ int ceildiv(int a, int b) { return -floordiv(-a, b); }

}  // namespace dw
