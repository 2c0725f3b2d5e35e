// dw_dyn.hpp -- pieces shared by the dynamic multi-dilation filter's forward
// (dw_dynconv.hip) and backward (dw_dynbwd.hip) kernels: 16-byte strips of
// RW pixels, the zero-padded fp32 tile of a row band, and its staging.
#pragma once

#include "dw_common.hpp"
#include "dw_internal.hpp"

namespace dw {
namespace dyn {

constexpr int kMaxBranches = 4;
constexpr int kLdsPref = 32 * 1024;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// RW elements (one 16-byte vector) starting at p, as fp32; lanes past `valid`
// read as 0 and are not touched in memory.
template <typename T, int RW>
__device__ __forceinline__ void load_strip(const T *p, float *v, int valid, bool vec) {
    if (vec && valid >= RW) {
        static_assert(sizeof(T) * RW == 16, "strip is one 16-byte vector");
        union {
            u32x4 u;
            T t[RW];
        } b;
        b.u = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
#pragma unroll
        for (int q = 0; q < RW; ++q) v[q] = to_f32(b.t[q]);
    } else {
#pragma unroll
        for (int q = 0; q < RW; ++q) v[q] = q < valid ? to_f32(p[q]) : 0.f;
    }
}

template <typename T, int RW>
__device__ __forceinline__ void store_strip(T *p, const float *acc, int valid, bool vec) {
    if (vec && valid >= RW) {
        union {
            uint4 u;
            T t[RW];
        } b;
#pragma unroll
        for (int q = 0; q < RW; ++q) b.t[q] = from_f32<T>(acc[q]);
        *reinterpret_cast<uint4 *>(p) = b.u;
    } else {
#pragma unroll
        for (int q = 0; q < RW; ++q)
            if (q < valid) p[q] = from_f32<T>(acc[q]);
    }
}

// As store_strip, bypassing the caches' retention for whole vectors (the
// stream is written once and not read again by this kernel).
template <typename T, int RW>
__device__ __forceinline__ void store_strip_nt(T *p, const float *acc, int valid, bool vec) {
    if (vec && valid >= RW) {
        union {
            u32x4 u;
            T t[RW];
        } b;
#pragma unroll
        for (int q = 0; q < RW; ++q) b.t[q] = from_f32<T>(acc[q]);
        __builtin_nontemporal_store(b.u, reinterpret_cast<u32x4 *>(p));
    } else {
#pragma unroll
        for (int q = 0; q < RW; ++q)
            if (q < valid) p[q] = from_f32<T>(acc[q]);
    }
}

// RW elements held in one 16-byte vector, as fp32.
template <typename T, int RW>
__device__ __forceinline__ void strip_values(const u32x4 &u, float *v) {
    static_assert(sizeof(T) * RW == 16, "strip is one 16-byte vector");
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        if constexpr (sizeof(T) == 4) {
            v[q] = __uint_as_float(w[q]);
        } else {
            const uint32_t h = (q & 1) ? (w[q >> 1] >> 16) : (w[q >> 1] & 0xffffu);
            T t;
            __builtin_memcpy(&t, &h, sizeof(T));
            v[q] = to_f32(t);
        }
    }
}

// Staged tile geometry: hp zero columns left of each row (the halo rounded
// up to 4, so a strip's own columns start 16-byte aligned in LDS) and a row
// pitch LW >= w + 2*hp, a multiple of 4.
inline void dyn_tile(int w, int halo, int &hp, int &LW) {
    hp = (halo + 3) / 4 * 4;
    LW = (w + 2 * hp + 3) / 4 * 4;
}

// Image rows rbase .. rbase+rows-1 of one plane `src` (h x w) into LDS as
// fp32: row r at xs[r*LW + hp ...], zero for rows outside the image and for
// the padding columns on both sides.  vin: src 16-byte aligned and w a
// multiple of the vector width, so rows are copied as 16-byte vectors (four
// loads in flight per thread before the LDS stores).  fVPR divides by the
// vectors per row, fPAD by the padding columns per row (LW - w), fLW by LW.
template <typename T>
__device__ __forceinline__ void stage_rows_f32(float *xs, const T *src, int rbase, int rows, int h, int w,
                                               int LW, int hp, FastDiv fVPR, FastDiv fPAD, FastDiv fLW,
                                               bool vin, int tid) {
    if (vin) {
        constexpr int VE = Vec<T>::N;
        constexpr int NB = 4;
        const int vpr = w / VE;
        const int nvec = rows * vpr;
        for (int v0 = tid; v0 < nvec; v0 += NB * kThreads) {
            uint4 raw[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                raw[k] = make_uint4(0u, 0u, 0u, 0u);
                const int v = v0 + k * kThreads;
                const int r = v < nvec ? static_cast<int>(fdiv(static_cast<uint32_t>(v), fVPR)) : 0;
                const int ih = rbase + r;
                if (v < nvec && ih >= 0 && ih < h)
                    raw[k] = *reinterpret_cast<const uint4 *>(src + static_cast<int64_t>(ih) * w +
                                                               static_cast<int64_t>(v - r * vpr) * VE);
            }
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int v = v0 + k * kThreads;
                if (v < nvec) {
                    const int r = static_cast<int>(fdiv(static_cast<uint32_t>(v), fVPR));
                    float *d = xs + r * LW + hp + (v - r * vpr) * VE;
                    union {
                        uint4 u;
                        T t[VE];
                    } b;
                    b.u = raw[k];
#pragma unroll
                    for (int e = 0; e < VE; e += 4)
                        *reinterpret_cast<float4 *>(d + e) =
                            make_float4(to_f32(b.t[e]), to_f32(b.t[e + 1]), to_f32(b.t[e + 2]), to_f32(b.t[e + 3]));
                }
            }
        }
        const int padw = LW - w;
        for (int e = tid; e < rows * padw; e += kThreads) {
            const int r = static_cast<int>(fdiv(static_cast<uint32_t>(e), fPAD));
            const int j = e - r * padw;
            xs[r * LW + (j < hp ? j : w + j)] = 0.f;
        }
    } else {
        for (int e = tid; e < rows * LW; e += kThreads) {
            const int r = static_cast<int>(fdiv(static_cast<uint32_t>(e), fLW));
            const int col = e - r * LW - hp;
            const int ih = rbase + r;
            xs[e] = (col >= 0 && col < w && ih >= 0 && ih < h) ? to_f32(src[static_cast<int64_t>(ih) * w + col])
                                                                  : 0.f;
        }
    }
}

// Row bands over the planes of one (n, c) grid: band height BH so that each
// thread gets about `per_thread` strips, the tile (BH + 2*halo rows) within
// the LDS budget, and >= 1024 workgroups when the problem allows.
struct DynPlan {
    int BH, nbands, lds_bytes;
};

template <typename T>
bool plan_dyn(int n, int c, int h, int w, int k, int maxdil, DynPlan &p, int per_thread = 2) {
    constexpr int RW = Vec<T>::N;
    const int NS = (w + RW - 1) / RW;
    const int halo = (k - 1) / 2 * maxdil;
    int hp, LW;
    dyn_tile(w, halo, hp, LW);
    auto bytes = [&](int bh) -> int64_t {
        const int64_t rows = std::min<int64_t>(bh, h) + 2 * static_cast<int64_t>(halo);  // zero rows included
        const int64_t cnt = rows * LW + RW;  // + RW: a partial last strip may read past the last row
        if (cnt > (1 << 24)) return INT64_MAX;
        return cnt * static_cast<int64_t>(sizeof(float));
    };
    const int lim = bytes(1) <= kLdsPref ? kLdsPref : kLdsCap;
    if (bytes(1) > lim) return false;
    int bh = std::max(1, (per_thread * kThreads + NS - 1) / NS);
    bh = std::min(bh, h);
    while (bh > 1 && bytes(bh) > lim) --bh;
    const int64_t planes = static_cast<int64_t>(n) * c;
    while (bh > 1 && planes * ((h + bh - 1) / bh) < 1024) bh = (bh + 1) / 2;
    p.nbands = (h + bh - 1) / bh;
    p.BH = (h + p.nbands - 1) / p.nbands;
    p.lds_bytes = static_cast<int>(bytes(p.BH));
    return true;
}

}  // namespace dyn
}  // namespace dw
