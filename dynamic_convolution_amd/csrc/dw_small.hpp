// dw_small.hpp -- shared pieces of the channel-group kernels for small planes
// (grad-weight in dw_small.hip, forward in dw_small_fwd.hip, grad-input in
// dw_small_bwdin.hip).
//
// A workgroup owns G adjacent channels and a chunk of images.  For a fixed
// image the G channels' planes of one tensor are one contiguous range of NCHW
// memory, so staging an image is a straight copy of one or two ranges into
// LDS, and an output image is one contiguous range too.  When every range is
// whole, aligned 16-byte vectors, the next image's vectors are loaded into
// registers (kCgPV per lane) while the current image is computed; otherwise
// elements are copied at the top of each iteration.  Each lane owns one
// (channel, row) of the plane it produces for the whole chunk.
#pragma once

#include "dw_common.hpp"
#include "dw_internal.hpp"

namespace dw {

constexpr int kCgStageCap = 16 * 1024;                // staged input bytes per image and workgroup
constexpr int kCgPV = kCgStageCap / (16 * kThreads);  // 16-byte vectors per lane and image
typedef unsigned int cg_v4u __attribute__((ext_vector_type(4)));

// Loads flat vectors tid + k*kThreads of [range a: na vectors | range b: nv - na
// vectors].  Lanes past the end load the first vector of a again (a valid
// address), so no load sits behind a branch.
template <typename T>
__device__ __forceinline__ void cg_issue(cg_v4u (&pf)[kCgPV], const T *a, int na, const T *b, int nv, int tid) {
    constexpr int VE = Vec<T>::N;
#pragma unroll
    for (int k = 0; k < kCgPV; ++k) {
        const int f = tid + k * kThreads;
        const T *p = f < na ? a + f * VE : (f < nv ? b + (f - na) * VE : a);
        pf[k] = *reinterpret_cast<const cg_v4u *>(p);
    }
}

// Stores what cg_issue loaded into the LDS ranges la (na vectors) and lb.
template <typename T>
__device__ __forceinline__ void cg_commit(const cg_v4u (&pf)[kCgPV], T *la, int na, T *lb, int nv, int tid) {
    constexpr int VE = Vec<T>::N;
#pragma unroll
    for (int k = 0; k < kCgPV; ++k) {
        const int f = tid + k * kThreads;
        if (f < nv) {
            T *q = f < na ? la + f * VE : lb + (f - na) * VE;
            *reinterpret_cast<cg_v4u *>(q) = pf[k];
        }
    }
}

// Element copy (ranges that are not whole aligned vectors).
template <typename T>
__device__ __forceinline__ void cg_copy_elems(T *dst, const T *src, int n, int tid) {
    for (int e = tid; e < n; e += kThreads) dst[e] = src[e];
}

// Writes n elements staged in LDS to global memory, as 16-byte vectors when vec.
template <typename T>
__device__ __forceinline__ void cg_store_out(T *dst, const T *src, int n, bool vec, int tid) {
    if (vec) {
        constexpr int VE = Vec<T>::N;
        for (int f = tid; f < n / VE; f += kThreads)
            reinterpret_cast<cg_v4u *>(dst)[f] = reinterpret_cast<const cg_v4u *>(src)[f];
    } else {
        cg_copy_elems(dst, src, n, tid);
    }
}

// Wave-uniform mask of the window positions p < NP whose column p + c0 lies in [0, n).
template <int NP>
__device__ __forceinline__ uint64_t cg_colmask(int c0, int n) {
    static_assert(NP <= 64, "window wider than the mask");
    uint64_t m = 0;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int c = p + c0;
        if (c >= 0 && c < n) m |= 1ull << p;
    }
    return m;
}

// Filter geometries the channel-group kernels are compiled for: square 3x3
// (stride 1 or 2, dilation 1) and 5x5 (stride 1 dilation 1, stride 2 dilation
// 2), multiplier 1 or 2; the padding is a runtime value.
inline bool cg_combo_ok(const Geo &g) {
    const bool sq = g.kh == g.kw && g.sh == g.sw && g.dh == g.dw;
    return g.mult <= 2 && sq &&
           ((g.kh == 3 && g.dh == 1 && g.sh <= 2) || (g.kh == 5 && ((g.sh == 1 && g.dh == 1) || (g.sh == 2 && g.dh == 2))));
}

struct CgPlan {
    int G;         // channels per workgroup
    int NC, npc;   // image chunks, images per chunk
    int grid;      // workgroups
    int vec;       // ranges are whole 16-byte vectors (base pointers are checked at launch)
};

// Group size and image chunks for kernels whose lanes own `lanes_per_ch` rows
// of each channel and which stage `stage_per_ch` bytes per channel and image.
inline bool cg_plan(const Geo &g, int lanes_per_ch, int64_t stage_per_ch, int sz, CgPlan &p) {
    if (lanes_per_ch < 1 || lanes_per_ch > kThreads) return false;
    const int VE = 16 / sz;
    const int64_t iplane = static_cast<int64_t>(g.ih) * g.iw;
    const int64_t oplanes = static_cast<int64_t>(g.mult) * g.oh * g.ow;  // dy or y elements per channel
    int G = static_cast<int>(std::min<int64_t>(kThreads / lanes_per_ch, g.ic));
    while (G > 1 && G * stage_per_ch > kCgStageCap) --G;
    if (G * stage_per_ch > kCgStageCap) return false;
    // whole 16-byte vectors: every image's range of every channel group starts
    // and ends on a vector boundary
    bool vec = (g.ic * iplane) % VE == 0 && (g.ic * oplanes) % VE == 0;
    if (vec) {
        int Gv = G;
        while (Gv > 0 && ((Gv * iplane) % VE != 0 || (Gv * oplanes) % VE != 0)) --Gv;
        if (Gv > 0) G = Gv; else vec = false;
    }
    const int ngroups = (g.ic + G - 1) / G;
    // about 1536 workgroups (six per CU) with at least four images each when
    // the batch allows, so loads of the next image overlap the current one
    int NC = std::max(1, (1536 + ngroups - 1) / ngroups);
    NC = std::min(NC, std::max(1, g.n / 4));
    const int npc = (g.n + NC - 1) / NC;
    p.G = G;
    p.NC = (g.n + npc - 1) / npc;
    p.npc = npc;
    p.grid = ngroups * p.NC;
    p.vec = vec;
    return true;
}

}  // namespace dw
