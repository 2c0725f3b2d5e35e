// dw_bwd_weight.hip -- depthwise gradient with respect to the filters (and bias)
// on gfx950.
//
//   dw[o,i,j] = sum_{n,p,q} dy[n,o,p,q] * x[n,o/M, p*sh-ph+i*dh, q*sw-pw+j*dw]
//   db[o]     = sum_{n,p,q} dy[n,o,p,q]
// (PyTorch PR #3057: the grad-weight kernel, extended to padding, stride and
// dilation, and the bias gradient.)
//
// Two passes, no atomics, so the result is bitwise reproducible:
//  pass 1  the reduction axis (n, p, q) of input channel ic is cut into units
//          (a group of images x a band of output rows); a workgroup takes a
//          fixed chunk of consecutive units, stages x and dy of each unit in
//          LDS, accumulates partial sums for all M*(kh*kw+1) outputs of the
//          channel and writes them to workspace[ic][chunk][slot].
//  pass 2  one thread per (o, tap) adds the chunk partials in chunk order.
// Small filters use pixel-parallel accumulation (every thread holds all taps
// of its pixels, then a workgroup reduction); other filters use tap-parallel
// accumulation (each thread owns up to SPT taps and walks every pixel).
#include "dw_common.hpp"
#include "dw_internal.hpp"

#include <type_traits>

namespace dw {
namespace {

constexpr int kLdsPref = 32 * 1024;
constexpr int kTargetWG = 2048;
constexpr int kRW = 4;
constexpr int kWaves = kThreads / 64;

struct BwPlan {
    int G;          // images per unit
    int BH;         // output rows per band
    int nbands;     // bands per plane
    int R;          // x rows staged per band (upper bound)
    int units;      // units per input channel
    int NC, upc;    // chunks per input channel, units per chunk
    int nslots;     // M * (kh*kw + 1)
    int SPT, nsg;   // tap-parallel: slots per thread, slot groups
    int small;      // pixel-parallel kernel
    int lds_bytes;
    int64_t ws_bytes;
};

template <typename T> struct BwArgs {
    const T *x;
    const T *dy;
    float *ws;
    Geo g;
    BwPlan p;
    int NS;
    FastDiv fNS, fBH;
    int xseg, dseg;  // LDS elements per staged x / dy segment
};

// Stages x rows [rlo, rhi) of the unit's images and dy rows [oh0, oh1) of the
// M output planes of each image.  Segments of >= kThreads elements are copied
// by the whole workgroup one after another, shorter ones one per wave.
template <typename T>
__device__ __forceinline__ void stage_unit(const BwArgs<T> &a, T *xs, T *ds, int ic, int n0, int Gu,
                                           int rlo, int rhi, int oh0, int oh1, int tid) {
    const Geo &g = a.g;
    const int M = g.mult;
    const int xlen = max(rhi - rlo, 0) * g.iw;
    const int dlen = (oh1 - oh0) * g.ow;
    const int64_t xplane = static_cast<int64_t>(g.ih) * g.iw;
    const int64_t dplane = static_cast<int64_t>(g.oh) * g.ow;
    const int wave = tid >> 6, lane = tid & 63;
    const int nseg = Gu + Gu * M;
    for (int k = 0; k < nseg; ++k) {
        const bool isx = k < Gu;
        const int len = isx ? xlen : dlen;
        if (len < kThreads) continue;
        const T *src;
        T *dst;
        if (isx) {
            src = a.x + (static_cast<int64_t>(n0 + k) * g.ic + ic) * xplane + static_cast<int64_t>(rlo) * g.iw;
            dst = xs + k * a.xseg;
        } else {
            const int kk = k - Gu, gi = kk / M, m = kk - gi * M;
            src = a.dy + (static_cast<int64_t>(n0 + gi) * g.oc + ic * M + m) * dplane + static_cast<int64_t>(oh0) * g.ow;
            dst = ds + kk * a.dseg;
        }
        for (int e = tid; e < len; e += kThreads) dst[e] = src[e];
    }
    for (int k = wave; k < nseg; k += kWaves) {
        const bool isx = k < Gu;
        const int len = isx ? xlen : dlen;
        if (len >= kThreads) continue;
        const T *src;
        T *dst;
        if (isx) {
            src = a.x + (static_cast<int64_t>(n0 + k) * g.ic + ic) * xplane + static_cast<int64_t>(rlo) * g.iw;
            dst = xs + k * a.xseg;
        } else {
            const int kk = k - Gu, gi = kk / M, m = kk - gi * M;
            src = a.dy + (static_cast<int64_t>(n0 + gi) * g.oc + ic * M + m) * dplane + static_cast<int64_t>(oh0) * g.ow;
            dst = ds + kk * a.dseg;
        }
        for (int e = lane; e < len; e += 64) dst[e] = src[e];
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

template <typename T>
__device__ __forceinline__ void unit_bounds(const BwArgs<T> &a, int unit, int SH, int DH, int KH, int &n0,
                                            int &Gu, int &oh0, int &oh1, int &rlo, int &rhi) {
    const Geo &g = a.g;
    const int ng = unit / a.p.nbands;
    const int band = unit - ng * a.p.nbands;
    n0 = ng * a.p.G;
    Gu = min(a.p.G, g.n - n0);
    oh0 = band * a.p.BH;
    oh1 = min(oh0 + a.p.BH, g.oh);
    // exactly the input rows this band of output rows reads (<= the staged segment)
    rlo = max(oh0 * SH - g.ph, 0);
    rhi = min((oh1 - 1) * SH - g.ph + (KH - 1) * DH + 1, g.ih);
}

// Pixel-parallel pass 1 for compile-time filter geometry and multiplier MM.
template <typename T, int KH, int KW, int S, int D, int MM, int RW>
__global__ __launch_bounds__(kThreads) void bwd_weight_small_kernel(BwArgs<T> a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int KK = KH * KW;
    constexpr int A = MM * (KK + 1);
    constexpr int WW = (RW - 1) * S + (KW - 1) * D + 1;
    __shared__ float red[kWaves][A];
    const Geo &g = a.g;
    const int tid = threadIdx.x;
    const int ic = blockIdx.x / a.p.NC;
    const int c = blockIdx.x - ic * a.p.NC;
    T *xs = reinterpret_cast<T *>(smem);
    T *ds = xs + a.p.G * a.xseg;

    float acc[MM][KK + 1];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t <= KK; ++t) acc[m][t] = 0.f;

    const int ubeg = c * a.p.upc;
    const int uend = min(ubeg + a.p.upc, a.p.units);
    for (int unit = ubeg; unit < uend; ++unit) {
        int n0, Gu, oh0, oh1, rlo, rhi;
        unit_bounds(a, unit, S, D, KH, n0, Gu, oh0, oh1, rlo, rhi);
        __syncthreads();  // previous unit's LDS reads are done
        stage_unit(a, xs, ds, ic, n0, Gu, rlo, rhi, oh0, oh1, tid);
        __syncthreads();
        const int items = Gu * a.p.BH * a.NS;
        const int rows = oh1 - oh0;
        for (int u = tid; u < items; u += kThreads) {
            const int q1 = static_cast<int>(fdiv(static_cast<uint32_t>(u), a.fNS));
            const int s = u - q1 * a.NS;
            const int gi = static_cast<int>(fdiv(static_cast<uint32_t>(q1), a.fBH));
            const int r = q1 - gi * a.p.BH;
            if (r >= rows) continue;
            const int oh = oh0 + r;
            const int ow0 = s * RW;
            float gy[MM][RW];
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                const T *dp = ds + (gi * MM + m) * a.dseg + r * g.ow + ow0;
                float sb = 0.f;
#pragma unroll
                for (int q = 0; q < RW; ++q) {
                    gy[m][q] = (ow0 + q < g.ow) ? to_f32(dp[q]) : 0.f;
                    sb += gy[m][q];
                }
                acc[m][KK] += sb;
            }
            const T *xp = xs + gi * a.xseg;
            const int c0 = ow0 * S - g.pw;
#pragma unroll
            for (int i = 0; i < KH; ++i) {
                const int ih = oh * S - g.ph + i * D;
                if (ih < rlo || ih >= rhi) continue;
                const T *rp = xp + (ih - rlo) * g.iw;
                float win[WW];
#pragma unroll
                for (int cc = 0; cc < WW; ++cc) {
                    const int col = c0 + cc;
                    win[cc] = (col >= 0 && col < g.iw) ? to_f32(rp[col]) : 0.f;
                }
#pragma unroll
                for (int j = 0; j < KW; ++j)
#pragma unroll
                    for (int m = 0; m < MM; ++m)
#pragma unroll
                        for (int q = 0; q < RW; ++q)
                            acc[m][i * KW + j] = fmaf(gy[m][q], win[q * S + j * D], acc[m][i * KW + j]);
            }
        }
    }
    // workgroup reduction in a fixed order
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t <= KK; ++t) {
            const float v = wave_sum(acc[m][t]);
            if (lane == 0) red[wave][m * (KK + 1) + t] = v;
        }
    __syncthreads();
    if (tid < A) {
        float v = red[0][tid];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) v += red[w][tid];
        a.ws[(static_cast<int64_t>(ic) * a.p.NC + c) * A + tid] = v;
    }
}

// Tap-parallel pass 1 for any geometry: thread tid of slot group sg owns
// slots sg*kThreads*SPT + k*kThreads + tid (k < SPT).
template <typename T, int SPT>
__global__ __launch_bounds__(kThreads) void bwd_weight_taps_kernel(BwArgs<T> a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const Geo &g = a.g;
    const int KK = g.kh * g.kw;
    const int M = g.mult;
    const int tid = threadIdx.x;
    const int sg = blockIdx.x % a.p.nsg;
    const int cc = blockIdx.x / a.p.nsg;
    const int ic = cc / a.p.NC;
    const int c = cc - ic * a.p.NC;
    T *xs = reinterpret_cast<T *>(smem);
    T *ds = xs + a.p.G * a.xseg;

    float acc[SPT];
    int sm[SPT], si[SPT], sj[SPT];
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        acc[k] = 0.f;
        const int slot = (sg * SPT + k) * kThreads + tid;
        sm[k] = slot / (KK + 1);
        const int t = slot - sm[k] * (KK + 1);
        si[k] = t < KK ? t / g.kw : -1;  // -1: bias slot
        sj[k] = t < KK ? t - si[k] * g.kw : 0;
    }
    const int ubeg = c * a.p.upc;
    const int uend = min(ubeg + a.p.upc, a.p.units);
    for (int unit = ubeg; unit < uend; ++unit) {
        int n0, Gu, oh0, oh1, rlo, rhi;
        unit_bounds(a, unit, g.sh, g.dh, g.kh, n0, Gu, oh0, oh1, rlo, rhi);
        __syncthreads();
        stage_unit(a, xs, ds, ic, n0, Gu, rlo, rhi, oh0, oh1, tid);
        __syncthreads();
        const int rows = oh1 - oh0;
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            if (sm[k] >= M) continue;
            for (int gi = 0; gi < Gu; ++gi) {
                const T *dp = ds + (gi * M + sm[k]) * a.dseg;
                if (si[k] < 0) {
                    float s = 0.f;
                    for (int e = 0; e < rows * g.ow; ++e) s += to_f32(dp[e]);
                    acc[k] += s;
                    continue;
                }
                const int j = sj[k];
                const int ow_lo = max(ceildiv(g.pw - j * g.dw, g.sw), 0);
                const int ow_hi = min(floordiv(g.iw - 1 + g.pw - j * g.dw, g.sw) + 1, g.ow);
                const T *xp = xs + gi * a.xseg;
                for (int r = 0; r < rows; ++r) {
                    const int ih = (oh0 + r) * g.sh - g.ph + si[k] * g.dh;
                    if (ih < rlo || ih >= rhi) continue;
                    const T *xr = xp + (ih - rlo) * g.iw - g.pw + j * g.dw;
                    const T *dr = dp + r * g.ow;
                    float s = 0.f;
                    for (int ow = ow_lo; ow < ow_hi; ++ow) s = fmaf(to_f32(dr[ow]), to_f32(xr[ow * g.sw]), s);
                    acc[k] += s;
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        const int slot = (sg * SPT + k) * kThreads + tid;
        if (slot < a.p.nslots) a.ws[(static_cast<int64_t>(ic) * a.p.NC + c) * a.p.nslots + slot] = acc[k];
    }
}

// Pass 2: dw[o, t] (t < kk) and db[o] (t == kk) from the chunk partials.
// 2^lrl adjacent lanes share one output slot: lane l adds chunks l, l + 2^lrl,
// ... in order and the lanes are then combined by a fixed xor tree, so the
// result does not depend on scheduling.  Each lane issues its (up to four per
// round) loads before adding any of them: the partials were just written by
// pass 1 and every load is a full memory round trip.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_weight_reduce_kernel(const float *__restrict__ ws, T *dwt,
                                                                     T *db, int oc, int mult, int kk,
                                                                     int NC, int nslots, int lrl) {
    const int gid = blockIdx.x * kThreads + threadIdx.x;
    const int RL = 1 << lrl;
    const int idx = gid >> lrl, lane = gid & (RL - 1);
    const bool valid = idx < oc * (kk + 1);
    int o = 0, t = 0;
    float s = 0.f;
    if (valid) {
        o = idx / (kk + 1);
        t = idx - o * (kk + 1);
        const int ic = o / mult, m = o - ic * mult;
        const float *p = ws + static_cast<int64_t>(ic) * NC * nslots + m * (kk + 1) + t;
        for (int c0 = lane; c0 < NC; c0 += 4 * RL) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)  // clamped index: always a valid address, no branch around the load
                v[u] = p[static_cast<int64_t>(min(c0 + u * RL, NC - 1)) * nslots];
#pragma unroll
            for (int u = 0; u < 4; ++u) s += c0 + u * RL < NC ? v[u] : 0.f;
        }
    }
    for (int off = RL >> 1; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (!valid || lane != 0) return;
    if (t < kk)
        dwt[static_cast<int64_t>(o) * kk + t] = from_f32<T>(s);
    else if (db != nullptr)
        db[o] = from_f32<T>(s);
}

// Launches pass 2 with about four chunks per lane (at most 64 lanes per slot).
template <typename T>
int launch_reduce(const Geo &g, const void *ws, void *dwt, void *db, int NC, int nslots, hipStream_t s) {
    const int kk = g.kh * g.kw;
    const int64_t total = static_cast<int64_t>(g.oc) * (kk + 1);
    int lrl = 0;
    while (lrl < 6 && (1 << (lrl + 2)) < NC && (total << (lrl + 1)) <= 0x7fff0000LL) ++lrl;
    const int64_t threads = total << lrl;
    hipLaunchKernelGGL((bwd_weight_reduce_kernel<T>), dim3(static_cast<unsigned>((threads + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, static_cast<const float *>(ws), static_cast<T *>(dwt),
                       static_cast<T *>(db), g.oc, g.mult, kk, NC, nslots, lrl);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

bool small_variant(const Geo &g) {
    const bool sq = g.kh == g.kw && g.sh == g.sw && g.dh == g.dw;
    if (!sq || g.mult > 2) return false;
    return (g.kh == 3 && g.dh == 1 && (g.sh == 1 || g.sh == 2)) ||
           (g.kh == 5 && ((g.sh == 1 && g.dh == 1) || (g.sh == 2 && g.dh == 2)));
}

bool plan_bwd_weight(const Geo &g, int elem, BwPlan &p) {
    const int KK = g.kh * g.kw;
    p.nslots = g.mult * (KK + 1);
    p.small = small_variant(g) ? 1 : 0;
    if (p.small) {
        p.SPT = 1;
        p.nsg = 1;
    } else {
        p.SPT = p.nslots <= kThreads ? 1 : (p.nslots <= 2 * kThreads ? 2 : 4);
        p.nsg = (p.nslots + kThreads * p.SPT - 1) / (kThreads * p.SPT);
    }
    const int NS = (g.ow + kRW - 1) / kRW;
    const int64_t xplane = static_cast<int64_t>(g.ih) * g.iw;
    const int64_t dplane = static_cast<int64_t>(g.oh) * g.ow;
    auto rows_x = [&](int bh) {
        return std::min<int64_t>((static_cast<int64_t>(bh) - 1) * g.sh + static_cast<int64_t>(g.kh - 1) * g.dh + 1, g.ih);
    };
    const int64_t full1 = (xplane + g.mult * dplane) * elem;
    if (full1 <= kLdsPref) {
        p.nbands = 1;
        p.BH = g.oh;
        p.R = g.ih;
        const int64_t items_pp = static_cast<int64_t>(g.oh) * NS;
        int G = static_cast<int>(std::min<int64_t>(g.n, std::max<int64_t>(1, (1024 + items_pp - 1) / items_pp)));
        while (G > 1 && G * full1 > kLdsPref) --G;
        p.G = G;
    } else {
        auto bytes = [&](int bh) { return (rows_x(bh) * g.iw + static_cast<int64_t>(g.mult) * bh * g.ow) * elem; };
        // the pixel-parallel kernel adds a small static reduction buffer
        const int cap = bytes(1) <= kLdsPref ? kLdsPref : kLdsCap - 1024;
        if (bytes(1) > cap) return false;
        int lo = 1, hi = g.oh;
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (bytes(mid) <= cap) lo = mid; else hi = mid - 1;
        }
        p.nbands = (g.oh + lo - 1) / lo;
        p.BH = (g.oh + p.nbands - 1) / p.nbands;
        p.R = static_cast<int>(rows_x(p.BH));
        p.G = 1;
    }
    p.units = ((g.n + p.G - 1) / p.G) * p.nbands;
    const int per_ch = std::max(1, (kTargetWG + g.ic * p.nsg - 1) / (g.ic * p.nsg));
    p.NC = std::min(p.units, per_ch);
    p.upc = (p.units + p.NC - 1) / p.NC;
    p.NC = (p.units + p.upc - 1) / p.upc;
    const int64_t xseg = static_cast<int64_t>(p.R) * g.iw;
    const int64_t dseg = static_cast<int64_t>(p.BH) * g.ow;
    p.lds_bytes = static_cast<int>((p.G * xseg + static_cast<int64_t>(p.G) * g.mult * dseg) * elem);
    p.ws_bytes = static_cast<int64_t>(g.ic) * p.NC * p.nslots * 4;
    return true;
}

template <typename T>
void fill_args(BwArgs<T> &a, const Geo &g, const BwPlan &p, const void *x, const void *dy, void *ws) {
    a.x = static_cast<const T *>(x);
    a.dy = static_cast<const T *>(dy);
    a.ws = static_cast<float *>(ws);
    a.g = g;
    a.p = p;
    a.NS = (g.ow + kRW - 1) / kRW;
    const uint64_t items = static_cast<uint64_t>(p.G) * p.BH * a.NS;
    a.fNS = make_fastdiv(a.NS, items);
    a.fBH = make_fastdiv(p.BH, items / a.NS);
    a.xseg = p.R * g.iw;
    a.dseg = p.BH * g.ow;
}

template <typename T, int KH, int KW, int S, int D>
int run_small(const Geo &g, const BwPlan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    BwArgs<T> a;
    fill_args(a, g, p, x, dy, ws);
    const dim3 grid(g.ic * p.NC);
    if (g.mult == 1)
        hipLaunchKernelGGL((bwd_weight_small_kernel<T, KH, KW, S, D, 1, kRW>), grid, dim3(kThreads), p.lds_bytes, s, a);
    else
        hipLaunchKernelGGL((bwd_weight_small_kernel<T, KH, KW, S, D, 2, kRW>), grid, dim3(kThreads), p.lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

enum BwAlgo {
    kBwChannelGroup = 0, kBwLargek, kBwRowwalk, kBwDecim, kBwBandPixel, kBwBandTaps, kBwLargekMfma, kBwLargekMfma32,
    kBwDirect, kBwLargekMfma16, kBwStream7, kBwLargekMfmaH16, kBwRoll16, kBwCount
};

const char *const kBwNames[kBwCount] = {"channelgroup_small", "largek_regtile", "rowwalk_3x3", "decimated_s2d2",
                                        "band_pixel",         "band_taps",      "largek_mfma",  "largek_mfma_f32",
                                        "direct",             "largek_mfma_t16", "stream_7x7",     "largek_mfma_h16", "largek_roll16"};

bool band_bw_plans(const Geo &g, int dt) {
    BwPlan p;
    return plan_bwd_weight(g, dt == 0 ? 4 : 2, p);
}

// Whether pass-1 family `algo` can run this geometry (the band kernel's
// pixel and taps variants are decided by the geometry, not alternatives).
bool feasible_bw(int algo, const Geo &g, int dt) {
    switch (algo) {
        case kBwChannelGroup: return small_fits(g, dt, 2);
        case kBwLargek: return largek_bwdw_fits(g);
        case kBwRowwalk: return rowwalk_fits(g, dt, 2);
        case kBwDecim: return decim_fits(g, 2);
        case kBwLargekMfma: return largek_mfma_bwdw_fits(g, dt);
        case kBwLargekMfma32: return largek_wgrad32_fits(g, dt);
        case kBwBandPixel: return small_variant(g) && band_bw_plans(g, dt);
        case kBwBandTaps: return !small_variant(g) && band_bw_plans(g, dt);
        case kBwDirect: return true;
        case kBwLargekMfma16: return largek_wgrad16_fits(g, dt);
        case kBwStream7: return stream7_bwdw_fits(g);
        case kBwLargekMfmaH16: return largek_mfma_bwdw16_fits(g, dt);
        case kBwRoll16: return largek_wroll16_fits(g, dt);
        default: return false;
    }
}

// The pass-1 kernel family a grad-weight call launches (pass 2 is always the
// fixed-order chunk reduction): the selection table's entry, else the rules.
int select_bwd_weight(const Geo &g, int dt) {
    const int tuned = tuned_algo(2, g, dt);
    if (tuned >= 0 && feasible_bw(tuned, g, dt)) return tuned;
    if (small_fits(g, dt, 2)) return kBwChannelGroup;
    // 16-bit, k = 13: 16 x 16 tiles measured 1.45-1.75x faster than 32 x 32 ones
    // 16-bit 13 x 13 and 31 x 31: input rows streamed past the dy rows held in
    // the filter-row slots, measured 1.25-1.55x faster than the tile kernels
    if (largek_wroll16_fits(g, dt)) return kBwRoll16;
    if (g.kh == 13 && largek_mfma_bwdw16_fits(g, dt)) return kBwLargekMfmaH16;
    if (largek_mfma_bwdw_fits(g, dt)) return kBwLargekMfma;  // 16-bit: measured faster than 16 x 16 fp32 tiles
    if (largek_wgrad16_fits(g, dt)) return kBwLargekMfma16;
    if (largek_wgrad32_fits(g, dt)) return kBwLargekMfma32;
    if (stream7_bwdw_fits(g)) return kBwStream7;  // measured 1.2-2.2x faster than the register tiles
    if (largek_bwdw_fits(g)) return kBwLargek;
    if (rowwalk_fits(g, dt, 2)) return kBwRowwalk;
    if (decim_fits(g, 2)) return kBwDecim;
    if (!band_bw_plans(g, dt)) return kBwDirect;  // rows too wide to stage
    return small_variant(g) ? kBwBandPixel : kBwBandTaps;
}

// Workspace bytes family `algo` needs for this geometry (-1: cannot run it).
int64_t ws_for(int algo, const Geo &g, int dtype) {
    const int64_t slots = static_cast<int64_t>(g.mult) * (g.kh * g.kw + 1);
    switch (algo) {
        case kBwChannelGroup: return std::max<int64_t>(g.ic * small_bwd_weight_chunks(g, dtype) * slots * 4, 16);
        case kBwLargek: return std::max<int64_t>(g.ic * largek_bwd_weight_chunks(g) * slots * 4, 16);
        case kBwLargekMfma: return std::max<int64_t>(g.ic * largek_mfma_bwd_weight_chunks(g) * slots * 4, 16);
        case kBwLargekMfma32: return std::max<int64_t>(g.ic * largek_wgrad32_chunks(g) * slots * 4, 16);
        case kBwLargekMfma16: return std::max<int64_t>(g.ic * largek_wgrad16_chunks(g) * slots * 4, 16);
        case kBwStream7: return std::max<int64_t>(g.ic * stream7_bwdw_chunks(g) * slots * 4, 16);
        case kBwLargekMfmaH16: return std::max<int64_t>(g.ic * largek_mfma_bwd_weight_chunks(g) * slots * 4, 16);
        case kBwRoll16: return std::max<int64_t>(static_cast<int64_t>(g.ic) * largek_wroll16_chunks(g) * slots * 4, 16);
        case kBwDirect: return std::max<int64_t>(static_cast<int64_t>(g.ic) * direct_bwd_weight_chunks(g) * slots * 4, 16);
        case kBwRowwalk: return std::max<int64_t>(g.ic * rowwalk_bwd_weight_chunks(g, dtype) * slots * 4, 16);
        case kBwDecim: return std::max<int64_t>(g.ic * decim_bwd_weight_chunks(g) * slots * 4, 16);
        default: {
            BwPlan p;
            if (!plan_bwd_weight(g, dtype == 0 ? 4 : 2, p)) return -1;
            return std::max<int64_t>(p.ws_bytes, 16);
        }
    }
}

template <typename T>
int dispatch_bwd_weight(const Geo &g, const void *x, const void *dy, void *dwt, void *db, void *ws,
                        hipStream_t s) {
    const int dt = sizeof(T) == 4 ? 0 : (std::is_same<T, __half>::value ? 1 : 2);
    const int kk = g.kh * g.kw;
    int NC, nslots, rc;
    const int algo = select_bwd_weight(g, dt);
    const bool small = algo == kBwChannelGroup;
    const bool large = algo == kBwLargek;
    const bool decim = algo == kBwDecim;
    if (algo == kBwLargekMfma) {
        rc = largek_mfma_bwd_weight(g, x, dy, ws, dt, s);
        if (rc != kOk) return rc;
        return launch_reduce<T>(g, ws, dwt, db, largek_mfma_bwd_weight_chunks(g), kk + 1, s);
    }
    if (algo == kBwDirect) {
        rc = direct_bwd_weight(g, x, dy, ws, dt, s);
        if (rc != kOk) return rc;
        return launch_reduce<T>(g, ws, dwt, db, direct_bwd_weight_chunks(g), g.mult * (kk + 1), s);
    }
    if (algo == kBwLargekMfma16) {
        rc = largek_wgrad16(g, x, dy, ws, dt, s);
        if (rc != kOk) return rc;
        return launch_reduce<T>(g, ws, dwt, db, largek_wgrad16_chunks(g), kk + 1, s);
    }
    if (algo == kBwLargekMfmaH16) {
        rc = largek_mfma_bwd_weight16(g, x, dy, ws, dt, s);
        if (rc != kOk) return rc;
        return launch_reduce<T>(g, ws, dwt, db, largek_mfma_bwd_weight_chunks(g), kk + 1, s);
    }
    if (algo == kBwRoll16) {
        rc = largek_wroll16(g, x, dy, ws, dt, s);
        if (rc != kOk) return rc;
        return launch_reduce<T>(g, ws, dwt, db, largek_wroll16_chunks(g), kk + 1, s);
    }
    if (algo == kBwStream7) {
        rc = stream7_bwdw(g, x, dy, ws, dt, s);
        if (rc != kOk) return rc;
        return launch_reduce<T>(g, ws, dwt, db, stream7_bwdw_chunks(g), kk + 1, s);
    }
    if (algo == kBwLargekMfma32) {
        rc = largek_wgrad32(g, x, dy, ws, s);
        if (rc != kOk) return rc;
        return launch_reduce<T>(g, ws, dwt, db, largek_wgrad32_chunks(g), kk + 1, s);
    }
    if (small || large || decim || algo == kBwRowwalk) {
        // channel-group (small planes), register-tile (large k) or streaming (3x3, pad 1)
        // pass 1: workspace [ic][NC][M*(kk+1)]
        NC = small ? small_bwd_weight_chunks(g, dt)
                   : large ? largek_bwd_weight_chunks(g)
                           : decim ? decim_bwd_weight_chunks(g) : rowwalk_bwd_weight_chunks(g, dt);
        nslots = g.mult * (kk + 1);
        rc = small   ? small_bwd_weight(g, x, dy, ws, dt, s)
             : large ? largek_bwd_weight(g, x, dy, ws, dt, s)
             : decim ? decim_bwd_weight(g, x, dy, ws, dt, s)
                     : rowwalk_bwd_weight(g, x, dy, ws, dt, s);
        if (rc != kOk) return rc;
        return launch_reduce<T>(g, ws, dwt, db, NC, nslots, s);
    }
    BwPlan p;
    if (!plan_bwd_weight(g, sizeof(T), p)) return kErrUnsupported;
    if (p.small) {
        if (g.kh == 3 && g.sh == 1) rc = run_small<T, 3, 3, 1, 1>(g, p, x, dy, ws, s);
        else if (g.kh == 3) rc = run_small<T, 3, 3, 2, 1>(g, p, x, dy, ws, s);
        else if (g.sh == 1) rc = run_small<T, 5, 5, 1, 1>(g, p, x, dy, ws, s);
        else rc = run_small<T, 5, 5, 2, 2>(g, p, x, dy, ws, s);
    } else {
        BwArgs<T> a;
        fill_args(a, g, p, x, dy, ws);
        const dim3 grid(g.ic * p.NC * p.nsg);
        if (p.SPT == 1)
            hipLaunchKernelGGL((bwd_weight_taps_kernel<T, 1>), grid, dim3(kThreads), p.lds_bytes, s, a);
        else if (p.SPT == 2)
            hipLaunchKernelGGL((bwd_weight_taps_kernel<T, 2>), grid, dim3(kThreads), p.lds_bytes, s, a);
        else
            hipLaunchKernelGGL((bwd_weight_taps_kernel<T, 4>), grid, dim3(kThreads), p.lds_bytes, s, a);
        rc = hipGetLastError() == hipSuccess ? kOk : kErrHip;
    }
    if (rc != kOk) return rc;
    return launch_reduce<T>(g, ws, dwt, db, p.NC, p.nslots, s);
}

}  // namespace

const char *bwd_weight_algo_name(const Geo &g, int dtype) { return kBwNames[select_bwd_weight(g, dtype)]; }

int bwd_weight_algo_count() { return kBwCount; }
const char *bwd_weight_algo_name_of(int algo) { return algo >= 0 && algo < kBwCount ? kBwNames[algo] : nullptr; }
bool bwd_weight_algo_feasible(int algo, const Geo &g, int dtype) { return feasible_bw(algo, g, dtype); }

// The largest workspace any family that can run this geometry needs, so a
// buffer sized by it serves whichever family the selection table picks
// (-1 when no family can run it).
int64_t bwd_weight_workspace(const Geo &g, int dtype) {
    int64_t need = -1;
    for (int a = 0; a < kBwCount; ++a)
        if (feasible_bw(a, g, dtype)) need = std::max(need, ws_for(a, g, dtype));
    return need;
}

// Workspace bytes of the family the selection picks for this geometry alone.
int64_t bwd_weight_workspace_selected(const Geo &g, int dtype) { return ws_for(select_bwd_weight(g, dtype), g, dtype); }

int launch_bwd_weight(const Geo &g, const void *x, const void *dy, void *dwt, void *db, void *ws, int dtype,
                      hipStream_t s) {
    switch (dtype) {
        case 0: return dispatch_bwd_weight<float>(g, x, dy, dwt, db, ws, s);
        case 1: return dispatch_bwd_weight<__half>(g, x, dy, dwt, db, ws, s);
        default: return dispatch_bwd_weight<bf16_t>(g, x, dy, dwt, db, ws, s);
    }
}

}  // namespace dw
