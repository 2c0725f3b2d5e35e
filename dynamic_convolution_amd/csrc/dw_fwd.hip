// dw_fwd.hip -- depthwise forward on gfx950.
//
// Computes y[n,o,p,q] = b[o] + sum_ij w[o,i,j] x[n,o/M, p*sh-ph+i*dh, q*sw-pw+j*dw]
// (PyTorch PR #3057, depthwise forward with padding, stride, dilation,
// multiplier and bias; problem shapes as in the MegEngine large-kernel
// depthwise article's im2col problem statement).
//
// Design: one workgroup owns a band of output rows of one (n, ic) plane, or
// several whole small planes.  The input rows the band needs form one
// contiguous range of NCHW memory, so they are staged into LDS with 16-byte
// coalesced loads; then each thread produces a strip of RW adjacent outputs of
// one row for every one of the M output channels that read this input plane,
// and stores them with one vector store when the row layout allows.  For the
// common small filters the kernel size, stride and dilation are compile-time
// constants and each input row segment a strip needs is read from LDS once
// into registers (a sliding window) and reused by all its taps.
#include "dw_common.hpp"
#include "dw_internal.hpp"

#include <type_traits>

namespace dw {
namespace {

constexpr int kLdsPref = 32 * 1024;  // preferred LDS per workgroup: 5 workgroups per CU
constexpr int kTargetWG = 2048;      // aim for >= 8 workgroups per CU
constexpr int kRW = 4;               // outputs per thread strip

template <typename T> struct FwdArgs {
    const T *x;
    const T *w;
    const T *b;
    T *y;
    Geo g;
    int G;       // input planes per workgroup
    int BH;      // output rows per band
    int nbands;  // bands per plane
    int NS;      // strips per output row
    FastDiv fNS, fBH;
    int nplanes;   // n * ic
    int full;      // whole planes staged (nbands == 1)
    int vin;       // x is 16-byte aligned: vector staging
    int vout;      // y rows start on RW-vector boundaries
    int xs_slots;  // LDS elements reserved for staged x
};

template <typename T, int RW>
__device__ __forceinline__ void store_strip(T *p, const float *acc, int valid, bool vec) {
    if (vec && valid >= RW) {
        union {
            T t[RW];
            uint4 v4;
            uint2 v2;
            uint32_t v1;
        } u;
#pragma unroll
        for (int q = 0; q < RW; ++q) u.t[q] = from_f32<T>(acc[q]);
        if constexpr (sizeof(T) * RW == 16) {
            *reinterpret_cast<uint4 *>(p) = u.v4;
        } else if constexpr (sizeof(T) * RW == 8) {
            *reinterpret_cast<uint2 *>(p) = u.v2;
        } else {
#pragma unroll
            for (int q = 0; q < RW; ++q) p[q] = u.t[q];
        }
    } else {
#pragma unroll
        for (int q = 0; q < RW; ++q)
            if (q < valid) p[q] = from_f32<T>(acc[q]);
    }
}

template <typename T, int KH_, int KW_, int SH_, int SW_, int DH_, int DW_, int RW>
__global__ __launch_bounds__(kThreads) void fwd_band_kernel(FwdArgs<T> a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const Geo &g = a.g;
    const int KH = KH_ ? KH_ : g.kh;
    const int KW = KW_ ? KW_ : g.kw;
    const int SH = SH_ ? SH_ : g.sh;
    const int SW = SW_ ? SW_ : g.sw;
    const int DH = DH_ ? DH_ : g.dh;
    const int DW = DW_ ? DW_ : g.dw;
    const int KK = KH * KW;
    const int M = g.mult;
    const int tid = threadIdx.x;

    const int pg = blockIdx.x / a.nbands;
    const int band = blockIdx.x - pg * a.nbands;
    const int P0 = pg * a.G;
    const int Gc = min(a.G, a.nplanes - P0);
    const int oh0 = band * a.BH;
    const int oh1 = min(oh0 + a.BH, g.oh);
    int rlo, rhi;
    if (a.full) {
        rlo = 0;
        rhi = g.ih;
    } else {
        rlo = max(oh0 * SH - g.ph, 0);
        rhi = min((oh1 - 1) * SH - g.ph + (KH - 1) * DH + 1, g.ih);
    }
    const int R = rhi - rlo;

    T *xs = reinterpret_cast<T *>(smem);
    float *wsm = reinterpret_cast<float *>(smem + static_cast<size_t>(a.xs_slots) * sizeof(T));
    const int64_t plane_elems = static_cast<int64_t>(g.ih) * g.iw;
    int off = 0;
    if (R > 0) {
        const int64_t gbeg = static_cast<int64_t>(P0) * plane_elems + static_cast<int64_t>(rlo) * g.iw;
        const int64_t gend = a.full ? static_cast<int64_t>(P0 + Gc) * plane_elems
                                    : gbeg + static_cast<int64_t>(R) * g.iw;
        off = a.vin ? lds_copy_range(xs, a.x, gbeg, gend, tid, kThreads)
                    : lds_copy_range_scalar(xs, a.x, gbeg, gend, tid, kThreads);
    }
    const int MKK = M * KK;
    for (int e = tid; e < Gc * MKK; e += kThreads) {
        const int p = e / MKK;
        const int ic = (P0 + p) % g.ic;
        wsm[e] = to_f32(a.w[static_cast<int64_t>(ic) * MKK + (e - p * MKK)]);
    }
    __syncthreads();

    const int rows_out = oh1 - oh0;
    const int items = Gc * a.BH * a.NS;
    const int pstride = a.full ? static_cast<int>(plane_elems) : R * g.iw;
    for (int u = tid; u < items; u += kThreads) {
        const int q1 = static_cast<int>(fdiv(static_cast<uint32_t>(u), a.fNS));
        const int s = u - q1 * a.NS;
        const int p = static_cast<int>(fdiv(static_cast<uint32_t>(q1), a.fBH));
        const int r = q1 - p * a.BH;
        if (r >= rows_out) continue;
        const int oh = oh0 + r;
        const int ow0 = s * RW;
        const int P = P0 + p;
        const int ic = P % g.ic;
        const T *xp = xs + off + p * pstride;
        const int valid = g.ow - ow0;
        for (int m = 0; m < M; ++m) {
            const float bv = a.b ? to_f32(a.b[ic * M + m]) : 0.f;
            float acc[RW];
#pragma unroll
            for (int q = 0; q < RW; ++q) acc[q] = bv;
            const float *wp = wsm + (p * M + m) * KK;
            if constexpr (KW_ > 0 && SW_ > 0 && DW_ > 0) {
                // sliding window: each needed input element of the row read once
                constexpr int WW = (RW - 1) * SW_ + (KW_ - 1) * DW_ + 1;
                const int c0 = ow0 * SW_ - g.pw;
#pragma unroll
                for (int i = 0; i < KH; ++i) {
                    const int ih = oh * SH - g.ph + i * DH;
                    if (ih < rlo || ih >= rhi) continue;
                    const T *rp = xp + (ih - rlo) * g.iw;
                    float win[WW];
#pragma unroll
                    for (int c = 0; c < WW; ++c) {
                        const int col = c0 + c;
                        win[c] = (col >= 0 && col < g.iw) ? to_f32(rp[col]) : 0.f;
                    }
#pragma unroll
                    for (int j = 0; j < KW_; ++j) {
                        const float wv = wp[i * KW_ + j];
#pragma unroll
                        for (int q = 0; q < RW; ++q) acc[q] = fmaf(wv, win[q * SW_ + j * DW_], acc[q]);
                    }
                }
            } else {
                for (int i = 0; i < KH; ++i) {
                    const int ih = oh * SH - g.ph + i * DH;
                    if (ih < rlo || ih >= rhi) continue;
                    const T *rp = xp + (ih - rlo) * g.iw;
                    for (int j = 0; j < KW; ++j) {
                        const float wv = wp[i * KW + j];
                        const int cb = ow0 * SW - g.pw + j * DW;
#pragma unroll
                        for (int q = 0; q < RW; ++q) {
                            const int col = cb + q * SW;
                            const float v = (col >= 0 && col < g.iw) ? to_f32(rp[col]) : 0.f;
                            acc[q] = fmaf(wv, v, acc[q]);
                        }
                    }
                }
            }
            T *yp = a.y + (static_cast<int64_t>(P * M + m) * g.oh + oh) * g.ow + ow0;
            store_strip<T, RW>(yp, acc, valid, a.vout != 0);
        }
    }
}

template <typename T>
bool plan_fwd(const Geo &g, BandPlan &bp) {
    const int elem = sizeof(T);
    const int64_t wbytes_pp = static_cast<int64_t>(g.mult) * g.kh * g.kw * 4;  // staged weights per plane
    const int64_t plane_in = static_cast<int64_t>(g.ih) * g.iw;
    const int NS = (g.ow + kRW - 1) / kRW;
    auto full_bytes = [&](int G) -> int64_t {
        const int64_t cnt = G * plane_in;
        if (cnt > (1 << 24)) return INT64_MAX;
        return static_cast<int64_t>(lds_slots<T>(static_cast<int>(cnt))) * elem + G * wbytes_pp;
    };
    auto band_bytes = [&](int bh) -> int64_t {
        const int64_t rows = std::min<int64_t>(
            (static_cast<int64_t>(bh) - 1) * g.sh + static_cast<int64_t>(g.kh - 1) * g.dh + 1, g.ih);
        const int64_t cnt = rows * g.iw;
        if (cnt > (1 << 24)) return INT64_MAX;
        return static_cast<int64_t>(lds_slots<T>(static_cast<int>(cnt))) * elem + wbytes_pp;
    };
    return plan_bands(g.n * g.ic, g.oh, NS, kLdsPref, kLdsCap, kTargetWG, 1024, full_bytes,
                      band_bytes, bp);
}

template <typename T, int KH, int KW, int SH, int SW, int DH, int DW>
int run_fwd(const Geo &g, const BandPlan &bp, const void *x, const void *w, const void *b, void *y,
            hipStream_t s) {
    FwdArgs<T> a;
    a.x = static_cast<const T *>(x);
    a.w = static_cast<const T *>(w);
    a.b = static_cast<const T *>(b);
    a.y = static_cast<T *>(y);
    a.g = g;
    a.G = bp.G;
    a.BH = bp.BH;
    a.nbands = bp.nbands;
    a.NS = (g.ow + kRW - 1) / kRW;
    const uint64_t items = static_cast<uint64_t>(bp.G) * bp.BH * a.NS;
    a.fNS = make_fastdiv(a.NS, items);
    a.fBH = make_fastdiv(bp.BH, items / a.NS);
    a.nplanes = g.n * g.ic;
    a.full = bp.full;
    a.vin = (reinterpret_cast<uintptr_t>(x) % 16) == 0;
    a.vout = (g.ow % kRW == 0) && (reinterpret_cast<uintptr_t>(y) % (kRW * sizeof(T)) == 0);
    if (bp.full) {
        a.xs_slots = lds_slots<T>(bp.G * g.ih * g.iw);
    } else {
        const int rows = std::min((bp.BH - 1) * g.sh + (g.kh - 1) * g.dh + 1, g.ih);
        a.xs_slots = lds_slots<T>(rows * g.iw);
    }
    hipLaunchKernelGGL((fwd_band_kernel<T, KH, KW, SH, SW, DH, DW, kRW>), dim3(bp.grid), dim3(kThreads),
                       bp.lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

enum FwdAlgo {
    kFwdRowwalk = 0, kFwdLargek, kFwdDecim, kFwdBand33s1, kFwdBand33s2, kFwdBand55s1, kFwdBand55s2d2, kFwdBandGeneric,
    kFwdChannelGroup, kFwdLargekMfma, kFwdLargekMfma32, kFwdDirect, kFwdLargekMfmaH16, kFwdLargekRoll16, kFwdLargekRollF32, kFwdCount
};

const char *const kFwdNames[kFwdCount] = {"rowwalk_3x3",    "largek_regtile", "decimated_s2d2",
                                          "band_3x3_s1",    "band_3x3_s2",    "band_5x5_s1",
                                          "band_5x5_s2_d2", "band_generic",   "channelgroup_small",
                                          "largek_mfma",    "largek_mfma_f32", "direct",
                                          "largek_mfma_h16", "largek_roll16",  "largek_roll_f32"};

bool band_fwd_plans(const Geo &g, int dt) {
    BandPlan bp;
    return dt == 0 ? plan_fwd<float>(g, bp) : plan_fwd<__half>(g, bp);
}

// Whether family `algo` can run this geometry (each family's own fit test;
// the specialised band variants need their exact geometry).
bool feasible_fwd(int algo, const Geo &g, int dt) {
    const bool sq = g.kh == g.kw && g.sh == g.sw && g.dh == g.dw;
    switch (algo) {
        case kFwdRowwalk: return rowwalk_fits(g, dt, 0);
        case kFwdLargek: return largek_fits(g, 0);
        case kFwdDecim: return decim_fits(g, 0);
        case kFwdChannelGroup: return small_fwd_fits(g, dt);
        case kFwdLargekMfma: return largek_mfma_fits(g, 0, dt);
        case kFwdLargekMfma32: return largek_fwd32_fits(g, 0, dt);
        case kFwdLargekMfmaH16: return largek_mfma16_fits(g, 0, dt);
        case kFwdLargekRoll16: return largek_roll16_fits(g, 0, dt);
        case kFwdLargekRollF32: return largek_rollf32_fits(g, 0, dt);
        case kFwdBand33s1: return sq && g.kh == 3 && g.sh == 1 && g.dh == 1 && band_fwd_plans(g, dt);
        case kFwdBand33s2: return sq && g.kh == 3 && g.sh == 2 && g.dh == 1 && band_fwd_plans(g, dt);
        case kFwdBand55s1: return sq && g.kh == 5 && g.sh == 1 && g.dh == 1 && band_fwd_plans(g, dt);
        case kFwdBand55s2d2: return sq && g.kh == 5 && g.sh == 2 && g.dh == 2 && band_fwd_plans(g, dt);
        case kFwdBandGeneric: return band_fwd_plans(g, dt);
        case kFwdDirect: return true;
        default: return false;
    }
}

// The kernel family a forward call launches (the dispatcher and the
// introspection helper both use this one decision): a family recorded in the
// selection table for this geometry, else the built-in rules.
int select_fwd(const Geo &g, int dt) {
    const int tuned = tuned_algo(0, g, dt);
    if (tuned >= 0 && feasible_fwd(tuned, g, dt)) return tuned;
    if (rowwalk_fits(g, dt, 0)) return kFwdRowwalk;
    // 16-bit 7 x 7 and 13 x 13 on planes of at least 32 x 32: input rows streamed
    // past slots of output rows on the matrix cores, measured 1.2-1.5x faster
    // than the tiles at 48 and 64 rows, level at 32
    if ((g.kh == 7 || g.kh == 13) && g.ih >= 32 && g.ow >= 32 && largek_roll16_fits(g, 0, dt)) return kFwdLargekRoll16;
    // 16-bit k = 7 planes wider or taller than 32: 16 x 16 tiles measured ~10 % faster
    if (g.kh == 7 && (g.oh > 32 || g.ow > 32) && largek_mfma16_fits(g, 0, dt)) return kFwdLargekMfmaH16;
    // 16-bit 31 x 31: input rows streamed through rotating filter rows
    if (g.kh == 31 && largek_roll16_fits(g, 0, dt)) return kFwdLargekRoll16;
    // fp32 31 x 31 on planes of at least 32 x 32: input rows streamed past
    // rotating filter rows, measured 1.05-1.27x faster than the kernel-row
    // contraction, whose anti-diagonal sums add vector work to the matrix time
    if (g.kh == 31 && g.ih >= 32 && g.ow >= 32 && largek_rollf32_fits(g, 0, dt)) return kFwdLargekRollF32;
    if (largek_mfma_fits(g, 0, dt)) return kFwdLargekMfma;
    if (largek_fwd32_fits(g, 0, dt) && largek_fwd32_preferred(g, 0)) return kFwdLargekMfma32;
    if (largek_fits(g, 0)) return kFwdLargek;
    if (decim_fits(g, 0)) return kFwdDecim;
    if (small_fwd_fits(g, dt)) return kFwdChannelGroup;
    if (!band_fwd_plans(g, dt)) return kFwdDirect;  // rows too wide to stage
    const bool sq = g.kh == g.kw && g.sh == g.sw && g.dh == g.dw;
    if (sq && g.kh == 3 && g.sh == 1 && g.dh == 1) return kFwdBand33s1;
    if (sq && g.kh == 3 && g.sh == 2 && g.dh == 1) return kFwdBand33s2;
    if (sq && g.kh == 5 && g.sh == 1 && g.dh == 1) return kFwdBand55s1;
    if (sq && g.kh == 5 && g.sh == 2 && g.dh == 2) return kFwdBand55s2d2;
    return kFwdBandGeneric;
}

template <typename T>
int dispatch_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, hipStream_t s) {
    const int dt = sizeof(T) == 4 ? 0 : (std::is_same<T, __half>::value ? 1 : 2);
    const int algo = select_fwd(g, dt);
    if (algo == kFwdRowwalk) return rowwalk_fwd(g, x, w, b, y, dt, s);
    if (algo == kFwdLargek) return largek_fwd(g, x, w, b, y, dt, s);
    if (algo == kFwdLargekMfma) return largek_mfma_fwd(g, x, w, b, y, dt, s);
    if (algo == kFwdLargekMfma32) return largek_fwd32(g, x, w, b, y, s);
    if (algo == kFwdLargekMfmaH16) return largek_mfma16_fwd(g, x, w, b, y, dt, s);
    if (algo == kFwdLargekRoll16) return largek_roll16_fwd(g, x, w, b, y, dt, s);
    if (algo == kFwdLargekRollF32) return largek_rollf32_fwd(g, x, w, b, y, s);
    if (algo == kFwdDecim) return decim_fwd(g, x, w, b, y, dt, s);
    if (algo == kFwdChannelGroup) return small_fwd(g, x, w, b, y, dt, s);
    if (algo == kFwdDirect) return direct_fwd(g, x, w, b, y, dt, s);
    BandPlan bp;
    if (!plan_fwd<T>(g, bp)) return kErrUnsupported;
    switch (algo) {
        case kFwdBand33s1: return run_fwd<T, 3, 3, 1, 1, 1, 1>(g, bp, x, w, b, y, s);
        case kFwdBand33s2: return run_fwd<T, 3, 3, 2, 2, 1, 1>(g, bp, x, w, b, y, s);
        case kFwdBand55s1: return run_fwd<T, 5, 5, 1, 1, 1, 1>(g, bp, x, w, b, y, s);
        case kFwdBand55s2d2: return run_fwd<T, 5, 5, 2, 2, 2, 2>(g, bp, x, w, b, y, s);
        default: return run_fwd<T, 0, 0, 0, 0, 0, 0>(g, bp, x, w, b, y, s);
    }
}

}  // namespace

const char *fwd_algo_name(const Geo &g, int dtype) { return kFwdNames[select_fwd(g, dtype)]; }

int fwd_algo_count() { return kFwdCount; }
const char *fwd_algo_name_of(int algo) { return algo >= 0 && algo < kFwdCount ? kFwdNames[algo] : nullptr; }
bool fwd_algo_feasible(int algo, const Geo &g, int dtype) { return feasible_fwd(algo, g, dtype); }

bool fwd_supported(const Geo &, int) { return true; }  // the direct kernel serves every geometry

int launch_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype,
               hipStream_t s) {
    switch (dtype) {
        case 0: return dispatch_fwd<float>(g, x, w, b, y, s);
        case 1: return dispatch_fwd<__half>(g, x, w, b, y, s);
        default: return dispatch_fwd<bf16_t>(g, x, w, b, y, s);
    }
}

}  // namespace dw
