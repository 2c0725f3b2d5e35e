// dw_bwd_input.hip -- depthwise gradient with respect to the input on gfx950.
//
// dx is the adjoint of the forward in x (PyTorch PR #3057 ships it as the
// depthwise grad-input kernel).  Instead of scattering every w*dy product into
// dx, each dx element gathers the products that reach it:
//   dx[n,g,h,c] = sum_{m<M} sum_{i,j} w[g*M+m,i,j] * dy[n,g*M+m,(h+ph-i*dh)/sh,(c+pw-j*dw)/sw]
// over the taps where both divisions are exact and land inside dy; every dx
// element is written, including those no tap reaches (they get 0).
//
// Layout mirrors the forward: a workgroup owns a band of dx rows of one input
// plane (or several whole small planes); the dy rows of the M output planes
// that feed it are staged in LDS with 16-byte coalesced loads; each thread
// produces RW adjacent dx values of one row.  With stride 1 the dy row segment
// a strip needs is read into registers once and reused by all its taps.
#include "dw_common.hpp"
#include "dw_internal.hpp"

#include <type_traits>

namespace dw {
namespace {

constexpr int kLdsPref = 32 * 1024;
constexpr int kTargetWG = 2048;
constexpr int kRW = 4;

template <typename T> struct BinArgs {
    const T *dy;
    const T *w;
    T *dx;
    Geo g;
    int G, BH, nbands, NS;
    FastDiv fNS, fBH;
    int nplanes;    // n * ic
    int full;       // whole planes staged
    int vin, vout;
    int seg_slots;  // LDS elements per staged dy segment (band mode), or the whole region
};

template <typename T, int RW>
__device__ __forceinline__ void store_strip(T *p, const float *acc, int valid, bool vec) {
    if (vec && valid >= RW) {
        union {
            T t[RW];
            uint4 v4;
            uint2 v2;
        } u;
#pragma unroll
        for (int q = 0; q < RW; ++q) u.t[q] = from_f32<T>(acc[q]);
        if constexpr (sizeof(T) * RW == 16) {
            *reinterpret_cast<uint4 *>(p) = u.v4;
        } else {
            static_assert(sizeof(T) * RW == 8, "strip store is 8 or 16 bytes");
            *reinterpret_cast<uint2 *>(p) = u.v2;
        }
    } else {
#pragma unroll
        for (int q = 0; q < RW; ++q)
            if (q < valid) p[q] = from_f32<T>(acc[q]);
    }
}

template <typename T, int KH_, int KW_, int S_, int D_, int RW>
__global__ __launch_bounds__(kThreads) void bwd_input_band_kernel(BinArgs<T> a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const Geo &g = a.g;
    const int KH = KH_ ? KH_ : g.kh;
    const int KW = KW_ ? KW_ : g.kw;
    const int SH = S_ ? S_ : g.sh;
    const int SW = S_ ? S_ : g.sw;
    const int DH = D_ ? D_ : g.dh;
    const int DW = D_ ? D_ : g.dw;
    const int KK = KH * KW;
    const int M = g.mult;
    const int tid = threadIdx.x;
    constexpr int VE = Vec<T>::N;

    const int pg = blockIdx.x / a.nbands;
    const int band = blockIdx.x - pg * a.nbands;
    const int P0 = pg * a.G;
    const int Gc = min(a.G, a.nplanes - P0);
    const int h0 = band * a.BH;
    const int h1 = min(h0 + a.BH, g.ih);
    int olo, ohi;
    if (a.full) {
        olo = 0;
        ohi = g.oh;
    } else {
        olo = max(ceildiv(h0 + g.ph - (KH - 1) * DH, SH), 0);
        ohi = min(floordiv(h1 - 1 + g.ph, SH) + 1, g.oh);
    }
    const int R = max(ohi - olo, 0);

    T *ds = reinterpret_cast<T *>(smem);
    const int nseg = a.full ? 1 : M;
    float *wsm = reinterpret_cast<float *>(smem + static_cast<size_t>(nseg) * a.seg_slots * sizeof(T));
    const int64_t oplane = static_cast<int64_t>(g.oh) * g.ow;
    int off0 = 0;
    if (a.full) {
        const int64_t gbeg = static_cast<int64_t>(P0) * M * oplane;
        const int64_t gend = static_cast<int64_t>(P0 + Gc) * M * oplane;
        off0 = a.vin ? lds_copy_range(ds, a.dy, gbeg, gend, tid, kThreads)
                     : lds_copy_range_scalar(ds, a.dy, gbeg, gend, tid, kThreads);
    } else if (R > 0) {
        for (int m = 0; m < M; ++m) {
            const int64_t gbeg = (static_cast<int64_t>(P0) * M + m) * oplane + static_cast<int64_t>(olo) * g.ow;
            const int64_t gend = gbeg + static_cast<int64_t>(R) * g.ow;
            if (a.vin)
                lds_copy_range(ds + m * a.seg_slots, a.dy, gbeg, gend, tid, kThreads);
            else
                lds_copy_range_scalar(ds + m * a.seg_slots, a.dy, gbeg, gend, tid, kThreads);
        }
    }
    const int MKK = M * KK;
    for (int e = tid; e < Gc * MKK; e += kThreads) {
        const int p = e / MKK;
        const int ic = (P0 + p) % g.ic;
        wsm[e] = to_f32(a.w[static_cast<int64_t>(ic) * MKK + (e - p * MKK)]);
    }
    __syncthreads();

    const int rows_out = h1 - h0;
    const int items = Gc * a.BH * a.NS;
    for (int u = tid; u < items; u += kThreads) {
        const int q1 = static_cast<int>(fdiv(static_cast<uint32_t>(u), a.fNS));
        const int s = u - q1 * a.NS;
        const int p = static_cast<int>(fdiv(static_cast<uint32_t>(q1), a.fBH));
        const int r = q1 - p * a.BH;
        if (r >= rows_out) continue;
        const int h = h0 + r;
        const int w0 = s * RW;
        const int P = P0 + p;
        float acc[RW];
#pragma unroll
        for (int q = 0; q < RW; ++q) acc[q] = 0.f;
        for (int m = 0; m < M; ++m) {
            // row o of dy plane (P, m) sits at base + (o - olo) * ow
            const T *base;
            if (a.full) {
                base = ds + off0 + (static_cast<int64_t>(p) * M + m) * oplane;
            } else {
                const int64_t gbeg = (static_cast<int64_t>(P0) * M + m) * oplane + static_cast<int64_t>(olo) * g.ow;
                base = ds + m * a.seg_slots + (a.vin ? static_cast<int>(gbeg & (VE - 1)) : 0);
            }
            const float *wp = wsm + (p * M + m) * KK;
            for (int i = 0; i < KH; ++i) {
                const int t = h + g.ph - i * DH;
                if (t < 0) break;  // t decreases with i
                if (S_ != 1 && (t % SH) != 0) continue;
                const int o = t / SH;
                if (o < olo || o >= ohi) continue;
                const T *rp = base + (o - olo) * g.ow;
                if constexpr (S_ == 1 && KW_ > 0 && D_ > 0) {
                    // dy columns c + pw - j*dw for c in the strip: one window
                    constexpr int WW = (KW_ - 1) * D_ + RW;
                    const int cb = w0 + g.pw - (KW_ - 1) * D_;
                    float win[WW];
#pragma unroll
                    for (int c = 0; c < WW; ++c) {
                        const int col = cb + c;
                        win[c] = (col >= 0 && col < g.ow) ? to_f32(rp[col]) : 0.f;
                    }
#pragma unroll
                    for (int j = 0; j < KW_; ++j) {
                        const float wv = wp[i * KW_ + j];
#pragma unroll
                        for (int q = 0; q < RW; ++q)
                            acc[q] = fmaf(wv, win[(KW_ - 1 - j) * D_ + q], acc[q]);
                    }
                } else {
                    for (int j = 0; j < KW; ++j) {
                        const float wv = wp[i * KW + j];
#pragma unroll
                        for (int q = 0; q < RW; ++q) {
                            const int tc = w0 + q + g.pw - j * DW;
                            if (tc < 0) continue;
                            if (S_ != 1 && (tc % SW) != 0) continue;
                            const int col = tc / SW;
                            if (col < g.ow) acc[q] = fmaf(wv, to_f32(rp[col]), acc[q]);
                        }
                    }
                }
            }
        }
        T *xp = a.dx + (static_cast<int64_t>(P) * g.ih + h) * g.iw + w0;
        store_strip<T, RW>(xp, acc, g.iw - w0, a.vout != 0);
    }
}

template <typename T>
bool plan_bwd_input(const Geo &g, BandPlan &bp, int &seg_slots) {
    const int elem = sizeof(T);
    const int64_t wbytes_pp = static_cast<int64_t>(g.mult) * g.kh * g.kw * 4;
    const int64_t oplane = static_cast<int64_t>(g.oh) * g.ow;
    const int NS = (g.iw + kRW - 1) / kRW;
    auto full_bytes = [&](int G) -> int64_t {
        const int64_t cnt = static_cast<int64_t>(G) * g.mult * oplane;
        if (cnt > (1 << 24)) return INT64_MAX;
        return static_cast<int64_t>(lds_slots<T>(static_cast<int>(cnt))) * elem + G * wbytes_pp;
    };
    auto rows_for = [&](int bh) -> int64_t {
        return std::min<int64_t>((static_cast<int64_t>(bh) - 1 + static_cast<int64_t>(g.kh - 1) * g.dh) / g.sh + 2, g.oh);
    };
    auto band_bytes = [&](int bh) -> int64_t {
        const int64_t cnt = rows_for(bh) * g.ow;
        if (cnt > (1 << 24)) return INT64_MAX;
        return static_cast<int64_t>(g.mult) * lds_slots<T>(static_cast<int>(cnt)) * elem + wbytes_pp;
    };
    if (!plan_bands(g.n * g.ic, g.ih, NS, kLdsPref, kLdsCap, kTargetWG, 1024, full_bytes, band_bytes, bp))
        return false;
    seg_slots = bp.full ? lds_slots<T>(static_cast<int>(bp.G * g.mult * oplane))
                        : lds_slots<T>(static_cast<int>(rows_for(bp.BH) * g.ow));
    return true;
}

template <typename T, int KH, int KW, int S, int D>
int run_bwd_input(const Geo &g, const BandPlan &bp, int seg_slots, const void *dy, const void *w,
                  void *dx, hipStream_t s) {
    BinArgs<T> a;
    a.dy = static_cast<const T *>(dy);
    a.w = static_cast<const T *>(w);
    a.dx = static_cast<T *>(dx);
    a.g = g;
    a.G = bp.G;
    a.BH = bp.BH;
    a.nbands = bp.nbands;
    a.NS = (g.iw + kRW - 1) / kRW;
    const uint64_t items = static_cast<uint64_t>(bp.G) * bp.BH * a.NS;
    a.fNS = make_fastdiv(a.NS, items);
    a.fBH = make_fastdiv(bp.BH, items / a.NS);
    a.nplanes = g.n * g.ic;
    a.full = bp.full;
    a.vin = (reinterpret_cast<uintptr_t>(dy) % 16) == 0;
    a.vout = (g.iw % kRW == 0) && (reinterpret_cast<uintptr_t>(dx) % (kRW * sizeof(T)) == 0);
    a.seg_slots = seg_slots;
    hipLaunchKernelGGL((bwd_input_band_kernel<T, KH, KW, S, D, kRW>), dim3(bp.grid), dim3(kThreads),
                       bp.lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

enum BinAlgo {
    kBinRowwalk = 0, kBinLargek, kBinDecim, kBinBand33s1, kBinBand33s2, kBinBand55s1, kBinBand55s2d2, kBinBandGeneric,
    kBinChannelGroup, kBinLargekMfma, kBinLargekMfma32, kBinDirect, kBinLargekMfmaH16, kBinLargekRoll16, kBinLargekRollF32, kBinCount
};

const char *const kBinNames[kBinCount] = {"rowwalk_3x3",    "largek_regtile", "decimated_s2d2",
                                          "band_3x3_s1",    "band_3x3_s2",    "band_5x5_s1",
                                          "band_5x5_s2_d2", "band_generic",   "channelgroup_small",
                                          "largek_mfma",    "largek_mfma_f32", "direct",
                                          "largek_mfma_h16", "largek_roll16",  "largek_roll_f32"};

bool band_bin_plans(const Geo &g, int dt) {
    BandPlan bp;
    int ss;
    return dt == 0 ? plan_bwd_input<float>(g, bp, ss) : plan_bwd_input<__half>(g, bp, ss);
}

bool feasible_bin(int algo, const Geo &g, int dt) {
    const bool sq = g.kh == g.kw && g.sh == g.sw && g.dh == g.dw;
    switch (algo) {
        case kBinRowwalk: return rowwalk_fits(g, dt, 1);
        case kBinLargek: return largek_fits(g, 1);
        case kBinDecim: return decim_fits(g, 1);
        case kBinChannelGroup: return small_bwd_input_fits(g, dt);
        case kBinLargekMfma: return largek_mfma_fits(g, 1, dt);
        case kBinLargekMfma32: return largek_fwd32_fits(g, 1, dt);
        case kBinLargekMfmaH16: return largek_mfma16_fits(g, 1, dt);
        case kBinLargekRoll16: return largek_roll16_fits(g, 1, dt);
        case kBinLargekRollF32: return largek_rollf32_fits(g, 1, dt);
        case kBinBand33s1: return sq && g.kh == 3 && g.sh == 1 && g.dh == 1 && band_bin_plans(g, dt);
        case kBinBand33s2: return sq && g.kh == 3 && g.sh == 2 && g.dh == 1 && band_bin_plans(g, dt);
        case kBinBand55s1: return sq && g.kh == 5 && g.sh == 1 && g.dh == 1 && band_bin_plans(g, dt);
        case kBinBand55s2d2: return sq && g.kh == 5 && g.sh == 2 && g.dh == 2 && band_bin_plans(g, dt);
        case kBinBandGeneric: return band_bin_plans(g, dt);
        case kBinDirect: return true;
        default: return false;
    }
}

// The kernel family a grad-input call launches: the selection table's entry
// for this geometry, else the built-in rules.
int select_bwd_input(const Geo &g, int dt) {
    const int tuned = tuned_algo(1, g, dt);
    if (tuned >= 0 && feasible_bin(tuned, g, dt)) return tuned;
    if (decim_fits(g, 1)) return kBinDecim;
    if (small_bwd_input_fits(g, dt)) return kBinChannelGroup;
    if (rowwalk_fits(g, dt, 1)) return kBinRowwalk;
    // 16-bit 7 x 7 and 13 x 13 on planes of at least 32 x 32: input rows streamed
    // past slots of output rows on the matrix cores, measured 1.2-1.5x faster
    // than the tiles at 48 and 64 rows, level at 32
    if ((g.kh == 7 || g.kh == 13) && g.ih >= 32 && g.ow >= 32 && largek_roll16_fits(g, 1, dt)) return kBinLargekRoll16;
    // 16-bit k = 7 planes wider or taller than 32: 16 x 16 tiles measured ~5 % faster
    if (g.kh == 7 && (g.ih > 32 || g.iw > 32) && largek_mfma16_fits(g, 1, dt)) return kBinLargekMfmaH16;
    // 16-bit 31 x 31: input rows streamed through rotating filter rows
    if (g.kh == 31 && largek_roll16_fits(g, 1, dt)) return kBinLargekRoll16;
    // fp32 31 x 31 on planes of at least 32 x 32: input rows streamed past
    // rotating filter rows, measured 1.05-1.27x faster than the kernel-row
    // contraction, whose anti-diagonal sums add vector work to the matrix time
    if (g.kh == 31 && g.ih >= 32 && g.ow >= 32 && largek_rollf32_fits(g, 1, dt)) return kBinLargekRollF32;
    if (largek_mfma_fits(g, 1, dt)) return kBinLargekMfma;
    if (largek_fwd32_fits(g, 1, dt) && largek_fwd32_preferred(g, 1)) return kBinLargekMfma32;
    if (largek_fits(g, 1)) return kBinLargek;
    if (!band_bin_plans(g, dt)) return kBinDirect;  // rows too wide to stage
    const bool sq = g.kh == g.kw && g.sh == g.sw && g.dh == g.dw;
    if (sq && g.kh == 3 && g.sh == 1 && g.dh == 1) return kBinBand33s1;
    if (sq && g.kh == 3 && g.sh == 2 && g.dh == 1) return kBinBand33s2;
    if (sq && g.kh == 5 && g.sh == 1 && g.dh == 1) return kBinBand55s1;
    if (sq && g.kh == 5 && g.sh == 2 && g.dh == 2) return kBinBand55s2d2;
    return kBinBandGeneric;
}

template <typename T>
int dispatch_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t s) {
    const int dt = sizeof(T) == 4 ? 0 : (std::is_same<T, __half>::value ? 1 : 2);
    const int algo = select_bwd_input(g, dt);
    if (algo == kBinRowwalk) return rowwalk_bwd_input(g, dy, w, dx, dt, s);
    if (algo == kBinLargek) return largek_bwd_input(g, dy, w, dx, dt, s);
    if (algo == kBinLargekMfma) return largek_mfma_bwd_input(g, dy, w, dx, dt, s);
    if (algo == kBinLargekMfma32) return largek_bwd_input32(g, dy, w, dx, s);
    if (algo == kBinLargekMfmaH16) return largek_mfma16_bwd_input(g, dy, w, dx, dt, s);
    if (algo == kBinLargekRoll16) return largek_roll16_bwd_input(g, dy, w, dx, dt, s);
    if (algo == kBinLargekRollF32) return largek_rollf32_bwd_input(g, dy, w, dx, s);
    if (algo == kBinDecim) return decim_bwd_input(g, dy, w, dx, dt, s);
    if (algo == kBinChannelGroup) return small_bwd_input(g, dy, w, dx, dt, s);
    if (algo == kBinDirect) return direct_bwd_input(g, dy, w, dx, dt, s);
    BandPlan bp;
    int seg_slots = 0;
    if (!plan_bwd_input<T>(g, bp, seg_slots)) return kErrUnsupported;
    switch (algo) {
        case kBinBand33s1: return run_bwd_input<T, 3, 3, 1, 1>(g, bp, seg_slots, dy, w, dx, s);
        case kBinBand33s2: return run_bwd_input<T, 3, 3, 2, 1>(g, bp, seg_slots, dy, w, dx, s);
        case kBinBand55s1: return run_bwd_input<T, 5, 5, 1, 1>(g, bp, seg_slots, dy, w, dx, s);
        case kBinBand55s2d2: return run_bwd_input<T, 5, 5, 2, 2>(g, bp, seg_slots, dy, w, dx, s);
        default: return run_bwd_input<T, 0, 0, 0, 0>(g, bp, seg_slots, dy, w, dx, s);
    }
}

}  // namespace

const char *bwd_input_algo_name(const Geo &g, int dtype) { return kBinNames[select_bwd_input(g, dtype)]; }

int bwd_input_algo_count() { return kBinCount; }
const char *bwd_input_algo_name_of(int algo) { return algo >= 0 && algo < kBinCount ? kBinNames[algo] : nullptr; }
bool bwd_input_algo_feasible(int algo, const Geo &g, int dtype) { return feasible_bin(algo, g, dtype); }

bool bwd_input_supported(const Geo &, int) { return true; }  // the direct kernel serves every geometry

int launch_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return dispatch_bwd_input<float>(g, dy, w, dx, s);
        case 1: return dispatch_bwd_input<__half>(g, dy, w, dx, s);
        default: return dispatch_bwd_input<bf16_t>(g, dy, w, dx, s);
    }
}

}  // namespace dw
