// dw_small.hip -- depthwise grad-weight for small planes on gfx950.
//
//   dw[o,i,j] = sum_{n,p,q} dy[n,o,p,q] * x[n,o/M, p*s-pad+i*d, q*s-pad+j*d],  db[o] = sum dy
// (PyTorch PR #3057: grad-weight and grad-bias of the depthwise convolution.)
//
// For small planes (up to 14x14 outputs) one channel's data is a
// 200-4000 byte piece per image, scattered with the stride of a whole image,
// and a per-channel walk reads short rows from many places.  Here a workgroup
// owns G adjacent channels instead: for a fixed image their x planes are one
// contiguous range and their dy planes another, and the workgroup walks a
// chunk of images, staging one image's two ranges in LDS at a time.  When the
// ranges are whole 16-byte vectors the next image's vectors are loaded into
// registers while the current image is computed.
//
// Each lane owns one (channel, output row) for the whole chunk: per image it
// reads its dy row and the kh input rows under it from LDS and accumulates the
// kh*kw tap sums and the bias sum in registers, so the sum over images needs
// no cross-lane step.  At the end the output rows of each channel are added
// in a fixed order through LDS and one lane per (channel, slot) writes the
// (channel, image chunk) partial to the workspace [ic][chunk][M*(kh*kw+1)]
// that pass 2 adds up.
#include "dw_common.hpp"
#include "dw_internal.hpp"

namespace dw {
namespace {

constexpr int kStageCap = 16 * 1024;  // staged bytes per image and workgroup
constexpr int kPV = kStageCap / (16 * kThreads);  // 16-byte vectors per lane and image
constexpr int kRedCh = 16;            // accumulators per lane per reduction step

template <typename T> struct SwArgs {
    const T *x;
    const T *dy;
    float *ws;
    Geo g;
    int G;             // channels per workgroup
    int NC, npc;       // image chunks, images per chunk
    int gpre;          // LDS elements before the x planes (left-pad reads)
    int dofs;          // LDS element index of the first dy plane
    int vec;           // every staged range is whole, aligned 16-byte vectors
};

// In-row positions a lane touches: q*S + j*D for q < OWM, j < K.
template <int K, int S, int D, int OWM> struct RowSpan {
    static constexpr int IWM = (OWM - 1) * S + (K - 1) * D + 1;
};

template <typename T, int K, int S, int D, int MM, int OWM>
__global__ __launch_bounds__(kThreads) void sp_bwdw_kernel(SwArgs<T> a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int KK = K * K;
    constexpr int NT = MM * (KK + 1);
    constexpr int IWM = RowSpan<K, S, D, OWM>::IWM;
    constexpr int VE = Vec<T>::N;
    const Geo &g = a.g;
    const int tid = threadIdx.x;
    // consecutive workgroups take adjacent channel groups of the same images,
    // so the groups in flight read a few long stretches of memory
    const int ngroups = (g.ic + a.G - 1) / a.G;
    const int chunk = blockIdx.x / ngroups;
    const int cg = blockIdx.x - chunk * ngroups;
    const int c0 = cg * a.G;
    const int Gc = min(a.G, g.ic - c0);
    const int iplane = g.ih * g.iw, oplane = g.oh * g.ow;
    const int ch = tid / g.oh;
    const int r = tid - ch * g.oh;
    const bool active = ch < Gc;
    T *lds = reinterpret_cast<T *>(smem);
    T *xs = lds + a.gpre;
    T *ds = lds + a.dofs;
    const int xlen = Gc * iplane, dlen = Gc * MM * oplane;
    const int nvx = xlen / VE, nv = nvx + dlen / VE;

    float acc[MM][KK + 1];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t <= KK; ++t) acc[m][t] = 0.f;

    const int n_beg = chunk * a.npc;
    const int n_end = min(n_beg + a.npc, g.n);
    auto xbase = [&](int n) { return (static_cast<int64_t>(n) * g.ic + c0) * iplane; };
    auto dbase = [&](int n) { return (static_cast<int64_t>(n) * g.oc + static_cast<int64_t>(c0) * MM) * oplane; };

    // register-staged 16-byte vectors of one image: lane vector k is flat
    // vector tid + k*kThreads of [x range | dy range]; lanes past the end load
    // the first x vector again (a valid address) and store nothing
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    v4u pf[kPV];
    auto issue = [&](int n) {
        const T *xb = a.x + xbase(n), *db = a.dy + dbase(n);
#pragma unroll
        for (int k = 0; k < kPV; ++k) {
            const int f = tid + k * kThreads;
            const T *p = f < nvx ? xb + f * VE : (f < nv ? db + (f - nvx) * VE : xb);
            pf[k] = *reinterpret_cast<const v4u *>(p);
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int k = 0; k < kPV; ++k) {
            const int f = tid + k * kThreads;
            if (f < nv) {
                T *q = f < nvx ? xs + f * VE : ds + (f - nvx) * VE;
                *reinterpret_cast<v4u *>(q) = pf[k];
            }
        }
    };

    // uniform column masks: position p of a row window reads column p - pw
    uint64_t colok = 0;
#pragma unroll
    for (int p = 0; p < IWM; ++p) {
        const int c = p - g.pw;
        if (c >= 0 && c < g.iw) colok |= 1ull << p;
    }

    if (a.vec && n_beg < n_end) issue(n_beg);
    for (int n = n_beg; n < n_end; ++n) {
        __syncthreads();  // the previous image's LDS reads are done
        if (a.vec) {
            commit();
        } else {
            const int64_t xb = xbase(n), db = dbase(n);
            for (int e = tid; e < xlen; e += kThreads) xs[e] = a.x[xb + e];
            for (int e = tid; e < dlen; e += kThreads) ds[e] = a.dy[db + e];
        }
        __syncthreads();
        if (a.vec && n + 1 < n_end) issue(n + 1);
        if (active) {
            const T *dp = ds + ch * MM * oplane + r * g.ow;
            float dv[MM][OWM];
#pragma unroll
            for (int m = 0; m < MM; ++m)
#pragma unroll
                for (int q = 0; q < OWM; ++q) {
                    const float v = to_f32(dp[m * oplane + q]);
                    dv[m][q] = q < g.ow ? v : 0.f;
                    acc[m][KK] += dv[m][q];
                }
#pragma unroll
            for (int i = 0; i < K; ++i) {
                const int ih = r * S - g.ph + i * D;
                const bool rowok = ih >= 0 && ih < g.ih;
                const T *xr = xs + ch * iplane + (rowok ? ih : 0) * g.iw - g.pw;
                float xv[IWM];
#pragma unroll
                for (int p = 0; p < IWM; ++p) {
                    const float v = to_f32(xr[p]);
                    xv[p] = (colok >> p) & 1 ? v : 0.f;
                }
#pragma unroll
                for (int j = 0; j < K; ++j)
#pragma unroll
                    for (int m = 0; m < MM; ++m) {
                        float t = 0.f;
#pragma unroll
                        for (int q = 0; q < OWM; ++q) t = fmaf(dv[m][q], xv[q * S + j * D], t);
                        acc[m][i * K + j] += rowok ? t : 0.f;
                    }
            }
        }
    }

    // fixed-order sum over the output rows of each channel, kRedCh slots at a time
    float *red = reinterpret_cast<float *>(smem);
    constexpr int RC = NT < kRedCh ? NT : kRedCh;
#pragma unroll
    for (int t0 = 0; t0 < NT; t0 += RC) {
        __syncthreads();
#pragma unroll
        for (int tt = 0; tt < RC; ++tt) {
            const int t = t0 + tt;
            if (t < NT) red[tid * RC + tt] = acc[t / (KK + 1)][t % (KK + 1)];
        }
        __syncthreads();
        for (int idx = tid; idx < Gc * RC; idx += kThreads) {
            const int c = idx / RC, tt = idx - c * RC;
            if (t0 + tt >= NT) continue;
            float s = 0.f;
            for (int rr = 0; rr < g.oh; ++rr) s += red[(c * g.oh + rr) * RC + tt];
            a.ws[(static_cast<int64_t>(c0 + c) * a.NC + chunk) * NT + t0 + tt] = s;
        }
    }
}

struct SwPlan {
    int G, NC, npc, grid, gpre, dofs, lds_bytes, vec, owm;
};

bool combo_ok(const Geo &g) {
    const bool sq = g.kh == g.kw && g.sh == g.sw && g.dh == g.dw;
    return g.mult <= 2 && sq &&
           ((g.kh == 3 && g.dh == 1 && g.sh <= 2) || (g.kh == 5 && ((g.sh == 1 && g.dh == 1) || (g.sh == 2 && g.dh == 2))));
}

int row_span(const Geo &g, int owm) { return (owm - 1) * g.sw + (g.kw - 1) * g.dw + 1; }

template <typename T>
bool plan_sp_bwdw(const Geo &g, SwPlan &p) {
    if (!combo_ok(g)) return false;
    const int sz = sizeof(T), VE = 16 / sz;
    const int64_t iplane = static_cast<int64_t>(g.ih) * g.iw, oplane = static_cast<int64_t>(g.oh) * g.ow;
    // used for planes of at most 256 output pixels and rows of at most 16
    // (7x7, 14x14, 28x28 at stride 2): larger planes measured faster with the
    // streaming row walk
    if (oplane > 256 || g.ow > 16 || g.oh > kThreads) return false;
    p.owm = g.ow <= 4 ? 4 : (g.ow <= 8 ? 8 : 16);
    const int64_t per_ch = (iplane + g.mult * oplane) * sz;
    int G = std::min<int64_t>(kThreads / g.oh, g.ic);
    while (G > 1 && G * per_ch > kStageCap) --G;
    if (G * per_ch > kStageCap) return false;
    // whole 16-byte vectors: every image's range of every channel group starts
    // and ends on a vector boundary (base pointers are checked at launch)
    bool vec = (g.ic * iplane) % VE == 0 && (static_cast<int64_t>(g.oc) * oplane) % VE == 0;
    if (vec) {
        int Gv = G;
        while (Gv > 0 && ((Gv * iplane) % VE != 0 || (Gv * g.mult * oplane) % VE != 0)) --Gv;
        if (Gv > 0) G = Gv; else vec = false;
    }
    const int ngroups = (g.ic + G - 1) / G;
    // about 1536 workgroups (six per CU) with at least four images each when
    // the batch allows, so loads of the next image overlap the current one
    int NC = std::max(1, (1536 + ngroups - 1) / ngroups);
    NC = std::min(NC, std::max(1, g.n / 4));
    const int npc = (g.n + NC - 1) / NC;
    NC = (g.n + npc - 1) / npc;
    const int iwm = row_span(g, p.owm);
    p.G = G;
    p.NC = NC;
    p.npc = npc;
    p.grid = ngroups * NC;
    p.vec = vec;
    // LDS: [left guard][x planes][pad][dy planes][right guard]; the guards and
    // the pad keep every row-window read inside the allocation
    p.gpre = (g.pw + VE - 1) / VE * VE;
    const int xl = static_cast<int>(G * iplane), dl = static_cast<int>(G * g.mult * oplane);
    p.dofs = p.gpre + (xl + VE - 1) / VE * VE;
    const int post = std::max(iwm, p.owm) + VE;
    const int stage = (p.dofs + dl + post) * sz;
    const int NT = g.mult * (g.kh * g.kw + 1);
    const int red = kThreads * std::min(NT, kRedCh) * 4;
    p.lds_bytes = (std::max(stage, red) + 15) / 16 * 16;
    return true;
}

template <typename T, int K, int S, int D, int MM, int OWM>
int run_sp_bwdw(const Geo &g, const SwPlan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    SwArgs<T> a{};
    a.x = static_cast<const T *>(x);
    a.dy = static_cast<const T *>(dy);
    a.ws = static_cast<float *>(ws);
    a.g = g;
    a.G = p.G;
    a.NC = p.NC;
    a.npc = p.npc;
    a.gpre = p.gpre;
    a.dofs = p.dofs;
    a.vec = p.vec && reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(dy) % 16 == 0;
    hipLaunchKernelGGL((sp_bwdw_kernel<T, K, S, D, MM, OWM>), dim3(p.grid), dim3(kThreads), p.lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, int K, int S, int D, int MM>
int run_w(const Geo &g, const SwPlan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    if (p.owm == 4) return run_sp_bwdw<T, K, S, D, MM, 4>(g, p, x, dy, ws, s);
    if (p.owm == 8) return run_sp_bwdw<T, K, S, D, MM, 8>(g, p, x, dy, ws, s);
    return run_sp_bwdw<T, K, S, D, MM, 16>(g, p, x, dy, ws, s);
}

template <typename T, int K, int S, int D>
int run_m(const Geo &g, const SwPlan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    return g.mult == 2 ? run_w<T, K, S, D, 2>(g, p, x, dy, ws, s) : run_w<T, K, S, D, 1>(g, p, x, dy, ws, s);
}

template <typename T>
int sp_bwdw_t(const Geo &g, const void *x, const void *dy, void *ws, hipStream_t s) {
    SwPlan p;
    if (!plan_sp_bwdw<T>(g, p)) return kErrUnsupported;
    if (g.kh == 3) return g.sh == 1 ? run_m<T, 3, 1, 1>(g, p, x, dy, ws, s) : run_m<T, 3, 2, 1>(g, p, x, dy, ws, s);
    return g.sh == 1 ? run_m<T, 5, 1, 1>(g, p, x, dy, ws, s) : run_m<T, 5, 2, 2>(g, p, x, dy, ws, s);
}

}  // namespace

bool small_fits(const Geo &g, int dtype, int pass) {
    if (pass != 2) return false;  // forward and grad-input use the band kernels for small planes
    SwPlan p;
    return dtype == 0 ? plan_sp_bwdw<float>(g, p) : plan_sp_bwdw<__half>(g, p);
}

int small_bwd_weight_chunks(const Geo &g, int dtype) {
    SwPlan p;
    const bool ok = dtype == 0 ? plan_sp_bwdw<float>(g, p) : plan_sp_bwdw<__half>(g, p);
    return ok ? p.NC : 0;
}

int small_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return sp_bwdw_t<float>(g, x, dy, ws, s);
        case 1: return sp_bwdw_t<__half>(g, x, dy, ws, s);
        default: return sp_bwdw_t<bf16_t>(g, x, dy, ws, s);
    }
}

}  // namespace dw
