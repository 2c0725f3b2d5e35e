// dw_small.hip -- depthwise grad-weight for small planes on gfx950.
//
//   dw[o,i,j] = sum_{n,p,q} dy[n,o,p,q] * x[n,o/M, p*s-pad+i*d, q*s-pad+j*d],  db[o] = sum dy
// (PyTorch PR #3057: grad-weight and grad-bias of the depthwise convolution.)
//
// For small planes (up to 16x16 outputs) one channel's data is a few hundred
// bytes to 4 KB per image, scattered with the stride of a whole image, and a
// per-channel walk reads short rows from many places.  Here a workgroup owns G
// adjacent channels and walks a chunk of images, staging one image's x range
// and dy range in LDS at a time (dw_small.hpp).
//
// Each lane owns one (channel, output row) for the whole chunk: per image it
// reads its dy row and the kh input rows under it from LDS and accumulates the
// kh*kw tap sums and the bias sum in registers, so the sum over images needs
// no cross-lane step.  At the end the output rows of each channel are added
// in a fixed order through LDS and one lane per (channel, slot) writes the
// (channel, image chunk) partial to the workspace [ic][chunk][M*(kh*kw+1)]
// that pass 2 adds up.
#include "dw_small.hpp"

namespace dw {
namespace {

constexpr int kRedCh = 16;  // accumulators per lane per reduction step

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

    cg_v4u pf[kCgPV];
    auto issue = [&](int n) { cg_issue(pf, a.x + xbase(n), nvx, a.dy + dbase(n), nv, tid); };

    // uniform column mask: position p of a row window reads column p - pw
    const uint64_t colok = cg_colmask<IWM>(-g.pw, g.iw);

    if (a.vec && n_beg < n_end) issue(n_beg);
    for (int n = n_beg; n < n_end; ++n) {
        __syncthreads();  // the previous image's LDS reads are done
        if (a.vec) {
            cg_commit(pf, xs, nvx, ds, nv, tid);
        } else {
            cg_copy_elems(xs, a.x + xbase(n), xlen, tid);
            cg_copy_elems(ds, a.dy + dbase(n), dlen, tid);
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
    CgPlan c;
    int gpre, dofs, lds_bytes, owm;
};

int row_span(const Geo &g, int owm) { return (owm - 1) * g.sw + (g.kw - 1) * g.dw + 1; }

template <typename T>
bool plan_sp_bwdw(const Geo &g, SwPlan &p) {
    if (!cg_combo_ok(g)) return false;
    const int sz = sizeof(T), VE = 16 / sz;
    const int64_t iplane = static_cast<int64_t>(g.ih) * g.iw, oplane = static_cast<int64_t>(g.oh) * g.ow;
    // used for planes of at most 256 output pixels and rows of at most 16
    // (7x7, 14x14, 28x28 at stride 2): larger planes measured faster with the
    // streaming row walk
    if (oplane > 256 || g.ow > 16) return false;
    if (!cg_plan(g, g.oh, (iplane + g.mult * oplane) * sz, sz, p.c)) return false;
    p.owm = g.ow <= 4 ? 4 : (g.ow <= 8 ? 8 : 16);
    const int iwm = row_span(g, p.owm);
    // LDS: [left guard][x planes][pad][dy planes][right guard]; the guards and
    // the pad keep every row-window read inside the allocation
    p.gpre = (g.pw + VE - 1) / VE * VE;
    const int xl = static_cast<int>(p.c.G * iplane), dl = static_cast<int>(p.c.G * g.mult * oplane);
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
    a.G = p.c.G;
    a.NC = p.c.NC;
    a.npc = p.c.npc;
    a.gpre = p.gpre;
    a.dofs = p.dofs;
    a.vec = p.c.vec && reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(dy) % 16 == 0;
    hipLaunchKernelGGL((sp_bwdw_kernel<T, K, S, D, MM, OWM>), dim3(p.c.grid), dim3(kThreads), p.lds_bytes, s, a);
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
    return ok ? p.c.NC : 0;
}

int small_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return sp_bwdw_t<float>(g, x, dy, ws, s);
        case 1: return sp_bwdw_t<__half>(g, x, dy, ws, s);
        default: return sp_bwdw_t<bf16_t>(g, x, dy, ws, s);
    }
}

}  // namespace dw
