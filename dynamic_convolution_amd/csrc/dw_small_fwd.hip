// dw_small_fwd.hip -- depthwise forward for small planes on gfx950.
//
//   y[n,o,p,q] = b[o] + sum_ij w[o,i,j] * x[n,o/M, p*s-pad+i*d, q*s-pad+j*d]
// (PyTorch PR #3057: depthwise forward with padding, stride, dilation,
// multiplier and bias.)
//
// Input planes of up to 256 pixels: a workgroup owns G adjacent channels and a
// chunk of images and stages one image's x range in LDS at a time
// (dw_small.hpp).  Each lane owns one (channel, output row) for the chunk, so
// its channel's taps and bias stay in registers; per image it reads the kh
// input rows under its output row from LDS (a window of compile-time width,
// columns outside the plane masked by a wave-uniform mask), writes its M output
// rows to an LDS copy of the output range, and the workgroup then stores that
// range to y as 16-byte vectors.
#include "dw_small.hpp"

namespace dw {
namespace {

template <typename T> struct CfArgs {
    const T *x;
    const T *w;
    const T *b;
    T *y;
    Geo g;
    int G;        // channels per workgroup
    int NC, npc;  // image chunks, images per chunk
    int gpre;     // LDS elements before the x planes (left-pad reads)
    int yofs;     // LDS element index of the staged output planes
    int vec;      // x and y ranges are whole, aligned 16-byte vectors
};

template <typename T, int K, int S, int D, int MM, int OWM>
__global__ __launch_bounds__(kThreads) void cg_fwd_kernel(CfArgs<T> a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int KK = K * K;
    constexpr int IWM = (OWM - 1) * S + (K - 1) * D + 1;  // input columns under a window of outputs
    constexpr int VE = Vec<T>::N;
    const Geo &g = a.g;
    const int tid = threadIdx.x;
    const int ngroups = (g.ic + a.G - 1) / a.G;
    const int chunk = blockIdx.x / ngroups;
    const int c0 = (blockIdx.x - chunk * ngroups) * a.G;
    const int Gc = min(a.G, g.ic - c0);
    const int iplane = g.ih * g.iw, oplane = g.oh * g.ow;
    const int ch = tid / g.oh;
    const int r = tid - ch * g.oh;
    const bool active = ch < Gc;
    T *lds = reinterpret_cast<T *>(smem);
    T *xs = lds + a.gpre;
    T *ys = lds + a.yofs;
    const int xlen = Gc * iplane, ylen = Gc * MM * oplane;
    const int nvx = xlen / VE;

    // this lane's taps and biases: its channel is fixed for the whole chunk
    const int cc = c0 + (active ? ch : 0);
    float wv[MM][KK], bv[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) {
#pragma unroll
        for (int t = 0; t < KK; ++t) wv[m][t] = to_f32(a.w[(static_cast<int64_t>(cc) * MM + m) * KK + t]);
        bv[m] = a.b ? to_f32(a.b[cc * MM + m]) : 0.f;
    }

    const int n_beg = chunk * a.npc;
    const int n_end = min(n_beg + a.npc, g.n);
    auto xbase = [&](int n) { return (static_cast<int64_t>(n) * g.ic + c0) * iplane; };
    auto ybase = [&](int n) { return (static_cast<int64_t>(n) * g.oc + static_cast<int64_t>(c0) * MM) * oplane; };
    cg_v4u pf[kCgPV];
    auto issue = [&](int n) {
        const T *xb = a.x + xbase(n);
        cg_issue(pf, xb, nvx, xb, nvx, tid);
    };
    // uniform column mask: position p of a row window reads column p - pw
    const uint64_t colok = cg_colmask<IWM>(-g.pw, g.iw);

    if (a.vec && n_beg < n_end) issue(n_beg);
    for (int n = n_beg; n < n_end; ++n) {
        __syncthreads();  // the previous image's LDS reads (x rows, staged y) are done
        if (a.vec)
            cg_commit(pf, xs, nvx, xs, nvx, tid);
        else
            cg_copy_elems(xs, a.x + xbase(n), xlen, tid);
        __syncthreads();
        if (a.vec && n + 1 < n_end) issue(n + 1);
        if (active) {
            float acc[MM][OWM];
#pragma unroll
            for (int m = 0; m < MM; ++m)
#pragma unroll
                for (int q = 0; q < OWM; ++q) acc[m][q] = bv[m];
#pragma unroll
            for (int i = 0; i < K; ++i) {
                const int ih = r * S - g.ph + i * D;
                const bool rowok = ih >= 0 && ih < g.ih;
                const T *xr = xs + ch * iplane + (rowok ? ih : 0) * g.iw - g.pw;
                float xv[IWM];
#pragma unroll
                for (int p = 0; p < IWM; ++p) {
                    const float v = to_f32(xr[p]);
                    xv[p] = rowok && ((colok >> p) & 1) ? v : 0.f;
                }
#pragma unroll
                for (int j = 0; j < K; ++j)
#pragma unroll
                    for (int m = 0; m < MM; ++m)
#pragma unroll
                        for (int q = 0; q < OWM; ++q) acc[m][q] = fmaf(wv[m][i * K + j], xv[q * S + j * D], acc[m][q]);
            }
            T *yr = ys + ch * MM * oplane + r * g.ow;
#pragma unroll
            for (int m = 0; m < MM; ++m)
#pragma unroll
                for (int q = 0; q < OWM; ++q)
                    if (q < g.ow) yr[m * oplane + q] = from_f32<T>(acc[m][q]);
        }
        __syncthreads();
        cg_store_out(a.y + ybase(n), ys, ylen, a.vec, tid);
    }
}

struct CfPlan {
    CgPlan c;
    int gpre, yofs, lds_bytes, owm;
};

template <typename T>
bool plan_cg_fwd(const Geo &g, CfPlan &p) {
    if (!cg_combo_ok(g)) return false;
    const int sz = sizeof(T), VE = 16 / sz;
    const int64_t iplane = static_cast<int64_t>(g.ih) * g.iw, oplane = static_cast<int64_t>(g.oh) * g.ow;
    // input planes of at most 256 pixels with output rows of at most 16 (7x7,
    // 14x14; a 28x28 input leaves too few channels per workgroup for the 16 KB
    // of staging and measured faster with the band kernel)
    if (iplane > 256 || oplane > 256 || g.ow > 16) return false;
    if (!cg_plan(g, g.oh, iplane * sz, sz, p.c)) return false;
    p.owm = g.ow <= 4 ? 4 : (g.ow <= 8 ? 8 : 16);
    const int iwm = (p.owm - 1) * g.sw + (g.kw - 1) * g.dw + 1;
    // LDS: [left guard][x planes][right guard][staged y planes]; the guards
    // keep every row-window read inside the allocation
    p.gpre = (g.pw + VE - 1) / VE * VE;
    const int xl = static_cast<int>(p.c.G * iplane), yl = static_cast<int>(p.c.G * g.mult * oplane);
    p.yofs = (p.gpre + xl + iwm + VE - 1) / VE * VE;
    p.lds_bytes = ((p.yofs + yl) * sz + 15) / 16 * 16;
    return true;
}

template <typename T, int K, int S, int D, int MM, int OWM>
int run_cg_fwd(const Geo &g, const CfPlan &p, const void *x, const void *w, const void *b, void *y, hipStream_t s) {
    CfArgs<T> a{};
    a.x = static_cast<const T *>(x);
    a.w = static_cast<const T *>(w);
    a.b = static_cast<const T *>(b);
    a.y = static_cast<T *>(y);
    a.g = g;
    a.G = p.c.G;
    a.NC = p.c.NC;
    a.npc = p.c.npc;
    a.gpre = p.gpre;
    a.yofs = p.yofs;
    a.vec = p.c.vec && reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0;
    hipLaunchKernelGGL((cg_fwd_kernel<T, K, S, D, MM, OWM>), dim3(p.c.grid), dim3(kThreads), p.lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, int K, int S, int D, int MM>
int run_w(const Geo &g, const CfPlan &p, const void *x, const void *w, const void *b, void *y, hipStream_t s) {
    if (p.owm == 4) return run_cg_fwd<T, K, S, D, MM, 4>(g, p, x, w, b, y, s);
    if (p.owm == 8) return run_cg_fwd<T, K, S, D, MM, 8>(g, p, x, w, b, y, s);
    return run_cg_fwd<T, K, S, D, MM, 16>(g, p, x, w, b, y, s);
}

template <typename T, int K, int S, int D>
int run_m(const Geo &g, const CfPlan &p, const void *x, const void *w, const void *b, void *y, hipStream_t s) {
    return g.mult == 2 ? run_w<T, K, S, D, 2>(g, p, x, w, b, y, s) : run_w<T, K, S, D, 1>(g, p, x, w, b, y, s);
}

template <typename T>
int cg_fwd_t(const Geo &g, const void *x, const void *w, const void *b, void *y, hipStream_t s) {
    CfPlan p;
    if (!plan_cg_fwd<T>(g, p)) return kErrUnsupported;
    if (g.kh == 3) return g.sh == 1 ? run_m<T, 3, 1, 1>(g, p, x, w, b, y, s) : run_m<T, 3, 2, 1>(g, p, x, w, b, y, s);
    return g.sh == 1 ? run_m<T, 5, 1, 1>(g, p, x, w, b, y, s) : run_m<T, 5, 2, 2>(g, p, x, w, b, y, s);
}

}  // namespace

bool small_fwd_fits(const Geo &g, int dtype) {
    CfPlan p;
    return dtype == 0 ? plan_cg_fwd<float>(g, p) : plan_cg_fwd<__half>(g, p);
}

int small_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return cg_fwd_t<float>(g, x, w, b, y, s);
        case 1: return cg_fwd_t<__half>(g, x, w, b, y, s);
        default: return cg_fwd_t<bf16_t>(g, x, w, b, y, s);
    }
}

}  // namespace dw
