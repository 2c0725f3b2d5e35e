// dw_small_bwdin.hip -- depthwise grad-input for small planes on gfx950.
//
//   dx[n,c,h,w] = sum_{m,i,j} w[cM+m,i,j] * dy[n,cM+m,p,q]
//                 over (p, q) with p*s - pad + i*d = h and q*s - pad + j*d = w
// (PyTorch PR #3057: the grad-input of the depthwise convolution.)
//
// dx planes of up to 256 pixels (1024 with rows of up to 32 at stride 2): a
// workgroup owns G adjacent channels and a chunk of images and stages one
// image's dy range in LDS at a time (dw_small.hpp).  Each lane owns one
// (channel, dx row) for the chunk with its channel's M*kh*kw taps in
// registers.  For each (m, i) the dy row that reaches its dx row is read from
// LDS into a window of compile-time width; at stride 2 only taps whose column
// offset has the right parity reach a dx column, which is decided at compile
// time from the parity of the padding (a template parameter), and a dy row of
// the wrong parity is masked.  The dx rows go to an LDS copy of the dx range,
// stored as 16-byte vectors.
#include "dw_small.hpp"

namespace dw {
namespace {

template <typename T> struct CbArgs {
    const T *dy;
    const T *w;
    T *dx;
    Geo g;
    int G;        // channels per workgroup
    int NC, npc;  // image chunks, images per chunk
    int gpre;     // LDS elements before the dy planes (reads left of a row)
    int xofs;     // LDS element index of the staged dx planes
    int vec;      // dy and dx ranges are whole, aligned 16-byte vectors
};

constexpr int floordiv_c(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Window of dy positions one dx row of IWM columns reads for one tap row.
template <int K, int S, int D, int IWM, int PP> struct BinWin {
    // stride 1: position u is dy column u + pw - (K-1)*D, dx column iw uses u = iw + (K-1-j)*D
    // stride 2: position u is dy column u + (pw-PP)/2 + C0, dx column iw uses u = (iw+PP-j*D)/2 - C0
    static constexpr int C0 = S == 1 ? 0 : floordiv_c(PP - (K - 1) * D, 2);
    static constexpr int U = S == 1 ? IWM + (K - 1) * D : (IWM - 1 + PP) / 2 - C0 + 1;
};

template <typename T, int K, int S, int D, int MM, int IWM, int PP>
__global__ __launch_bounds__(kThreads) void cg_bwdin_kernel(CbArgs<T> a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int KK = K * K;
    constexpr int VE = Vec<T>::N;
    using W = BinWin<K, S, D, IWM, PP>;
    constexpr int U = W::U;
    const Geo &g = a.g;
    const int tid = threadIdx.x;
    const int ngroups = (g.ic + a.G - 1) / a.G;
    const int chunk = blockIdx.x / ngroups;
    const int c0 = (blockIdx.x - chunk * ngroups) * a.G;
    const int Gc = min(a.G, g.ic - c0);
    const int iplane = g.ih * g.iw, oplane = g.oh * g.ow;
    const int ch = tid / g.ih;
    const int r = tid - ch * g.ih;  // dx row
    const bool active = ch < Gc;
    T *lds = reinterpret_cast<T *>(smem);
    T *ds = lds + a.gpre;
    T *xs = lds + a.xofs;
    const int dlen = Gc * MM * oplane, xlen = Gc * iplane;
    const int nvd = dlen / VE;

    const int cc = c0 + (active ? ch : 0);
    float wv[MM][KK];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t < KK; ++t) wv[m][t] = to_f32(a.w[(static_cast<int64_t>(cc) * MM + m) * KK + t]);

    const int n_beg = chunk * a.npc;
    const int n_end = min(n_beg + a.npc, g.n);
    auto dbase = [&](int n) { return (static_cast<int64_t>(n) * g.oc + static_cast<int64_t>(c0) * MM) * oplane; };
    auto xbase = [&](int n) { return (static_cast<int64_t>(n) * g.ic + c0) * iplane; };
    cg_v4u pf[kCgPV];
    auto issue = [&](int n) {
        const T *db = a.dy + dbase(n);
        cg_issue(pf, db, nvd, db, nvd, tid);
    };
    // dy column of window position 0, and the uniform mask of positions inside the row
    const int u0 = S == 1 ? g.pw - (K - 1) * D : (g.pw - PP) / 2 + W::C0;
    const uint64_t colok = cg_colmask<U>(u0, g.ow);

    if (a.vec && n_beg < n_end) issue(n_beg);
    for (int n = n_beg; n < n_end; ++n) {
        __syncthreads();  // the previous image's LDS reads (dy rows, staged dx) are done
        if (a.vec)
            cg_commit(pf, ds, nvd, ds, nvd, tid);
        else
            cg_copy_elems(ds, a.dy + dbase(n), dlen, tid);
        __syncthreads();
        if (a.vec && n + 1 < n_end) issue(n + 1);
        if (active) {
            float acc[IWM];
#pragma unroll
            for (int c = 0; c < IWM; ++c) acc[c] = 0.f;
#pragma unroll
            for (int m = 0; m < MM; ++m)
#pragma unroll
                for (int i = 0; i < K; ++i) {
                    // dy row p with p*S - ph + i*D = r
                    const int num = r + g.ph - i * D;
                    const int p = S == 1 ? num : (num >> 1);
                    const bool rowok = num >= 0 && (S == 1 || (num & 1) == 0) && p < g.oh;
                    const T *dr = ds + (ch * MM + m) * oplane + (rowok ? p : 0) * g.ow + u0;
                    float dv[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const float v = to_f32(dr[u]);
                        dv[u] = rowok && ((colok >> u) & 1) ? v : 0.f;
                    }
#pragma unroll
                    for (int j = 0; j < K; ++j) {
                        const float wt = wv[m][i * K + j];
#pragma unroll
                        for (int c = 0; c < IWM; ++c) {
                            if constexpr (S == 1) {
                                acc[c] = fmaf(wt, dv[c + (K - 1 - j) * D], acc[c]);
                            } else {
                                if ((c + PP - j * D) % 2 == 0) acc[c] = fmaf(wt, dv[(c + PP - j * D) / 2 - W::C0], acc[c]);
                            }
                        }
                    }
                }
            T *xr = xs + ch * iplane + r * g.iw;
#pragma unroll
            for (int c = 0; c < IWM; ++c)
                if (c < g.iw) xr[c] = from_f32<T>(acc[c]);
        }
        __syncthreads();
        cg_store_out(a.dx + xbase(n), xs, xlen, a.vec, tid);
    }
}

struct CbPlan {
    CgPlan c;
    int gpre, xofs, lds_bytes, iwm;
};

template <typename T>
bool plan_cg_bwdin(const Geo &g, CbPlan &p) {
    if (!cg_combo_ok(g)) return false;
    const int sz = sizeof(T), VE = 16 / sz;
    const int64_t iplane = static_cast<int64_t>(g.ih) * g.iw, oplane = static_cast<int64_t>(g.oh) * g.ow;
    // dx planes of at most 256 pixels (7x7, 14x14), or 1024 with rows of at
    // most 32 at stride 2 (28x28): at stride 1 a 28x28 plane leaves too few
    // channels per workgroup and measured faster with the band kernel
    if (iplane > (g.sh == 2 ? 1024 : 256) || g.iw > 32) return false;
    if (!cg_plan(g, g.ih, g.mult * oplane * sz, sz, p.c)) return false;
    p.iwm = g.iw <= 8 ? 8 : (g.iw <= 16 ? 16 : 32);
    const int K = g.kh, D = g.dh, PP = g.pw & 1;
    int u0, U;
    if (g.sw == 1) {
        u0 = g.pw - (K - 1) * D;
        U = p.iwm + (K - 1) * D;
    } else {
        const int c0 = floordiv_c(PP - (K - 1) * D, 2);
        u0 = (g.pw - PP) / 2 + c0;
        U = (p.iwm - 1 + PP) / 2 - c0 + 1;
    }
    // LDS: [left guard][dy planes][right guard][staged dx planes]; the guards
    // keep every window read inside the allocation
    p.gpre = (std::max(0, -u0) + VE - 1) / VE * VE;
    const int dl = static_cast<int>(p.c.G * g.mult * oplane), xl = static_cast<int>(p.c.G * iplane);
    p.xofs = (p.gpre + dl + std::max(0, u0) + U + VE - 1) / VE * VE;
    p.lds_bytes = ((p.xofs + xl) * sz + 15) / 16 * 16;
    return true;
}

template <typename T, int K, int S, int D, int MM, int IWM, int PP>
int run_cg_bwdin(const Geo &g, const CbPlan &p, const void *dy, const void *w, void *dx, hipStream_t s) {
    CbArgs<T> a{};
    a.dy = static_cast<const T *>(dy);
    a.w = static_cast<const T *>(w);
    a.dx = static_cast<T *>(dx);
    a.g = g;
    a.G = p.c.G;
    a.NC = p.c.NC;
    a.npc = p.c.npc;
    a.gpre = p.gpre;
    a.xofs = p.xofs;
    a.vec = p.c.vec && reinterpret_cast<uintptr_t>(dy) % 16 == 0 && reinterpret_cast<uintptr_t>(dx) % 16 == 0;
    hipLaunchKernelGGL((cg_bwdin_kernel<T, K, S, D, MM, IWM, PP>), dim3(p.c.grid), dim3(kThreads), p.lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, int K, int S, int D, int MM, int IWM>
int run_p(const Geo &g, const CbPlan &p, const void *dy, const void *w, void *dx, hipStream_t s) {
    if (S == 2 && (g.pw & 1)) return run_cg_bwdin<T, K, S, D, MM, IWM, 1>(g, p, dy, w, dx, s);
    return run_cg_bwdin<T, K, S, D, MM, IWM, 0>(g, p, dy, w, dx, s);
}

template <typename T, int K, int S, int D, int MM>
int run_w(const Geo &g, const CbPlan &p, const void *dy, const void *w, void *dx, hipStream_t s) {
    if (p.iwm == 8) return run_p<T, K, S, D, MM, 8>(g, p, dy, w, dx, s);
    if (p.iwm == 16) return run_p<T, K, S, D, MM, 16>(g, p, dy, w, dx, s);
    return run_p<T, K, S, D, MM, 32>(g, p, dy, w, dx, s);
}

template <typename T, int K, int S, int D>
int run_m(const Geo &g, const CbPlan &p, const void *dy, const void *w, void *dx, hipStream_t s) {
    return g.mult == 2 ? run_w<T, K, S, D, 2>(g, p, dy, w, dx, s) : run_w<T, K, S, D, 1>(g, p, dy, w, dx, s);
}

template <typename T>
int cg_bwdin_t(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t s) {
    CbPlan p;
    if (!plan_cg_bwdin<T>(g, p)) return kErrUnsupported;
    if (g.kh == 3) return g.sh == 1 ? run_m<T, 3, 1, 1>(g, p, dy, w, dx, s) : run_m<T, 3, 2, 1>(g, p, dy, w, dx, s);
    return g.sh == 1 ? run_m<T, 5, 1, 1>(g, p, dy, w, dx, s) : run_m<T, 5, 2, 2>(g, p, dy, w, dx, s);
}

}  // namespace

bool small_bwd_input_fits(const Geo &g, int dtype) {
    CbPlan p;
    return dtype == 0 ? plan_cg_bwdin<float>(g, p) : plan_cg_bwdin<__half>(g, p);
}

int small_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return cg_bwdin_t<float>(g, dy, w, dx, s);
        case 1: return cg_bwdin_t<__half>(g, dy, w, dx, s);
        default: return cg_bwdin_t<bf16_t>(g, dy, w, dx, s);
    }
}

}  // namespace dw
