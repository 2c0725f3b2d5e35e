// dw_small.hip -- depthwise grad-weight for small planes on gfx950.
//
//   dw[o,i,j] = sum_{n,p,q} dy[n,o,p,q] * x[n,o/M, p*s-pad+i*d, q*s-pad+j*d],  db[o] = sum dy
// (PyTorch PR #3057: grad-weight and grad-bias of the depthwise convolution.)
//
// For small planes (7x7, or 14x14 at stride 2) one channel's data is a
// 200-800 byte piece per image, scattered with the stride of a whole image,
// and a per-channel walk reads short rows from many places.  Here a workgroup
// owns G adjacent channels instead: for a fixed image their x planes are one
// contiguous range and their dy planes another.  Each iteration stages NI
// images' worth of both ranges in LDS, every lane issuing all of its 16-byte
// loads before any LDS store (2*NI requests in flight per lane).  Each
// channel's output pixels are split over TPC lanes accumulating the kh*kw tap
// sums and the bias sum; the TPC lanes of a channel are reduced with shuffles
// in a fixed order and one lane writes the (channel, image chunk) partial to
// the workspace [ic][chunk][M*(kh*kw+1)] that pass 2 adds up.
#include "dw_common.hpp"
#include "dw_internal.hpp"

namespace dw {
namespace {

constexpr int kSmallLds = 32 * 1024;  // staged bytes per workgroup
constexpr int kNI = 4;                // images staged per iteration

template <typename T> struct SwArgs {
    const T *x;
    const T *dy;
    float *ws;
    Geo g;
    int G;          // channels per workgroup
    int NC, npc;    // image chunks, images per chunk
    int TPC;        // lanes per channel (power of two <= 64)
    FastDiv fPW;    // output width
    int xslots, dslots;  // LDS elements per staged image (x, dy)
    int vec;        // x and dy 16-byte aligned
};

// Stages the x range and the dy range of images n0 .. n0+NI-1 (those < n1).
template <typename T>
__device__ __forceinline__ void stage_images(const SwArgs<T> &a, T *xs, T *ds, int c0, int Gc, int n0, int n1,
                                             int (&xo)[kNI], int (&dof)[kNI], int tid) {
    constexpr int VE = Vec<T>::N;
    const Geo &g = a.g;
    const int64_t iplane = static_cast<int64_t>(g.ih) * g.iw, oplane = static_cast<int64_t>(g.oh) * g.ow;
    const int64_t xlen = Gc * iplane, dlen = Gc * g.mult * oplane;
    int64_t xb[kNI], db[kNI];
    int nvx = 0, nvd = 0;
#pragma unroll
    for (int u = 0; u < kNI; ++u) {
        const int n = n0 + u;
        xb[u] = (static_cast<int64_t>(n) * g.ic + c0) * iplane;
        db[u] = (static_cast<int64_t>(n) * g.oc + static_cast<int64_t>(c0) * g.mult) * oplane;
        xo[u] = static_cast<int>(xb[u] & (VE - 1));
        dof[u] = static_cast<int>(db[u] & (VE - 1));
        nvx = max(nvx, static_cast<int>((xo[u] + xlen + VE - 1) / VE));
        nvd = max(nvd, static_cast<int>((dof[u] + dlen + VE - 1) / VE));
    }
    if (!a.vec) {  // base pointers not 16-byte aligned: element copies
#pragma unroll
        for (int u = 0; u < kNI; ++u) {
            xo[u] = dof[u] = 0;
            if (n0 + u >= n1) continue;
            for (int e = tid; e < xlen; e += kThreads) xs[u * a.xslots + e] = a.x[xb[u] + e];
            for (int e = tid; e < dlen; e += kThreads) ds[u * a.dslots + e] = a.dy[db[u] + e];
        }
        return;
    }
    const int nv = max(nvx, nvd);
    for (int v = tid; v < nv; v += kThreads) {
        uint4 rx[kNI], rd[kNI];
#pragma unroll
        for (int u = 0; u < kNI; ++u) rx[u] = rd[u] = make_uint4(0, 0, 0, 0);
        // all loads of this lane first ...
#pragma unroll
        for (int u = 0; u < kNI; ++u) {
            if (n0 + u >= n1) continue;
            const int64_t ex = (xb[u] - xo[u]) + static_cast<int64_t>(v) * VE;
            if (v < nvx && ex >= xb[u] && ex + VE <= xb[u] + xlen) rx[u] = *reinterpret_cast<const uint4 *>(a.x + ex);
            const int64_t ed = (db[u] - dof[u]) + static_cast<int64_t>(v) * VE;
            if (v < nvd && ed >= db[u] && ed + VE <= db[u] + dlen) rd[u] = *reinterpret_cast<const uint4 *>(a.dy + ed);
        }
        // ... then the LDS stores (partial end vectors element by element)
#pragma unroll
        for (int u = 0; u < kNI; ++u) {
            if (n0 + u >= n1) continue;
            const int64_t ex = (xb[u] - xo[u]) + static_cast<int64_t>(v) * VE;
            T *lx = xs + u * a.xslots + v * VE;
            if (v < nvx) {
                if (ex >= xb[u] && ex + VE <= xb[u] + xlen) {
                    *reinterpret_cast<uint4 *>(lx) = rx[u];
                } else {
#pragma unroll
                    for (int k = 0; k < VE; ++k)
                        lx[k] = (ex + k >= xb[u] && ex + k < xb[u] + xlen) ? a.x[ex + k] : T{};
                }
            }
            const int64_t ed = (db[u] - dof[u]) + static_cast<int64_t>(v) * VE;
            T *ld = ds + u * a.dslots + v * VE;
            if (v < nvd) {
                if (ed >= db[u] && ed + VE <= db[u] + dlen) {
                    *reinterpret_cast<uint4 *>(ld) = rd[u];
                } else {
#pragma unroll
                    for (int k = 0; k < VE; ++k)
                        ld[k] = (ed + k >= db[u] && ed + k < db[u] + dlen) ? a.dy[ed + k] : T{};
                }
            }
        }
    }
}

template <typename T, int KH, int KW, int S, int D, int MM>
__global__ __launch_bounds__(kThreads) void sp_bwdw_kernel(SwArgs<T> a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int KK = KH * KW;
    const Geo &g = a.g;
    const int tid = threadIdx.x;
    const int cg = blockIdx.x / a.NC;
    const int chunk = blockIdx.x - cg * a.NC;
    const int c0 = cg * a.G;
    const int Gc = min(a.G, g.ic - c0);
    const int lch = tid / a.TPC;  // local channel of this lane
    const int sub = tid - lch * a.TPC;
    const int iplane = g.ih * g.iw, oplane = g.oh * g.ow;
    T *xs = reinterpret_cast<T *>(smem);
    T *ds = xs + kNI * a.xslots;
    float acc[MM][KK + 1];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t <= KK; ++t) acc[m][t] = 0.f;
    const int n_beg = chunk * a.npc;
    const int n_end = min(n_beg + a.npc, g.n);
    for (int n0 = n_beg; n0 < n_end; n0 += kNI) {
        int xo[kNI], dof[kNI];
        __syncthreads();  // the previous images' LDS reads are done
        stage_images(a, xs, ds, c0, Gc, n0, n_end, xo, dof, tid);
        __syncthreads();
        if (lch < Gc) {
#pragma unroll
            for (int u = 0; u < kNI; ++u) {
                if (n0 + u >= n_end) continue;
                const T *xp = xs + u * a.xslots + xo[u] + lch * iplane;
                const T *dp = ds + u * a.dslots + dof[u] + lch * MM * oplane;
                for (int pix = sub; pix < oplane; pix += a.TPC) {
                    const int oh = static_cast<int>(fdiv(static_cast<uint32_t>(pix), a.fPW));
                    const int ow = pix - oh * g.ow;
                    float gy[MM];
#pragma unroll
                    for (int m = 0; m < MM; ++m) {
                        gy[m] = to_f32(dp[m * oplane + pix]);
                        acc[m][KK] += gy[m];
                    }
#pragma unroll
                    for (int i = 0; i < KH; ++i) {
                        const int ih = oh * S - g.ph + i * D;
                        if (ih < 0 || ih >= g.ih) continue;
#pragma unroll
                        for (int j = 0; j < KW; ++j) {
                            const int iw = ow * S - g.pw + j * D;
                            if (iw < 0 || iw >= g.iw) continue;
                            const float xv = to_f32(xp[ih * g.iw + iw]);
#pragma unroll
                            for (int m = 0; m < MM; ++m) acc[m][i * KW + j] = fmaf(gy[m], xv, acc[m][i * KW + j]);
                        }
                    }
                }
            }
        }
    }
    // fixed-order reduction over the TPC lanes of each channel (aligned groups in one wave)
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t <= KK; ++t) {
            float v = acc[m][t];
            for (int off = a.TPC >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            acc[m][t] = v;
        }
    if (sub == 0 && lch < Gc) {
        float *dst = a.ws + (static_cast<int64_t>(c0 + lch) * a.NC + chunk) * (MM * (KK + 1));
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int t = 0; t <= KK; ++t) dst[m * (KK + 1) + t] = acc[m][t];
    }
}

struct SwPlan {
    int G, TPC, NC, npc, grid, xslots, dslots, lds_bytes;
};

bool combo_ok(const Geo &g) {
    const bool sq = g.kh == g.kw && g.sh == g.sw && g.dh == g.dw;
    return g.mult <= 2 && sq &&
           ((g.kh == 3 && g.dh == 1 && g.sh <= 2) || (g.kh == 5 && ((g.sh == 1 && g.dh == 1) || (g.sh == 2 && g.dh == 2))));
}

template <typename T>
bool plan_sp_bwdw(const Geo &g, SwPlan &p) {
    if (!combo_ok(g)) return false;
    const int64_t iplane = static_cast<int64_t>(g.ih) * g.iw, oplane = static_cast<int64_t>(g.oh) * g.ow;
    // used for planes of at most 64 output pixels (7x7, and 14x14 at stride 2):
    // larger planes measured faster with the streaming row walk
    if (oplane > 64) return false;
    int tpc = 4;
    while (tpc < 64 && tpc * 4 < oplane) tpc <<= 1;
    int G = std::min(kThreads / tpc, g.ic);
    auto bytes = [&](int Gx, int &xs, int &dsl) {
        xs = lds_slots<T>(static_cast<int>(Gx * iplane));
        dsl = lds_slots<T>(static_cast<int>(Gx * g.mult * oplane));
        return static_cast<int64_t>(kNI) * (xs + dsl) * static_cast<int64_t>(sizeof(T));
    };
    int xs, dsl;
    while (G > 1 && bytes(G, xs, dsl) > kSmallLds) --G;
    if (bytes(G, xs, dsl) > kSmallLds) return false;
    int t = 1;
    while (t * 2 <= std::min(64, kThreads / G)) t *= 2;
    tpc = t;
    const int ngroups = (g.ic + G - 1) / G;
    // image chunks: >= 2048 workgroups, each staging at least one full batch of kNI images
    int NC = std::max(1, (2048 + ngroups - 1) / ngroups);
    NC = std::min(NC, std::max(1, g.n / kNI));
    const int npc = (g.n + NC - 1) / NC;
    NC = (g.n + npc - 1) / npc;
    p.G = G;
    p.TPC = tpc;
    p.NC = NC;
    p.npc = npc;
    p.grid = ngroups * NC;
    p.xslots = xs;
    p.dslots = dsl;
    p.lds_bytes = static_cast<int>(bytes(G, xs, dsl));
    return true;
}

template <typename T, int KH, int KW, int S, int D, int MM>
int run_sp_bwdw(const Geo &g, const SwPlan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    SwArgs<T> a{};
    a.x = static_cast<const T *>(x);
    a.dy = static_cast<const T *>(dy);
    a.ws = static_cast<float *>(ws);
    a.g = g;
    a.G = p.G;
    a.NC = p.NC;
    a.npc = p.npc;
    a.TPC = p.TPC;
    a.fPW = make_fastdiv(g.ow, static_cast<uint64_t>(g.oh) * g.ow + 64);
    a.xslots = p.xslots;
    a.dslots = p.dslots;
    a.vec = reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(dy) % 16 == 0;
    hipLaunchKernelGGL((sp_bwdw_kernel<T, KH, KW, S, D, MM>), dim3(p.grid), dim3(kThreads), p.lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, int KH, int S, int D>
int run_m(const Geo &g, const SwPlan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    return g.mult == 2 ? run_sp_bwdw<T, KH, KH, S, D, 2>(g, p, x, dy, ws, s)
                       : run_sp_bwdw<T, KH, KH, S, D, 1>(g, p, x, dy, ws, s);
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
