// dw_dynbwd.hip -- backward of the fused per-pixel dynamic filter at several
// dilations on gfx950.
//
// Forward (lartpang/DynamicConvolutionOperator: HDFNet's Dynamic Dilated
// Pyramid computation, written straight into the branch-concatenated output):
//   y[n, b*C + c, p] = sum_{t = i*k + j} F_b[n, c, t, p] * x[n, c, p + o_b(t)],
//   o_b(t) = ((i - r) d_b, (j - r) d_b),  r = (k - 1)/2,  zero outside the image.
// The page's benchmark times this op with its backward (its "--backward"
// flag).  y is bilinear in x and the filters, so the chain rule gives
//   dF_b[n, c, t, p] = dy[n, b*C + c, p] * x[n, c, p + o_b(t)]   (0 outside)
//   dx[n, c, s]      = sum_b sum_t F_b[n, c, t, s - o_b(t)] * dy[n, b*C + c, s - o_b(t)]
// (terms whose source pixel s - o_b(t) is outside the image vanish).
//
// Two kernels, both HBM-bound streams of about 1 + nb + nb*k*k planes:
//  - filter gradient: the forward's tile (x rows of a band plus the largest
//    dilation's halo, fp32, zero columns) is staged in LDS once; each thread
//    takes RW adjacent pixels of one row, loads dy of every branch as one
//    16-byte strip and writes the nb*k*k gradient strips (nearly all of the
//    kernel's traffic is these writes);
//  - input gradient, a gather with no atomics: a workgroup owns a band of dx
//    rows and walks the (branch, tap row i) pairs.  For each pair it stages
//    G_j = F_b[t = i*k + j] * dy_b on the source rows of the band (shifted by
//    (i - r) d_b) into an fp32 LDS tile with zero columns, k slabs, double
//    buffered so that the next pair's 16-byte loads are in flight while the
//    current pair is summed; each dx strip then adds the k column-shifted
//    reads of its row.  Every dx element is summed by one thread in a fixed
//    order (branch, i, j), so results are bitwise reproducible.
#include "dw_dyn.hpp"

namespace dw {
namespace {

using namespace dyn;

template <typename T> struct DynBwdArgs {
    const T *x;
    const T *f[kMaxBranches];
    const T *dy;              // (n, dych, h, w): branch b, channel ch at plane dyoff + b*c + ch
    T *dx;                    // (n, c, h, w)
    T *df[kMaxBranches];      // (n, c, k*k, h, w) each; NULL: not wanted
    int dil[kMaxBranches];
    int nb;
    int n, c, h, w, k;
    int dych, dyoff;
    int BH, nbands, NS;       // row bands of the launched kernel, strips per row
    FastDiv fNS;
    int halo;                 // r * max dilation
    int hp, LW;               // zero columns left of a staged row, row pitch (floats)
    FastDiv fLW, fVPR, fPAD;
    int vin;                  // x 16-byte aligned and rows of whole 16-byte vectors
    int vf;                   // every tensor 16-byte aligned and w a multiple of RW
};

// ---------------------------------------------------------------- filter gradient
template <typename T, int K_, int RW, bool VF>
__global__ __launch_bounds__(kThreads) void dynbwd_filter_kernel(DynBwdArgs<T> a) {
    extern __shared__ __align__(16) float xs[];
    const int K = K_ ? K_ : a.k;
    const int KK = K * K;
    const int rr = (K - 1) / 2;
    const int tid = threadIdx.x;
    const int plane = blockIdx.x / a.nbands;
    const int band = blockIdx.x - plane * a.nbands;
    const int nn = plane / a.c;
    const int ch = plane - nn * a.c;
    const int h0 = band * a.BH;
    const int h1 = min(h0 + a.BH, a.h);
    const int64_t hw = static_cast<int64_t>(a.h) * a.w;
    const int rbase = h0 - a.halo;
    const int rows = (h1 - h0) + 2 * a.halo;
    const int LW = a.LW, hp = a.hp;
    const bool vec = VF || a.vf != 0;

    stage_rows_f32<T>(xs, a.x + static_cast<int64_t>(plane) * hw, rbase, rows, a.h, a.w, LW, hp, a.fVPR,
                      a.fPAD, a.fLW, a.vin != 0, tid);
    __syncthreads();

    const int items = a.BH * a.NS;
    for (int u = tid; u < items; u += kThreads) {
        const int r = static_cast<int>(fdiv(static_cast<uint32_t>(u), a.fNS));
        const int s = u - r * a.NS;
        const int hh = h0 + r;
        if (hh >= h1) continue;
        const int w0 = s * RW;
        const int valid = a.w - w0;
        const int64_t pix = static_cast<int64_t>(hh) * a.w + w0;
        for (int b = 0; b < a.nb; ++b) {
            T *ob = a.df[b];
            if (!ob) continue;
            const int d = a.dil[b];
            float g[RW];
            load_strip<T, RW>(a.dy + (static_cast<int64_t>(nn) * a.dych + a.dyoff + b * a.c + ch) * hw + pix, g, valid, vec);
            ob += static_cast<int64_t>(plane) * KK * hw + pix;
            // LDS holds every row a tap of the band reaches (zeros outside the
            // image) and zero columns on both sides: no bounds test per tap
            for (int i = 0; i < K; ++i) {
                const float *rp = xs + (hh + (i - rr) * d - rbase) * LW + hp + w0;
                for (int j = 0; j < K; ++j) {
                    const int off = (j - rr) * d;
                    float o[RW];
#pragma unroll
                    for (int q = 0; q < RW; ++q) o[q] = g[q] * rp[off + q];
                    store_strip_nt<T, RW>(ob + static_cast<int64_t>(i * K + j) * hw, o, valid, vec);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- input gradient
// LDS layout: buffer q (0, 1) holds K slabs; slab j holds BH rows of LW floats;
// row rr of slab j of the pair (b, i) is G_j on source row h0 + rr - (i - r) d_b,
// column c at index hp + c.  The padding columns are zeroed once and never
// written again.
__device__ __forceinline__ void zero_pad_columns(float *gs, int nrows, int w, int LW, int hp, FastDiv fPAD,
                                                 int tid) {
    const int padw = LW - w;
    for (int e = tid; e < nrows * padw; e += kThreads) {
        const int r = static_cast<int>(fdiv(static_cast<uint32_t>(e), fPAD));
        const int j = e - r * padw;
        gs[r * LW + (j < hp ? j : w + j)] = 0.f;
    }
}

// Fast path: k = K_ and the branch count NB_ at compile time, every strip a
// whole 16-byte vector, one strip per thread per pair (BH * NS <= kThreads).
// The pair loop is fully unrolled and free of branches around loads and LDS
// writes (idle lanes repeat the last live lane's strip, writing the same
// values to the same place), so the compiler tracks every load exactly: the
// loads of pairs p + 1 and p + 2 stay in flight (issued from a clamped,
// always valid row) while pair p is summed, and pair p + 1 is then
// multiplied and written to the other buffer.
template <typename T, int K_, int RW, int NB_>
__global__ __launch_bounds__(kThreads) void dynbwd_input_kernel(DynBwdArgs<T> a) {
    extern __shared__ __align__(16) float gs[];
    constexpr int rr = (K_ - 1) / 2;
    constexpr int KK = K_ * K_;
    constexpr int NP = NB_ * K_;  // (branch, tap row) pairs
    const int tid = threadIdx.x;
    const int plane = blockIdx.x / a.nbands;
    const int band = blockIdx.x - plane * a.nbands;
    const int nn = plane / a.c;
    const int ch = plane - nn * a.c;
    const int h0 = band * a.BH;
    const int h1 = min(h0 + a.BH, a.h);
    const int64_t hw = static_cast<int64_t>(a.h) * a.w;
    const int LW = a.LW, hp = a.hp;
    const int slab = a.BH * LW;
    const int bufsz = K_ * slab;

    zero_pad_columns(gs, 2 * K_ * a.BH, a.w, LW, hp, a.fPAD, tid);

    const int items = a.BH * a.NS;
    const int u = min(tid, items - 1);
    const int row = static_cast<int>(fdiv(static_cast<uint32_t>(u), a.fNS));
    const int w0 = (u - row * a.NS) * RW;
    const bool mine = tid < items && h0 + row < h1;  // this thread owns dx strip (h0 + row, w0)

    // one pair's loads: dy and the K filter strips of tap row i on the source row
    struct Pend {
        u32x4 g, f[K_];
        bool in;
    };
    auto issue = [&](int p, Pend &r) {
        const int b = p / K_;
        const int i = p - b * K_;
        const int sr = h0 + row - (i - rr) * a.dil[b];
        r.in = sr >= 0 && sr < a.h;
        const int64_t pix = static_cast<int64_t>(min(max(sr, 0), a.h - 1)) * a.w + w0;
        r.g = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
            a.dy + (static_cast<int64_t>(nn) * a.dych + a.dyoff + b * a.c + ch) * hw + pix));
        const T *fb = a.f[b] + (static_cast<int64_t>(plane) * KK + i * K_) * hw + pix;
#pragma unroll
        for (int j = 0; j < K_; ++j)
            r.f[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(fb + static_cast<int64_t>(j) * hw));
    };
    auto put = [&](int p, const Pend &r) {
        float g[RW];
        strip_values<T, RW>(r.g, g);
        const float m = r.in ? 1.f : 0.f;  // source row outside the image: the pair adds nothing
#pragma unroll
        for (int q = 0; q < RW; ++q) g[q] *= m;
        float *dst = gs + (p & 1) * bufsz + row * LW + hp + w0;
#pragma unroll
        for (int j = 0; j < K_; ++j) {
            float fv[RW];
            strip_values<T, RW>(r.f[j], fv);
#pragma unroll
            for (int q = 0; q < RW; q += 4)
                *reinterpret_cast<float4 *>(dst + j * slab + q) =
                    make_float4(fv[q] * g[q], fv[q + 1] * g[q + 1], fv[q + 2] * g[q + 2], fv[q + 3] * g[q + 3]);
        }
    };

    float acc[RW];
#pragma unroll
    for (int q = 0; q < RW; ++q) acc[q] = 0.f;
    auto sum = [&](int p) {
        const int d = a.dil[p / K_];
        const float *src = gs + (p & 1) * bufsz + row * LW + hp + w0;
#pragma unroll
        for (int j = 0; j < K_; ++j) {
            const float *sp = src + j * slab - (j - rr) * d;
#pragma unroll
            for (int q = 0; q < RW; ++q) acc[q] += sp[q];
        }
    };

    Pend P[NP];
    issue(0, P[0]);
    if constexpr (NP > 1) issue(1, P[1]);
    put(0, P[0]);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        if (p + 2 < NP) issue(p + 2, P[p + 2]);
        // all of pair p + 2's loads ahead of pair p + 1's uses: the in-order
        // load counter then lets the waits for p + 1 leave them in flight
        __builtin_amdgcn_sched_barrier(0);
        sum(p);
        if (p + 1 < NP) put(p + 1, P[p + 1]);
        __syncthreads();
    }
    if (mine) store_strip<T, RW>(a.dx + static_cast<int64_t>(plane) * hw + static_cast<int64_t>(h0 + row) * a.w + w0,
                                 acc, RW, true);
}

// Any k, alignment and width: one pair at a time through a single buffer.
template <typename T, int RW>
__global__ __launch_bounds__(kThreads) void dynbwd_input_generic_kernel(DynBwdArgs<T> a) {
    extern __shared__ __align__(16) float gs[];
    const int K = a.k;
    const int KK = K * K;
    const int rr = (K - 1) / 2;
    const int tid = threadIdx.x;
    const int plane = blockIdx.x / a.nbands;
    const int band = blockIdx.x - plane * a.nbands;
    const int nn = plane / a.c;
    const int ch = plane - nn * a.c;
    const int h0 = band * a.BH;
    const int h1 = min(h0 + a.BH, a.h);
    const int64_t hw = static_cast<int64_t>(a.h) * a.w;
    const int LW = a.LW, hp = a.hp;
    const int slab = a.BH * LW;
    const bool vec = a.vf != 0;

    zero_pad_columns(gs, K * a.BH, a.w, LW, hp, a.fPAD, tid);

    const int items = a.BH * a.NS;
    const int per = (items + kThreads - 1) / kThreads;  // strips per thread
    constexpr int kMaxPer = 4;
    float acc[kMaxPer][RW];
#pragma unroll
    for (int m = 0; m < kMaxPer; ++m)
#pragma unroll
        for (int q = 0; q < RW; ++q) acc[m][q] = 0.f;

    for (int b = 0; b < a.nb; ++b) {
        const int d = a.dil[b];
        const T *dyb = a.dy + (static_cast<int64_t>(nn) * a.dych + a.dyoff + b * a.c + ch) * hw;
        for (int i = 0; i < K; ++i) {
            const T *fb = a.f[b] + (static_cast<int64_t>(plane) * KK + i * K) * hw;
            for (int u = tid; u < items; u += kThreads) {
                const int row = static_cast<int>(fdiv(static_cast<uint32_t>(u), a.fNS));
                const int w0 = (u - row * a.NS) * RW;
                const int valid = min(a.w - w0, RW);
                const int sr = h0 + row - (i - rr) * d;
                float *dst = gs + row * LW + hp + w0;
                if (sr < 0 || sr >= a.h) {
                    for (int j = 0; j < K; ++j)
                        for (int q = 0; q < valid; ++q) dst[j * slab + q] = 0.f;
                    continue;
                }
                const int64_t pix = static_cast<int64_t>(sr) * a.w + w0;
                float g[RW];
                load_strip<T, RW>(dyb + pix, g, valid, vec);
                for (int j = 0; j < K; ++j) {
                    float fv[RW];
                    load_strip<T, RW>(fb + static_cast<int64_t>(j) * hw + pix, fv, valid, vec);
#pragma unroll
                    for (int q = 0; q < RW; ++q)
                        if (q < valid) dst[j * slab + q] = fv[q] * g[q];
                }
            }
            __syncthreads();
#pragma unroll
            for (int m = 0; m < kMaxPer; ++m) {
                const int u = tid + m * kThreads;
                if (m >= per || u >= items) continue;
                const int row = static_cast<int>(fdiv(static_cast<uint32_t>(u), a.fNS));
                if (h0 + row >= h1) continue;
                const int w0 = (u - row * a.NS) * RW;
                const float *src = gs + row * LW + hp + w0;
                for (int j = 0; j < K; ++j) {
                    const float *sp = src + j * slab - (j - rr) * d;
#pragma unroll
                    for (int q = 0; q < RW; ++q) acc[m][q] += sp[q];
                }
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int m = 0; m < kMaxPer; ++m) {
        const int u = tid + m * kThreads;
        if (m >= per || u >= items) continue;
        const int row = static_cast<int>(fdiv(static_cast<uint32_t>(u), a.fNS));
        if (h0 + row >= h1) continue;
        const int w0 = (u - row * a.NS) * RW;
        store_strip<T, RW>(a.dx + static_cast<int64_t>(plane) * hw + static_cast<int64_t>(h0 + row) * a.w + w0,
                           acc[m], a.w - w0, vec);
    }
}

// Band plan of the input-gradient kernels: about one strip per thread
// (the generic kernel allows up to four), the K-slab tile (two buffers on
// the fast path) within the LDS budget.  Returns false when even one row
// does not fit.
struct InPlan {
    int BH, nbands, lds_bytes;
    bool fast;
};

template <typename T>
bool plan_dynbwd_input(int n, int c, int h, int w, int k, int maxdil, bool vf, InPlan &p) {
    constexpr int RW = Vec<T>::N;
    const int NS = (w + RW - 1) / RW;
    int hp, LW;
    dyn_tile(w, (k - 1) / 2 * maxdil, hp, LW);
    auto bytes = [&](int bh, int nbuf) -> int64_t {
        // + RW: a partial last strip may read past the last row of the last slab
        const int64_t cnt = static_cast<int64_t>(nbuf) * k * bh * LW + RW;
        if (cnt > (1 << 24)) return INT64_MAX;
        return cnt * static_cast<int64_t>(sizeof(float));
    };
    const bool kfast = (k == 3 || k == 5) && vf;
    const int bh1 = std::max(1, std::min(h, kThreads / NS));
    if (kfast && NS <= kThreads) {
        int bh = bh1;
        while (bh > 1 && bytes(bh, 2) > kLdsCap) --bh;
        if (bytes(bh, 2) <= kLdsCap) {
            p.nbands = (h + bh - 1) / bh;
            p.BH = (h + p.nbands - 1) / p.nbands;
            p.lds_bytes = static_cast<int>(bytes(p.BH, 2));
            p.fast = true;
            return true;
        }
    }
    if (NS > 4 * kThreads) return false;
    int bh = bh1;
    while (bh > 1 && bytes(bh, 1) > kLdsCap) --bh;
    if (bytes(bh, 1) > kLdsCap) return false;
    p.nbands = (h + bh - 1) / bh;
    p.BH = (h + p.nbands - 1) / p.nbands;
    p.lds_bytes = static_cast<int>(bytes(p.BH, 1));
    p.fast = false;
    return true;
}

template <typename T, int K_, int RW>
void launch_input_fast(int nb, dim3 grid, int lds, hipStream_t s, const DynBwdArgs<T> &g) {
    switch (nb) {
        case 1: hipLaunchKernelGGL((dynbwd_input_kernel<T, K_, RW, 1>), grid, dim3(kThreads), lds, s, g); break;
        case 2: hipLaunchKernelGGL((dynbwd_input_kernel<T, K_, RW, 2>), grid, dim3(kThreads), lds, s, g); break;
        case 3: hipLaunchKernelGGL((dynbwd_input_kernel<T, K_, RW, 3>), grid, dim3(kThreads), lds, s, g); break;
        default: hipLaunchKernelGGL((dynbwd_input_kernel<T, K_, RW, 4>), grid, dim3(kThreads), lds, s, g); break;
    }
}

template <typename T>
int run_dynbwd(const void *x, const void *const *filters, const void *dy, int dych, int dyoff, const int32_t *dil,
               int nb, void *dx, void *const *dfilters, int n, int c, int h, int w, int k, hipStream_t s) {
    constexpr int RW = Vec<T>::N;
    int maxdil = 1;
    for (int b = 0; b < nb; ++b) maxdil = std::max(maxdil, static_cast<int>(dil[b]));
    bool want_df = false;
    for (int b = 0; b < nb; ++b) want_df = want_df || (dfilters && dfilters[b]);

    DynBwdArgs<T> a;
    a.x = static_cast<const T *>(x);
    a.dy = static_cast<const T *>(dy);
    a.dych = dych;
    a.dyoff = dyoff;
    a.dx = static_cast<T *>(dx);
    bool al = reinterpret_cast<uintptr_t>(dy) % 16 == 0 && (!dx || reinterpret_cast<uintptr_t>(dx) % 16 == 0);
    for (int b = 0; b < kMaxBranches; ++b) {
        const bool on = b < nb;
        a.f[b] = on ? static_cast<const T *>(filters[b]) : nullptr;
        a.df[b] = on && dfilters ? static_cast<T *>(dfilters[b]) : nullptr;
        a.dil[b] = on ? dil[b] : 1;
        if (on) al = al && reinterpret_cast<uintptr_t>(filters[b]) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(a.df[b]) % 16 == 0;
    }
    a.nb = nb;
    a.n = n;
    a.c = c;
    a.h = h;
    a.w = w;
    a.k = k;
    a.NS = (w + RW - 1) / RW;
    a.halo = (k - 1) / 2 * maxdil;
    dyn_tile(w, a.halo, a.hp, a.LW);
    a.vin = reinterpret_cast<uintptr_t>(x) % 16 == 0 && w % Vec<T>::N == 0;
    a.vf = al && (w % RW == 0);
    const int vpr = std::max(w / Vec<T>::N, 1);
    const int64_t planes = static_cast<int64_t>(n) * c;

    if (want_df) {
        DynPlan p;
        if (!plan_dyn<T>(n, c, h, w, k, maxdil, p, 1)) return kErrUnsupported;
        DynBwdArgs<T> f = a;
        f.BH = p.BH;
        f.nbands = p.nbands;
        f.fNS = make_fastdiv(f.NS, static_cast<uint64_t>(p.BH) * f.NS);
        const int rows_max = p.BH + 2 * a.halo;
        f.fLW = make_fastdiv(a.LW, static_cast<uint64_t>(rows_max) * a.LW);
        f.fVPR = make_fastdiv(vpr, static_cast<uint64_t>(rows_max) * vpr);
        f.fPAD = make_fastdiv(a.LW - w, static_cast<uint64_t>(rows_max) * (a.LW - w));
        const dim3 grid(static_cast<unsigned>(planes * p.nbands));
        const bool vf = a.vf != 0;
        if (k == 3 && vf)
            hipLaunchKernelGGL((dynbwd_filter_kernel<T, 3, RW, true>), grid, dim3(kThreads), p.lds_bytes, s, f);
        else if (k == 3)
            hipLaunchKernelGGL((dynbwd_filter_kernel<T, 3, RW, false>), grid, dim3(kThreads), p.lds_bytes, s, f);
        else if (k == 5 && vf)
            hipLaunchKernelGGL((dynbwd_filter_kernel<T, 5, RW, true>), grid, dim3(kThreads), p.lds_bytes, s, f);
        else
            hipLaunchKernelGGL((dynbwd_filter_kernel<T, 0, RW, false>), grid, dim3(kThreads), p.lds_bytes, s, f);
        if (hipGetLastError() != hipSuccess) return kErrHip;
    }
    if (dx) {
        InPlan p;
        if (!plan_dynbwd_input<T>(n, c, h, w, k, maxdil, a.vf != 0, p)) return kErrUnsupported;
        DynBwdArgs<T> g = a;
        g.BH = p.BH;
        g.nbands = p.nbands;
        g.fNS = make_fastdiv(g.NS, static_cast<uint64_t>(p.BH) * g.NS);
        const int nrows = (p.fast ? 2 : 1) * k * p.BH;
        g.fPAD = make_fastdiv(a.LW - w, static_cast<uint64_t>(nrows) * (a.LW - w));
        const dim3 grid(static_cast<unsigned>(planes * p.nbands));
        if (p.fast && k == 3)
            launch_input_fast<T, 3, RW>(nb, grid, p.lds_bytes, s, g);
        else if (p.fast)
            launch_input_fast<T, 5, RW>(nb, grid, p.lds_bytes, s, g);
        else
            hipLaunchKernelGGL((dynbwd_input_generic_kernel<T, RW>), grid, dim3(kThreads), p.lds_bytes, s, g);
        if (hipGetLastError() != hipSuccess) return kErrHip;
    }
    return kOk;
}

template <typename T>
bool dynbwd_fits(int h, int w, int k, int maxdil) {
    DynPlan p;
    InPlan q;
    return plan_dyn<T>(1, 1, h, w, k, maxdil, p) && plan_dynbwd_input<T>(1, 1, h, w, k, maxdil, false, q);
}

}  // namespace

bool dynconv_bwd_supported(int h, int w, int k, int maxdil, int dtype) {
    return dtype == 0 ? dynbwd_fits<float>(h, w, k, maxdil) : dynbwd_fits<__half>(h, w, k, maxdil);
}

int launch_dynconv_bwd(const void *x, const void *const *filters, const void *dy, int dych, int dyoff,
                       const int32_t *dil, int nb, void *dx, void *const *dfilters, int n, int c, int h, int w,
                       int k, int dtype, hipStream_t s) {
    int maxdil = 1;
    for (int b = 0; b < nb; ++b) maxdil = std::max(maxdil, static_cast<int>(dil[b]));
    if (!dynconv_bwd_supported(h, w, k, maxdil, dtype))  // rows too wide to stage: direct kernels
        return direct_dynconv_bwd(x, filters, dy, dych, dyoff, dil, nb, dx, dfilters, n, c, h, w, k, dtype, s);
    switch (dtype) {
        case 0: return run_dynbwd<float>(x, filters, dy, dych, dyoff, dil, nb, dx, dfilters, n, c, h, w, k, s);
        case 1: return run_dynbwd<__half>(x, filters, dy, dych, dyoff, dil, nb, dx, dfilters, n, c, h, w, k, s);
        default: return run_dynbwd<bf16_t>(x, filters, dy, dych, dyoff, dil, nb, dx, dfilters, n, c, h, w, k, s);
    }
}

}  // namespace dw
