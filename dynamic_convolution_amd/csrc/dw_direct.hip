// dw_direct.hip -- direct kernels that serve every valid geometry: one thread
// per output element, every operand read from global memory (through the
// caches), no LDS staging and therefore no size limit beyond the library's
// 2^31-element tensors.
//
// The specialised families stage whole input rows (or bands of them) in LDS;
// a row too wide for the 64 KiB a workgroup may stage (a 31 x 31 filter over
// rows of 600, a 3 x 3 filter over rows of 16384) used to be refused.  These
// kernels compute the same sums straight from the definitions (PR #3057:
// depthwise forward, grad-input and grad-weight with padding, stride,
// dilation and multiplier; lartpang/DynamicConvolutionOperator: the fused
// per-pixel filter at several dilations and its backward), fp32 accumulation,
// taps in a fixed order.  They are the last choice of the selection rules.
#include "dw_common.hpp"
#include "dw_internal.hpp"

namespace dw {
namespace {

constexpr int kDirectThreads = 256;
constexpr int kDirectMaxBlocks = 65536;
constexpr int kDirectBranches = 4;

// Per-branch filter pointers and dilations of the dynamic filter (by value).
template <typename T> struct DynPtrs {
    const T *p[kDirectBranches];
    int dil[kDirectBranches];
};

inline unsigned direct_blocks(int64_t items) {
    const int64_t b = (items + kDirectThreads - 1) / kDirectThreads;
    return static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(b, kDirectMaxBlocks)));
}

// y[n, o, p, q] = b[o] + sum_{i, j} w[o, i, j] x[n, o / M, p*sh - ph + i*dh, q*sw - pw + j*dw]
template <typename T>
__global__ __launch_bounds__(kDirectThreads) void direct_fwd_kernel(const T *__restrict__ x, const T *__restrict__ w,
                                                                   const T *__restrict__ b, T *__restrict__ y,
                                                                   Geo g) {
    const int64_t total = static_cast<int64_t>(g.n) * g.oc * g.oh * g.ow;
    for (int64_t e = blockIdx.x * static_cast<int64_t>(kDirectThreads) + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * kDirectThreads) {
        const int q = static_cast<int>(e % g.ow);
        int64_t r = e / g.ow;
        const int p = static_cast<int>(r % g.oh);
        r /= g.oh;
        const int o = static_cast<int>(r % g.oc);
        const int n = static_cast<int>(r / g.oc);
        const T *xp = x + (static_cast<int64_t>(n) * g.ic + o / g.mult) * g.ih * g.iw;
        const T *wp = w + static_cast<int64_t>(o) * g.kh * g.kw;
        float acc = b ? to_f32(b[o]) : 0.f;
        for (int i = 0; i < g.kh; ++i) {
            const int h = p * g.sh - g.ph + i * g.dh;
            if (h < 0 || h >= g.ih) continue;
            for (int j = 0; j < g.kw; ++j) {
                const int c = q * g.sw - g.pw + j * g.dw;
                if (c < 0 || c >= g.iw) continue;
                acc = fmaf(to_f32(wp[i * g.kw + j]), to_f32(xp[static_cast<int64_t>(h) * g.iw + c]), acc);
            }
        }
        y[e] = from_f32<T>(acc);
    }
}

// dx[n, gi, h, c] = sum over m, i, j with (h + ph - i*dh) = p*sh and (c + pw - j*dw) = q*sw
// (p, q inside the output) of w[gi*M + m, i, j] dy[n, gi*M + m, p, q]
template <typename T>
__global__ __launch_bounds__(kDirectThreads) void direct_bwd_input_kernel(const T *__restrict__ dy,
                                                                         const T *__restrict__ w,
                                                                         T *__restrict__ dx, Geo g) {
    const int64_t total = static_cast<int64_t>(g.n) * g.ic * g.ih * g.iw;
    for (int64_t e = blockIdx.x * static_cast<int64_t>(kDirectThreads) + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * kDirectThreads) {
        const int c = static_cast<int>(e % g.iw);
        int64_t r = e / g.iw;
        const int h = static_cast<int>(r % g.ih);
        r /= g.ih;
        const int gi = static_cast<int>(r % g.ic);
        const int n = static_cast<int>(r / g.ic);
        float acc = 0.f;
        for (int m = 0; m < g.mult; ++m) {
            const int o = gi * g.mult + m;
            const T *dp = dy + (static_cast<int64_t>(n) * g.oc + o) * g.oh * g.ow;
            const T *wp = w + static_cast<int64_t>(o) * g.kh * g.kw;
            for (int i = 0; i < g.kh; ++i) {
                const int tp = h + g.ph - i * g.dh;
                if (tp < 0 || tp % g.sh != 0) continue;
                const int p = tp / g.sh;
                if (p >= g.oh) continue;
                for (int j = 0; j < g.kw; ++j) {
                    const int tq = c + g.pw - j * g.dw;
                    if (tq < 0 || tq % g.sw != 0) continue;
                    const int q = tq / g.sw;
                    if (q >= g.ow) continue;
                    acc = fmaf(to_f32(wp[i * g.kw + j]), to_f32(dp[static_cast<int64_t>(p) * g.ow + q]), acc);
                }
            }
        }
        dx[e] = from_f32<T>(acc);
    }
}

// Pass 1 of grad-weight: workgroup (input channel, chunk of output rows (n, p),
// group of slots); thread = slot s = m * (kk + 1) + t of the chunk partial
// [ic][NC][M (kk + 1)]: tap t < kk of output channel ic*M + m, or its dy sum at
// t == kk.  Each thread walks the chunk's rows in order.
template <typename T>
__global__ __launch_bounds__(kDirectThreads) void direct_bwd_weight_kernel(const T *__restrict__ x,
                                                                          const T *__restrict__ dy,
                                                                          float *__restrict__ ws, Geo g, int NC,
                                                                          int rpc, int nsg) {
    const int kk = g.kh * g.kw;
    const int nslots = g.mult * (kk + 1);
    const int sg = blockIdx.x % nsg;
    const int chunk = (blockIdx.x / nsg) % NC;
    const int gi = blockIdx.x / (nsg * NC);
    const int slot = sg * kDirectThreads + threadIdx.x;
    if (slot >= nslots) return;
    const int m = slot / (kk + 1), t = slot - m * (kk + 1);
    const int o = gi * g.mult + m;
    const int i = t < kk ? t / g.kw : 0, j = t < kk ? t - (t / g.kw) * g.kw : 0;
    const int64_t rows = static_cast<int64_t>(g.n) * g.oh;
    const int64_t r0 = static_cast<int64_t>(chunk) * rpc;
    const int64_t r1 = r0 + rpc < rows ? r0 + rpc : rows;
    float acc = 0.f;
    for (int64_t rr = r0; rr < r1; ++rr) {
        const int n = static_cast<int>(rr / g.oh), p = static_cast<int>(rr % g.oh);
        const T *dp = dy + ((static_cast<int64_t>(n) * g.oc + o) * g.oh + p) * g.ow;
        if (t == kk) {
            for (int q = 0; q < g.ow; ++q) acc += to_f32(dp[q]);
            continue;
        }
        const int h = p * g.sh - g.ph + i * g.dh;
        if (h < 0 || h >= g.ih) continue;
        const T *xp = x + ((static_cast<int64_t>(n) * g.ic + gi) * g.ih + h) * g.iw;
        for (int q = 0; q < g.ow; ++q) {
            const int c = q * g.sw - g.pw + j * g.dw;
            if (c < 0 || c >= g.iw) continue;
            acc = fmaf(to_f32(dp[q]), to_f32(xp[c]), acc);
        }
    }
    ws[(static_cast<int64_t>(gi) * NC + chunk) * nslots + slot] = acc;
}

// Dynamic filter forward: y[n, yoff + b*c + ch, h, w] = sum_{i, j} F_b[n, ch, i*k + j, h, w]
// x[n, ch, h + (i - r) d_b, w + (j - r) d_b]
template <typename T>
__global__ __launch_bounds__(kDirectThreads) void direct_dyn_fwd_kernel(const T *__restrict__ x, DynPtrs<T> f,
                                                                       T *__restrict__ y, int ych, int yoff, int nb,
                                                                       int n, int c, int h, int w, int k) {
    const int64_t hw = static_cast<int64_t>(h) * w;
    const int64_t total = static_cast<int64_t>(n) * nb * c * hw;
    const int rad = (k - 1) / 2;
    for (int64_t e = blockIdx.x * static_cast<int64_t>(kDirectThreads) + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * kDirectThreads) {
        const int64_t pix = e % hw;
        int64_t r = e / hw;
        const int ch = static_cast<int>(r % c);
        r /= c;
        const int b = static_cast<int>(r % nb);
        const int nn = static_cast<int>(r / nb);
        const int hh = static_cast<int>(pix / w), ww = static_cast<int>(pix % w);
        const int d = f.dil[b];
        const T *xp = x + (static_cast<int64_t>(nn) * c + ch) * hw;
        const T *fp = f.p[b] + (static_cast<int64_t>(nn) * c + ch) * k * k * hw + pix;
        float acc = 0.f;
        for (int i = 0; i < k; ++i) {
            const int sh = hh + (i - rad) * d;
            for (int j = 0; j < k; ++j) {
                const int sw = ww + (j - rad) * d;
                if (sh < 0 || sh >= h || sw < 0 || sw >= w) continue;
                acc = fmaf(to_f32(fp[(i * k + j) * hw]), to_f32(xp[static_cast<int64_t>(sh) * w + sw]), acc);
            }
        }
        y[(static_cast<int64_t>(nn) * ych + yoff + b * c + ch) * hw + pix] = from_f32<T>(acc);
    }
}

// Dynamic filter gradients: dF_b[n, ch, t, h, w] = dy[n, dyoff + b*c + ch, h, w] x(shifted), 0 outside
template <typename T>
__global__ __launch_bounds__(kDirectThreads) void direct_dyn_dfilter_kernel(const T *__restrict__ x,
                                                                           const T *__restrict__ dy,
                                                                           T *__restrict__ out, int d, int dych,
                                                                           int dyoff, int b, int n, int c, int h,
                                                                           int w, int k) {
    const int64_t hw = static_cast<int64_t>(h) * w;
    const int kk = k * k;
    const int64_t total = static_cast<int64_t>(n) * c * kk * hw;
    const int rad = (k - 1) / 2;
    for (int64_t e = blockIdx.x * static_cast<int64_t>(kDirectThreads) + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * kDirectThreads) {
        const int64_t pix = e % hw;
        int64_t r = e / hw;
        const int t = static_cast<int>(r % kk);
        r /= kk;
        const int ch = static_cast<int>(r % c);
        const int nn = static_cast<int>(r / c);
        const int hh = static_cast<int>(pix / w), ww = static_cast<int>(pix % w);
        const int sh = hh + (t / k - rad) * d, sw = ww + (t % k - rad) * d;
        float v = 0.f;
        if (sh >= 0 && sh < h && sw >= 0 && sw < w)
            v = to_f32(dy[(static_cast<int64_t>(nn) * dych + dyoff + b * c + ch) * hw + pix]) *
                to_f32(x[(static_cast<int64_t>(nn) * c + ch) * hw + static_cast<int64_t>(sh) * w + sw]);
        out[e] = from_f32<T>(v);
    }
}

// Dynamic input gradient: dx[n, ch, s, u] = sum_b sum_t F_b[n, ch, t, p] dy[n, dyoff + b*c + ch, p]
// at the pixel p = (s - (i - r) d_b, u - (j - r) d_b) inside the image; branches then taps in order
template <typename T>
__global__ __launch_bounds__(kDirectThreads) void direct_dyn_dx_kernel(DynPtrs<T> f, const T *__restrict__ dy,
                                                                      T *__restrict__ dx, int dych, int dyoff,
                                                                      int nb, int n, int c, int h, int w, int k) {
    const int64_t hw = static_cast<int64_t>(h) * w;
    const int64_t total = static_cast<int64_t>(n) * c * hw;
    const int rad = (k - 1) / 2;
    for (int64_t e = blockIdx.x * static_cast<int64_t>(kDirectThreads) + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * kDirectThreads) {
        const int64_t pix = e % hw;
        const int64_t plane = e / hw;  // n * c + ch
        const int ch = static_cast<int>(plane % c);
        const int nn = static_cast<int>(plane / c);
        const int ss = static_cast<int>(pix / w), uu = static_cast<int>(pix % w);
        float acc = 0.f;
        for (int b = 0; b < nb; ++b) {
            const int d = f.dil[b];
            const T *fp = f.p[b] + plane * k * k * hw;
            const T *dp = dy + (static_cast<int64_t>(nn) * dych + dyoff + b * c + ch) * hw;
            for (int i = 0; i < k; ++i) {
                const int ph = ss - (i - rad) * d;
                if (ph < 0 || ph >= h) continue;
                for (int j = 0; j < k; ++j) {
                    const int pw = uu - (j - rad) * d;
                    if (pw < 0 || pw >= w) continue;
                    const int64_t q = static_cast<int64_t>(ph) * w + pw;
                    acc = fmaf(to_f32(fp[(i * k + j) * hw + q]), to_f32(dp[q]), acc);
                }
            }
        }
        dx[e] = from_f32<T>(acc);
    }
}

struct DirectBwPlan {
    int NC, rpc, nsg;
};

DirectBwPlan plan_direct_bw(const Geo &g) {
    DirectBwPlan p;
    const int nslots = g.mult * (g.kh * g.kw + 1);
    p.nsg = (nslots + kDirectThreads - 1) / kDirectThreads;
    const int64_t rows = static_cast<int64_t>(g.n) * g.oh;
    // about 2048 workgroups, chunks of at least one output row
    const int64_t want = std::max<int64_t>(1, 2048 / std::max<int64_t>(1, static_cast<int64_t>(g.ic) * p.nsg));
    const int64_t nc = std::min<int64_t>(rows, std::min<int64_t>(want, 4096));
    p.rpc = static_cast<int>((rows + nc - 1) / nc);
    p.NC = static_cast<int>((rows + p.rpc - 1) / p.rpc);
    return p;
}

template <typename T>
int dyn_fwd_t(const void *x, const void *const *filters, const int32_t *dil, int nb, void *y, int ych, int yoff,
              int n, int c, int h, int w, int k, hipStream_t s) {
    DynPtrs<T> f{};
    for (int b = 0; b < nb; ++b) {
        f.p[b] = static_cast<const T *>(filters[b]);
        f.dil[b] = dil[b];
    }
    const int64_t total = static_cast<int64_t>(n) * nb * c * h * w;
    hipLaunchKernelGGL((direct_dyn_fwd_kernel<T>), dim3(direct_blocks(total)), dim3(kDirectThreads), 0, s,
                       static_cast<const T *>(x), f, static_cast<T *>(y), ych, yoff, nb, n, c, h, w, k);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T>
int dyn_bwd_t(const void *x, const void *const *filters, const void *dy, int dych, int dyoff, const int32_t *dil,
              int nb, void *dx, void *const *dfilters, int n, int c, int h, int w, int k, hipStream_t s) {
    DynPtrs<T> f{};
    for (int b = 0; b < nb; ++b) {
        f.p[b] = static_cast<const T *>(filters[b]);
        f.dil[b] = dil[b];
    }
    if (dfilters) {
        for (int b = 0; b < nb; ++b) {
            if (!dfilters[b]) continue;
            const int64_t total = static_cast<int64_t>(n) * c * k * k * h * w;
            hipLaunchKernelGGL((direct_dyn_dfilter_kernel<T>), dim3(direct_blocks(total)), dim3(kDirectThreads), 0, s,
                               static_cast<const T *>(x), static_cast<const T *>(dy), static_cast<T *>(dfilters[b]),
                               static_cast<int>(dil[b]), dych, dyoff, b, n, c, h, w, k);
            if (hipGetLastError() != hipSuccess) return kErrHip;
        }
    }
    if (dx) {
        const int64_t total = static_cast<int64_t>(n) * c * h * w;
        hipLaunchKernelGGL((direct_dyn_dx_kernel<T>), dim3(direct_blocks(total)), dim3(kDirectThreads), 0, s, f,
                           static_cast<const T *>(dy), static_cast<T *>(dx), dych, dyoff, nb, n, c, h, w, k);
        if (hipGetLastError() != hipSuccess) return kErrHip;
    }
    return kOk;
}

}  // namespace

int direct_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s) {
    const int64_t total = static_cast<int64_t>(g.n) * g.oc * g.oh * g.ow;
    const dim3 grid(direct_blocks(total)), block(kDirectThreads);
    switch (dtype) {
        case 0:
            hipLaunchKernelGGL((direct_fwd_kernel<float>), grid, block, 0, s, static_cast<const float *>(x),
                               static_cast<const float *>(w), static_cast<const float *>(b), static_cast<float *>(y), g);
            break;
        case 1:
            hipLaunchKernelGGL((direct_fwd_kernel<__half>), grid, block, 0, s, static_cast<const __half *>(x),
                               static_cast<const __half *>(w), static_cast<const __half *>(b), static_cast<__half *>(y),
                               g);
            break;
        default:
            hipLaunchKernelGGL((direct_fwd_kernel<bf16_t>), grid, block, 0, s, static_cast<const bf16_t *>(x),
                               static_cast<const bf16_t *>(w), static_cast<const bf16_t *>(b), static_cast<bf16_t *>(y),
                               g);
            break;
    }
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

int direct_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s) {
    const int64_t total = static_cast<int64_t>(g.n) * g.ic * g.ih * g.iw;
    const dim3 grid(direct_blocks(total)), block(kDirectThreads);
    switch (dtype) {
        case 0:
            hipLaunchKernelGGL((direct_bwd_input_kernel<float>), grid, block, 0, s, static_cast<const float *>(dy),
                               static_cast<const float *>(w), static_cast<float *>(dx), g);
            break;
        case 1:
            hipLaunchKernelGGL((direct_bwd_input_kernel<__half>), grid, block, 0, s, static_cast<const __half *>(dy),
                               static_cast<const __half *>(w), static_cast<__half *>(dx), g);
            break;
        default:
            hipLaunchKernelGGL((direct_bwd_input_kernel<bf16_t>), grid, block, 0, s, static_cast<const bf16_t *>(dy),
                               static_cast<const bf16_t *>(w), static_cast<bf16_t *>(dx), g);
            break;
    }
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

int direct_bwd_weight_chunks(const Geo &g) { return plan_direct_bw(g).NC; }

int direct_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s) {
    const DirectBwPlan p = plan_direct_bw(g);
    const dim3 grid(static_cast<unsigned>(g.ic) * p.NC * p.nsg), block(kDirectThreads);
    float *wsf = static_cast<float *>(ws);
    switch (dtype) {
        case 0:
            hipLaunchKernelGGL((direct_bwd_weight_kernel<float>), grid, block, 0, s, static_cast<const float *>(x),
                               static_cast<const float *>(dy), wsf, g, p.NC, p.rpc, p.nsg);
            break;
        case 1:
            hipLaunchKernelGGL((direct_bwd_weight_kernel<__half>), grid, block, 0, s, static_cast<const __half *>(x),
                               static_cast<const __half *>(dy), wsf, g, p.NC, p.rpc, p.nsg);
            break;
        default:
            hipLaunchKernelGGL((direct_bwd_weight_kernel<bf16_t>), grid, block, 0, s, static_cast<const bf16_t *>(x),
                               static_cast<const bf16_t *>(dy), wsf, g, p.NC, p.rpc, p.nsg);
            break;
    }
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

int direct_dynconv(const void *x, const void *const *filters, const int32_t *dil, int nb, void *y, int ych, int yoff,
                   int n, int c, int h, int w, int k, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return dyn_fwd_t<float>(x, filters, dil, nb, y, ych, yoff, n, c, h, w, k, s);
        case 1: return dyn_fwd_t<__half>(x, filters, dil, nb, y, ych, yoff, n, c, h, w, k, s);
        default: return dyn_fwd_t<bf16_t>(x, filters, dil, nb, y, ych, yoff, n, c, h, w, k, s);
    }
}

int direct_dynconv_bwd(const void *x, const void *const *filters, const void *dy, int dych, int dyoff,
                       const int32_t *dil, int nb, void *dx, void *const *dfilters, int n, int c, int h, int w, int k,
                       int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return dyn_bwd_t<float>(x, filters, dy, dych, dyoff, dil, nb, dx, dfilters, n, c, h, w, k, s);
        case 1: return dyn_bwd_t<__half>(x, filters, dy, dych, dyoff, dil, nb, dx, dfilters, n, c, h, w, k, s);
        default: return dyn_bwd_t<bf16_t>(x, filters, dy, dych, dyoff, dil, nb, dx, dfilters, n, c, h, w, k, s);
    }
}

}  // namespace dw
