// dw_dynconv.hip -- fused per-pixel dynamic filter at several dilations on gfx950.
//
//   y[n, b*C + c, h, w] = sum_{i,j<k} F_b[n, c, i*k + j, h, w] * x[n, c, h + (i-r)d_b, w + (j-r)d_b]
// with r = (k-1)/2 and zero outside the image (lartpang/DynamicConvolutionOperator:
// HDFNet's Dynamic Dilated Pyramid computation; its fused design gathers all
// dilation branches in one program and stores each branch's pixels straight
// into the concatenated output, so no unfolded copy and no concatenation).
//
// The op moves ~k*k*nb filter values per output pixel and does one FMA per
// value, so it is bound by HBM bandwidth.  A workgroup owns a band of rows of
// one (n, c) plane: the x rows of the band plus the largest dilation's halo
// are staged in LDS once, as fp32 with zero columns on both sides (so no tap
// needs a column test and no conversion), and serve every branch; each thread
// produces RW adjacent pixels of one row for all branches, streaming every
// filter tap as one 16-byte coalesced load and writing each branch's strip at
// its channel offset b*C + c of the concatenated output (or, for a caller's
// larger concatenation, at channel yoff + b*C + c of an output of ych channels).
#include "dw_dyn.hpp"

namespace dw {
namespace {

using namespace dyn;

template <typename T> struct DynArgs {
    const T *x;
    const T *f[kMaxBranches];
    T *y;
    int dil[kMaxBranches];
    int nb;
    int n, c, h, w, k;
    int ych, yoff;  // channels of the output tensor, channel of branch 0's first plane
    int BH, nbands, NS;
    FastDiv fNS;
    int halo;   // r * max dilation
    int hp;     // zero columns left of the staged rows: halo rounded up to 4
    int LW;     // staged row pitch in floats (multiple of 4)
    FastDiv fLW, fVPR, fPAD;
    int vin;    // x 16-byte aligned and rows of whole 16-byte vectors
    int vf;     // filters and y rows allow 16-byte strips
};

// VF: every strip is a whole aligned 16-byte vector (w a multiple of RW), so
// the filter loads of a branch are issued together, unconditionally, before
// any of them is used (behind a per-strip branch each load was waited on at
// once, serialising the nine loads).
template <typename T, int K_, int RW, bool VF>
__global__ __launch_bounds__(kThreads) void dynconv_kernel(DynArgs<T> a) {
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
    // LDS row r holds image row rbase + r (zeros outside the image), for every
    // row a tap of the band can reach: no tap needs a row test
    const int rbase = h0 - a.halo;
    const int rows = (h1 - h0) + 2 * a.halo;
    const int LW = a.LW, hp = a.hp;

    // stage x rows as fp32: row r at xs[r*LW + hp ...], zeros elsewhere in the row
    const T *src = a.x + static_cast<int64_t>(plane) * hw;
    stage_rows_f32<T>(xs, src, rbase, rows, a.h, a.w, LW, hp, a.fVPR, a.fPAD, a.fLW, a.vin != 0, tid);
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
            const int d = a.dil[b];
            const T *fb = a.f[b] + static_cast<int64_t>(plane) * KK * hw + pix;
            float acc[RW];
#pragma unroll
            for (int q = 0; q < RW; ++q) acc[q] = 0.f;
            if constexpr (VF && K_ > 0) {
                constexpr int KK_ = K_ * K_;
                u32x4 fr[KK_];
#pragma unroll
                for (int t = 0; t < KK_; ++t)
                    fr[t] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4 *>(fb + static_cast<int64_t>(t) * hw));
                __builtin_amdgcn_sched_barrier(0);  // all taps in flight before the first use
#pragma unroll
                for (int i = 0; i < K_; ++i) {
                    const float *rp = xs + (hh + (i - rr) * d - rbase) * LW + hp + w0;
#pragma unroll
                    for (int j = 0; j < K_; ++j) {
                        float fv[RW], xv[RW];
                        strip_values<T, RW>(fr[i * K_ + j], fv);
                        if (j == rr) {
#pragma unroll
                            for (int q = 0; q < RW; q += 4) {
                                const float4 v4 = *reinterpret_cast<const float4 *>(rp + q);
                                xv[q] = v4.x;
                                xv[q + 1] = v4.y;
                                xv[q + 2] = v4.z;
                                xv[q + 3] = v4.w;
                            }
                        } else {
                            const int off = (j - rr) * d;
#pragma unroll
                            for (int q = 0; q < RW; ++q) xv[q] = rp[off + q];
                        }
#pragma unroll
                        for (int q = 0; q < RW; ++q) acc[q] = fmaf(fv[q], xv[q], acc[q]);
                    }
                }
                T *yp = a.y + (static_cast<int64_t>(nn) * a.ych + a.yoff + b * a.c + ch) * hw + pix;
                store_strip<T, RW>(yp, acc, RW, true);
                continue;
            }
            for (int i = 0; i < K; ++i) {  // K is a constant unless k is a runtime size
                const int sy = hh + (i - rr) * d;
                if (sy < 0 || sy >= a.h) continue;  // whole filter row multiplies zero padding
                const float *rp = xs + (sy - rbase) * LW + hp + w0;  // column w0 of row sy
                for (int j = 0; j < K; ++j) {
                    float fv[RW], xv[RW];
                    load_strip<T, RW>(fb + static_cast<int64_t>(i * K + j) * hw, fv, valid, a.vf != 0);
                    if (K_ && j == rr) {
                        // centre column: RW floats at a 16-byte aligned address
#pragma unroll
                        for (int q = 0; q < RW; q += 4) {
                            const float4 v4 = *reinterpret_cast<const float4 *>(rp + q);
                            xv[q] = v4.x;
                            xv[q + 1] = v4.y;
                            xv[q + 2] = v4.z;
                            xv[q + 3] = v4.w;
                        }
                    } else {
                        const int off = (j - rr) * d;
#pragma unroll
                        for (int q = 0; q < RW; ++q) xv[q] = rp[off + q];
                    }
#pragma unroll
                    for (int q = 0; q < RW; ++q) acc[q] = fmaf(fv[q], xv[q], acc[q]);
                }
            }
            T *yp = a.y + (static_cast<int64_t>(nn) * a.ych + a.yoff + b * a.c + ch) * hw + pix;
            store_strip<T, RW>(yp, acc, valid, a.vf != 0);
        }
    }
}

template <typename T>
int run_dyn(const void *x, const void *const *filters, const int32_t *dil, int nb, void *y, int ych, int yoff,
            int n, int c, int h, int w, int k, hipStream_t s) {
    constexpr int RW = Vec<T>::N;
    int maxdil = 1;
    for (int b = 0; b < nb; ++b) maxdil = std::max(maxdil, static_cast<int>(dil[b]));
    DynPlan p;
    if (!plan_dyn<T>(n, c, h, w, k, maxdil, p)) return kErrUnsupported;
    DynArgs<T> a;
    a.x = static_cast<const T *>(x);
    bool fal = true;
    for (int b = 0; b < kMaxBranches; ++b) {
        a.f[b] = b < nb ? static_cast<const T *>(filters[b]) : nullptr;
        a.dil[b] = b < nb ? dil[b] : 1;
        if (b < nb) fal = fal && (reinterpret_cast<uintptr_t>(filters[b]) % 16 == 0);
    }
    a.y = static_cast<T *>(y);
    a.ych = ych;
    a.yoff = yoff;
    a.nb = nb;
    a.n = n;
    a.c = c;
    a.h = h;
    a.w = w;
    a.k = k;
    a.BH = p.BH;
    a.nbands = p.nbands;
    a.NS = (w + RW - 1) / RW;
    a.fNS = make_fastdiv(a.NS, static_cast<uint64_t>(p.BH) * a.NS);
    a.halo = (k - 1) / 2 * maxdil;
    dyn_tile(w, a.halo, a.hp, a.LW);
    const int rows_max = p.BH + 2 * a.halo;
    const int vpr = w / Vec<T>::N;
    a.fLW = make_fastdiv(a.LW, static_cast<uint64_t>(rows_max) * a.LW);
    a.fVPR = make_fastdiv(std::max(vpr, 1), static_cast<uint64_t>(rows_max) * std::max(vpr, 1));
    a.fPAD = make_fastdiv(a.LW - w, static_cast<uint64_t>(rows_max) * (a.LW - w));
    a.vin = reinterpret_cast<uintptr_t>(x) % 16 == 0 && w % Vec<T>::N == 0;
    a.vf = fal && (w % RW == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(n) * c * p.nbands));
    const bool vf = a.vf != 0;
    if (k == 3 && vf)
        hipLaunchKernelGGL((dynconv_kernel<T, 3, RW, true>), grid, dim3(kThreads), p.lds_bytes, s, a);
    else if (k == 3)
        hipLaunchKernelGGL((dynconv_kernel<T, 3, RW, false>), grid, dim3(kThreads), p.lds_bytes, s, a);
    else if (k == 5 && vf)
        hipLaunchKernelGGL((dynconv_kernel<T, 5, RW, true>), grid, dim3(kThreads), p.lds_bytes, s, a);
    else if (k == 5)
        hipLaunchKernelGGL((dynconv_kernel<T, 5, RW, false>), grid, dim3(kThreads), p.lds_bytes, s, a);
    else
        hipLaunchKernelGGL((dynconv_kernel<T, 0, RW, false>), grid, dim3(kThreads), p.lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

}  // namespace

bool dynconv_supported(int h, int w, int k, int maxdil, int dtype) {
    DynPlan p;
    return dtype == 0 ? plan_dyn<float>(1, 1, h, w, k, maxdil, p) : plan_dyn<__half>(1, 1, h, w, k, maxdil, p);
}

int launch_dynconv(const void *x, const void *const *filters, const int32_t *dil, int nb, void *y, int ych,
                   int yoff, int n, int c, int h, int w, int k, int dtype, hipStream_t s) {
    int maxdil = 1;
    for (int b = 0; b < nb; ++b) maxdil = std::max(maxdil, static_cast<int>(dil[b]));
    if (!dynconv_supported(h, w, k, maxdil, dtype))  // rows too wide to stage: direct kernel
        return direct_dynconv(x, filters, dil, nb, y, ych, yoff, n, c, h, w, k, dtype, s);
    switch (dtype) {
        case 0: return run_dyn<float>(x, filters, dil, nb, y, ych, yoff, n, c, h, w, k, s);
        case 1: return run_dyn<__half>(x, filters, dil, nb, y, ych, yoff, n, c, h, w, k, s);
        default: return run_dyn<bf16_t>(x, filters, dil, nb, y, ych, yoff, n, c, h, w, k, s);
    }
}

}  // namespace dw
