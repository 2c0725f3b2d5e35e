// dw_rowwalk.hip -- streaming kernels for the 3x3, pad 1, dilation 1 depthwise
// layers (stride 1 and 2) on gfx950: forward, grad-input, grad-weight.
//
// These layers move ~8 bytes per multiply-add group and are bound by HBM
// bandwidth (the MobileNet layer table of PyTorch PR #3057 "Spatial Depthwise
// Convolution on the GPU" is this case).  Instead of staging tiles in LDS
// behind barriers, every lane owns one 16-byte column strip of a plane and
// walks down a band of rows:
//   - each input row segment is read once with a 16-byte load and converted
//     to fp32 registers; the column halo (one element left/right) comes from
//     the neighbouring lanes with a shuffle, the row halo from a rolling window
//     of the previous rows kept in registers;
//   - each output strip is written with one 16-byte store;
//   - no LDS tile and no barrier, so waves stream independently.
// A wave holds 64 / NS strips-of-a-row "slots" (NS = strips per row), each slot
// walking one (plane, band) unit; all slots of a wave take the same number of
// steps so the shuffles always see every lane active.
#include "dw_common.hpp"
#include "dw_internal.hpp"

namespace dw {
namespace {

constexpr int kWaves = kThreads / 64;

template <typename T> struct RwArgs {
    const T *in;    // forward: x; grad-input: dy; grad-weight: x
    const T *in2;   // grad-weight: dy
    const T *w;
    const T *b;
    T *out;         // y, dx
    float *ws;      // grad-weight partials [ic][chunk][M*10]
    Geo g;
    int NS;         // strips per row of the strip-defining tensor
    int SPW;        // slots per wave
    int BH;         // rows walked per unit
    int nbands;     // bands per plane
    int nunits;     // forward/grad-input: units in total; grad-weight: units per channel
    int NC;         // grad-weight: chunks per channel
    int upc;        // grad-weight: units per chunk
    int vin, vout;  // 16-byte loads / stores allowed
};

// Lane's IRW consecutive elements [c0, c0 + IRW) of row r (zero outside the image).
template <typename T, int IRW>
__device__ __forceinline__ void load_seg(const T *plane, int r, int H, int W, int c0, bool vec, bool act,
                                         float (&v)[IRW]) {
    constexpr int VE = Vec<T>::N;
    static_assert(IRW % VE == 0, "segment is whole vectors");
#pragma unroll
    for (int e = 0; e < IRW; ++e) v[e] = 0.f;
    if (!act || r < 0 || r >= H) return;
    const T *p = plane + static_cast<int64_t>(r) * W + c0;
    if (vec) {
#pragma unroll
        for (int k = 0; k < IRW / VE; ++k) {
            if (c0 + (k + 1) * VE <= W) {
                union {
                    uint4 u;
                    T t[VE];
                } b;
                b.u = *reinterpret_cast<const uint4 *>(p + k * VE);
#pragma unroll
                for (int e = 0; e < VE; ++e) v[k * VE + e] = to_f32(b.t[e]);
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < IRW; ++e)
            if (c0 + e < W) v[e] = to_f32(p[e]);
    }
}

template <typename T, int RW>
__device__ __forceinline__ void store_seg(T *p, const float *acc, int valid, bool vec) {
    if (vec && valid >= RW) {
        union {
            uint4 u;
            T t[RW];
        } b;
        static_assert(sizeof(T) * RW == 16, "strip is one 16-byte vector");
#pragma unroll
        for (int q = 0; q < RW; ++q) b.t[q] = from_f32<T>(acc[q]);
        *reinterpret_cast<uint4 *>(p) = b.u;
    } else {
#pragma unroll
        for (int q = 0; q < RW; ++q)
            if (q < valid) p[q] = from_f32<T>(acc[q]);
    }
}

// Window of one input row for a strip: win[0] = column c0 - 1 (from the left
// lane), win[1..IRW] = the lane's own segment, and for stride 1 win[IRW+1] =
// column c0 + IRW (from the right lane).
template <int IRW, int S>
__device__ __forceinline__ void make_window(const float (&v)[IRW], int lane, bool has_left, bool has_right,
                                            float (&win)[IRW + (S == 1 ? 2 : 1)]) {
    const float l = __shfl(v[IRW - 1], lane - 1, 64);
    win[0] = has_left ? l : 0.f;
#pragma unroll
    for (int e = 0; e < IRW; ++e) win[1 + e] = v[e];
    if constexpr (S == 1) {
        const float r = __shfl(v[0], lane + 1, 64);
        win[IRW + 1] = has_right ? r : 0.f;
    }
}

// ---------------------------------------------------------------- forward / grad-input (stride 1)
// FWD: one input plane x[P] -> MM output planes y[P*MM+m].
// BWD (stride 1 only): MM input planes dy[P*MM+m] -> one output plane dx[P],
// with the kernel flipped (for stride 1, pad 1 the adjoint is the same
// stencil with w[2-i][2-j]).
template <typename T, int S, int MM, bool BWD>
__global__ __launch_bounds__(kThreads) void rw_conv3_kernel(RwArgs<T> a) {
    constexpr int RW = Vec<T>::N;
    constexpr int IRW = RW * S;
    constexpr int WW = IRW + (S == 1 ? 2 : 1);
    constexpr int NIN = BWD ? MM : 1;   // input planes per unit
    constexpr int NOUT = BWD ? 1 : MM;  // output planes per unit
    static_assert(!BWD || S == 1, "stride-2 grad-input has its own kernel");
    const Geo &g = a.g;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slot = lane / a.NS;
    const int s = lane - slot * a.NS;
    const int unit = (blockIdx.x * kWaves + wave) * a.SPW + slot;
    const bool act = slot < a.SPW && unit < a.nunits;
    const int P = act ? unit / a.nbands : 0;
    const int band = act ? unit - P * a.nbands : 0;
    const int IH = BWD ? g.oh : g.ih, IW = BWD ? g.ow : g.iw;  // rows/cols of the input planes
    const int OH = BWD ? g.ih : g.oh, OW = BWD ? g.iw : g.ow;
    const int c_in = s * IRW;
    const int c_out = s * RW;
    const bool has_left = s > 0;
    const bool has_right = s < a.NS - 1;
    const int ic = P % g.ic;

    float wt[MM][9];
    float bias[NOUT];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t < 9; ++t)
            wt[m][t] = act ? to_f32(a.w[(ic * MM + m) * 9 + (BWD ? 8 - t : t)]) : 0.f;
#pragma unroll
    for (int o = 0; o < NOUT; ++o) bias[o] = (!BWD && act && a.b) ? to_f32(a.b[ic * MM + o]) : 0.f;

    const int64_t in_plane = static_cast<int64_t>(IH) * IW;
    const T *inp[NIN];
#pragma unroll
    for (int k = 0; k < NIN; ++k) inp[k] = a.in + (static_cast<int64_t>(P) * NIN + k) * in_plane;

    const int oh0 = band * a.BH;
    const int oh_end = min(oh0 + a.BH, OH);
    const bool vin = a.vin != 0;
    // rolling window: rows S*oh - 1 (w0, carried), S*oh (w1), S*oh + 1 (w2); the
    // raw segments of the next step's rows are loaded one step ahead (nx*)
    float w0[NIN][WW], w1[NIN][WW], w2[NIN][WW];
    float nxa[NIN][IRW], nxb[NIN][IRW];  // next step: row S*oh+S (stride 2: and S*oh+1 of next)
#pragma unroll
    for (int k = 0; k < NIN; ++k) {
        float v[IRW];
        load_seg<T, IRW>(inp[k], S * oh0 - 1, IH, IW, c_in, vin, act, v);
        make_window<IRW, S>(v, lane, has_left, has_right, w0[k]);
        if constexpr (S == 1) {
            load_seg<T, IRW>(inp[k], oh0, IH, IW, c_in, vin, act, v);
            make_window<IRW, S>(v, lane, has_left, has_right, w1[k]);
            load_seg<T, IRW>(inp[k], oh0 + 1, IH, IW, c_in, vin, act, nxb[k]);
        } else {
            load_seg<T, IRW>(inp[k], 2 * oh0, IH, IW, c_in, vin, act, nxa[k]);
            load_seg<T, IRW>(inp[k], 2 * oh0 + 1, IH, IW, c_in, vin, act, nxb[k]);
        }
    }
    for (int step = 0; step < a.BH; ++step) {
        const int oh = oh0 + step;
#pragma unroll
        for (int k = 0; k < NIN; ++k) {
            float cb[IRW];
#pragma unroll
            for (int e = 0; e < IRW; ++e) cb[e] = nxb[k][e];
            if constexpr (S == 2) {
                float ca[IRW];
#pragma unroll
                for (int e = 0; e < IRW; ++e) ca[e] = nxa[k][e];
                load_seg<T, IRW>(inp[k], 2 * oh + 2, IH, IW, c_in, vin, act, nxa[k]);
                load_seg<T, IRW>(inp[k], 2 * oh + 3, IH, IW, c_in, vin, act, nxb[k]);
                make_window<IRW, S>(ca, lane, has_left, has_right, w1[k]);
            } else {
                load_seg<T, IRW>(inp[k], oh + 2, IH, IW, c_in, vin, act, nxb[k]);
            }
            make_window<IRW, S>(cb, lane, has_left, has_right, w2[k]);
        }
        if (act && oh < oh_end) {
#pragma unroll
            for (int o = 0; o < NOUT; ++o) {
                float acc[RW];
#pragma unroll
                for (int q = 0; q < RW; ++q) acc[q] = bias[o];
#pragma unroll
                for (int k = 0; k < NIN; ++k) {
                    const float *wk = wt[BWD ? k : o];
#pragma unroll
                    for (int j = 0; j < 3; ++j)
#pragma unroll
                        for (int q = 0; q < RW; ++q) {
                            acc[q] = fmaf(wk[j], w0[k][q * S + j], acc[q]);
                            acc[q] = fmaf(wk[3 + j], w1[k][q * S + j], acc[q]);
                            acc[q] = fmaf(wk[6 + j], w2[k][q * S + j], acc[q]);
                        }
                }
                T *op = a.out + ((static_cast<int64_t>(P) * NOUT + o) * OH + oh) * OW + c_out;
                store_seg<T, RW>(op, acc, OW - c_out, a.vout != 0);
            }
        }
        // slide the window down
#pragma unroll
        for (int k = 0; k < NIN; ++k)
#pragma unroll
            for (int e = 0; e < WW; ++e) {
                if constexpr (S == 1) {
                    w0[k][e] = w1[k][e];
                    w1[k][e] = w2[k][e];
                } else {
                    w0[k][e] = w2[k][e];
                }
            }
    }
}

// ---------------------------------------------------------------- grad-input, stride 2
// For 3x3, pad 1, stride 2 the taps reaching dx split by parity:
//   dx[2r  ][2c  ] = w11 dy[r][c]
//   dx[2r  ][2c+1] = w10 dy[r][c+1] + w12 dy[r][c]
//   dx[2r+1][2c  ] = w01 dy[r+1][c] + w21 dy[r][c]
//   dx[2r+1][2c+1] = w00 dy[r+1][c+1] + w02 dy[r+1][c] + w20 dy[r][c+1] + w22 dy[r][c]
// (summed over the M output planes of the input channel; dy outside its plane
// is zero).  dx is four times dy, so the kernel is store-bound: a lane owns the
// DRW = RW/2 dy columns [c0, c0+DRW) and writes the RW dx columns [2c0, 2c0+RW)
// of dx rows 2r and 2r+1 as one 16-byte store each, so every store instruction
// of a wave covers one contiguous run of dx.
template <typename T, int DRW>
__device__ __forceinline__ void load_half(const T *plane, int r, int H, int W, int c0, bool vec, bool act,
                                          float (&v)[DRW]) {
    static_assert(sizeof(T) * DRW == 8, "half strip is 8 bytes");
#pragma unroll
    for (int e = 0; e < DRW; ++e) v[e] = 0.f;
    if (!act || r < 0 || r >= H) return;
    const T *p = plane + static_cast<int64_t>(r) * W + c0;
    if (vec && c0 + DRW <= W) {
        union {
            uint2 u;
            T t[DRW];
        } b;
        b.u = *reinterpret_cast<const uint2 *>(p);
#pragma unroll
        for (int e = 0; e < DRW; ++e) v[e] = to_f32(b.t[e]);
    } else {
#pragma unroll
        for (int e = 0; e < DRW; ++e)
            if (c0 + e < W) v[e] = to_f32(p[e]);
    }
}

template <typename T, int MM>
__global__ __launch_bounds__(kThreads) void rw_bwdin3_s2_kernel(RwArgs<T> a) {
    constexpr int RW = Vec<T>::N;
    constexpr int DRW = RW / 2;
    const Geo &g = a.g;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slot = lane / a.NS;
    const int s = lane - slot * a.NS;
    const int unit = (blockIdx.x * kWaves + wave) * a.SPW + slot;
    const bool act = slot < a.SPW && unit < a.nunits;
    const int P = act ? unit / a.nbands : 0;
    const int band = act ? unit - P * a.nbands : 0;
    const int c0 = s * DRW;
    const bool has_right = s < a.NS - 1;
    const int ic = P % g.ic;
    float wt[MM][9];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t < 9; ++t) wt[m][t] = act ? to_f32(a.w[(ic * MM + m) * 9 + t]) : 0.f;
    const int64_t dplane = static_cast<int64_t>(g.oh) * g.ow;
    const T *dp[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) dp[m] = a.in + (static_cast<int64_t>(P) * MM + m) * dplane;
    const int r0 = band * a.BH;
    // dy row r (cur) and r+1 (nxt), each with the right neighbour column; the
    // raw segment of row r+2 is loaded one step ahead (pre)
    float cur[MM][DRW + 1], nxt[MM][DRW + 1], pre[MM][DRW];
    const bool vin = a.vin != 0;
#pragma unroll
    for (int m = 0; m < MM; ++m) {
        float v[DRW];
        load_half<T, DRW>(dp[m], r0, g.oh, g.ow, c0, vin, act, v);
        const float rr = __shfl(v[0], lane + 1, 64);
#pragma unroll
        for (int e = 0; e < DRW; ++e) cur[m][e] = v[e];
        cur[m][DRW] = has_right ? rr : 0.f;
        load_half<T, DRW>(dp[m], r0 + 1, g.oh, g.ow, c0, vin, act, pre[m]);
    }
    // dx rows 2r and 2r+1 for r in the band; the band covers dx rows [2*r0, 2*(r0+BH))
    for (int step = 0; step < a.BH; ++step) {
        const int r = r0 + step;
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            float v[DRW];
#pragma unroll
            for (int e = 0; e < DRW; ++e) v[e] = pre[m][e];
            load_half<T, DRW>(dp[m], r + 2, g.oh, g.ow, c0, vin, act, pre[m]);
            const float rr = __shfl(v[0], lane + 1, 64);
#pragma unroll
            for (int e = 0; e < DRW; ++e) nxt[m][e] = v[e];
            nxt[m][DRW] = has_right ? rr : 0.f;
        }
        if (act && 2 * r < g.ih) {
            float e0[RW], e1[RW];  // dx rows 2r and 2r+1, columns 2c0 .. 2c0+RW-1
#pragma unroll
            for (int q = 0; q < RW; ++q) e0[q] = e1[q] = 0.f;
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                const float *w = wt[m];
#pragma unroll
                for (int q = 0; q < DRW; ++q) {
                    e0[2 * q] = fmaf(w[4], cur[m][q], e0[2 * q]);
                    e0[2 * q + 1] = fmaf(w[3], cur[m][q + 1], fmaf(w[5], cur[m][q], e0[2 * q + 1]));
                    e1[2 * q] = fmaf(w[1], nxt[m][q], fmaf(w[7], cur[m][q], e1[2 * q]));
                    e1[2 * q + 1] = fmaf(w[0], nxt[m][q + 1],
                                         fmaf(w[2], nxt[m][q], fmaf(w[6], cur[m][q + 1], fmaf(w[8], cur[m][q], e1[2 * q + 1]))));
                }
            }
            T *xp = a.out + (static_cast<int64_t>(P) * g.ih + 2 * r) * g.iw + 2 * c0;
            const int valid = g.iw - 2 * c0;
            store_seg<T, RW>(xp, e0, valid, a.vout != 0);
            if (2 * r + 1 < g.ih) store_seg<T, RW>(xp + g.iw, e1, valid, a.vout != 0);
        }
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int e = 0; e <= DRW; ++e) cur[m][e] = nxt[m][e];
    }
}

// ---------------------------------------------------------------- grad-weight
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Workgroup (ic, chunk): its lanes walk units (n, band) of input channel ic,
// accumulating for each of the MM output channels the 9 taps and the bias sum;
// one fixed-order workgroup reduction writes the chunk's partials.
template <typename T, int S, int MM>
__global__ __launch_bounds__(kThreads) void rw_bwdw3_kernel(RwArgs<T> a) {
    constexpr int RW = Vec<T>::N;
    constexpr int IRW = RW * S;
    constexpr int WW = IRW + (S == 1 ? 2 : 1);
    constexpr int A = MM * 10;
    __shared__ float red[kWaves][A];
    const Geo &g = a.g;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slot = lane / a.NS;
    const int s = lane - slot * a.NS;
    const int ic = blockIdx.x / a.NC;
    const int chunk = blockIdx.x - ic * a.NC;
    const int c_in = s * IRW;
    const int c_out = s * RW;
    const bool has_left = s > 0;
    const bool has_right = s < a.NS - 1;
    const int64_t xplane = static_cast<int64_t>(g.ih) * g.iw;
    const int64_t dplane = static_cast<int64_t>(g.oh) * g.ow;

    float acc[MM][10];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t < 10; ++t) acc[m][t] = 0.f;

    const int ubeg = chunk * a.upc;
    const int uend = min(ubeg + a.upc, a.nunits);
    for (int base = ubeg; base < uend; base += kWaves * a.SPW) {
        const int unit = base + wave * a.SPW + slot;
        const bool act = slot < a.SPW && unit < uend;
        const int n = act ? unit / a.nbands : 0;
        const int band = act ? unit - n * a.nbands : 0;
        const T *xp = a.in + (static_cast<int64_t>(n) * g.ic + ic) * xplane;
        const T *dyp = a.in2 + (static_cast<int64_t>(n) * g.oc + ic * MM) * dplane;
        const int oh0 = band * a.BH;
        const int oh_end = min(oh0 + a.BH, g.oh);
        const bool vin = a.vin != 0, vdy = a.vout != 0;
        float w0[WW], w1[WW], w2[WW];
        float nxa[IRW], nxb[IRW], ndy[MM][RW];  // next step's raw rows, loaded one step ahead
        {
            float v[IRW];
            load_seg<T, IRW>(xp, S * oh0 - 1, g.ih, g.iw, c_in, vin, act, v);
            make_window<IRW, S>(v, lane, has_left, has_right, w0);
            if constexpr (S == 1) {
                load_seg<T, IRW>(xp, oh0, g.ih, g.iw, c_in, vin, act, v);
                make_window<IRW, S>(v, lane, has_left, has_right, w1);
                load_seg<T, IRW>(xp, oh0 + 1, g.ih, g.iw, c_in, vin, act, nxb);
            } else {
                load_seg<T, IRW>(xp, 2 * oh0, g.ih, g.iw, c_in, vin, act, nxa);
                load_seg<T, IRW>(xp, 2 * oh0 + 1, g.ih, g.iw, c_in, vin, act, nxb);
            }
#pragma unroll
            for (int m = 0; m < MM; ++m)
                load_seg<T, RW>(dyp + m * dplane, oh0, g.oh, g.ow, c_out, vdy, act && oh0 < oh_end, ndy[m]);
        }
        for (int step = 0; step < a.BH; ++step) {
            const int oh = oh0 + step;
            float cb[IRW], gy[MM][RW];
#pragma unroll
            for (int e = 0; e < IRW; ++e) cb[e] = nxb[e];
#pragma unroll
            for (int m = 0; m < MM; ++m)
#pragma unroll
                for (int q = 0; q < RW; ++q) gy[m][q] = ndy[m][q];
            if constexpr (S == 2) {
                float ca[IRW];
#pragma unroll
                for (int e = 0; e < IRW; ++e) ca[e] = nxa[e];
                load_seg<T, IRW>(xp, 2 * oh + 2, g.ih, g.iw, c_in, vin, act, nxa);
                load_seg<T, IRW>(xp, 2 * oh + 3, g.ih, g.iw, c_in, vin, act, nxb);
                make_window<IRW, S>(ca, lane, has_left, has_right, w1);
            } else {
                load_seg<T, IRW>(xp, oh + 2, g.ih, g.iw, c_in, vin, act, nxb);
            }
#pragma unroll
            for (int m = 0; m < MM; ++m)
                load_seg<T, RW>(dyp + m * dplane, oh + 1, g.oh, g.ow, c_out, vdy, act && oh + 1 < oh_end, ndy[m]);
            make_window<IRW, S>(cb, lane, has_left, has_right, w2);
#pragma unroll
            for (int m = 0; m < MM; ++m) {
#pragma unroll
                for (int q = 0; q < RW; ++q) {
                    acc[m][9] += gy[m][q];
#pragma unroll
                    for (int j = 0; j < 3; ++j) {
                        acc[m][j] = fmaf(gy[m][q], w0[q * S + j], acc[m][j]);
                        acc[m][3 + j] = fmaf(gy[m][q], w1[q * S + j], acc[m][3 + j]);
                        acc[m][6 + j] = fmaf(gy[m][q], w2[q * S + j], acc[m][6 + j]);
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < WW; ++e) {
                if constexpr (S == 1) {
                    w0[e] = w1[e];
                    w1[e] = w2[e];
                } else {
                    w0[e] = w2[e];
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t < 10; ++t) {
            const float v = wave_sum(acc[m][t]);
            if (lane == 0) red[wave][m * 10 + t] = v;
        }
    __syncthreads();
    if (threadIdx.x < A) {
        float v = red[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) v += red[w][threadIdx.x];
        a.ws[(static_cast<int64_t>(ic) * a.NC + chunk) * A + threadIdx.x] = v;
    }
}

// ---------------------------------------------------------------- planning
struct RwPlan {
    int NS, SPW, BH, nbands, nunits, grid, NC, upc;
};

// Strips of 16 bytes per row of the strip-defining tensor (output rows for the
// forward, dy rows for grad-input stride 2, output rows for grad-weight).
template <typename T> int strips(int width) { return (width + Vec<T>::N - 1) / Vec<T>::N; }

// rows walked per unit: enough waves for the chip (>= ~8192 slots' worth of
// lanes) while keeping the 2-row halo re-read small.
inline int pick_bh(int64_t planes, int rows, int SPW, int min_bh) {
    int bh = rows;
    while (bh > min_bh && planes * ((rows + bh - 1) / bh) < int64_t{8192} * SPW / 2) bh = (bh + 1) / 2;
    const int nb = (rows + bh - 1) / bh;
    return (rows + nb - 1) / nb;
}

}  // namespace

bool rowwalk_applicable(const Geo &g, int pass) {
    if (g.kh != 3 || g.kw != 3 || g.ph != 1 || g.pw != 1 || g.dh != 1 || g.dw != 1) return false;
    if (g.sh != g.sw || (g.sh != 1 && g.sh != 2)) return false;
    if (g.mult > 2) return false;
    (void)pass;
    return true;
}

bool rowwalk_fits(const Geo &g, int dtype, int pass) {
    if (!rowwalk_applicable(g, pass)) return false;
    const int ve = dtype == 0 ? 4 : 8;
    // strip-defining width: output rows (forward, grad-weight), dx rows (grad-input
    // stride 1) or dy rows (grad-input stride 2)
    const int width = pass == 1 ? (g.sh == 1 ? g.iw : g.ow) : g.ow;
    if (pass == 1 && g.sh == 2) return (width + ve / 2 - 1) / (ve / 2) <= 64 && width >= 28;  // half strips of dy
    if ((width + ve - 1) / ve > 64) return false;
    // narrow rows leave most lanes of a slot idle; the LDS band kernels measure
    // faster there for the forward and grad-input (grad-weight streams always)
    return pass == 2 || width >= 56;
}

namespace {

template <typename T>
bool rw_strip_layout(int width, RwPlan &p) {
    p.NS = strips<T>(width);
    if (p.NS > 64) return false;
    p.SPW = 64 / p.NS;
    return true;
}

template <typename T, int S, int MM, bool BWD>
int launch_conv3(const Geo &g, const void *in, const void *w, const void *b, void *out, hipStream_t st) {
    constexpr int RW = Vec<T>::N;
    RwPlan p;
    const int OW = BWD ? g.iw : g.ow, OH = BWD ? g.ih : g.oh;
    const int IW = BWD ? g.ow : g.iw;
    if (!rw_strip_layout<T>(OW, p)) return kErrUnsupported;
    const int64_t planes = static_cast<int64_t>(g.n) * g.ic;
    p.BH = pick_bh(planes, OH, p.SPW, 4);
    p.nbands = (OH + p.BH - 1) / p.BH;
    p.nunits = static_cast<int>(planes * p.nbands);
    const int per_wg = kWaves * p.SPW;
    p.grid = (p.nunits + per_wg - 1) / per_wg;
    RwArgs<T> a{};
    a.in = static_cast<const T *>(in);
    a.w = static_cast<const T *>(w);
    a.b = static_cast<const T *>(b);
    a.out = static_cast<T *>(out);
    a.g = g;
    a.NS = p.NS;
    a.SPW = p.SPW;
    a.BH = p.BH;
    a.nbands = p.nbands;
    a.nunits = p.nunits;
    a.vin = (IW % RW == 0) && (reinterpret_cast<uintptr_t>(in) % 16 == 0);
    a.vout = (OW % RW == 0) && (reinterpret_cast<uintptr_t>(out) % 16 == 0);
    hipLaunchKernelGGL((rw_conv3_kernel<T, S, MM, BWD>), dim3(p.grid), dim3(kThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, int MM>
int launch_bwdin_s2(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t st) {
    constexpr int RW = Vec<T>::N;
    constexpr int DRW = RW / 2;
    RwPlan p;
    p.NS = (g.ow + DRW - 1) / DRW;  // half strips of dy columns
    if (p.NS > 64) return kErrUnsupported;
    p.SPW = 64 / p.NS;
    // dx must be covered by dy rows/cols: 2*oh >= ih and 2*ow >= iw hold for pad 1, k 3, stride 2
    const int64_t planes = static_cast<int64_t>(g.n) * g.ic;
    p.BH = pick_bh(planes, g.oh, p.SPW, 2);
    p.nbands = (g.oh + p.BH - 1) / p.BH;
    p.nunits = static_cast<int>(planes * p.nbands);
    const int per_wg = kWaves * p.SPW;
    p.grid = (p.nunits + per_wg - 1) / per_wg;
    RwArgs<T> a{};
    a.in = static_cast<const T *>(dy);
    a.w = static_cast<const T *>(w);
    a.out = static_cast<T *>(dx);
    a.g = g;
    a.NS = p.NS;
    a.SPW = p.SPW;
    a.BH = p.BH;
    a.nbands = p.nbands;
    a.nunits = p.nunits;
    a.vin = (g.ow % DRW == 0) && (reinterpret_cast<uintptr_t>(dy) % 8 == 0);
    a.vout = (g.iw % RW == 0) && (reinterpret_cast<uintptr_t>(dx) % 16 == 0);
    hipLaunchKernelGGL((rw_bwdin3_s2_kernel<T, MM>), dim3(p.grid), dim3(kThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T>
bool plan_bwdw(const Geo &g, RwPlan &p) {
    if (!rw_strip_layout<T>(g.ow, p)) return false;
    p.BH = pick_bh(static_cast<int64_t>(g.n) * g.ic, g.oh, p.SPW, 4);
    p.nbands = (g.oh + p.BH - 1) / p.BH;
    p.nunits = g.n * p.nbands;  // per channel
    const int per_round = kWaves * p.SPW;
    const int rounds = (p.nunits + per_round - 1) / per_round;
    // chunks per channel: >= 2048 workgroups when there is enough work
    const int want = std::max(1, (2048 + g.ic - 1) / g.ic);
    const int nc = std::min(rounds, want);
    const int rpc = (rounds + nc - 1) / nc;  // rounds per chunk
    p.upc = rpc * per_round;
    p.NC = (p.nunits + p.upc - 1) / p.upc;
    p.grid = g.ic * p.NC;
    return true;
}

template <typename T, int S, int MM>
int launch_bwdw(const Geo &g, const RwPlan &p, const void *x, const void *dy, void *ws, hipStream_t st) {
    constexpr int RW = Vec<T>::N;
    RwArgs<T> a{};
    a.in = static_cast<const T *>(x);
    a.in2 = static_cast<const T *>(dy);
    a.ws = static_cast<float *>(ws);
    a.g = g;
    a.NS = p.NS;
    a.SPW = p.SPW;
    a.BH = p.BH;
    a.nbands = p.nbands;
    a.nunits = p.nunits;
    a.NC = p.NC;
    a.upc = p.upc;
    a.vin = (g.iw % RW == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0);
    a.vout = (g.ow % RW == 0) && (reinterpret_cast<uintptr_t>(dy) % 16 == 0);
    hipLaunchKernelGGL((rw_bwdw3_kernel<T, S, MM>), dim3(p.grid), dim3(kThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T>
int fwd_t(const Geo &g, const void *x, const void *w, const void *b, void *y, hipStream_t s) {
    if (g.sh == 1) return g.mult == 1 ? launch_conv3<T, 1, 1, false>(g, x, w, b, y, s) : launch_conv3<T, 1, 2, false>(g, x, w, b, y, s);
    return g.mult == 1 ? launch_conv3<T, 2, 1, false>(g, x, w, b, y, s) : launch_conv3<T, 2, 2, false>(g, x, w, b, y, s);
}

template <typename T>
int bwdin_t(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t s) {
    if (g.sh == 1) return g.mult == 1 ? launch_conv3<T, 1, 1, true>(g, dy, w, nullptr, dx, s) : launch_conv3<T, 1, 2, true>(g, dy, w, nullptr, dx, s);
    return g.mult == 1 ? launch_bwdin_s2<T, 1>(g, dy, w, dx, s) : launch_bwdin_s2<T, 2>(g, dy, w, dx, s);
}

template <typename T>
int bwdw_t(const Geo &g, const void *x, const void *dy, void *ws, hipStream_t s) {
    RwPlan p;
    if (!plan_bwdw<T>(g, p)) return kErrUnsupported;
    if (g.sh == 1) return g.mult == 1 ? launch_bwdw<T, 1, 1>(g, p, x, dy, ws, s) : launch_bwdw<T, 1, 2>(g, p, x, dy, ws, s);
    return g.mult == 1 ? launch_bwdw<T, 2, 1>(g, p, x, dy, ws, s) : launch_bwdw<T, 2, 2>(g, p, x, dy, ws, s);
}

}  // namespace

// Row-walk launchers; they return kErrUnsupported when the row is wider than
// 64 strips (the caller then uses the band kernels).
int rowwalk_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return fwd_t<float>(g, x, w, b, y, s);
        case 1: return fwd_t<__half>(g, x, w, b, y, s);
        default: return fwd_t<bf16_t>(g, x, w, b, y, s);
    }
}

int rowwalk_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return bwdin_t<float>(g, dy, w, dx, s);
        case 1: return bwdin_t<__half>(g, dy, w, dx, s);
        default: return bwdin_t<bf16_t>(g, dy, w, dx, s);
    }
}

// Chunks per channel of the row-walk grad-weight (its workspace is [ic][NC][M*10]); 0 if not usable.
int rowwalk_bwd_weight_chunks(const Geo &g, int dtype) {
    RwPlan p;
    const bool ok = dtype == 0 ? plan_bwdw<float>(g, p) : plan_bwdw<__half>(g, p);
    return ok ? p.NC : 0;
}

int rowwalk_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return bwdw_t<float>(g, x, dy, ws, s);
        case 1: return bwdw_t<__half>(g, x, dy, ws, s);
        default: return bwdw_t<bf16_t>(g, x, dy, ws, s);
    }
}

}  // namespace dw
