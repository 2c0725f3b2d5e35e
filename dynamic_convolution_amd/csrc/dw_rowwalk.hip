// dw_rowwalk.hip -- streaming kernels for the 3x3, pad 1, dilation 1 depthwise
// layers (stride 1 and 2) on gfx950: forward, grad-input, grad-weight.
//
// These layers move ~8 bytes per multiply-add group and are bound by HBM
// bandwidth (the MobileNet layer table of PyTorch PR #3057 "Spatial Depthwise
// Convolution on the GPU" is this case).  Instead of staging tiles in LDS
// behind barriers, every lane owns one 16-byte column strip of a plane and
// walks down a band of rows:
//   - each input row segment is read with one 16-byte load (two for a stride-2
//     forward segment) three steps ahead of its use and kept as raw words
//     until it enters the window, so those loads stay in flight across the
//     arithmetic of the rows before it; the raw rows sit in one buffer per
//     row of an unrolled pass of the row loop, indexed at compile time (a
//     buffer copied into another would make the compiler wait for its load);
//     rows outside the plane are read from a clamped row and zeroed on
//     conversion, so the loads need no branch;
//   - the column halo (one element left/right) comes from the neighbouring
//     lanes by shuffle, the row halo from a ring of the last three rows kept
//     in registers and indexed at compile time (the row loop is unrolled by 3);
//   - each output strip is written with one 16-byte store;
//   - no LDS tile and no barrier, so waves stream independently.
// A wave serves one channel (its taps are wave-uniform, in scalar registers)
// and holds 64 / NS slots (NS = strips per row), each slot walking one
// (image, band) unit; all slots of a wave take the same number of steps so the
// shuffles always see every lane active.
#include "dw_internal.hpp"
#include "dw_stream.hpp"

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
    int nunits;     // units (image, band) per channel
    int wpc;        // forward / grad-input: waves per channel
    int NC;         // grad-weight: chunks per channel
    int upc;        // grad-weight: units per chunk
};

// Window of one input row for a strip: win[0] = column c0 - 1 (from the left
// lane), win[1..IRW] = the lane's own segment, and for stride 1 win[IRW+1] =
// column c0 + IRW (from the right lane).
template <int IRW, int S>
__device__ __forceinline__ void make_window(const float (&v)[IRW], int lane, bool has_left, bool has_right,
                                            float (&win)[IRW + (S == 1 ? 2 : 1)]) {
    const float l = lane_left(v[IRW - 1]);
    win[0] = has_left ? l : 0.f;
#pragma unroll
    for (int e = 0; e < IRW; ++e) win[1 + e] = v[e];
    if constexpr (S == 1) {
        const float r = lane_right(v[0]);
        win[IRW + 1] = has_right ? r : 0.f;
    }
}

// Rows are loaded three steps (one unrolled pass of the row loop) ahead of use:
// S input rows and one dy row per step.
constexpr int kAhead = 3;

// ---------------------------------------------------------------- forward / grad-input (stride 1)
// FWD: one input plane x[P] -> MM output planes y[P*MM+m].
// BWD (stride 1 only): MM input planes dy[P*MM+m] -> one output plane dx[P],
// with the kernel flipped (for stride 1, pad 1 the adjoint is the same
// stencil with w[2-i][2-j]).
// Relative input row j (row S*oh0 - 1 + j of the band) lives in window slot
// j % 3; output step t reads rows S*t .. S*t + 2 and brings in the S rows
// S*t + 3 - S .. S*t + 2.
template <typename T, int S, int MM, bool BWD, int VB, bool CS>
__global__ __launch_bounds__(kThreads) void rw_conv3_kernel(RwArgs<T> a) {
    constexpr int RW = Vec<T>::N;
    constexpr int IRW = RW * S;
    constexpr int WW = IRW + (S == 1 ? 2 : 1);
    constexpr int NWI = IRW / kPerWord<T>;  // raw words of an input segment
    constexpr int R = S * kAhead;           // raw rows in flight, buffer S*uu+e at step uu
    constexpr int NIN = BWD ? MM : 1;       // input planes per unit
    constexpr int NOUT = BWD ? 1 : MM;      // output planes per unit
    static_assert(!BWD || S == 1, "stride-2 grad-input has its own kernel");
    const Geo &g = a.g;
    // CS: slots are consecutive channels of one image (taps per lane); else
    // slots are (image, band) units of one channel (taps wave-uniform, in SGPRs)
    const WaveUnit u = CS ? chan_unit(a.wpc, a.NS, a.SPW, g.ic, g.n)
                          : wave_unit(a.wpc, a.NS, a.SPW, a.nunits, a.nbands, g.ic);
    float wt[MM][9];
    float bias[NOUT];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            const float v = to_f32(a.w[(u.ic * MM + m) * 9 + (BWD ? 8 - t : t)]);
            wt[m][t] = CS ? v : uniform(v);
        }
#pragma unroll
    for (int o = 0; o < NOUT; ++o) {
        const float v = (!BWD && a.b) ? to_f32(a.b[u.ic * MM + o]) : 0.f;
        bias[o] = CS ? v : uniform(v);
    }

    const int P = u.n * g.ic + u.ic;  // plane (n, ic)
    const int IH = BWD ? g.oh : g.ih, IW = BWD ? g.ow : g.iw;  // rows/cols of the input planes
    const int OH = BWD ? g.ih : g.oh, OW = BWD ? g.iw : g.ow;
    const int c_in = u.s * IRW, c_out = u.s * RW;
    const int nin = VB == 16 ? IRW : IW - c_in;  // valid columns of the lane's input segment
    const bool hl = u.s > 0, hr = u.s < a.NS - 1;
    const int64_t in_plane = static_cast<int64_t>(IH) * IW;
    const T *inp[NIN];
#pragma unroll
    for (int k = 0; k < NIN; ++k) inp[k] = a.in + (static_cast<int64_t>(P) * NIN + k) * in_plane;
    const int oh0 = u.band * a.BH;
    const int oh_end = min(oh0 + a.BH, OH);
    const int rb = S * oh0 - 1;             // input row of relative row 0
    const int jlast = S * (a.BH - 1) + 2;   // last relative row any step reads

    float win[NIN][3][WW];
    uint32_t rq[NIN][R][NWI];
    bool rk[NIN][R];
#pragma unroll
    for (int k = 0; k < NIN; ++k) {
#pragma unroll
        for (int j = 0; j < 3 - S; ++j) {
            uint32_t w[NWI];
            bool ok;
            float v[IRW];
            load_row<T, NWI, VB>(inp[k], rb + j, IH, IW, c_in, u.act, w, ok);
            row_values<T>(w, ok, nin, v);
            make_window<IRW, S>(v, u.lane, hl, hr, win[k][j]);
        }
    }
    // first refills in the loop's own order (step, input plane, row), so the
    // wait counts at the loop's head are the same on entry as around the loop
#pragma unroll
    for (int uu = 0; uu < 3; ++uu) {
#pragma unroll
        for (int k = 0; k < NIN; ++k)
#pragma unroll
            for (int e = 0; e < S; ++e) {
                const int f = S * uu + e;
                load_row<T, NWI, VB>(inp[k], rb + 3 - S + f, IH, IW, c_in, u.act, rq[k][f], rk[k][f]);
            }
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int t0 = 0; t0 < a.BH; t0 += 3) {  // BH is a multiple of 3
#pragma unroll
        for (int uu = 0; uu < 3; ++uu) {
            const int t = t0 + uu;
            {
#pragma unroll
                for (int k = 0; k < NIN; ++k)
#pragma unroll
                    for (int e = 0; e < S; ++e) {
                        float v[IRW];
                        const int f = S * uu + e;
                        uint32_t cw[NWI];
                        take_words<T>(rq[k][f], cw);
                        row_values<T>(cw, rk[k][f], nin, v);
                        make_window<IRW, S>(v, u.lane, hl, hr, win[k][(S * uu + 3 - S + e) % 3]);
                        // refill with relative row S*t + 3 - S + e + R; past the last row a
                        // step reads, re-read that row (a cache hit, never used) so the
                        // load stays unconditional
                        const int jn = min(S * t + 3 - S + e + R, jlast);
                        load_row<T, NWI, VB>(inp[k], rb + jn, IH, IW, c_in, u.act, rq[k][f], rk[k][f]);
                    }
                __builtin_amdgcn_sched_barrier(0);
                const int oh = oh0 + t;
                if (u.act && oh < oh_end) {
#pragma unroll
                    for (int o = 0; o < NOUT; ++o) {
                        float acc[RW];
#pragma unroll
                        for (int q = 0; q < RW; ++q) acc[q] = bias[o];
#pragma unroll
                        for (int k = 0; k < NIN; ++k) {
                            const float *wk = wt[BWD ? k : o];
#pragma unroll
                            for (int i = 0; i < 3; ++i)
#pragma unroll
                                for (int j = 0; j < 3; ++j)
#pragma unroll
                                    for (int q = 0; q < RW; ++q)
                                        acc[q] = fmaf(wk[3 * i + j], win[k][(S * uu + i) % 3][q * S + j], acc[q]);
                        }
                        T *op = a.out + ((static_cast<int64_t>(P) * NOUT + o) * OH + oh) * OW + c_out;
                        store_values<T, RW, VB>(op, acc, OW - c_out);
                    }
                }
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
template <typename T, int MM, int VB, bool CS>
__global__ __launch_bounds__(kThreads) void rw_bwdin3_s2_kernel(RwArgs<T> a) {
    constexpr int RW = Vec<T>::N;
    constexpr int DRW = RW / 2;
    constexpr int ND = DRW / kPerWord<T>;  // raw words of a half strip (8 bytes)
    constexpr int R = 3;                   // dy rows in flight
    constexpr int VD = VB < 8 ? VB : 8;    // vector bytes of the dy loads
    const Geo &g = a.g;
    const WaveUnit u = CS ? chan_unit(a.wpc, a.NS, a.SPW, g.ic, g.n)
                          : wave_unit(a.wpc, a.NS, a.SPW, a.nunits, a.nbands, g.ic);
    const int c0 = u.s * DRW;
    const int nd = VB == 16 ? DRW : g.ow - c0;  // valid dy columns of the half strip
    const bool has_right = u.s < a.NS - 1;
    float wt[MM][9];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t < 9; ++t) {
            const float v = to_f32(a.w[(u.ic * MM + m) * 9 + t]);
            wt[m][t] = CS ? v : uniform(v);
        }
    const int P = u.n * g.ic + u.ic;
    const int64_t dplane = static_cast<int64_t>(g.oh) * g.ow;
    const T *dp[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) dp[m] = a.in + (static_cast<int64_t>(P) * MM + m) * dplane;
    const int r0 = u.band * a.BH;
    const int rlast = r0 + a.BH;  // last dy row any step reads (later refills re-read it)
    // dy row r (cur) and r+1 (nxt), each with the right neighbour column
    float cur[MM][DRW + 1], nxt[MM][DRW + 1];
    uint32_t rq[MM][R][ND];
    bool rk[MM][R];
#pragma unroll
    for (int m = 0; m < MM; ++m) {
        uint32_t w[ND];
        bool ok;
        float v[DRW];
        load_row<T, ND, VD>(dp[m], r0, g.oh, g.ow, c0, u.act, w, ok);
        row_values<T>(w, ok, nd, v);
        const float rr = lane_right(v[0]);
#pragma unroll
        for (int e = 0; e < DRW; ++e) cur[m][e] = v[e];
        cur[m][DRW] = has_right ? rr : 0.f;
#pragma unroll
        for (int f = 0; f < R; ++f) load_row<T, ND, VD>(dp[m], r0 + 1 + f, g.oh, g.ow, c0, u.act, rq[m][f], rk[m][f]);
    }
    for (int step = 0; step < a.BH; ++step) {
        const int r = r0 + step;
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            float v[DRW];
            row_values<T>(rq[m][0], rk[m][0], nd, v);
            ring_pop<R, ND>(rq[m], rk[m]);
            load_row<T, ND, VD>(dp[m], min(r + 1 + R, rlast), g.oh, g.ow, c0, u.act, rq[m][R - 1], rk[m][R - 1]);
            const float rr = lane_right(v[0]);
#pragma unroll
            for (int e = 0; e < DRW; ++e) nxt[m][e] = v[e];
            nxt[m][DRW] = has_right ? rr : 0.f;
        }
        if (u.act && 2 * r < g.ih) {
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
            // dx is four times dy: streaming stores keep L2 for the dy rows
            store_values<T, RW, VB, true>(xp, e0, valid);
            if (2 * r + 1 < g.ih) store_values<T, RW, VB, true>(xp + g.iw, e1, valid);
        }
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int e = 0; e <= DRW; ++e) cur[m][e] = nxt[m][e];
    }
}

// ---------------------------------------------------------------- grad-weight
// Workgroup (ic, chunk): its lanes walk units (n, band) of input channel ic,
// accumulating for each of the MM output channels the 9 taps and the bias sum;
// one fixed-order workgroup reduction writes the chunk's partials.  The x rows
// move through the same window ring as the forward; dy rows are loaded ahead
// as raw words too.
template <typename T, int S, int MM, int VB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu((sizeof(T) == 4 && S == 1 && MM == 1 && VB == 16) ? 6 : 1))) void rw_bwdw3_kernel(RwArgs<T> a) {
    constexpr int RW = Vec<T>::N;
    constexpr int IRW = RW * S;
    constexpr int WW = IRW + (S == 1 ? 2 : 1);
    constexpr int NWI = IRW / kPerWord<T>;
    constexpr int NWO = RW / kPerWord<T>;
    constexpr int R = S * kAhead;  // x rows in flight, buffer S*uu+e at step uu
    constexpr int RD = kAhead;     // dy rows in flight, buffer uu at step uu
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
    const int nin = VB == 16 ? IRW : g.iw - c_in;   // valid columns of the x segment
    const int nout = VB == 16 ? RW : g.ow - c_out;  // valid columns of the dy strip
    const bool hl = s > 0;
    const bool hr = s < a.NS - 1;
    const int64_t xplane = static_cast<int64_t>(g.ih) * g.iw;
    const int64_t dplane = static_cast<int64_t>(g.oh) * g.ow;
    const int jlast = S * (a.BH - 1) + 2;

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
        const int rb = S * oh0 - 1;
        float win[3][WW];
        uint32_t rq[R][NWI], gq[MM][RD][NWO];
        bool rk[R], gk[MM][RD];
#pragma unroll
        for (int j = 0; j < 3 - S; ++j) {
            uint32_t w[NWI];
            bool ok;
            float v[IRW];
            load_row<T, NWI, VB>(xp, rb + j, g.ih, g.iw, c_in, act, w, ok);
            row_values<T>(w, ok, nin, v);
            make_window<IRW, S>(v, lane, hl, hr, win[j]);
        }
        // first loads in the loop's own order (step: x rows, then dy rows), so
        // the wait counts at the loop's head are the same on entry as around it
#pragma unroll
        for (int uu = 0; uu < 3; ++uu) {
#pragma unroll
            for (int e = 0; e < S; ++e)
                load_row<T, NWI, VB>(xp, rb + 3 - S + S * uu + e, g.ih, g.iw, c_in, act, rq[S * uu + e],
                                     rk[S * uu + e]);
#pragma unroll
            for (int m = 0; m < MM; ++m)
                load_row<T, NWO, VB>(dyp + m * dplane, oh0 + uu, oh_end, g.ow, c_out, act, gq[m][uu], gk[m][uu]);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int t0 = 0; t0 < a.BH; t0 += 3) {  // BH is a multiple of 3
#pragma unroll
            for (int uu = 0; uu < 3; ++uu) {
                const int t = t0 + uu;
                {
#pragma unroll
                    for (int e = 0; e < S; ++e) {
                        float v[IRW];
                        const int f = S * uu + e;
                        uint32_t cw[NWI];
                        take_words<T>(rq[f], cw);
                        row_values<T>(cw, rk[f], nin, v);
                        make_window<IRW, S>(v, lane, hl, hr, win[(S * uu + 3 - S + e) % 3]);
                        const int jn = min(S * t + 3 - S + e + R, jlast);
                        load_row<T, NWI, VB>(xp, rb + jn, g.ih, g.iw, c_in, act, rq[f], rk[f]);
                    }
                    float gy[MM][RW];
#pragma unroll
                    for (int m = 0; m < MM; ++m) {
                        uint32_t cw[NWO];
                        take_words<T>(gq[m][uu], cw);
                        row_values<T>(cw, gk[m][uu], nout, gy[m]);
                        load_row<T, NWO, VB>(dyp + m * dplane, oh0 + min(t + RD, a.BH - 1), oh_end, g.ow, c_out, act,
                                               gq[m][uu], gk[m][uu]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int m = 0; m < MM; ++m)
#pragma unroll
                        for (int q = 0; q < RW; ++q) {
                            acc[m][9] += gy[m][q];
#pragma unroll
                            for (int i = 0; i < 3; ++i)
#pragma unroll
                                for (int j = 0; j < 3; ++j)
                                    acc[m][3 * i + j] =
                                        fmaf(gy[m][q], win[(S * uu + i) % 3][q * S + j], acc[m][3 * i + j]);
                        }
                }
            }
        }
    }
    {
        float flat[A];
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int t = 0; t < 10; ++t) flat[m * 10 + t] = acc[m][t];
        const float v = wave_transpose_sum<A>(flat, lane);
        if (lane < A) red[wave][lane] = v;
    }
    __syncthreads();
    if (threadIdx.x < A) {
        float v = red[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) v += red[w][threadIdx.x];
        a.ws[(static_cast<int64_t>(ic) * a.NC + chunk) * A + threadIdx.x] = v;
    }
}

// Grad-weight for small planes with channel slots: workgroup (channel group,
// image chunk); each of its waves walks whole planes of one image at a time
// (images chunk*upc + wave, + 4, ...), its slots on SPW consecutive channels,
// so each lane accumulates the taps of its own channel.  The partials of a
// channel's NS strips and 4 waves are summed in a fixed order through LDS.
template <typename T, int S, int MM, int VB>
__global__ __launch_bounds__(kThreads) void rw_bwdw3_cs_kernel(RwArgs<T> a) {
    constexpr int RW = Vec<T>::N;
    constexpr int IRW = RW * S;
    constexpr int WW = IRW + (S == 1 ? 2 : 1);
    constexpr int NWI = IRW / kPerWord<T>;
    constexpr int NWO = RW / kPerWord<T>;
    constexpr int R = S * kAhead;
    constexpr int RD = kAhead;
    constexpr int A = MM * 10;
    __shared__ float red[kWaves][64][A + 1];
    const Geo &g = a.g;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slot = lane / a.NS;
    const int s = lane - slot * a.NS;
    const int cg = blockIdx.x / a.NC;
    const int chunk = blockIdx.x - cg * a.NC;
    const int c = cg * a.SPW + slot;
    const bool act = slot < a.SPW && c < g.ic;
    const int cc = act ? c : 0;
    const int c_in = s * IRW;
    const int c_out = s * RW;
    const int nin = VB == 16 ? IRW : g.iw - c_in;
    const int nout = VB == 16 ? RW : g.ow - c_out;
    const bool hl = s > 0;
    const bool hr = s < a.NS - 1;
    const int64_t xplane = static_cast<int64_t>(g.ih) * g.iw;
    const int64_t dplane = static_cast<int64_t>(g.oh) * g.ow;
    const int jlast = S * (a.BH - 1) + 2;

    float acc[MM][10];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t < 10; ++t) acc[m][t] = 0.f;

    const int n_end = min((chunk + 1) * a.upc, g.n);
    for (int n = chunk * a.upc + wave; n < n_end; n += kWaves) {
        const T *xp = a.in + (static_cast<int64_t>(n) * g.ic + cc) * xplane;
        const T *dyp = a.in2 + (static_cast<int64_t>(n) * g.oc + cc * MM) * dplane;
        const int rb = -1;
        float win[3][WW];
        uint32_t rq[R][NWI], gq[MM][RD][NWO];
        bool rk[R], gk[MM][RD];
#pragma unroll
        for (int j = 0; j < 3 - S; ++j) {
            uint32_t w[NWI];
            bool ok;
            float v[IRW];
            load_row<T, NWI, VB>(xp, rb + j, g.ih, g.iw, c_in, act, w, ok);
            row_values<T>(w, ok, nin, v);
            make_window<IRW, S>(v, lane, hl, hr, win[j]);
        }
        // first loads in the loop's own order (as in rw_bwdw3_kernel)
#pragma unroll
        for (int uu = 0; uu < 3; ++uu) {
#pragma unroll
            for (int e = 0; e < S; ++e)
                load_row<T, NWI, VB>(xp, rb + 3 - S + S * uu + e, g.ih, g.iw, c_in, act, rq[S * uu + e],
                                     rk[S * uu + e]);
#pragma unroll
            for (int m = 0; m < MM; ++m)
                load_row<T, NWO, VB>(dyp + m * dplane, uu, g.oh, g.ow, c_out, act, gq[m][uu], gk[m][uu]);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int t0 = 0; t0 < a.BH; t0 += 3) {  // BH is a multiple of 3
#pragma unroll
            for (int uu = 0; uu < 3; ++uu) {
                const int t = t0 + uu;
#pragma unroll
                for (int e = 0; e < S; ++e) {
                    float v[IRW];
                    const int f = S * uu + e;
                    uint32_t cw[NWI];
                    take_words<T>(rq[f], cw);
                    row_values<T>(cw, rk[f], nin, v);
                    make_window<IRW, S>(v, lane, hl, hr, win[(S * uu + 3 - S + e) % 3]);
                    const int jn = min(S * t + 3 - S + e + R, jlast);
                    load_row<T, NWI, VB>(xp, rb + jn, g.ih, g.iw, c_in, act, rq[f], rk[f]);
                }
                float gy[MM][RW];
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    uint32_t cw[NWO];
                    take_words<T>(gq[m][uu], cw);
                    row_values<T>(cw, gk[m][uu], nout, gy[m]);
                    load_row<T, NWO, VB>(dyp + m * dplane, min(t + RD, a.BH - 1), g.oh, g.ow, c_out, act, gq[m][uu],
                                         gk[m][uu]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < MM; ++m)
#pragma unroll
                    for (int q = 0; q < RW; ++q) {
                        acc[m][9] += gy[m][q];
#pragma unroll
                        for (int i = 0; i < 3; ++i)
#pragma unroll
                            for (int j = 0; j < 3; ++j)
                                acc[m][3 * i + j] = fmaf(gy[m][q], win[(S * uu + i) % 3][q * S + j], acc[m][3 * i + j]);
                    }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t < 10; ++t) red[wave][lane][m * 10 + t] = acc[m][t];
    __syncthreads();
    for (int e = threadIdx.x; e < a.SPW * A; e += kThreads) {
        const int j = e / A;
        const int k = e - j * A;
        const int cj = cg * a.SPW + j;
        if (cj < g.ic) {
            float v = 0.f;
            for (int w = 0; w < kWaves; ++w)
                for (int q = 0; q < a.NS; ++q) v += red[w][j * a.NS + q][k];
            a.ws[(static_cast<int64_t>(cj) * a.NC + chunk) * A + k] = v;
        }
    }
}

// ---------------------------------------------------------------- planning
struct RwPlan {
    int NS, SPW, BH, nbands, nunits, wpc, grid, NC, upc;
    bool cs;  // channel slots (small planes)
};

// Planes of at most this many outputs are walked with channel slots: the
// slots of a wave then read one contiguous run of planes instead of one row of
// each of 64/NS planes that lie a whole image apart.
constexpr int64_t kCsMaxOut = 1024;

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
    if (pass == 1 && g.sh == 2) return (width + ve / 2 - 1) / (ve / 2) <= 64 && width >= 14;  // half strips of dy
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

// Channel-uniform waves over units (image, band): wpc waves per channel.
// Bands of BH rows, BH rounded up to a multiple of `step` (the row loop's
// unroll factor: steps past the band's last row compute nothing that is stored).
inline bool finish_plan(const Geo &g, RwPlan &p, int rows, int min_bh, int step) {
    const int64_t planes = static_cast<int64_t>(g.n) * g.ic;
    p.BH = (pick_bh(planes, rows, p.SPW, min_bh) + step - 1) / step * step;
    p.nbands = (rows + p.BH - 1) / p.BH;
    p.nunits = g.n * p.nbands;
    p.wpc = (p.nunits + p.SPW - 1) / p.SPW;
    const int64_t waves = static_cast<int64_t>(g.ic) * p.wpc;
    if (waves > (int64_t{1} << 30)) return false;
    p.grid = static_cast<int>((waves + kWaves - 1) / kWaves);
    return true;
}

// Channel-slot plan: one wave per (image, group of SPW channels), whole planes
// of `rows` rows, rounded up to a multiple of `step`.
inline bool cs_plan(const Geo &g, RwPlan &p, int rows, int step) {
    p.cs = true;
    p.BH = (rows + step - 1) / step * step;
    p.nbands = 1;
    p.nunits = 0;
    p.wpc = (g.ic + p.SPW - 1) / p.SPW;
    const int64_t waves = static_cast<int64_t>(g.n) * p.wpc;
    if (waves > (int64_t{1} << 30)) return false;
    p.grid = static_cast<int>((waves + kWaves - 1) / kWaves);
    return true;
}

template <typename T>
RwArgs<T> rw_args(const Geo &g, const RwPlan &p) {
    RwArgs<T> a{};
    a.g = g;
    a.NS = p.NS;
    a.SPW = p.SPW;
    a.BH = p.BH;
    a.nbands = p.nbands;
    a.nunits = p.nunits;
    a.wpc = p.wpc;
    a.NC = p.NC;
    a.upc = p.upc;
    return a;
}

template <typename T, int S, int MM, bool BWD>
int launch_conv3(const Geo &g, const void *in, const void *w, const void *b, void *out, hipStream_t st) {
    RwPlan p{};
    const int OW = BWD ? g.iw : g.ow, OH = BWD ? g.ih : g.oh;
    const int IW = BWD ? g.ow : g.iw;
    if (!rw_strip_layout<T>(OW, p)) return kErrUnsupported;
    if (static_cast<int64_t>(OH) * OW <= kCsMaxOut ? !cs_plan(g, p, OH, 3) : !finish_plan(g, p, OH, 4, 3))
        return kErrUnsupported;
    RwArgs<T> a = rw_args<T>(g, p);
    a.in = static_cast<const T *>(in);
    a.w = static_cast<const T *>(w);
    a.b = static_cast<const T *>(b);
    a.out = static_cast<T *>(out);
    // vector width of the row accesses: 16 bytes means every strip [c_out, c_out+RW)
    // and segment [S*c_out, S*(c_out+RW)) lies inside its row
    const int vb = row_vector_bytes<T>({IW, OW}, {in, out});
    return with_vector_bytes<T>(vb, [&](auto V) {
        if (p.cs)
            hipLaunchKernelGGL((rw_conv3_kernel<T, S, MM, BWD, decltype(V)::value, true>), dim3(p.grid), dim3(kThreads),
                               0, st, a);
        else
            hipLaunchKernelGGL((rw_conv3_kernel<T, S, MM, BWD, decltype(V)::value, false>), dim3(p.grid), dim3(kThreads),
                               0, st, a);
        return hipGetLastError() == hipSuccess ? kOk : kErrHip;
    });
}

template <typename T, int MM>
int launch_bwdin_s2(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t st) {
    constexpr int RW = Vec<T>::N;
    constexpr int DRW = RW / 2;
    RwPlan p{};
    p.NS = (g.ow + DRW - 1) / DRW;  // half strips of dy columns
    if (p.NS > 64) return kErrUnsupported;
    p.SPW = 64 / p.NS;
    // dx must be covered by dy rows/cols: 2*oh >= ih and 2*ow >= iw hold for pad 1, k 3, stride 2
    if (static_cast<int64_t>(g.ih) * g.iw <= kCsMaxOut ? !cs_plan(g, p, g.oh, 1) : !finish_plan(g, p, g.oh, 2, 1))
        return kErrUnsupported;
    RwArgs<T> a = rw_args<T>(g, p);
    a.in = static_cast<const T *>(dy);
    a.w = static_cast<const T *>(w);
    a.out = static_cast<T *>(dx);
    // vector width of the row accesses (dy loads use at most 8 bytes, a half strip)
    const int vb = row_vector_bytes<T>({g.ow, g.iw}, {dy, dx});
    return with_vector_bytes<T>(vb, [&](auto V) {
        if (p.cs)
            hipLaunchKernelGGL((rw_bwdin3_s2_kernel<T, MM, decltype(V)::value, true>), dim3(p.grid), dim3(kThreads), 0, st, a);
        else
            hipLaunchKernelGGL((rw_bwdin3_s2_kernel<T, MM, decltype(V)::value, false>), dim3(p.grid), dim3(kThreads), 0, st,
                               a);
        return hipGetLastError() == hipSuccess ? kOk : kErrHip;
    });
}

template <typename T>
bool plan_bwdw(const Geo &g, RwPlan &p) {
    if (!rw_strip_layout<T>(g.ow, p)) return false;
    if (static_cast<int64_t>(g.oh) * g.ow <= kCsMaxOut) {
        // channel slots: workgroup (channel group, chunk of upc images), one image per wave at a time
        p.cs = true;
        p.BH = (g.oh + 2) / 3 * 3;
        p.nbands = 1;
        p.nunits = 0;
        p.wpc = (g.ic + p.SPW - 1) / p.SPW;
        p.upc = kWaves;
        while (p.upc < g.n && static_cast<int64_t>(p.wpc) * ((g.n + 2 * p.upc - 1) / (2 * p.upc)) >= 1024) p.upc *= 2;
        p.NC = (g.n + p.upc - 1) / p.upc;
        const int64_t grid = static_cast<int64_t>(p.wpc) * p.NC;
        if (grid > (int64_t{1} << 30)) return false;
        p.grid = static_cast<int>(grid);
        return true;
    }
    p.cs = false;
    p.BH = (pick_bh(static_cast<int64_t>(g.n) * g.ic, g.oh, p.SPW, 4) + 2) / 3 * 3;  // unroll factor 3
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
    RwArgs<T> a = rw_args<T>(g, p);
    a.in = static_cast<const T *>(x);
    a.in2 = static_cast<const T *>(dy);
    a.ws = static_cast<float *>(ws);
    const int vb = row_vector_bytes<T>({g.iw, g.ow}, {x, dy});
    return with_vector_bytes<T>(vb, [&](auto V) {
        if (p.cs)
            hipLaunchKernelGGL((rw_bwdw3_cs_kernel<T, S, MM, decltype(V)::value>), dim3(p.grid), dim3(kThreads), 0, st, a);
        else
            hipLaunchKernelGGL((rw_bwdw3_kernel<T, S, MM, decltype(V)::value>), dim3(p.grid), dim3(kThreads), 0, st, a);
        return hipGetLastError() == hipSuccess ? kOk : kErrHip;
    });
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
