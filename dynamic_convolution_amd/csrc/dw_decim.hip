// dw_decim.hip -- depthwise passes with stride 2, dilation 2 and pad k-1
// (k = 3, 5; multiplier 1 or 2) on gfx950.
//
// With stride s = 2, dilation d = 2 and pad p = k - 1 every tap of every output
// reads an input element at an even row and an even column:
//   x[2*oh - p + 2*i][2*ow - p + 2*j] = xe[oh - h + i][ow - h + j],   h = (k-1)/2,
// where xe[r][c] = x[2r][2c] is the decimated input.  So all three passes are
// stride-1, dilation-1 "same" convolutions on the decimated grid (this is the
// multiplier-2 / dilation-2 / stride-2 layer of PyTorch PR #3057's feature set):
//   forward      y = sum_ij w[i][j] xe[oh-h+i][ow-h+j]  -- only even x rows are read;
//   grad-input   dx[2r][2c] = sum_m sum_ij w_m[i][j] dy_m[r+h-i][c+h-j], and every
//                other dx element is a structural zero (75 % of dx), written as such;
//   grad-weight  dw_m[i][j] = sum dy_m[oh][ow] xe[oh-h+i][ow-h+j].
//
// Each lane owns RO = 4 decimated columns of a plane and walks a band of rows:
// the lane's x segment [2c0, 2c0+8) is one 16-byte load (two for fp32) whose
// even elements are kept, the column halo of h values on each side comes from
// the neighbouring lanes by shuffle, and the k rows of the window stay in
// registers as a ring indexed at compile time (the row loop is unrolled by k).
// Rows are loaded k rows ahead and kept as raw 32-bit words until they enter
// the window, in k buffers indexed by the row's step modulo k (a compile-time
// index in the row loop unrolled by k, so no buffer is ever copied to another:
// a copy would make the compiler wait for that buffer's load and leave one
// load in flight); those loads stay in flight across the arithmetic of the
// rows before them.  Rows outside the plane are read from a clamped address
// and replaced by zeros on conversion, which keeps the loads branch-free.
// Forward and grad-input waves each serve one channel (several images or row
// bands of it), so the filter taps are wave-uniform and live in scalar registers.
#include "dw_internal.hpp"
#include "dw_stream.hpp"

namespace dw {
namespace {

constexpr int kWaves = kThreads / 64;
constexpr int RO = 4;  // decimated columns per lane

// 32-bit words of a lane's x segment (2*RO elements) and of a dy / y strip (RO elements).
template <typename T> constexpr int kXWords = 2 * RO * static_cast<int>(sizeof(T)) / 4;
template <typename T> constexpr int kDWords = RO * static_cast<int>(sizeof(T)) / 4;

// Raw x segment of decimated row r (x row 2r, columns [2c0, 2c0 + 2*RO)).
template <typename T, bool FULL>
__device__ __forceinline__ void load_xrow(const T *plane, int r, int XH, int IW, int c0, bool act,
                                          uint32_t (&w)[kXWords<T>], bool &ok) {
    ok = act && r >= 0 && r < XH;
    const int rc = min(max(r, 0), XH - 1);
    const T *p = plane + static_cast<int64_t>(2 * rc) * IW + 2 * c0;
    if constexpr (FULL)
        load_words<kXWords<T>>(p, w);
    else
        load_words_tail<T, kXWords<T>>(p, IW - 2 * c0, w);
}

// Raw strip [c0, c0 + RO) of row r of a plane of H rows and W columns.
template <typename T, bool FULL>
__device__ __forceinline__ void load_drow(const T *plane, int r, int H, int W, int c0, bool act,
                                          uint32_t (&w)[kDWords<T>], bool &ok) {
    ok = act && r >= 0 && r < H;
    const int rc = min(max(r, 0), H - 1);
    const T *p = plane + static_cast<int64_t>(rc) * W + c0;
    if constexpr (FULL)
        load_words<kDWords<T>>(p, w);
    else
        load_words_tail<T, kDWords<T>>(p, W - c0, w);
}

// win[0..H) = the left lane's last H values, win[H..H+RO) = own, then the right lane's first H.
template <int HH>
__device__ __forceinline__ void halo_window(const float (&v)[RO], int lane, bool has_left, bool has_right,
                                            float (&win)[RO + 2 * HH]) {
#pragma unroll
    for (int e = 0; e < HH; ++e) {
        const float l = lane_left(v[RO - HH + e]);
        win[e] = has_left ? l : 0.f;
        const float r = lane_right(v[e]);
        win[HH + RO + e] = has_right ? r : 0.f;
    }
#pragma unroll
    for (int e = 0; e < RO; ++e) win[HH + e] = v[e];
}

// Window row from a raw x segment: its even elements, zero when the row is outside the plane.
template <typename T, int HH>
__device__ __forceinline__ void xrow_window(const uint32_t (&w)[kXWords<T>], bool ok, int lane, bool hl, bool hr,
                                            float (&row)[RO + 2 * HH]) {
    float v[RO];
#pragma unroll
    for (int e = 0; e < RO; ++e) v[e] = ok ? word_elem<T>(w, 2 * e) : 0.f;
    halo_window<HH>(v, lane, hl, hr, row);
}

template <typename T>
__device__ __forceinline__ void drow_values(const uint32_t (&w)[kDWords<T>], bool ok, float (&v)[RO]) {
#pragma unroll
    for (int e = 0; e < RO; ++e) v[e] = ok ? word_elem<T>(w, e) : 0.f;
}

template <typename T> struct DcArgs {
    const T *in;
    const T *in2;   // grad-weight: dy
    const T *w;
    const T *b;
    T *out;
    float *ws;
    Geo g;
    int XH, XW;     // decimated input plane: ceil(ih/2) x ceil(iw/2)
    int NS, SPW, BH, nbands;
    int wpc;        // forward / grad-input: waves per channel
    int nunits;     // units (image, band) per channel
    int NC, upc;    // grad-weight chunking
};

// ---------------------------------------------------------------- forward
template <typename T, int K, int MM, bool FULL>
__global__ __launch_bounds__(kThreads) void dec_fwd_kernel(DcArgs<T> a) {
    constexpr int HH = (K - 1) / 2, WW = RO + 2 * HH, NX = kXWords<T>, ND = kDWords<T>;
    const Geo &g = a.g;
    const WaveUnit u = wave_unit(a.wpc, a.NS, a.SPW, a.nunits, a.nbands, g.ic);
    float wt[MM][K * K], bias[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) {
#pragma unroll
        for (int t = 0; t < K * K; ++t) wt[m][t] = uniform(to_f32(a.w[(u.ic * MM + m) * K * K + t]));
        bias[m] = a.b ? uniform(to_f32(a.b[u.ic * MM + m])) : 0.f;
    }
    const int P = u.n * g.ic + u.ic;  // input plane (n, ic)
    const T *xp = a.in + static_cast<int64_t>(P) * g.ih * g.iw;
    const int c0 = u.s * RO;
    const bool hl = u.s > 0, hr = u.s < a.NS - 1;
    const int oh0 = u.band * a.BH, oh_end = min(oh0 + a.BH, g.oh);
    // relative row j (absolute decimated row oh0 - HH + j) lives in window slot j % K
    float win[K][WW];
    // rq[f]: raw relative row K-1+f, +K per pass of the row loop (it enters the
    // window at step f of the pass)
    uint32_t rq[K][NX];
    bool rk[K];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
        uint32_t w[NX];
        bool ok;
        load_xrow<T, FULL>(xp, oh0 - HH + j, a.XH, g.iw, c0, u.act, w, ok);
        xrow_window<T, HH>(w, ok, u.lane, hl, hr, win[j]);
    }
#pragma unroll
    for (int f = 0; f < K; ++f) load_xrow<T, FULL>(xp, oh0 - HH + K - 1 + f, a.XH, g.iw, c0, u.act, rq[f], rk[f]);
    for (int t0 = 0; t0 < a.BH; t0 += K) {  // BH is a multiple of K
        uint32_t ybuf[K][MM][ND];  // packed outputs of this iteration's K rows
#pragma unroll
        for (int uu = 0; uu < K; ++uu) {
            const int t = t0 + uu;
            {
                {
                    uint32_t cw[NX];
                    take_words<T>(rq[uu], cw);
                    xrow_window<T, HH>(cw, rk[uu], u.lane, hl, hr, win[(uu + K - 1) % K]);
                }
                load_xrow<T, FULL>(xp, oh0 - HH + t + 2 * K - 1, a.XH, g.iw, c0, u.act, rq[uu], rk[uu]);
                __builtin_amdgcn_sched_barrier(0);
                const int oh = oh0 + t;
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    float acc[RO];
#pragma unroll
                    for (int q = 0; q < RO; ++q) acc[q] = bias[m];
#pragma unroll
                    for (int i = 0; i < K; ++i)
#pragma unroll
                        for (int j = 0; j < K; ++j)
#pragma unroll
                            for (int q = 0; q < RO; ++q)
                                acc[q] = fmaf(wt[m][i * K + j], win[(uu + i) % K][q + j], acc[q]);
                    if constexpr (FULL) {
                        pack_words<T, ND>(acc, ybuf[uu][m]);
                    } else if (u.act && oh < oh_end) {
                        T *yp = a.out + ((static_cast<int64_t>(P) * MM + m) * g.oh + oh) * g.ow + c0;
#pragma unroll
                        for (int q = 0; q < RO; ++q)
                            if (q < g.ow - c0) yp[q] = from_f32<T>(acc[q]);
                    }
                }
            }
        }
        if constexpr (FULL) {
            // the K rows of this iteration back to back: a slot's rows are adjacent
            // in memory, so each cache line is completed by one burst of stores
            // (rows written one step apart were evicted half-written and cost
            // extra HBM writes and read-modify-writes)
#pragma unroll
            for (int m = 0; m < MM; ++m)
#pragma unroll
                for (int uu = 0; uu < K; ++uu) {
                    const int oh = oh0 + t0 + uu;
                    if (u.act && oh < oh_end)
                        store_words<ND>(a.out + ((static_cast<int64_t>(P) * MM + m) * g.oh + oh) * g.ow + c0,
                                        ybuf[uu][m]);
                }
        }
    }
}

// ---------------------------------------------------------------- forward, 16-bit pairs
// The forward with 16-bit whole-vector rows: two taps per instruction.  The
// decimated values of a lane's raw x segment are the low halves of its four
// words, so the window is kept as words W[k] (low half = decimated column
// c0 - HH + k) and as pairs P[k] = (W[k].lo, W[k+1].lo) built with one byte
// permute each; each output q then sums, per kernel row i and multiplier m,
// the dot products of P[q + 2p] with the tap pairs (w[i][2p], w[i][2p+1])
// (the last pair of an odd k is (w[i][k-1], 0)).  v_dot2c_f32_{bf16,f16}
// multiplies the 16-bit values exactly and adds in fp32 (Dot2).
// Pairs of a window row from a raw x segment (zeros outside the plane / image).
template <typename T, int HH>
__device__ __forceinline__ void xrow_pairs(const uint32_t (&w)[kXWords<T>], bool ok, int lane, bool hl, bool hr,
                                           uint32_t (&P)[RO + 2 * HH]) {
    static_assert(kXWords<T> == RO, "16-bit segment: one word per decimated column");
    constexpr int WW = RO + 2 * HH;
    uint32_t W[WW];
    uint32_t v[RO];
#pragma unroll
    for (int e = 0; e < RO; ++e) v[e] = ok ? w[e] : 0u;
#pragma unroll
    for (int e = 0; e < HH; ++e) {
        const uint32_t l = static_cast<uint32_t>(lane_left(static_cast<uint32_t>(v[RO - HH + e])));
        W[e] = hl ? l : 0u;
        const uint32_t r = static_cast<uint32_t>(lane_right(static_cast<uint32_t>(v[e])));
        W[HH + RO + e] = hr ? r : 0u;
    }
#pragma unroll
    for (int e = 0; e < RO; ++e) W[HH + e] = v[e];
#pragma unroll
    for (int k = 0; k + 1 < WW; ++k) P[k] = __builtin_amdgcn_perm(W[k + 1], W[k], 0x05040100u);
    P[WW - 1] = W[WW - 1] & 0xffffu;
}

template <typename T, int K, int MM>
__global__ __launch_bounds__(kThreads) void dec_fwd_dot2_kernel(DcArgs<T> a) {
    constexpr int HH = (K - 1) / 2, WW = RO + 2 * HH, NX = kXWords<T>, ND = kDWords<T>, KP = (K + 1) / 2;
    const Geo &g = a.g;
    const WaveUnit u = wave_unit(a.wpc, a.NS, a.SPW, a.nunits, a.nbands, g.ic);
    // tap pairs (w[i][2p], w[i][2p+1]) as 16-bit pairs, wave-uniform
    uint32_t wp[MM][K][KP];
    float bias[MM];
    const uint16_t *wr = reinterpret_cast<const uint16_t *>(a.w);
#pragma unroll
    for (int m = 0; m < MM; ++m) {
#pragma unroll
        for (int i = 0; i < K; ++i)
#pragma unroll
            for (int p = 0; p < KP; ++p) {
                const int t = (u.ic * MM + m) * K * K + i * K + 2 * p;
                const uint32_t lo = wr[t], hi = 2 * p + 1 < K ? wr[t + 1] : 0u;
                wp[m][i][p] = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lo | (hi << 16))));
            }
        bias[m] = a.b ? uniform(to_f32(a.b[u.ic * MM + m])) : 0.f;
    }
    const int P = u.n * g.ic + u.ic;  // input plane (n, ic)
    const T *xp = a.in + static_cast<int64_t>(P) * g.ih * g.iw;
    const int c0 = u.s * RO;
    const bool hl = u.s > 0, hr = u.s < a.NS - 1;
    const int oh0 = u.band * a.BH, oh_end = min(oh0 + a.BH, g.oh);
    // relative row j (absolute decimated row oh0 - HH + j) lives in window slot j % K
    uint32_t win[K][WW];
    uint32_t rq[K][NX];
    bool rk[K];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
        uint32_t w[NX];
        bool ok;
        load_xrow<T, true>(xp, oh0 - HH + j, a.XH, g.iw, c0, u.act, w, ok);
        xrow_pairs<T, HH>(w, ok, u.lane, hl, hr, win[j]);
    }
#pragma unroll
    for (int f = 0; f < K; ++f) load_xrow<T, true>(xp, oh0 - HH + K - 1 + f, a.XH, g.iw, c0, u.act, rq[f], rk[f]);
    for (int t0 = 0; t0 < a.BH; t0 += K) {  // BH is a multiple of K
        uint32_t ybuf[K][MM][ND];
#pragma unroll
        for (int uu = 0; uu < K; ++uu) {
            const int t = t0 + uu;
            {
                uint32_t cw[NX];
                take_words<T>(rq[uu], cw);
                xrow_pairs<T, HH>(cw, rk[uu], u.lane, hl, hr, win[(uu + K - 1) % K]);
            }
            load_xrow<T, true>(xp, oh0 - HH + t + 2 * K - 1, a.XH, g.iw, c0, u.act, rq[uu], rk[uu]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                float acc[RO];
#pragma unroll
                for (int q = 0; q < RO; ++q) acc[q] = bias[m];
#pragma unroll
                for (int i = 0; i < K; ++i)
#pragma unroll
                    for (int p = 0; p < KP; ++p)
#pragma unroll
                        for (int q = 0; q < RO; ++q)
                            acc[q] = Dot2<T>::run(win[(uu + i) % K][q + 2 * p], wp[m][i][p], acc[q]);
                pack_words<T, ND>(acc, ybuf[uu][m]);
            }
        }
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int uu = 0; uu < K; ++uu) {
                const int oh = oh0 + t0 + uu;
                if (u.act && oh < oh_end)
                    store_words<ND>(a.out + ((static_cast<int64_t>(P) * MM + m) * g.oh + oh) * g.ow + c0, ybuf[uu][m]);
            }
    }
}

// ---------------------------------------------------------------- grad-input
template <typename T, int K, int MM, bool FULL>
__global__ __launch_bounds__(kThreads) void dec_bwdin_kernel(DcArgs<T> a) {
    constexpr int HH = (K - 1) / 2, WW = RO + 2 * HH, ND = kDWords<T>, NX = kXWords<T>;
    const Geo &g = a.g;
    const WaveUnit u = wave_unit(a.wpc, a.NS, a.SPW, a.nunits, a.nbands, g.ic);
    // flipped taps: dxe[r][c] = sum_m sum_ij wf_m[i][j] dy_m[r-h+i][c-h+j]
    float wf[MM][K * K];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int i = 0; i < K; ++i)
#pragma unroll
            for (int j = 0; j < K; ++j)
                wf[m][i * K + j] = uniform(to_f32(a.w[(u.ic * MM + m) * K * K + (K - 1 - i) * K + (K - 1 - j)]));
    const int P = u.n * g.ic + u.ic;  // dx plane (n, ic)
    const int64_t dplane = static_cast<int64_t>(g.oh) * g.ow;
    const T *dp[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) dp[m] = a.in + (static_cast<int64_t>(P) * MM + m) * dplane;
    const int c0 = u.s * RO;  // decimated dx columns [c0, c0+RO) = dy columns of the same index
    const bool hl = u.s > 0, hr = u.s < a.NS - 1;
    const int r0 = u.band * a.BH, r_end = min(r0 + a.BH, a.XH);
    // relative row j (dy row r0 - HH + j) lives in window slot j % K
    float win[MM][K][WW];
#pragma unroll
    for (int m = 0; m < MM; ++m) {
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
            uint32_t w[ND];
            bool ok;
            float v[RO];
            load_drow<T, FULL>(dp[m], r0 - HH + j, g.oh, g.ow, c0, u.act, w, ok);
            drow_values<T>(w, ok, v);
            halo_window<HH>(v, u.lane, hl, hr, win[m][j]);
        }
    }
    // The K new dy rows of an iteration (relative rows t0+K-1 .. t0+2K-2) are
    // loaded as one burst an iteration ahead, into two alternating buffers: a
    // slot's consecutive dy rows share cache lines, and rows read one step
    // apart were evicted and fetched again in between.
    auto load_iter = [&](int jbase, uint32_t (&buf)[MM][K][ND], bool (&ok)[MM][K]) {
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int uu = 0; uu < K; ++uu)
                load_drow<T, FULL>(dp[m], r0 - HH + jbase + uu, g.oh, g.ow, c0, u.act, buf[m][uu], ok[m][uu]);
    };
    auto run_iter = [&](int t0, const uint32_t (&buf)[MM][K][ND], const bool (&ok)[MM][K]) {
#pragma unroll
        for (int uu = 0; uu < K; ++uu) {
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                float v[RO];
                drow_values<T>(buf[m][uu], ok[m][uu], v);
                halo_window<HH>(v, u.lane, hl, hr, win[m][(uu + K - 1) % K]);
            }
            const int r = r0 + t0 + uu;
            if (u.act && r < r_end) {
                float acc[RO];
#pragma unroll
                for (int q = 0; q < RO; ++q) acc[q] = 0.f;
#pragma unroll
                for (int m = 0; m < MM; ++m)
#pragma unroll
                    for (int i = 0; i < K; ++i)
#pragma unroll
                        for (int j = 0; j < K; ++j)
#pragma unroll
                            for (int q = 0; q < RO; ++q)
                                acc[q] = fmaf(wf[m][i * K + j], win[m][(uu + i) % K][q + j], acc[q]);
                // dx row 2r: values at even columns, zeros at odd; dx row 2r+1: zeros
                float e0[2 * RO];
#pragma unroll
                for (int q = 0; q < RO; ++q) {
                    e0[2 * q] = acc[q];
                    e0[2 * q + 1] = 0.f;
                }
                uint32_t we[NX], wz[NX];
                pack_words<T, NX>(e0, we);
#pragma unroll
                for (int k = 0; k < NX; ++k) wz[k] = 0u;
                T *xq = a.out + (static_cast<int64_t>(P) * g.ih + 2 * r) * g.iw + 2 * c0;
                if constexpr (FULL) {
                    store_words<NX>(xq, we);
                    if (2 * r + 1 < g.ih) store_words<NX>(xq + g.iw, wz);
                } else {
                    store_words_tail<T, NX>(xq, g.iw - 2 * c0, we);
                    if (2 * r + 1 < g.ih) store_words_tail<T, NX>(xq + g.iw, g.iw - 2 * c0, wz);
                }
            }
        }
    };
    uint32_t bA[MM][K][ND], bB[MM][K][ND];
    bool kA[MM][K], kB[MM][K];
    load_iter(K - 1, bA, kA);
    for (int t0 = 0; t0 < a.BH; t0 += 2 * K) {  // BH is a multiple of 2K
        load_iter(t0 + 2 * K - 1, bB, kB);
        run_iter(t0, bA, kA);
        load_iter(t0 + 3 * K - 1, bA, kA);
        run_iter(t0 + K, bB, kB);
    }
}

// ---------------------------------------------------------------- grad-weight
template <typename T, int K, int MM, bool FULL>
__global__ __launch_bounds__(kThreads) void dec_bwdw_kernel(DcArgs<T> a) {
    constexpr int HH = (K - 1) / 2, WW = RO + 2 * HH, KK = K * K, A = MM * (KK + 1);
    constexpr int NX = kXWords<T>, ND = kDWords<T>;
    __shared__ float red[kWaves][A];
    const Geo &g = a.g;
    const int ic = blockIdx.x / a.NC;
    const int chunk = blockIdx.x - ic * a.NC;
    float acc[MM][KK + 1];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int t = 0; t <= KK; ++t) acc[m][t] = 0.f;
    const int ubeg = chunk * a.upc, uend = min(ubeg + a.upc, a.nunits);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane / a.NS, s = lane - slot * a.NS;
    const int c0 = s * RO;
    const bool hl = s > 0, hr = s < a.NS - 1;
    const int64_t dplane = static_cast<int64_t>(g.oh) * g.ow;
    for (int base = ubeg; base < uend; base += kWaves * a.SPW) {
        const int unit = base + wave * a.SPW + slot;
        const bool act = slot < a.SPW && unit < uend;
        const int n = act ? unit / a.nbands : 0;
        const int band = act ? unit - n * a.nbands : 0;
        const T *xp = a.in + (static_cast<int64_t>(n) * g.ic + ic) * g.ih * g.iw;
        const T *dyp = a.in2 + (static_cast<int64_t>(n) * g.oc + static_cast<int64_t>(ic) * MM) * dplane;
        const int oh0 = band * a.BH, oh_end = min(oh0 + a.BH, g.oh);
        // relative x row j (decimated row oh0 - HH + j) lives in window slot j % K;
        // dy row oh0 + t is used at step t
        float win[K][WW];
        // rq[f]: raw relative x row K-1+f, +K per K steps (as in the forward)
        uint32_t rq[K][NX];
        bool rk[K];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
            uint32_t w[NX];
            bool ok;
            load_xrow<T, FULL>(xp, oh0 - HH + j, a.XH, g.iw, c0, act, w, ok);
            xrow_window<T, HH>(w, ok, lane, hl, hr, win[j]);
        }
#pragma unroll
        for (int f = 0; f < K; ++f) load_xrow<T, FULL>(xp, oh0 - HH + K - 1 + f, a.XH, g.iw, c0, act, rq[f], rk[f]);
        // dy rows: the K rows of an iteration are loaded as one burst an
        // iteration ahead into two alternating buffers (a slot's consecutive dy
        // rows share cache lines; rows read one step apart were fetched twice)
        auto load_dy = [&](int tbase, uint32_t (&buf)[MM][K][ND], bool (&ok)[MM][K]) {
#pragma unroll
            for (int m = 0; m < MM; ++m)
#pragma unroll
                for (int uu = 0; uu < K; ++uu)
                    load_drow<T, FULL>(dyp + m * dplane, oh0 + tbase + uu, oh_end, g.ow, c0, act, buf[m][uu],
                                       ok[m][uu]);
        };
        auto run_iter = [&](int t0, const uint32_t (&buf)[MM][K][ND], const bool (&ok)[MM][K]) {
#pragma unroll
            for (int uu = 0; uu < K; ++uu) {
                const int t = t0 + uu;
                {
                    uint32_t cw[NX];
                    take_words<T>(rq[uu], cw);
                    xrow_window<T, HH>(cw, rk[uu], lane, hl, hr, win[(uu + K - 1) % K]);
                }
                load_xrow<T, FULL>(xp, oh0 - HH + t + 2 * K - 1, a.XH, g.iw, c0, act, rq[uu], rk[uu]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < MM; ++m) {
                    float gy[RO];
                    drow_values<T>(buf[m][uu], ok[m][uu], gy);
#pragma unroll
                    for (int q = 0; q < RO; ++q) {
                        acc[m][KK] += gy[q];
#pragma unroll
                        for (int i = 0; i < K; ++i)
#pragma unroll
                            for (int j = 0; j < K; ++j)
                                acc[m][i * K + j] = fmaf(gy[q], win[(uu + i) % K][q + j], acc[m][i * K + j]);
                    }
                }
            }
        };
        uint32_t dA[MM][K][ND], dB[MM][K][ND];
        bool kA[MM][K], kB[MM][K];
        load_dy(0, dA, kA);
        for (int t0 = 0; t0 < a.BH; t0 += 2 * K) {  // BH is a multiple of 2K
            load_dy(t0 + K, dB, kB);
            run_iter(t0, dA, kA);
            load_dy(t0 + 2 * K, dA, kA);
            run_iter(t0 + K, dB, kB);
        }
    }
    {
        float flat[A];
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
            for (int t = 0; t <= KK; ++t) flat[m * (KK + 1) + t] = acc[m][t];
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

// ---------------------------------------------------------------- planning
struct DcPlan {
    int NS, SPW, BH, nbands, nunits, wpc, grid, NC, upc;
};

bool plan_dec(const Geo &g, int pass, DcPlan &p) {
    // strips of RO decimated columns over the output width (= decimated width)
    p.NS = (g.ow + RO - 1) / RO;
    if (p.NS > 64) return false;
    p.SPW = 64 / p.NS;
    const int rows = pass == 1 ? (g.ih + 1) / 2 : g.oh;  // rows walked: decimated dx rows or output rows
    const int64_t planes = static_cast<int64_t>(g.n) * g.ic;
    int bh = rows;
    // few long bands: the halo rows are re-read once per band, and longer
    // streams per slot measure faster (8192 * SPW / 4 units is ~2000+ waves)
    while (bh > 4 && planes * ((rows + bh - 1) / bh) < int64_t{8192} * p.SPW / 4) bh = (bh + 1) / 2;
    p.nbands = (rows + bh - 1) / bh;
    // rows per band, a multiple of the row loop's unroll factor (k; 2k for
    // the backward passes, which alternate two dy row buffers): steps past the
    // band's last row store nothing and read dy as zero
    const int step = pass == 0 ? g.kh : 2 * g.kh;
    p.BH = ((rows + p.nbands - 1) / p.nbands + step - 1) / step * step;
    p.nbands = (rows + p.BH - 1) / p.BH;
    p.nunits = g.n * p.nbands;  // units per channel
    if (pass == 2) {
        const int per_round = kWaves * p.SPW;
        const int rounds = (p.nunits + per_round - 1) / per_round;
        const int nc = std::min(rounds, std::max(1, (2048 + g.ic - 1) / g.ic));
        p.upc = ((rounds + nc - 1) / nc) * per_round;
        p.NC = (p.nunits + p.upc - 1) / p.upc;
        p.wpc = 0;
        p.grid = g.ic * p.NC;
    } else {
        p.wpc = (p.nunits + p.SPW - 1) / p.SPW;
        p.NC = p.upc = 0;
        const int64_t waves = static_cast<int64_t>(g.ic) * p.wpc;
        if (waves > int64_t{1} << 30) return false;
        p.grid = static_cast<int>((waves + kWaves - 1) / kWaves);
    }
    return true;
}

template <typename T>
DcArgs<T> dec_args(const Geo &g, const DcPlan &p) {
    DcArgs<T> a{};
    a.g = g;
    a.XH = (g.ih + 1) / 2;
    a.XW = (g.iw + 1) / 2;
    a.NS = p.NS;
    a.SPW = p.SPW;
    a.BH = p.BH;
    a.nbands = p.nbands;
    a.wpc = p.wpc;
    a.nunits = p.nunits;
    a.NC = p.NC;
    a.upc = p.upc;
    return a;
}

bool aligned16(const void *p) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % 16 == 0; }

template <typename T, int K, int MM, bool FULL>
void launch_dec(int pass, int grid, const DcArgs<T> &a, hipStream_t s) {
    if (pass == 0) {
        if constexpr (sizeof(T) == 2 && FULL)
            hipLaunchKernelGGL((dec_fwd_dot2_kernel<T, K, MM>), dim3(grid), dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((dec_fwd_kernel<T, K, MM, FULL>), dim3(grid), dim3(kThreads), 0, s, a);
    }
    else if (pass == 1)
        hipLaunchKernelGGL((dec_bwdin_kernel<T, K, MM, FULL>), dim3(grid), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((dec_bwdw_kernel<T, K, MM, FULL>), dim3(grid), dim3(kThreads), 0, s, a);
}

template <typename T, int K, int MM>
int run_dec(int pass, const Geo &g, const void *in, const void *in2, const void *w, const void *b, void *out,
            void *ws, hipStream_t s) {
    DcPlan p;
    if (!plan_dec(g, pass, p)) return kErrUnsupported;
    DcArgs<T> a = dec_args<T>(g, p);
    a.in = static_cast<const T *>(in);
    a.in2 = static_cast<const T *>(in2);
    a.w = static_cast<const T *>(w);
    a.b = static_cast<const T *>(b);
    a.out = static_cast<T *>(out);
    a.ws = static_cast<float *>(ws);
    // Whole-vector path: every lane's x segment [2c0, 2c0+8) and strip [c0, c0+4)
    // lie inside their rows (iw a multiple of 8 makes ow = iw/2 a multiple of 4),
    // and every row starts 16-byte aligned.
    const bool full = g.iw % 8 == 0 && aligned16(in) && aligned16(in2) && aligned16(out);
    if (full)
        launch_dec<T, K, MM, true>(pass, p.grid, a, s);
    else
        launch_dec<T, K, MM, false>(pass, p.grid, a, s);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T>
int dec_t(int pass, const Geo &g, const void *in, const void *in2, const void *w, const void *b, void *out, void *ws,
          hipStream_t s) {
    if (g.kh == 3) return g.mult == 1 ? run_dec<T, 3, 1>(pass, g, in, in2, w, b, out, ws, s)
                                      : run_dec<T, 3, 2>(pass, g, in, in2, w, b, out, ws, s);
    return g.mult == 1 ? run_dec<T, 5, 1>(pass, g, in, in2, w, b, out, ws, s)
                       : run_dec<T, 5, 2>(pass, g, in, in2, w, b, out, ws, s);
}

int dec_dispatch(int pass, const Geo &g, const void *in, const void *in2, const void *w, const void *b, void *out,
                 void *ws, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return dec_t<float>(pass, g, in, in2, w, b, out, ws, s);
        case 1: return dec_t<__half>(pass, g, in, in2, w, b, out, ws, s);
        default: return dec_t<bf16_t>(pass, g, in, in2, w, b, out, ws, s);
    }
}

}  // namespace

bool decim_fits(const Geo &g, int pass) {
    if (g.kh != g.kw || (g.kh != 3 && g.kh != 5)) return false;
    if (g.sh != 2 || g.sw != 2 || g.dh != 2 || g.dw != 2) return false;
    if (g.ph != g.kh - 1 || g.pw != g.kw - 1 || g.mult > 2) return false;
    DcPlan p;
    return plan_dec(g, pass, p);
}

int decim_bwd_weight_chunks(const Geo &g) {
    DcPlan p;
    return plan_dec(g, 2, p) ? p.NC : 0;
}

int decim_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s) {
    return dec_dispatch(0, g, x, nullptr, w, b, y, nullptr, dtype, s);
}

int decim_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s) {
    return dec_dispatch(1, g, dy, nullptr, w, nullptr, dx, nullptr, dtype, s);
}

int decim_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s) {
    return dec_dispatch(2, g, x, dy, nullptr, nullptr, nullptr, ws, dtype, s);
}

}  // namespace dw
