// dw_largek_wgrad7.hip -- 7 x 7 "same" depthwise grad-weight as a row stream
// on the vector units (stride 1, dilation 1, padding 3, multiplier 1, any
// I/O dtype).
//
//   dw[i][j] = sum_{n, oh, ow} dy[n, oh, ow] * x[n, oh + i - 3, ow + j - 3],
//   db       = sum dy
// (PR #3057's grad-weight with the padding its commits add).  With 49 taps a
// band staged in LDS feeds the multiply-adds from LDS at about one value per
// three of them, which the LDS cannot sustain, so nothing is staged here:
// each lane owns 4 adjacent columns of a plane (one 16- or 8-byte load per
// row of x and of dy) and walks a band of dy rows.  The 3 columns on either
// side that its 7-column windows also read come from the neighbouring lanes
// of the same plane row through cross-lane moves (DPP whole-wave shifts by
// one lane), zero at the row's ends.  The 7 x rows under the current dy row
// are kept as a register ring, the 49 tap sums and the dy sum in registers,
// and the loads run two (fp32) or three (16-bit) rows ahead.  The row loop is
// unrolled by 7 times that so ring slots and load buffers are compile-time
// registers that keep their roles across the back edge.
//   fp32: the ring holds the 10-column windows as floats; 196 v_fmac_f32 a row.
//   16-bit: the ring holds the 9 overlapping pairs (w[p], w[p+1]) of each
//   window (own words as they are, the others built with one funnel shift
//   each) and dy as its two raw words, so one v_dot2c_f32_{f16,bf16} takes two
//   dy columns of a tap: 98 a row (the products are exact, the sums fp32).
// At the end the lanes' sums are reduced over the wave (transpose-sum), then
// over the workgroup's waves in a fixed order, into the chunk partial of the
// two-pass, atomics-free reduction.
#include "dw_internal.hpp"
#include "dw_stream.hpp"

namespace dw {
namespace {

constexpr int kS7K = 7;
constexpr int kS7P = 3;                     // padding: the window is own 4 columns plus 3 each side
constexpr int kS7W = 4 + 2 * kS7P;          // x columns of a lane's window
constexpr int kS7A = kS7K * kS7K + 1;       // accumulated values: 49 taps, dy sum

template <typename T> struct S7Args {
    const T *x, *dy;
    float *ws;          // [c][NC][50]
    int C, IH, IW;      // OH = IH, OW = IW
    int NS, SPW;        // lanes per row, row slots per wave
    int BH, nbands;     // dy rows per band, bands per plane
    int NC, upc;        // chunks per channel, units (image, band) per chunk
    int nunits;         // units per channel
};

// words holding a lane's 4 elements
template <typename T> constexpr int kS7Words = static_cast<int>(sizeof(T));

// The 4 elements at columns col .. col + 3 of a row of w elements as raw
// words: one vector load (VEC: whole aligned 4-element runs), else element by
// element with the columns at and past w read as zero.
template <typename T, bool VEC>
__device__ __forceinline__ void s7_load(uint32_t (&r)[kS7Words<T>], const T *row, int col, int w) {
    if constexpr (VEC) {
        load_words<kS7Words<T>>(row + col, r);
    } else {
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = col + e < w ? bits_of(row[min(col + e, w - 1)]) : 0u;
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = b[e];
        } else {
            r[0] = b[0] | (b[1] << 16);
            r[1] = b[2] | (b[3] << 16);
        }
    }
}

// Value of lane - 1 (DPP wave_shr:1) and lane + 1 (wave_shl:1), 0 past the
// wave's ends.  A DPP move reads a lane that EXEC disables as zero, so it must
// run with every lane enabled: the empty volatile asm keeps the compiler from
// moving it under the branch of a later select.
__device__ __forceinline__ uint32_t from_left(uint32_t v) {
    uint32_t r = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x138, 0xf, 0xf, true));
    asm volatile("" : "+v"(r));
    return r;
}
__device__ __forceinline__ uint32_t from_right(uint32_t v) {
    uint32_t r = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x130, 0xf, 0xf, true));
    asm volatile("" : "+v"(r));
    return r;
}

// Rows loaded ahead: three, two for fp32 (a third would leave room for only
// two waves per SIMD).
template <typename T> constexpr int kS7Ahead = sizeof(T) == 4 ? 2 : 3;

// One ring row: fp32 -- the window's 10 values; 16-bit -- its 9 pairs.
template <typename T> constexpr int kS7Ring = sizeof(T) == 4 ? kS7W : kS7W - 1;

template <typename T>
__device__ __forceinline__ void s7_window(const uint32_t (&r)[kS7Words<T>], bool ok, bool first, bool last,
                                          uint32_t (&w)[kS7Ring<T>]) {
    uint32_t v[kS7Words<T>];
#pragma unroll
    for (int e = 0; e < kS7Words<T>; ++e) v[e] = ok ? r[e] : 0u;
    if constexpr (sizeof(T) == 4) {
        // w[0..2] = left lane's columns 1..3, w[3..6] own, w[7..9] = right lane's columns 0..2
#pragma unroll
        for (int e = 0; e < kS7P; ++e) {
            const uint32_t l = from_left(v[4 - kS7P + e]);
            const uint32_t rr = from_right(v[e]);
            w[e] = first ? 0u : l;
            w[kS7P + 4 + e] = last ? 0u : rr;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) w[kS7P + e] = v[e];
    } else {
        // words L0 L1 | O0 O1 | R0 R1 hold elements -4..-1 | 0..3 | 4..7 of the lane's
        // columns; the window starts at element -3, so pair p = elements (p - 3, p - 2)
        const uint32_t dl0 = from_left(v[0]), dl1 = from_left(v[1]);
        const uint32_t dr0 = from_right(v[0]), dr1 = from_right(v[1]);
        const uint32_t l0 = first ? 0u : dl0, l1 = first ? 0u : dl1;
        const uint32_t r0 = last ? 0u : dr0, r1 = last ? 0u : dr1;
        w[0] = __builtin_amdgcn_alignbit(l1, l0, 16);
        w[1] = l1;
        w[2] = __builtin_amdgcn_alignbit(v[0], l1, 16);
        w[3] = v[0];
        w[4] = __builtin_amdgcn_alignbit(v[1], v[0], 16);
        w[5] = v[1];
        w[6] = __builtin_amdgcn_alignbit(r0, v[1], 16);
        w[7] = r0;
        w[8] = __builtin_amdgcn_alignbit(r1, r0, 16);
    }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void s7_wgrad_kernel(S7Args<T> a) {
    constexpr int K = kS7K, A = kS7A, D = kS7Ahead<T>, NW = kS7Words<T>, RW = kS7Ring<T>;
    constexpr bool F32 = sizeof(T) == 4;
    __shared__ float red[4][A];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = blockIdx.x / a.NC;
    const int chunk = blockIdx.x - c * a.NC;
    const int slot = lane / a.NS;
    const int s = lane - slot * a.NS;
    const int c0 = 4 * s;                      // this lane's columns c0 .. c0 + 3
    const bool first = s == 0, last = s == a.NS - 1;
    const int H = a.IH, W = a.IW;
    float acc[A];
#pragma unroll
    for (int t = 0; t < A; ++t) acc[t] = 0.f;
    const uint32_t ones = sizeof(T) == 4 ? 0u : bits_of(from_f32<T>(1.f)) * 0x10001u;

    const int ubeg = chunk * a.upc, uend = min(ubeg + a.upc, a.nunits);
    for (int base = ubeg; base < uend; base += 4 * a.SPW) {
        const int unit = base + wave * a.SPW + slot;
        const bool act = slot < a.SPW && unit < uend;
        const int n = act ? unit / a.nbands : 0;
        const int band = act ? unit - n * a.nbands : 0;
        const int64_t plane = (static_cast<int64_t>(n) * a.C + c) * H * W;
        const T *xp = a.x + plane;
        const T *dp = a.dy + plane;
        const int oh0 = band * a.BH, rows = act ? min(a.BH, H - oh0) : 0;
        // x row q of the band is image row oh0 - 3 + q (q < rows + 6); dy row t is oh0 + t (t < rows)
        auto xrow_ok = [&](int q) { return q < rows + K - 1 && oh0 - kS7P + q >= 0 && oh0 - kS7P + q < H; };
        auto xrow_ptr = [&](int q) { return xp + static_cast<int64_t>(min(max(oh0 - kS7P + q, 0), H - 1)) * W; };
        auto drow_ptr = [&](int t) { return dp + static_cast<int64_t>(min(oh0 + t, H - 1)) * W; };
        // loads D steps ahead into buffer t % D: step t needs x row t + 6 and dy row t
        uint32_t xq[D][NW], dq[D][NW];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            s7_load<T, VEC>(xq[d], xrow_ptr(K - 1 + d), c0, W);
            s7_load<T, VEC>(dq[d], drow_ptr(d), c0, W);
        }
        // ring slot v holds x row v modulo 7; rows 0 .. 5 first (all loads issued before the first wait)
        uint32_t win[K][RW];
        {
            uint32_t r[K - 1][NW];
#pragma unroll
            for (int q = 0; q < K - 1; ++q) s7_load<T, VEC>(r[q], xrow_ptr(q), c0, W);
#pragma unroll
            for (int q = 0; q < K - 1; ++q) s7_window<T>(r[q], xrow_ok(q), first, last, win[q]);
        }
        for (int t0 = 0; t0 < rows; t0 += K * D) {
#pragma unroll
            for (int uu = 0; uu < K * D; ++uu) {
                const int t = t0 + uu;
                if (t >= rows) break;
                const int b = uu % D;
                s7_window<T>(xq[b], xrow_ok(t + K - 1), first, last, win[(uu + K - 1) % K]);
                uint32_t dv[NW];
#pragma unroll
                for (int e = 0; e < NW; ++e) dv[e] = dq[b][e];
                s7_load<T, VEC>(xq[b], xrow_ptr(t + K - 1 + D), c0, W);
                s7_load<T, VEC>(dq[b], drow_ptr(t + D), c0, W);
                if constexpr (F32) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float d = __uint_as_float(dv[q]);
                        acc[A - 1] += d;
#pragma unroll
                        for (int i = 0; i < K; ++i)
#pragma unroll
                            for (int j = 0; j < K; ++j)
                                acc[i * K + j] = fmaf(d, __uint_as_float(win[(uu + i) % K][q + j]), acc[i * K + j]);
                    }
                } else {
                    // dy word h holds columns 2h, 2h + 1: with window pair 2h + j it gives tap j
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        acc[A - 1] = Dot2<T>::run(dv[h], ones, acc[A - 1]);
#pragma unroll
                        for (int i = 0; i < K; ++i)
#pragma unroll
                            for (int j = 0; j < K; ++j)
                                acc[i * K + j] = Dot2<T>::run(dv[h], win[(uu + i) % K][2 * h + j], acc[i * K + j]);
                    }
                }
            }
        }
    }
    // fixed-order sums: over the wave, then over the 4 waves
    const float v = wave_transpose_sum<A>(acc, lane);
    if (lane < A) red[wave][lane] = v;
    __syncthreads();
    if (tid < A)
        a.ws[(static_cast<int64_t>(c) * a.NC + chunk) * A + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

struct S7Plan {
    int NS, SPW, BH, nbands, NC, upc, nunits;
};

bool plan_s7(const Geo &g, S7Plan &p) {
    p.NS = (g.iw + 3) / 4;
    if (p.NS > 64) return false;
    p.SPW = 64 / p.NS;
    // bands: enough units for about 2048 waves, bands of at least 14 rows
    const int64_t planes = static_cast<int64_t>(g.n) * g.ic;
    const int nb = static_cast<int>(std::min<int64_t>(std::max<int64_t>(1, (int64_t{2048} * p.SPW + planes - 1) / planes),
                                                       std::max(1, g.oh / (2 * kS7K))));
    p.BH = (g.oh + nb - 1) / nb;
    p.nbands = (g.oh + p.BH - 1) / p.BH;
    p.nunits = g.n * p.nbands;
    const int per_round = 4 * p.SPW;
    const int rounds = (p.nunits + per_round - 1) / per_round;
    const int nc = std::max(1, std::min(rounds, (2048 + g.ic - 1) / g.ic));
    p.upc = (rounds + nc - 1) / nc * per_round;
    p.NC = (p.nunits + p.upc - 1) / p.upc;
    return true;
}

template <typename T>
int run_s7(const Geo &g, const S7Plan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    S7Args<T> a{};
    a.x = static_cast<const T *>(x);
    a.dy = static_cast<const T *>(dy);
    a.ws = static_cast<float *>(ws);
    a.C = g.ic;
    a.IH = g.ih;
    a.IW = g.iw;
    a.NS = p.NS;
    a.SPW = p.SPW;
    a.BH = p.BH;
    a.nbands = p.nbands;
    a.NC = p.NC;
    a.upc = p.upc;
    a.nunits = p.nunits;
    const bool vec = g.iw % 4 == 0 && reinterpret_cast<uintptr_t>(x) % (4 * sizeof(T)) == 0 &&
                     reinterpret_cast<uintptr_t>(dy) % (4 * sizeof(T)) == 0;
    if (vec)
        hipLaunchKernelGGL((s7_wgrad_kernel<T, true>), dim3(g.ic * p.NC), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((s7_wgrad_kernel<T, false>), dim3(g.ic * p.NC), dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

}  // namespace

// 7 x 7 square filter, stride 1, dilation 1, padding 3 on both axes (so the
// output plane is the input plane), multiplier 1, rows of at most 256.
bool stream7_bwdw_fits(const Geo &g) {
    if (g.n < 1 || g.ih < 1 || g.iw < 1) return false;
    if (g.kh != kS7K || g.kw != kS7K) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.mult != 1) return false;
    if (g.ph != kS7P || g.pw != kS7P) return false;
    S7Plan p;
    return plan_s7(g, p);
}

int stream7_bwdw_chunks(const Geo &g) {
    S7Plan p;
    return plan_s7(g, p) ? p.NC : 0;
}

int stream7_bwdw(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s) {
    S7Plan p;
    if (!plan_s7(g, p)) return kErrUnsupported;
    switch (dtype) {
        case 0: return run_s7<float>(g, p, x, dy, ws, s);
        case 1: return run_s7<__half>(g, p, x, dy, ws, s);
        default: return run_s7<bf16_t>(g, p, x, dy, ws, s);
    }
}

}  // namespace dw
