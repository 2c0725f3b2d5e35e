// dw_largek_wgrad16.hip -- depthwise grad-weight for filters of up to 16 x 16
// (k = 13 in the large-kernel sweep) on the gfx950 matrix cores, any I/O
// dtype (stride 1, dilation 1, multiplier 1).
//
// The same contraction as the 31 x 31 matrix-core grad-weight: for one image n
// and one output row oh,
//   dw[i][j] += sum_m X[oh + i - P][m] * dy[oh][m - j + P],
// a product over the input columns m of A[i][m] = X[oh + i - P][m] (tap rows x
// input columns) and B[m][j] = dy[oh][m - j + P] (the dy row arranged by
// shift), zero where the dy column leaves [0, ow).  A 13 x 13 filter fills 42 %
// of a 32 x 32 tile but 66 % of a 16 x 16 one, so the tile here is one
// v_mfma_f32_16x16x4_f32 accumulator (fp32 multiply-add, fp32 sums; 16-bit
// inputs are widened to fp32 when staged).
//
// Lane layout of v_mfma_f32_16x16x4_f32 (checked on the MI355X with an
// in-bounds probe): A lane l holds row l % 16, k = l / 16; B lane l holds
// column l % 16, k = l / 16; D register r of lane l holds row 4 (l / 16) + r,
// column l % 16.  Instruction t of a 16-column step takes input column
// base + 4 (l / 16) + t, so the four instructions of a step consume one
// 16-byte LDS read of x per lane and four 4-byte reads of dy.
//
// A workgroup (4 waves) owns one channel and a chunk of images.  Per band of
// dy rows it stages the input rows the band reads (zero rows outside the
// image) and the dy rows, each at column offset 15 - P of a zeroed row so
// every B read is in bounds and reads zero outside the row; the waves take the
// band's dy rows in turn, alternating two accumulators.  The waves' tiles are
// summed in a fixed order into the chunk partial of the two-pass, atomics-free
// reduction.
#include "dw_common.hpp"
#include "dw_internal.hpp"

namespace dw {
namespace {

typedef float f32x4_w __attribute__((ext_vector_type(4)));

constexpr int kW16Off = 15;      // largest kernel column reach left of a dy column
constexpr int kW16TargetWG = 6144;

template <typename T> struct Lw16Args {
    const T *x;
    const T *dy;
    float *ws;      // [c][NC][k*k + 1]
    int C, N, IH, IW, OH, OW, P;
    int NC, npc;    // image chunks, images per chunk
    int BH, nbands; // dy rows per band, bands per plane
    int XW;         // x columns the instructions walk: iw rounded up to 16
    int XP;         // LDS pitch of an x row: XW + 4 (the 16 rows a read touches in distinct banks)
    int L;          // LDS pitch of a dz row: XW + 20
    int D0;         // dz column of dy column 0: 15 - P rounded up to a multiple of 4
                    // (16-byte stores; the B reads start at D0 + P - 15 >= 0)
    int vx, vd;     // x / dy rows are whole aligned 16-byte vectors
};

__device__ __forceinline__ f32x4_w mfma16(float a, float b, f32x4_w c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Rows [r0, r0 + nrows) of a plane with `w` elements per row into fp32 LDS rows
// of `pitch` floats (row r at dst + (r - r0) * pitch), rows outside [0, h) as
// zeros; 16-byte loads when vec.
template <typename T>
__device__ __forceinline__ void stage_f32(float *dst, int pitch, const T *src, int r0, int nrows, int h, int w,
                                          bool vec, int tid) {
    if (vec) {
        constexpr int VE = Vec<T>::N;
        const int vpr = w / VE;
        for (int v = tid; v < nrows * vpr; v += 256) {
            const int r = v / vpr;
            const int c0 = (v - r * vpr) * VE;
            const int ih = r0 + r;
            union {
                uint4 u;
                T t[VE];
            } raw;
            raw.u = make_uint4(0u, 0u, 0u, 0u);
            if (ih >= 0 && ih < h) raw.u = *reinterpret_cast<const uint4 *>(src + static_cast<int64_t>(ih) * w + c0);
            float4 *d = reinterpret_cast<float4 *>(dst + r * pitch + c0);
#pragma unroll
            for (int e = 0; e < VE / 4; ++e)
                d[e] = make_float4(to_f32(raw.t[4 * e]), to_f32(raw.t[4 * e + 1]), to_f32(raw.t[4 * e + 2]),
                                   to_f32(raw.t[4 * e + 3]));
        }
    } else {
        for (int e = tid; e < nrows * w; e += 256) {
            const int r = e / w;
            const int col = e - r * w;
            const int ih = r0 + r;
            dst[r * pitch + col] = (ih >= 0 && ih < h) ? to_f32(src[static_cast<int64_t>(ih) * w + col]) : 0.f;
        }
    }
}

// 16-byte vectors per thread that hold a band's rows while the previous band
// is computed (x rows, dy rows), for rows of at most kW16PfCols elements.
constexpr int kW16PfCols = 64;
template <typename T> constexpr int kW16Nx = ((32 + 16 - 1) * (kW16PfCols / Vec<T>::N) + 255) / 256;
template <typename T> constexpr int kW16Nd = (32 * (kW16PfCols / Vec<T>::N) + 255) / 256;

template <typename T, int K, bool PF>
__global__ __launch_bounds__(256) void lk_wgrad16_kernel(Lw16Args<T> a) {
    static_assert(K <= 16, "one 16 x 16 tile");
    extern __shared__ __align__(16) unsigned char smem[];
    float *xs = reinterpret_cast<float *>(smem);          // [BH + K - 1][XP]
    float *dz = xs + (a.BH + K - 1) * a.XP;               // [BH][L]
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the row loop branches on it
    const int lane = tid & 63;
    const int mj = lane & 15, kq = lane >> 4;
    const int c = blockIdx.x / a.NC;
    const int chunk = blockIdx.x - c * a.NC;
    const int n0 = chunk * a.npc, n1 = min(n0 + a.npc, a.N);

    // zero once: x columns iw .. XP - 1 of every row and every dz column
    // outside the dy row are never rewritten
    const int xtot = (a.BH + K - 1) * a.XP, dtot = a.BH * a.L;
    for (int e = tid; e < xtot + dtot; e += 256) xs[e] = 0.f;

    f32x4_w acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    float dsum = 0.f;
    // tap rows K .. 15 (outside the filter) read tap row K - 1's input row so
    // every read stays in the staged rows; their results are discarded
    const int mi = min(mj, K - 1);

    // (image, band) steps; with PF the next step's rows are loaded into
    // registers while the current band is computed
    constexpr int VE = Vec<T>::N;
    constexpr int NXV = PF ? kW16Nx<T> : 1, NDV = PF ? kW16Nd<T> : 1;
    const int nsteps = (n1 - n0) * a.nbands;
    uint4 pfx[NXV], pfd[NDV];
    // each thread's vectors (row, element column) are the same for every band:
    // divided once here, not per band
    const int xv = PF ? a.IW / VE : 1, dv = PF ? a.OW / VE : 1;
    int xr_[NXV], xc_[NXV], dr_[NDV], dc_[NDV];
#pragma unroll
    for (int k = 0; k < NXV; ++k) {
        const int v = tid + 256 * k;
        xr_[k] = v / xv;
        xc_[k] = (v - xr_[k] * xv) * VE;
    }
#pragma unroll
    for (int k = 0; k < NDV; ++k) {
        const int v = tid + 256 * k;
        dr_[k] = v / dv;
        dc_[k] = (v - dr_[k] * dv) * VE;
    }
    auto prefetch = [&](int t) {
        const int n = n0 + t / a.nbands, oh0 = (t % a.nbands) * a.BH;
        const int rows = min(a.BH, a.OH - oh0);
        const T *xp = a.x + (static_cast<int64_t>(n) * a.C + c) * a.IH * a.IW;
        const T *dp = a.dy + (static_cast<int64_t>(n) * a.C + c) * a.OH * a.OW;
#pragma unroll
        for (int k = 0; k < NXV; ++k) {
            const int ih = oh0 + xr_[k] - a.P;
            pfx[k] = make_uint4(0u, 0u, 0u, 0u);
            if (xr_[k] < rows + K - 1 && ih >= 0 && ih < a.IH)
                pfx[k] = *reinterpret_cast<const uint4 *>(xp + static_cast<int64_t>(ih) * a.IW + xc_[k]);
        }
#pragma unroll
        for (int k = 0; k < NDV; ++k) {
            pfd[k] = make_uint4(0u, 0u, 0u, 0u);
            if (dr_[k] < rows)
                pfd[k] = *reinterpret_cast<const uint4 *>(dp + static_cast<int64_t>(oh0 + dr_[k]) * a.OW + dc_[k]);
        }
    };
    if (PF && nsteps > 0) prefetch(0);

    for (int t = 0; t < nsteps; ++t) {
        const int n = n0 + t / a.nbands, band = t % a.nbands;
        const T *xp = a.x + (static_cast<int64_t>(n) * a.C + c) * a.IH * a.IW;
        const T *dp = a.dy + (static_cast<int64_t>(n) * a.C + c) * a.OH * a.OW;
        {
            const int oh0 = band * a.BH;
            const int rows = min(a.BH, a.OH - oh0);
            __syncthreads();  // the previous band's reads are done
            // staged x row r is image row oh0 + r - P; dy row r sits at dz column D0
            if constexpr (PF) {
                const int xv = a.IW / VE, dv = a.OW / VE;
#pragma unroll
                for (int k = 0; k < NXV; ++k) {
                    if (xr_[k] < rows + K - 1) {
                        union {
                            uint4 u;
                            T t[VE];
                        } raw;
                        raw.u = pfx[k];
                        float4 *d = reinterpret_cast<float4 *>(xs + xr_[k] * a.XP + xc_[k]);
#pragma unroll
                        for (int e = 0; e < VE / 4; ++e)
                            d[e] = make_float4(to_f32(raw.t[4 * e]), to_f32(raw.t[4 * e + 1]), to_f32(raw.t[4 * e + 2]),
                                               to_f32(raw.t[4 * e + 3]));
                    }
                }
#pragma unroll
                for (int k = 0; k < NDV; ++k) {
                    if (dr_[k] < rows) {
                        union {
                            uint4 u;
                            T t[VE];
                        } raw;
                        raw.u = pfd[k];
                        float4 *d = reinterpret_cast<float4 *>(dz + a.D0 + dr_[k] * a.L + dc_[k]);
#pragma unroll
                        for (int e = 0; e < VE / 4; ++e) {
                            const float4 q = make_float4(to_f32(raw.t[4 * e]), to_f32(raw.t[4 * e + 1]),
                                                         to_f32(raw.t[4 * e + 2]), to_f32(raw.t[4 * e + 3]));
                            d[e] = q;
                            dsum += (q.x + q.y) + (q.z + q.w);  // bias gradient, this thread's vectors in order
                        }
                    }
                }
            } else {
                stage_f32<T>(xs, a.XP, xp, oh0 - a.P, rows + K - 1, a.IH, a.IW, a.vx != 0, tid);
                stage_f32<T>(dz + a.D0, a.L, dp, oh0, rows, a.OH, a.OW, a.vd != 0, tid);
            }
            __syncthreads();
            if (PF && t + 1 < nsteps) prefetch(t + 1);
            // bias gradient (the prefetching variant sums the dy vectors as it
            // stages them): the band's dy values, summed per thread in a fixed order
            if constexpr (!PF) {
                for (int e = tid; e < rows * a.OW; e += 256) {
                    const int r = e / a.OW;
                    dsum += dz[r * a.L + a.D0 + (e - r * a.OW)];
                }
            }
            for (int oh = wave; oh < rows; oh += 4) {
                // A: x row oh + i, column base + 4 kq + t; B: dz[oh][base + 4 kq + t - j + 15]
                const float *xr = xs + (oh + mi) * a.XP + 4 * kq;
                const float *dr = dz + oh * a.L + a.D0 + a.P - mj + 4 * kq;
                for (int base = 0; base < a.XW; base += 16) {
                    const float4 av = *reinterpret_cast<const float4 *>(xr + base);
                    const float b0 = dr[base], b1 = dr[base + 1], b2 = dr[base + 2], b3 = dr[base + 3];
                    acc0 = mfma16(av.x, b0, acc0);
                    acc1 = mfma16(av.y, b1, acc1);
                    acc0 = mfma16(av.z, b2, acc0);
                    acc1 = mfma16(av.w, b3, acc1);
                }
            }
        }
    }

    // fixed-order sum of the 4 waves' tiles and of the 256 dy partial sums
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);  // [wave][lane][5]
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 64 + lane) * 5 + r] = acc0[r] + acc1[r];
    red[(wave * 64 + lane) * 5 + 4] = dsum;
    __syncthreads();
    float *dst = a.ws + (static_cast<int64_t>(c) * a.NC + chunk) * (K * K + 1);
    for (int e = tid; e < K * K + 1; e += 256) {
        float v = 0.f;
        if (e < K * K) {
            const int i = e / K, j = e - (e / K) * K;
            const int ln = 16 * (i >> 2) + j, r = i & 3;
            for (int w = 0; w < 4; ++w) v += red[(w * 64 + ln) * 5 + r];
        } else {
            for (int t = 0; t < 256; ++t) v += red[t * 5 + 4];
        }
        dst[e] = v;
    }
}

struct Lw16Plan {
    int NC, npc, BH, nbands, XW, XP, L, lds_bytes;
};

bool plan_lw16(const Geo &g, Lw16Plan &p) {
    p.XW = (g.iw + 15) & ~15;
    p.XP = p.XW + 4;
    p.L = p.XW + 20;
    const int K = g.kh;
    auto bytes = [&](int bh) {
        const int64_t stage = (static_cast<int64_t>(bh + K - 1) * p.XP + static_cast<int64_t>(bh) * p.L) * 4;
        return std::max<int64_t>(stage, 4 * 64 * 5 * 4);
    };
    // bands of at most 32 dy rows within 32 KiB, so several workgroups share a
    // CU and one's staging overlaps the others' matrix work
    int bh = std::min(g.oh, 32);
    while (bh > 1 && bytes(bh) > 32 * 1024) --bh;
    if (bytes(bh) > 64 * 1024) return false;
    p.nbands = (g.oh + bh - 1) / bh;
    p.BH = (g.oh + p.nbands - 1) / p.nbands;
    p.lds_bytes = static_cast<int>(bytes(p.BH));
    int NC = std::max(1, (kW16TargetWG + g.ic - 1) / g.ic);
    NC = std::min(NC, g.n);
    p.npc = (g.n + NC - 1) / NC;
    p.NC = (g.n + p.npc - 1) / p.npc;
    return true;
}

template <typename T>
int run_lw16(const Geo &g, const Lw16Plan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    Lw16Args<T> a{};
    a.x = static_cast<const T *>(x);
    a.dy = static_cast<const T *>(dy);
    a.ws = static_cast<float *>(ws);
    a.C = g.ic;
    a.N = g.n;
    a.IH = g.ih;
    a.IW = g.iw;
    a.OH = g.oh;
    a.OW = g.ow;
    a.P = g.ph;
    a.NC = p.NC;
    a.npc = p.npc;
    a.BH = p.BH;
    a.nbands = p.nbands;
    a.XW = p.XW;
    a.XP = p.XP;
    a.L = p.L;
    a.D0 = (kW16Off - g.ph + 3) & ~3;
    a.vx = g.iw % Vec<T>::N == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
    a.vd = g.ow % Vec<T>::N == 0 && reinterpret_cast<uintptr_t>(dy) % 16 == 0;
    // register prefetch for whole-vector rows of at most kW16PfCols elements
    const bool pf = a.vx && a.vd && g.iw <= kW16PfCols && g.ow <= kW16PfCols && p.BH <= 32;
    if (pf)
        hipLaunchKernelGGL((lk_wgrad16_kernel<T, 13, true>), dim3(g.ic * p.NC), dim3(256), p.lds_bytes, s, a);
    else
        hipLaunchKernelGGL((lk_wgrad16_kernel<T, 13, false>), dim3(g.ic * p.NC), dim3(256), p.lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

}  // namespace

// 13 x 13 square filter, stride 1, dilation 1, multiplier 1, the same padding
// on both axes (at most 12: the dz offset covers it), rows of at most 256.
bool largek_wgrad16_fits(const Geo &g, int dtype) {
    (void)dtype;  // every dtype is staged as fp32
    if (g.kh != 13 || g.kw != 13) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.ph != g.pw || g.mult != 1) return false;
    if (g.ph > g.kh - 1 || g.iw > 256) return false;
    Lw16Plan p;
    return plan_lw16(g, p);
}

int largek_wgrad16_chunks(const Geo &g) {
    Lw16Plan p;
    return plan_lw16(g, p) ? p.NC : 0;
}

int largek_wgrad16(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s) {
    Lw16Plan p;
    if (!plan_lw16(g, p)) return kErrUnsupported;
    switch (dtype) {
        case 0: return run_lw16<float>(g, p, x, dy, ws, s);
        case 1: return run_lw16<__half>(g, p, x, dy, ws, s);
        default: return run_lw16<bf16_t>(g, p, x, dy, ws, s);
    }
}

}  // namespace dw
