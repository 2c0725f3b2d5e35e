// dw_largek.hip -- large-kernel depthwise forward and grad-input on gfx950
// (k = 7, 13, 31; stride 1, dilation 1).
//
// With a k x k filter each input element feeds k*k multiply-adds, so for
// k >= 13 these passes are bound by fp32 VALU throughput, not by HBM (the
// MegEngine large-kernel depthwise article: batch 64, 384 channels, kernels up
// to 31x31; its DirectConv splits kernel columns over 4 lanes and reduces with
// a shuffle butterfly).  On CDNA the filter of a plane is uniform across the
// workgroup, so here it is staged once as fp32 in LDS, each kernel row is
// read into VGPRs with broadcast 16-byte LDS reads and feeds TR*k*TC FMAs per
// input row, and each lane keeps a whole TR x TC output tile in VGPRs -- no
// cross-lane reduction is needed:
//   1. the workgroup stages its plane (or a band of rows) into LDS as fp32 with
//      the zero padding written out, so the inner loop has no bounds tests;
//   2. a lane walks the TR + k - 1 padded input rows its tile reads; each row
//      segment of TC + k - 1 values is read from LDS once and feeds up to
//      TR*k*TC FMAs (0.08 LDS words per FMA at k = 31);
//   3. grad-input is the same correlation of dy with the kernel flipped in
//      both axes and padding k - 1 - pad (stride 1, dilation 1, multiplier 1).
#include "dw_common.hpp"
#include "dw_internal.hpp"

namespace dw {
namespace {

template <typename T> struct LkArgs {
    const T *in;   // forward: x; grad-input: dy
    const T *w;
    const T *b;
    T *out;        // y or dx
    int IH, IW;    // input plane of this pass
    int OH, OW;    // output plane of this pass
    int P;         // top/left zero padding of this pass
    int C;         // output channels of this pass (planes per image)
    int mult;      // forward: output channels per input channel
    int pitch;     // LDS row pitch (floats)
    int BH;        // output rows per band
    int nbands;
    int NCB, NRB;  // column / row blocks of output tiles in a band
    int wsm_off;   // float offset of the fp32 filter copy in LDS
    int vin;       // input rows are whole 16-byte vectors (aligned): vector staging
    int vout;      // output tiles are whole (OW % TC == 0) and aligned: vector stores
    FastDiv fpitch, fvpr, fpad;
};

// TC fp32 values rounded to T and stored as 16-byte (or 8-byte) vectors.
template <typename T, int TC>
__device__ __forceinline__ void store_tile_row(T *p, const float (&v)[TC]) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int q = 0; q < TC; q += 4)
            *reinterpret_cast<float4 *>(p + q) = make_float4(v[q], v[q + 1], v[q + 2], v[q + 3]);
    } else if constexpr (TC == 8) {
        *reinterpret_cast<uint4 *>(p) =
            make_uint4(pack2<T>(v[0], v[1]), pack2<T>(v[2], v[3]), pack2<T>(v[4], v[5]), pack2<T>(v[6], v[7]));
    } else {
        *reinterpret_cast<uint2 *>(p) = make_uint2(pack2<T>(v[0], v[1]), pack2<T>(v[2], v[3]));
    }
}

template <typename T, int K, int TR, int TC, bool FLIP>
__global__ __launch_bounds__(256) void lk_conv_kernel(LkArgs<T> a) {
    extern __shared__ __align__(16) unsigned char smem[];
    float *xs = reinterpret_cast<float *>(smem);
    constexpr int WW4 = (TC + K - 1 + 3) / 4 * 4;
    static_assert(TC % 4 == 0, "column tile is whole 16-byte vectors");
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int plane = blockIdx.x / a.nbands;  // output plane (n, c)
    const int band = blockIdx.x - plane * a.nbands;
    const int n = plane / a.C;
    const int c = plane - n * a.C;
    const int cin = FLIP ? c : c / a.mult;  // input plane channel
    const int oh0 = band * a.BH;
    const int rows = min(a.BH, a.OH - oh0) + K - 1;  // padded input rows of this band
    const T *src = a.in + (static_cast<int64_t>(n) * (FLIP ? a.C : a.C / a.mult) + cin) * a.IH * a.IW;

    // 1. stage padded rows [oh0 - P, oh0 - P + rows) x cols [-P, pitch - P)
    if (a.vin) {
        // tile rows r_lo .. r_hi - 1 hold image rows; their image part is copied
        // with 16-byte loads (4 in flight per lane), the rest of the tile is zeroed
        constexpr int VE = Vec<T>::N;
        constexpr int NB = 4;
        const int r_lo = max(0, a.P - oh0), r_hi = min(rows, a.IH + a.P - oh0);
        const int vpr = a.IW / VE;
        const int nvec = max(r_hi - r_lo, 0) * vpr;
        const T *s0 = src + static_cast<int64_t>(oh0 - a.P + r_lo) * a.IW;
        for (int v0 = tid; v0 < nvec; v0 += NB * nthr) {
            uint4 raw[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                raw[k] = make_uint4(0u, 0u, 0u, 0u);
                const int v = v0 + k * nthr;
                if (v < nvec) raw[k] = *reinterpret_cast<const uint4 *>(s0 + static_cast<int64_t>(v) * VE);
            }
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int v = v0 + k * nthr;
                if (v < nvec) {
                    const int rr = static_cast<int>(fdiv(static_cast<uint32_t>(v), a.fvpr));
                    float *d = xs + (r_lo + rr) * a.pitch + a.P + (v - rr * vpr) * VE;
                    union {
                        uint4 u;
                        T t[VE];
                    } b;
                    b.u = raw[k];
#pragma unroll
                    for (int e = 0; e < VE; ++e) d[e] = to_f32(b.t[e]);
                }
            }
        }
        const int padw = a.pitch - a.IW;  // zero columns of an image row: P left, the rest right
        for (int e = tid; e < max(r_hi - r_lo, 0) * padw; e += nthr) {
            const int rr = static_cast<int>(fdiv(static_cast<uint32_t>(e), a.fpad));
            const int j = e - rr * padw;
            xs[(r_lo + rr) * a.pitch + (j < a.P ? j : a.IW + j)] = 0.f;
        }
        const int top = min(r_lo, rows) * a.pitch;  // whole zero rows above and below the image
        for (int e = tid; e < top; e += nthr) xs[e] = 0.f;
        const int bot0 = max(r_hi, r_lo) * a.pitch;
        for (int e = bot0 + tid; e < rows * a.pitch; e += nthr) xs[e] = 0.f;
    } else {
        const int total = rows * a.pitch;
        for (int e = tid; e < total; e += nthr) {
            const int r = static_cast<int>(fdiv(static_cast<uint32_t>(e), a.fpitch));
            const int col = e - r * a.pitch;
            const int ih = oh0 - a.P + r, iw = col - a.P;
            xs[e] = (ih >= 0 && ih < a.IH && iw >= 0 && iw < a.IW) ? to_f32(src[ih * a.IW + iw]) : 0.f;
        }
    }
    // The filter is staged once as fp32 in LDS, one row per KP floats (16-byte
    // aligned, zero past k).  A kernel row is read into VGPRs with KP/4
    // uniform-address (broadcast) 16-byte LDS reads when the row walk first
    // needs it and stays there for the TR steps that use it, so the FMAs take
    // both multiplicands from VGPRs and wait for no LDS read of their own.
    // (Scalar loads of an fp32 filter measured slower: the scalar cache misses
    // stall each row's FMAs; 16-bit taps at odd offsets cannot be scalar-loaded.)
    constexpr int KP = (K + 3) / 4 * 4;
    float *wsm = xs + a.wsm_off;
    for (int e = tid; e < K * KP; e += nthr) {
        const int i = e / KP, j = e - (e / KP) * KP;
        wsm[e] = j < K ? to_f32(a.w[(static_cast<int64_t>(c) * K + i) * K + j]) : 0.f;
    }
    __syncthreads();

    const float bias = (!FLIP && a.b) ? to_f32(a.b[c]) : 0.f;
    const int items = a.NRB * a.NCB;
    for (int it = tid; it < items; it += nthr) {
        const int rb = it / a.NCB;
        const int cb = it - rb * a.NCB;
        float acc[TR][TC];
#pragma unroll
        for (int tr = 0; tr < TR; ++tr)
#pragma unroll
            for (int q = 0; q < TC; ++q) acc[tr][q] = bias;
        const float *base = xs + (rb * TR) * a.pitch + cb * TC;
        // wr[u]: kernel row r of the step r = r0 + u that loaded it; tile row tr
        // at step r uses kernel row r - tr, loaded tr steps earlier
        float wr[TR][KP];
        static_assert((TR + K - 1) % TR == 0, "the row walk is whole passes of TR steps");
#pragma unroll 1
        for (int r0 = 0; r0 < TR + K - 1; r0 += TR) {
#pragma unroll
            for (int u = 0; u < TR; ++u) {
                const int r = r0 + u;
                if (r < K) {
                    const float4 *wp = reinterpret_cast<const float4 *>(wsm + (FLIP ? K - 1 - r : r) * KP);
#pragma unroll
                    for (int e = 0; e < KP / 4; ++e) {
                        const float4 v = wp[e];
                        wr[u][4 * e] = v.x;
                        wr[u][4 * e + 1] = v.y;
                        wr[u][4 * e + 2] = v.z;
                        wr[u][4 * e + 3] = v.w;
                    }
                }
                // TC and the pitch are multiples of 4: the window is read as 16-byte vectors
                float win[WW4];
                const float4 *rp = reinterpret_cast<const float4 *>(base + r * a.pitch);
#pragma unroll
                for (int e = 0; e < WW4 / 4; ++e) {
                    const float4 v = rp[e];
                    win[4 * e] = v.x;
                    win[4 * e + 1] = v.y;
                    win[4 * e + 2] = v.z;
                    win[4 * e + 3] = v.w;
                }
#pragma unroll
                for (int tr = 0; tr < TR; ++tr) {
                    const int i = r - tr;  // kernel row; uniform across the workgroup
                    if (i < 0 || i >= K) continue;
                    const float *wv = wr[(u - tr + TR) % TR];
#pragma unroll
                    for (int j = 0; j < K; ++j)
#pragma unroll
                        for (int q = 0; q < TC; ++q) acc[tr][q] = fmaf(wv[FLIP ? K - 1 - j : j], win[q + j], acc[tr][q]);
                }
            }
        }
        T *op = a.out + (static_cast<int64_t>(plane) * a.OH + oh0 + rb * TR) * a.OW + cb * TC;
#pragma unroll
        for (int tr = 0; tr < TR; ++tr) {
            if (oh0 + rb * TR + tr >= min(oh0 + a.BH, a.OH)) continue;
            if (a.vout) {
                store_tile_row<T, TC>(op + tr * a.OW, acc[tr]);
            } else {
#pragma unroll
                for (int q = 0; q < TC; ++q)
                    if (cb * TC + q < a.OW) op[tr * a.OW + q] = from_f32<T>(acc[tr][q]);
            }
        }
    }
}

struct LkPlan {
    int TC, BH, nbands, NCB, NRB, pitch, threads, lds_bytes;
};

constexpr int kTR = 2;

bool plan_lk(int OH, int OW, int K, LkPlan &p) {
    // column tile 8 unless that wastes more than a quarter of the row, else 4
    p.TC = 8;
    if (((OW + 7) / 8) * 8 - OW > OW / 4) p.TC = 4;
    p.NCB = (OW + p.TC - 1) / p.TC;
    p.pitch = p.NCB * p.TC + K - 1;
    p.pitch = (p.pitch + 3) & ~3;
    // rows per band: whole plane while the tile count fits 256 lanes and LDS fits 64 KiB
    int bh = OH;
    // padded input tile + an fp32 copy of the filter
    auto lds = [&](int b) { return (static_cast<int64_t>(b + K - 1) * p.pitch + K * ((K + 3) / 4 * 4)) * 4; };
    while (bh > kTR && (((bh + kTR - 1) / kTR) * p.NCB > 256 || lds(bh) > 64 * 1024)) bh = (bh + 1) / 2;
    if (lds(bh) > 64 * 1024) return false;
    p.nbands = (OH + bh - 1) / bh;
    p.BH = (OH + p.nbands - 1) / p.nbands;
    p.BH = (p.BH + kTR - 1) / kTR * kTR;
    p.nbands = (OH + p.BH - 1) / p.BH;
    p.NRB = p.BH / kTR;
    p.threads = std::min(256, ((p.NRB * p.NCB + 63) / 64) * 64);
    if (lds(p.BH) > 64 * 1024) return false;
    p.lds_bytes = static_cast<int>(lds(p.BH));
    return true;
}

template <typename T, int K, int TC, bool FLIP>
int run_lk(const LkArgs<T> &a0, const LkPlan &p, int planes, hipStream_t s) {
    LkArgs<T> a = a0;
    a.pitch = p.pitch;
    a.BH = p.BH;
    a.nbands = p.nbands;
    a.NCB = p.NCB;
    a.NRB = p.NRB;
    a.fpitch = make_fastdiv(p.pitch, static_cast<uint64_t>(p.BH + K) * p.pitch);
    a.wsm_off = (p.BH + K - 1) * p.pitch;
    const int rows_max = p.BH + K - 1;
    a.vin = a.IW % Vec<T>::N == 0 && reinterpret_cast<uintptr_t>(a.in) % 16 == 0;
    a.vout = a.OW % TC == 0 && reinterpret_cast<uintptr_t>(a.out) % 16 == 0;
    a.fvpr = make_fastdiv(std::max(a.IW / Vec<T>::N, 1), static_cast<uint64_t>(rows_max) * (a.IW / Vec<T>::N + 1));
    a.fpad = make_fastdiv(std::max(p.pitch - a.IW, 1), static_cast<uint64_t>(rows_max) * p.pitch);
    hipLaunchKernelGGL((lk_conv_kernel<T, K, kTR, TC, FLIP>), dim3(planes * p.nbands), dim3(p.threads), p.lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, bool FLIP>
int run_k(const LkArgs<T> &a, const LkPlan &p, int K, int planes, hipStream_t s) {
    if (p.TC == 8) {
        if (K == 7) return run_lk<T, 7, 8, FLIP>(a, p, planes, s);
        if (K == 13) return run_lk<T, 13, 8, FLIP>(a, p, planes, s);
        return run_lk<T, 31, 8, FLIP>(a, p, planes, s);
    }
    if (K == 7) return run_lk<T, 7, 4, FLIP>(a, p, planes, s);
    if (K == 13) return run_lk<T, 13, 4, FLIP>(a, p, planes, s);
    return run_lk<T, 31, 4, FLIP>(a, p, planes, s);
}

template <typename T>
int lk_fwd_t(const Geo &g, const void *x, const void *w, const void *b, void *y, hipStream_t s) {
    LkPlan p;
    if (!plan_lk(g.oh, g.ow, g.kh, p)) return kErrUnsupported;
    LkArgs<T> a{};
    a.in = static_cast<const T *>(x);
    a.w = static_cast<const T *>(w);
    a.b = static_cast<const T *>(b);
    a.out = static_cast<T *>(y);
    a.IH = g.ih;
    a.IW = g.iw;
    a.OH = g.oh;
    a.OW = g.ow;
    a.P = g.ph;
    a.C = g.oc;
    a.mult = g.mult;
    return run_k<T, false>(a, p, g.kh, g.n * g.oc, s);
}

template <typename T>
int lk_bwdin_t(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t s) {
    LkPlan p;
    if (!plan_lk(g.ih, g.iw, g.kh, p)) return kErrUnsupported;
    LkArgs<T> a{};
    a.in = static_cast<const T *>(dy);
    a.w = static_cast<const T *>(w);
    a.out = static_cast<T *>(dx);
    a.IH = g.oh;
    a.IW = g.ow;
    a.OH = g.ih;
    a.OW = g.iw;
    a.P = g.kh - 1 - g.ph;
    a.C = g.ic;
    a.mult = 1;
    return run_k<T, true>(a, p, g.kh, g.n * g.ic, s);
}


// ---------------------------------------------------------------- grad-weight
// dw[c,i,j] = sum_{n,oh,ow} dy[n,c,oh,ow] * xpad[n,c,oh+i,ow+j]: the same sliding
// correlation with the roles swapped (dy is the long "filter", dw the small
// output).  A workgroup owns (channel, image chunk); a lane holds a TR x TC
// tile of dw; the ceil(k/TR)*ceil(k/TC) tiles are replicated over NG lane groups
// that take every NG-th dy row, and the groups are summed at the end in a
// fixed order.  Per image the padded x plane and the dy plane are staged in
// LDS as fp32; a lane reads a 16-byte-vector x window and the dy values (the
// same for all lanes of a group, so the reads broadcast).
template <typename T> struct LkwArgs {
    const T *x;
    const T *dy;
    float *ws;     // [c][NC][k*k+1]
    int C, IH, IW, OH, OW, P;
    int N, NC, npc;
    int BH, nbands;  // dy rows per band, bands per plane
    int xpitch;    // LDS pitch of the padded x rows
    int xrows;     // LDS rows reserved for x: BH + k - 1
    int dpitch;    // LDS pitch of the dy rows (multiple of 8)
    int vx, vd;    // x / dy rows are whole aligned 16-byte vectors: vector staging
    FastDiv fxp, fdp, fxv, fdv;
};

// Copies `nrows` rows of `w` elements (whole 16-byte vectors, row stride w in
// global memory) into fp32 LDS rows of `pitch` floats starting at column
// col0; 4 loads in flight per lane.  fvpr divides by w / VE.
template <typename T>
__device__ __forceinline__ void stage_rows_vec(float *lds, int pitch, int col0, const T *src, int nrows, int w,
                                               FastDiv fvpr, int tid, int nthr) {
    constexpr int VE = Vec<T>::N;
    constexpr int NB = 4;
    const int vpr = w / VE;
    const int nvec = nrows * vpr;
    for (int v0 = tid; v0 < nvec; v0 += NB * nthr) {
        uint4 raw[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            raw[k] = make_uint4(0u, 0u, 0u, 0u);
            const int v = v0 + k * nthr;
            if (v < nvec) raw[k] = *reinterpret_cast<const uint4 *>(src + static_cast<int64_t>(v) * VE);
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int v = v0 + k * nthr;
            if (v < nvec) {
                const int r = static_cast<int>(fdiv(static_cast<uint32_t>(v), fvpr));
                float *d = lds + r * pitch + col0 + (v - r * vpr) * VE;
                union {
                    uint4 u;
                    T t[VE];
                } b;
                b.u = raw[k];
#pragma unroll
                for (int e = 0; e < VE; ++e) d[e] = to_f32(b.t[e]);
            }
        }
    }
}

template <typename T, int K, int TR, int TC, int SEG>
__global__ __launch_bounds__(256, 3) void lk_bwdw_kernel(LkwArgs<T> a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NRB = (K + TR - 1) / TR, NCB = (K + TC - 1) / TC, NT = NRB * NCB;
    constexpr int NG = 256 / NT;  // lane groups
    constexpr int XW = SEG + TC - 1, XW4 = (XW + 3) / 4 * 4;
    float *xs = reinterpret_cast<float *>(smem);
    float *ds = xs + a.xrows * a.xpitch;
    const int tid = threadIdx.x;
    // workgroup (channel, image chunk, band of dy rows)
    const int units = a.NC * a.nbands;
    const int c = blockIdx.x / units;
    const int rest = blockIdx.x - c * units;
    const int chunk = rest / a.nbands;
    const int band = rest - chunk * a.nbands;
    const int oh0 = band * a.BH, oh1 = min(oh0 + a.BH, a.OH);
    const int grp = tid / NT;
    const int tile = tid - grp * NT;
    const int rb = tile / NCB, cb = tile - (tile / NCB) * NCB;
    const bool lane_ok = grp < NG;
    float acc[TR][TC];
#pragma unroll
    for (int tr = 0; tr < TR; ++tr)
#pragma unroll
        for (int q = 0; q < TC; ++q) acc[tr][q] = 0.f;
    float dbs = 0.f;
    const int n0 = chunk * a.npc, n1 = min(n0 + a.npc, a.N);
    // padded x rows oh0 .. oh1 + k - 2 (image rows minus P) and dy rows oh0 .. oh1 - 1
    const int xtot = (oh1 - oh0 + K - 1) * a.xpitch, dtot = (oh1 - oh0) * a.dpitch;
    // tile rows r_lo .. r_hi - 1 hold image rows (at columns P .. P + IW - 1)
    const int r_lo = max(0, a.P - oh0), r_hi = min(oh1 - oh0 + K - 1, a.IH + a.P - oh0);
    if (a.vx && a.vd) {
        // the zero padding is the same for every image: write the whole tile once,
        // then each image overwrites only its data
        for (int e = tid; e < xtot; e += 256) xs[e] = 0.f;
        for (int e = tid; e < dtot; e += 256) ds[e] = 0.f;
    }
    for (int n = n0; n < n1; ++n) {
        __syncthreads();
        const T *xp = a.x + (static_cast<int64_t>(n) * a.C + c) * a.IH * a.IW;
        const T *dp = a.dy + (static_cast<int64_t>(n) * a.C + c) * a.OH * a.OW;
        if (a.vx && a.vd) {
            if (r_hi > r_lo)
                stage_rows_vec<T>(xs + r_lo * a.xpitch, a.xpitch, a.P, xp + static_cast<int64_t>(oh0 + r_lo - a.P) * a.IW,
                                  r_hi - r_lo, a.IW, a.fxv, tid, 256);
            stage_rows_vec<T>(ds, a.dpitch, 0, dp + static_cast<int64_t>(oh0) * a.OW, oh1 - oh0, a.OW, a.fdv, tid, 256);
        } else {
            for (int e = tid; e < xtot; e += 256) {
                const int r = static_cast<int>(fdiv(static_cast<uint32_t>(e), a.fxp));
                const int col = e - r * a.xpitch;
                const int ih = oh0 + r - a.P, iw = col - a.P;
                xs[e] = (ih >= 0 && ih < a.IH && iw >= 0 && iw < a.IW) ? to_f32(xp[ih * a.IW + iw]) : 0.f;
            }
            for (int e = tid; e < dtot; e += 256) {
                const int r = static_cast<int>(fdiv(static_cast<uint32_t>(e), a.fdp));
                const int col = e - r * a.dpitch;
                ds[e] = col < a.OW ? to_f32(dp[(oh0 + r) * a.OW + col]) : 0.f;
            }
        }
        __syncthreads();
        if (!lane_ok) continue;
        // lane groups take (dy row, segment) items in turn, so a band with fewer
        // rows than lane groups still keeps every group busy
        const int nseg = (a.OW + SEG - 1) / SEG;
        const int items = (oh1 - oh0) * nseg;
        for (int it = grp; it < items; it += NG) {
            const int oh = it / nseg;  // band-relative dy row
            const int s0 = (it - oh * nseg) * SEG;
            const float *drow = ds + oh * a.dpitch;
            {
                float dv[SEG];
                const float4 *d4 = reinterpret_cast<const float4 *>(drow + s0);
#pragma unroll
                for (int e = 0; e < SEG / 4; ++e) {
                    const float4 v = d4[e];
                    dv[4 * e] = v.x;
                    dv[4 * e + 1] = v.y;
                    dv[4 * e + 2] = v.z;
                    dv[4 * e + 3] = v.w;
                }
                if (tile == 0) {
#pragma unroll
                    for (int u = 0; u < SEG; ++u) dbs += dv[u];
                }
#pragma unroll
                for (int tr = 0; tr < TR; ++tr) {
                    const int i = rb * TR + tr;
                    if (i >= K) continue;
                    float xv[XW4];
                    const float4 *x4 = reinterpret_cast<const float4 *>(xs + (oh + i) * a.xpitch + cb * TC + s0);
#pragma unroll
                    for (int e = 0; e < XW4 / 4; ++e) {
                        const float4 v = x4[e];
                        xv[4 * e] = v.x;
                        xv[4 * e + 1] = v.y;
                        xv[4 * e + 2] = v.z;
                        xv[4 * e + 3] = v.w;
                    }
#pragma unroll
                    for (int u = 0; u < SEG; ++u)
#pragma unroll
                        for (int q = 0; q < TC; ++q) acc[tr][q] = fmaf(dv[u], xv[u + q], acc[tr][q]);
                }
            }
        }
    }
    // fixed-order sum over the lane groups, one tile row of every lane per
    // round (the buffer holds TC + 1 values per lane: the taps and the dy sum)
    float *red = xs;  // reuse: [256][TC + 1]
    constexpr int RS = TC + 1;
    float *dst = a.ws + (static_cast<int64_t>(c) * units + rest) * (K * K + 1);
#pragma unroll
    for (int tr = 0; tr < TR; ++tr) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < TC; ++q) red[tid * RS + q] = acc[tr][q];
        red[tid * RS + TC] = dbs;
        __syncthreads();
        for (int e = tid; e < NT * RS; e += 256) {
            const int t = e / RS, k = e - (e / RS) * RS;
            if (k == TC && (tr != 0 || t != 0)) continue;  // the dy sum once, from tile 0
            float v = 0.f;
            for (int gq = 0; gq < NG; ++gq) v += red[(gq * NT + t) * RS + k];
            if (k == TC) {
                dst[K * K] = v;
                continue;
            }
            const int i = (t / NCB) * TR + tr, j = (t - (t / NCB) * NCB) * TC + k;
            if (i < K && j < K) dst[i * K + j] = v;
        }
    }
}

struct LkwPlan {
    int NC, npc, BH, nbands, xpitch, xrows, dpitch, lds_bytes;
};

// Tile shape of the grad-weight lanes: TR x TC taps per lane over dy segments
// of SEG columns.  Each segment reads a TC + SEG - 1 wide x window per tile
// row from LDS, so the LDS bytes per FMA fall as the segment and the tile
// widen: at k = 31 a 16 x 16 tile halves them against 8 x 8 (1.1-1.25x
// faster; the kernel is held to 168 VGPRs so three waves share a SIMD, which
// measured faster than two waves with more registers), and at k = 7 and 13
// (8 tap columns per lane) 16-column segments measured 1.1-1.2x faster than
// 8-column ones.
constexpr int lkw_tc(int K) { return K == 31 ? 16 : 8; }
constexpr int kLkwSeg = 16;

bool plan_lkw(const Geo &g, int K, LkwPlan &p) {
    const int TC = lkw_tc(K), SEG = kLkwSeg;
    const int owr = (g.ow + SEG - 1) / SEG * SEG;  // dy columns walked (zero beyond ow)
    // x window of the last segment and tile: owr + ceil(k/TC)*TC + 3 columns at most
    p.xpitch = (owr + (K + TC - 1) / TC * TC + 3 + 3) & ~3;
    p.dpitch = owr;
    const int64_t red = 256 * (TC + 1) * 4;
    auto bytes = [&](int bh) {
        return std::max((static_cast<int64_t>(bh + K - 1) * p.xpitch + static_cast<int64_t>(bh) * p.dpitch) * 4, red);
    };
    // bands of dy rows within 48 KiB of LDS: the kernel's 168 VGPRs allow three
    // workgroups per CU, and three such bands still fit its 160 KiB, so the
    // staging of one image overlaps the arithmetic of the other workgroups
    // (larger bands also re-stage fewer halo rows; 24 KiB bands measured
    // 3-9 % slower at 48 x 48 and 64 x 64)
    int bh = g.oh;
    while (bh > 8 && bytes(bh) > 48 * 1024) bh = (bh + 1) / 2;
    if (bytes(bh) > 64 * 1024) return false;
    p.nbands = (g.oh + bh - 1) / bh;
    p.BH = (g.oh + p.nbands - 1) / p.nbands;
    p.xrows = p.BH + K - 1;
    p.lds_bytes = static_cast<int>(bytes(p.BH));
    // image chunks: about 2048 workgroups in total
    int NC = std::max(1, (2048 + g.ic * p.nbands - 1) / (g.ic * p.nbands));
    NC = std::min(NC, g.n);
    p.npc = (g.n + NC - 1) / NC;
    p.NC = (g.n + p.npc - 1) / p.npc;
    return true;
}

template <typename T, int K>
int run_lkw(const Geo &g, const LkwPlan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    LkwArgs<T> a{};
    a.x = static_cast<const T *>(x);
    a.dy = static_cast<const T *>(dy);
    a.ws = static_cast<float *>(ws);
    a.C = g.ic;
    a.IH = g.ih;
    a.IW = g.iw;
    a.OH = g.oh;
    a.OW = g.ow;
    a.P = g.ph;
    a.N = g.n;
    a.NC = p.NC;
    a.npc = p.npc;
    a.BH = p.BH;
    a.nbands = p.nbands;
    a.xpitch = p.xpitch;
    a.xrows = p.xrows;
    a.dpitch = p.dpitch;
    a.fxp = make_fastdiv(p.xpitch, static_cast<uint64_t>(p.xrows) * p.xpitch + 256);
    a.fdp = make_fastdiv(p.dpitch, static_cast<uint64_t>(p.BH) * p.dpitch + 256);
    a.vx = g.iw % Vec<T>::N == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
    a.vd = g.ow % Vec<T>::N == 0 && reinterpret_cast<uintptr_t>(dy) % 16 == 0;
    a.fxv = make_fastdiv(std::max(g.iw / Vec<T>::N, 1), static_cast<uint64_t>(p.xrows) * (g.iw / Vec<T>::N + 1) + 1024);
    a.fdv = make_fastdiv(std::max(g.ow / Vec<T>::N, 1), static_cast<uint64_t>(p.BH) * (g.ow / Vec<T>::N + 1) + 1024);
    hipLaunchKernelGGL((lk_bwdw_kernel<T, K, kTR, lkw_tc(K), kLkwSeg>), dim3(g.ic * p.NC * p.nbands), dim3(256),
                       p.lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T>
int lk_bwdw_t(const Geo &g, const void *x, const void *dy, void *ws, hipStream_t s) {
    LkwPlan p;
    if (!plan_lkw(g, g.kh, p)) return kErrUnsupported;
    if (g.kh == 7) return run_lkw<T, 7>(g, p, x, dy, ws, s);
    if (g.kh == 13) return run_lkw<T, 13>(g, p, x, dy, ws, s);
    return run_lkw<T, 31>(g, p, x, dy, ws, s);
}

}  // namespace

bool largek_bwdw_fits(const Geo &g) {
    if (g.kh != g.kw || (g.kh != 7 && g.kh != 13 && g.kh != 31)) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.ph != g.pw || g.mult != 1) return false;
    LkwPlan p;
    return plan_lkw(g, g.kh, p);
}

int largek_bwd_weight_chunks(const Geo &g) {
    LkwPlan p;
    return plan_lkw(g, g.kh, p) ? p.NC * p.nbands : 0;
}

int largek_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return lk_bwdw_t<float>(g, x, dy, ws, s);
        case 1: return lk_bwdw_t<__half>(g, x, dy, ws, s);
        default: return lk_bwdw_t<bf16_t>(g, x, dy, ws, s);
    }
}

namespace {
}  // namespace

bool largek_fits(const Geo &g, int pass) {
    if (g.kh != g.kw || (g.kh != 7 && g.kh != 13 && g.kh != 31)) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.ph != g.pw) return false;
    if (pass == 1 && (g.mult != 1 || g.ph > g.kh - 1)) return false;
    LkPlan p;
    return pass == 1 ? plan_lk(g.ih, g.iw, g.kh, p) : plan_lk(g.oh, g.ow, g.kh, p);
}

int largek_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return lk_fwd_t<float>(g, x, w, b, y, s);
        case 1: return lk_fwd_t<__half>(g, x, w, b, y, s);
        default: return lk_fwd_t<bf16_t>(g, x, w, b, y, s);
    }
}

int largek_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s) {
    switch (dtype) {
        case 0: return lk_bwdin_t<float>(g, dy, w, dx, s);
        case 1: return lk_bwdin_t<__half>(g, dy, w, dx, s);
        default: return lk_bwdin_t<bf16_t>(g, dy, w, dx, s);
    }
}

}  // namespace dw
