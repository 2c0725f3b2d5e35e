// dw_largek_mfma.hip -- large-kernel depthwise forward and grad-input for
// 16-bit I/O on the gfx950 matrix cores (k = 7, 13, 31; stride 1, dilation 1;
// planes of at most 64 x 64 outputs).
//
// The MegEngine large-kernel depthwise article turns depthwise convolution
// into an implicit batched GEMM (section on ImplicitBatchedGEMM) and notes
// that its flop inflation shrinks as the kernel grows toward the input size.
// Here the GEMM is built per plane from one kernel row at a time: with
// zero-padded input rows X[r] (r = oh + i) the output tile is
//   y[oh][ow] = sum_i sum_c T_i[ow][c] * X[oh + i][c],
//   T_i[ow][c] = w[i][c - ow]   (0 <= c - ow < k, else 0),
// a banded Toeplitz matrix of filter row i.  A 32 x 32 output tile reads the
// 32 + k - 1 input columns of its window, padded to KP = 16 * KPS, so the
// matrix cores do KP / k times the useful multiply-adds (2.06x at k = 31)
// at 16x the fp32 vector rate.  Products of 16-bit values are exact and the
// sums are fp32 (v_mfma_f32_32x32x16_{f16,bf16}).
//
// Roles in D = A * B (M = 32 output columns, N = 32 output rows, K = 16
// window columns per instruction):
//   A[m][kk] = T_i[m][kk]: lane l reads the 8 filter values
//              w[i][16 s + 8 (l / 32) + e - l % 32], e < 8, from a zero-padded
//              copy of filter row i in LDS (two copies shifted by one element,
//              so every run of 8 starts on a 4-byte boundary);
//   B[kk][n] = X[32 mt + n + i][32 nt + 16 s + kk]: lane l reads 8 adjacent
//              columns of input row 32 mt + l % 32 + i -- one aligned 16-byte
//              LDS read;
//   D: register r of lane l is output (32 mt + l % 32, 32 nt + 8 (r / 4)
//      + 4 (l / 32) + r % 4), so a lane stores runs of 4 adjacent outputs.
// A workgroup (4 waves) serves one channel and 4 / MT images, one wave per
// (image, 32-row output tile): the filter table is built once, the waves stage
// the images' zero-padded planes in LDS together, and each wave accumulates its
// row tile's NT column tiles over the k kernel rows (one B read feeds the NT
// tiles it overlaps).  Two 32-row tiles of a 64-row plane on two waves keep
// three workgroups (12 waves) per CU where whole planes per wave fit one.
// Grad-input is the same correlation of dy with the filter flipped in both
// axes and padding k - 1 - pad.
#include "dw_common.hpp"
#include "dw_internal.hpp"

namespace dw {
namespace {

typedef _Float16 f16x8_v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x16_v __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));

constexpr int kZoff = 31;  // zero columns left of a filter row in the table (largest tile column)

template <typename T> struct Mfma;
template <> struct Mfma<__half> {
    static __device__ __forceinline__ f32x16_v run(u32x4_v a, u32x4_v b, f32x16_v c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_v, a), __builtin_bit_cast(f16x8_v, b),
                                                      c, 0, 0, 0);
    }
};
template <> struct Mfma<bf16_t> {
    static __device__ __forceinline__ f32x16_v run(u32x4_v a, u32x4_v b, f32x16_v c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                       __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
    }
};

template <typename T> struct LkmArgs {
    const T *in;   // forward: x; grad-input: dy
    const T *w;
    const T *b;    // bias (forward) or NULL
    T *out;        // y or dx
    int N;         // images
    int IH, IW;    // input plane of this pass
    int OH, OW;    // output plane of this pass
    int P;         // top/left zero padding of this pass
    int C;         // output channels of this pass (planes per image)
    int Cin;       // input channels of this pass
    int mult;      // output channels per input channel
    int ngroups;   // workgroups per channel, each walking gpc image groups
    int gpc;       // image groups (one image per wave of a workgroup) per workgroup
    int ngtot;     // image groups per channel
    int vin;       // input rows are whole 16-byte vectors (and aligned)
    int pre;       // vin, and a group's planes fit the prefetch registers (2 NT vectors a thread)
    int vout;      // output rows are whole 4-element runs (and 8-byte aligned)
};

// LDS geometry of one (K, KPS, MT, NT) instance: the filter table plus one
// input tile per wave, as many waves (up to 4) as fit the LDS budget.
template <int K, int KPS, int MT, int NT> struct LkmGeo {
    static constexpr int QD = 8 * KPS + 20;              // dwords per copy of a filter row (even)
    static constexpr int W1 = K * QD + 17;               // dword offset of copy 1 (17 banks from copy 0)
    static constexpr int XR = 32 * MT + K - 1;           // staged input rows
    static constexpr int XC = 32 * (NT - 1) + 16 * KPS;  // staged input columns
    static constexpr int XP = XC + 8;                    // row pitch (halves): an odd multiple of 16 bytes mod 32
    static constexpr int table_bytes = ((W1 + K * QD) * 4 + 15) / 16 * 16;
    static constexpr int tile_halves = XR * XP;
    static constexpr int IPG = 4 / MT;                   // images per workgroup: one wave per (image, row tile)
    static constexpr int lds_bytes = table_bytes + IPG * tile_halves * 2;
    static_assert(lds_bytes <= kLdsCap, "tiles exceed the LDS budget");
};

template <typename T, int K, int KPS, int MT, int NT, bool FLIP>
__global__ __launch_bounds__(256) void lk_mfma_kernel(LkmArgs<T> a) {
    using G = LkmGeo<K, KPS, MT, NT>;
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *wtab = reinterpret_cast<uint32_t *>(smem);  // copy 0 [i][QD], copy 1 at W1
    uint16_t *tiles = reinterpret_cast<uint16_t *>(smem + G::table_bytes);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int img = wave / MT;     // image of the workgroup's group this wave serves
    const int mt = wave - img * MT;  // its 32-row output tile
    const int c = blockIdx.x / a.ngroups;  // output plane channel of this pass
    const int g0 = (blockIdx.x - c * a.ngroups) * a.gpc;
    const int g1 = min(g0 + a.gpc, a.ngtot);

    // 1. filter table: copy q (0, 1) of row i holds, in dword d, the 16-bit
    //    values of padded positions 2d + q and 2d + q + 1, where padded
    //    position p is w[i][p - kZoff] (flipped for grad-input), 0 outside.
    const uint16_t *wr = reinterpret_cast<const uint16_t *>(a.w) + static_cast<int64_t>(c) * K * K;
    for (int e = tid; e < 2 * K * G::QD; e += 256) {
        const int q = e / (K * G::QD);
        const int rem = e - q * K * G::QD;
        const int i = rem / G::QD;
        const int d = rem - i * G::QD;
        uint32_t v = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int j = 2 * d + q + u - kZoff;
            if (j >= 0 && j < K) {
                const uint16_t bits = FLIP ? wr[(K - 1 - i) * K + (K - 1 - j)] : wr[i * K + j];
                v |= static_cast<uint32_t>(bits) << (16 * u);
            }
        }
        wtab[q * G::W1 + rem] = v;
    }

    // 2. per image group, the padded input planes: tile[r][col] = in[r - P][col - P],
    //    0 outside (the zeros are written once: every group writes the same
    //    interior positions); the MT waves of an image stage its plane together.
    //    With whole 16-byte rows that fit the registers (planes no larger than
    //    the output tiles) the next group's planes are loaded into registers
    //    while the matrix cores work on this one.
    {
        uint4 *z = reinterpret_cast<uint4 *>(tiles);
        for (int e = tid; e < G::IPG * G::tile_halves / 8; e += 256) z[e] = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();  // zeros before any plane data
    const int cin = FLIP ? c : c / a.mult;
    const int64_t plane = static_cast<int64_t>(a.IH) * a.IW;
    const int64_t istride = static_cast<int64_t>(a.Cin) * plane;  // one image
    const uint16_t *ib = reinterpret_cast<const uint16_t *>(a.in) + cin * plane;
    // vector v = tid + 256 k of a group: image v / nvec, row, 8-column run; its
    // offset from the group's first plane and its place in the tiles
    constexpr int NV = 2 * NT;  // IPG * 32 MT * 32 NT halves / 8 per vector / 256 threads
    const int vpr = a.IW / 8, nvec = a.IH * vpr;
    int64_t goff[NV];
    int loff[NV], vidx[NV];
    if (a.pre) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int v = tid + 256 * k;
            const int im = v / nvec;
            const int vv = v - im * nvec;
            const int r = vv / vpr;
            const int c8 = (vv - r * vpr) * 8;
            vidx[k] = v;
            goff[k] = im * istride + static_cast<int64_t>(r) * a.IW + c8;
            loff[k] = im * G::tile_halves + (r + a.P) * G::XP + c8 + a.P;
        }
    }
    uint4 raw[NV];
    auto load_group = [&](int gi) {
        const int nv = min(G::IPG, a.N - gi * G::IPG) * nvec;
        const uint16_t *src = ib + static_cast<int64_t>(gi) * G::IPG * istride;
#pragma unroll
        for (int k = 0; k < NV; ++k)
            if (vidx[k] < nv) raw[k] = *reinterpret_cast<const uint4 *>(src + goff[k]);
    };
    if (a.pre && g0 < g1) load_group(g0);

    const int m = lane & 31;
    const int h = lane >> 5;
    const float bias = (!FLIP && a.b) ? to_f32(a.b[c]) : 0.f;
    const uint16_t *xt = tiles + img * G::tile_halves;
    for (int gi = g0; gi < g1; ++gi) {
        const int n0 = gi * G::IPG;
        const int nimg = min(G::IPG, a.N - n0);
        if (a.pre) {
            const int nv = nimg * nvec;
#pragma unroll
            for (int k = 0; k < NV; ++k)
                if (vidx[k] < nv) {
                    uint16_t *d = tiles + loff[k];
                    const uint32_t wd[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) d[e] = static_cast<uint16_t>(wd[e >> 1] >> ((e & 1) * 16));
                }
        } else if (a.vin) {
            const uint16_t *src = ib + static_cast<int64_t>(n0) * istride;
            for (int v = tid; v < nimg * nvec; v += 256) {
                const int im = v / nvec;
                const int vv = v - im * nvec;
                const int r = vv / vpr;
                const int c8 = (vv - r * vpr) * 8;
                const uint4 rv = *reinterpret_cast<const uint4 *>(src + im * istride + static_cast<int64_t>(r) * a.IW + c8);
                uint16_t *d = tiles + im * G::tile_halves + (r + a.P) * G::XP + c8 + a.P;
                const uint32_t wd[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) d[e] = static_cast<uint16_t>(wd[e >> 1] >> ((e & 1) * 16));
            }
        } else {
            const uint16_t *src = ib + static_cast<int64_t>(n0) * istride;
            for (int e = tid; e < nimg * a.IH * a.IW; e += 256) {
                const int im = e / (a.IH * a.IW);
                const int ee = e - im * a.IH * a.IW;
                const int r = ee / a.IW;
                const int col = ee - r * a.IW;
                tiles[im * G::tile_halves + (r + a.P) * G::XP + col + a.P] = src[im * istride + ee];
            }
        }
        __syncthreads();
        if (a.pre && gi + 1 < g1) load_group(gi + 1);
        const int n = n0 + img;
        if (n < a.N) {
            // 3. k kernel rows x KPS window steps x (MT x NT) tiles of MFMAs
            f32x16_v acc[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[nt][r] = 0.f;
#pragma unroll 1
            for (int i = 0; i < K; ++i) {
                u32x4_v af[KPS];
#pragma unroll
                for (int s = 0; s < KPS; ++s) {
                    const int t = 16 * s + 8 * h - m + kZoff;  // first padded position of this lane's run
                    const int q = t & 1;
                    const uint32_t *p = wtab + q * G::W1 + i * G::QD + ((t - q) >> 1);
                    af[s] = u32x4_v{p[0], p[1], p[2], p[3]};
                }
#pragma unroll
                for (int sp = 0; sp < KPS + 2 * (NT - 1); ++sp) {
                    const u32x4_v bf =
                        *reinterpret_cast<const u32x4_v *>(xt + (32 * mt + m + i) * G::XP + 16 * sp + 8 * h);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const int s = sp - 2 * nt;
                        if (s >= 0 && s < KPS) acc[nt] = Mfma<T>::run(af[s], bf, acc[nt]);
                    }
                }
            }
            // 4. store: lane holds, per tile and r4, outputs (32 mt + m, 32 nt + 8 r4 + 4 h + 0..3)
            T *op = a.out + (static_cast<int64_t>(n) * a.C + c) * a.OH * a.OW;
            const int oh = 32 * mt + m;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int ow = 32 * nt + 8 * r4 + 4 * h;
                    const float v0 = acc[nt][4 * r4] + bias, v1 = acc[nt][4 * r4 + 1] + bias;
                    const float v2 = acc[nt][4 * r4 + 2] + bias, v3 = acc[nt][4 * r4 + 3] + bias;
                    T *dst = op + oh * a.OW + ow;
                    if (oh >= a.OH) continue;
                    if (a.vout && ow + 4 <= a.OW) {
                        *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2<T>(v0, v1), pack2<T>(v2, v3));
                    } else {
                        const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (ow + q < a.OW) dst[q] = from_f32<T>(vv[q]);
                    }
                }
        }
        __syncthreads();  // the tiles are read before the next group overwrites them
    }
}

// Window steps of 16 columns a 32-column output tile needs: 32 + K - 1 columns.
constexpr int kps_of(int K) { return (32 + K - 1 + 15) / 16; }

template <typename T, int K, bool FLIP, int MT, int NT>
int run_lkm_t(const LkmArgs<T> &a, hipStream_t s) {
    constexpr int KPS = kps_of(K);
    using G = LkmGeo<K, KPS, MT, NT>;
    LkmArgs<T> b = a;
    // image groups per channel, walked by about 2048 workgroups in all where the
    // matrix work per group is short (k = 7, 13: the next group's loads then
    // overlap it); at k = 31 one group per workgroup measured faster
    b.ngtot = (a.N + G::IPG - 1) / G::IPG;
    const int64_t all = static_cast<int64_t>(a.C) * b.ngtot;
    const int gpc = K > 13 ? 1 : static_cast<int>(std::max<int64_t>(1, all / 2048));
    b.ngroups = (b.ngtot + gpc - 1) / gpc;
    b.gpc = (b.ngtot + b.ngroups - 1) / b.ngroups;
    b.pre = a.vin && G::IPG * a.IH * (a.IW / 8) <= 256 * 2 * NT;
    const dim3 grid(static_cast<unsigned>(a.C * b.ngroups));
    hipLaunchKernelGGL((lk_mfma_kernel<T, K, KPS, MT, NT, FLIP>), grid, dim3(256), G::lds_bytes, s, b);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, int K, bool FLIP>
int run_lkm_k(const LkmArgs<T> &a, hipStream_t s) {
    const int MT = (a.OH + 31) / 32, NT = (a.OW + 31) / 32;
    if (MT == 1 && NT == 1) return run_lkm_t<T, K, FLIP, 1, 1>(a, s);
    if (MT == 1) return run_lkm_t<T, K, FLIP, 1, 2>(a, s);
    if (NT == 1) return run_lkm_t<T, K, FLIP, 2, 1>(a, s);
    return run_lkm_t<T, K, FLIP, 2, 2>(a, s);
}

template <typename T, bool FLIP>
int run_lkm(const LkmArgs<T> &a, int K, hipStream_t s) {
    if (K == 7) return run_lkm_k<T, 7, FLIP>(a, s);
    if (K == 13) return run_lkm_k<T, 13, FLIP>(a, s);
    return run_lkm_k<T, 31, FLIP>(a, s);
}

template <typename T>
void fill_io(LkmArgs<T> &a) {
    a.vin = a.IW % 8 == 0 && reinterpret_cast<uintptr_t>(a.in) % 16 == 0;
    a.vout = a.OW % 4 == 0 && reinterpret_cast<uintptr_t>(a.out) % 8 == 0;
}

template <typename T>
int lkm_fwd_t(const Geo &g, const void *x, const void *w, const void *b, void *y, hipStream_t s) {
    LkmArgs<T> a{};
    a.in = static_cast<const T *>(x);
    a.w = static_cast<const T *>(w);
    a.b = static_cast<const T *>(b);
    a.out = static_cast<T *>(y);
    a.N = g.n;
    a.IH = g.ih;
    a.IW = g.iw;
    a.OH = g.oh;
    a.OW = g.ow;
    a.P = g.ph;
    a.C = g.oc;
    a.Cin = g.ic;
    a.mult = g.mult;
    fill_io(a);
    return run_lkm<T, false>(a, g.kh, s);
}

template <typename T>
int lkm_bwdin_t(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t s) {
    LkmArgs<T> a{};
    a.in = static_cast<const T *>(dy);
    a.w = static_cast<const T *>(w);
    a.out = static_cast<T *>(dx);
    a.N = g.n;
    a.IH = g.oh;
    a.IW = g.ow;
    a.OH = g.ih;
    a.OW = g.iw;
    a.P = g.kh - 1 - g.ph;
    a.C = g.ic;
    a.Cin = g.oc;
    a.mult = 1;
    fill_io(a);
    return run_lkm<T, true>(a, g.kh, s);
}

}  // namespace

// 16-bit I/O, k = 7 / 13 / 31 square, stride 1, dilation 1, symmetric padding,
// an output plane of at most 64 x 64 and an input plane that fits the staged
// tile (pad + input extent <= tile extent).  Grad-input needs multiplier 1 and
// pad <= k - 1 (its own padding k - 1 - pad is then >= 0).
bool largek_mfma_fits(const Geo &g, int pass, int dtype) {
    if (dtype == 0) return false;
    if (g.kh != g.kw || (g.kh != 7 && g.kh != 13 && g.kh != 31)) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.ph != g.pw) return false;
    if (pass == 1 && (g.mult != 1 || g.ph > g.kh - 1)) return false;
    const int OH = pass == 1 ? g.ih : g.oh, OW = pass == 1 ? g.iw : g.ow;
    const int IH = pass == 1 ? g.oh : g.ih, IW = pass == 1 ? g.ow : g.iw;
    const int P = pass == 1 ? g.kh - 1 - g.ph : g.ph;
    if (OH > 64 || OW > 64) return false;
    const int MT = (OH + 31) / 32, NT = (OW + 31) / 32;
    const int XR = 32 * MT + g.kh - 1, XC = 32 * (NT - 1) + 16 * kps_of(g.kh);
    // every staged input element lands inside the tile
    return IH + P <= XR && IW + P <= XC;
}

int largek_mfma_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s) {
    return dtype == 1 ? lkm_fwd_t<__half>(g, x, w, b, y, s) : lkm_fwd_t<bf16_t>(g, x, w, b, y, s);
}

int largek_mfma_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s) {
    return dtype == 1 ? lkm_bwdin_t<__half>(g, dy, w, dx, s) : lkm_bwdin_t<bf16_t>(g, dy, w, dx, s);
}

namespace {

typedef float f32x4_v __attribute__((ext_vector_type(4)));

template <typename T> struct Mfma16;
template <> struct Mfma16<__half> {
    static __device__ __forceinline__ f32x4_v run(u32x4_v a, u32x4_v b, f32x4_v c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_v, a), __builtin_bit_cast(f16x8_v, b),
                                                      c, 0, 0, 0);
    }
};
template <> struct Mfma16<bf16_t> {
    static __device__ __forceinline__ f32x4_v run(u32x4_v a, u32x4_v b, f32x4_v c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                       __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
    }
};

// ---------------------------------------------------------------- forward, 16 x 16 tiles
// The same Toeplitz product on v_mfma_f32_16x16x32_{f16,bf16}: 16 x 16 output
// tiles (M = 16 output columns, N = 16 output rows, K = 32 window columns per
// instruction).  A 16-column tile reads 16 + k - 1 window columns, padded to
// 32 KPS: 32 for k = 7, 13 (4.6x and 2.5x the useful multiply-adds against
// 6.9x and 3.7x with 32-column tiles) and 64 for k = 31 (2.06x, the same), and
// 48-wide planes take 3 x 3 tiles instead of four 32 x 32 ones that are 44 %
// empty.  Measured on N64 C384: ~10 % faster than the 32 x 32 tiles at k = 7
// on 48 and 64 planes, about even at k = 13 and 2.5-3x slower at k = 31 (twice
// the LDS reads per multiply-add), so the default only at k = 7.
//   A[m][kk] = T_i[m][kk]: lane l reads the 8 filter values of window columns
//              32 s + 8 (l / 16) .. for output column l % 16 from the table;
//   B[kk][n] = X[16 mt + n + i][16 nt + 32 s + kk]: lane l reads 8 adjacent
//              columns of input row 16 mt + l % 16 + i (one 16-byte LDS read;
//              tiles whose windows start at the same column share it);
//   D: register r of lane l is output (16 mt + l % 16, 16 nt + 4 (l / 16) + r).
// A workgroup serves one channel and IPG images, one wave per (image, 16-row
// tile), and walks several image groups, loading the next group's planes into
// registers during the matrix work.
template <int K> constexpr int kps16_of() { return (16 + K - 1 + 31) / 32; }

template <typename T> struct Lkm16Args {
    const T *in, *w, *b;
    T *out;
    int N, IH, IW, OH, OW, P, C, Cin, mult;
    int MT, NT;          // 16-row / 16-column output tiles of a plane (NT <= 4)
    int IPG;             // images per group (one wave per image and row tile)
    int XR, XP;          // staged rows, row pitch (halves) of an input plane
    int ngroups, gpc, ngtot;
    int vin, vout, pre;
};

template <typename T, int K, bool FLIP>
__global__ __launch_bounds__(256) void lk_mfma16_kernel(Lkm16Args<T> a) {
    constexpr int KPS = kps16_of<K>();
    constexpr int QD = 16 * KPS + 20;   // dwords per copy of a filter row (even)
    constexpr int W1 = K * QD + 17;     // dword offset of copy 1 (17 banks from copy 0)
    constexpr int table_bytes = ((W1 + K * QD) * 4 + 15) / 16 * 16;
    constexpr int NTM = 4;              // largest column-tile count (planes up to 64 wide)
    constexpr int NV = 2;               // prefetch vectors per thread: IPG * 16 MT * 16 NT / 8 <= 2 * threads
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *wtab = reinterpret_cast<uint32_t *>(smem);  // copy 0 [i][QD], copy 1 at W1
    uint16_t *tiles = reinterpret_cast<uint16_t *>(smem + table_bytes);
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int img = wave / a.MT;
    const int mt = wave - img * a.MT;
    const int c = blockIdx.x / a.ngroups;
    const int g0 = (blockIdx.x - c * a.ngroups) * a.gpc;
    const int g1 = min(g0 + a.gpc, a.ngtot);
    const int tile_halves = a.XR * a.XP;

    // 1. filter table: copy q holds, in dword d of row i, padded positions
    //    2d + q and 2d + q + 1 (position p is w[i][p - kZoff], flipped for grad-input)
    const uint16_t *wr = reinterpret_cast<const uint16_t *>(a.w) + static_cast<int64_t>(c) * K * K;
    for (int e = tid; e < 2 * K * QD; e += nthr) {
        const int q = e / (K * QD);
        const int rem = e - q * K * QD;
        const int i = rem / QD;
        const int d = rem - i * QD;
        uint32_t v = 0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int j = 2 * d + q + u - kZoff;
            if (j >= 0 && j < K) {
                const uint16_t bits = FLIP ? wr[(K - 1 - i) * K + (K - 1 - j)] : wr[i * K + j];
                v |= static_cast<uint32_t>(bits) << (16 * u);
            }
        }
        wtab[q * W1 + rem] = v;
    }
    // 2. zero planes once; every group writes the same interior positions
    for (int e = tid; e < a.IPG * tile_halves / 8; e += nthr)
        reinterpret_cast<uint4 *>(tiles)[e] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    const int cin = FLIP ? c : c / a.mult;
    const int64_t plane = static_cast<int64_t>(a.IH) * a.IW;
    const int64_t istride = static_cast<int64_t>(a.Cin) * plane;
    const uint16_t *ib = reinterpret_cast<const uint16_t *>(a.in) + cin * plane;
    const int vpr = a.IW / 8, nvec = a.IH * vpr;
    int64_t goff[NV];
    int loff[NV], vidx[NV];
    if (a.pre) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int v = tid + nthr * k;
            const int im = v / nvec;
            const int vv = v - im * nvec;
            const int r = vv / vpr;
            const int c8 = (vv - r * vpr) * 8;
            vidx[k] = v;
            goff[k] = im * istride + static_cast<int64_t>(r) * a.IW + c8;
            loff[k] = im * tile_halves + (r + a.P) * a.XP + c8 + a.P;
        }
    }
    uint4 raw[NV];
    auto load_group = [&](int gi) {
        const int nv = min(a.IPG, a.N - gi * a.IPG) * nvec;
        const uint16_t *src = ib + static_cast<int64_t>(gi) * a.IPG * istride;
#pragma unroll
        for (int k = 0; k < NV; ++k)
            if (vidx[k] < nv) raw[k] = *reinterpret_cast<const uint4 *>(src + goff[k]);
    };
    if (a.pre && g0 < g1) load_group(g0);

    const int m = lane & 15, g4 = lane >> 4;
    const float bias = (!FLIP && a.b) ? to_f32(a.b[c]) : 0.f;
    const uint16_t *xt = tiles + img * tile_halves;
    for (int gi = g0; gi < g1; ++gi) {
        const int n0 = gi * a.IPG;
        const int nimg = min(a.IPG, a.N - n0);
        if (a.pre) {
            const int nv = nimg * nvec;
#pragma unroll
            for (int k = 0; k < NV; ++k)
                if (vidx[k] < nv) {
                    uint16_t *d = tiles + loff[k];
                    const uint32_t wd[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) d[e] = static_cast<uint16_t>(wd[e >> 1] >> ((e & 1) * 16));
                }
        } else {
            const uint16_t *src = ib + static_cast<int64_t>(n0) * istride;
            for (int e = tid; e < nimg * a.IH * a.IW; e += nthr) {
                const int im = e / (a.IH * a.IW);
                const int ee = e - im * a.IH * a.IW;
                const int r = ee / a.IW;
                const int col = ee - r * a.IW;
                tiles[im * tile_halves + (r + a.P) * a.XP + col + a.P] = src[im * istride + ee];
            }
        }
        __syncthreads();
        if (a.pre && gi + 1 < g1) load_group(gi + 1);
        const int n = n0 + img;
        if (img < nimg) {
            // 3. kernel rows x window positions x column tiles
            f32x4_v acc[NTM];
#pragma unroll
            for (int nt = 0; nt < NTM; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[nt][r] = 0.f;
#pragma unroll 1
            for (int i = 0; i < K; ++i) {
                u32x4_v af[KPS];
#pragma unroll
                for (int s2 = 0; s2 < KPS; ++s2) {
                    const int t = 32 * s2 + 8 * g4 - m + kZoff;  // first padded position of this lane's run
                    const int q = t & 1;
                    const uint32_t *p = wtab + q * W1 + i * QD + ((t - q) >> 1);
                    af[s2] = u32x4_v{p[0], p[1], p[2], p[3]};
                }
                // window position p (16 columns): tile nt, step s with nt + 2 s = p
#pragma unroll
                for (int p = 0; p < NTM + 2 * (KPS - 1); ++p) {
                    if (p >= a.NT + 2 * (KPS - 1)) break;
                    const u32x4_v bf =
                        *reinterpret_cast<const u32x4_v *>(xt + (16 * mt + m + i) * a.XP + 16 * p + 8 * g4);
#pragma unroll
                    for (int nt = 0; nt < NTM; ++nt) {
                        const int d = p - nt;
                        if (nt < a.NT && d >= 0 && (d & 1) == 0 && (d >> 1) < KPS)
                            acc[nt] = Mfma16<T>::run(af[d >> 1], bf, acc[nt]);
                    }
                }
            }
            // 4. store: lane holds outputs (16 mt + m, 16 nt + 4 g4 + 0..3)
            T *op = a.out + (static_cast<int64_t>(n) * a.C + c) * a.OH * a.OW;
            const int oh = 16 * mt + m;
            if (oh < a.OH) {
#pragma unroll
                for (int nt = 0; nt < NTM; ++nt) {
                    if (nt >= a.NT) break;
                    const int ow = 16 * nt + 4 * g4;
                    const float v0 = acc[nt][0] + bias, v1 = acc[nt][1] + bias;
                    const float v2 = acc[nt][2] + bias, v3 = acc[nt][3] + bias;
                    T *dst = op + oh * a.OW + ow;
                    if (a.vout && ow + 4 <= a.OW) {
                        *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2<T>(v0, v1), pack2<T>(v2, v3));
                    } else {
                        const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (ow + q < a.OW) dst[q] = from_f32<T>(vv[q]);
                    }
                }
            }
        }
        __syncthreads();  // the planes are read before the next group overwrites them
    }
}

template <typename T, int K, bool FLIP>
int run_lkm16(Lkm16Args<T> a, hipStream_t s) {
    constexpr int KPS = kps16_of<K>();
    constexpr int QD = 16 * KPS + 20;
    constexpr int table_bytes = ((K * QD + 17 + K * QD) * 4 + 15) / 16 * 16;
    a.MT = (a.OH + 15) / 16;
    a.NT = (a.OW + 15) / 16;
    a.IPG = std::max(1, 4 / a.MT);
    a.XR = 16 * a.MT + K - 1;
    a.XP = 16 * (a.NT - 1) + 32 * KPS + 8;
    const int threads = 64 * a.MT * a.IPG;
    const int lds = table_bytes + a.IPG * a.XR * a.XP * 2;
    if (a.NT > 4 || a.MT > 4 || lds > kLdsCap) return kErrUnsupported;
    a.ngtot = (a.N + a.IPG - 1) / a.IPG;
    const int64_t all = static_cast<int64_t>(a.C) * a.ngtot;
    const int gpc = K > 13 ? 1 : static_cast<int>(std::max<int64_t>(1, all / 2048));
    a.ngroups = (a.ngtot + gpc - 1) / gpc;
    a.gpc = (a.ngtot + a.ngroups - 1) / a.ngroups;
    a.pre = a.vin && a.IPG * a.IH * (a.IW / 8) <= 2 * threads;
    hipLaunchKernelGGL((lk_mfma16_kernel<T, K, FLIP>), dim3(static_cast<unsigned>(a.C * a.ngroups)), dim3(threads), lds, s,
                       a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, bool FLIP>
int run_lkm16_k(const Lkm16Args<T> &a, int K, hipStream_t s) {
    if (K == 7) return run_lkm16<T, 7, FLIP>(a, s);
    if (K == 13) return run_lkm16<T, 13, FLIP>(a, s);
    return run_lkm16<T, 31, FLIP>(a, s);
}

template <typename T>
void fill_io16(Lkm16Args<T> &a) {
    a.vin = a.IW % 8 == 0 && reinterpret_cast<uintptr_t>(a.in) % 16 == 0;
    a.vout = a.OW % 4 == 0 && reinterpret_cast<uintptr_t>(a.out) % 8 == 0;
}

template <typename T>
int lkm16_fwd_t(const Geo &g, const void *x, const void *w, const void *b, void *y, hipStream_t s) {
    Lkm16Args<T> a{};
    a.in = static_cast<const T *>(x);
    a.w = static_cast<const T *>(w);
    a.b = static_cast<const T *>(b);
    a.out = static_cast<T *>(y);
    a.N = g.n;
    a.IH = g.ih;
    a.IW = g.iw;
    a.OH = g.oh;
    a.OW = g.ow;
    a.P = g.ph;
    a.C = g.oc;
    a.Cin = g.ic;
    a.mult = g.mult;
    fill_io16(a);
    return run_lkm16_k<T, false>(a, g.kh, s);
}

template <typename T>
int lkm16_bwdin_t(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t s) {
    Lkm16Args<T> a{};
    a.in = static_cast<const T *>(dy);
    a.w = static_cast<const T *>(w);
    a.out = static_cast<T *>(dx);
    a.N = g.n;
    a.IH = g.oh;
    a.IW = g.ow;
    a.OH = g.ih;
    a.OW = g.iw;
    a.P = g.kh - 1 - g.ph;
    a.C = g.ic;
    a.Cin = g.oc;
    a.mult = 1;
    fill_io16(a);
    return run_lkm16_k<T, true>(a, g.kh, s);
}

}  // namespace

// The same conditions on 16 x 16 tiles (16-row / 16-column tiles of an output
// plane of at most 64 x 64, the input inside the staged window).
bool largek_mfma16_fits(const Geo &g, int pass, int dtype) {
    if (dtype == 0) return false;
    if (g.kh != g.kw || (g.kh != 7 && g.kh != 13 && g.kh != 31)) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.ph != g.pw) return false;
    if (pass == 1 && (g.mult != 1 || g.ph > g.kh - 1)) return false;
    const int OH = pass == 1 ? g.ih : g.oh, OW = pass == 1 ? g.iw : g.ow;
    const int IH = pass == 1 ? g.oh : g.ih, IW = pass == 1 ? g.ow : g.iw;
    const int P = pass == 1 ? g.kh - 1 - g.ph : g.ph;
    if (OH < 1 || OW < 1 || OH > 64 || OW > 64) return false;
    const int MT = (OH + 15) / 16, NT = (OW + 15) / 16;
    const int kps = (16 + g.kh - 1 + 31) / 32;
    const int XR = 16 * MT + g.kh - 1, XC = 16 * (NT - 1) + 32 * kps;
    return IH + P <= XR && IW + P <= XC;
}

int largek_mfma16_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s) {
    return dtype == 1 ? lkm16_fwd_t<__half>(g, x, w, b, y, s) : lkm16_fwd_t<bf16_t>(g, x, w, b, y, s);
}

int largek_mfma16_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s) {
    return dtype == 1 ? lkm16_bwdin_t<__half>(g, dy, w, dx, s) : lkm16_bwdin_t<bf16_t>(g, dy, w, dx, s);
}

// ---------------------------------------------------------------- grad-weight
// dw[i][j] = sum_{n, oh, c} X[oh + i][c] * dz[oh][c - j], with X the
// zero-padded input rows and dz[oh][u] = dy[oh][u] for 0 <= u < ow, else 0:
// a contraction over (image, dy row, window column) with M = kernel row i and
// N = kernel column j, one 32 x 32 output tile (k <= 32).  Per dy row and
// window step of 16 columns one v_mfma_f32_32x32x16:
//   A[i][kk] = X[oh + i][16 s + kk]: lane l reads 8 adjacent columns of input
//              row oh + l % 32 -- one aligned 16-byte LDS read;
//   B[kk][j] = dz[oh][16 s + kk - j]: lane l reads the run of 8 dy values
//              starting at column 16 s + 8 (l / 32) - l % 32 from a zero-padded
//              copy of dy row oh (two copies shifted by one element, so every
//              run starts on a 4-byte boundary);
//   D: register r of lane l is dw[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
// A workgroup (4 waves) serves one channel and a chunk of images: per image
// and band of BH dy rows it stages the BH + k - 1 padded input rows and the dy
// rows in LDS, each wave takes every 4th dy row of the band, and at the end
// the waves' tiles (and the dy sums for the bias gradient) are added in a
// fixed order into the chunk's partial [k*k + 1] of the workspace, which the
// fixed-order pass 2 reduces over chunks.
namespace {

constexpr int kDzOff = 32;  // zero columns left of a dy row in the table (even: copy 0 is dword aligned)

template <typename T> struct LkmwArgs {
    const T *x, *dy;
    float *ws;           // [c][NC][k*k + 1]
    int C, N, IH, IW, OH, OW, P;
    int NC, npc, nbands;
    int vx, vd;          // x / dy rows are whole aligned 16-byte vectors
};

template <int K, int CS, int BH> struct LkmwGeo {
    static constexpr int QD = 8 * CS + 20;          // dwords per copy of a dy row (multiple of 4)
    static constexpr int D1 = BH * QD + 17;         // dword offset of copy 1 (17 banks from copy 0)
    static constexpr int XR = BH + K - 1;           // staged input rows
    static constexpr int XP = 16 * CS + 8;          // input row pitch (halves)
    static constexpr int dz_bytes = ((D1 + BH * QD) * 4 + 15) / 16 * 16;
    static constexpr int x_bytes = XR * XP * 2;
    static constexpr int red_bytes = 4 * 64 * 17 * 4;  // per-wave tiles and dy sums for the final sum
    static constexpr int lds_bytes = (dz_bytes + x_bytes) > red_bytes ? dz_bytes + x_bytes : red_bytes;
    static_assert(lds_bytes <= kLdsCap, "band tiles exceed the LDS budget");
};

template <typename T, int K, int CS, int BH>
__global__ __launch_bounds__(256) void lk_mfma_bwdw_kernel(LkmwArgs<T> a) {
    using G = LkmwGeo<K, CS, BH>;
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *dz = reinterpret_cast<uint32_t *>(smem);                    // copy 0 [BH][QD], copy 1 at D1
    uint16_t *xt = reinterpret_cast<uint16_t *>(smem + G::dz_bytes);      // [XR][XP]
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int m = lane & 31, h = lane >> 5;
    const int c = blockIdx.x / a.NC;
    const int chunk = blockIdx.x - c * a.NC;
    const int n0 = chunk * a.npc, n1 = min(n0 + a.npc, a.N);

    // zero padding that never changes: every x column and every dy column
    // outside the image (the image part is rewritten per band)
    for (int e = tid; e < G::x_bytes / 16; e += 256) reinterpret_cast<uint4 *>(xt)[e] = make_uint4(0u, 0u, 0u, 0u);
    for (int e = tid; e < G::dz_bytes / 16; e += 256) reinterpret_cast<uint4 *>(dz)[e] = make_uint4(0u, 0u, 0u, 0u);

    f32x16_v acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    float dsum = 0.f;

    // (image, band) steps; with whole 16-byte rows the next step's input and
    // dy rows are loaded into registers while the current band is computed
    constexpr int NXV = ((BH + K - 1) * 2 * CS + 255) / 256;  // x vectors per thread (iw <= 16 CS)
    constexpr int NDV = (BH * 8 + 255) / 256;                 // dy vectors per thread (ow <= 64)
    const bool vec = a.vx && a.vd;
    const int nsteps = (n1 - n0) * a.nbands;
    uint4 pfx[NXV], pfd[NDV];
    auto prefetch = [&](int t) {
        const int n = n0 + t / a.nbands, oh0 = (t % a.nbands) * BH;
        const int rows = min(BH, a.OH - oh0);
        const uint16_t *xp = reinterpret_cast<const uint16_t *>(a.x) + (static_cast<int64_t>(n) * a.C + c) * a.IH * a.IW;
        const uint16_t *dp = reinterpret_cast<const uint16_t *>(a.dy) + (static_cast<int64_t>(n) * a.C + c) * a.OH * a.OW;
        const int xv = a.IW / 8, dv = a.OW / 8;
#pragma unroll
        for (int k = 0; k < NXV; ++k) {
            const int v = tid + 256 * k;
            const int r = v / xv;
            const int ih = oh0 + r - a.P;
            pfx[k] = make_uint4(0u, 0u, 0u, 0u);
            if (v < (rows + K - 1) * xv && ih >= 0 && ih < a.IH)
                pfx[k] = *reinterpret_cast<const uint4 *>(xp + static_cast<int64_t>(ih) * a.IW + (v - r * xv) * 8);
        }
#pragma unroll
        for (int k = 0; k < NDV; ++k) {
            const int v = tid + 256 * k;
            const int r = v / dv;
            pfd[k] = make_uint4(0u, 0u, 0u, 0u);
            if (v < rows * dv)
                pfd[k] = *reinterpret_cast<const uint4 *>(dp + static_cast<int64_t>(oh0 + r) * a.OW + (v - r * dv) * 8);
        }
    };
    if (vec && nsteps > 0) prefetch(0);

    for (int t = 0; t < nsteps; ++t) {
        const int n = n0 + t / a.nbands, band = t % a.nbands;
        const uint16_t *xp = reinterpret_cast<const uint16_t *>(a.x) + (static_cast<int64_t>(n) * a.C + c) * a.IH * a.IW;
        const uint16_t *dp = reinterpret_cast<const uint16_t *>(a.dy) + (static_cast<int64_t>(n) * a.C + c) * a.OH * a.OW;
        {
            const int oh0 = band * BH;
            const int rows = min(BH, a.OH - oh0);
            __syncthreads();  // the previous band's reads are done
            // input rows oh0 .. oh0 + rows + k - 2 of the padded plane (image row = that - P)
            const int xrows = rows + K - 1;
            if (vec) {
                const int xv = a.IW / 8, dv = a.OW / 8;
#pragma unroll
                for (int k = 0; k < NXV; ++k) {
                    const int v = tid + 256 * k;
                    if (v < xrows * xv) {
                        const int r = v / xv;
                        uint16_t *d = xt + r * G::XP + a.P + (v - r * xv) * 8;
                        const uint32_t wd[4] = {pfx[k].x, pfx[k].y, pfx[k].z, pfx[k].w};
#pragma unroll
                        for (int e = 0; e < 8; ++e) d[e] = static_cast<uint16_t>(wd[e >> 1] >> ((e & 1) * 16));
                    }
                }
#pragma unroll
                for (int k = 0; k < NDV; ++k) {
                    const int v = tid + 256 * k;
                    if (v < rows * dv) {
                        const int r = v / dv;
                        const int c8 = (v - r * dv) * 8;
                        *reinterpret_cast<uint4 *>(dz + r * G::QD + (kDzOff + c8) / 2) = pfd[k];
                        const uint32_t wd[4] = {pfd[k].x, pfd[k].y, pfd[k].z, pfd[k].w};
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const uint16_t bits = static_cast<uint16_t>(wd[e >> 1] >> ((e & 1) * 16));
                            T tv;
                            __builtin_memcpy(&tv, &bits, 2);
                            dsum += to_f32(tv);
                        }
                    }
                }
            } else {
                for (int e = tid; e < xrows * a.IW; e += 256) {
                    const int r = e / a.IW;
                    const int col = e - r * a.IW;
                    const int ih = oh0 + r - a.P;
                    xt[r * G::XP + a.P + col] = (ih >= 0 && ih < a.IH) ? xp[static_cast<int64_t>(ih) * a.IW + col] : 0;
                }
                // dy rows oh0 .. oh0 + rows - 1 into copy 0: dword d holds columns 2d - kDzOff, 2d + 1 - kDzOff
                uint16_t *dz16 = reinterpret_cast<uint16_t *>(dz);
                for (int e = tid; e < rows * a.OW; e += 256) {
                    const int r = e / a.OW;
                    const int col = e - r * a.OW;
                    const uint16_t bits = dp[static_cast<int64_t>(oh0 + r) * a.OW + col];
                    dz16[2 * r * G::QD + kDzOff + col] = bits;
                    T tv;
                    __builtin_memcpy(&tv, &bits, 2);
                    dsum += to_f32(tv);
                }
            }
            __syncthreads();
            // copy 1: dword d holds copy-0 positions 2d + 1 and 2d + 2
            uint32_t *dz1 = dz + G::D1;
            for (int e = tid; e < rows * G::QD; e += 256) {
                const int r = e / G::QD;
                const int d = e - r * G::QD;
                const uint32_t lo = dz[r * G::QD + d];
                const uint32_t hi = d + 1 < G::QD ? dz[r * G::QD + d + 1] : 0u;
                dz1[r * G::QD + d] = (lo >> 16) | (hi << 16);
            }
            __syncthreads();
            if (vec && t + 1 < nsteps) prefetch(t + 1);
            // kernel rows i >= k (lanes m >= k) are not part of dw: they read row k - 1
            // instead, so every read stays inside the staged rows
            const int mi = min(m, K - 1);
            for (int oh = wave; oh < rows; oh += 4) {
#pragma unroll
                for (int s = 0; s < CS; ++s) {
                    const u32x4_v af = *reinterpret_cast<const u32x4_v *>(xt + (oh + mi) * G::XP + 16 * s + 8 * h);
                    const int t = 16 * s + 8 * h - m + kDzOff;  // first padded position of this lane's dy run
                    const int q = t & 1;
                    const uint32_t *p = dz + q * G::D1 + oh * G::QD + ((t - q) >> 1);
                    const u32x4_v bf = u32x4_v{p[0], p[1], p[2], p[3]};
                    acc = Mfma<T>::run(af, bf, acc);
                }
            }
        }
    }

    // fixed-order sum of the 4 waves' tiles and of the 256 dy partial sums
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);  // [wave][lane][17]
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 64 + lane) * 17 + r] = acc[r];
    red[(wave * 64 + lane) * 17 + 16] = dsum;
    __syncthreads();
    float *dst = a.ws + (static_cast<int64_t>(c) * a.NC + chunk) * (K * K + 1);
    for (int e = tid; e < K * K + 1; e += 256) {
        float v = 0.f;
        if (e < K * K) {
            const int i = e / K, j = e - (e / K) * K;
            const int ln = 32 * ((i & 7) >> 2) + j, r = 4 * (i >> 3) + (i & 3);
            for (int w = 0; w < 4; ++w) v += red[(w * 64 + ln) * 17 + r];
        } else {
            for (int t2 = 0; t2 < 256; ++t2) v += red[t2 * 17 + 16];
        }
        dst[e] = v;
    }
}

constexpr int kBwBH = 32;  // dy rows per band

struct LkmwPlan {
    int NC, npc, nbands;
};

inline bool plan_lkmw(const Geo &g, LkmwPlan &p) {
    p.nbands = (g.oh + kBwBH - 1) / kBwBH;
    // image chunks: about 2048 workgroups in total
    int NC = std::max(1, (2048 + g.ic - 1) / g.ic);
    NC = std::min(NC, g.n);
    p.npc = (g.n + NC - 1) / NC;
    p.NC = (g.n + p.npc - 1) / p.npc;
    return true;
}

template <typename T, int K, int CS>
int run_lkmw_cs(const Geo &g, const LkmwPlan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    using G = LkmwGeo<K, CS, kBwBH>;
    LkmwArgs<T> a{};
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
    a.nbands = p.nbands;
    a.vx = g.iw % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
    a.vd = g.ow % 8 == 0 && reinterpret_cast<uintptr_t>(dy) % 16 == 0;
    hipLaunchKernelGGL((lk_mfma_bwdw_kernel<T, K, CS, kBwBH>), dim3(g.ic * p.NC), dim3(256), G::lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, int K>
int run_lkmw(const Geo &g, const LkmwPlan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    switch ((g.ow + K - 1 + 15) / 16) {
        case 1: return run_lkmw_cs<T, K, 1>(g, p, x, dy, ws, s);
        case 2: return run_lkmw_cs<T, K, 2>(g, p, x, dy, ws, s);
        case 3: return run_lkmw_cs<T, K, 3>(g, p, x, dy, ws, s);
        case 4: return run_lkmw_cs<T, K, 4>(g, p, x, dy, ws, s);
        case 5: return run_lkmw_cs<T, K, 5>(g, p, x, dy, ws, s);
        default: return run_lkmw_cs<T, K, 6>(g, p, x, dy, ws, s);
    }
}

// ---------------------------------------------------------------- grad-weight, 16 x 16 tiles
// The same contraction for k <= 16 on v_mfma_f32_16x16x32_{f16,bf16}: one
// 16 x 16 output tile (M = kernel row i, N = kernel column j) holds the k x k
// filter, 13 x 13 of 16 x 16 at k = 13 against 13 x 13 of 32 x 32 in the 32 x 32
// tile, so the matrix cores execute a quarter of the multiply-adds.  Per dy
// row and window step of 32 columns one instruction:
//   A[i][kk] = X[oh + i][32 s + kk]: lane l reads 8 adjacent columns
//              (kk = 8 (l / 16) ..) of input row oh + l % 16 -- one aligned
//              16-byte LDS read;
//   B[kk][j] = dz[oh][32 s + kk - j]: lane l reads the run of 8 dy values
//              starting at column 32 s + 8 (l / 16) - l % 16 from the two
//              shifted copies of the dy row (copy 1 placed 17 dwords further
//              in the bank order, so the lanes reading either copy use
//              distinct banks);
//   D: register r of lane l is dw[4 (l / 16) + r][l % 16].
template <int K, int CS, int BH> struct Lkmw16Geo {
    static constexpr int QD = 16 * CS + 20;         // dwords per copy of a dy row
    static constexpr int D1 = BH * QD + 17;         // dword offset of copy 1
    static constexpr int XR = BH + K - 1;           // staged input rows
    static constexpr int XP = 32 * CS + 8;          // input row pitch (halves)
    static constexpr int dz_bytes = ((D1 + BH * QD) * 4 + 15) / 16 * 16;
    static constexpr int x_bytes = XR * XP * 2;
    static constexpr int red_bytes = 4 * 64 * 5 * 4;  // per-wave tiles and dy sums for the final sum
    static constexpr int lds_bytes = (dz_bytes + x_bytes) > red_bytes ? dz_bytes + x_bytes : red_bytes;
    static_assert(lds_bytes <= kLdsCap, "band tiles exceed the LDS budget");
};

template <typename T, int K, int CS, int BH>
__global__ __launch_bounds__(256) void lk_mfma_bwdw16_kernel(LkmwArgs<T> a) {
    using G = Lkmw16Geo<K, CS, BH>;
    static_assert(K <= 16, "one 16 x 16 tile holds the filter");
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *dz = reinterpret_cast<uint32_t *>(smem);                    // copy 0 [BH][QD], copy 1 at D1
    uint16_t *xt = reinterpret_cast<uint16_t *>(smem + G::dz_bytes);      // [XR][XP]
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int jl = lane & 15, g4 = lane >> 4;
    const int c = blockIdx.x / a.NC;
    const int chunk = blockIdx.x - c * a.NC;
    const int n0 = chunk * a.npc, n1 = min(n0 + a.npc, a.N);

    for (int e = tid; e < G::x_bytes / 16; e += 256) reinterpret_cast<uint4 *>(xt)[e] = make_uint4(0u, 0u, 0u, 0u);
    for (int e = tid; e < G::dz_bytes / 16; e += 256) reinterpret_cast<uint4 *>(dz)[e] = make_uint4(0u, 0u, 0u, 0u);

    f32x4_v acc0, acc1;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc0[r] = acc1[r] = 0.f;
    float dsum = 0.f;

    constexpr int NXV = ((BH + K - 1) * 4 * CS + 255) / 256;  // x vectors per thread (iw <= 32 CS)
    constexpr int NDV = (BH * 8 + 255) / 256;                 // dy vectors per thread (ow <= 64)
    const bool vec = a.vx && a.vd;
    const int nsteps = (n1 - n0) * a.nbands;
    uint4 pfx[NXV], pfd[NDV];
    auto prefetch = [&](int t) {
        const int n = n0 + t / a.nbands, oh0 = (t % a.nbands) * BH;
        const int rows = min(BH, a.OH - oh0);
        const uint16_t *xp = reinterpret_cast<const uint16_t *>(a.x) + (static_cast<int64_t>(n) * a.C + c) * a.IH * a.IW;
        const uint16_t *dp = reinterpret_cast<const uint16_t *>(a.dy) + (static_cast<int64_t>(n) * a.C + c) * a.OH * a.OW;
        const int xv = a.IW / 8, dv = a.OW / 8;
#pragma unroll
        for (int k = 0; k < NXV; ++k) {
            const int v = tid + 256 * k;
            const int r = v / xv;
            const int ih = oh0 + r - a.P;
            pfx[k] = make_uint4(0u, 0u, 0u, 0u);
            if (v < (rows + K - 1) * xv && ih >= 0 && ih < a.IH)
                pfx[k] = *reinterpret_cast<const uint4 *>(xp + static_cast<int64_t>(ih) * a.IW + (v - r * xv) * 8);
        }
#pragma unroll
        for (int k = 0; k < NDV; ++k) {
            const int v = tid + 256 * k;
            const int r = v / dv;
            pfd[k] = make_uint4(0u, 0u, 0u, 0u);
            if (v < rows * dv)
                pfd[k] = *reinterpret_cast<const uint4 *>(dp + static_cast<int64_t>(oh0 + r) * a.OW + (v - r * dv) * 8);
        }
    };
    if (vec && nsteps > 0) prefetch(0);

    for (int t = 0; t < nsteps; ++t) {
        const int n = n0 + t / a.nbands, band = t % a.nbands;
        const uint16_t *xp = reinterpret_cast<const uint16_t *>(a.x) + (static_cast<int64_t>(n) * a.C + c) * a.IH * a.IW;
        const uint16_t *dp = reinterpret_cast<const uint16_t *>(a.dy) + (static_cast<int64_t>(n) * a.C + c) * a.OH * a.OW;
        const int oh0 = band * BH;
        const int rows = min(BH, a.OH - oh0);
        __syncthreads();  // the previous band's reads are done
        const int xrows = rows + K - 1;
        if (vec) {
            const int xv = a.IW / 8, dv = a.OW / 8;
#pragma unroll
            for (int k = 0; k < NXV; ++k) {
                const int v = tid + 256 * k;
                if (v < xrows * xv) {
                    const int r = v / xv;
                    uint16_t *d = xt + r * G::XP + a.P + (v - r * xv) * 8;
                    const uint32_t wd[4] = {pfx[k].x, pfx[k].y, pfx[k].z, pfx[k].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) d[e] = static_cast<uint16_t>(wd[e >> 1] >> ((e & 1) * 16));
                }
            }
#pragma unroll
            for (int k = 0; k < NDV; ++k) {
                const int v = tid + 256 * k;
                if (v < rows * dv) {
                    const int r = v / dv;
                    const int c8 = (v - r * dv) * 8;
                    *reinterpret_cast<uint4 *>(dz + r * G::QD + (kDzOff + c8) / 2) = pfd[k];
                    const uint32_t wd[4] = {pfd[k].x, pfd[k].y, pfd[k].z, pfd[k].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint16_t bits = static_cast<uint16_t>(wd[e >> 1] >> ((e & 1) * 16));
                        T tv;
                        __builtin_memcpy(&tv, &bits, 2);
                        dsum += to_f32(tv);
                    }
                }
            }
        } else {
            for (int e = tid; e < xrows * a.IW; e += 256) {
                const int r = e / a.IW;
                const int col = e - r * a.IW;
                const int ih = oh0 + r - a.P;
                xt[r * G::XP + a.P + col] = (ih >= 0 && ih < a.IH) ? xp[static_cast<int64_t>(ih) * a.IW + col] : 0;
            }
            uint16_t *dz16 = reinterpret_cast<uint16_t *>(dz);
            for (int e = tid; e < rows * a.OW; e += 256) {
                const int r = e / a.OW;
                const int col = e - r * a.OW;
                const uint16_t bits = dp[static_cast<int64_t>(oh0 + r) * a.OW + col];
                dz16[2 * r * G::QD + kDzOff + col] = bits;
                T tv;
                __builtin_memcpy(&tv, &bits, 2);
                dsum += to_f32(tv);
            }
        }
        __syncthreads();
        // copy 1: dword d holds copy-0 positions 2d + 1 and 2d + 2
        for (int e = tid; e < rows * G::QD; e += 256) {
            const int r = e / G::QD;
            const int d = e - r * G::QD;
            const uint32_t lo = dz[r * G::QD + d];
            const uint32_t hi = d + 1 < G::QD ? dz[r * G::QD + d + 1] : 0u;
            dz[G::D1 + r * G::QD + d] = (lo >> 16) | (hi << 16);
        }
        __syncthreads();
        if (vec && t + 1 < nsteps) prefetch(t + 1);
        // kernel rows i >= k (lanes with l % 16 >= k) are not part of dw: they read
        // row k - 1 instead, so every read stays inside the staged rows
        const int mi = min(jl, K - 1);
        for (int oh = wave; oh < rows; oh += 4) {
#pragma unroll
            for (int s2 = 0; s2 < CS; ++s2) {
                const u32x4_v af = *reinterpret_cast<const u32x4_v *>(xt + (oh + mi) * G::XP + 32 * s2 + 8 * g4);
                const int tp = 32 * s2 + 8 * g4 - jl + kDzOff;  // first padded position of this lane's dy run
                const int q = tp & 1;
                const uint32_t *p = dz + q * G::D1 + oh * G::QD + ((tp - q) >> 1);
                const u32x4_v bf = u32x4_v{p[0], p[1], p[2], p[3]};
                if (s2 & 1)
                    acc1 = Mfma16<T>::run(af, bf, acc1);
                else
                    acc0 = Mfma16<T>::run(af, bf, acc0);
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
            for (int t2 = 0; t2 < 256; ++t2) v += red[t2 * 5 + 4];
        }
        dst[e] = v;
    }
}

template <typename T, int K, int CS>
int run_lkmw16_cs(const Geo &g, const LkmwPlan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    using G = Lkmw16Geo<K, CS, kBwBH>;
    LkmwArgs<T> a{};
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
    a.nbands = p.nbands;
    a.vx = g.iw % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
    a.vd = g.ow % 8 == 0 && reinterpret_cast<uintptr_t>(dy) % 16 == 0;
    hipLaunchKernelGGL((lk_mfma_bwdw16_kernel<T, K, CS, kBwBH>), dim3(g.ic * p.NC), dim3(256), G::lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, int K>
int run_lkmw16(const Geo &g, const LkmwPlan &p, const void *x, const void *dy, void *ws, hipStream_t s) {
    switch ((g.ow + K - 1 + 31) / 32) {
        case 1: return run_lkmw16_cs<T, K, 1>(g, p, x, dy, ws, s);
        case 2: return run_lkmw16_cs<T, K, 2>(g, p, x, dy, ws, s);
        default: return run_lkmw16_cs<T, K, 3>(g, p, x, dy, ws, s);
    }
}

}  // namespace

// 16-bit I/O, k = 13 or 31 square, stride 1, dilation 1, multiplier 1,
// symmetric padding, dy rows of at most 64 (so the window, ow + k - 1 <= 94
// columns, is at most six 16-column steps) and an input that fits the staged
// columns.
bool largek_mfma_bwdw_fits(const Geo &g, int dtype) {
    if (dtype == 0) return false;
    if (g.kh != g.kw || (g.kh != 13 && g.kh != 31)) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.ph != g.pw || g.mult != 1) return false;
    if (g.ow > 64) return false;
    const int XC = 16 * ((g.ow + g.kh - 1 + 15) / 16);
    return g.iw + g.ph <= XC;
}

int largek_mfma_bwd_weight_chunks(const Geo &g) {
    LkmwPlan p;
    plan_lkmw(g, p);
    return p.NC;
}

// 16-bit I/O, k = 7 or 13 square, stride 1, dilation 1, multiplier 1,
// symmetric padding, dy rows of at most 64 (the window, ow + k - 1 <= 76
// columns, is at most three 32-column steps) and an input that fits them.
bool largek_mfma_bwdw16_fits(const Geo &g, int dtype) {
    if (dtype == 0) return false;
    if (g.kh != g.kw || (g.kh != 7 && g.kh != 13)) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.ph != g.pw || g.mult != 1) return false;
    if (g.ow > 64) return false;
    const int XC = 32 * ((g.ow + g.kh - 1 + 31) / 32);
    return g.iw + g.ph <= XC;
}

int largek_mfma_bwd_weight16(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s) {
    LkmwPlan p;
    plan_lkmw(g, p);
    if (dtype == 1) return g.kh == 7 ? run_lkmw16<__half, 7>(g, p, x, dy, ws, s) : run_lkmw16<__half, 13>(g, p, x, dy, ws, s);
    return g.kh == 7 ? run_lkmw16<bf16_t, 7>(g, p, x, dy, ws, s) : run_lkmw16<bf16_t, 13>(g, p, x, dy, ws, s);
}

int largek_mfma_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s) {
    LkmwPlan p;
    plan_lkmw(g, p);
    if (dtype == 1) return g.kh == 13 ? run_lkmw<__half, 13>(g, p, x, dy, ws, s) : run_lkmw<__half, 31>(g, p, x, dy, ws, s);
    return g.kh == 13 ? run_lkmw<bf16_t, 13>(g, p, x, dy, ws, s) : run_lkmw<bf16_t, 31>(g, p, x, dy, ws, s);
}

}  // namespace dw
