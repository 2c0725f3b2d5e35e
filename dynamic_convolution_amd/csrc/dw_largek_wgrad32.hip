// dw_largek_wgrad32.hip -- large-kernel (k = 31) depthwise grad-weight for
// fp32 I/O on the gfx950 matrix cores (stride 1, dilation 1, multiplier 1).
//
// The grad-weight is a correlation of the input with the output gradient
// (PR #3057's grad-weight kernel; the MegEngine large-kernel depthwise article
// states the problem as (n, ic, ih, iw) x (oc, kh, kw)).  For one image n and
// one output row oh it is a dense product over the input columns m:
//   dw[i][j] += sum_m X[oh + i - P][m] * dy[oh][m - j + P],
// terms whose dy column m - j + P falls outside [0, ow) being zero.  So with
//   A[i][m] = X[oh + i - P][m]        (tap rows x input columns)
//   B[m][j] = dy[oh][m - j + P]        (the dy row arranged by shift)
// a (32 x 32) tile of dw accumulates A * B, the contraction running over the
// iw input columns only: unlike the forward's banded (Toeplitz) form no
// structural zeros of a band are multiplied.  What the tile executes beyond
// the useful multiply-adds is (a) tap rows whose input row lies outside the
// image, (b) the (m, j) corners where the dy column falls outside the row and
// (c) the 32nd tap row and column of a 31 x 31 filter: 1.38x the useful work
// at 64 x 64 planes, 1.85x at 32 x 32.  v_mfma_f32_32x32x2_f32 multiplies
// and adds in fp32 and was measured at 130-144 TFLOP/s on the MI355X against
// 100-112 for the best v_fmac_f32 code, which is why fp32 grad-weight of the
// 31 x 31 filter runs here and not on the vector units.
//
// Lane layout of v_mfma_f32_32x32x2_f32 (checked on the MI355X with an
// in-bounds probe): A lane l holds row l % 32, k = l / 32; B lane l holds
// column l % 32, k = l / 32; D register r of lane l holds row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
//
// A workgroup (4 waves) owns one channel and a chunk of images.  Per band of
// dy rows it stages the input rows the band reads (zero rows outside the
// image) and the dy rows, each placed at column offset 31 - P of a zeroed row
// so every B read is in bounds and reads zero outside the row; the waves take
// the band's dy rows in turn.  Four instructions consume one 16-byte LDS read
// of x per lane (instruction t takes input column base + 4 (l / 32) + t) and
// four 4-byte reads of dy.  The waves' tiles are summed in a fixed order into
// the chunk partial of the two-pass, atomics-free reduction.
#include "dw_common.hpp"
#include "dw_internal.hpp"

namespace dw {
namespace {

typedef float f32x16_w __attribute__((ext_vector_type(16)));

constexpr int kW32K = 31;       // filter size this family serves
constexpr int kW32Off = 31;     // dz column of dy column -P (so m - j + 31 indexes dz directly)
constexpr int kW32TargetWG = 6144;

struct Lw32Args {
    const float *x;
    const float *dy;
    float *ws;      // [c][NC][k*k + 1]
    int C, N, IH, IW, OH, OW, P;
    int NC, npc;    // image chunks, images per chunk
    int BH, nbands; // dy rows per band, bands per plane
    int XW;         // x columns the instructions walk: iw rounded up to 8
    int XP;         // LDS pitch of an x row: XW + 4 (lanes read 32 different rows: the
                    // odd multiple of 4 floats puts 16 consecutive rows in distinct banks)
    int L;          // LDS pitch of a dz row: XW + 32
    int vx, vd;     // x / dy rows are whole aligned 16-byte vectors
};

__device__ __forceinline__ f32x16_w mfma32(float a, float b, f32x16_w c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int K>
__global__ __launch_bounds__(256) void lk_wgrad32_kernel(Lw32Args a) {
    extern __shared__ __align__(16) unsigned char smem[];
    float *xs = reinterpret_cast<float *>(smem);          // [BH + K - 1][XP]
    float *dz = xs + (a.BH + K - 1) * a.XP;               // [BH][L]
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the row loop branches on it
    const int lane = tid & 63;
    const int mj = lane & 31, h = lane >> 5;
    const int c = blockIdx.x / a.NC;
    const int chunk = blockIdx.x - c * a.NC;
    const int n0 = chunk * a.npc, n1 = min(n0 + a.npc, a.N);

    // zero once: x columns iw .. XP - 1 of every row and every dz column
    // outside the dy row are never rewritten
    const int xtot = (a.BH + K - 1) * a.XP, dtot = a.BH * a.L;
    for (int e = tid; e < xtot + dtot; e += 256) xs[e] = 0.f;

    // two accumulators, alternating, so consecutive instructions do not wait on each other
    f32x16_w acc0, acc1;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;
    float dsum = 0.f;
    // tap row 31 (outside the 31 x 31 filter) reads tap row 30's input row so
    // every read stays in the staged rows; its results are discarded
    const int mi = min(mj, K - 1);

    for (int n = n0; n < n1; ++n) {
        const float *xp = a.x + (static_cast<int64_t>(n) * a.C + c) * a.IH * a.IW;
        const float *dp = a.dy + (static_cast<int64_t>(n) * a.C + c) * a.OH * a.OW;
        for (int band = 0; band < a.nbands; ++band) {
            const int oh0 = band * a.BH;
            const int rows = min(a.BH, a.OH - oh0);
            const int xrows = rows + K - 1;
            __syncthreads();  // the previous band's reads are done
            // input rows: staged row r is image row oh0 + r - P (zeros outside the image)
            if (a.vx) {
                const int vpr = a.IW >> 2;
                for (int v = tid; v < xrows * vpr; v += 256) {
                    const int r = v / vpr;
                    const int c4 = (v - r * vpr) << 2;
                    const int ih = oh0 + r - a.P;
                    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (ih >= 0 && ih < a.IH) t = *reinterpret_cast<const float4 *>(xp + static_cast<int64_t>(ih) * a.IW + c4);
                    *reinterpret_cast<float4 *>(xs + r * a.XP + c4) = t;
                }
            } else {
                for (int e = tid; e < xrows * a.IW; e += 256) {
                    const int r = e / a.IW;
                    const int col = e - r * a.IW;
                    const int ih = oh0 + r - a.P;
                    xs[r * a.XP + col] = (ih >= 0 && ih < a.IH) ? xp[static_cast<int64_t>(ih) * a.IW + col] : 0.f;
                }
            }
            // dy rows oh0 .. oh0 + rows - 1 at dz column kW32Off - P + ow
            float *dzb = dz + kW32Off - a.P;
            if (a.vd) {
                const int vpr = a.OW >> 2;
                for (int v = tid; v < rows * vpr; v += 256) {
                    const int r = v / vpr;
                    const int c4 = (v - r * vpr) << 2;
                    const float4 t = *reinterpret_cast<const float4 *>(dp + static_cast<int64_t>(oh0 + r) * a.OW + c4);
                    float *d = dzb + r * a.L + c4;
                    d[0] = t.x;
                    d[1] = t.y;
                    d[2] = t.z;
                    d[3] = t.w;
                    dsum += (t.x + t.y) + (t.z + t.w);
                }
            } else {
                for (int e = tid; e < rows * a.OW; e += 256) {
                    const int r = e / a.OW;
                    const int col = e - r * a.OW;
                    const float t = dp[static_cast<int64_t>(oh0 + r) * a.OW + col];
                    dzb[r * a.L + col] = t;
                    dsum += t;
                }
            }
            __syncthreads();
            for (int oh = wave; oh < rows; oh += 4) {
                // A: x row oh + i (staged), columns base + 4h + t; B: dz[oh][base + 4h + t - j + 31]
                const float *xr = xs + (oh + mi) * a.XP + 4 * h;
                const float *dr = dz + oh * a.L + kW32Off - mj + 4 * h;
                for (int base = 0; base < a.XW; base += 8) {
                    const float4 av = *reinterpret_cast<const float4 *>(xr + base);
                    const float b0 = dr[base], b1 = dr[base + 1], b2 = dr[base + 2], b3 = dr[base + 3];
                    acc0 = mfma32(av.x, b0, acc0);
                    acc1 = mfma32(av.y, b1, acc1);
                    acc0 = mfma32(av.z, b2, acc0);
                    acc1 = mfma32(av.w, b3, acc1);
                }
            }
        }
    }

    // fixed-order sum of the 4 waves' tiles and of the 256 dy partial sums
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);  // [wave][lane][17]
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 64 + lane) * 17 + r] = acc0[r] + acc1[r];
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
            for (int t = 0; t < 256; ++t) v += red[t * 17 + 16];
        }
        dst[e] = v;
    }
}

struct Lw32Plan {
    int NC, npc, BH, nbands, XW, XP, L, lds_bytes;
};

bool plan_lw32(const Geo &g, Lw32Plan &p) {
    p.XW = (g.iw + 7) & ~7;
    p.XP = p.XW + 4;
    p.L = p.XW + 32;
    auto bytes = [&](int bh) {
        const int64_t stage = (static_cast<int64_t>(bh + kW32K - 1) * p.XP + static_cast<int64_t>(bh) * p.L) * 4;
        return std::max<int64_t>(stage, 4 * 64 * 17 * 4);
    };
    // bands of at most 32 dy rows within 40 KiB, so four or more workgroups
    // share a CU and one's staging overlaps the others' matrix work
    int bh = std::min(g.oh, 32);
    while (bh > 1 && bytes(bh) > 40 * 1024) --bh;
    if (bytes(bh) > 64 * 1024) return false;
    p.nbands = (g.oh + bh - 1) / bh;
    p.BH = (g.oh + p.nbands - 1) / p.nbands;
    p.lds_bytes = static_cast<int>(bytes(p.BH));
    int NC = std::max(1, (kW32TargetWG + g.ic - 1) / g.ic);
    NC = std::min(NC, g.n);
    p.npc = (g.n + NC - 1) / NC;
    p.NC = (g.n + p.npc - 1) / p.npc;
    return true;
}

}  // namespace

// fp32, 31 x 31 square filter, stride 1, dilation 1, multiplier 1, the same
// padding on both axes and at most 31 (the dz offset), rows of at most 256.
bool largek_wgrad32_fits(const Geo &g, int dtype) {
    if (dtype != 0) return false;
    if (g.kh != kW32K || g.kw != kW32K) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.ph != g.pw || g.mult != 1) return false;
    if (g.ph > kW32Off || g.iw > 256) return false;
    Lw32Plan p;
    return plan_lw32(g, p);
}

int largek_wgrad32_chunks(const Geo &g) {
    Lw32Plan p;
    return plan_lw32(g, p) ? p.NC : 0;
}

int largek_wgrad32(const Geo &g, const void *x, const void *dy, void *ws, hipStream_t s) {
    Lw32Plan p;
    if (!plan_lw32(g, p)) return kErrUnsupported;
    Lw32Args a{};
    a.x = static_cast<const float *>(x);
    a.dy = static_cast<const float *>(dy);
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
    a.vx = g.iw % 4 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
    a.vd = g.ow % 4 == 0 && reinterpret_cast<uintptr_t>(dy) % 16 == 0;
    hipLaunchKernelGGL((lk_wgrad32_kernel<kW32K>), dim3(g.ic * p.NC), dim3(256), p.lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

}  // namespace dw
