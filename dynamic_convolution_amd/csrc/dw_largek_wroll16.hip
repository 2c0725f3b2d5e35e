// dw_largek_wroll16.hip -- large-kernel (k = 13, 31) depthwise grad-weight
// for 16-bit I/O on the gfx950 matrix cores, streaming input rows (stride 1,
// dilation 1, multiplier 1, output rows of at most 64).
//
// The grad-weight correlates the input with the output gradient (PR #3057's
// grad-weight kernel; the MegEngine large-kernel depthwise article's
// (n, ic, ih, iw) x (oc, kh, kw) problem).  Taken one input row r at a time:
//   dw[i][j] += sum_ow dy[r + P - i][ow] * X[r][ow + j - P]
// for every kernel row i at once -- a product D = A B with A[i][ow] the dy
// rows r + P - i (M = kernel rows, K = output columns) and B[ow][j] a Hankel
// matrix of input row r (B[ow][j] = X[r][ow + j - P]: each lane reads 8
// adjacent values of the staged row).  D is the grad-weight tile itself and
// stays in registers for all rows and images of a wave.  From one input row
// to the next the dy rows of A move down one kernel row: every lane takes
// its neighbour's registers (a DPP row rotation), the first lane of the
// second 16-row block the last of the first, and the first lane of the first
// block the dy row entering the window (read from a ring of staged dy rows).
// Only products of kernel rows whose dy row lies outside the plane, of
// (column, kernel column) pairs whose input column lies outside the row, and
// of the padding up to 16-row / 16-column blocks are executed beyond the
// useful ones -- not the k / (16 + k - 1) band of a Toeplitz tile.
//
// v_mfma_f32_16x16x32_{f16,bf16} lane layout (checked on the MI355X): A lane l
// holds row l % 16, k = 8 (l / 16) .. + 8; B lane l holds column l % 16, the
// same k; D register q of lane l holds row 4 (l / 16) + q, column l % 16.
// Products of 16-bit values are exact and sums are fp32.
//
// One wave owns one channel and a group of images (a chunk of the two-pass,
// atomics-free reduction: it writes its k*k sums and its dy sum, the bias
// gradient's share, to the workspace).  Input rows and dy rows arrive four at
// a time from 16-byte buffer loads one batch ahead into LDS rings of the
// wave's own; input rows are stored twice, the second copy shifted by one
// element so every 8-value run starts on a 4-byte boundary.
#include "dw_common.hpp"
#include "dw_internal.hpp"

#include <type_traits>

namespace dw {
namespace {

typedef _Float16 f16x8_g __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_g __attribute__((ext_vector_type(8)));
typedef float f32x4_g __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_g __attribute__((ext_vector_type(4)));

template <typename T> struct WrMfma;
template <> struct WrMfma<__half> {
    static __device__ __forceinline__ f32x4_g run(u32x4_g a, u32x4_g b, f32x4_g c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_g, a), __builtin_bit_cast(f16x8_g, b),
                                                      c, 0, 0, 0);
    }
};
template <> struct WrMfma<bf16_t> {
    static __device__ __forceinline__ f32x4_g run(u32x4_g a, u32x4_g b, f32x4_g c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_g, a),
                                                       __builtin_bit_cast(bf16x8_g, b), c, 0, 0, 0);
    }
};

constexpr int kWrSkip = 0x40000000;  // buffer offset past any plane: loads read zeros

struct WrArgs {
    const void *x;
    const void *dy;
    float *ws;     // [c][NC][k*k + 1]
    int N, C, IH, IW, OH, OW, P;
    int NC, ipw;   // image chunks of a channel (one wave each), images per chunk
};

// Staged input row (NS 32-column steps of output columns, kernel columns in
// blocks of 16): copy 0 at halves [0, XP), copy 1 from dword D1 (+1 for an odd
// alignment shift, which keeps the two copies' lanes in different banks); ring
// slot k of dword d at RS d + k.  Staged dy rows: DYP dwords a row, slot-major.
template <int K, int NS> struct WrGeo {
    static constexpr int NB = (K + 15) / 16;           // 16-row / 16-column blocks
    static constexpr int SLOTS = 8;                    // rows in flight: two batches of four
    static constexpr int RS = SLOTS + 1;
    static constexpr int XW = 32 * NS + 16 * NB - 1;   // input columns a row step reads
    static constexpr int XP = (XW + 23 + 7) / 8 * 8;
    static constexpr int D1 = (XP / 2 + 1 + 15) / 32 * 32 + 16;
    static constexpr int ROWD = D1 + 1 + XP / 2;
    static constexpr int XRING = RS * ROWD;            // dwords of the input ring
    static constexpr int DYP = 16 * NS + 4;            // dwords of a staged dy row (32 NS halves, padded)
    static constexpr int DRING = SLOTS * DYP;
    static constexpr int NVEC = (XW + 7 + 7) / 8;      // 8-column vectors an input row may need
    static_assert(NVEC <= 16, "a staged row is loaded by 16 lanes");
    static constexpr int lds_bytes = 4 * (XRING + DRING) * 4;
};

__device__ __forceinline__ void wr_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Lane l takes lane (l - 1) mod 16 of its 16-lane row (DPP row_ror:1), every lane enabled.
__device__ __forceinline__ uint32_t wr_rot(uint32_t v) {
    uint32_t r = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x121, 0xf, 0xf, true));
    asm volatile("" : "+v"(r));
    return r;
}

__device__ __forceinline__ float wr_f32(uint32_t h, __half *) { return __half2float(__ushort_as_half(static_cast<unsigned short>(h))); }
__device__ __forceinline__ float wr_f32(uint32_t h, bf16_t *) { return __uint_as_float(h << 16); }

template <typename T, int K, int NS, bool VX, bool VD>
__global__ __launch_bounds__(256) void lk_wroll16_kernel(WrArgs a) {
    using G = WrGeo<K, NS>;
    constexpr int NB = G::NB;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wid = blockIdx.x * 4 + wave;
    if (wid >= a.C * a.NC) return;  // whole waves; the kernel has no workgroup barrier
    uint32_t *xring = reinterpret_cast<uint32_t *>(smem) + wave * (G::XRING + G::DRING);
    uint32_t *dring = xring + G::XRING;

    const int c = wid / a.NC;
    const int chunk = wid - c * a.NC;
    const int n0 = chunk * a.ipw, n1 = min(n0 + a.ipw, a.N);

    const int m = lane & 15, g = lane >> 4;
    const int cb = -a.P;             // input column of window position 0
    const int cb8 = cb & ~7;
    const int AL = cb - cb8;
    const int d1 = G::D1 + (AL & 1);
    // B operand of (column block bj, step s): staged position AL + 32 s + 16 bj + 8 g + m
    const int s0 = AL + 8 * g + m;
    const int boff = G::RS * ((s0 & 1) ? d1 + ((s0 - 1) >> 1) : (s0 >> 1));
    const int sk = lane & 15;
    const int gc = cb8 + 8 * sk;
    const bool vk = sk < G::NVEC && gc >= 0 && gc + 8 <= a.IW;
    const bool vd = 8 * sk < a.OW;   // dy staging lane: output columns 8 sk .. 8 sk + 7

    for (int e = lane; e < G::XRING + G::DRING; e += 64) xring[e] = 0u;
    wr_lds_sync();

    const int64_t iplane = static_cast<int64_t>(a.IH) * a.IW;
    const int64_t oplane = static_cast<int64_t>(a.OH) * a.OW;
    constexpr int PD = K > 16 ? 2 : 4;  // batches loaded ahead
    const int nq = ((a.IH + 4 * PD - 1) / (4 * PD)) * PD;  // batches of four input rows, whole groups of PD
    f32x4_g d[NB][NB];
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
        for (int bj = 0; bj < NB; ++bj) d[bi][bj] = f32x4_g{0.f, 0.f, 0.f, 0.f};
    float dsum = 0.f;  // this lane's share of the dy sum (bias gradient)

    for (int nimg = n0; nimg < n1; ++nimg) {
        const uint16_t *ip = static_cast<const uint16_t *>(a.x) + (static_cast<int64_t>(nimg) * a.C + c) * iplane;
        const uint16_t *gp = static_cast<const uint16_t *>(a.dy) + (static_cast<int64_t>(nimg) * a.C + c) * oplane;
        const __amdgpu_buffer_rsrc_t xr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(ip), 0, static_cast<int>(iplane * 2), 0x00020000);
        const __amdgpu_buffer_rsrc_t gr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(gp), 0, static_cast<int>(oplane * 2), 0x00020000);

        // A at input row 0: lane (m, g) of block bi, step s holds dy row
        // P - 16 bi - m, columns 32 s + 8 g .. + 7 (zero outside the plane)
        u32x4_g A[NB][NS];
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int oh = a.P - 16 * bi - m, oc0 = 32 * s + 8 * g;
                if constexpr (VD) {
                    const int off = (oh >= 0 && oh < a.OH && oc0 < a.OW) ? (oh * a.OW + oc0) * 2 : kWrSkip;
                    A[bi][s] = __builtin_amdgcn_raw_buffer_load_b128(gr, off, 0, 0);
                } else {
#pragma unroll
                    for (int k2 = 0; k2 < 4; ++k2) {
                        uint32_t v = 0;
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int ow = oc0 + 2 * k2 + hh;
                            if (oh >= 0 && oh < a.OH && ow < a.OW)
                                v |= static_cast<uint32_t>(gp[static_cast<int64_t>(oh) * a.OW + ow]) << (16 * hh);
                        }
                        A[bi][s][k2] = v;
                    }
                }
            }
        // the dy rows A starts with (0 .. P) enter the bias sum here: each is
        // held by exactly one lane row of block 0 or 1
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2)
                    dsum += wr_f32(A[bi][s][k2] & 0xffffu, static_cast<T *>(nullptr)) +
                            wr_f32(A[bi][s][k2] >> 16, static_cast<T *>(nullptr));

        // batch qb: input rows 4 qb .. + 3 (zeros past the plane) and the dy
        // rows that enter A after them, 4 qb + P + 1 .. + 4
        auto load_x = [&](int qb) -> uint4 {
            const int r = 4 * qb + (lane >> 4);
            const int off = (vk && r < a.IH) ? (r * a.IW + gc) * 2 : kWrSkip;
            const u32x4_g v = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
            return make_uint4(v[0], v[1], v[2], v[3]);
        };
        auto load_d = [&](int qb) -> uint4 {
            const int oh = 4 * qb + (lane >> 4) + a.P + 1;
            const int off = (vd && oh < a.OH) ? (oh * a.OW + 8 * sk) * 2 : kWrSkip;
            const u32x4_g v = __builtin_amdgcn_raw_buffer_load_b128(gr, off, 0, 0);
            return make_uint4(v[0], v[1], v[2], v[3]);
        };
        auto put = [&](int qb, const uint4 &rx, const uint4 &rd) {
            const int k = (4 * qb + (lane >> 4)) & (G::SLOTS - 1);
            if (vk) {
                uint32_t *p0 = xring + G::RS * (4 * sk) + k;
                p0[0] = rx.x;
                p0[G::RS] = rx.y;
                p0[2 * G::RS] = rx.z;
                p0[3 * G::RS] = rx.w;
                uint32_t *p1 = xring + G::RS * (d1 + 4 * sk) + k;
                reinterpret_cast<uint16_t *>(p1 - G::RS)[1] = static_cast<uint16_t>(rx.x);
                p1[0] = __builtin_amdgcn_alignbit(rx.y, rx.x, 16);
                p1[G::RS] = __builtin_amdgcn_alignbit(rx.z, rx.y, 16);
                p1[2 * G::RS] = __builtin_amdgcn_alignbit(rx.w, rx.z, 16);
                reinterpret_cast<uint16_t *>(p1 + 3 * G::RS)[0] = static_cast<uint16_t>(rx.w >> 16);
            }
            if (vd) {
                *reinterpret_cast<uint4 *>(dring + k * G::DYP + 4 * sk) = rd;
                const uint32_t w4[4] = {rd.x, rd.y, rd.z, rd.w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    dsum += wr_f32(w4[q] & 0xffffu, static_cast<T *>(nullptr)) + wr_f32(w4[q] >> 16, static_cast<T *>(nullptr));
            }
        };
        // element-wise staging (rows that are not whole aligned vectors)
        auto stage_scalar = [&](int qb) {
            const int span = AL + G::XW;
            for (int e = lane; e < 4 * span; e += 64) {
                const int q = e / span;
                const int p = e - q * span;
                const int r = 4 * qb + q;
                const int col = cb8 + p;
                if (col < 0 || col >= a.IW) continue;
                const uint16_t v = r < a.IH ? ip[static_cast<int64_t>(r) * a.IW + col] : uint16_t{0};
                const int k = (4 * qb + q) & (G::SLOTS - 1);
                reinterpret_cast<uint16_t *>(xring + G::RS * (p >> 1) + k)[p & 1] = v;
                const int q1 = 2 * d1 + p - 1;
                reinterpret_cast<uint16_t *>(xring + G::RS * (q1 >> 1) + k)[q1 & 1] = v;
            }
            for (int e = lane; e < 4 * 32 * NS; e += 64) {
                const int q = e / (32 * NS);
                const int ow = e - q * 32 * NS;
                const int oh = 4 * qb + q + a.P + 1;
                const uint16_t v = (ow < a.OW && oh < a.OH) ? gp[static_cast<int64_t>(oh) * a.OW + ow] : uint16_t{0};
                const int k = (4 * qb + q) & (G::SLOTS - 1);
                reinterpret_cast<uint16_t *>(dring + k * G::DYP)[ow] = v;
                dsum += wr_f32(v, static_cast<T *>(nullptr));
            }
        };

        // Input and dy rows are loaded PD batches before they are staged:
        // nothing else uses vector memory in the loop and every batch issues
        // the same loads (rows past the plane read zeros), so each wait is for
        // the oldest loads only.  A batch is a few hundred cycles of matrix
        // work; a load from memory takes several batches.
        uint4 rx[PD], rd[PD];
        if constexpr (VX && VD) {
            put(0, load_x(0), load_d(0));
#pragma unroll
            for (int b = 0; b < PD; ++b) {
                rx[b] = load_x(b + 1);
                rd[b] = load_d(b + 1);
            }
        } else {
            stage_scalar(0);
        }

        auto step = [&](int r) {
            const int k = r & (G::SLOTS - 1);
            u32x4_g bv[NB][NS];
            const uint32_t *bp = xring + boff + k;
#pragma unroll
            for (int bj = 0; bj < NB; ++bj)
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const uint32_t *q = bp + G::RS * (16 * s + 8 * bj);
                    bv[bj][s] = u32x4_g{q[0], q[G::RS], q[2 * G::RS], q[3 * G::RS]};
                }
            // the dy row entering A after this input row: only the first lane of
            // each lane row reads it (an LDS read returns data to every active
            // lane, and 16 lanes of one run would cost 16 times its bytes)
            u32x4_g nw[NS];
            if (m == 0) {
#pragma unroll
                for (int s = 0; s < NS; ++s) nw[s] = *reinterpret_cast<const u32x4_g *>(dring + k * G::DYP + 16 * s + 4 * g);
            }
#pragma unroll
            for (int bi = 0; bi < NB; ++bi)
#pragma unroll
                for (int bj = 0; bj < NB; ++bj)
#pragma unroll
                    for (int s = 0; s < NS; ++s) d[bi][bj] = WrMfma<T>::run(A[bi][s], bv[bj][s], d[bi][bj]);
            // move the dy rows down one kernel row
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) {
                    uint32_t prev = nw[s][k2];  // what lane 0 of block 0 takes
#pragma unroll
                    for (int bi = 0; bi < NB; ++bi) {
                        const uint32_t rot = wr_rot(A[bi][s][k2]);  // lane 0: this block's lane 15
                        A[bi][s][k2] = m == 0 ? prev : rot;
                        prev = rot;
                    }
                }
        };
        // batch q (register set b = q % PD holds batch q + 1 on entry)
        auto batch = [&](auto b_c, int q) {
            constexpr int B = decltype(b_c)::value;
            wr_lds_sync();  // batch q is in the rings; batch q - 1's reads are done
            {
                if constexpr (VX && VD) {
                    put(q + 1, rx[B], rd[B]);
                    rx[B] = load_x(q + 1 + PD);
                    rd[B] = load_d(q + 1 + PD);
                } else {
                    stage_scalar(q + 1);
                }
            }
            const int r = 4 * q;
            step(r);
            step(r + 1);
            step(r + 2);
            step(r + 3);
        };
        for (int q = 0; q < nq; q += PD) {
            batch(std::integral_constant<int, 0>{}, q);
            batch(std::integral_constant<int, 1>{}, q + 1);
            if constexpr (PD == 4) {
                batch(std::integral_constant<int, 2>{}, q + 2);
                batch(std::integral_constant<int, 3>{}, q + 3);
            }
        }
        wr_lds_sync();  // the rings' reads are done before the next image writes them
        // dy rows past the last batch never enter A: they sit below the last
        // input row + P and pair with no input row; rows the last batch staged
        // that lie past OH are zero
    }

    // the chunk's sums: dw[i][j] (D register q of lane (m, g): i = 16 bi + 4 g + q,
    // j = 16 bj + m) and the dy sum
    float *wsp = a.ws + (static_cast<int64_t>(c) * a.NC + chunk) * (K * K + 1);
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
        for (int bj = 0; bj < NB; ++bj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = 16 * bi + 4 * g + q, j = 16 * bj + m;
                if (i < K && j < K) wsp[i * K + j] = d[bi][bj][q];
            }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) dsum += __shfl_xor(dsum, o, 64);
    if (lane == 0) wsp[K * K] = dsum;
}

struct WrPlan {
    int NC, ipw;
};

// about three rounds of four waves per SIMD, a few images a wave
void plan_wr(const Geo &g, WrPlan &p) {
    const int64_t want = std::max<int64_t>(1, 12288 / std::max(1, g.ic));
    p.NC = static_cast<int>(std::min<int64_t>(g.n, want));
    p.ipw = (g.n + p.NC - 1) / p.NC;
    p.NC = (g.n + p.ipw - 1) / p.ipw;
}

template <typename T, int K, int NS>
int run_wr(const Geo &g, const void *x, const void *dy, void *ws, hipStream_t s) {
    using G = WrGeo<K, NS>;
    WrPlan p;
    plan_wr(g, p);
    WrArgs a{};
    a.x = x;
    a.dy = dy;
    a.ws = static_cast<float *>(ws);
    a.N = g.n;
    a.C = g.ic;
    a.IH = g.ih;
    a.IW = g.iw;
    a.OH = g.oh;
    a.OW = g.ow;
    a.P = g.ph;
    a.NC = p.NC;
    a.ipw = p.ipw;
    const int64_t nw = static_cast<int64_t>(g.ic) * p.NC;
    const dim3 grid(static_cast<unsigned>((nw + 3) / 4));
    const bool vx = g.iw % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
    const bool vd = g.ow % 8 == 0 && reinterpret_cast<uintptr_t>(dy) % 16 == 0;
    if (vx && vd)
        hipLaunchKernelGGL((lk_wroll16_kernel<T, K, NS, true, true>), grid, dim3(256), G::lds_bytes, s, a);
    else
        hipLaunchKernelGGL((lk_wroll16_kernel<T, K, NS, false, false>), grid, dim3(256), G::lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, int K>
int run_wr_k(const Geo &g, const void *x, const void *dy, void *ws, hipStream_t s) {
    if (g.ow <= 32) return run_wr<T, K, 1>(g, x, dy, ws, s);
    return run_wr<T, K, 2>(g, x, dy, ws, s);
}

}  // namespace

// 16-bit, k = 13 or 31 square, stride 1, dilation 1, multiplier 1, equal
// paddings below k, output rows of at most 64 and planes below 1 GiB.
bool largek_wroll16_fits(const Geo &g, int dtype) {
    if (dtype == 0) return false;
    if (g.kh != g.kw || (g.kh != 13 && g.kh != 31)) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.mult != 1) return false;
    if (g.ph != g.pw || g.ph > g.kh - 1) return false;
    if (g.oh < 1 || g.ow < 1 || g.ow > 64) return false;
    const int64_t ip = static_cast<int64_t>(g.ih) * g.iw, op = static_cast<int64_t>(g.oh) * g.ow;
    return std::max(ip, op) * 2 < (int64_t{1} << 30);
}

int largek_wroll16_chunks(const Geo &g) {
    WrPlan p;
    plan_wr(g, p);
    return p.NC;
}

int largek_wroll16(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s) {
    if (g.kh == 13)
        return dtype == 1 ? run_wr_k<__half, 13>(g, x, dy, ws, s) : run_wr_k<bf16_t, 13>(g, x, dy, ws, s);
    return dtype == 1 ? run_wr_k<__half, 31>(g, x, dy, ws, s) : run_wr_k<bf16_t, 31>(g, x, dy, ws, s);
}

}  // namespace dw
