// dw_largek_fwd32.hip -- large-kernel (k = 31) depthwise forward and
// grad-input for fp32 I/O on the gfx950 matrix cores (stride 1, dilation 1).
//
// The forward (MegEngine large-kernel depthwise article: the im2col problem
// statement; its implicit batched GEMM) is split by kernel column:
//   y[oh][ow] = b + sum_j U_j[oh][ow + j - P],
//   U_j[oh][c] = sum_i w[i][j] * X[oh + i - P][c].
// For one output row oh and a tile of 32 input columns, U is a dense
// 32 x 32 x 31 product D[j][c] = sum_i A[j][i] B[i][c] with A[j][i] = w[i][j]
// (the filter, transposed: the same for every row, so it is held in 16
// registers per lane for the whole kernel) and B[i][c] = X[oh + i - P][c0 + c]
// (the input rows the output row reads).  The contraction runs over kernel
// rows, so pairs of kernel rows whose input rows are both outside the image
// are skipped with a wave-uniform branch; the only multiply-adds executed
// beyond the useful ones are the (j, c) corners of a tile whose output column
// ow = c0 + c - j + P falls outside the row, and the 32nd kernel row and
// column.  The anti-diagonal sums y[ow] += D[j][ow + j - P - c0] are taken
// with cross-lane reads (ds_bpermute): each lane gathers the elements of one
// diagonal from the lanes holding them and adds them in a fixed order into a
// per-wave fp32 row accumulator in LDS (one lane per output column: no
// atomics, bitwise reproducible).  v_mfma_f32_32x32x2_f32 multiplies and
// adds in fp32; it was measured at 130-144 TFLOP/s on the MI355X against
// 100-112 for the best v_fmac_f32 code.
//
// Lane layout of v_mfma_f32_32x32x2_f32 (checked on the MI355X): A lane l
// holds row l % 32, k = l / 32; B lane l holds column l % 32, k = l / 32;
// D register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4, column
// l % 32.  Instruction s takes kernel rows 2s (k = 0) and 2s + 1 (k = 1).
//
// A workgroup (4 waves) owns one output channel and a chunk of images; per
// band of output rows it stages the input rows the band reads (zero rows
// outside the image, zero columns up to a multiple of 32) and the waves take
// the band's output rows in turn.  Grad-input is the same correlation of dy
// with the filter flipped in both axes and padding k - 1 - pad (multiplier 1).
#include "dw_common.hpp"
#include "dw_internal.hpp"

namespace dw {
namespace {

typedef float f32x16_f __attribute__((ext_vector_type(16)));
typedef float f32x4_f __attribute__((ext_vector_type(4)));

constexpr int kF32K = 31;            // filter size this family serves
constexpr int kF32TargetWG = 6144;

template <typename T> struct Lf32Args {
    const T *in;    // forward: x; grad-input: dy
    const T *w;
    const T *b;     // forward bias or nullptr
    T *out;         // y or dx
    int N, C, Cin, mult;
    int IH, IW, OH, OW, P;
    int NC, npc;    // image chunks, images per chunk
    int BH, nbands; // output rows per band, bands per plane
    int NCT;        // 32-column tiles of an input row (its LDS pitch is 32 NCT)
    int OWP;        // floats of a wave's row accumulator
    int vin;        // input rows are whole aligned 16-byte vectors
};

__device__ __forceinline__ f32x16_f mfma_f32(float a, float b, f32x16_f c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Orders this wave's LDS accesses: its earlier LDS writes complete before any
// later LDS access of the wave (lanes read what other lanes of the wave wrote).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited on
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

template <typename T, int K, int NCT, bool FLIP>
__global__ __launch_bounds__(256, 6) void lk_fwd32_kernel(Lf32Args<T> a) {
    constexpr int XP = 32 * NCT;  // LDS pitch of a staged input row
    constexpr int NS = 16;  // instructions per 32-column tile: kernel rows 2s, 2s + 1
    static_assert(K <= 2 * NS, "one 32-row contraction covers the filter");
    extern __shared__ __align__(16) unsigned char smem[];
    const int xrows = a.BH + K;  // rows of a band, one zero row past the last kernel row
    float *xs = reinterpret_cast<float *>(smem);                  // [xrows][XP]
    float *yacc = xs + xrows * XP;                                // [4][OWP]
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the row loop branches on it
    const int lane = tid & 63;
    const int jl = lane & 31, h = lane >> 5;
    const int c = blockIdx.x / a.NC;
    const int chunk = blockIdx.x - c * a.NC;
    const int n0 = chunk * a.npc, n1 = min(n0 + a.npc, a.N);
    const int cin = FLIP ? c : c / a.mult;
    float *ya = yacc + wave * a.OWP;

    // A operand: w[i][j] at i = 2s + h, j = jl (the filter flipped in both
    // axes for grad-input), zero outside the k x k filter
    float wreg[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int i = 2 * s + h;
        float v = 0.f;
        if (i < K && jl < K) {
            const int si = FLIP ? K - 1 - i : i, sj = FLIP ? K - 1 - jl : jl;
            v = to_f32(a.w[(static_cast<int64_t>(c) * K + si) * K + sj]);
        }
        wreg[s] = v;
    }
    // the filter loads complete here: later waits in the loops then count only
    // LDS reads (output stores share the vector-memory counter with loads)
    __builtin_amdgcn_s_waitcnt(0);
    const float bias = (!FLIP && a.b) ? to_f32(a.b[c]) : 0.f;
    for (int e = tid; e < xrows * XP; e += 256) xs[e] = 0.f;
    for (int e = tid; e < 4 * a.OWP; e += 256) yacc[e] = 0.f;

    for (int n = n0; n < n1; ++n) {
        const T *ip = a.in + (static_cast<int64_t>(n) * a.Cin + cin) * a.IH * a.IW;
        T *op = a.out + (static_cast<int64_t>(n) * a.C + c) * a.OH * a.OW;
        for (int band = 0; band < a.nbands; ++band) {
            const int oh0 = band * a.BH;
            const int rows = min(a.BH, a.OH - oh0);
            const int srows = rows + K;
            __syncthreads();  // the previous band's reads are done
            // staged row r is input row oh0 + r - P (zeros outside the image)
            if (a.vin) {
                constexpr int VE = Vec<T>::N;
                const int vpr = a.IW / VE;
                for (int v = tid; v < srows * vpr; v += 256) {
                    const int r = v / vpr;
                    const int c0 = (v - r * vpr) * VE;
                    const int ih = oh0 + r - a.P;
                    union {
                        uint4 u;
                        T t[VE];
                    } raw;
                    raw.u = make_uint4(0u, 0u, 0u, 0u);
                    if (ih >= 0 && ih < a.IH) raw.u = *reinterpret_cast<const uint4 *>(ip + static_cast<int64_t>(ih) * a.IW + c0);
                    float *d = xs + r * XP + c0;
#pragma unroll
                    for (int e = 0; e < VE; ++e) d[e] = to_f32(raw.t[e]);
                }
            } else {
                for (int e = tid; e < srows * a.IW; e += 256) {
                    const int r = e / a.IW;
                    const int col = e - r * a.IW;
                    const int ih = oh0 + r - a.P;
                    xs[r * XP + col] = (ih >= 0 && ih < a.IH) ? to_f32(ip[static_cast<int64_t>(ih) * a.IW + col]) : 0.f;
                }
            }
            __syncthreads();
            // this wave's items: output row wave + 4 (q / NCT), column tile q % NCT,
            // each issued and then reduced: one accumulator and B operands read
            // four at a time keep the kernel at 71 VGPRs, seven waves per SIMD,
            // whose matrix work covers the others' reductions (8-10 % faster than
            // issuing item q + 1 before reducing item q at four waves per SIMD).
            const int nq = (rows > wave ? (rows - wave + 3) / 4 : 0) * NCT;
            auto issue = [&](f32x16_f &acc, int q) {
                const int r = wave + 4 * (q / NCT), ct = q % NCT;
                const int oh = oh0 + r;
                // kernel rows whose input row is inside the image; pairs with neither are skipped
                const int i_lo = max(0, a.P - oh), i_hi = min(K, a.IH + a.P - oh);
                const int s_lo = i_lo >> 1, s_hi = (i_hi + 1) >> 1;
                // every B operand row is in the staged band
                const float *bp = xs + (r + h) * XP + 32 * ct + jl;
#pragma unroll
                for (int u = 0; u < 16; ++u) acc[u] = 0.f;
                // B operands read four at a time (fewer live registers)
#pragma unroll
                for (int u0 = 0; u0 < NS; u0 += 4) {
                    float bv[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) bv[k] = bp[2 * (u0 + k) * XP];
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (u0 + k >= s_lo && u0 + k < s_hi) acc = mfma_f32(wreg[u0 + k], bv[k], acc);
                }
            };
            auto reduce = [&](const f32x16_f &acc, int q) {
                const int r = wave + 4 * (q / NCT), ct = q % NCT;
                // Lane (t, h) gathers, from register u of lane ((t + j) mod 32, h),
                // D[j][(t + j) mod 32] with j = 8 (u / 4) + 4 h + u % 4: the diagonal
                // c - j = t when t + j < 32, else t - 32.  j grows with u, so the
                // registers of diagonal t are a prefix of u: one running sum in a
                // fixed order, captured where the prefix ends; diagonal t - 32 gets
                // the total minus that prefix (two vector instructions per register
                // instead of four).
                float run = 0.f, spos = 0.f;
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int j = 8 * (u >> 2) + 4 * h + (u & 3);
                    const int src = ((jl + j) & 31) + 32 * h;
                    const float v = __int_as_float(
                        __builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(acc[u])));
                    run += v;
                    spos = (jl + j < 32) ? run : spos;
                }
                const float sneg = run - spos;
                // both halves' sums of a diagonal: lanes t (h = 0) and t + 32 (h = 1)
                const float opos = __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(spos)));
                const float oneg = __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(sneg)));
                // lane t adds diagonal t, lane t + 32 diagonal t - 32 (h = 0's sum first)
                const float tot = h == 0 ? spos + opos : oneg + sneg;
                const int ow = 32 * ct + jl - 32 * h + a.P;
                if (ow >= 0 && ow < a.OW) ya[ow] += tot;
                if (ct == NCT - 1) {  // the row is complete
                    wave_lds_sync();
                    T *yr = op + static_cast<int64_t>(oh0 + r) * a.OW;
                    for (int u = lane; u < a.OW; u += 64) {
                        yr[u] = from_f32<T>(ya[u] + bias);
                        ya[u] = 0.f;
                    }
                    wave_lds_sync();
                }
            };
            f32x16_f acc_a;
            for (int q = 0; q < nq; ++q) {
                issue(acc_a, q);
                reduce(acc_a, q);
            }
        }
    }
}

// The same split on 16 x 16 x 4 fp32 tiles (v_mfma_f32_16x16x4_f32), for rows
// whose width leaves at most half of a last 32-column tile used (48 = 32 + 16
// columns: 32-column tiles execute 64 columns' work, 16-column tiles 48).  A
// 16-column tile of one output row is two instructions per 4 kernel rows:
//   D_h[j][c] = sum_i w[i][16 h + j] X[oh + i - P][c0 + c],  h = 0, 1,
// A lane l holding j = l % 16, i = 4 u + l / 16 (16 filter registers per lane
// for the whole kernel); B lane l holding c = l % 16, i = 4 u + l / 16 (one
// 4-byte LDS read feeds both instructions); D register r of lane l holding
// j = 4 (l / 16) + r, c = l % 16 (layout checked on the MI355X).  Diagonal
// sums: lane (t, g) = (l % 16, l / 16) gathers D[j][(t + j) mod 16] for its 4
// rows j = 4 g + r (one ds_bpermute each within its 16-lane row, j growing
// with r so the diagonal-t terms are a prefix: running sum, captured), then
// the 4 rows of lanes are summed with v_permlane16_swap / v_permlane32_swap
// (both halves added in the same order in every lane).  Lane t then holds
// local diagonals t and t - 16 of each tile half; the three output columns a
// lane adds (diagonals t, t - 16, t - 32 of the 47 a tile touches) go to the
// wave's LDS row accumulator from lane rows 0, 1 and 2.
__device__ __forceinline__ f32x4_f mfma_f32x16(float a, float b, f32x4_f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// sum of v over the lanes l ^ 16, l ^ 32, l ^ 48 and l (fixed order, same in every lane)
__device__ __forceinline__ float rowsum4(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <typename T, int K, int NCT, bool FLIP>
__global__ __launch_bounds__(256, 8) void lk_fwd16t_kernel(Lf32Args<T> a) {
    constexpr int XP = 16 * NCT;  // LDS pitch of a staged input row
    constexpr int NU = 8;          // instructions per tile half: kernel rows 4u .. 4u + 3
    static_assert(K <= 4 * NU, "one 32-row contraction covers the filter");
    extern __shared__ __align__(16) unsigned char smem[];
    const int xrows = a.BH + K;
    float *xs = reinterpret_cast<float *>(smem);                  // [xrows][XP]
    float *yacc = xs + xrows * XP;                                // [4][OWP]
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int t = lane & 15, g = lane >> 4;
    const int c = blockIdx.x / a.NC;
    const int chunk = blockIdx.x - c * a.NC;
    const int n0 = chunk * a.npc, n1 = min(n0 + a.npc, a.N);
    const int cin = FLIP ? c : c / a.mult;
    float *ya = yacc + wave * a.OWP;

    // A operands: w[i][j] at i = 4u + g, j = 16 h + t (flipped for grad-input), zero outside
    float wreg[2][NU];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int i = 4 * u + g, j = 16 * hh + t;
            float v = 0.f;
            if (i < K && j < K) {
                const int si = FLIP ? K - 1 - i : i, sj = FLIP ? K - 1 - j : j;
                v = to_f32(a.w[(static_cast<int64_t>(c) * K + si) * K + sj]);
            }
            wreg[hh][u] = v;
        }
    __builtin_amdgcn_s_waitcnt(0);
    const float bias = (!FLIP && a.b) ? to_f32(a.b[c]) : 0.f;
    for (int e = tid; e < xrows * XP; e += 256) xs[e] = 0.f;
    for (int e = tid; e < 4 * a.OWP; e += 256) yacc[e] = 0.f;

    for (int n = n0; n < n1; ++n) {
        const T *ip = a.in + (static_cast<int64_t>(n) * a.Cin + cin) * a.IH * a.IW;
        T *op = a.out + (static_cast<int64_t>(n) * a.C + c) * a.OH * a.OW;
        for (int band = 0; band < a.nbands; ++band) {
            const int oh0 = band * a.BH;
            const int rows = min(a.BH, a.OH - oh0);
            const int srows = rows + K;
            __syncthreads();
            if (a.vin) {
                constexpr int VE = Vec<T>::N;
                const int vpr = a.IW / VE;
                for (int v = tid; v < srows * vpr; v += 256) {
                    const int r = v / vpr;
                    const int c0 = (v - r * vpr) * VE;
                    const int ih = oh0 + r - a.P;
                    union {
                        uint4 u;
                        T t[VE];
                    } raw;
                    raw.u = make_uint4(0u, 0u, 0u, 0u);
                    if (ih >= 0 && ih < a.IH) raw.u = *reinterpret_cast<const uint4 *>(ip + static_cast<int64_t>(ih) * a.IW + c0);
                    float *d = xs + r * XP + c0;
#pragma unroll
                    for (int e = 0; e < VE; ++e) d[e] = to_f32(raw.t[e]);
                }
            } else {
                for (int e = tid; e < srows * a.IW; e += 256) {
                    const int r = e / a.IW;
                    const int col = e - r * a.IW;
                    const int ih = oh0 + r - a.P;
                    xs[r * XP + col] = (ih >= 0 && ih < a.IH) ? to_f32(ip[static_cast<int64_t>(ih) * a.IW + col]) : 0.f;
                }
            }
            __syncthreads();
            // items: output row wave + 4 (q / NCT), 16-column tile q % NCT, each
            // issued and then reduced (53 VGPRs: eight waves per SIMD)
            const int nq = (rows > wave ? (rows - wave + 3) / 4 : 0) * NCT;
            auto issue = [&](f32x4_f &d0, f32x4_f &d1, int q) {
                const int r = wave + 4 * (q / NCT), ct = q % NCT;
                const int oh = oh0 + r;
                const int i_lo = max(0, a.P - oh), i_hi = min(K, a.IH + a.P - oh);
                const int u_lo = i_lo >> 2, u_hi = (i_hi + 3) >> 2;
                const float *bp = xs + (r + g) * XP + 16 * ct + t;
#pragma unroll
                for (int e = 0; e < 4; ++e) d0[e] = d1[e] = 0.f;
#pragma unroll
                for (int u0 = 0; u0 < NU; u0 += 4) {
                    float bv[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) bv[k] = bp[4 * (u0 + k) * XP];
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (u0 + k >= u_lo && u0 + k < u_hi) {
                            d0 = mfma_f32x16(wreg[0][u0 + k], bv[k], d0);
                            d1 = mfma_f32x16(wreg[1][u0 + k], bv[k], d1);
                        }
                }
            };
            auto reduce = [&](const f32x4_f &d0, const f32x4_f &d1, int q) {
                const int r = wave + 4 * (q / NCT), ct = q % NCT;
                // per tile half: lane (t, g) gathers D[4g + e][(t + 4g + e) mod 16] from
                // register e of lane 16 g + ((t + 4 g + e) & 15); the terms with
                // t + 4g + e < 16 are diagonal t (a prefix of e), the others t - 16
                float pos[2], neg[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    float run = 0.f, sp = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int jj = 4 * g + e;
                        const int src = 16 * g + ((t + jj) & 15);
                        const float dv = hh == 0 ? d0[e] : d1[e];
                        const float v = __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(dv)));
                        run += v;
                        sp = (t + jj < 16) ? run : sp;
                    }
                    pos[hh] = rowsum4(sp);
                    neg[hh] = rowsum4(run - sp);
                }
                // diagonals t (half 0 pos), t - 16 (half 0 neg + half 1 pos), t - 32 (half 1 neg)
                const float v = g == 0 ? pos[0] : g == 1 ? neg[0] + pos[1] : neg[1];
                const int ow = 16 * ct + t - 16 * g + a.P;
                if (g < 3 && ow >= 0 && ow < a.OW) ya[ow] += v;
                if (ct == NCT - 1) {
                    wave_lds_sync();
                    T *yr = op + static_cast<int64_t>(oh0 + r) * a.OW;
                    for (int u = lane; u < a.OW; u += 64) {
                        yr[u] = from_f32<T>(ya[u] + bias);
                        ya[u] = 0.f;
                    }
                    wave_lds_sync();
                }
            };
            f32x4_f a0, a1;
            for (int q = 0; q < nq; ++q) {
                issue(a0, a1, q);
                reduce(a0, a1, q);
            }
        }
    }
}

struct Lf32Plan {
    int NC, npc, BH, nbands, XP, OWP, lds_bytes, tile;
};

// Column tile of the input rows: 16 where a last 32-column tile would be at
// most half used.
inline int lf32_tile(int IW) {
    const int r = IW % 32;
    return (r != 0 && r <= 16) ? 16 : 32;
}

// ih x iw: input plane of this pass, oh x ow: its output plane
bool plan_lf32(int N, int C, int IH, int IW, int OH, int OW, Lf32Plan &p) {
    (void)IH;
    p.tile = lf32_tile(IW);
    p.XP = (IW + p.tile - 1) / p.tile * p.tile;
    p.OWP = (OW + 63) / 64 * 64;
    const int64_t fixed = 4LL * p.OWP * 4;
    auto bytes = [&](int bh) { return static_cast<int64_t>(bh + kF32K) * p.XP * 4 + fixed; };
    // bands of at most 32 rows within 40 KiB
    int bh = std::min(OH, 32);
    while (bh > 1 && bytes(bh) > 40 * 1024) --bh;
    if (bytes(bh) > 64 * 1024) return false;
    p.nbands = (OH + bh - 1) / bh;
    p.BH = (OH + p.nbands - 1) / p.nbands;
    p.lds_bytes = static_cast<int>(bytes(p.BH));
    int NC = std::max(1, (kF32TargetWG + C - 1) / C);
    NC = std::min(NC, N);
    p.npc = (N + NC - 1) / NC;
    p.NC = (N + p.npc - 1) / p.npc;
    return true;
}

template <typename T, bool FLIP>
int run_lf32(Lf32Args<T> a, const Lf32Plan &p, hipStream_t s) {
    a.NC = p.NC;
    a.npc = p.npc;
    a.BH = p.BH;
    a.nbands = p.nbands;
    a.NCT = p.XP / p.tile;
    a.OWP = p.OWP;
    a.vin = a.IW % Vec<T>::N == 0 && reinterpret_cast<uintptr_t>(a.in) % 16 == 0;
    const dim3 grid(a.C * p.NC), block(256);
    if (p.tile == 16) {
        // an odd count of 16-column tiles (the width leaves the last 32-column tile half used)
        switch (a.NCT) {
            case 1: hipLaunchKernelGGL((lk_fwd16t_kernel<T, kF32K, 1, FLIP>), grid, block, p.lds_bytes, s, a); break;
            case 3: hipLaunchKernelGGL((lk_fwd16t_kernel<T, kF32K, 3, FLIP>), grid, block, p.lds_bytes, s, a); break;
            case 5: hipLaunchKernelGGL((lk_fwd16t_kernel<T, kF32K, 5, FLIP>), grid, block, p.lds_bytes, s, a); break;
            case 7: hipLaunchKernelGGL((lk_fwd16t_kernel<T, kF32K, 7, FLIP>), grid, block, p.lds_bytes, s, a); break;
            case 9: hipLaunchKernelGGL((lk_fwd16t_kernel<T, kF32K, 9, FLIP>), grid, block, p.lds_bytes, s, a); break;
            case 11: hipLaunchKernelGGL((lk_fwd16t_kernel<T, kF32K, 11, FLIP>), grid, block, p.lds_bytes, s, a); break;
            case 13: hipLaunchKernelGGL((lk_fwd16t_kernel<T, kF32K, 13, FLIP>), grid, block, p.lds_bytes, s, a); break;
            default: hipLaunchKernelGGL((lk_fwd16t_kernel<T, kF32K, 15, FLIP>), grid, block, p.lds_bytes, s, a); break;
        }
        return hipGetLastError() == hipSuccess ? kOk : kErrHip;
    }
    switch (a.NCT) {
        case 1: hipLaunchKernelGGL((lk_fwd32_kernel<T, kF32K, 1, FLIP>), grid, block, p.lds_bytes, s, a); break;
        case 2: hipLaunchKernelGGL((lk_fwd32_kernel<T, kF32K, 2, FLIP>), grid, block, p.lds_bytes, s, a); break;
        case 3: hipLaunchKernelGGL((lk_fwd32_kernel<T, kF32K, 3, FLIP>), grid, block, p.lds_bytes, s, a); break;
        case 4: hipLaunchKernelGGL((lk_fwd32_kernel<T, kF32K, 4, FLIP>), grid, block, p.lds_bytes, s, a); break;
        case 5: hipLaunchKernelGGL((lk_fwd32_kernel<T, kF32K, 5, FLIP>), grid, block, p.lds_bytes, s, a); break;
        case 6: hipLaunchKernelGGL((lk_fwd32_kernel<T, kF32K, 6, FLIP>), grid, block, p.lds_bytes, s, a); break;
        case 7: hipLaunchKernelGGL((lk_fwd32_kernel<T, kF32K, 7, FLIP>), grid, block, p.lds_bytes, s, a); break;
        default: hipLaunchKernelGGL((lk_fwd32_kernel<T, kF32K, 8, FLIP>), grid, block, p.lds_bytes, s, a); break;
    }
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

}  // namespace

// fp32, 31 x 31 square filter, stride 1, dilation 1, the same padding on both
// axes (grad-input: multiplier 1 and pad <= k - 1), rows of at most 256.
bool largek_fwd32_fits(const Geo &g, int pass, int dtype) {
    if (dtype != 0) return false;
    if (g.kh != kF32K || g.kw != kF32K) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.ph != g.pw) return false;
    Lf32Plan p;
    if (pass == 1) {
        if (g.mult != 1 || g.ph > g.kh - 1 || g.ow > 256) return false;
        return plan_lf32(g.n, g.ic, g.oh, g.ow, g.ih, g.iw, p);
    }
    if (g.iw > 256) return false;
    return plan_lf32(g.n, g.oc, g.ih, g.iw, g.oh, g.ow, p);
}

// Whether the family is the better default: its tiles must be mostly input
// (32-column tiles on 48-column rows leave a quarter of the work empty and
// measured slower than the register-tile kernels: 1.49 against 1.44 ms at
// N64 C384 48 x 48; those rows take 16-column tiles).
bool largek_fwd32_preferred(const Geo &g, int pass) {
    const int iw = pass == 1 ? g.ow : g.iw;
    const int tile = lf32_tile(iw);
    return tile == 16 || 5 * iw >= 4 * tile * ((iw + tile - 1) / tile);
}

int largek_fwd32(const Geo &g, const void *x, const void *w, const void *b, void *y, hipStream_t s) {
    Lf32Plan p;
    if (!plan_lf32(g.n, g.oc, g.ih, g.iw, g.oh, g.ow, p)) return kErrUnsupported;
    Lf32Args<float> a{};
    a.in = static_cast<const float *>(x);
    a.w = static_cast<const float *>(w);
    a.b = static_cast<const float *>(b);
    a.out = static_cast<float *>(y);
    a.N = g.n;
    a.C = g.oc;
    a.Cin = g.ic;
    a.mult = g.mult;
    a.IH = g.ih;
    a.IW = g.iw;
    a.OH = g.oh;
    a.OW = g.ow;
    a.P = g.ph;
    return run_lf32<float, false>(a, p, s);
}

int largek_bwd_input32(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t s) {
    Lf32Plan p;
    if (!plan_lf32(g.n, g.ic, g.oh, g.ow, g.ih, g.iw, p)) return kErrUnsupported;
    Lf32Args<float> a{};
    a.in = static_cast<const float *>(dy);
    a.w = static_cast<const float *>(w);
    a.b = nullptr;
    a.out = static_cast<float *>(dx);
    a.N = g.n;
    a.C = g.ic;
    a.Cin = g.oc;
    a.mult = 1;
    a.IH = g.oh;
    a.IW = g.ow;
    a.OH = g.ih;
    a.OW = g.iw;
    a.P = g.kh - 1 - g.ph;
    return run_lf32<float, true>(a, p, s);
}

}  // namespace dw
