// dw_largek_rollf32.hip -- large-kernel (k = 31) depthwise forward and
// grad-input for fp32 I/O on the gfx950 matrix cores, streaming input rows
// (stride 1, dilation 1, any plane size).
//
// The formulation is the 16-bit one of dw_largek_roll16.hip (MegEngine
// large-kernel depthwise article, its im2col problem statement and implicit
// GEMM): input row v, read once, adds to output row oh = v + P - i for every
// kernel row i at once, D[i][ow] = sum_j A[i][j] B[j][ow] with A the filter
// (M = kernel rows, K = kernel columns) and B[j][ow] = X[v][ow + j - P].  An
// accumulator row m of a 16-row block keeps one output row while the block's
// 16 kernel rows pass; the filter rows rotate one lane per input row (DPP),
// and a row's partial sum moves from block 0 to block 1 in place.  Only the
// multiply-adds of kernel rows and columns that fall outside the plane, and
// the 32nd kernel row and column, are executed beyond the useful ones; nothing
// is reduced across lanes afterwards.
//
// Why not the kernel-row contraction of dw_largek_fwd32.hip here: the fp32
// matrix instructions do not run alongside vector instructions on the same
// SIMD (the co-execution counter stays at zero for them, where 16-bit matrix
// work overlaps), so the anti-diagonal sums that contraction needs -- five to
// six vector instructions per matrix instruction -- add to the matrix time.
// Streaming rows needs about one vector instruction per eight matrix ones.
//
// v_mfma_f32_16x16x4_f32 lane layout (checked on the MI355X): A lane l holds
// row l % 16, k = l / 16; B lane l holds column l % 16, k = l / 16; D register
// r of lane l holds row 4 (l / 16) + r, column l % 16.  Instruction J of an
// input row takes kernel columns j = 8 k + J (k = 0 .. 3): lane (n, k) then
// reads 8 adjacent staged values for its 8 instructions.
//
// One wave streams one (channel, 16 NT-column chunk) of an image: input rows
// arrive R at a time (R = 2 or 4) from 16-byte buffer loads one batch ahead,
// into an LDS ring of the wave's own (two batches).  Grad-input is the same
// correlation of dy with the filter flipped in both axes and padding
// k - 1 - pad.
#include "dw_common.hpp"
#include "dw_internal.hpp"

#include <type_traits>

namespace dw {
namespace {

typedef float f32x4_r __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_r __attribute__((ext_vector_type(4)));

constexpr int kRfK = 31;               // filter size this family serves
constexpr int kRfSkip = 0x40000000;    // an offset past every plane (planes are below 1 GiB)

struct RfArgs {
    const float *in;  // forward: x; grad-input: dy
    const float *w;
    const float *b;   // forward bias or nullptr
    float *out;       // y or dx
    int N, C, Cin, mult;
    int IH, IW, OH, OW, P;
    int nchunk;       // column chunks of an output row (16 NT columns each)
    int ipw;          // images per wave
    int nimgw;        // image groups of a (channel, chunk): ceil(N / ipw)
    int nwaves;       // C * nchunk * nimgw
    int vin;          // input rows are whole aligned 16-byte vectors
};

// Staged row of an NT-tile chunk: window position 0 (input column c_lo - P)
// sits at staged position AL (0 .. 3, the shift to a 16-byte boundary); a
// step reads positions AL .. AL + 16 NT + 30 + 3.  NV 4-value vectors cover
// them; a batch of R rows takes NVP lanes a row.
template <int NT> struct RfGeo {
    static constexpr int NV = (16 * NT + kRfK + 3 + 3) / 4;  // vectors a staged row
    static constexpr int NVP = NV <= 16 ? 16 : 32;           // staging lanes a row
    static constexpr int R = 64 / NVP;                        // rows a batch
    static constexpr int SLOTS = 2 * R;                       // ring rows: two batches
    static constexpr int RP = 4 * NV + 4;                     // dwords a ring row (16-byte multiple)
    static constexpr int lds_bytes = 4 * SLOTS * RP * 4;      // four waves
};

__device__ __forceinline__ void rf_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Lane l takes lane (l - 1) mod 16 of its 16-lane row (DPP row_ror:1), every lane enabled.
__device__ __forceinline__ float rf_rot(float v) {
    int r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xf, 0xf, true);
    asm volatile("" : "+v"(r));
    return __int_as_float(r);
}

template <int NT, bool FLIP, bool VIN>
__global__ __launch_bounds__(256) void lk_rollf32_kernel(RfArgs a) {
    using G = RfGeo<NT>;
    constexpr int K = kRfK;
    constexpr int NB = 2;   // 16-row blocks of kernel rows
    constexpr int NJ = 8;   // instructions an input row: kernel columns 8 k + J
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wid = blockIdx.x * 4 + wave;
    if (wid >= a.nwaves) return;  // whole waves; the kernel has no workgroup barrier
    float *ring = reinterpret_cast<float *>(smem) + wave * G::SLOTS * G::RP;

    const int per_c = a.nchunk * a.nimgw;
    const int c = wid / per_c;
    const int rem = wid - c * per_c;
    const int chunk = rem / a.nimgw;
    const int ig = rem - chunk * a.nimgw;
    const int n0 = ig * a.ipw, n1 = min(n0 + a.ipw, a.N);
    const int cin = FLIP ? c : c / a.mult;
    const int c_lo = chunk * 16 * NT;   // first output column of the chunk
    const int cb = c_lo - a.P;          // input column of window position 0
    const int cb4 = cb & ~3;            // rounded down to a multiple of 4
    const int AL = cb - cb4;            // its staged position

    const int n = lane & 15, g = lane >> 4;
    const int boff = AL + n + 8 * g;    // staged position of instruction 0's B value, tile 0
    // staging lane: row rr of the batch, vector sk (lanes past the last vector
    // repeat it: same load, same LDS write); vectors outside the plane and
    // rows past it read zeros (offsets past the buffer's range)
    const int rr = lane / G::NVP;
    const int sk = min(lane % G::NVP, G::NV - 1);
    const int gc = cb4 + 4 * sk;
    const bool vk = gc >= 0 && gc + 4 <= a.IW;
    const int lbase = vk ? (rr * a.IW + gc) * 4 : kRfSkip;
    const int bstep = G::R * a.IW * 4;

    const float bias = (!FLIP && a.b) ? a.b[c] : 0.f;
    const float *wc = a.w + static_cast<int64_t>(c) * K * K;
    const int64_t iplane = static_cast<int64_t>(a.IH) * a.IW;
    // steps in groups of four (rows past the plane are zero)
    const int nv = (a.IH + 3) & ~3;
    const int nq = nv / G::R;  // batches

    for (int nimg = n0; nimg < n1; ++nimg) {
        const float *ip = a.in + (static_cast<int64_t>(nimg) * a.Cin + cin) * iplane;
        float *op = a.out + (static_cast<int64_t>(nimg) * a.C + c) * a.OH * a.OW;
        const __amdgpu_buffer_rsrc_t irsrc =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(ip), 0, static_cast<int>(iplane * 4), 0x00020000);
        const __amdgpu_buffer_rsrc_t orsrc =
            __builtin_amdgcn_make_buffer_rsrc(op, 0, a.OH * a.OW * 4, 0x00020000);

        // Step v consumes input row v.  Accumulator row m of block b then holds
        // output row v + P - i with kernel row i = 16 b + ((v - m) mod 16): lane
        // (m, k) of instruction J's A holds w[i][8 k + J] (zero past the filter).
        float A[NB][NJ];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int i = 16 * b + ((-n) & 15);
#pragma unroll
            for (int J = 0; J < NJ; ++J) {
                const int j = 8 * g + J;
                float v = 0.f;
                if (i < K && j < K) v = FLIP ? wc[(K - 1 - i) * K + (K - 1 - j)] : wc[i * K + j];
                A[b][J] = v;
            }
        }
        f32x4_r d[NB][NT];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int t = 0; t < NT; ++t) d[b][t] = f32x4_r{bias, bias, bias, bias};

        auto load_batch = [&](int qb) -> u32x4_r {
            return __builtin_amdgcn_raw_buffer_load_b128(irsrc, lbase + qb * bstep, 0, 0);
        };
        auto write_batch = [&](int qb, const u32x4_r &raw) {
            const int slot = (qb * G::R + rr) & (G::SLOTS - 1);
            *reinterpret_cast<u32x4_r *>(ring + slot * G::RP + 4 * sk) = raw;
        };
        // element-wise staging (rows that are not whole aligned vectors)
        auto stage_scalar = [&](int qb) {
            constexpr int SP = 4 * G::NV;
            for (int e = lane; e < G::R * SP; e += 64) {
                const int q = e / SP;
                const int p = e - q * SP;
                const int r = qb * G::R + q;
                const int col = cb4 + p;
                const float v = (r < a.IH && col >= 0 && col < a.IW) ? ip[static_cast<int64_t>(r) * a.IW + col] : 0.f;
                ring[((qb * G::R + q) & (G::SLOTS - 1)) * G::RP + p] = v;
            }
        };

        u32x4_r raw = u32x4_r{0u, 0u, 0u, 0u};
        if constexpr (VIN) {
            write_batch(0, load_batch(0));
            if (nq > 1) raw = load_batch(1);
        } else {
            stage_scalar(0);
        }

        auto step = [&](auto rr_c, int v) {
            constexpr int RR = decltype(rr_c)::value;  // v mod 4
            const float *bp = ring + (v & (G::SLOTS - 1)) * G::RP + boff;
            // accumulator row v mod 16 (register RR of lane row (v / 4) mod 4): the
            // last block's output row v + P - 32 is complete, block 1 takes block
            // 0's partial sum, block 0 starts output row v + P at its bias
            const bool sel = g == ((v >> 2) & 3);
            float e[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                e[t] = d[1][t][RR];
                d[1][t][RR] = sel ? d[0][t][RR] : d[1][t][RR];
                d[0][t][RR] = sel ? bias : d[0][t][RR];
            }
            const int oh = v + a.P - 16 * NB;
            const int ub = (sel && oh >= 0 && oh < a.OH) ? (oh * a.OW + c_lo + n) * 4 : kRfSkip;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(e[t]), orsrc,
                                                      c_lo + 16 * t + n < a.OW ? ub + 64 * t : kRfSkip, 0, 0);
            // instruction J: kernel columns 8 k + J of both blocks and every tile
#pragma unroll
            for (int J = 0; J < NJ; ++J) {
                float bv[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t) bv[t] = bp[16 * t + J];
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        d[b][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[b][J], bv[t], d[b][t], 0, 0, 0);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int J = 0; J < NJ; ++J) A[b][J] = rf_rot(A[b][J]);
        };
        // batch boundary before step v (v a multiple of R): batch v / R is in
        // the ring once this wave's LDS writes are done; the next one is staged
        auto stage_next = [&](int qv) {
            rf_lds_sync();
            if (qv + 1 < nq) {
                if constexpr (VIN) {
                    write_batch(qv + 1, raw);
                    if (qv + 2 < nq) raw = load_batch(qv + 2);
                } else {
                    stage_scalar(qv + 1);
                }
            }
        };

        for (int v0 = 0; v0 < nv; v0 += 4) {
            stage_next(v0 / G::R);
            step(std::integral_constant<int, 0>{}, v0);
            step(std::integral_constant<int, 1>{}, v0 + 1);
            if constexpr (G::R == 2) stage_next(v0 / G::R + 1);  // rows v0 + 2, v0 + 3: the next batch
            step(std::integral_constant<int, 2>{}, v0 + 2);
            step(std::integral_constant<int, 3>{}, v0 + 3);
        }
        rf_lds_sync();  // the ring's reads are done before the next image writes it

        // every output row still in an accumulator is complete: input rows past
        // the plane add nothing
        const int vl = nv - 1;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * g + r;
                const int oh = vl + a.P - 16 * b - ((vl - m) & 15);
                if (oh < 0 || oh >= a.OH) continue;
                float *orow = op + static_cast<int64_t>(oh) * a.OW + c_lo + n;
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    if (c_lo + 16 * t + n < a.OW) orow[16 * t] = d[b][t][r];
            }
    }
}

template <int NT, bool FLIP>
int run_rf_t(RfArgs a, hipStream_t s) {
    using G = RfGeo<NT>;
    a.nchunk = (a.OW + 16 * NT - 1) / (16 * NT);
    // one image a wave (many waves leave no partial last round of resident
    // waves), a few where there are more than 2^18 of them
    const int64_t items = static_cast<int64_t>(a.C) * a.nchunk;
    const int64_t want = std::max<int64_t>(1, (static_cast<int64_t>(a.N) * items) >> 18);
    a.ipw = static_cast<int>(std::min<int64_t>(want, a.N));
    a.nimgw = (a.N + a.ipw - 1) / a.ipw;
    const int64_t nw = items * a.nimgw;
    if (nw > (int64_t{1} << 30)) return kErrUnsupported;
    a.nwaves = static_cast<int>(nw);
    const dim3 grid(static_cast<unsigned>((nw + 3) / 4));
    if (a.vin)
        hipLaunchKernelGGL((lk_rollf32_kernel<NT, FLIP, true>), grid, dim3(256), G::lds_bytes, s, a);
    else
        hipLaunchKernelGGL((lk_rollf32_kernel<NT, FLIP, false>), grid, dim3(256), G::lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <bool FLIP>
int run_rf(const RfArgs &a, hipStream_t s) {
    const int nt = std::min(4, (a.OW + 15) / 16);
    if (nt == 1) return run_rf_t<1, FLIP>(a, s);
    if (nt == 2) return run_rf_t<2, FLIP>(a, s);
    if (nt == 3) return run_rf_t<3, FLIP>(a, s);
    return run_rf_t<4, FLIP>(a, s);
}

}  // namespace

// fp32, k = 31 square, stride 1, dilation 1, equal paddings below k; the
// grad-input pass with multiplier 1.  Any plane size.
bool largek_rollf32_fits(const Geo &g, int pass, int dtype) {
    if (dtype != 0) return false;
    if (g.kh != kRfK || g.kw != kRfK) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.ph != g.pw || g.ph > g.kh - 1) return false;
    if (pass == 1 && g.mult != 1) return false;
    // input and output planes addressed by 32-bit buffer offsets below 1 GiB
    const int64_t ip = static_cast<int64_t>(g.ih) * g.iw, op = static_cast<int64_t>(g.oh) * g.ow;
    return g.oh >= 1 && g.ow >= 1 && std::max(ip, op) * 4 < (int64_t{1} << 30);
}

int largek_rollf32_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, hipStream_t s) {
    RfArgs a{};
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
    a.vin = a.IW % 4 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
    return run_rf<false>(a, s);
}

int largek_rollf32_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t s) {
    RfArgs a{};
    a.in = static_cast<const float *>(dy);
    a.w = static_cast<const float *>(w);
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
    a.vin = a.IW % 4 == 0 && reinterpret_cast<uintptr_t>(dy) % 16 == 0;
    return run_rf<true>(a, s);
}

}  // namespace dw
