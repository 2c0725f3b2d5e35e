// dw_largek_roll16.hip -- large-kernel (k = 31) depthwise forward and
// grad-input for 16-bit I/O on the gfx950 matrix cores, streaming input rows
// (stride 1, dilation 1, any plane size).
//
// The MegEngine large-kernel depthwise article writes depthwise convolution as
// an implicit GEMM (its im2col problem statement and ImplicitBatchedGEMM
// section).  Here the contraction is taken over kernel columns, one input row
// at a time: input row r, read once, adds to output row oh = r + P - i
//   U_i[ow] = sum_j w[i][j] X[r][ow + j - P]
// for every kernel row i at once -- a product D[i][ow] = sum_j A[i][j] B[j][ow]
// with A the filter (M = kernel rows, K = kernel columns) and B a Hankel matrix
// of the input row (B[j][ow] = X[r][ow + j - P]: each lane reads 8 adjacent
// values of the staged row).  Each row of D belongs to a different output row;
// rather than moving partial sums, the rows of A rotate: an accumulator row m
// of a 16-row block keeps one output row (oh = m mod 16) for the 16 input rows
// that block's kernel rows cover, and at input row u - P holds kernel row
//   i = 16 b + ((u - m) mod 16)        (block b = 0, 1 for k = 31),
// so from one input row to the next every lane of A takes its neighbour's
// filter row (one DPP row rotation per register).  When an output row has had
// its 16 kernel rows of block 0 its partial sum moves into block 1's register
// of the same row; when block 1 is done the row is complete and is stored.
// Only the multiply-adds of kernel columns and rows that fall outside the
// plane are executed beyond the useful ones (and the 32nd kernel row and
// column), not the k / (16 + k - 1) band of a Toeplitz tile.
//
// v_mfma_f32_16x16x32_{f16,bf16} lane layout (checked on the MI355X): A lane l
// holds row l % 16, k = 8 (l / 16) .. + 8; B lane l holds column l % 16, the
// same k; D register r of lane l holds row 4 (l / 16) + r, column l % 16.
// Products of 16-bit values are exact and sums are fp32.
//
// One wave streams one (channel, 16 NT-column chunk) of a few images: input
// rows arrive four at a time from 16-byte global loads one batch ahead, into
// an LDS ring of the wave's own (two batches; each row stored twice, the
// second copy shifted by one element so that every 8-value run starts on a
// 4-byte boundary).  Grad-input is the same correlation of dy with the filter
// flipped in both axes and padding k - 1 - pad.
#include "dw_common.hpp"
#include "dw_internal.hpp"

#include <type_traits>

namespace dw {
namespace {

typedef _Float16 f16x8_r __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_r __attribute__((ext_vector_type(8)));
typedef float f32x4_r __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_r __attribute__((ext_vector_type(4)));

template <typename T> struct RollMfma;
template <> struct RollMfma<__half> {
    static __device__ __forceinline__ f32x4_r run(u32x4_r a, u32x4_r b, f32x4_r c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_r, a), __builtin_bit_cast(f16x8_r, b),
                                                      c, 0, 0, 0);
    }
};
template <> struct RollMfma<bf16_t> {
    static __device__ __forceinline__ f32x4_r run(u32x4_r a, u32x4_r b, f32x4_r c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_r, a),
                                                       __builtin_bit_cast(bf16x8_r, b), c, 0, 0, 0);
    }
};

constexpr int kR16K = 31;     // filter size this family serves

template <typename T> struct Lr16Args {
    const T *in;  // forward: x; grad-input: dy
    const T *w;
    const T *b;   // forward bias or nullptr
    T *out;       // y or dx
    int N, C, Cin, mult;
    int IH, IW, OH, OW, P;
    int nchunk;   // column chunks of an output row (16 NT columns each)
    int ipw;      // images per wave
    int nimgw;    // image groups of a (channel, chunk): ceil(N / ipw)
    int nwaves;   // C * nchunk * nimgw
    int vin;      // input rows are whole aligned 16-byte vectors
};

// Staged row geometry of an NT-tile chunk (16 NT columns): XW input columns;
// copy 0 at halves [0, XP) (room for the alignment shift and the 8-value runs'
// ends), copy 1 from dword D1 (its position -1 included).  Dword d of ring
// slot k sits at ring dword 9 d + k: every dword a step reads is one base
// register plus an immediate below 256 (one ds_read2_b32 per two dwords, for
// any slot).  With 32 banks, two lanes of a half-wave reading dwords d (copy 0)
// and D1 + d' (copy 1) share a bank when 9 d = 9 (D1 + d') mod 32, i.e.
// d - d' = D1 mod 32; 32 lanes whose runs start at 32 consecutive positions
// give d - d' in [-15, 15] (even first position) or [-14, 16] (odd), so copy 1
// starts at a dword = 16 mod 32, one dword later for an odd first position.
template <int K, int NT, int NSLOT> struct Lr16Geo {
    static constexpr int SLOTS = NSLOT;   // ring rows (input rows in flight)
    static constexpr int RS = SLOTS + 1;  // ring stride: dword d of slot k at RS d + k (RS odd)
    static_assert(SLOTS == 8 || SLOTS == 16, "two or four batches of four rows");
    static constexpr int XW = 16 * NT + K - 1;
    static constexpr int XP = (XW + 23 + 7) / 8 * 8;
    static constexpr int D1 = (XP / 2 + 1 + 15) / 32 * 32 + 16;  // copy 1's first dword (+1 for an odd start)
    static constexpr int ROWD = D1 + 1 + XP / 2;  // dwords of a staged row, both copies
    static constexpr int RING = RS * ROWD;    // dwords of a wave's ring
    static constexpr int NVEC = (XW + 7 + 7) / 8;  // 8-column vectors a row may need
    static_assert(NVEC <= 16, "a staged row is loaded by 16 lanes");
    static constexpr int lds_bytes = 4 * RING * 4;
};

// Ring dword of the lane's B-operand run starting at staged position s0
// (copy 1 from dword d1).
template <int RS> __device__ __forceinline__ int ring_run(int s0, int d1) {
    return RS * ((s0 & 1) ? d1 + ((s0 - 1) >> 1) : (s0 >> 1));
}

// Stages one 8-value vector (raw, staged positions 8 sk .. 8 sk + 7) of slot k:
// copy 0, and copy 1 from dword d1 (its position q holds copy-0 position q + 1).
template <int RS> __device__ __forceinline__ void ring_put_vec(uint32_t *ring, int d1, int k, int sk, const uint4 &raw) {
    uint32_t *p0 = ring + RS * (4 * sk) + k;
    p0[0] = raw.x;
    p0[RS] = raw.y;
    p0[2 * RS] = raw.z;
    p0[3 * RS] = raw.w;
    uint32_t *p1 = ring + RS * (d1 + 4 * sk) + k;
    reinterpret_cast<uint16_t *>(p1 - RS)[1] = static_cast<uint16_t>(raw.x);  // position 8 sk - 1
    p1[0] = __builtin_amdgcn_alignbit(raw.y, raw.x, 16);
    p1[RS] = __builtin_amdgcn_alignbit(raw.z, raw.y, 16);
    p1[2 * RS] = __builtin_amdgcn_alignbit(raw.w, raw.z, 16);
    reinterpret_cast<uint16_t *>(p1 + 3 * RS)[0] = static_cast<uint16_t>(raw.w >> 16);  // position 8 sk + 6
}

// Stages one value at staged position p of slot k (both copies).
template <int RS> __device__ __forceinline__ void ring_put_one(uint32_t *ring, int d1, int k, int p, uint16_t v) {
    reinterpret_cast<uint16_t *>(ring + RS * (p >> 1) + k)[p & 1] = v;
    const int q = 2 * d1 + p - 1;
    reinterpret_cast<uint16_t *>(ring + RS * (q >> 1) + k)[q & 1] = v;
}

// Orders this wave's LDS accesses: its earlier LDS operations complete before
// any later one (lanes read what other lanes of the wave wrote).
__device__ __forceinline__ void roll_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Lane l takes lane (l - 1) mod 16 of its 16-lane row (DPP row_ror:1), every lane enabled.
__device__ __forceinline__ uint32_t rot_row(uint32_t v) {
    uint32_t r = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x121, 0xf, 0xf, true));
    asm volatile("" : "+v"(r));
    return r;
}

// Input rows are read and output rows written with raw buffer accesses: a
// lane with nothing to load or store gives an offset past the plane, which the
// hardware's range check turns into zeros (loads) or drops (stores): no branch
// around the access.
constexpr int kR16Skip = 0x40000000;  // planes are below 1 GiB

__device__ __forceinline__ uint16_t bits16(float v, __half *) { return __half_as_ushort(__float2half_rn(v)); }
__device__ __forceinline__ uint16_t bits16(float v, bf16_t *) { return from_f32<bf16_t>(v).bits; }

template <typename T, int K, int NT, bool FLIP, bool VIN>
__global__ __launch_bounds__(256) void lk_roll16_kernel(Lr16Args<T> a) {
    using G = Lr16Geo<K, NT, 8>;
    constexpr int NB = (K + 15) / 16;  // 16-row blocks of kernel rows
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wid = blockIdx.x * 4 + wave;
    if (wid >= a.nwaves) return;  // whole waves; the kernel has no workgroup barrier
    uint32_t *ring = reinterpret_cast<uint32_t *>(smem) + wave * G::RING;

    const int per_c = a.nchunk * a.nimgw;
    const int c = wid / per_c;
    const int rem = wid - c * per_c;
    const int chunk = rem / a.nimgw;
    const int ig = rem - chunk * a.nimgw;
    const int n0 = ig * a.ipw, n1 = min(n0 + a.ipw, a.N);
    const int cin = FLIP ? c : c / a.mult;
    const int c_lo = chunk * 16 * NT;   // first output column of the chunk
    const int cb = c_lo - a.P;          // input column of window position 0
    const int cb8 = cb & ~7;            // rounded down to a multiple of 8
    const int AL = cb - cb8;            // staged position of window position 0

    const int n = lane & 15, g = lane >> 4;
    const int n2 = n * static_cast<int>(sizeof(T));
    // B operand: staged position s = AL + 16 t + n + 8 g; odd runs read copy 1
    const int s0 = AL + n + 8 * g;
    const int d1 = G::D1 + (AL & 1);  // copy 1's first dword
    const int boff = ring_run<G::RS>(s0, d1);
    // staging: lane = (row of the batch, 8-column vector)
    const int sk = lane & 15;
    const int gc = cb8 + 8 * sk;
    const bool vk = sk < G::NVEC && gc >= 0 && gc + 8 <= a.IW;

    for (int e = lane; e < G::RING; e += 64) ring[e] = 0u;
    roll_lds_sync();

    const float bias = (!FLIP && a.b) ? to_f32(a.b[c]) : 0.f;
    const uint16_t *wc = reinterpret_cast<const uint16_t *>(a.w) + static_cast<int64_t>(c) * K * K;
    const int64_t iplane = static_cast<int64_t>(a.IH) * a.IW;
    const int nq = (a.IH + 3) >> 2;  // batches of four input rows (rows past the plane are zero)
    const bool colfull = c_lo + 16 * NT <= a.OW;  // every tile column is inside the row

    for (int nimg = n0; nimg < n1; ++nimg) {
        const uint16_t *ip = reinterpret_cast<const uint16_t *>(a.in) + (static_cast<int64_t>(nimg) * a.Cin + cin) * iplane;
        T *op = a.out + (static_cast<int64_t>(nimg) * a.C + c) * a.OH * a.OW;
        const __amdgpu_buffer_rsrc_t orsrc =
            __builtin_amdgcn_make_buffer_rsrc(op, 0, a.OH * a.OW * static_cast<int>(sizeof(T)), 0x00020000);

        // Step v consumes input row v.  Accumulator row m of block b then holds
        // output row v + P - i with kernel row i = 16 b + ((v - m) mod 16): lane
        // (m, g) of A holds w[i][8 g .. 8 g + 7] (zero past the filter).
        u32x4_r A[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int i = 16 * b + ((-n) & 15);
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) {
                uint32_t v = 0;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int j = 8 * g + 2 * k2 + hh;
                    if (i < K && j < K) {
                        const uint16_t bits = FLIP ? wc[(K - 1 - i) * K + (K - 1 - j)] : wc[i * K + j];
                        v |= static_cast<uint32_t>(bits) << (16 * hh);
                    }
                }
                A[b][k2] = v;
            }
        }
        f32x4_r d[NB][NT];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int t = 0; t < NT; ++t) d[b][t] = f32x4_r{bias, bias, bias, bias};  // each output row starts at its bias

        // batch qb = input rows 4 qb .. 4 qb + 3, lane row lane / 16; zeros past the plane
        // rows past the plane and vectors outside it read as zeros (buffer range
        // check): the load has no branch, so nothing waits for it before the
        // batch is written to the ring
        const __amdgpu_buffer_rsrc_t irsrc =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(ip), 0, static_cast<int>(iplane * 2), 0x00020000);
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        auto load_batch = [&](int qb) {
            const int r = 4 * qb + (lane >> 4);
            const int off = (vk && r < a.IH) ? (r * a.IW + gc) * 2 : kR16Skip;
            const u32x4_r v = __builtin_amdgcn_raw_buffer_load_b128(irsrc, off, 0, 0);
            raw = make_uint4(v[0], v[1], v[2], v[3]);
        };
        auto write_batch = [&](int qb) {
            if (vk) ring_put_vec<G::RS>(ring, d1, (4 * qb + (lane >> 4)) & (G::SLOTS - 1), sk, raw);
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
                ring_put_one<G::RS>(ring, d1, (4 * qb + q) & (G::SLOTS - 1), p, v);
            }
        };

        if constexpr (VIN) {
            load_batch(0);
            write_batch(0);
            if (nq > 1) load_batch(1);
        } else {
            stage_scalar(0);
        }

        auto step = [&](auto rr_c, int v) {
            constexpr int rr = decltype(rr_c)::value;
            // B operands first: their LDS latency overlaps the accumulator bookkeeping
            const uint32_t *bp = ring + boff + (v & (G::SLOTS - 1));
            u32x4_r bv[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint32_t *q = bp + G::RS * 8 * t;
                bv[t] = u32x4_r{q[0], q[G::RS], q[2 * G::RS], q[3 * G::RS]};
            }
            // accumulator row v mod 16 (register rr of lane row (v / 4) mod 4): the
            // last block's output row v + P - 16 NB is complete, each block takes
            // the previous block's partial sum, block 0 starts output row v + P
            const bool sel = g == ((v >> 2) & 3);
            float e[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                e[t] = d[NB - 1][t][rr];
#pragma unroll
                for (int b = NB - 1; b > 0; --b) d[b][t][rr] = sel ? d[b - 1][t][rr] : d[b][t][rr];
                d[0][t][rr] = sel ? bias : d[0][t][rr];
            }
            const int oh = v + a.P - 16 * NB;
            const int ub = (oh >= 0 && oh < a.OH) ? (oh * a.OW + c_lo) * static_cast<int>(sizeof(T)) : kR16Skip;
            const int off = sel ? ub + n2 : kR16Skip;
            if (colfull) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    __builtin_amdgcn_raw_buffer_store_b16(bits16(e[t], static_cast<T *>(nullptr)), orsrc, off + 32 * t, 0, 0);
            } else {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    __builtin_amdgcn_raw_buffer_store_b16(bits16(e[t], static_cast<T *>(nullptr)), orsrc,
                                                          c_lo + 16 * t + n < a.OW ? off + 32 * t : kR16Skip, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int b = 0; b < NB; ++b) d[b][t] = RollMfma<T>::run(A[b], bv[t], d[b][t]);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) A[b][k2] = rot_row(A[b][k2]);
        };

        for (int q = 0; q < nq; ++q) {
            roll_lds_sync();  // batch q is in the ring; batch q - 1's reads are done
            if (q + 1 < nq) {
                if constexpr (VIN) {
                    write_batch(q + 1);
                    if (q + 2 < nq) load_batch(q + 2);
                } else {
                    stage_scalar(q + 1);
                }
            }
            const int v = 4 * q;
            step(std::integral_constant<int, 0>{}, v);
            step(std::integral_constant<int, 1>{}, v + 1);
            step(std::integral_constant<int, 2>{}, v + 2);
            step(std::integral_constant<int, 3>{}, v + 3);
        }
        roll_lds_sync();  // the ring's reads are done before the next image writes it

        // every output row still in an accumulator is complete: input rows past
        // the plane add nothing
        const int vl = 4 * nq - 1;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int m = 4 * g + rr;
                const int oh = vl + a.P - 16 * b - ((vl - m) & 15);
                if (oh < 0 || oh >= a.OH) continue;
                T *orow = op + static_cast<int64_t>(oh) * a.OW + c_lo + n;
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    if (c_lo + 16 * t + n < a.OW) orow[16 * t] = from_f32<T>(d[b][t][rr]);
            }
    }
}

// The same streaming on 32 x 32 x 16 tiles for rows whose width is a
// multiple of 32: one instruction covers all 32 kernel-row slots of a 32-column
// tile (lanes 0-15 of each half hold block 0's slots, lanes 16-31 block 1's, so
// the rotation stays inside 16-lane DPP rows), and a block's partial sum moves
// to the other block inside one lane (registers r and r + 8).  Per input row
// and 64 columns: 4 instructions, 8 rotations, 4 selects and 2 stores,
// against 8, 8, 8 and 4 on 16-column tiles.
// v_mfma_f32_32x32x16_{f16,bf16} lane layout (checked on the MI355X): A lane l
// holds row l % 32, k = 8 (l / 32) .. + 8; B lane l holds column l % 32, the
// same k; D register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.
typedef float f32x16_r __attribute__((ext_vector_type(16)));
template <typename T> struct RollMfma32;
template <> struct RollMfma32<__half> {
    static __device__ __forceinline__ f32x16_r run(u32x4_r a, u32x4_r b, f32x16_r c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_r, a), __builtin_bit_cast(f16x8_r, b),
                                                      c, 0, 0, 0);
    }
};
template <> struct RollMfma32<bf16_t> {
    static __device__ __forceinline__ f32x16_r run(u32x4_r a, u32x4_r b, f32x16_r c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_r, a),
                                                       __builtin_bit_cast(bf16x8_r, b), c, 0, 0, 0);
    }
};

template <typename T, int K, int NT, bool FLIP, bool VIN>
__global__ __launch_bounds__(256) void lk_roll32_kernel(Lr16Args<T> a) {
    static_assert(K > 16 && K <= 32, "two 16-row blocks of kernel rows");
    using G = Lr16Geo<K, 2 * NT, 8>;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wid = blockIdx.x * 4 + wave;
    if (wid >= a.nwaves) return;  // whole waves; the kernel has no workgroup barrier
    uint32_t *ring = reinterpret_cast<uint32_t *>(smem) + wave * G::RING;

    const int per_c = a.nchunk * a.nimgw;
    const int c = wid / per_c;
    const int rem = wid - c * per_c;
    const int chunk = rem / a.nimgw;
    const int ig = rem - chunk * a.nimgw;
    const int n0 = ig * a.ipw, n1 = min(n0 + a.ipw, a.N);
    const int cin = FLIP ? c : c / a.mult;
    const int c_lo = chunk * 32 * NT;
    const int cb = c_lo - a.P;
    const int cb8 = cb & ~7;
    const int AL = cb - cb8;

    const int n = lane & 31, h = lane >> 5;
    const int n2 = n * static_cast<int>(sizeof(T));
    // B operand of instruction s: staged position AL + 32 t + 16 s + n + 8 h
    const int s0 = AL + n + 8 * h;
    const int d1 = G::D1 + (AL & 1);  // copy 1's first dword
    const int boff = ring_run<G::RS>(s0, d1);
    const int sk = lane & 15;
    const int gc = cb8 + 8 * sk;
    const bool vk = sk < G::NVEC && gc >= 0 && gc + 8 <= a.IW;

    for (int e = lane; e < G::RING; e += 64) ring[e] = 0u;
    roll_lds_sync();

    const float bias = (!FLIP && a.b) ? to_f32(a.b[c]) : 0.f;
    const uint16_t *wc = reinterpret_cast<const uint16_t *>(a.w) + static_cast<int64_t>(c) * K * K;
    const int64_t iplane = static_cast<int64_t>(a.IH) * a.IW;
    const int nq = ((a.IH + 15) >> 4) << 2;  // batches of four rows, whole groups of 16 (rows past the plane are zero)
    const bool colfull = c_lo + 32 * NT <= a.OW;

    for (int nimg = n0; nimg < n1; ++nimg) {
        const uint16_t *ip = reinterpret_cast<const uint16_t *>(a.in) + (static_cast<int64_t>(nimg) * a.Cin + cin) * iplane;
        T *op = a.out + (static_cast<int64_t>(nimg) * a.C + c) * a.OH * a.OW;
        const __amdgpu_buffer_rsrc_t orsrc =
            __builtin_amdgcn_make_buffer_rsrc(op, 0, a.OH * a.OW * static_cast<int>(sizeof(T)), 0x00020000);

        // A of instruction s: lane row R = 16 b + m holds, at step v, w[i][16 s +
        // 8 h .. + 7] with i = 16 b + ((v - m) mod 16) (zero past the filter)
        u32x4_r A[2];
        {
            const int b = n >> 4, m = n & 15;
            const int i = 16 * b + ((-m) & 15);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) {
                    uint32_t v = 0;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int j = 16 * s + 8 * h + 2 * k2 + hh;
                        if (i < K && j < K) {
                            const uint16_t bits = FLIP ? wc[(K - 1 - i) * K + (K - 1 - j)] : wc[i * K + j];
                            v |= static_cast<uint32_t>(bits) << (16 * hh);
                        }
                    }
                    A[s][k2] = v;
                }
        }
        f32x16_r d[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) d[t][r] = bias;

        // rows past the plane and vectors outside it read as zeros (buffer range
        // check): the load has no branch, so nothing waits for it before the
        // batch is written to the ring
        const __amdgpu_buffer_rsrc_t irsrc =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(ip), 0, static_cast<int>(iplane * 2), 0x00020000);
        auto load_batch = [&](int qb) -> uint4 {
            const int r = 4 * qb + (lane >> 4);
            const int off = (vk && r < a.IH) ? (r * a.IW + gc) * 2 : kR16Skip;
            const u32x4_r v = __builtin_amdgcn_raw_buffer_load_b128(irsrc, off, 0, 0);
            return make_uint4(v[0], v[1], v[2], v[3]);
        };
        auto write_batch = [&](int qb, const uint4 &raw) {
            if (vk) ring_put_vec<G::RS>(ring, d1, (4 * qb + (lane >> 4)) & (G::SLOTS - 1), sk, raw);
        };
        auto stage_scalar = [&](int qb) {
            const int span = AL + G::XW;
            for (int e = lane; e < 4 * span; e += 64) {
                const int q = e / span;
                const int p = e - q * span;
                const int r = 4 * qb + q;
                const int col = cb8 + p;
                if (col < 0 || col >= a.IW) continue;
                const uint16_t v = r < a.IH ? ip[static_cast<int64_t>(r) * a.IW + col] : uint16_t{0};
                ring_put_one<G::RS>(ring, d1, (4 * qb + q) & (G::SLOTS - 1), p, v);
            }
        };
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (VIN) {
            write_batch(0, load_batch(0));
            raw = load_batch(1);
        } else {
            stage_scalar(0);
        }

        // step v (v mod 16 = MM): slot m* = MM of both blocks is register r0 =
        // 4 (MM / 8) + MM % 4 (block 0) and r0 + 8 (block 1) of lane half (MM / 4) % 2
        auto step = [&](auto mm_c, int v) {
            constexpr int MM = decltype(mm_c)::value;
            constexpr int HH = (MM >> 2) & 1;
            constexpr int R0 = 4 * (MM >> 3) + (MM & 3), R1 = R0 + 8;
            const uint32_t *bp = ring + boff + (v & (G::SLOTS - 1));
            u32x4_r bv[NT][2];
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const uint32_t *q = bp + G::RS * (16 * t + 8 * s);
                    bv[t][s] = u32x4_r{q[0], q[G::RS], q[2 * G::RS], q[3 * G::RS]};
                }
            const bool sel = h == HH;
            float e[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                e[t] = d[t][R1];
                d[t][R1] = sel ? d[t][R0] : d[t][R1];
                d[t][R0] = sel ? bias : d[t][R0];
            }
            const int oh = v + a.P - 32;
            const int ub = (oh >= 0 && oh < a.OH) ? (oh * a.OW + c_lo) * static_cast<int>(sizeof(T)) : kR16Skip;
            const int off = sel ? ub + n2 : kR16Skip;
            if (colfull) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    __builtin_amdgcn_raw_buffer_store_b16(bits16(e[t], static_cast<T *>(nullptr)), orsrc, off + 64 * t, 0, 0);
            } else {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    __builtin_amdgcn_raw_buffer_store_b16(bits16(e[t], static_cast<T *>(nullptr)), orsrc,
                                                          c_lo + 32 * t + n < a.OW ? off + 64 * t : kR16Skip, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int s = 0; s < 2; ++s) d[t] = RollMfma32<T>::run(A[s], bv[t][s], d[t]);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) A[s][k2] = rot_row(A[s][k2]);
        };
        auto batch = [&](auto jb_c, int q) {
            constexpr int JB = decltype(jb_c)::value;
            roll_lds_sync();
            if (q + 1 < nq) {
                if constexpr (VIN) {
                    write_batch(q + 1, raw);
                    if (q + 2 < nq) raw = load_batch(q + 2);
                } else {
                    stage_scalar(q + 1);
                }
            }
            const int v = 4 * q;
            step(std::integral_constant<int, 4 * JB>{}, v);
            step(std::integral_constant<int, 4 * JB + 1>{}, v + 1);
            step(std::integral_constant<int, 4 * JB + 2>{}, v + 2);
            step(std::integral_constant<int, 4 * JB + 3>{}, v + 3);
        };
        for (int q = 0; q < nq; q += 4) {
            batch(std::integral_constant<int, 0>{}, q);
            batch(std::integral_constant<int, 1>{}, q + 1);
            batch(std::integral_constant<int, 2>{}, q + 2);
            batch(std::integral_constant<int, 3>{}, q + 3);
        }
        roll_lds_sync();

        const int vl = 4 * nq - 1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int R = 8 * (r >> 2) + 4 * h + (r & 3);
            const int b = R >> 4, m = R & 15;
            const int oh = vl + a.P - 16 * b - ((vl - m) & 15);
            if (oh < 0 || oh >= a.OH) continue;
            T *orow = op + static_cast<int64_t>(oh) * a.OW + c_lo + n;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (c_lo + 32 * t + n < a.OW) orow[32 * t] = from_f32<T>(d[t][r]);
        }
    }
}

// The same streaming for k <= 13 on 16 x 16 x 32 tiles, the contraction
// covering several input rows: RPS = 4 rows of 8 kernel columns (k <= 8) or
// 2 rows of 16 (k <= 13) per instruction, lane k-group g holding 8 adjacent
// values of input row RPS p + delta(g).  One 16-row block of accumulator
// slots: the output row whose kernel row 0 is input row rho lives in slot
// s = rho mod 16 while input rows rho .. rho + 15 stream past; at step p slot s
// holds kernel rows i0 + delta with i0 = RPS p - rho (mod 16), so the filter
// rows a lane needs repeat every 16 / RPS steps: all of those phases are held
// in registers (no data movement between steps).  Slot s sits in accumulator
// row 4 (s mod 4) + s / 4, so slots 4 R .. 4 R + 3 are register R of all four
// lane rows.  With RPS = 4 a step finishes exactly those four slots; with
// RPS = 2 a step finishes two of them, and the other two are already complete
// (their last two kernel rows, 14 and 15 or 13 and 14, are zero for k <= 13),
// so every second step emits one whole register.
//
// Output rows are collected in LDS (32 rows of the chunk) and leave in a
// fixed number of stores once per 32 rows: with no stores between, the waits on
// vector memory are for the oldest input loads only, so the inputs can be
// loaded several batches (a few hundred cycles of matrix work each) ahead.
template <int K, int NT> struct RsOut {
    static constexpr int ROWS = 32;
    static constexpr int PITCH = 8 * NT + 4;   // dwords of a buffered output row (16 NT halves, padded)
    static constexpr int DW = ROWS * PITCH;    // dwords of the buffer
    static constexpr int RINGA = (Lr16Geo<K, NT, 8>::RING + 3) / 4 * 4;  // ring, 16-byte aligned
    static constexpr int WAVE = RINGA + DW;    // dwords of LDS a wave
};

template <typename T, int K, int NT, bool FLIP, bool VIN>
__global__ __launch_bounds__(256) void lk_rolls_kernel(Lr16Args<T> a) {
    constexpr int RPS = K <= 8 ? 4 : 2;  // input rows per step
    // a slot restarts while the rows of its step still stream past, and with
    // RPS = 2 a register is emitted one step before half of its slots restart:
    // kernel rows 13 .. 15 must be zero
    static_assert(K <= 13, "one 16-row block of slots");
    constexpr int NPH = 16 / RPS;        // filter phases
    constexpr int JW = 32 / RPS;         // kernel columns per input row of the contraction
    constexpr int SPB = 4 / RPS;         // steps per batch of four rows
    constexpr int PD = 4;                // batches loaded ahead
    using G = Lr16Geo<K, NT, 8>;
    using O = RsOut<K, NT>;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wid = blockIdx.x * 4 + wave;
    if (wid >= a.nwaves) return;  // whole waves; the kernel has no workgroup barrier
    uint32_t *ring = reinterpret_cast<uint32_t *>(smem) + wave * O::WAVE;
    uint16_t *obuf = reinterpret_cast<uint16_t *>(ring + O::RINGA);

    const int per_c = a.nchunk * a.nimgw;
    const int c = wid / per_c;
    const int rem = wid - c * per_c;
    const int chunk = rem / a.nimgw;
    const int ig = rem - chunk * a.nimgw;
    const int n0 = ig * a.ipw, n1 = min(n0 + a.ipw, a.N);
    const int cin = FLIP ? c : c / a.mult;
    const int c_lo = chunk * 16 * NT;
    const int cb = c_lo - a.P;
    const int cb8 = cb & ~7;
    const int AL = cb - cb8;

    const int n = lane & 15, g = lane >> 4;
    const int dl = (8 * g) / JW;        // this lane row's input row within a step
    const int j0 = (8 * g) % JW;        // its first kernel column
    const int s0 = AL + n + j0;
    const int d1 = G::D1 + (AL & 1);
    const int boff = ring_run<G::RS>(s0, d1) + dl;  // + slot of the step's first row
    // lanes past the last vector repeat it (same load, same LDS writes), so
    // every lane stages without a branch; vectors outside the plane, and rows
    // past it, load zeros (offsets past the buffer's range)
    const int sk = min(lane & 15, G::NVEC - 1);
    const int gc = cb8 + 8 * sk;
    const bool vk = gc >= 0 && gc + 8 <= a.IW;
    const int lbase = vk ? ((lane >> 4) * a.IW + gc) * 2 : kR16Skip;  // batch 0's offset
    const int bstep = 8 * a.IW;                                        // bytes of four rows

    for (int e = lane; e < O::RINGA / 4; e += 64) reinterpret_cast<uint4 *>(ring)[e] = make_uint4(0u, 0u, 0u, 0u);

    const float bias = (!FLIP && a.b) ? to_f32(a.b[c]) : 0.f;
    const uint16_t *wc = reinterpret_cast<const uint16_t *>(a.w) + static_cast<int64_t>(c) * K * K;
    // the filter (flipped for grad-input), staged in the output buffer's place
    // as rows i = -4 .. 15 of 16 values, zero outside the k x k filter: each
    // phase's 8 values of a lane are one 16-byte LDS read
    constexpr int FO = 4;  // rows of zeros before kernel row 0
    static_assert(RPS - 1 <= FO && (FO + 16) * 8 <= O::DW, "staged filter fits");
    for (int e = lane; e < (FO + 16) * 16; e += 64) {
        const int i = e / 16 - FO, j = e % 16;
        uint16_t v = 0;
        if (i >= 0 && i < K && j < K) v = FLIP ? wc[(K - 1 - i) * K + (K - 1 - j)] : wc[i * K + j];
        obuf[e] = v;
    }
    roll_lds_sync();
    const int64_t iplane = static_cast<int64_t>(a.IH) * a.IW;
    const int nq = ((a.IH + 15) >> 4) << 2;  // batches of four rows, whole groups of 16
    // A of phase f: lane (m, g) holds w[i0 + dl][j0 .. j0 + 7] (zero outside
    // the filter), i0 = (RPS (f + 1) - 1 - s mod 16) - (RPS - 1) for the slot
    // s = 4 (m mod 4) + m / 4 of accumulator row m
    const int slot = 4 * (n & 3) + (n >> 2);
    u32x4_r A[NPH];
#pragma unroll
    for (int f = 0; f < NPH; ++f) {
        const int i = (((RPS * (f + 1) - 1 - slot) & 15) - (RPS - 1)) + dl;
        const uint4 v = *reinterpret_cast<const uint4 *>(obuf + (i + FO) * 16 + j0);
        A[f] = u32x4_r{v.x, v.y, v.z, v.w};
    }
    // output row oh sits in buffer row (oh - oh0) mod 32, oh0 = P - 16 the first
    // row a step finishes, so a group of 32 buffer rows is whole steps
    const int oh0 = a.P - 16;
    const bool vout = a.OW % 8 == 0 && reinterpret_cast<uintptr_t>(a.out) % 16 == 0;

    for (int nimg = n0; nimg < n1; ++nimg) {
        const uint16_t *ip = reinterpret_cast<const uint16_t *>(a.in) + (static_cast<int64_t>(nimg) * a.Cin + cin) * iplane;
        T *op = a.out + (static_cast<int64_t>(nimg) * a.C + c) * a.OH * a.OW;
        const __amdgpu_buffer_rsrc_t orsrc =
            __builtin_amdgcn_make_buffer_rsrc(op, 0, a.OH * a.OW * static_cast<int>(sizeof(T)), 0x00020000);
        const __amdgpu_buffer_rsrc_t irsrc =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(ip), 0, static_cast<int>(iplane * 2), 0x00020000);

        // buffered rows gb .. gb + 31 (those inside the plane) to memory, in the
        // same number of stores every time
        auto flush = [&](int gb) {
            roll_lds_sync();  // the rows' LDS writes are done
            if (vout) {
                // 16-byte runs: 2 NT a row
#pragma unroll
                for (int it = 0; it < O::ROWS * 2 * NT / 64; ++it) {
                    const int e = lane + 64 * it;
                    const int rl = e / (2 * NT);
                    const int v8 = e % (2 * NT);
                    const int rr = gb + rl;
                    const int col = c_lo + 8 * v8;
                    const uint4 val = *reinterpret_cast<const uint4 *>(obuf + 2 * ((rr - oh0) & (O::ROWS - 1)) * O::PITCH + 8 * v8);
                    const int off = (rr >= 0 && rr < a.OH && col < a.OW) ? (rr * a.OW + col) * static_cast<int>(sizeof(T)) : kR16Skip;
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4_r{val.x, val.y, val.z, val.w}, orsrc, off, 0, 0);
                }
            } else {
#pragma unroll 1
                for (int it = 0; it < O::ROWS * 16 * NT / 64; ++it) {
                    const int e = lane + 64 * it;
                    const int rl = e / (16 * NT);
                    const int cc = e % (16 * NT);
                    const int rr = gb + rl;
                    const uint16_t val = obuf[2 * ((rr - oh0) & (O::ROWS - 1)) * O::PITCH + cc];
                    const int off = (rr >= 0 && rr < a.OH && c_lo + cc < a.OW) ? (rr * a.OW + c_lo + cc) * static_cast<int>(sizeof(T)) : kR16Skip;
                    __builtin_amdgcn_raw_buffer_store_b16(val, orsrc, off, 0, 0);
                }
            }
            roll_lds_sync();  // the rows are read before the buffer is reused
        };

        f32x4_r d[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) d[t] = f32x4_r{bias, bias, bias, bias};

        auto load_batch = [&](int qb) -> uint4 {
            const u32x4_r v = __builtin_amdgcn_raw_buffer_load_b128(irsrc, lbase + qb * bstep, 0, 0);
            return make_uint4(v[0], v[1], v[2], v[3]);
        };
        auto write_batch = [&](int qb, const uint4 &raw) {
            ring_put_vec<G::RS>(ring, d1, (4 * qb + (lane >> 4)) & (G::SLOTS - 1), sk, raw);
        };
        auto stage_scalar = [&](int qb) {
            const int span = AL + G::XW;
            for (int e = lane; e < 4 * span; e += 64) {
                const int q = e / span;
                const int p = e - q * span;
                const int r = 4 * qb + q;
                const int col = cb8 + p;
                if (col < 0 || col >= a.IW) continue;
                const uint16_t v = r < a.IH ? ip[static_cast<int64_t>(r) * a.IW + col] : uint16_t{0};
                ring_put_one<G::RS>(ring, d1, (4 * qb + q) & (G::SLOTS - 1), p, v);
            }
        };
        // every batch loads the same way (rows past the plane read zeros): the
        // waits then count loads exactly
        uint4 raw[PD];
        if constexpr (VIN) {
            write_batch(0, load_batch(0));
#pragma unroll
            for (int b = 0; b < PD; ++b) raw[b] = load_batch(b + 1);
        } else {
            stage_scalar(0);
        }

        // step p (PP = p mod 16 / RPS, the filter phase): input rows RPS p .. RPS p + RPS - 1
        auto step = [&](auto pp_c, int p) {
            constexpr int PP = decltype(pp_c)::value;
            // a base of its own per step: the reads of two steps are not paired
            // into one ds_read2 (which would scatter each operand's registers)
            int boffs = boff + ((RPS * PP) & (G::SLOTS - 1));
            asm volatile("" : "+v"(boffs));
            const uint32_t *bp = ring + boffs;
            u32x4_r bv[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint32_t *q = bp + G::RS * 8 * t;
                bv[t] = u32x4_r{q[0], q[G::RS], q[2 * G::RS], q[3 * G::RS]};
            }
            // register R's four slots finish the output rows RPS p + g + oh0 (buffer
            // row (RPS p + g) mod 32) and start the rows 16 later at the bias:
            // every step (RPS 4) or every even step (RPS 2)
            if constexpr (RPS == 4 || PP % 2 == 0) {
                constexpr int R = RPS == 4 ? PP : PP / 2;
                uint16_t *orow = obuf + 2 * ((RPS * p + g) & (O::ROWS - 1)) * O::PITCH + n;
#pragma unroll
                for (int t = 0; t < NT; t += 2) {
                    if (t + 1 < NT) {
                        const uint32_t w2 = pack2<T>(d[t][R], d[t + 1][R]);
                        orow[16 * t] = static_cast<uint16_t>(w2);
                        orow[16 * t + 16] = static_cast<uint16_t>(w2 >> 16);
                    } else {
                        orow[16 * t] = bits16(d[t][R], static_cast<T *>(nullptr));
                    }
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) d[t][R] = bias;
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) d[t] = RollMfma<T>::run(A[PP], bv[t], d[t]);
        };
        auto batch = [&](auto jb_c, int q) {
            constexpr int JB = decltype(jb_c)::value;
            roll_lds_sync();
            if constexpr (VIN) {
                write_batch(q + 1, raw[JB]);
                raw[JB] = load_batch(q + 1 + PD);
            } else {
                if (q + 1 < nq) stage_scalar(q + 1);
            }
            const int p = SPB * q;
            if constexpr (RPS == 4) {
                step(std::integral_constant<int, JB>{}, p);
            } else {
                step(std::integral_constant<int, 2 * JB>{}, p);
                step(std::integral_constant<int, 2 * JB + 1>{}, p + 1);
            }
        };
        for (int q = 0; q < nq; q += 4) {
            batch(std::integral_constant<int, 0>{}, q);
            batch(std::integral_constant<int, 1>{}, q + 1);
            batch(std::integral_constant<int, 2>{}, q + 2);
            batch(std::integral_constant<int, 3>{}, q + 3);
            // 16 rows a pass: after every second pass 32 buffer rows are whole
            if (((q + 4) & 7) == 0) flush(oh0 + 4 * (q + 4) - O::ROWS);
        }

        // every output row still in a slot is complete
        const int pl = SPB * nq - 1;  // last step
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int sl = 4 * r + g;  // slot of accumulator row 4 g + r
            // the last step is odd for RPS 2: no slot is between its early
            // emission and its restart
            const int i0 = ((RPS * pl - sl + RPS - 1) & 15) - (RPS - 1);
            const int oh = RPS * pl - i0 + a.P;
            uint16_t *orow = obuf + 2 * ((oh - oh0) & (O::ROWS - 1)) * O::PITCH + n;
#pragma unroll
            for (int t = 0; t < NT; ++t) orow[16 * t] = bits16(d[t][r], static_cast<T *>(nullptr));
        }
        // the slots held relative rows 4 nq .. 4 nq + 15; with the 0 or 16 rows
        // since the last whole group (4 nq is a multiple of 16) they fill at most
        // one group, so none overwrote a row still to go out
        flush(oh0 + 4 * nq - ((4 * nq) & (O::ROWS - 1)));
    }
}

template <typename T, int K, int NT, bool FLIP>
int run_lrs_t(Lr16Args<T> a, hipStream_t s) {
    using G = Lr16Geo<K, NT, 8>;
    constexpr int lds = 4 * 4 * RsOut<K, NT>::WAVE;
    a.nchunk = (a.OW + 16 * NT - 1) / (16 * NT);
    const int64_t items = static_cast<int64_t>(a.C) * a.nchunk;
    // two images a wave on planes of at most 32 rows (the wave's set-up, its
    // filter phases and first loads, then covers two planes: measured 6-12 %
    // faster at 32 x 32, 3-15 % slower at 64 x 64), more past 2^18 waves
    const int64_t want = std::max<int64_t>(a.IH <= 32 ? 2 : 1, (static_cast<int64_t>(a.N) * items) >> 18);
    a.ipw = static_cast<int>(std::min<int64_t>(want, a.N));
    a.nimgw = (a.N + a.ipw - 1) / a.ipw;
    const int64_t nw = items * a.nimgw;
    if (nw > (int64_t{1} << 30)) return kErrUnsupported;
    a.nwaves = static_cast<int>(nw);
    const dim3 grid(static_cast<unsigned>((nw + 3) / 4));
    if (a.vin)
        hipLaunchKernelGGL((lk_rolls_kernel<T, K, NT, FLIP, true>), grid, dim3(256), lds, s, a);
    else
        hipLaunchKernelGGL((lk_rolls_kernel<T, K, NT, FLIP, false>), grid, dim3(256), lds, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, int K, bool FLIP>
int run_lrs(const Lr16Args<T> &a, hipStream_t s) {
    const int nt = std::min(4, (a.OW + 15) / 16);
    if (nt == 1) return run_lrs_t<T, K, 1, FLIP>(a, s);
    if (nt == 2) return run_lrs_t<T, K, 2, FLIP>(a, s);
    if (nt == 3) return run_lrs_t<T, K, 3, FLIP>(a, s);
    return run_lrs_t<T, K, 4, FLIP>(a, s);
}

template <typename T, int NT, bool FLIP>
int run_lr32_t(Lr16Args<T> a, hipStream_t s) {
    using G = Lr16Geo<kR16K, 2 * NT, 8>;
    a.nchunk = (a.OW + 32 * NT - 1) / (32 * NT);
    const int64_t items = static_cast<int64_t>(a.C) * a.nchunk;
    const int64_t want = std::max<int64_t>(1, (static_cast<int64_t>(a.N) * items) >> 18);
    a.ipw = static_cast<int>(std::min<int64_t>(want, a.N));
    a.nimgw = (a.N + a.ipw - 1) / a.ipw;
    const int64_t nw = items * a.nimgw;
    if (nw > (int64_t{1} << 30)) return kErrUnsupported;
    a.nwaves = static_cast<int>(nw);
    const dim3 grid(static_cast<unsigned>((nw + 3) / 4));
    if (a.vin)
        hipLaunchKernelGGL((lk_roll32_kernel<T, kR16K, NT, FLIP, true>), grid, dim3(256), G::lds_bytes, s, a);
    else
        hipLaunchKernelGGL((lk_roll32_kernel<T, kR16K, NT, FLIP, false>), grid, dim3(256), G::lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, int NT, bool FLIP>
int run_lr16_t(Lr16Args<T> a, hipStream_t s) {
    using G = Lr16Geo<kR16K, NT, 8>;
    a.nchunk = (a.OW + 16 * NT - 1) / (16 * NT);
    // one image a wave (many short waves leave no partial last round of
    // resident waves), a few where there are more than 2^18 of them
    const int64_t items = static_cast<int64_t>(a.C) * a.nchunk;
    const int64_t want = std::max<int64_t>(1, (static_cast<int64_t>(a.N) * items) >> 18);
    a.ipw = static_cast<int>(std::min<int64_t>(want, a.N));
    a.nimgw = (a.N + a.ipw - 1) / a.ipw;
    const int64_t nw = items * a.nimgw;
    if (nw > (int64_t{1} << 30)) return kErrUnsupported;
    a.nwaves = static_cast<int>(nw);
    const dim3 grid(static_cast<unsigned>((nw + 3) / 4));
    if (a.vin)
        hipLaunchKernelGGL((lk_roll16_kernel<T, kR16K, NT, FLIP, true>), grid, dim3(256), G::lds_bytes, s, a);
    else
        hipLaunchKernelGGL((lk_roll16_kernel<T, kR16K, NT, FLIP, false>), grid, dim3(256), G::lds_bytes, s, a);
    return hipGetLastError() == hipSuccess ? kOk : kErrHip;
}

template <typename T, bool FLIP>
int run_lr16(const Lr16Args<T> &a, int K, hipStream_t s) {
    if (K == 7) return run_lrs<T, 7, FLIP>(a, s);
    if (K == 13) return run_lrs<T, 13, FLIP>(a, s);
    // rows a multiple of 32 wide: 32-column tiles
    if (a.OW % 32 == 0) return a.OW == 32 ? run_lr32_t<T, 1, FLIP>(a, s) : run_lr32_t<T, 2, FLIP>(a, s);
    const int nt = std::min(4, (a.OW + 15) / 16);
    if (nt == 1) return run_lr16_t<T, 1, FLIP>(a, s);
    if (nt == 2) return run_lr16_t<T, 2, FLIP>(a, s);
    if (nt == 3) return run_lr16_t<T, 3, FLIP>(a, s);
    return run_lr16_t<T, 4, FLIP>(a, s);
}

template <typename T>
int lr16_fwd_t(const Geo &g, const void *x, const void *w, const void *b, void *y, hipStream_t s) {
    Lr16Args<T> a{};
    a.in = static_cast<const T *>(x);
    a.w = static_cast<const T *>(w);
    a.b = static_cast<const T *>(b);
    a.out = static_cast<T *>(y);
    a.N = g.n;
    a.C = g.oc;
    a.Cin = g.ic;
    a.mult = g.mult;
    a.IH = g.ih;
    a.IW = g.iw;
    a.OH = g.oh;
    a.OW = g.ow;
    a.P = g.ph;
    a.vin = a.IW % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
    return run_lr16<T, false>(a, g.kh, s);
}

template <typename T>
int lr16_bwdin_t(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t s) {
    Lr16Args<T> a{};
    a.in = static_cast<const T *>(dy);
    a.w = static_cast<const T *>(w);
    a.out = static_cast<T *>(dx);
    a.N = g.n;
    a.C = g.ic;
    a.Cin = g.oc;
    a.mult = 1;
    a.IH = g.oh;
    a.IW = g.ow;
    a.OH = g.ih;
    a.OW = g.iw;
    a.P = g.kh - 1 - g.ph;
    a.vin = a.IW % 8 == 0 && reinterpret_cast<uintptr_t>(dy) % 16 == 0;
    return run_lr16<T, true>(a, g.kh, s);
}

}  // namespace

// 16-bit, k = 7, 13 or 31 square, stride 1, dilation 1, equal paddings below
// k; the grad-input pass with multiplier 1.  Any plane size.
bool largek_roll16_fits(const Geo &g, int pass, int dtype) {
    if (dtype == 0) return false;
    if (g.kh != g.kw || (g.kh != 7 && g.kh != 13 && g.kh != kR16K)) return false;
    if (g.sh != 1 || g.sw != 1 || g.dh != 1 || g.dw != 1 || g.ph != g.pw || g.ph > g.kh - 1) return false;
    if (pass == 1 && g.mult != 1) return false;
    // input and output planes addressed by 32-bit buffer offsets below 1 GiB
    const int64_t ip = static_cast<int64_t>(g.ih) * g.iw, op = static_cast<int64_t>(g.oh) * g.ow;
    return g.oh >= 1 && g.ow >= 1 && std::max(ip, op) * 2 < (int64_t{1} << 30);
}

int largek_roll16_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s) {
    return dtype == 1 ? lr16_fwd_t<__half>(g, x, w, b, y, s) : lr16_fwd_t<bf16_t>(g, x, w, b, y, s);
}

int largek_roll16_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s) {
    return dtype == 1 ? lr16_bwdin_t<__half>(g, dy, w, dx, s) : lr16_bwdin_t<bf16_t>(g, dy, w, dx, s);
}

}  // namespace dw
