// dw_stream.hpp -- device helpers of the streaming (row-walk) kernels:
// rows moved as raw 32-bit words so that loads issued ahead stay in flight
// until the row is used, element access and rounding on those words, and
// wave-level reductions.
#pragma once

#include "dw_common.hpp"
#include "dw_internal.hpp"

#include <initializer_list>
#include <type_traits>

namespace dw {

// Elements of T per 32-bit word.
template <typename T> constexpr int kPerWord = 4 / static_cast<int>(sizeof(T));

__device__ __forceinline__ uint32_t bits_of(float v) { return __float_as_uint(v); }
__device__ __forceinline__ uint32_t bits_of(__half v) { return __half_as_ushort(v); }
__device__ __forceinline__ uint32_t bits_of(bf16_t v) { return v.bits; }

template <typename T> __device__ __forceinline__ T from_bits(uint32_t b);
template <> __device__ __forceinline__ float from_bits<float>(uint32_t b) { return __uint_as_float(b); }
template <> __device__ __forceinline__ __half from_bits<__half>(uint32_t b) {
    return __ushort_as_half(static_cast<unsigned short>(b));
}
template <> __device__ __forceinline__ bf16_t from_bits<bf16_t>(uint32_t b) {
    bf16_t r;
    r.bits = static_cast<uint16_t>(b);
    return r;
}

// Element e of a packed run of words, as fp32 (e is a constant after unrolling).
template <typename T, int NW>
__device__ __forceinline__ float word_elem(const uint32_t (&w)[NW], int e) {
    if constexpr (sizeof(T) == 4) {
        return __uint_as_float(w[e]);
    } else {
        const uint32_t h = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu);
        if constexpr (std::is_same<T, bf16_t>::value)
            return __uint_as_float(h << 16);
        else
            return __half2float(__ushort_as_half(static_cast<unsigned short>(h)));
    }
}

// NW words from NW * kPerWord<T> fp32 values, each rounded to T.
template <typename T, int NW>
__device__ __forceinline__ void pack_words(const float *v, uint32_t (&w)[NW]) {
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        if constexpr (sizeof(T) == 4)
            w[k] = __float_as_uint(v[k]);
        else
            w[k] = pack2<T>(v[2 * k], v[2 * k + 1]);
    }
}

template <int NW>
__device__ __forceinline__ void load_words(const void *p, uint32_t (&w)[NW]) {
    if constexpr (NW == 2) {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        w[0] = u.x;
        w[1] = u.y;
    } else {
        static_assert(NW % 4 == 0, "whole 16-byte vectors");
#pragma unroll
        for (int k = 0; k < NW / 4; ++k) {
            const uint4 u = reinterpret_cast<const uint4 *>(p)[k];
            w[4 * k] = u.x;
            w[4 * k + 1] = u.y;
            w[4 * k + 2] = u.z;
            w[4 * k + 3] = u.w;
        }
    }
}

// NT: nontemporal (streaming) 16-byte stores, for outputs much larger than
// the inputs of the kernel (they then leave L2 to the input rows).
template <int NW, bool NT = false>
__device__ __forceinline__ void store_words(void *p, const uint32_t (&w)[NW]) {
    if constexpr (NW == 2) {
        *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
    } else {
        static_assert(NW % 4 == 0, "whole 16-byte vectors");
        typedef unsigned int v4u __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int k = 0; k < NW / 4; ++k) {
            const v4u t = {w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
            if constexpr (NT)
                __builtin_nontemporal_store(t, reinterpret_cast<v4u *>(p) + k);
            else
                reinterpret_cast<v4u *>(p)[k] = t;
        }
    }
}

// The same words assembled element by element; elements at index >= avail read as zero.
template <typename T, int NW>
__device__ __forceinline__ void load_words_tail(const T *p, int avail, uint32_t (&w)[NW]) {
    constexpr int PW = kPerWord<T>;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < PW; ++e)
            if (k * PW + e < avail) v |= bits_of(p[k * PW + e]) << (16 * e);
        w[k] = v;
    }
}

template <typename T, int NW>
__device__ __forceinline__ void store_words_tail(T *p, int avail, const uint32_t (&w)[NW]) {
    constexpr int PW = kPerWord<T>;
#pragma unroll
    for (int k = 0; k < NW; ++k)
#pragma unroll
        for (int e = 0; e < PW; ++e)
            if (k * PW + e < avail) p[k * PW + e] = from_bits<T>(PW == 1 ? w[k] : (w[k] >> (16 * e)) & 0xffffu);
}

// acc + a.lo * b.lo + a.hi * b.hi for two packed 16-bit pairs
// (v_dot2c_f32_{f16,bf16}: the products are exact, the sums fp32).
template <typename T> struct Dot2;
template <> struct Dot2<bf16_t> {
    static __device__ __forceinline__ float run(uint32_t a, uint32_t b, float c) {
        typedef __bf16 v2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2, a), __builtin_bit_cast(v2, b), c, false);
    }
};
template <> struct Dot2<__half> {
    static __device__ __forceinline__ float run(uint32_t a, uint32_t b, float c) {
        typedef _Float16 v2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(v2, a), __builtin_bit_cast(v2, b), c, false);
    }
};

// Wave-uniform value kept in a scalar register (the filter taps of a channel).
__device__ __forceinline__ float uniform(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Value of lane - 1 (DPP wave_shr:1) and of lane + 1 (wave_shl:1), 0 past the
// wave's ends, without LDS traffic.  A DPP move reads a lane that EXEC
// disables as zero, so callers run it with every lane enabled; the empty
// volatile asm keeps the compiler from sinking it under a later branch.
__device__ __forceinline__ float lane_left(float v) {
    int r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xf, 0xf, true);
    asm volatile("" : "+v"(r));
    return __int_as_float(r);
}
__device__ __forceinline__ float lane_right(float v) {
    int r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x130, 0xf, 0xf, true);
    asm volatile("" : "+v"(r));
    return __int_as_float(r);
}
__device__ __forceinline__ uint32_t lane_left(uint32_t v) {
    return __float_as_uint(lane_left(__uint_as_float(v)));
}
__device__ __forceinline__ uint32_t lane_right(uint32_t v) {
    return __float_as_uint(lane_right(__uint_as_float(v)));
}

// Partner value of the lane paired with this one inside its 16-lane row at
// halving step o <= 8 (DPP, no LDS): row_mirror (lane i ^ 15) for o = 8,
// row_half_mirror (i ^ 7) for o = 4, quad_perm (i ^ 2, i ^ 1) for o = 2, 1.
// Each partner differs from the lane in bit o and agrees on every bit above
// it, which is all the halving below needs.
template <int O> __device__ __forceinline__ float row_partner(float v) {
    constexpr int ctrl = O == 8 ? 0x140 : O == 4 ? 0x141 : O == 2 ? 0x4e : 0xb1;
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xf, 0xf, true));
}

// Sums of N <= 64 per-lane values over the wave, by recursive halving: at the
// step with lane offset o every lane keeps one half of its current vector,
// sends the other half to its partner (a lane that differs in bit o) and adds
// what it receives, so after six steps lane l holds the total of value l
// (63 exchanges instead of 6 per value).  The exchanges across 32 and 16
// lanes are v_permlane32_swap / v_permlane16_swap of the two halves (one swap
// leaves each lane its kept value and its partner's sent one, the sum of the
// two results), the ones inside 16-lane rows are DPP moves: no LDS traffic.
template <int N>
__device__ __forceinline__ float wave_transpose_sum(const float (&v)[N], int lane) {
    static_assert(N <= 64, "one value per lane");
    float c[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) c[i] = i < N ? v[i] : 0.f;
    auto swap_step = [&](auto o_c) {
        constexpr int o = decltype(o_c)::value;
#pragma unroll
        for (int i = 0; i < o; ++i) {
            // lower lanes keep c[i], upper lanes c[i + o]: after the swap the
            // first result holds the lower lanes' c[i] and the upper lanes'
            // partner c[i + o], the second the partner c[i] and own c[i + o]
            const uint32_t x = __float_as_uint(c[i]), y = __float_as_uint(c[i + o]);
            auto r = o == 32 ? __builtin_amdgcn_permlane32_swap(x, y, false, false)
                             : __builtin_amdgcn_permlane16_swap(x, y, false, false);
            c[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    };
    auto row_step = [&](auto o_c) {
        constexpr int o = decltype(o_c)::value;
        const bool upper = (lane & o) != 0;  // this lane keeps indices [o, 2o) of the current vector
#pragma unroll
        for (int i = 0; i < o; ++i) {
            const float keep = upper ? c[i + o] : c[i];
            const float send = upper ? c[i] : c[i + o];
            c[i] = keep + row_partner<o>(send);
        }
    };
    swap_step(std::integral_constant<int, 32>{});
    swap_step(std::integral_constant<int, 16>{});
    row_step(std::integral_constant<int, 8>{});
    row_step(std::integral_constant<int, 4>{});
    row_step(std::integral_constant<int, 2>{});
    row_step(std::integral_constant<int, 1>{});
    return c[0];
}

// Raw words moved out of a prefetch buffer before the buffer is refilled.
// 32-bit elements are used as they are, so the compiler would otherwise keep
// them in the buffer's registers for the whole step, load the refill into
// other registers and copy it back at the loop's back edge, which makes every
// pass wait for the loads it has just issued.  The copy is opaque to the
// compiler (one v_mov_b32 per word), so the buffer's registers are free for
// the refill as soon as it has run.  16-bit words are unpacked into new
// registers anyway and are passed through.
template <typename T, int NW>
__device__ __forceinline__ void take_words(const uint32_t (&src)[NW], uint32_t (&dst)[NW]) {
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        if constexpr (sizeof(T) == 4)
            asm("v_mov_b32 %0, %1" : "=v"(dst[k]) : "v"(src[k]));
        else
            dst[k] = src[k];
    }
}

// Drops the front of a ring of R raw rows: q[f] = q[f + 1]; the back slot is
// refilled by the caller.  Call it after the front row has been used: the
// scheduling barrier keeps the refill load below that use, so the register
// allocator can give each refill the registers of the row it replaces and the
// ring needs no copies (a copy of a row still in flight would wait for it).
template <int R, int NW>
__device__ __forceinline__ void ring_pop(uint32_t (&q)[R][NW], bool (&ok)[R]) {
#pragma unroll
    for (int f = 0; f + 1 < R; ++f) {
#pragma unroll
        for (int k = 0; k < NW; ++k) q[f][k] = q[f + 1][k];
        ok[f] = ok[f + 1];
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Raw words of columns [c0, c0 + NW * kPerWord<T>) of row r of a plane with H
// rows of W elements, read as vectors of VB bytes.  Rows outside [0, H) are
// read from the nearest row and flagged !ok, so the load needs no branch.
// VB == 16: the caller guarantees the columns lie inside the row (and the
// alignment).  VB < 16: each vector's start is clamped to the row's last whole
// vector, so the read stays inside the row; the caller masks the columns at
// and beyond W when converting (row_values with nvalid = W - c0).  Requires
// W * sizeof(T) to be a multiple of VB, at least VB, and a VB-aligned plane.
template <typename T, int NW, int VB>
__device__ __forceinline__ void load_row(const T *plane, int r, int H, int W, int c0, bool act, uint32_t (&w)[NW],
                                         bool &ok) {
    static_assert(VB == 16 || VB == 8 || VB == 4 || VB == 2, "vector width");
    static_assert(VB >= static_cast<int>(sizeof(T)), "whole elements");
    ok = act && r >= 0 && r < H;
    const int rc = min(max(r, 0), H - 1);
    const T *row = plane + static_cast<int64_t>(rc) * W;
    if constexpr (VB == 16) {
        load_words<NW>(row + c0, w);
    } else {
        constexpr int VE = VB / static_cast<int>(sizeof(T));  // elements per vector
        constexpr int NV = NW * 4 / VB;                         // vectors per segment
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const T *q = row + min(c0 + k * VE, W - VE);
            if constexpr (VB == 8) {
                const uint2 u = *reinterpret_cast<const uint2 *>(q);
                w[2 * k] = u.x;
                w[2 * k + 1] = u.y;
            } else if constexpr (VB == 4) {
                w[k] = *reinterpret_cast<const uint32_t *>(q);
            } else {
                const uint32_t h = *reinterpret_cast<const uint16_t *>(q);
                if (k & 1)
                    w[k >> 1] |= h << 16;
                else
                    w[k >> 1] = h;
            }
        }
    }
}

// The N elements held in a raw row as fp32; zero when the row is flagged !ok
// and for elements at index >= nvalid (columns past the end of the row).
template <typename T, int N, int NW>
__device__ __forceinline__ void row_values(const uint32_t (&w)[NW], bool ok, int nvalid, float (&v)[N]) {
    static_assert(N <= NW * kPerWord<T>, "elements held in the words");
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] = (ok && e < nvalid) ? word_elem<T>(w, e) : 0.f;
}

// N fp32 values rounded to T and stored at p as vectors of VB bytes: all of
// them when VB == 16 (the caller guarantees the strip lies inside the row),
// else only the vectors that start before `avail` (W * sizeof(T) a multiple
// of VB, so a vector that starts inside the row ends inside it).
template <typename T, int N, int VB, bool NT = false>
__device__ __forceinline__ void store_values(T *p, const float (&v)[N], int avail) {
    constexpr int NW = N / kPerWord<T>;
    static_assert(NW * kPerWord<T> == N, "whole words");
    uint32_t w[NW];
    pack_words<T, NW>(v, w);
    if constexpr (VB == 16) {
        store_words<NW, NT>(p, w);
    } else {
        constexpr int VE = VB / static_cast<int>(sizeof(T));
        constexpr int NV = NW * 4 / VB;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            if (k * VE < avail) {
                T *q = p + k * VE;
                if constexpr (VB == 8)
                    *reinterpret_cast<uint2 *>(q) = make_uint2(w[2 * k], w[2 * k + 1]);
                else if constexpr (VB == 4)
                    *reinterpret_cast<uint32_t *>(q) = w[k];
                else
                    *reinterpret_cast<uint16_t *>(q) = static_cast<uint16_t>((k & 1) ? w[k >> 1] >> 16 : w[k >> 1]);
            }
        }
    }
}

// Wave -> work of the streaming kernels: wave wv of the grid serves channel
// wv / wpc and its units [j*SPW, (j+1)*SPW), j = wv % wpc, a unit being one
// (image, row band) pair; within the wave, slot = lane / NS picks the unit
// and s = lane % NS the column strip.  Waves past the last channel are idle.
struct WaveUnit {
    int ic, n, band, lane, s;
    bool act;
};

__device__ __forceinline__ WaveUnit wave_unit(int wpc, int NS, int SPW, int nunits, int nbands, int nch) {
    WaveUnit u;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * (kThreads / 64) +
                                                  static_cast<int>(threadIdx.x >> 6));
    const int ic = wv / wpc;
    const int jw = wv - ic * wpc;
    const bool wave_ok = ic < nch;
    u.ic = wave_ok ? ic : nch - 1;
    u.lane = threadIdx.x & 63;
    const int slot = u.lane / NS;
    u.s = u.lane - slot * NS;
    const int ul = jw * SPW + slot;
    u.act = wave_ok && slot < SPW && ul < nunits;
    u.n = u.act ? ul / nbands : 0;
    u.band = u.act ? ul - u.n * nbands : 0;
    return u;
}

// Channel-slot mapping for small planes: wave wv serves image wv / wpc and the
// SPW consecutive channels of group wv % wpc, slot = lane / NS picking the
// channel and s = lane % NS the column strip; every slot walks its whole
// plane.  The planes a wave touches are one contiguous run of memory, and the
// channel (so the taps) differs per slot.
__device__ __forceinline__ WaveUnit chan_unit(int wpc, int NS, int SPW, int nch, int nimg) {
    WaveUnit u;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * (kThreads / 64) +
                                                  static_cast<int>(threadIdx.x >> 6));
    const int n = wv / wpc;
    const int cg = wv - n * wpc;
    u.lane = threadIdx.x & 63;
    const int slot = u.lane / NS;
    u.s = u.lane - slot * NS;
    const int c = cg * SPW + slot;
    u.act = n < nimg && slot < SPW && c < nch;
    u.ic = u.act ? c : 0;
    u.n = u.act ? n : 0;
    u.band = 0;
    return u;
}

// Widest vector (16, 8, 4 or 2 bytes, at least one element of T) that divides
// the byte length of every listed row width and every listed base address: the
// VB for load_row / store_values on those rows (a row vector never straddles
// two rows).  Never 0 for element-aligned bases, as 2- or 4-byte vectors fit.
template <typename T>
inline int row_vector_bytes(std::initializer_list<int> widths, std::initializer_list<const void *> bases) {
    for (int vb = 16; vb >= static_cast<int>(sizeof(T)); vb /= 2) {
        bool ok = true;
        for (int w : widths) {
            const int64_t bytes = static_cast<int64_t>(w) * static_cast<int64_t>(sizeof(T));
            ok = ok && bytes % vb == 0 && bytes >= vb;
        }
        for (const void *p : bases) ok = ok && reinterpret_cast<uintptr_t>(p) % vb == 0;
        if (ok) return vb;
    }
    return 0;
}

// Calls f(std::integral_constant<int, VB>) for the runtime vector width vb.
template <typename T, typename F>
int with_vector_bytes(int vb, F &&f) {
    switch (vb) {
        case 16: return f(std::integral_constant<int, 16>{});
        case 8: return f(std::integral_constant<int, 8>{});
        case 4:
            if constexpr (sizeof(T) <= 4) return f(std::integral_constant<int, 4>{});
            break;
        case 2:
            if constexpr (sizeof(T) <= 2) return f(std::integral_constant<int, 2>{});
            break;
        default: break;
    }
    return kErrUnsupported;
}

}  // namespace dw
