// dw_probe.hip -- achievable-rate probes of the device, for the benchmark's
// roofline (not part of the convolution library): how fast this GPU streams
// HBM with 16-byte nontemporal accesses (copy, read-only, write-only), how
// fast its matrix cores retire fp32 and fp16 multiply-adds and its vector
// units fp32 fused multiply-adds.  The
// convolution kernels are compared against these measured ceilings as well
// as against the published peaks.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// b[i] = a[i] for i < nv, four vectors per thread in flight.
__global__ __launch_bounds__(kThreads) void copy_kernel(const v4u *__restrict__ a, v4u *__restrict__ b, int64_t nv) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < nv; i += kUnroll * stride) {
        v4u t[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) t[u] = __builtin_nontemporal_load(a + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(t[u], b + i + u * stride);
    }
    for (; i < nv; i += stride) b[i] = a[i];
}

// Reads a[0, nv); writes one word only when the folded value matches a key the
// data never produces (the store keeps the loads live).
__global__ __launch_bounds__(kThreads) void read_kernel(const v4u *__restrict__ a, unsigned *out, int64_t nv) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    unsigned acc = 0;
    for (; i + (kUnroll - 1) * stride < nv; i += kUnroll * stride) {
        v4u t[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) t[u] = __builtin_nontemporal_load(a + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= t[u].x ^ t[u].y ^ t[u].z ^ t[u].w;
    }
    for (; i < nv; i += stride) acc ^= a[i].x;
    if (acc == 0x9e3779b9u) out[0] = acc;
}

__global__ __launch_bounds__(kThreads) void write_kernel(v4u *__restrict__ b, int64_t nv) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const v4u z = {0u, 0u, 0u, 0u};
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < nv; i += stride)
        __builtin_nontemporal_store(z, b + i);
}

// Four independent accumulation chains of v_mfma_f32_32x32x2_f32 per wave
// (2 * 32 * 32 * 2 flops each), `iters` rounds; one float per thread out.
__global__ __launch_bounds__(kThreads) void mfma_f32_kernel(float *out, int iters) {
    const float a = 1e-3f * threadIdx.x, b = 2e-3f * threadIdx.x;
    f32x16 acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[k], 0, 0, 0);
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) t += acc[k][r];
    out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = t;
}

// The same with v_mfma_f32_32x32x16_f16 (2 * 32 * 32 * 16 flops each).
__global__ __launch_bounds__(kThreads) void mfma_f16_kernel(float *out, int iters) {
    f16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<_Float16>(1e-3f * (threadIdx.x + e));
        b[e] = static_cast<_Float16>(2e-3f * (threadIdx.x - e));
    }
    f32x16 acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) t += acc[k][r];
    out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = t;
}

// Eight independent fp32 fused multiply-add chains per lane on the vector
// units (2 * 8 flops per lane and round).
__global__ __launch_bounds__(kThreads) void valu_f32_kernel(float *out, int iters) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 1e-3f * threadIdx.x + k;
    const float m = 0.999f, c = 1e-4f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = fmaf(v[k], m, c);
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) t += v[k];
    out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = t;
}

constexpr unsigned kStreamGrid = 8192;

}  // namespace

extern "C" {

// kind 0: copy `bytes` from src to dst; 1: read src; 2: write dst.  bytes is
// a multiple of 16 and both buffers are 16-byte aligned; out (kind 1) is a
// 4-byte device word.  Returns 0, or -1 for bad arguments, -2 on a launch error.
int dw_probe_stream(int kind, const void *src, void *dst, size_t bytes, void *out, void *stream) {
    if (bytes == 0 || bytes % 16 != 0) return -1;
    if ((kind == 0 || kind == 1) && (!src || reinterpret_cast<uintptr_t>(src) % 16 != 0)) return -1;
    if ((kind == 0 || kind == 2) && (!dst || reinterpret_cast<uintptr_t>(dst) % 16 != 0)) return -1;
    if (kind == 1 && !out) return -1;
    const int64_t nv = static_cast<int64_t>(bytes / 16);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (kind) {
        case 0:
            hipLaunchKernelGGL(copy_kernel, dim3(kStreamGrid), dim3(kThreads), 0, s, static_cast<const v4u *>(src),
                               static_cast<v4u *>(dst), nv);
            break;
        case 1:
            hipLaunchKernelGGL(read_kernel, dim3(kStreamGrid), dim3(kThreads), 0, s, static_cast<const v4u *>(src),
                               static_cast<unsigned *>(out), nv);
            break;
        case 2:
            hipLaunchKernelGGL(write_kernel, dim3(kStreamGrid), dim3(kThreads), 0, s, static_cast<v4u *>(dst), nv);
            break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// kind 0: fp32 matrix instructions, 1: fp16 matrix instructions, 2: fp32
// vector fused multiply-adds.  out holds blocks * 256 floats.  Writes the
// flops the launch performs to *flops.  Returns as dw_probe_stream.
int dw_probe_compute(int kind, float *out, int blocks, int iters, double *flops, void *stream) {
    if (!out || !flops || blocks < 1 || iters < 1 || kind < 0 || kind > 2) return -1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const double waves = static_cast<double>(blocks) * kThreads / 64;
    if (kind == 0) {
        *flops = 2.0 * 32 * 32 * 2 * 4 * iters * waves;
        hipLaunchKernelGGL(mfma_f32_kernel, dim3(blocks), dim3(kThreads), 0, s, out, iters);
    } else if (kind == 1) {
        *flops = 2.0 * 32 * 32 * 16 * 4 * iters * waves;
        hipLaunchKernelGGL(mfma_f16_kernel, dim3(blocks), dim3(kThreads), 0, s, out, iters);
    } else {
        *flops = 2.0 * 8 * iters * static_cast<double>(blocks) * kThreads;
        hipLaunchKernelGGL(valu_f32_kernel, dim3(blocks), dim3(kThreads), 0, s, out, iters);
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
