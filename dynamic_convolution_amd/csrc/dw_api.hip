// dw_api.hip -- the extern "C" entry points declared in include/dwconv.h.
//
// Every argument is validated on the host before any HIP call, so invalid
// calls launch nothing and touch no output.  Valid calls plan the launch and
// enqueue the kernels of dw_fwd / dw_bwd_input / dw_bwd_weight / dw_dynconv /
// dw_dynbwd (and the specialised families they dispatch to) on the caller's
// stream.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <cstring>
#include <mutex>

#include "dw_internal.hpp"
#include "dwconv.h"

namespace {

constexpr int64_t kMaxElems = (int64_t{1} << 31) - 1;  // every tensor below 2^31 elements
constexpr int64_t kMaxExtent = int64_t{1} << 30;        // keeps in-kernel index math in int32

size_t elem_size(int dtype) { return dtype == DW_F32 ? 4 : 2; }

// a * b * c * d < 2^31 without overflow (all factors >= 1).
bool product_ok(int64_t a, int64_t b, int64_t c = 1, int64_t d = 1) {
    int64_t p = a;
    for (int64_t f : {b, c, d}) {
        if (p > kMaxElems / f) return false;
        p *= f;
    }
    return p <= kMaxElems;
}

bool aligned(const void *p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// [a, a+na) and [b, b+nb) share a byte.
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Validates the 13 geometry integers and fills g.  Order of checks: size
// ranges, multiplier, output size, element counts.
int check_geometry(int64_t n, int64_t ic, int64_t ih, int64_t iw, int64_t oc, int64_t kh, int64_t kw,
                   int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw_, dw::Geo *g) {
    if (n < 1 || ic < 1 || ih < 1 || iw < 1 || oc < 1 || kh < 1 || kw < 1 || sh < 1 || sw < 1 || dh < 1 ||
        dw_ < 1 || ph < 0 || pw < 0)
        return DW_ESHAPE;
    for (int64_t v : {n, ic, ih, iw, oc, kh, kw, sh, sw, ph, pw, dh, dw_})
        if (v > kMaxExtent) return DW_ETOOLARGE;
    if (oc % ic != 0) return DW_EMULT;
    if (ih + 2 * ph > kMaxExtent || iw + 2 * pw > kMaxExtent || (kh - 1) * dh > kMaxExtent ||
        (kw - 1) * dw_ > kMaxExtent)
        return DW_ETOOLARGE;
    const int64_t nh = ih + 2 * ph - dh * (kh - 1) - 1;
    const int64_t nw = iw + 2 * pw - dw_ * (kw - 1) - 1;
    if (nh < 0 || nw < 0) return DW_ESHAPE;
    const int64_t oh = nh / sh + 1, ow = nw / sw + 1;
    if (!product_ok(n, ic, ih, iw) || !product_ok(n, oc, oh, ow) || !product_ok(oc, kh, kw))
        return DW_ETOOLARGE;
    if (g) {
        g->n = static_cast<int>(n);
        g->ic = static_cast<int>(ic);
        g->ih = static_cast<int>(ih);
        g->iw = static_cast<int>(iw);
        g->oc = static_cast<int>(oc);
        g->kh = static_cast<int>(kh);
        g->kw = static_cast<int>(kw);
        g->sh = static_cast<int>(sh);
        g->sw = static_cast<int>(sw);
        g->ph = static_cast<int>(ph);
        g->pw = static_cast<int>(pw);
        g->dh = static_cast<int>(dh);
        g->dw = static_cast<int>(dw_);
        g->oh = static_cast<int>(oh);
        g->ow = static_cast<int>(ow);
        g->mult = static_cast<int>(oc / ic);
    }
    return DW_OK;
}

size_t x_bytes(const dw::Geo &g, size_t e) { return static_cast<size_t>(g.n) * g.ic * g.ih * g.iw * e; }
size_t y_bytes(const dw::Geo &g, size_t e) { return static_cast<size_t>(g.n) * g.oc * g.oh * g.ow * e; }
size_t w_bytes(const dw::Geo &g, size_t e) { return static_cast<size_t>(g.oc) * g.kh * g.kw * e; }
size_t b_bytes(const dw::Geo &g, size_t e) { return static_cast<size_t>(g.oc) * e; }

int map_launch(int rc) {
    if (rc == dw::kOk) return DW_OK;
    if (rc == dw::kErrUnsupported) return DW_EUNSUPPORTED;
    return DW_EHIP;
}

// Validates the arguments the dynamic filter's forward and backward share:
// dtype, sizes, branch count, dilations, x and the filter pointers, element
// counts.  Writes the largest dilation.
int check_dyn(const void *x, const void *const *filters, const int32_t *dilations, int32_t nb, int64_t n,
              int64_t c, int64_t h, int64_t w, int64_t k, int dtype, int *maxdil) {
    if (dtype != DW_F32 && dtype != DW_F16 && dtype != DW_BF16) return DW_EDTYPE;
    if (n < 1 || c < 1 || h < 1 || w < 1 || k < 1) return DW_ESHAPE;
    for (int64_t v : {n, c, h, w, k})
        if (v > kMaxExtent) return DW_ETOOLARGE;
    if (nb < 1 || nb > 4 || (k % 2) == 0) return DW_EDYN;
    if (!x || !filters || !dilations) return DW_EPTR;
    int md = 1;
    for (int b = 0; b < nb; ++b) {
        if (dilations[b] < 1) return DW_EDYN;
        if (!filters[b]) return DW_EPTR;
        if ((k - 1) / 2 * static_cast<int64_t>(dilations[b]) > kMaxExtent) return DW_ETOOLARGE;
        if (dilations[b] > md) md = dilations[b];
    }
    if (!product_ok(n, c, h, w) || !product_ok(n * nb, c, h, w) || !product_ok(n * c, k * k, h, w))
        return DW_ETOOLARGE;
    const size_t e = elem_size(dtype);
    if (!aligned(x, e)) return DW_EPTR;
    for (int b = 0; b < nb; ++b)
        if (!aligned(filters[b], e)) return DW_EPTR;
    *maxdil = md;
    return DW_OK;
}

}  // namespace

// ---------------------------------------------------------------- kernel selection
namespace {

struct PassFns {
    int (*count)();
    const char *(*name_of)(int);
    bool (*feasible)(int, const dw::Geo &, int);
};
const PassFns kPassFns[3] = {{dw::fwd_algo_count, dw::fwd_algo_name_of, dw::fwd_algo_feasible},
                             {dw::bwd_input_algo_count, dw::bwd_input_algo_name_of, dw::bwd_input_algo_feasible},
                             {dw::bwd_weight_algo_count, dw::bwd_weight_algo_name_of, dw::bwd_weight_algo_feasible}};

// Times every family that can run (pass, g, dtype) with `run` (one compute
// call) and records the fastest; on an error the previous entry is restored.
template <class Run>
int tune_pass(int pass, const dw::Geo &g, int dtype, int reps, hipStream_t s, Run run, const char **chosen) {
    const PassFns &f = kPassFns[pass];
    const int prev = dw::tuned_algo(pass, g, dtype);
    reps = reps < 1 ? 1 : (reps > 1000 ? 1000 : reps);
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return DW_EHIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return DW_EHIP;
    }
    int best = -1, rc = DW_OK;
    float best_ms = 0.f;
    for (int a = 0; a < f.count() && rc == DW_OK; ++a) {
        if (!f.feasible(a, g, dtype)) continue;
        dw::set_tuned_algo(pass, g, dtype, a);
        rc = run();  // warm-up, and the first error stops the search
        if (rc != DW_OK) break;
        if (hipEventRecord(e0, s) != hipSuccess) {
            rc = DW_EHIP;
            break;
        }
        for (int r = 0; r < reps && rc == DW_OK; ++r) rc = run();
        if (rc != DW_OK) break;
        float ms = 0.f;
        if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
            hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
            rc = DW_EHIP;
            break;
        }
        if (best < 0 || ms < best_ms) {
            best = a;
            best_ms = ms;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (rc != DW_OK || best < 0) {
        dw::set_tuned_algo(pass, g, dtype, prev);
        return rc != DW_OK ? rc : DW_EUNSUPPORTED;
    }
    dw::set_tuned_algo(pass, g, dtype, best);
    if (chosen) *chosen = f.name_of(best);
    return DW_OK;
}

}  // namespace

// Device scratch of dwconv2d_bwd_weight_noalloc: the grad-weight's per-block
// partial sums (pass 1) that the fixed-order reduction (pass 2) reads back.
// Each GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// only the address hipGetSymbolAddress returns for a device is passed on.
static __device__ __align__(256) unsigned char scratch[DWCONV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device ordinal

// The current device's copy of `scratch`, resolved once per device with that
// device current.  Fails when the stream belongs to another device.
int scratch_for(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DW_EHIP;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return DW_EHIP;
        if (sdev != dev) return DW_ESCRATCH;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return DW_EHIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DW_OK;
}

}  // namespace

extern "C" {

int dwconv2d_out_size(int64_t n, int64_t ic, int64_t ih, int64_t iw, int64_t oc, int64_t kh, int64_t kw,
                      int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w, int64_t dil_h,
                      int64_t dil_w, int64_t *oh, int64_t *ow) {
    dw::Geo g;
    const int rc = check_geometry(n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, &g);
    if (rc != DW_OK) return rc;
    if (oh) *oh = g.oh;
    if (ow) *ow = g.ow;
    return DW_OK;
}

int dwconv2d_fwd(const void *x, const void *w, const void *bias, void *y, int64_t n, int64_t ic, int64_t ih,
                 int64_t iw, int64_t oc, int64_t kh, int64_t kw, int64_t stride_h, int64_t stride_w,
                 int64_t pad_h, int64_t pad_w, int64_t dil_h, int64_t dil_w, int dtype, void *stream) {
    if (dtype != DW_F32 && dtype != DW_F16 && dtype != DW_BF16) return DW_EDTYPE;
    dw::Geo g;
    const int rc = check_geometry(n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, &g);
    if (rc != DW_OK) return rc;
    const size_t e = elem_size(dtype);
    if (!x || !w || !y) return DW_EPTR;
    if (!aligned(x, e) || !aligned(w, e) || !aligned(y, e) || (bias && !aligned(bias, e))) return DW_EPTR;
    const size_t yb = y_bytes(g, e);
    if (overlap(y, yb, x, x_bytes(g, e)) || overlap(y, yb, w, w_bytes(g, e)) ||
        (bias && overlap(y, yb, bias, b_bytes(g, e))))
        return DW_EALIAS;
    return map_launch(dw::launch_fwd(g, x, w, bias, y, dtype, static_cast<hipStream_t>(stream)));
}

int dwconv2d_bwd_input(const void *dy, const void *w, void *dx, int64_t n, int64_t ic, int64_t ih, int64_t iw,
                       int64_t oc, int64_t kh, int64_t kw, int64_t stride_h, int64_t stride_w, int64_t pad_h,
                       int64_t pad_w, int64_t dil_h, int64_t dil_w, int dtype, void *stream) {
    if (dtype != DW_F32 && dtype != DW_F16 && dtype != DW_BF16) return DW_EDTYPE;
    dw::Geo g;
    const int rc = check_geometry(n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, &g);
    if (rc != DW_OK) return rc;
    const size_t e = elem_size(dtype);
    if (!dy || !w || !dx) return DW_EPTR;
    if (!aligned(dy, e) || !aligned(w, e) || !aligned(dx, e)) return DW_EPTR;
    const size_t xb = x_bytes(g, e);
    if (overlap(dx, xb, dy, y_bytes(g, e)) || overlap(dx, xb, w, w_bytes(g, e))) return DW_EALIAS;
    return map_launch(dw::launch_bwd_input(g, dy, w, dx, dtype, static_cast<hipStream_t>(stream)));
}

int dwconv2d_bwd_weight_workspace_bytes(int64_t n, int64_t ic, int64_t ih, int64_t iw, int64_t oc, int64_t kh,
                                        int64_t kw, int64_t stride_h, int64_t stride_w, int64_t pad_h,
                                        int64_t pad_w, int64_t dil_h, int64_t dil_w, int dtype, size_t *bytes) {
    if (dtype != DW_F32 && dtype != DW_F16 && dtype != DW_BF16) return DW_EDTYPE;
    dw::Geo g;
    const int rc = check_geometry(n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, &g);
    if (rc != DW_OK) return rc;
    const int64_t ws = dw::bwd_weight_workspace(g, dtype);
    if (ws < 0) return DW_EUNSUPPORTED;
    if (bytes) *bytes = static_cast<size_t>(ws);
    return DW_OK;
}

int dwconv2d_bwd_weight(const void *x, const void *dy, void *dwt, void *db, void *workspace,
                        size_t workspace_bytes, int64_t n, int64_t ic, int64_t ih, int64_t iw, int64_t oc,
                        int64_t kh, int64_t kw, int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                        int64_t dil_h, int64_t dil_w, int dtype, void *stream) {
    if (dtype != DW_F32 && dtype != DW_F16 && dtype != DW_BF16) return DW_EDTYPE;
    dw::Geo g;
    const int rc = check_geometry(n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, &g);
    if (rc != DW_OK) return rc;
    const size_t e = elem_size(dtype);
    if (!x || !dy || !dwt) return DW_EPTR;
    if (!aligned(x, e) || !aligned(dy, e) || !aligned(dwt, e) || (db && !aligned(db, e))) return DW_EPTR;
    const int64_t need = dw::bwd_weight_workspace(g, dtype);
    if (need < 0) return DW_EUNSUPPORTED;
    if (!workspace || workspace_bytes < static_cast<size_t>(need) || !aligned(workspace, 16))
        return DW_EWORKSPACE;
    const size_t xb = x_bytes(g, e), yb = y_bytes(g, e), wb = w_bytes(g, e), bb = b_bytes(g, e);
    const size_t wsb = static_cast<size_t>(need);
    if (overlap(dwt, wb, x, xb) || overlap(dwt, wb, dy, yb) || overlap(dwt, wb, workspace, wsb) ||
        overlap(workspace, wsb, x, xb) || overlap(workspace, wsb, dy, yb) ||
        (db && (overlap(db, bb, x, xb) || overlap(db, bb, dy, yb) || overlap(db, bb, dwt, wb) ||
                overlap(db, bb, workspace, wsb))))
        return DW_EALIAS;
    return map_launch(dw::launch_bwd_weight(g, x, dy, dwt, db, workspace, dtype, static_cast<hipStream_t>(stream)));
}

int dwconv2d_bwd_weight_noalloc(const void *x, const void *dy, void *dwt, void *db, int64_t n, int64_t ic,
                                int64_t ih, int64_t iw, int64_t oc, int64_t kh, int64_t kw, int64_t stride_h,
                                int64_t stride_w, int64_t pad_h, int64_t pad_w, int64_t dil_h, int64_t dil_w,
                                int dtype, void *stream) {
    if (dtype != DW_F32 && dtype != DW_F16 && dtype != DW_BF16) return DW_EDTYPE;
    dw::Geo g;
    const int rc = check_geometry(n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, &g);
    if (rc != DW_OK) return rc;
    const size_t e = elem_size(dtype);
    if (!x || !dy || !dwt) return DW_EPTR;
    if (!aligned(x, e) || !aligned(dy, e) || !aligned(dwt, e) || (db && !aligned(db, e))) return DW_EPTR;
    const int64_t need = dw::bwd_weight_workspace_selected(g, dtype);
    if (need < 0) return DW_EUNSUPPORTED;
    if (static_cast<uint64_t>(need) > DWCONV_NOALLOC_SCRATCH_BYTES) return DW_ESCRATCH;
    const size_t xb = x_bytes(g, e), yb = y_bytes(g, e), wb = w_bytes(g, e), bb = b_bytes(g, e);
    if (overlap(dwt, wb, x, xb) || overlap(dwt, wb, dy, yb) ||
        (db && (overlap(db, bb, x, xb) || overlap(db, bb, dy, yb) || overlap(db, bb, dwt, wb))))
        return DW_EALIAS;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    const int src = scratch_for(s, &ws);
    if (src != DW_OK) return src;
    // pass 1 overwrites every partial-sum slot pass 2 reads, so the scratch
    // needs no clearing between calls
    return map_launch(dw::launch_bwd_weight(g, x, dy, dwt, db, ws, dtype, s));
}

int dynconv_multidil_fwd_into(const void *x, const void *const *filters, const int32_t *dilations, int32_t nb,
                              void *y, int64_t y_channels, int64_t y_offset, int64_t n, int64_t c, int64_t h,
                              int64_t w, int64_t k, int dtype, void *stream) {
    int maxdil = 1;
    const int rc = check_dyn(x, filters, dilations, nb, n, c, h, w, k, dtype, &maxdil);
    if (rc != DW_OK) return rc;
    if (!y) return DW_EPTR;
    if (y_channels < 1 || y_offset < 0 || y_offset + nb * c > y_channels) return DW_ESHAPE;
    if (y_channels > kMaxExtent || !product_ok(n, y_channels, h, w)) return DW_ETOOLARGE;
    const size_t e = elem_size(dtype);
    if (!aligned(y, e)) return DW_EPTR;
    const size_t xb = static_cast<size_t>(n * c * h * w) * e;
    const size_t yb = static_cast<size_t>(n * y_channels * h * w) * e;
    const size_t fb = static_cast<size_t>(n * c * k * k * h * w) * e;
    if (overlap(y, yb, x, xb)) return DW_EALIAS;
    for (int b = 0; b < nb; ++b)
        if (overlap(y, yb, filters[b], fb)) return DW_EALIAS;
    return map_launch(dw::launch_dynconv(x, filters, dilations, nb, y, static_cast<int>(y_channels),
                                         static_cast<int>(y_offset), static_cast<int>(n), static_cast<int>(c),
                                         static_cast<int>(h), static_cast<int>(w), static_cast<int>(k), dtype,
                                         static_cast<hipStream_t>(stream)));
}

int dynconv_multidil_fwd(const void *x, const void *const *filters, const int32_t *dilations, int32_t nb,
                         void *y, int64_t n, int64_t c, int64_t h, int64_t w, int64_t k, int dtype, void *stream) {
    // the branch-concatenated output alone: nb*c channels, branch 0 at channel 0
    const int64_t ych = (nb >= 1 && nb <= 4) ? nb * c : 1;
    return dynconv_multidil_fwd_into(x, filters, dilations, nb, y, ych, 0, n, c, h, w, k, dtype, stream);
}

int dynconv_multidil_bwd_from(const void *x, const void *const *filters, const void *dy, int64_t dy_channels,
                              int64_t dy_offset, const int32_t *dilations, int32_t nb, void *dx,
                              void *const *dfilters, int64_t n, int64_t c, int64_t h, int64_t w, int64_t k,
                              int dtype, void *stream) {
    int maxdil = 1;
    const int rc = check_dyn(x, filters, dilations, nb, n, c, h, w, k, dtype, &maxdil);
    if (rc != DW_OK) return rc;
    if (!dy) return DW_EPTR;
    if (dy_channels < 1 || dy_offset < 0 || dy_offset + nb * c > dy_channels) return DW_ESHAPE;
    if (dy_channels > kMaxExtent || !product_ok(n, dy_channels, h, w)) return DW_ETOOLARGE;
    const size_t e = elem_size(dtype);
    if (!aligned(dy, e) || (dx && !aligned(dx, e))) return DW_EPTR;
    for (int b = 0; dfilters && b < nb; ++b)
        if (dfilters[b] && !aligned(dfilters[b], e)) return DW_EPTR;
    const size_t xb = static_cast<size_t>(n * c * h * w) * e;
    const size_t yb = static_cast<size_t>(n * dy_channels * h * w) * e;
    const size_t fb = static_cast<size_t>(n * c * k * k * h * w) * e;
    // every output against every input and every other output
    const void *outs[1 + 4];
    size_t osz[1 + 4];
    int no = 0;
    if (dx) {
        outs[no] = dx;
        osz[no++] = xb;
    }
    for (int b = 0; dfilters && b < nb; ++b)
        if (dfilters[b]) {
            outs[no] = dfilters[b];
            osz[no++] = fb;
        }
    for (int o = 0; o < no; ++o) {
        if (overlap(outs[o], osz[o], x, xb) || overlap(outs[o], osz[o], dy, yb)) return DW_EALIAS;
        for (int b = 0; b < nb; ++b)
            if (overlap(outs[o], osz[o], filters[b], fb)) return DW_EALIAS;
        for (int q = o + 1; q < no; ++q)
            if (overlap(outs[o], osz[o], outs[q], osz[q])) return DW_EALIAS;
    }
    if (no == 0) return DW_OK;  // nothing requested
    return map_launch(dw::launch_dynconv_bwd(x, filters, dy, static_cast<int>(dy_channels), static_cast<int>(dy_offset),
                                             dilations, nb, dx, dfilters, static_cast<int>(n), static_cast<int>(c),
                                             static_cast<int>(h), static_cast<int>(w), static_cast<int>(k), dtype,
                                             static_cast<hipStream_t>(stream)));
}

int dynconv_multidil_bwd(const void *x, const void *const *filters, const void *dy, const int32_t *dilations,
                         int32_t nb, void *dx, void *const *dfilters, int64_t n, int64_t c, int64_t h, int64_t w,
                         int64_t k, int dtype, void *stream) {
    const int64_t dych = (nb >= 1 && nb <= 4) ? nb * c : 1;
    return dynconv_multidil_bwd_from(x, filters, dy, dych, 0, dilations, nb, dx, dfilters, n, c, h, w, k, dtype,
                                     stream);
}

const char *dwconv2d_algo(int pass, int64_t n, int64_t ic, int64_t ih, int64_t iw, int64_t oc, int64_t kh,
                          int64_t kw, int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                          int64_t dil_h, int64_t dil_w, int dtype) {
    if (dtype != DW_F32 && dtype != DW_F16 && dtype != DW_BF16) return nullptr;
    dw::Geo g;
    if (check_geometry(n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, &g) != DW_OK)
        return nullptr;
    switch (pass) {
        case 0: return dw::fwd_supported(g, dtype) ? dw::fwd_algo_name(g, dtype) : nullptr;
        case 1: return dw::bwd_input_supported(g, dtype) ? dw::bwd_input_algo_name(g, dtype) : nullptr;
        case 2: return dw::bwd_weight_workspace(g, dtype) >= 0 ? dw::bwd_weight_algo_name(g, dtype) : nullptr;
        default: return nullptr;
    }
}

int dwconv2d_algo_candidates(int pass, int64_t n, int64_t ic, int64_t ih, int64_t iw, int64_t oc, int64_t kh,
                             int64_t kw, int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                             int64_t dil_h, int64_t dil_w, int dtype, const char **names, int cap) {
    if (dtype != DW_F32 && dtype != DW_F16 && dtype != DW_BF16) return DW_EDTYPE;
    if (pass < 0 || pass > 2) return DW_ESHAPE;
    dw::Geo g;
    const int rc = check_geometry(n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, &g);
    if (rc != DW_OK) return rc;
    if (cap > 0 && !names) return DW_EPTR;
    const PassFns &f = kPassFns[pass];
    int cnt = 0;
    for (int a = 0; a < f.count(); ++a) {
        if (!f.feasible(a, g, dtype)) continue;
        if (cnt < cap) names[cnt] = f.name_of(a);
        ++cnt;
    }
    return cnt;
}

int dwconv2d_set_algo(int pass, int64_t n, int64_t ic, int64_t ih, int64_t iw, int64_t oc, int64_t kh, int64_t kw,
                      int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w, int64_t dil_h,
                      int64_t dil_w, int dtype, const char *algo) {
    if (dtype != DW_F32 && dtype != DW_F16 && dtype != DW_BF16) return DW_EDTYPE;
    if (pass < 0 || pass > 2) return DW_ESHAPE;
    dw::Geo g;
    const int rc = check_geometry(n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, &g);
    if (rc != DW_OK) return rc;
    if (!algo) {
        dw::set_tuned_algo(pass, g, dtype, -1);
        return DW_OK;
    }
    const PassFns &f = kPassFns[pass];
    for (int a = 0; a < f.count(); ++a) {
        if (std::strcmp(f.name_of(a), algo) == 0 && f.feasible(a, g, dtype)) {
            dw::set_tuned_algo(pass, g, dtype, a);
            return DW_OK;
        }
    }
    return DW_EUNSUPPORTED;
}

int dwconv2d_tune_fwd(const void *x, const void *w, const void *bias, void *y, int64_t n, int64_t ic, int64_t ih,
                      int64_t iw, int64_t oc, int64_t kh, int64_t kw, int64_t stride_h, int64_t stride_w,
                      int64_t pad_h, int64_t pad_w, int64_t dil_h, int64_t dil_w, int dtype, int reps, void *stream,
                      const char **chosen) {
    auto run = [&] {
        return dwconv2d_fwd(x, w, bias, y, n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w,
                            dtype, stream);
    };
    const int rc = run();  // full validation with the current choice
    if (rc != DW_OK) return rc;
    dw::Geo g;
    check_geometry(n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, &g);
    return tune_pass(0, g, dtype, reps, static_cast<hipStream_t>(stream), run, chosen);
}

int dwconv2d_tune_bwd_input(const void *dy, const void *w, void *dx, int64_t n, int64_t ic, int64_t ih, int64_t iw,
                            int64_t oc, int64_t kh, int64_t kw, int64_t stride_h, int64_t stride_w, int64_t pad_h,
                            int64_t pad_w, int64_t dil_h, int64_t dil_w, int dtype, int reps, void *stream,
                            const char **chosen) {
    auto run = [&] {
        return dwconv2d_bwd_input(dy, w, dx, n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h,
                                  dil_w, dtype, stream);
    };
    const int rc = run();
    if (rc != DW_OK) return rc;
    dw::Geo g;
    check_geometry(n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, &g);
    return tune_pass(1, g, dtype, reps, static_cast<hipStream_t>(stream), run, chosen);
}

int dwconv2d_tune_bwd_weight(const void *x, const void *dy, void *dwt, void *db, void *workspace,
                             size_t workspace_bytes, int64_t n, int64_t ic, int64_t ih, int64_t iw, int64_t oc,
                             int64_t kh, int64_t kw, int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                             int64_t dil_h, int64_t dil_w, int dtype, int reps, void *stream, const char **chosen) {
    auto run = [&] {
        return dwconv2d_bwd_weight(x, dy, dwt, db, workspace, workspace_bytes, n, ic, ih, iw, oc, kh, kw, stride_h,
                                   stride_w, pad_h, pad_w, dil_h, dil_w, dtype, stream);
    };
    const int rc = run();
    if (rc != DW_OK) return rc;
    dw::Geo g;
    check_geometry(n, ic, ih, iw, oc, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, &g);
    return tune_pass(2, g, dtype, reps, static_cast<hipStream_t>(stream), run, chosen);
}

const char *dw_status_str(int status) {
    switch (status) {
        case DW_OK: return "ok";
        case DW_EPTR: return "a required pointer is NULL or not aligned to its element size";
        case DW_ESHAPE: return "invalid size, stride, dilation or padding, or empty output";
        case DW_EMULT: return "output channels are not a multiple of input channels";
        case DW_EDTYPE: return "unknown dtype";
        case DW_EWORKSPACE: return "workspace missing, too small or not 16-byte aligned";
        case DW_ETOOLARGE: return "a tensor has 2^31 elements or more, or an extent exceeds 2^30";
        case DW_EALIAS: return "an output overlaps an input or another output";
        case DW_EHIP: return "HIP kernel launch failed";
        case DW_EDYN: return "dynamic filter: k must be odd, 1 <= nb <= 4, dilations >= 1";
        case DW_EUNSUPPORTED: return "kernel family cannot run this geometry";
        case DW_ESCRATCH:
            return "no-alloc grad-weight: partial sums exceed the fixed device scratch, or the stream is on "
                   "another device";
        default: return "unknown status";
    }
}

}  // extern "C"
