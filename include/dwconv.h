/*
 * dwconv.h -- C ABI of the MI355X (gfx950) depthwise and dynamic-filter
 * convolution library (libdwconv.so).
 *
 * Problem statement (MegEngine large-kernel depthwise article, section on
 * going from convolution to matrix multiplication): input x is (n, ic, ih, iw),
 * the kernel is (oc, ic, kh, kw) and the output is (n, oc, oh, ow).  In the
 * depthwise case each output channel sees one input channel only, so the
 * kernel is stored as (oc, kh, kw) -- bitwise the same as (oc, 1, kh, kw).
 *
 * Features (PyTorch PR #3057 "Spatial Depthwise Convolution on the GPU": its
 * TODO list and commit history): zero padding, stride, dilation, a depth
 * multiplier M = oc / ic (output channel o reads input channel o / M, so the
 * M filters of one input channel are adjacent), an optional bias and its
 * gradient, and half precision with a wider accumulation type.
 *
 * Shared conventions
 * ------------------
 *  - Every tensor pointer is a DEVICE pointer to a dense, row-major (NCHW)
 *    array owned by the caller.  The library never allocates or frees device
 *    memory, never synchronises (the dwconv2d_tune_* calls excepted) and
 *    keeps no pointer after a call returns.
 *    Host arrays (filters[], dilations[]) are read during the call only.
 *  - dtype selects the element type of every tensor of the call: DW_F32,
 *    DW_F16 (IEEE binary16) or DW_BF16 (bfloat16).  Arithmetic is fp32;
 *    16-bit results are rounded to nearest-even on the final store.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns without waiting for it.
 *  - Every pointer must be aligned to its element size.
 *  - Geometry: cross-correlation (no kernel flip); symmetric zero padding per
 *    axis; oh = floor((ih + 2*pad_h - dil_h*(kh-1) - 1) / stride_h) + 1 and
 *    likewise ow.  All sizes, strides and dilations >= 1, pads >= 0,
 *    oc % ic == 0, oh >= 1, ow >= 1, and every tensor below 2^31 elements.
 *  - Errors: a negative status code, never an abort, exception or print.
 *    All argument checks run before any HIP call; when one fails nothing is
 *    launched and no output is touched.  DW_EHIP reports a failed launch.
 *  - Thread safety: concurrent calls on different streams with disjoint
 *    outputs are safe.  The only state is the kernel-selection table
 *    (dwconv2d_set_algo / dwconv2d_tune_*), guarded by a mutex; it changes
 *    which kernel family runs, never the values a call may produce beyond
 *    fp32 rounding order.
 */
#ifndef DWCONV_H
#define DWCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum dw_dtype { DW_F32 = 0, DW_F16 = 1, DW_BF16 = 2 };

enum dw_status {
    DW_OK = 0,
    DW_EPTR = -1,       /* a required pointer is NULL or not aligned to its element size */
    DW_ESHAPE = -2,     /* a size/stride/dilation < 1, a pad < 0, or an empty output */
    DW_EMULT = -3,      /* oc is not a multiple of ic */
    DW_EDTYPE = -4,     /* dtype is not one of enum dw_dtype */
    DW_EWORKSPACE = -5, /* workspace NULL or smaller than dwconv2d_bwd_weight_workspace_bytes */
    DW_ETOOLARGE = -6,  /* some tensor has 2^31 elements or more, or an extent
                           (size, stride, pad, dilated kernel span) exceeds 2^30 */
    DW_EALIAS = -7,     /* an output overlaps an input or another output */
    DW_EHIP = -8,       /* a HIP launch failed (hipGetLastError after the launch) */
    DW_EDYN = -9,       /* dynamic filter: k even, nb outside [1, 4], or a dilation < 1 */
    DW_EUNSUPPORTED = -10, /* dwconv2d_set_algo: a kernel-family name that cannot run the
                              geometry (the compute calls serve every valid geometry: rows
                              too wide for a family's LDS staging run on direct kernels) */
    DW_ESCRATCH = -11     /* dwconv2d_bwd_weight_noalloc: the partial sums need more than
                             DWCONV_NOALLOC_SCRATCH_BYTES, or the stream belongs to a device
                             other than the current one */
};

/* Size of the device array dwconv2d_bwd_weight_noalloc keeps its partial sums in. */
#define DWCONV_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * Output spatial size for the geometry above.  Writes *oh and *ow (either may
 * be NULL) and returns DW_OK, or returns DW_ESHAPE / DW_EMULT / DW_ETOOLARGE
 * exactly as the compute calls would for the same geometry.  Host only.
 */
int dwconv2d_out_size(int64_t n, int64_t ic, int64_t ih, int64_t iw,
                      int64_t oc, int64_t kh, int64_t kw,
                      int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                      int64_t dil_h, int64_t dil_w, int64_t *oh, int64_t *ow);

/*
 * Forward (PR #3057: depthwise forward kernel with padding, stride,
 * dilation, multiplier and bias):
 *   y[n, o, p, q] = bias[o]
 *       + sum_{i<kh, j<kw} w[o, i, j] * x[n, o/M, p*stride_h - pad_h + i*dil_h,
 *                                             q*stride_w - pad_w + j*dil_w]
 * with out-of-image taps contributing zero.
 *   x    (n, ic, ih, iw)   input
 *   w    (oc, kh, kw)      filters
 *   bias (oc) or NULL      added after accumulation, before rounding
 *   y    (n, oc, oh, ow)   output, fully overwritten
 */
int dwconv2d_fwd(const void *x, const void *w, const void *bias, void *y,
                 int64_t n, int64_t ic, int64_t ih, int64_t iw,
                 int64_t oc, int64_t kh, int64_t kw,
                 int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                 int64_t dil_h, int64_t dil_w, int dtype, void *stream);

/*
 * Gradient with respect to the input (PR #3057: the grad-input kernel of the
 * depthwise convolution): the adjoint of the forward in x,
 *   dx[n, g, h, c] = sum over (m < M, i, j, p, q) with
 *                    p*stride_h - pad_h + i*dil_h == h and
 *                    q*stride_w - pad_w + j*dil_w == c
 *                    of w[g*M + m, i, j] * dy[n, g*M + m, p, q].
 *   dy (n, oc, oh, ow)   incoming gradient
 *   w  (oc, kh, kw)      filters
 *   dx (n, ic, ih, iw)   output, fully overwritten (elements no tap reaches are 0)
 */
int dwconv2d_bwd_input(const void *dy, const void *w, void *dx,
                       int64_t n, int64_t ic, int64_t ih, int64_t iw,
                       int64_t oc, int64_t kh, int64_t kw,
                       int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                       int64_t dil_h, int64_t dil_w, int dtype, void *stream);

/*
 * Bytes of device workspace dwconv2d_bwd_weight needs for this geometry and
 * dtype (always > 0): the largest any kernel family that can run the
 * geometry needs, so the buffer serves whichever family is selected.
 * Writes *bytes; returns a status as dwconv2d_out_size.
 */
int dwconv2d_bwd_weight_workspace_bytes(int64_t n, int64_t ic, int64_t ih, int64_t iw,
                                        int64_t oc, int64_t kh, int64_t kw,
                                        int64_t stride_h, int64_t stride_w,
                                        int64_t pad_h, int64_t pad_w,
                                        int64_t dil_h, int64_t dil_w, int dtype,
                                        size_t *bytes);

/*
 * Gradient with respect to the filters and the bias (PR #3057: the
 * grad-weight kernel, later extended to padding, stride and dilation, and
 * the bias gradient added with it):
 *   dw[o, i, j] = sum_{n, p, q} dy[n, o, p, q] * x[n, o/M, p*stride_h - pad_h + i*dil_h,
 *                                                       q*stride_w - pad_w + j*dil_w]
 *   db[o]       = sum_{n, p, q} dy[n, o, p, q]
 *   x         (n, ic, ih, iw)   forward input
 *   dy        (n, oc, oh, ow)   incoming gradient
 *   dw        (oc, kh, kw)      output, overwritten
 *   db        (oc) or NULL      output, overwritten when non-NULL
 *   workspace device scratch of at least dwconv2d_bwd_weight_workspace_bytes
 *             bytes, aligned to 16 bytes, owned by the caller; its contents on
 *             entry do not matter and are garbage on exit.
 * Two kernels run in stream order (per-block partial sums, then a fixed-order
 * reduction); no atomics, so results are bitwise reproducible run to run.
 */
int dwconv2d_bwd_weight(const void *x, const void *dy, void *dw, void *db,
                        void *workspace, size_t workspace_bytes,
                        int64_t n, int64_t ic, int64_t ih, int64_t iw,
                        int64_t oc, int64_t kh, int64_t kw,
                        int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                        int64_t dil_h, int64_t dil_w, int dtype, void *stream);

/*
 * dwconv2d_bwd_weight without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and kernels as dwconv2d_bwd_weight, bit for bit; the
 * partial sums go to a fixed device array of DWCONV_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends
 * (resolved on the first call on each device, with that device current).
 *   Succeeds whenever dwconv2d_bwd_weight_workspace_bytes reports at most
 *   DWCONV_NOALLOC_SCRATCH_BYTES for the geometry (it needs only the selected
 *   kernel family's part of that figure); returns DW_ESCRATCH when the
 *   partial sums do not fit, or when `stream` is not on the current device.
 *   Calls no hipMalloc, hipFree or hipMemset: the array keeps the last call's
 *   contents, and the first kernel overwrites every value the second reads.
 *   Every call on one GPU shares that GPU's array: calls that may overlap on
 *   one GPU (different streams, different host threads) race and must be
 *   ordered by the caller.
 */
int dwconv2d_bwd_weight_noalloc(const void *x, const void *dy, void *dw, void *db,
                                int64_t n, int64_t ic, int64_t ih, int64_t iw,
                                int64_t oc, int64_t kh, int64_t kw,
                                int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                                int64_t dil_h, int64_t dil_w, int dtype, void *stream);

/*
 * Fused per-pixel dynamic filter at several dilations, written straight into
 * the channel-concatenated result (lartpang/DynamicConvolutionOperator: the
 * Dynamic Dilated Pyramid computation of HDFNet, sections on the
 * optimisation analysis and the solution -- no unfold buffer, no concat copy):
 *   y[n, b*c + ch, h, w] = sum_{i, j < k} F_b[n, ch, i*k + j, h, w]
 *                          * x[n, ch, h + (i - r)*d_b, w + (j - r)*d_b]
 * for every branch b < nb, with r = (k - 1)/2, d_b = dilations[b] and zero
 * outside the image (i.e. zero padding r*d_b, stride 1, output h x w).
 *   x          (n, c, h, w)            input
 *   filters    host array of nb device pointers; filters[b] is (n, c, k*k, h, w)
 *   dilations  host array of nb dilations (e.g. {1, 3, 5})
 *   nb         number of branches, 1..4
 *   y          (n, nb*c, h, w)         output, fully overwritten, branch-major
 *   k          odd window size
 */
int dynconv_multidil_fwd(const void *x, const void *const *filters,
                         const int32_t *dilations, int32_t nb, void *y,
                         int64_t n, int64_t c, int64_t h, int64_t w, int64_t k,
                         int dtype, void *stream);

/*
 * Backward of dynconv_multidil_fwd (the page's benchmark of the fused
 * operator times it together with its backward).  y is bilinear in x and
 * the filters, so with dy the gradient of y:
 *   dF_b[n, ch, i*k + j, h, w] = dy[n, b*c + ch, h, w] * x[n, ch, h + (i - r)*d_b, w + (j - r)*d_b]
 *                                (0 where that pixel is outside the image)
 *   dx[n, ch, sh, sw]          = sum over b, i, j of F_b[n, ch, i*k + j, h, w] * dy[n, b*c + ch, h, w]
 *                                at (h, w) = (sh - (i - r)*d_b, sw - (j - r)*d_b) inside the image.
 *   x, filters, dilations, nb, k   as for dynconv_multidil_fwd (all required)
 *   dy         (n, nb*c, h, w)     gradient of the branch-concatenated output
 *   dx         (n, c, h, w) or NULL: fully overwritten when non-NULL
 *   dfilters   host array of nb device pointers, or NULL; dfilters[b] is
 *              (n, c, k*k, h, w), fully overwritten, or NULL to skip branch b
 * Each dx element is summed by one thread in a fixed order, so results are
 * bitwise reproducible.  With dx NULL and no filter gradient requested the
 * call validates its arguments, launches nothing and returns DW_OK.
 */
int dynconv_multidil_bwd(const void *x, const void *const *filters, const void *dy,
                         const int32_t *dilations, int32_t nb, void *dx, void *const *dfilters,
                         int64_t n, int64_t c, int64_t h, int64_t w, int64_t k,
                         int dtype, void *stream);

/*
 * dynconv_multidil_fwd into a caller-owned larger concatenation: the page's
 * fused operator stores each branch straight into the tensor the downstream
 * aggregation reads.  Branch b, channel ch is written to channel
 * y_offset + b*c + ch of y, an (n, y_channels, h, w) tensor; its other
 * channels are not touched.  Requires y_offset >= 0 and
 * y_offset + nb*c <= y_channels (else DW_ESHAPE); the whole of y must not
 * overlap x or a filter (DW_EALIAS).  dynconv_multidil_fwd is this call with
 * y_channels = nb*c and y_offset = 0.
 */
int dynconv_multidil_fwd_into(const void *x, const void *const *filters,
                              const int32_t *dilations, int32_t nb, void *y,
                              int64_t y_channels, int64_t y_offset,
                              int64_t n, int64_t c, int64_t h, int64_t w, int64_t k,
                              int dtype, void *stream);

/*
 * dynconv_multidil_bwd with dy taken from a larger gradient tensor: the
 * gradient of branch b, channel ch is read from channel dy_offset + b*c + ch
 * of dy, an (n, dy_channels, h, w) tensor (the gradient of the concatenation
 * that dynconv_multidil_fwd_into wrote into).  Same requirements on the
 * channel range as above; dynconv_multidil_bwd is this call with
 * dy_channels = nb*c and dy_offset = 0.
 */
int dynconv_multidil_bwd_from(const void *x, const void *const *filters, const void *dy,
                              int64_t dy_channels, int64_t dy_offset,
                              const int32_t *dilations, int32_t nb, void *dx, void *const *dfilters,
                              int64_t n, int64_t c, int64_t h, int64_t w, int64_t k,
                              int dtype, void *stream);

/*
 * Kernel family a call would launch for this geometry and dtype (for
 * profiling and per-shape tuning; the same decision the compute calls make).
 * pass: 0 = dwconv2d_fwd, 1 = dwconv2d_bwd_input, 2 = dwconv2d_bwd_weight.
 * Returns a static string, or NULL for an invalid pass, dtype or geometry.
 * Host only; launches nothing.
 */
const char *dwconv2d_algo(int pass, int64_t n, int64_t ic, int64_t ih, int64_t iw,
                          int64_t oc, int64_t kh, int64_t kw,
                          int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                          int64_t dil_h, int64_t dil_w, int dtype);

/*
 * Kernel selection per geometry (the MegEngine large-kernel depthwise article
 * chooses among its algorithms automatically; here the choice is measured on
 * the device the library runs on).  Several kernel families can often run one
 * geometry -- the names dwconv2d_algo returns.  A process-wide table, keyed by
 * (pass, dtype, the 13 geometry integers), overrides the built-in choice; the
 * compute calls and dwconv2d_algo consult it.  Every family computes the same
 * sums (fp32 accumulation in its own order), so the table affects speed, not
 * the tolerance results meet.
 *
 * dwconv2d_algo_candidates: writes the names (static strings) of the families
 *   that can run `pass` for this geometry and dtype into names[0..cap) and
 *   returns how many there are (which may exceed cap; names may be NULL when
 *   cap is 0), or a negative status.  Host only.
 * dwconv2d_set_algo: records family `algo` (one of the candidates' names) for
 *   this key, or removes the key's entry when algo is NULL.  Returns
 *   DW_EUNSUPPORTED for a name that cannot run the geometry.  Host only.
 * dwconv2d_tune_fwd / _bwd_input / _bwd_weight: take exactly the arguments of
 *   the matching compute call (outputs are overwritten, several times), plus
 *   `reps` (timed calls per candidate, clamped to 1..1000) and `chosen`
 *   (NULL, or where to write the winner's name).  After one validating call
 *   they run every candidate once, then `reps` times between two HIP events
 *   on `stream`, and record the fastest for this key.  They synchronise on
 *   the events and must not be called during stream capture.  For
 *   grad-weight, dwconv2d_bwd_weight_workspace_bytes already covers every
 *   candidate.  On error the key's previous entry is restored.
 */
int dwconv2d_algo_candidates(int pass, int64_t n, int64_t ic, int64_t ih, int64_t iw,
                             int64_t oc, int64_t kh, int64_t kw,
                             int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                             int64_t dil_h, int64_t dil_w, int dtype, const char **names, int cap);

int dwconv2d_set_algo(int pass, int64_t n, int64_t ic, int64_t ih, int64_t iw,
                      int64_t oc, int64_t kh, int64_t kw,
                      int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                      int64_t dil_h, int64_t dil_w, int dtype, const char *algo);

int dwconv2d_tune_fwd(const void *x, const void *w, const void *bias, void *y,
                      int64_t n, int64_t ic, int64_t ih, int64_t iw,
                      int64_t oc, int64_t kh, int64_t kw,
                      int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                      int64_t dil_h, int64_t dil_w, int dtype, int reps, void *stream,
                      const char **chosen);

int dwconv2d_tune_bwd_input(const void *dy, const void *w, void *dx,
                            int64_t n, int64_t ic, int64_t ih, int64_t iw,
                            int64_t oc, int64_t kh, int64_t kw,
                            int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                            int64_t dil_h, int64_t dil_w, int dtype, int reps, void *stream,
                            const char **chosen);

int dwconv2d_tune_bwd_weight(const void *x, const void *dy, void *dw, void *db,
                             void *workspace, size_t workspace_bytes,
                             int64_t n, int64_t ic, int64_t ih, int64_t iw,
                             int64_t oc, int64_t kh, int64_t kw,
                             int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                             int64_t dil_h, int64_t dil_w, int dtype, int reps, void *stream,
                             const char **chosen);

/* Static, human-readable text for a status code (never NULL). */
const char *dw_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* DWCONV_H */
