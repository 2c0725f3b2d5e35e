/*
 * dwconv_oracle.c -- plain, slow, obviously correct CPU oracle for per-channel
 * (depthwise) 2-D convolution and the per-pixel dynamic multi-dilation filter.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, import or
 * call this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source, header, table or helper with the
 * HIP library.
 *
 * All arithmetic is fp64.  Callers pass fp64 arrays that hold the exact upcast
 * of whatever (possibly 16-bit) inputs the device sees; outputs stay fp64.
 * Loops follow the mathematical definitions directly, with no blocking,
 * fusion or reordering:
 *
 *   Problem statement (MegEngine large-kernel depthwise article, section
 *   "from convolution to matrix multiplication"): input (n, ic, ih, iw),
 *   kernel (oc, ic, kh, kw), output (n, oc, oh, ow).  For the depthwise case
 *   every output channel sees exactly one input channel, so the kernel is
 *   stored as (oc, kh, kw).
 *
 *   Depth multiplier, padding, stride and dilation (PyTorch PR #3057
 *   "Spatial Depthwise Convolution on the GPU": its TODO list and its commit
 *   history add padding, strides, dilation, a depthwise multiplier and bias).
 *   Output channel oc reads input channel oc / M with M = oc_count / ic_count,
 *   i.e. the M filters of one input channel are adjacent (the groups=ic
 *   ordering of nn.Conv2d).  Cross-correlation: no kernel flip.
 *
 *   Backward passes are the literal chain rule of the forward loop nest:
 *   grad-input scatters w*dy into every input element a forward tap read,
 *   grad-weight accumulates dy*x over every (n, oh, ow) of that tap, and
 *   grad-bias is the sum of dy.  This is deliberately the scatter form; the
 *   device path uses gathers.
 *
 *   Dynamic multi-dilation filter (lartpang/DynamicConvolutionOperator,
 *   sections "optimisation analysis" and "solution"): for every pixel a k x k
 *   window is sampled at dilation d_b, multiplied elementwise with that
 *   pixel's own per-channel filter and summed; the branch results for the
 *   dilations (1, 3, 5) are concatenated along channels, branch-major.
 *   Filter layout per branch: (n, c, k*k, h, w), tap t = i*k + j (row-major,
 *   the unfold ordering the page's baseline uses); zero padding r*d_b with
 *   r = (k-1)/2, so the output keeps the input's h x w.
 *
 * Parallelism: OpenMP over independent output planes only; each thread owns
 * the whole plane it writes, so results do not depend on the thread count.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of output positions along one axis: the positions o >= 0 with
 * o*s - p + (k-1)*d <= in - 1 + p, i.e. floor((in + 2p - d(k-1) - 1)/s) + 1.
 * Returns 0 when not even one window fits. */
int64_t oracle_out_size(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d)
{
    int64_t o = 0;
    if (in < 1 || k < 1 || s < 1 || p < 0 || d < 1) return 0;
    /* count by enumeration of the first input index each window touches */
    while (o * s - p + (k - 1) * d <= in - 1 + p) o++;
    return o;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of OpenMP threads later calls run on (timing at one thread
 * and at all of them); results do not depend on it. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* y[n, oc, oh, ow] = b[oc] + sum_{i<kh, j<kw} w[oc, i, j] * x[n, oc/M, oh*sh - ph + i*dh, ow*sw - pw + j*dw]
 * (out-of-image taps contribute nothing). b may be NULL. */
void oracle_dwconv_fwd(const double *x, const double *w, const double *b, double *y,
                       int64_t n, int64_t ic, int64_t ih, int64_t iw,
                       int64_t oc, int64_t kh, int64_t kw,
                       int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                       int64_t dh, int64_t dw)
{
    const int64_t oh_n = oracle_out_size(ih, kh, sh, ph, dh);
    const int64_t ow_n = oracle_out_size(iw, kw, sw, pw, dw);
    const int64_t mult = oc / ic;
    int64_t plane;
#pragma omp parallel for schedule(dynamic, 1)
    for (plane = 0; plane < n * oc; plane++) {
        const int64_t nn = plane / oc, o = plane % oc, g = o / mult;
        const double *xp = x + (nn * ic + g) * ih * iw;
        const double *wp = w + o * kh * kw;
        double *yp = y + (nn * oc + o) * oh_n * ow_n;
        for (int64_t oh = 0; oh < oh_n; oh++)
            for (int64_t ow = 0; ow < ow_n; ow++) {
                double acc = b ? b[o] : 0.0;
                for (int64_t i = 0; i < kh; i++)
                    for (int64_t j = 0; j < kw; j++) {
                        const int64_t h = oh * sh - ph + i * dh;
                        const int64_t c = ow * sw - pw + j * dw;
                        if (h >= 0 && h < ih && c >= 0 && c < iw)
                            acc += wp[i * kw + j] * xp[h * iw + c];
                    }
                yp[oh * ow_n + ow] = acc;
            }
    }
}

/* dx = d<dy, fwd(x, w)>/dx: for every forward tap that read x[n, g, h, c]
 * add w[o, i, j] * dy[n, o, oh, ow] to dx[n, g, h, c]; untouched elements stay 0. */
void oracle_dwconv_bwd_input(const double *dy, const double *w, double *dx,
                             int64_t n, int64_t ic, int64_t ih, int64_t iw,
                             int64_t oc, int64_t kh, int64_t kw,
                             int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                             int64_t dh, int64_t dw)
{
    const int64_t oh_n = oracle_out_size(ih, kh, sh, ph, dh);
    const int64_t ow_n = oracle_out_size(iw, kw, sw, pw, dw);
    const int64_t mult = oc / ic;
    int64_t plane;
#pragma omp parallel for schedule(dynamic, 1)
    for (plane = 0; plane < n * ic; plane++) {
        const int64_t nn = plane / ic, g = plane % ic;
        double *dxp = dx + (nn * ic + g) * ih * iw;
        memset(dxp, 0, (size_t)(ih * iw) * sizeof(double));
        for (int64_t m = 0; m < mult; m++) {
            const int64_t o = g * mult + m;
            const double *dyp = dy + (nn * oc + o) * oh_n * ow_n;
            const double *wp = w + o * kh * kw;
            for (int64_t oh = 0; oh < oh_n; oh++)
                for (int64_t ow = 0; ow < ow_n; ow++)
                    for (int64_t i = 0; i < kh; i++)
                        for (int64_t j = 0; j < kw; j++) {
                            const int64_t h = oh * sh - ph + i * dh;
                            const int64_t c = ow * sw - pw + j * dw;
                            if (h >= 0 && h < ih && c >= 0 && c < iw)
                                dxp[h * iw + c] += wp[i * kw + j] * dyp[oh * ow_n + ow];
                        }
        }
    }
}

/* dw[o, i, j] = sum_{n, oh, ow} dy[n, o, oh, ow] * x[n, o/M, oh*sh - ph + i*dh, ow*sw - pw + j*dw]
 * db[o] = sum_{n, oh, ow} dy[n, o, oh, ow]   (db may be NULL) */
void oracle_dwconv_bwd_weight(const double *x, const double *dy, double *dwt, double *db,
                              int64_t n, int64_t ic, int64_t ih, int64_t iw,
                              int64_t oc, int64_t kh, int64_t kw,
                              int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                              int64_t dh, int64_t dw)
{
    const int64_t oh_n = oracle_out_size(ih, kh, sh, ph, dh);
    const int64_t ow_n = oracle_out_size(iw, kw, sw, pw, dw);
    const int64_t mult = oc / ic;
    int64_t o;
#pragma omp parallel for schedule(dynamic, 1)
    for (o = 0; o < oc; o++) {
        const int64_t g = o / mult;
        double *wp = dwt + o * kh * kw;
        double bsum = 0.0;
        memset(wp, 0, (size_t)(kh * kw) * sizeof(double));
        for (int64_t nn = 0; nn < n; nn++) {
            const double *xp = x + (nn * ic + g) * ih * iw;
            const double *dyp = dy + (nn * oc + o) * oh_n * ow_n;
            for (int64_t oh = 0; oh < oh_n; oh++)
                for (int64_t ow = 0; ow < ow_n; ow++) {
                    const double gy = dyp[oh * ow_n + ow];
                    bsum += gy;
                    for (int64_t i = 0; i < kh; i++)
                        for (int64_t j = 0; j < kw; j++) {
                            const int64_t h = oh * sh - ph + i * dh;
                            const int64_t c = ow * sw - pw + j * dw;
                            if (h >= 0 && h < ih && c >= 0 && c < iw)
                                wp[i * kw + j] += gy * xp[h * iw + c];
                        }
                }
        }
        if (db) db[o] = bsum;
    }
}

/* y[n, b*C + c, h, w] = sum_{i, j < k} F_b[n, c, i*k + j, h, w] * x[n, c, h + (i - r)*d_b, w + (j - r)*d_b]
 * for b < nb, r = (k - 1)/2, zero outside the image.  filters[b] points to F_b. */
void oracle_dynconv_multidil_fwd(const double *x, const double *const *filters,
                                 const int32_t *dilations, int32_t nb, double *y,
                                 int64_t n, int64_t c, int64_t h, int64_t w, int64_t k)
{
    const int64_t r = (k - 1) / 2;
    int64_t task;
#pragma omp parallel for schedule(dynamic, 1)
    for (task = 0; task < (int64_t)nb * n * c; task++) {
        const int64_t br = task / (n * c), nn = (task / c) % n, ch = task % c;
        const int64_t d = dilations[br];
        const double *xp = x + (nn * c + ch) * h * w;
        const double *fp = filters[br] + (nn * c + ch) * k * k * h * w;
        double *yp = y + (nn * nb * c + br * c + ch) * h * w;
        for (int64_t py = 0; py < h; py++)
            for (int64_t px = 0; px < w; px++) {
                double acc = 0.0;
                for (int64_t i = 0; i < k; i++)
                    for (int64_t j = 0; j < k; j++) {
                        const int64_t sy = py + (i - r) * d, sx = px + (j - r) * d;
                        if (sy >= 0 && sy < h && sx >= 0 && sx < w)
                            acc += fp[(i * k + j) * h * w + py * w + px] * xp[sy * w + sx];
                    }
                yp[py * w + px] = acc;
            }
    }
}

/* Chain rule of oracle_dynconv_multidil_fwd (y is bilinear in x and the filters):
 *   dF_b[n, c, i*k + j, py, px] = dy[n, b*C + c, py, px] * x[n, c, py + (i - r)*d_b, px + (j - r)*d_b]
 *                                 (0 where that input pixel is outside the image)
 *   dx[n, c, sy, sx] += F_b[n, c, i*k + j, py, px] * dy[n, b*C + c, py, px]
 *                       for every in-image (sy, sx) = (py + (i - r)*d_b, px + (j - r)*d_b).
 * dx may be NULL; dfilters may be NULL, and so may any entry of it.  The loop nest is
 * the forward's, scattering into dx; each task owns one (n, c): its dx plane and its
 * filter-gradient planes of every branch. */
void oracle_dynconv_multidil_bwd(const double *x, const double *const *filters, const double *dy,
                                 const int32_t *dilations, int32_t nb, double *dx,
                                 double *const *dfilters, int64_t n, int64_t c, int64_t h,
                                 int64_t w, int64_t k)
{
    const int64_t r = (k - 1) / 2;
    int64_t task;
#pragma omp parallel for schedule(dynamic, 1)
    for (task = 0; task < n * c; task++) {
        const int64_t nn = task / c, ch = task % c;
        const double *xp = x + task * h * w;
        double *dxp = dx ? dx + task * h * w : NULL;
        if (dxp) memset(dxp, 0, sizeof(double) * (size_t)(h * w));
        for (int64_t br = 0; br < nb; br++) {
            const int64_t d = dilations[br];
            const double *fp = filters[br] + task * k * k * h * w;
            const double *gp = dy + (nn * nb * c + br * c + ch) * h * w;
            double *dfp = (dfilters && dfilters[br]) ? dfilters[br] + task * k * k * h * w : NULL;
            for (int64_t py = 0; py < h; py++)
                for (int64_t px = 0; px < w; px++) {
                    const double g = gp[py * w + px];
                    for (int64_t i = 0; i < k; i++)
                        for (int64_t j = 0; j < k; j++) {
                            const int64_t sy = py + (i - r) * d, sx = px + (j - r) * d;
                            const int inside = sy >= 0 && sy < h && sx >= 0 && sx < w;
                            const int64_t t = (i * k + j) * h * w + py * w + px;
                            if (dfp) dfp[t] = inside ? g * xp[sy * w + sx] : 0.0;
                            if (dxp && inside) dxp[sy * w + sx] += fp[t] * g;
                        }
                }
        }
    }
}
