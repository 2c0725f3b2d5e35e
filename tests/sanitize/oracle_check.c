/*
 * oracle_check.c -- runs every function of the C oracle under AddressSanitizer
 * and UndefinedBehaviorSanitizer on small seeded geometries, with each array
 * allocated at exactly its size so any read or write past it is reported.
 * Also checks the identities that tie the passes together (each backward is
 * the adjoint of the forward in one argument), so a wrong index that stays
 * inside a buffer still fails.  Exit status 0 when everything holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int64_t oracle_out_size(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d);
void oracle_set_threads(int n);
void oracle_dwconv_fwd(const double *x, const double *w, const double *b, double *y, int64_t n, int64_t ic,
                       int64_t ih, int64_t iw, int64_t oc, int64_t kh, int64_t kw, int64_t sh, int64_t sw,
                       int64_t ph, int64_t pw, int64_t dh, int64_t dw);
void oracle_dwconv_bwd_input(const double *dy, const double *w, double *dx, int64_t n, int64_t ic, int64_t ih,
                             int64_t iw, int64_t oc, int64_t kh, int64_t kw, int64_t sh, int64_t sw, int64_t ph,
                             int64_t pw, int64_t dh, int64_t dw);
void oracle_dwconv_bwd_weight(const double *x, const double *dy, double *dwt, double *db, int64_t n, int64_t ic,
                              int64_t ih, int64_t iw, int64_t oc, int64_t kh, int64_t kw, int64_t sh, int64_t sw,
                              int64_t ph, int64_t pw, int64_t dh, int64_t dw);
void oracle_dynconv_multidil_fwd(const double *x, const double *const *filters, const int32_t *dilations,
                                 int32_t nb, double *y, int64_t n, int64_t c, int64_t h, int64_t w, int64_t k);
void oracle_dynconv_multidil_bwd(const double *x, const double *const *filters, const double *dy,
                                 const int32_t *dilations, int32_t nb, double *dx, double *const *dfilters,
                                 int64_t n, int64_t c, int64_t h, int64_t w, int64_t k);

static int fails = 0;
static uint64_t state = 0x243F6A8885A308D3ull;

static uint64_t next(void)
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return state >> 11;
}
static int64_t pick(int64_t lo, int64_t hi) { return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1)); }

static double *filled(int64_t count)
{
    double *p = malloc(sizeof(double) * (size_t)count);
    for (int64_t i = 0; i < count; i++) p[i] = (double)(int64_t)(next() % 2001) / 1000.0 - 1.0;
    return p;
}

static double dot(const double *a, const double *b, int64_t count)
{
    double s = 0.0;
    for (int64_t i = 0; i < count; i++) s += a[i] * b[i];
    return s;
}

static void close_or_fail(double a, double b, double scale, const char *what, int it)
{
    if (fabs(a - b) > 1e-10 * (scale + 1.0)) {
        fprintf(stderr, "case %d: %s: %.17g vs %.17g\n", it, what, a, b);
        fails++;
    }
}

static void static_cases(int count)
{
    for (int it = 0; it < count; it++) {
        const int64_t n = pick(1, 3), ic = pick(1, 4), M = pick(1, 3), oc = ic * M;
        const int64_t kh = pick(1, 7), kw = pick(1, 7), sh = pick(1, 3), sw = pick(1, 3);
        const int64_t ph = pick(0, 4), pw = pick(0, 4), dh = pick(1, 3), dw = pick(1, 3);
        const int64_t ih = pick(1, 19), iw = pick(1, 19);
        const int64_t oh = oracle_out_size(ih, kh, sh, ph, dh), ow = oracle_out_size(iw, kw, sw, pw, dw);
        if (oh < 1 || ow < 1) continue;
        const int64_t nx = n * ic * ih * iw, ny = n * oc * oh * ow, nw = oc * kh * kw;
        double *x = filled(nx), *w = filled(nw), *b = filled(oc), *dy = filled(ny);
        double *y = malloc(sizeof(double) * (size_t)ny), *y0 = malloc(sizeof(double) * (size_t)ny);
        double *dx = malloc(sizeof(double) * (size_t)nx), *gw = malloc(sizeof(double) * (size_t)nw);
        double *gb = malloc(sizeof(double) * (size_t)oc);
        oracle_dwconv_fwd(x, w, b, y, n, ic, ih, iw, oc, kh, kw, sh, sw, ph, pw, dh, dw);
        oracle_dwconv_fwd(x, w, NULL, y0, n, ic, ih, iw, oc, kh, kw, sh, sw, ph, pw, dh, dw);
        oracle_dwconv_bwd_input(dy, w, dx, n, ic, ih, iw, oc, kh, kw, sh, sw, ph, pw, dh, dw);
        oracle_dwconv_bwd_weight(x, dy, gw, gb, n, ic, ih, iw, oc, kh, kw, sh, sw, ph, pw, dh, dw);
        oracle_dwconv_bwd_weight(x, dy, gw, NULL, n, ic, ih, iw, oc, kh, kw, sh, sw, ph, pw, dh, dw);
        /* <y0, dy> is bilinear in x and w: it equals <x, dx> and <w, gw> */
        const double ref = dot(y0, dy, ny);
        close_or_fail(ref, dot(x, dx, nx), (double)ny, "<fwd x, dy> vs <x, bwd_input dy>", it);
        close_or_fail(ref, dot(w, gw, nw), (double)ny, "<fwd x, dy> vs <w, bwd_weight>", it);
        /* the bias adds b[o] to every output of channel o, and db is the sum of dy */
        double bias_part = 0.0, ysum = 0.0, y0sum = 0.0;
        for (int64_t o = 0; o < oc; o++) bias_part += b[o] * gb[o];
        for (int64_t i = 0; i < ny; i++) {
            ysum += y[i] * dy[i];
            y0sum += y0[i] * dy[i];
        }
        close_or_fail(ysum - y0sum, bias_part, (double)ny, "bias term vs <b, db>", it);
        free(x); free(w); free(b); free(dy); free(y); free(y0); free(dx); free(gw); free(gb);
    }
}

static void dynamic_cases(int count)
{
    for (int it = 0; it < count; it++) {
        const int64_t n = pick(1, 2), c = pick(1, 3), h = pick(1, 14), w = pick(1, 14), k = 2 * pick(0, 3) + 1;
        const int32_t nb = (int32_t)pick(1, 4);
        int32_t dil[4];
        for (int b = 0; b < 4; b++) dil[b] = (int32_t)pick(1, 6);
        const int64_t nx = n * c * h * w, nf = n * c * k * k * h * w, ny = n * nb * c * h * w;
        double *x = filled(nx), *dy = filled(ny), *y = malloc(sizeof(double) * (size_t)ny);
        double *dx = malloc(sizeof(double) * (size_t)nx);
        double *f[4] = {0}, *df[4] = {0};
        for (int b = 0; b < nb; b++) {
            f[b] = filled(nf);
            df[b] = malloc(sizeof(double) * (size_t)nf);
        }
        oracle_dynconv_multidil_fwd(x, (const double *const *)f, dil, nb, y, n, c, h, w, k);
        oracle_dynconv_multidil_bwd(x, (const double *const *)f, dy, dil, nb, dx, df, n, c, h, w, k);
        oracle_dynconv_multidil_bwd(x, (const double *const *)f, dy, dil, nb, NULL, NULL, n, c, h, w, k);
        const double ref = dot(y, dy, ny);
        double fpart = 0.0;
        for (int b = 0; b < nb; b++) fpart += dot(f[b], df[b], nf);
        close_or_fail(ref, dot(x, dx, nx), (double)ny, "<dyn y, dy> vs <x, dx>", it);
        close_or_fail(ref, fpart, (double)ny, "<dyn y, dy> vs sum <F_b, dF_b>", it);
        for (int b = 0; b < nb; b++) {
            free(f[b]);
            free(df[b]);
        }
        free(x); free(dy); free(y); free(dx);
    }
}

int main(void)
{
    /* extremes of the output-size count must not overflow */
    if (oracle_out_size(1, 1, 1, 0, 1) != 1 || oracle_out_size(0, 3, 1, 1, 1) != 0 ||
        oracle_out_size(5, 3, 1, -1, 1) != 0 || oracle_out_size(1 << 20, 3, 1 << 19, 1, 1) != 2) {
        fprintf(stderr, "out_size extremes\n");
        fails++;
    }
    for (int threads = 1; threads <= 3; threads += 2) {
        oracle_set_threads(threads);
        static_cases(400);
        dynamic_cases(150);
    }
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle checks ok\n");
    return 0;
}
