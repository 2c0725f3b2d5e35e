// dw_internal.hpp -- host-side plan structures and kernel launchers shared by
// the C ABI (dw_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dw {

// Validated geometry in 32-bit ints (every tensor is below 2^31 elements).
struct Geo {
    int n, ic, ih, iw;
    int oc, kh, kw;
    int sh, sw, ph, pw, dh, dw;
    int oh, ow, mult;
};

// Largest LDS a single workgroup may use for staged tiles (bytes).
constexpr int kLdsCap = 64 * 1024;
// Threads per workgroup of every kernel in this library.
constexpr int kThreads = 256;

// Status codes returned by launchers (subset of the public enum).
constexpr int kOk = 0;
constexpr int kErrHip = -8;
constexpr int kErrUnsupported = -10;

int launch_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype,
               hipStream_t s);
int launch_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype,
                     hipStream_t s);
// Bytes of workspace launch_bwd_weight needs; -1 when the geometry is unsupported.
int64_t bwd_weight_workspace(const Geo &g, int dtype);
int64_t bwd_weight_workspace_selected(const Geo &g, int dtype);
int launch_bwd_weight(const Geo &g, const void *x, const void *dy, void *dwt, void *db,
                      void *ws, int dtype, hipStream_t s);
// Dynamic filter forward: branch b, channel ch is written to plane
// (n, yoff + b*c + ch) of an output with ych channels.
int launch_dynconv(const void *x, const void *const *filters, const int32_t *dil, int nb, void *y, int ych,
                   int yoff, int n, int c, int h, int w, int k, int dtype, hipStream_t s);
// Backward of the dynamic filter (dw_dynbwd.hip): dx when non-NULL, dF_b for
// every non-NULL dfilters[b] (dfilters itself may be NULL); dy is read at
// plane (n, dyoff + b*c + ch) of a gradient with dych channels.
int launch_dynconv_bwd(const void *x, const void *const *filters, const void *dy, int dych, int dyoff,
                       const int32_t *dil, int nb, void *dx, void *const *dfilters, int n, int c, int h, int w,
                       int k, int dtype, hipStream_t s);

// Streaming kernels for 3x3 / pad 1 / dilation 1 / stride 1-2 / multiplier <= 2
// (dw_rowwalk.hip).  The launchers return kErrUnsupported when the row is
// wider than one wave of 16-byte strips; callers then use the band kernels.
bool rowwalk_applicable(const Geo &g, int pass);
bool rowwalk_fits(const Geo &g, int dtype, int pass);  // pass: 0 fwd, 1 grad-input, 2 grad-weight
int rowwalk_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s);
int rowwalk_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s);
int rowwalk_bwd_weight_chunks(const Geo &g, int dtype);
int rowwalk_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s);

// Small planes over groups of adjacent channels, one lane per (channel, row):
// grad-weight (dw_small.hip; small_fits is true only for pass 2 geometries it
// handles), forward (dw_small_fwd.hip) and grad-input (dw_small_bwdin.hip).
bool small_fits(const Geo &g, int dtype, int pass);
int small_bwd_weight_chunks(const Geo &g, int dtype);
int small_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s);
bool small_fwd_fits(const Geo &g, int dtype);
int small_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s);
bool small_bwd_input_fits(const Geo &g, int dtype);
int small_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s);

// Large-kernel (k = 7, 13, 31; stride 1, dilation 1) register-tile kernels
// (dw_largek.hip).  pass: 0 forward, 1 grad-input.
bool largek_fits(const Geo &g, int pass);
int largek_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s);
int largek_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s);
bool largek_bwdw_fits(const Geo &g);
int largek_bwd_weight_chunks(const Geo &g);
int largek_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s);

// Large kernels (k = 7, 13, 31; stride 1, dilation 1) with 16-bit I/O on the
// matrix cores, planes of at most 64 x 64 outputs (dw_largek_mfma.hip).
// pass: 0 forward, 1 grad-input.
bool largek_mfma_fits(const Geo &g, int pass, int dtype);
int largek_mfma_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s);
int largek_mfma_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s);
// The same on 16 x 16 output tiles (dw_largek_mfma.hip).
bool largek_mfma16_fits(const Geo &g, int pass, int dtype);
int largek_mfma16_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s);
int largek_mfma16_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s);
// 16-bit k = 31 forward / grad-input streaming input rows through rotating
// filter rows on the matrix cores (dw_largek_roll16.hip); any plane size.
bool largek_roll16_fits(const Geo &g, int pass, int dtype);
int largek_roll16_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s);
int largek_roll16_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s);
// fp32 31 x 31 forward / grad-input streaming input rows through rotating
// filter rows on the matrix cores (dw_largek_rollf32.hip); any plane size.
bool largek_rollf32_fits(const Geo &g, int pass, int dtype);
int largek_rollf32_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, hipStream_t s);
int largek_rollf32_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t s);
// 16-bit k = 13 / 31 grad-weight streaming input rows, the dy rows moving
// through the filter-row slots (dw_largek_wroll16.hip); output rows <= 64.
bool largek_wroll16_fits(const Geo &g, int dtype);
int largek_wroll16_chunks(const Geo &g);
int largek_wroll16(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s);
// Grad-weight pass 1 of the same family (k = 13, 31; multiplier 1; dy rows <= 64):
// workspace [ic][chunks][k*k + 1].
bool largek_mfma_bwdw_fits(const Geo &g, int dtype);
int largek_mfma_bwd_weight_chunks(const Geo &g);
int largek_mfma_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s);
// The same on 16 x 16 tiles for k = 7, 13 (dw_largek_mfma.hip): workspace
// [ic][chunks][k*k + 1], chunks as largek_mfma_bwd_weight_chunks.
bool largek_mfma_bwdw16_fits(const Geo &g, int dtype);
int largek_mfma_bwd_weight16(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s);

// Forward and grad-input of the 31 x 31 filter with fp32 I/O on the matrix
// cores (dw_largek_fwd32.hip).  pass: 0 forward, 1 grad-input.
bool largek_fwd32_fits(const Geo &g, int pass, int dtype);
bool largek_fwd32_preferred(const Geo &g, int pass);
int largek_fwd32(const Geo &g, const void *x, const void *w, const void *b, void *y, hipStream_t s);
int largek_bwd_input32(const Geo &g, const void *dy, const void *w, void *dx, hipStream_t s);

// Grad-weight pass 1 of the 31 x 31 filter with fp32 I/O on the matrix cores
// (dw_largek_wgrad32.hip): workspace [ic][chunks][k*k + 1].
bool largek_wgrad32_fits(const Geo &g, int dtype);
int largek_wgrad32_chunks(const Geo &g);
int largek_wgrad32(const Geo &g, const void *x, const void *dy, void *ws, hipStream_t s);
// Grad-weight of 13 x 13 filters on the matrix cores with 16 x 16 tiles, any
// dtype (dw_largek_wgrad16.hip): workspace [ic][chunks][k*k + 1].
bool largek_wgrad16_fits(const Geo &g, int dtype);
int largek_wgrad16_chunks(const Geo &g);
int largek_wgrad16(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s);
// Grad-weight of 7 x 7 filters as a register row stream, any dtype
// (dw_largek_wgrad7.hip): workspace [ic][chunks][k*k + 1].
bool stream7_bwdw_fits(const Geo &g);
int stream7_bwdw_chunks(const Geo &g);
int stream7_bwdw(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s);

// Stride 2, dilation 2, pad k-1 (k = 3, 5) as stride-1 passes on the even grid (dw_decim.hip).
bool decim_fits(const Geo &g, int pass);
int decim_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s);
int decim_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s);
int decim_bwd_weight_chunks(const Geo &g);
int decim_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s);

// Direct kernels for every valid geometry (dw_direct.hip): one thread per
// output element, operands from global memory, no LDS size limit.  Grad-weight
// pass 1 writes the chunk partials [ic][chunks][M*(k*k + 1)].
int direct_fwd(const Geo &g, const void *x, const void *w, const void *b, void *y, int dtype, hipStream_t s);
int direct_bwd_input(const Geo &g, const void *dy, const void *w, void *dx, int dtype, hipStream_t s);
int direct_bwd_weight_chunks(const Geo &g);
int direct_bwd_weight(const Geo &g, const void *x, const void *dy, void *ws, int dtype, hipStream_t s);
int direct_dynconv(const void *x, const void *const *filters, const int32_t *dil, int nb, void *y, int ych, int yoff,
                   int n, int c, int h, int w, int k, int dtype, hipStream_t s);
int direct_dynconv_bwd(const void *x, const void *const *filters, const void *dy, int dych, int dyoff,
                       const int32_t *dil, int nb, void *dx, void *const *dfilters, int n, int c, int h, int w, int k,
                       int dtype, hipStream_t s);

// Name of the kernel family each pass would launch for this geometry.
const char *fwd_algo_name(const Geo &g, int dtype);
const char *bwd_input_algo_name(const Geo &g, int dtype);
const char *bwd_weight_algo_name(const Geo &g, int dtype);

// Every family of a pass, by index: its name and whether it can run a geometry.
int fwd_algo_count();
const char *fwd_algo_name_of(int algo);
bool fwd_algo_feasible(int algo, const Geo &g, int dtype);
int bwd_input_algo_count();
const char *bwd_input_algo_name_of(int algo);
bool bwd_input_algo_feasible(int algo, const Geo &g, int dtype);
int bwd_weight_algo_count();
const char *bwd_weight_algo_name_of(int algo);
bool bwd_weight_algo_feasible(int algo, const Geo &g, int dtype);

// Selection table (dw_tune.hip): the family recorded for (pass, geometry,
// dtype), or -1; set_tuned_algo records one (algo < 0 removes the entry).
int tuned_algo(int pass, const Geo &g, int dtype);
void set_tuned_algo(int pass, const Geo &g, int dtype, int algo);

// Shape checks the launchers need beyond argument validation (LDS fit).
bool fwd_supported(const Geo &g, int dtype);
bool bwd_input_supported(const Geo &g, int dtype);
bool dynconv_supported(int h, int w, int k, int maxdil, int dtype);
bool dynconv_bwd_supported(int h, int w, int k, int maxdil, int dtype);

}  // namespace dw
