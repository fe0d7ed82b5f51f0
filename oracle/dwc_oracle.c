/*
 * dwc_oracle.c -- plain CPU reference for depthwise convolution (DWC).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU library is
 * checked against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg may load it.  It shares no code, header or constant with the
 * HIP library, and the library never calls it.
 *
 * What it computes (Flash-DWC: Making Depthwise Convolution Compute-Efficient
 * on GPUs, TACO; the page's §2.1 "standard and depthwise convolution", §2.3
 * "unified channel-last layout", §5.1 "backward propagation"):
 *
 *   Layouts: X, Y, dX, dY are N x H x W x C (channel last); the filter W and
 *   its gradient dW are FH x FW x C.  IC = OC = C: each channel has its own
 *   filter (§2.1: every input patch takes an FH x FW inner product with the
 *   filter of its own channel).
 *
 *   Let Xz be X extended by zeros outside [0,IH) x [0,IW).
 *
 *   forward   Y[n,oh,ow,c]  = sum_{fh<FH} sum_{fw<FW}
 *                               Xz[n, oh*sh-ph+fh, ow*sw-pw+fw, c] * W[fh,fw,c]
 *   data grad dX[n,ih,iw,c] = sum over (oh,ow,fh,fw) with oh*sh-ph+fh = ih and
 *                               ow*sw-pw+fw = iw of dY[n,oh,ow,c] * W[fh,fw,c]
 *             (the adjoint of the forward map in X; for stride 1 this equals
 *              the forward map applied to dY with the filter turned by 180
 *              degrees, which is how §5.1 builds it)
 *   filter gr dW[fh,fw,c]   = sum_{n,oh,ow} Xz[n, oh*sh-ph+fh, ow*sw-pw+fw, c]
 *                                           * dY[n,oh,ow,c]
 *
 *   The output size is OH = floor((IH + 2*ph - FH)/sh) + 1 (same for OW); the
 *   pages print no formula, this is the usual reading.
 *
 * Every operand is float64 and every sum is accumulated in float64 (the pages
 * measure accuracy against an FP64 ground truth, §4.1 and §6.3.2).  The loops
 * are the definitions written out directly: no tiling, no reordering beyond
 * putting the channel loop innermost, which does not change any sum.
 * OpenMP splits independent outputs across threads; each output is summed by
 * one thread in a fixed order, so results do not depend on the thread count.
 *
 * Return value of every entry point: 0 on success, -1 on bad arguments.
 */
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t n, ih, iw, c;
    int64_t fh, fw;
    int64_t sh, sw, ph, pw;
    int64_t oh, ow;
} dims_t;

static int make_dims(dims_t* d, int64_t n, int64_t ih, int64_t iw, int64_t c,
                     int64_t fh, int64_t fw, int64_t sh, int64_t sw,
                     int64_t ph, int64_t pw) {
    if (n < 0 || ih < 1 || iw < 1 || c < 1 || fh < 1 || fw < 1 || sh < 1 ||
        sw < 1 || ph < 0 || pw < 0)
        return -1;
    d->n = n; d->ih = ih; d->iw = iw; d->c = c;
    d->fh = fh; d->fw = fw; d->sh = sh; d->sw = sw; d->ph = ph; d->pw = pw;
    int64_t a = ih + 2 * ph - fh, b = iw + 2 * pw - fw;
    if (a < 0 || b < 0) return -1;
    d->oh = a / sh + 1;
    d->ow = b / sw + 1;
    return 0;
}

int dwc_oracle_output_dims(int64_t ih, int64_t iw, int64_t fh, int64_t fw,
                           int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                           int64_t* oh, int64_t* ow) {
    dims_t d;
    if (make_dims(&d, 1, ih, iw, 1, fh, fw, sh, sw, ph, pw)) return -1;
    *oh = d.oh;
    *ow = d.ow;
    return 0;
}

#define XAT(d, x, n_, h_, w_, c_) \
    ((x)[(((n_) * (d)->ih + (h_)) * (d)->iw + (w_)) * (d)->c + (c_)])
#define YAT(d, y, n_, h_, w_, c_) \
    ((y)[(((n_) * (d)->oh + (h_)) * (d)->ow + (w_)) * (d)->c + (c_)])
#define WAT(d, w, fh_, fw_, c_) ((w)[((fh_) * (d)->fw + (fw_)) * (d)->c + (c_)])

/* forward: one output pixel (all channels) per iteration. */
int dwc_oracle_fwd(int64_t n, int64_t ih, int64_t iw, int64_t c, int64_t fh,
                   int64_t fw, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                   const double* x, const double* w, double* y) {
    dims_t d;
    if (make_dims(&d, n, ih, iw, c, fh, fw, sh, sw, ph, pw)) return -1;
    int64_t rows = d.n * d.oh;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t nn = r / d.oh, oh = r % d.oh;
        double* acc = (double*)malloc(sizeof(double) * (size_t)d.c);
        for (int64_t ow = 0; ow < d.ow; ++ow) {
            for (int64_t cc = 0; cc < d.c; ++cc) acc[cc] = 0.0;
            for (int64_t kh = 0; kh < d.fh; ++kh) {
                int64_t h = oh * d.sh - d.ph + kh;
                if (h < 0 || h >= d.ih) continue; /* zero padding */
                for (int64_t kw = 0; kw < d.fw; ++kw) {
                    int64_t ww = ow * d.sw - d.pw + kw;
                    if (ww < 0 || ww >= d.iw) continue;
                    const double* xp = &XAT(&d, x, nn, h, ww, 0);
                    const double* wp = &WAT(&d, w, kh, kw, 0);
                    for (int64_t cc = 0; cc < d.c; ++cc) acc[cc] += xp[cc] * wp[cc];
                }
            }
            memcpy(&YAT(&d, y, nn, oh, ow, 0), acc, sizeof(double) * (size_t)d.c);
        }
        free(acc);
    }
    return 0;
}

/* Channels per OpenMP work item in the two gradients: the widest of 128,
 * 64, 32, 16 that still leaves four work items per thread.  This only splits
 * independent outputs between threads; each output's sum runs over the same
 * terms in the same order whatever the block, so results do not depend on
 * it. */
static int64_t channel_block(int64_t outer, int64_t c) {
    int64_t want = 4 * (int64_t)omp_get_max_threads();
    int64_t b = 128;
    while (b > 16 && outer * ((c + b - 1) / b) < want) b /= 2;
    return b;
}

/* data gradient: the adjoint of the forward map, written as the scatter of
 * every (output pixel, tap) product onto the input pixel it came from.
 * A thread owns one image and one block of channels, so no two threads touch
 * the same dX element. */
int dwc_oracle_bwd_data(int64_t n, int64_t ih, int64_t iw, int64_t c,
                        int64_t fh, int64_t fw, int64_t sh, int64_t sw,
                        int64_t ph, int64_t pw, const double* dy,
                        const double* w, double* dx) {
    dims_t d;
    if (make_dims(&d, n, ih, iw, c, fh, fw, sh, sw, ph, pw)) return -1;
    const int64_t cblk = channel_block(d.n, d.c);
    int64_t nblk = (d.c + cblk - 1) / cblk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < d.n * nblk; ++t) {
        int64_t nn = t / nblk, c0 = (t % nblk) * cblk;
        int64_t c1 = c0 + cblk < d.c ? c0 + cblk : d.c;
        for (int64_t h = 0; h < d.ih; ++h)
            for (int64_t ww = 0; ww < d.iw; ++ww)
                for (int64_t cc = c0; cc < c1; ++cc) XAT(&d, dx, nn, h, ww, cc) = 0.0;
        for (int64_t oh = 0; oh < d.oh; ++oh)
            for (int64_t ow = 0; ow < d.ow; ++ow)
                for (int64_t kh = 0; kh < d.fh; ++kh) {
                    int64_t h = oh * d.sh - d.ph + kh;
                    if (h < 0 || h >= d.ih) continue;
                    for (int64_t kw = 0; kw < d.fw; ++kw) {
                        int64_t ww = ow * d.sw - d.pw + kw;
                        if (ww < 0 || ww >= d.iw) continue;
                        double* xp = &XAT(&d, dx, nn, h, ww, 0);
                        const double* gp = &YAT(&d, dy, nn, oh, ow, 0);
                        const double* wp = &WAT(&d, w, kh, kw, 0);
                        for (int64_t cc = c0; cc < c1; ++cc) xp[cc] += gp[cc] * wp[cc];
                    }
                }
    }
    return 0;
}

/* filter gradient: a thread owns one filter row and one block of channels
 * and sums over the whole batch. */
int dwc_oracle_bwd_filter(int64_t n, int64_t ih, int64_t iw, int64_t c,
                          int64_t fh, int64_t fw, int64_t sh, int64_t sw,
                          int64_t ph, int64_t pw, const double* x,
                          const double* dy, double* dw) {
    dims_t d;
    if (make_dims(&d, n, ih, iw, c, fh, fw, sh, sw, ph, pw)) return -1;
    const int64_t cblk = channel_block(d.fh, d.c);
    int64_t nblk = (d.c + cblk - 1) / cblk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < d.fh * nblk; ++t) {
        int64_t kh = t / nblk, c0 = (t % nblk) * cblk;
        int64_t c1 = c0 + cblk < d.c ? c0 + cblk : d.c;
        double* acc = &WAT(&d, dw, kh, 0, 0);
        for (int64_t kw = 0; kw < d.fw; ++kw)
            for (int64_t cc = c0; cc < c1; ++cc) acc[kw * d.c + cc] = 0.0;
        for (int64_t nn = 0; nn < d.n; ++nn)
            for (int64_t oh = 0; oh < d.oh; ++oh) {
                int64_t h = oh * d.sh - d.ph + kh;
                if (h < 0 || h >= d.ih) continue;
                for (int64_t ow = 0; ow < d.ow; ++ow)
                    for (int64_t kw = 0; kw < d.fw; ++kw) {
                        int64_t ww = ow * d.sw - d.pw + kw;
                        if (ww < 0 || ww >= d.iw) continue;
                        const double* xp = &XAT(&d, x, nn, h, ww, 0);
                        const double* gp = &YAT(&d, dy, nn, oh, ow, 0);
                        double* ap = &acc[kw * d.c];
                        for (int64_t cc = c0; cc < c1; ++cc) ap[cc] += xp[cc] * gp[cc];
                    }
            }
    }
    return 0;
}

/* ---- single-element forms, for checking sampled outputs of large runs ---- */

/* idx: k rows of (n, oh, ow, c); out[i] = Y at that index. */
int dwc_oracle_fwd_at(int64_t n, int64_t ih, int64_t iw, int64_t c, int64_t fh,
                      int64_t fw, int64_t sh, int64_t sw, int64_t ph,
                      int64_t pw, const double* x, const double* w,
                      const int64_t* idx, int64_t k, double* out) {
    dims_t d;
    if (make_dims(&d, n, ih, iw, c, fh, fw, sh, sw, ph, pw)) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < k; ++i) {
        int64_t nn = idx[4 * i], oh = idx[4 * i + 1], ow = idx[4 * i + 2],
                cc = idx[4 * i + 3];
        double s = 0.0;
        for (int64_t kh = 0; kh < d.fh; ++kh)
            for (int64_t kw = 0; kw < d.fw; ++kw) {
                int64_t h = oh * d.sh - d.ph + kh, ww = ow * d.sw - d.pw + kw;
                if (h < 0 || h >= d.ih || ww < 0 || ww >= d.iw) continue;
                s += XAT(&d, x, nn, h, ww, cc) * WAT(&d, w, kh, kw, cc);
            }
        out[i] = s;
    }
    return 0;
}

/* idx: k rows of (n, ih, iw, c); out[i] = dX there.  Gathers every
 * (oh, ow, fh, fw) whose tap lands on (ih, iw). */
int dwc_oracle_bwd_data_at(int64_t n, int64_t ih, int64_t iw, int64_t c,
                           int64_t fh, int64_t fw, int64_t sh, int64_t sw,
                           int64_t ph, int64_t pw, const double* dy,
                           const double* w, const int64_t* idx, int64_t k,
                           double* out) {
    dims_t d;
    if (make_dims(&d, n, ih, iw, c, fh, fw, sh, sw, ph, pw)) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < k; ++i) {
        int64_t nn = idx[4 * i], h = idx[4 * i + 1], ww = idx[4 * i + 2],
                cc = idx[4 * i + 3];
        double s = 0.0;
        for (int64_t kh = 0; kh < d.fh; ++kh)
            for (int64_t kw = 0; kw < d.fw; ++kw) {
                int64_t th = h + d.ph - kh, tw = ww + d.pw - kw;
                if (th < 0 || tw < 0 || th % d.sh || tw % d.sw) continue;
                int64_t oh = th / d.sh, ow = tw / d.sw;
                if (oh >= d.oh || ow >= d.ow) continue;
                s += YAT(&d, dy, nn, oh, ow, cc) * WAT(&d, w, kh, kw, cc);
            }
        out[i] = s;
    }
    return 0;
}

/* idx: k rows of (fh, fw, c); out[i] = dW there. */
int dwc_oracle_bwd_filter_at(int64_t n, int64_t ih, int64_t iw, int64_t c,
                             int64_t fh, int64_t fw, int64_t sh, int64_t sw,
                             int64_t ph, int64_t pw, const double* x,
                             const double* dy, const int64_t* idx, int64_t k,
                             double* out) {
    dims_t d;
    if (make_dims(&d, n, ih, iw, c, fh, fw, sh, sw, ph, pw)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < k; ++i) {
        int64_t kh = idx[3 * i], kw = idx[3 * i + 1], cc = idx[3 * i + 2];
        double s = 0.0;
        for (int64_t nn = 0; nn < d.n; ++nn)
            for (int64_t oh = 0; oh < d.oh; ++oh) {
                int64_t h = oh * d.sh - d.ph + kh;
                if (h < 0 || h >= d.ih) continue;
                for (int64_t ow = 0; ow < d.ow; ++ow) {
                    int64_t ww = ow * d.sw - d.pw + kw;
                    if (ww < 0 || ww >= d.iw) continue;
                    s += XAT(&d, x, nn, h, ww, cc) * YAT(&d, dy, nn, oh, ow, cc);
                }
            }
        out[i] = s;
    }
    return 0;
}
