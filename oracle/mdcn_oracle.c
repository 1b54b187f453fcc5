/*
 * mdcn_oracle.c -- reference evaluation of the modulated deformable 2-D
 * convolution forward pass (DCNv2), in double precision, on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, loads or calls it, and the two share no source.
 *
 * Source of the definition: the web page "TensorRT 插件解析：
 * modulatedDeformConvPlugin 可变形卷积插件的原理、参数与使用指南" (trdm.cn),
 * cited below as [plugin guide §N].  That page describes the operator as
 *   - layouts and shapes of x, offset, mask, weight, bias, output  [§二]
 *   - stride / padding / dilation / group / deformable_group       [§三]
 *   - step 1: per output position and input channel, an anchor
 *     (output coord * stride - pad), a sample point shifted by the
 *     kernel tap times dilation plus the learned offset, bilinear
 *     sampling that yields 0 outside the image, times the mask       [§五 step 1]
 *   - step 2: a per-group contraction over (C/group)*kh*kw           [§五 step 2]
 *   - step 3: broadcast add of the optional bias per output channel  [§五 step 3]
 * The page describes an im2col + GEMM pipeline; this file does NOT follow
 * that pipeline: it evaluates the definition directly, one output element
 * at a time, with a single double accumulator.
 *
 * Readings of points the page leaves open or that the text extraction
 * garbled (the extraction dropped '=', '+', '<', '>' and '&'):
 *   R1 sample point: h = ho*stride_h - pad_h + i*dil_h + dh,
 *                    w = wo*stride_w - pad_w + j*dil_w + dw.
 *   R2 a sample with h <= -1, h >= H, w <= -1 or w >= W reads 0; inside
 *      that window, each of the four bilinear corners that falls off the
 *      image reads 0.  A non-finite sample coordinate also reads 0.
 *   R3 floor() (not truncation) splits a coordinate into cell + fraction.
 *   R4 offset channels: for deformable group q and tap k = i*kw + j,
 *      channel q*2*K + 2*k holds dh and channel q*2*K + 2*k + 1 holds dw
 *      (K = kh*kw); mask channel q*K + k holds the modulation scalar.
 *   R5 deformable group q covers input channels [q*C/dg, (q+1)*C/dg).
 *   R6 group g covers input channels [g*C/G, (g+1)*C/G) and output
 *      channels [g*Co/G, (g+1)*Co/G); weight is [Co][C/G][kh][kw].
 *   R7 the mask multiplies the sampled value as given (no activation).
 *   R8 Ho, Wo are taken from the offset tensor, not from a formula.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Problem description, passed as an array of 17 int64 values in this order. */
enum {
    P_N, P_C, P_H, P_W, P_CO, P_KH, P_KW, P_HO, P_WO,
    P_SH, P_SW, P_PH, P_PW, P_DH, P_DW, P_GROUP, P_DGROUP, P_COUNT
};

/* Value of image plane X at integer pixel (y, x); 0 off the image [§五 step 1]. */
static double pixel_or_zero(const double *X, int64_t H, int64_t W, int64_t y, int64_t x)
{
    if (y < 0 || y >= H || x < 0 || x >= W)
        return 0.0;
    return X[y * W + x];
}

/* Bilinear sample of plane X at real point (h, w), zero outside (R2, R3). */
static double bilinear_zero(const double *X, int64_t H, int64_t W, double h, double w)
{
    if (!(h > -1.0 && h < (double)H && w > -1.0 && w < (double)W))
        return 0.0;
    double hf = floor(h);
    double wf = floor(w);
    int64_t y0 = (int64_t)hf;
    int64_t x0 = (int64_t)wf;
    double fy = h - hf; /* weight of the lower row */
    double fx = w - wf; /* weight of the right column */
    return (1.0 - fy) * (1.0 - fx) * pixel_or_zero(X, H, W, y0, x0)
         + (1.0 - fy) * fx         * pixel_or_zero(X, H, W, y0, x0 + 1)
         + fy         * (1.0 - fx) * pixel_or_zero(X, H, W, y0 + 1, x0)
         + fy         * fx         * pixel_or_zero(X, H, W, y0 + 1, x0 + 1);
}

double mdcn_oracle_e4m3(double v);

/* One output element out[n][co][ho][wo], straight from the definition.
 * FP8 mode (F1-F3 below) when scale is not NULL: weight then holds the
 * rounded scaled weights q(w * 2^e), each column value is rounded with
 * mdcn_oracle_e4m3, and the sum is multiplied by scale[co] = 2^-e before the
 * bias.  *abs_sum (if not NULL) gets the sum of |weight * column| (times
 * scale[co] in FP8 mode). */
static double output_element(const double *x, const double *offset, const double *mask,
                             const double *weight, const double *bias, const int64_t *p,
                             int64_t n, int64_t co, int64_t ho, int64_t wo,
                             const double *scale, double *abs_sum)
{
    const int64_t C = p[P_C], H = p[P_H], W = p[P_W], Co = p[P_CO];
    const int64_t kh = p[P_KH], kw = p[P_KW], Ho = p[P_HO], Wo = p[P_WO];
    const int64_t G = p[P_GROUP], DG = p[P_DGROUP];
    const int64_t K = kh * kw;
    const int64_t Cg = C / G;        /* input channels per group    (R6) */
    const int64_t Mg = Co / G;       /* output channels per group   (R6) */
    const int64_t Cdg = C / DG;      /* input channels per offset group (R5) */
    const int64_t g = co / Mg;       /* the group this output channel is in */
    const int64_t HoWo = Ho * Wo;
    const int64_t pix = ho * Wo + wo;

    double acc = 0.0, sa = 0.0;
    for (int64_t cl = 0; cl < Cg; ++cl) {
        const int64_t c = g * Cg + cl;
        const int64_t q = c / Cdg;
        const double *plane = x + (n * C + c) * H * W;
        for (int64_t i = 0; i < kh; ++i) {
            for (int64_t j = 0; j < kw; ++j) {
                const int64_t k = i * kw + j;
                const int64_t off_h_ch = n * 2 * DG * K + q * 2 * K + 2 * k;   /* R4 */
                const int64_t off_w_ch = off_h_ch + 1;
                const int64_t mask_ch = n * DG * K + q * K + k;
                const double dh = offset[off_h_ch * HoWo + pix];
                const double dw = offset[off_w_ch * HoWo + pix];
                const double m = mask[mask_ch * HoWo + pix];
                const double h = (double)(ho * p[P_SH] - p[P_PH] + i * p[P_DH]) + dh;  /* R1 */
                const double w = (double)(wo * p[P_SW] - p[P_PW] + j * p[P_DW]) + dw;
                const double val = bilinear_zero(plane, H, W, h, w) * m;            /* R7 */
                const double col = scale ? mdcn_oracle_e4m3(val) : val;               /* F1 */
                const double prod = weight[((co * Cg + cl) * kh + i) * kw + j] * col;
                acc += prod;
                sa += fabs(prod);
            }
        }
    }
    if (abs_sum)
        *abs_sum = scale ? sa * scale[co] : sa;
    if (scale)
        acc *= scale[co];                                                         /* F3 */
    if (bias)
        acc += bias[co];
    return acc;
}

/* Threads the OpenMP runtime will use for the calls below. */
int mdcn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets that thread count (n > 0); for timing the oracle on one thread.  The
 * results do not depend on it: every output element is one thread's
 * sequential sum. */
void mdcn_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Full forward: out is [N][Co][Ho][Wo].  bias may be NULL.
 * Returns 0, or -1 if the description is not one this definition covers. */
int mdcn_oracle_forward(const double *x, const double *offset, const double *mask,
                        const double *weight, const double *bias, const int64_t *p,
                        double *out)
{
    const int64_t N = p[P_N], Co = p[P_CO], Ho = p[P_HO], Wo = p[P_WO];
    if (p[P_GROUP] <= 0 || p[P_DGROUP] <= 0 || p[P_C] % p[P_GROUP] || Co % p[P_GROUP] ||
        p[P_C] % p[P_DGROUP])
        return -1;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t co = 0; co < Co; ++co)
            for (int64_t ho = 0; ho < Ho; ++ho)
                for (int64_t wo = 0; wo < Wo; ++wo)
                    out[((n * Co + co) * Ho + ho) * Wo + wo] =
                        output_element(x, offset, mask, weight, bias, p, n, co, ho, wo,
                                       NULL, NULL);
    return 0;
}

/* Selected outputs: idx holds npts flat indices into [N][Co][Ho][Wo];
 * out[t] receives the element at idx[t]. */
int mdcn_oracle_points(const double *x, const double *offset, const double *mask,
                       const double *weight, const double *bias, const int64_t *p,
                       int64_t npts, const int64_t *idx, double *out)
{
    const int64_t N = p[P_N], Co = p[P_CO], Ho = p[P_HO], Wo = p[P_WO];
    if (p[P_GROUP] <= 0 || p[P_DGROUP] <= 0 || p[P_C] % p[P_GROUP] || Co % p[P_GROUP] ||
        p[P_C] % p[P_DGROUP])
        return -1;
    const int64_t total = N * Co * Ho * Wo;
    for (int64_t t = 0; t < npts; ++t)
        if (idx[t] < 0 || idx[t] >= total)
            return -1;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < npts; ++t) {
        int64_t r = idx[t];
        const int64_t wo = r % Wo; r /= Wo;
        const int64_t ho = r % Ho; r /= Ho;
        const int64_t co = r % Co; r /= Co;
        const int64_t n = r;
        out[t] = output_element(x, offset, mask, weight, bias, p, n, co, ho, wo, NULL, NULL);
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * FP8 compute mode: the same operator with both contraction operands held
 * as OCP FP8 E4M3 numbers and the products summed in high precision.
 *
 * The pages fix no FP8 arithmetic (the plugin accepts fp32 and fp16 only,
 * [plugin guide §四]); this mode is this library's extension, and its
 * definition here is:
 *   F1 a column value (the modulated bilinear sample, computed exactly) is
 *      rounded to the nearest E4M3 number, ties to the even code, after
 *      clamping to [-448, 448] (saturation; NaN stays NaN);
 *   F2 each output channel's weight row is scaled by 2^e, e the largest
 *      integer with max|w_row| * 2^e <= 448 (e = 0 for an all-zero row;
 *      e clamped to [-126, 126]), then rounded as in F1;
 *   F3 out = 2^-e * sum(q(w) * q(column)) + bias.
 * E4M3 (OCP 8-bit floating point, E4M3 variant): sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; the
 * all-ones exponent with mantissa 7 is NaN; no infinities; the largest
 * finite value is 1.75 * 2^8 = 448.
 * ------------------------------------------------------------------------ */

/* F1: nearest E4M3 value, ties to even, saturating at +-448. */
double mdcn_oracle_e4m3(double v)
{
    if (isnan(v))
        return v;
    const double a = fabs(v);
    if (a >= 448.0)
        return copysign(448.0, v);
    /* spacing of E4M3 numbers around a: 2^-9 below the smallest normal
     * 2^-6, else 2^(floor(log2 a) - 3) (3 mantissa bits) */
    double step;
    if (a < 0x1p-6) {
        step = 0x1p-9;
    } else {
        int ex;
        frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
        step = ldexp(1.0, ex - 1 - 3);
    }
    /* a / step is exact (a power-of-two scaling); nearbyint rounds half to
     * even in the default rounding mode, and an even multiple of the step is
     * an even mantissa (also where the rounding carries into the next binade) */
    return copysign(nearbyint(a / step) * step, v);
}

/* F2: the exponent e of one weight row of n values. */
int mdcn_oracle_fp8_row_exponent(const double *row, int64_t n)
{
    double mx = 0.0;
    for (int64_t t = 0; t < n; ++t)
        if (fabs(row[t]) > mx)
            mx = fabs(row[t]);
    if (!(mx > 0.0) || isinf(mx))
        return 0;
    /* mx = f * 2^ex with f in [0.5, 1); 448 = 0.875 * 2^9, so
     * mx * 2^e <= 448 holds for e = 9 - ex when f <= 0.875, else 8 - ex */
    int ex;
    const double f = frexp(mx, &ex);
    int e = (f <= 0.875) ? 9 - ex : 8 - ex;
    if (e > 126)
        e = 126;
    if (e < -126)
        e = -126;
    return e;
}

/* F2 for every row: qw (Co*Cg*K values) and scale (Co values). */
static void quantize_weight(const double *weight, const int64_t *p, double *qw, double *scale)
{
    const int64_t Co = p[P_CO], Cg = p[P_C] / p[P_GROUP], K = p[P_KH] * p[P_KW];
    for (int64_t co = 0; co < Co; ++co) {
        const double *row = weight + co * Cg * K;
        const int e = mdcn_oracle_fp8_row_exponent(row, Cg * K);
        scale[co] = ldexp(1.0, -e);
        for (int64_t t = 0; t < Cg * K; ++t)
            qw[co * Cg * K + t] = mdcn_oracle_e4m3(ldexp(row[t], e));
    }
}

/* Selected outputs in the FP8 mode; qw and scale are caller-provided scratch
 * of Co*Cg*K and Co doubles; abs_sum (may be NULL) gets one value per point. */
int mdcn_oracle_points_fp8(const double *x, const double *offset, const double *mask,
                           const double *weight, const double *bias, const int64_t *p,
                           int64_t npts, const int64_t *idx, double *qw, double *scale,
                           double *out, double *abs_sum)
{
    const int64_t N = p[P_N], Co = p[P_CO], Ho = p[P_HO], Wo = p[P_WO];
    if (p[P_GROUP] <= 0 || p[P_DGROUP] <= 0 || p[P_C] % p[P_GROUP] || Co % p[P_GROUP] ||
        p[P_C] % p[P_DGROUP])
        return -1;
    const int64_t total = N * Co * Ho * Wo;
    for (int64_t t = 0; t < npts; ++t)
        if (idx[t] < 0 || idx[t] >= total)
            return -1;
    quantize_weight(weight, p, qw, scale);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < npts; ++t) {
        int64_t r = idx[t];
        const int64_t wo = r % Wo; r /= Wo;
        const int64_t ho = r % Ho; r /= Ho;
        const int64_t co = r % Co; r /= Co;
        const int64_t n = r;
        out[t] = output_element(x, offset, mask, qw, bias, p, n, co, ho, wo, scale,
                                abs_sum ? abs_sum + t : NULL);
    }
    return 0;
}

/* F1 applied to n values (for the tests of the quantizer itself). */
void mdcn_oracle_e4m3_array(const double *v, int64_t n, double *out)
{
    for (int64_t t = 0; t < n; ++t)
        out[t] = mdcn_oracle_e4m3(v[t]);
}

/* ------------------------------------------------------------------------
 * Backward pass: the gradients of a scalar loss L with respect to x, offset,
 * mask, weight and bias, given g = dL/dout ([N][Co][Ho][Wo]).  The pages
 * describe only the forward; these are the derivatives of its definition
 * above (R1-R8), read as:
 *   B1 the bilinear sample is differentiated on the cell that floor()
 *      selects: with h = y0 + a, w = x0 + b (a, b in [0, 1)),
 *      d sample/d h = (1-b)(v10 - v00) + b(v11 - v01),
 *      d sample/d w = (1-a)(v01 - v00) + a(v11 - v10),
 *      corners off the image counting as 0 (at integer h or w this is the
 *      derivative from above);
 *   B2 a sample outside the open window (h <= -1, h >= H, w <= -1, w >= W,
 *      or not finite) is 0 with zero derivatives;
 *   B3 the mask, weight and bias enter linearly, so their gradients are the
 *      sums of g times what multiplies them; x enters through the four
 *      corner weights times mask times weight.
 * ------------------------------------------------------------------------ */

/* Bilinear sample of plane X at (h, w) and its two partial derivatives
 * (B1, B2); dh, dw receive the derivatives. */
static double bilinear_grad(const double *X, int64_t H, int64_t W, double h, double w,
                            double *dh, double *dw)
{
    *dh = 0.0;
    *dw = 0.0;
    if (!(h > -1.0 && h < (double)H && w > -1.0 && w < (double)W))
        return 0.0;
    const double hf = floor(h), wf = floor(w);
    const int64_t y0 = (int64_t)hf, x0 = (int64_t)wf;
    const double a = h - hf, b = w - wf;
    const double v00 = pixel_or_zero(X, H, W, y0, x0);
    const double v01 = pixel_or_zero(X, H, W, y0, x0 + 1);
    const double v10 = pixel_or_zero(X, H, W, y0 + 1, x0);
    const double v11 = pixel_or_zero(X, H, W, y0 + 1, x0 + 1);
    *dh = (1.0 - b) * (v10 - v00) + b * (v11 - v01);
    *dw = (1.0 - a) * (v01 - v00) + a * (v11 - v10);
    return (1.0 - a) * (1.0 - b) * v00 + (1.0 - a) * b * v01 + a * (1.0 - b) * v10 + a * b * v11;
}

/* Adds s times the four corner weights of the sample at (h, w) to the
 * corners of plane GX that lie on the image (B1, B2, B3). */
static void scatter_corners(double *GX, int64_t H, int64_t W, double h, double w, double s)
{
    if (!(h > -1.0 && h < (double)H && w > -1.0 && w < (double)W))
        return;
    const double hf = floor(h), wf = floor(w);
    const int64_t y0 = (int64_t)hf, x0 = (int64_t)wf;
    const double a = h - hf, b = w - wf;
    const double cw[4] = {(1.0 - a) * (1.0 - b), (1.0 - a) * b, a * (1.0 - b), a * b};
    const int64_t cy[4] = {y0, y0, y0 + 1, y0 + 1}, cx[4] = {x0, x0 + 1, x0, x0 + 1};
    for (int t = 0; t < 4; ++t)
        if (cy[t] >= 0 && cy[t] < H && cx[t] >= 0 && cx[t] < W)
            GX[cy[t] * W + cx[t]] += s * cw[t];
}

/* All five gradients.  gx, goff, gmask, gw have the shapes of x, offset,
 * mask, weight; gb has Co values (may be NULL).  Sequential (the scatter
 * into gx has no fixed owner).  Returns 0, or -1 for an unsupported
 * description. */
int mdcn_oracle_backward(const double *x, const double *offset, const double *mask,
                         const double *weight, const double *grad_out, const int64_t *p,
                         double *gx, double *goff, double *gmask, double *gw, double *gb)
{
    const int64_t N = p[P_N], C = p[P_C], H = p[P_H], W = p[P_W], Co = p[P_CO];
    const int64_t kh = p[P_KH], kw = p[P_KW], Ho = p[P_HO], Wo = p[P_WO];
    const int64_t G = p[P_GROUP], DG = p[P_DGROUP];
    if (G <= 0 || DG <= 0 || C % G || Co % G || C % DG)
        return -1;
    const int64_t K = kh * kw, Cg = C / G, Mg = Co / G, Cdg = C / DG, HoWo = Ho * Wo;
    for (int64_t t = 0; t < N * C * H * W; ++t) gx[t] = 0.0;
    for (int64_t t = 0; t < N * 2 * DG * K * HoWo; ++t) goff[t] = 0.0;
    for (int64_t t = 0; t < N * DG * K * HoWo; ++t) gmask[t] = 0.0;
    for (int64_t t = 0; t < Co * Cg * K; ++t) gw[t] = 0.0;
    if (gb)
        for (int64_t t = 0; t < Co; ++t) gb[t] = 0.0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t co = 0; co < Co; ++co)
            for (int64_t ho = 0; ho < Ho; ++ho)
                for (int64_t wo = 0; wo < Wo; ++wo) {
                    const int64_t pix = ho * Wo + wo;
                    const double g = grad_out[(n * Co + co) * HoWo + pix];
                    if (gb)
                        gb[co] += g;
                    const int64_t grp = co / Mg;
                    for (int64_t cl = 0; cl < Cg; ++cl) {
                        const int64_t c = grp * Cg + cl;
                        const int64_t q = c / Cdg;
                        const double *plane = x + (n * C + c) * H * W;
                        for (int64_t i = 0; i < kh; ++i)
                            for (int64_t j = 0; j < kw; ++j) {
                                const int64_t k = i * kw + j;
                                const int64_t oh = (n * 2 * DG * K + q * 2 * K + 2 * k) * HoWo + pix;
                                const int64_t ow = oh + HoWo;
                                const int64_t mi = (n * DG * K + q * K + k) * HoWo + pix;
                                const double m = mask[mi];
                                const double h = (double)(ho * p[P_SH] - p[P_PH] + i * p[P_DH]) + offset[oh];
                                const double w = (double)(wo * p[P_SW] - p[P_PW] + j * p[P_DW]) + offset[ow];
                                const int64_t wi = ((co * Cg + cl) * kh + i) * kw + j;
                                double dh, dw;
                                const double v = bilinear_grad(plane, H, W, h, w, &dh, &dw);
                                const double gwt = g * weight[wi];       /* dL/d(modulated sample) */
                                gw[wi] += g * v * m;
                                gmask[mi] += gwt * v;
                                goff[oh] += gwt * m * dh;
                                goff[ow] += gwt * m * dw;
                                scatter_corners(gx + (n * C + c) * H * W, H, W, h, w, gwt * m);
                            }
                    }
                }
    return 0;
}
