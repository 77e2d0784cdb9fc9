/*
 * dc1d_oracle.c -- plain, slow CPU oracle for the 1D deformable convolution
 * forward, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the bench's
 * CPU-baseline leg have an independent answer to compare the GPU kernels
 * against.  It shares no header, helper, table or constant with the HIP
 * library, and includes nothing from it.
 *
 * What it computes (restated from the pages, cited by page and section):
 *
 *  - Output length, from the conv1d operator page ("conv1d", section
 *    Shape and the closing paragraph of Axis convention):
 *        L_out = floor((L_in + 2p - d(K-1) - 1) / s + 1).
 *  - Plain conv1d, same page, section Description: a cross-correlation,
 *        out[b,co,l] = bias[co] + sum_{ci,k} w[co,ci,k] * x[b,ci, l*s - p + k*d].
 *  - The deformable form, from the dilated/deformable convolution article
 *    (section Deformable Convolution, the y(p0) formula): each tap samples
 *    the input at its regular grid position plus a learned offset, and the
 *    two-stage workflow of that article (Step 2 deformable sampling, then
 *    Step 3 weighted summation) is followed literally: stage 1 builds the
 *    sampled tensor, stage 2 contracts it with the weight.
 *  - 1D sampling is linear interpolation between the two neighbouring
 *    integer positions (dc1d page, section Demo notebook: a fractional
 *    offset interpolates linearly; an integer offset is an exact shift).
 *    The weights are the 1D analogue of the article's bilinear weights:
 *    the integer part picks the left neighbour, the fractional part f
 *    weighs the right one by f and the left one by 1 - f.
 *  - Positions outside [0, L_in) read zero (the torchvision issue page's
 *    printed demo: samples shifted off the edge come back as 0).
 *  - Offsets have shape [B, G, L_out, K] with G (offset groups) dividing
 *    C_in (dc1d page, section Usage / DeformConv1d); channel ci uses
 *    offset group ci / (C_in / G) (reading: contiguous channel blocks, as
 *    the torchvision demo divides its input channels into groups).
 *  - The optional modulation mask has the offsets' shape and multiplies
 *    each sampled value as given (dc1d page, section Modulation (DCNv2)).
 *  - groups split C_in and C_out into contiguous independent blocks; the
 *    weight is [C_out, C_in/groups, K] (conv1d page, Arguments and Axis
 *    convention).
 *
 * Arithmetic: every input value arrives already converted exactly to
 * double; all arithmetic is double; the contraction sums over
 * (ci_local, k) in ascending order and then adds the bias.  Build with
 * -O2 -ffp-contract=off and without fast-math so the compiler neither
 * fuses nor reassociates.
 *
 * Non-finite inputs are outside the contract; the entry points reject them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Status codes of this file (independent of the GPU library's codes). */
#define OR_OK 0
#define OR_BAD_ARG 1
#define OR_NONFINITE 2
#define OR_NOMEM 3

/* conv1d output length; -1 when the arguments are out of range or the
 * result would not be positive. */
int64_t oracle_output_length(int64_t L_in, int64_t K, int64_t s, int64_t p, int64_t d)
{
    if (L_in < 0 || K < 1 || s < 1 || p < 0 || d < 1)
        return -1;
    int64_t num = L_in + 2 * p - d * (K - 1) - 1;
    if (num < 0)
        return -1; /* floor(num/s) + 1 <= 0 */
    return num / s + 1;
}

/* Zero-extended input: x~(i) = x[i] inside [0, L), 0 outside. */
static double x_ext(const double *row, int64_t L, int64_t i)
{
    return (i >= 0 && i < L) ? row[i] : 0.0;
}

/* Split a sampling position base + o into its integer left neighbour i0 and
 * fractional weight f in [0, 1).  The integer part of the grid term is
 * exact, so only the offset is floored. */
static void split_position(int64_t base, double o, int64_t *i0, double *f)
{
    double fl = floor(o);
    *i0 = base + (int64_t)fl;
    *f = o - fl;
}

/* One linearly interpolated, optionally modulated sample. */
static double sample(const double *row, int64_t L_in, int64_t base, double o, const double *m)
{
    int64_t i0;
    double f;
    split_position(base, o, &i0, &f);
    double v = (1.0 - f) * x_ext(row, L_in, i0) + f * x_ext(row, L_in, i0 + 1);
    return m ? v * (*m) : v;
}

static int all_finite(const double *a, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(a[i]))
            return 0;
    return 1;
}

typedef struct {
    int64_t B, C_in, L_in, C_out, K, s, p, d, groups, G, L_out;
} shape_t;

static int check_shape(shape_t *sh)
{
    if (sh->B < 0 || sh->C_in < 1 || sh->C_out < 1 || sh->groups < 1 || sh->G < 1)
        return OR_BAD_ARG;
    if (sh->C_in % sh->groups || sh->C_out % sh->groups || sh->C_in % sh->G)
        return OR_BAD_ARG;
    sh->L_out = oracle_output_length(sh->L_in, sh->K, sh->s, sh->p, sh->d);
    if (sh->L_out < 1)
        return OR_BAD_ARG;
    return OR_OK;
}

/*
 * Sampling positions only: for every (b, g, l, k) the left neighbour i0,
 * the fraction f and the two validity bits (bit0: 0 <= i0 < L_in,
 * bit1: 0 <= i0 + 1 < L_in).  offsets is [B, G, L_out, K].
 */
int oracle_positions(const double *offsets, int64_t B, int64_t G, int64_t L_in, int64_t K,
                     int64_t s, int64_t p, int64_t d, int64_t *i0_out, double *f_out,
                     uint8_t *valid_out)
{
    int64_t L_out = oracle_output_length(L_in, K, s, p, d);
    if (L_out < 1 || B < 0 || G < 1)
        return OR_BAD_ARG;
    int64_t n = B * G * L_out * K;
    if (!all_finite(offsets, n))
        return OR_NONFINITE;
    for (int64_t bg = 0; bg < B * G; ++bg)
        for (int64_t l = 0; l < L_out; ++l)
            for (int64_t k = 0; k < K; ++k) {
                int64_t idx = (bg * L_out + l) * K + k;
                int64_t base = l * s - p + k * d;
                int64_t i0;
                double f;
                split_position(base, offsets[idx], &i0, &f);
                i0_out[idx] = i0;
                f_out[idx] = f;
                valid_out[idx] = (uint8_t)((i0 >= 0 && i0 < L_in ? 1 : 0) |
                                           (i0 + 1 >= 0 && i0 + 1 < L_in ? 2 : 0));
            }
    return OR_OK;
}

/*
 * Full forward, two stages.
 *   x       [B, C_in, L_in]
 *   offsets [B, G, L_out, K]
 *   mask    [B, G, L_out, K] or NULL
 *   weight  [C_out, C_in/groups, K]
 *   bias    [C_out] or NULL
 *   out     [B, C_out, L_out]
 */
int oracle_forward(const double *x, const double *offsets, const double *mask,
                   const double *weight, const double *bias, int64_t B, int64_t C_in,
                   int64_t L_in, int64_t C_out, int64_t K, int64_t s, int64_t p, int64_t d,
                   int64_t groups, int64_t G, double *out)
{
    shape_t sh = {B, C_in, L_in, C_out, K, s, p, d, groups, G, 0};
    int st = check_shape(&sh);
    if (st)
        return st;
    const int64_t L_out = sh.L_out;
    const int64_t cpg = C_in / groups, opg = C_out / groups, cpo = C_in / G;
    const int64_t n_off = B * G * L_out * K;
    if (!all_finite(x, B * C_in * L_in) || !all_finite(offsets, n_off) ||
        (mask && !all_finite(mask, n_off)) || !all_finite(weight, C_out * cpg * K) ||
        (bias && !all_finite(bias, C_out)))
        return OR_NONFINITE;
    if (B == 0)
        return OR_OK;

    /* Stage 1: the sampled tensor S[b, ci, k, l]. */
    double *S = (double *)malloc(sizeof(double) * (size_t)(B * C_in * K * L_out));
    if (!S)
        return OR_NOMEM;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t ci = 0; ci < C_in; ++ci) {
            const int64_t g = ci / cpo;
            const double *row = x + (b * C_in + ci) * L_in;
            for (int64_t k = 0; k < K; ++k)
                for (int64_t l = 0; l < L_out; ++l) {
                    const int64_t oi = ((b * G + g) * L_out + l) * K + k;
                    S[((b * C_in + ci) * K + k) * L_out + l] =
                        sample(row, L_in, l * s - p + k * d, offsets[oi], mask ? mask + oi : NULL);
                }
        }

    /* Stage 2: weighted sum over the group's input channels and taps. */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t co = 0; co < C_out; ++co) {
            const int64_t grp = co / opg;
            for (int64_t l = 0; l < L_out; ++l) {
                double acc = 0.0;
                for (int64_t cl = 0; cl < cpg; ++cl)
                    for (int64_t k = 0; k < K; ++k)
                        acc += weight[(co * cpg + cl) * K + k] *
                               S[((b * C_in + grp * cpg + cl) * K + k) * L_out + l];
                out[(b * C_out + co) * L_out + l] = acc + (bias ? bias[co] : 0.0);
            }
        }
    free(S);
    return OR_OK;
}

/*
 * The same forward evaluated only at selected outputs, for shapes too big
 * to evaluate whole.  points holds npts triples (b, co, l); the arithmetic
 * per output is exactly that of oracle_forward (same sample(), same
 * ascending (ci_local, k) order, bias last), so each value equals the full
 * oracle's at that index.
 */
int oracle_forward_points(const double *x, const double *offsets, const double *mask,
                          const double *weight, const double *bias, int64_t B, int64_t C_in,
                          int64_t L_in, int64_t C_out, int64_t K, int64_t s, int64_t p,
                          int64_t d, int64_t groups, int64_t G, const int64_t *points,
                          int64_t npts, double *out)
{
    shape_t sh = {B, C_in, L_in, C_out, K, s, p, d, groups, G, 0};
    int st = check_shape(&sh);
    if (st)
        return st;
    const int64_t L_out = sh.L_out;
    const int64_t cpg = C_in / groups, opg = C_out / groups, cpo = C_in / G;
    for (int64_t q = 0; q < npts; ++q) {
        const int64_t b = points[3 * q], co = points[3 * q + 1], l = points[3 * q + 2];
        if (b < 0 || b >= B || co < 0 || co >= C_out || l < 0 || l >= L_out)
            return OR_BAD_ARG;
    }
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int64_t q = 0; q < npts; ++q) {
        const int64_t b = points[3 * q], co = points[3 * q + 1], l = points[3 * q + 2];
        const int64_t grp = co / opg;
        double acc = 0.0;
        for (int64_t cl = 0; cl < cpg; ++cl) {
            const int64_t ci = grp * cpg + cl;
            const int64_t g = ci / cpo;
            const double *row = x + (b * C_in + ci) * L_in;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t oi = ((b * G + g) * L_out + l) * K + k;
                if (!isfinite(offsets[oi]) || (mask && !isfinite(mask[oi])))
                    bad = 1;
                double v = sample(row, L_in, l * s - p + k * d, offsets[oi], mask ? mask + oi : NULL);
                acc += weight[(co * cpg + cl) * K + k] * v;
            }
        }
        out[q] = acc + (bias ? bias[co] : 0.0);
    }
    return bad ? OR_NONFINITE : OR_OK;
}

/*
 * Backward of oracle_forward: the gradients of the scalar
 * sum_{b,co,l} dout[b,co,l] * out[b,co,l] with respect to every input, for
 * a given dout [B, C_out, L_out].  The dc1d page trains the offsets and
 * checks the offset gradient against a finite difference (section Demo
 * notebook) and discusses what the backward keeps alive (section Going
 * faster); the formulas below are the derivatives of the forward as written
 * above, taken term by term:
 *
 *   dS[b,ci,k,l] = sum over the group's output channels co of
 *                  w[co, ci_local, k] * dout[b, co, l]
 *   gx[b,ci,i0]   += dS * m * (1 - f)     (only for 0 <= i0 < L_in)
 *   gx[b,ci,i0+1] += dS * m * f           (only for 0 <= i0+1 < L_in)
 *   goff[b,g,l,k]  = sum over ci in g of dS * m * (x~(i0+1) - x~(i0))
 *   gmask[b,g,l,k] = sum over ci in g of dS * ((1-f) x~(i0) + f x~(i0+1))
 *   gw[co,cl,k]    = sum over (b, l) of dout[b,co,l] * S[b, grp*cpg+cl, k, l]
 *   gb[co]         = sum over (b, l) of dout[b,co,l]
 *
 * The offset derivative is that of the interpolation formula with i0 held
 * fixed, i.e. the right derivative where the offset is an integer (the
 * forward is continuous there but not differentiable).  Any gradient
 * pointer may be NULL.  Sums run in ascending index order.
 */
int oracle_backward(const double *x, const double *offsets, const double *mask,
                    const double *weight, const double *dout, int64_t B, int64_t C_in,
                    int64_t L_in, int64_t C_out, int64_t K, int64_t s, int64_t p, int64_t d,
                    int64_t groups, int64_t G, double *gx, double *goff, double *gmask,
                    double *gw, double *gb)
{
    shape_t sh = {B, C_in, L_in, C_out, K, s, p, d, groups, G, 0};
    int st = check_shape(&sh);
    if (st)
        return st;
    const int64_t L_out = sh.L_out;
    const int64_t cpg = C_in / groups, opg = C_out / groups, cpo = C_in / G;
    const int64_t n_off = B * G * L_out * K;
    if (!all_finite(x, B * C_in * L_in) || !all_finite(offsets, n_off) ||
        (mask && !all_finite(mask, n_off)) || !all_finite(weight, C_out * cpg * K) ||
        !all_finite(dout, B * C_out * L_out))
        return OR_NONFINITE;

    /* dS for every (b, ci, k, l) */
    double *dS = (double *)malloc(sizeof(double) * (size_t)(B * C_in * K * L_out + 1));
    if (!dS)
        return OR_NOMEM;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t ci = 0; ci < C_in; ++ci) {
            const int64_t grp = ci / cpg, cl = ci - grp * cpg;
            for (int64_t k = 0; k < K; ++k)
                for (int64_t l = 0; l < L_out; ++l) {
                    double acc = 0.0;
                    for (int64_t oc = 0; oc < opg; ++oc) {
                        const int64_t co = grp * opg + oc;
                        acc += weight[(co * cpg + cl) * K + k] * dout[(b * C_out + co) * L_out + l];
                    }
                    dS[((b * C_in + ci) * K + k) * L_out + l] = acc;
                }
        }

    /* gx: each (b, ci) row receives only its own samples' contributions */
    if (gx) {
#pragma omp parallel for collapse(2) schedule(static)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t ci = 0; ci < C_in; ++ci) {
                const int64_t g = ci / cpo;
                double *grow = gx + (b * C_in + ci) * L_in;
                for (int64_t i = 0; i < L_in; ++i)
                    grow[i] = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    for (int64_t l = 0; l < L_out; ++l) {
                        const int64_t oi = ((b * G + g) * L_out + l) * K + k;
                        int64_t i0;
                        double f;
                        split_position(l * s - p + k * d, offsets[oi], &i0, &f);
                        const double m = mask ? mask[oi] : 1.0;
                        const double ds = dS[((b * C_in + ci) * K + k) * L_out + l];
                        if (i0 >= 0 && i0 < L_in)
                            grow[i0] += ds * m * (1.0 - f);
                        if (i0 + 1 >= 0 && i0 + 1 < L_in)
                            grow[i0 + 1] += ds * m * f;
                    }
            }
    }

    /* goff, gmask: sums over the offset group's channels */
    if (goff || gmask) {
#pragma omp parallel for collapse(2) schedule(static)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t g = 0; g < G; ++g)
                for (int64_t l = 0; l < L_out; ++l)
                    for (int64_t k = 0; k < K; ++k) {
                        const int64_t oi = ((b * G + g) * L_out + l) * K + k;
                        int64_t i0;
                        double f;
                        split_position(l * s - p + k * d, offsets[oi], &i0, &f);
                        const double m = mask ? mask[oi] : 1.0;
                        double ao = 0.0, am = 0.0;
                        for (int64_t ci = g * cpo; ci < (g + 1) * cpo; ++ci) {
                            const double *row = x + (b * C_in + ci) * L_in;
                            const double x0 = x_ext(row, L_in, i0), x1 = x_ext(row, L_in, i0 + 1);
                            const double ds = dS[((b * C_in + ci) * K + k) * L_out + l];
                            ao += ds * m * (x1 - x0);
                            am += ds * ((1.0 - f) * x0 + f * x1);
                        }
                        if (goff)
                            goff[oi] = ao;
                        if (gmask)
                            gmask[oi] = am;
                    }
    }
    free(dS);

    /* gw: dout against the sampled tensor, recomputed per term */
    if (gw) {
#pragma omp parallel for schedule(static)
        for (int64_t co = 0; co < C_out; ++co) {
            const int64_t grp = co / opg;
            for (int64_t cl = 0; cl < cpg; ++cl) {
                const int64_t ci = grp * cpg + cl, g = ci / cpo;
                for (int64_t k = 0; k < K; ++k) {
                    double acc = 0.0;
                    for (int64_t b = 0; b < B; ++b) {
                        const double *row = x + (b * C_in + ci) * L_in;
                        for (int64_t l = 0; l < L_out; ++l) {
                            const int64_t oi = ((b * G + g) * L_out + l) * K + k;
                            acc += dout[(b * C_out + co) * L_out + l] *
                                   sample(row, L_in, l * s - p + k * d, offsets[oi], mask ? mask + oi : NULL);
                        }
                    }
                    gw[(co * cpg + cl) * K + k] = acc;
                }
            }
        }
    }
    if (gb) {
        for (int64_t co = 0; co < C_out; ++co) {
            double acc = 0.0;
            for (int64_t b = 0; b < B; ++b)
                for (int64_t l = 0; l < L_out; ++l)
                    acc += dout[(b * C_out + co) * L_out + l];
            gb[co] = acc;
        }
    }
    return OR_OK;
}

/*
 * The offset (and mask) generator of the packed layer (dc1d page, section
 * PackedDeformConv1d, and its Modulation (DCNv2) paragraph): the layer
 * computes its own offsets from the input with a depthwise-separable
 * convolutional block, and when modulated, a second pointwise branch off
 * the same depthwise trunk, ending in a sigmoid, predicts the mask.  The
 * page only sketches the block; the readings taken here:
 *
 *  - trunk: one depthwise conv1d over x with the layer's kernel size,
 *    stride, padding and dilation (so it yields the L_out positions the
 *    offsets need), optional bias, no normalisation or activation:
 *        t[b,c,l] = tb[c] + sum_k tw[c,k] * x~[b,c, l*s - p + k*d];
 *  - offset head: a pointwise conv C_in -> G*K with optional bias;
 *    output channel g*K + k holds offsets[b,g,l,k]:
 *        offsets[b,g,l,k] = ob[g*K+k] + sum_c ow[g*K+k, c] * t[b,c,l];
 *  - mask head (only when mw is given): the same with (mw, mb), then the
 *    logistic sigmoid 1 / (1 + exp(-z)).
 *
 * Sums run over k (trunk) and c (heads) in ascending order, bias added
 * last.  tw is [C_in, K] (a [C_in, 1, K] depthwise weight), ow and mw are
 * [G*K, C_in] (pointwise [G*K, C_in, 1]).  mask_out is written only when
 * mw is given.
 */
int oracle_packed_heads(const double *x, const double *tw, const double *tb, const double *ow,
                        const double *ob, const double *mw, const double *mb, int64_t B, int64_t C_in,
                        int64_t L_in, int64_t K, int64_t s, int64_t p, int64_t d, int64_t G,
                        double *offsets_out, double *mask_out)
{
    if (B < 0 || C_in < 1 || G < 1 || C_in % G)
        return OR_BAD_ARG;
    int64_t L_out = oracle_output_length(L_in, K, s, p, d);
    if (L_out < 1)
        return OR_BAD_ARG;
    if (!all_finite(x, B * C_in * L_in) || !all_finite(tw, C_in * K) || (tb && !all_finite(tb, C_in)) ||
        !all_finite(ow, G * K * C_in) || (ob && !all_finite(ob, G * K)) || (mw && !all_finite(mw, G * K * C_in)) ||
        (mw && mb && !all_finite(mb, G * K)))
        return OR_NONFINITE;
    double *t = (double *)malloc((size_t)(C_in * L_out > 0 ? C_in * L_out : 1) * sizeof(double));
    if (!t)
        return OR_NOMEM;
    for (int64_t b = 0; b < B; ++b) {
        /* trunk */
        for (int64_t c = 0; c < C_in; ++c) {
            const double *row = x + (b * C_in + c) * L_in;
            for (int64_t l = 0; l < L_out; ++l) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += tw[c * K + k] * x_ext(row, L_in, l * s - p + k * d);
                t[c * L_out + l] = tb ? acc + tb[c] : acc;
            }
        }
        /* heads */
#pragma omp parallel for schedule(static)
        for (int64_t gk = 0; gk < G * K; ++gk) {
            const int64_t g = gk / K, k = gk % K;
            for (int64_t l = 0; l < L_out; ++l) {
                double zo = 0.0, zm = 0.0;
                for (int64_t c = 0; c < C_in; ++c) {
                    zo += ow[gk * C_in + c] * t[c * L_out + l];
                    if (mw)
                        zm += mw[gk * C_in + c] * t[c * L_out + l];
                }
                const int64_t o = ((b * G + g) * L_out + l) * K + k;
                offsets_out[o] = ob ? zo + ob[gk] : zo;
                if (mw) {
                    const double z = mb ? zm + mb[gk] : zm;
                    mask_out[o] = 1.0 / (1.0 + exp(-z));
                }
            }
        }
    }
    free(t);
    return OR_OK;
}

/*
 * 2D modulated deformable convolution (DCNv2), the variant the other pages
 * describe: the deformable convolution article (section Deformable
 * Convolution: the y(p0) formula, Step 2's bilinear sampling between the
 * four surrounding pixels, Step 3's weighted sum) and the torchvision
 * deform_conv2d issue (offset layout and its printed demo).
 *
 *   x       [B, C_in, H, W]
 *   offsets [B, 2*G*kh*kw, H_out, W_out]; channel ((g*kh + i)*kw + j)*2 holds
 *           the row (height) offset of tap (i, j) of offset group g, the next
 *           channel its column (width) offset (the order the issue settles
 *           on: groups, then kernel rows, then kernel columns, then the pair)
 *   mask    [B, G*kh*kw, H_out, W_out] or NULL, channel (g*kh + i)*kw + j
 *   weight  [C_out, C_in/groups, kh, kw]
 *   bias    [C_out] or NULL
 *   out     [B, C_out, H_out, W_out]
 *
 * Tap (i, j) of output (oh, ow) samples at row oh*sh - ph + i*dh + dy and
 * column ow*sw - pw + j*dw + dx.  Each axis is split as in 1D (exact
 * integer grid term plus the floor of the offset); the sample is the
 * bilinear blend of the four neighbours with weights (1-fy)(1-fx),
 * (1-fy)fx, fy(1-fx), fy fx, every neighbour outside the image reading 0;
 * the mask multiplies it as given.  H_out, W_out follow the conv1d closed
 * form per axis.  Contraction in ascending (ci_local, i, j), bias last.
 */
static double x_ext2(const double *plane, int64_t H, int64_t W, int64_t r, int64_t c)
{
    return (r >= 0 && r < H && c >= 0 && c < W) ? plane[r * W + c] : 0.0;
}

int oracle_forward2d(const double *x, const double *offsets, const double *mask, const double *weight,
                     const double *bias, int64_t B, int64_t C_in, int64_t H, int64_t W, int64_t C_out,
                     int64_t kh, int64_t kw, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                     int64_t dw, int64_t groups, int64_t G, double *out)
{
    if (B < 0 || C_in < 1 || C_out < 1 || groups < 1 || G < 1 || C_in % groups || C_out % groups || C_in % G)
        return OR_BAD_ARG;
    const int64_t H_out = oracle_output_length(H, kh, sh, ph, dh);
    const int64_t W_out = oracle_output_length(W, kw, sw, pw, dw);
    if (H_out < 1 || W_out < 1)
        return OR_BAD_ARG;
    const int64_t cpg = C_in / groups, opg = C_out / groups, cpo = C_in / G, T = kh * kw;
    const int64_t HWo = H_out * W_out;
    if (!all_finite(x, B * C_in * H * W) || !all_finite(offsets, B * 2 * G * T * HWo) ||
        (mask && !all_finite(mask, B * G * T * HWo)) || !all_finite(weight, C_out * cpg * T) ||
        (bias && !all_finite(bias, C_out)))
        return OR_NONFINITE;
    if (B == 0)
        return OR_OK;
    /* Stage 1: S[b, ci, i, j, oh, ow] */
    double *S = (double *)malloc(sizeof(double) * (size_t)(B * C_in * T * HWo));
    if (!S)
        return OR_NOMEM;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t ci = 0; ci < C_in; ++ci) {
            const int64_t g = ci / cpo;
            const double *plane = x + (b * C_in + ci) * H * W;
            for (int64_t i = 0; i < kh; ++i)
                for (int64_t j = 0; j < kw; ++j) {
                    const int64_t tap = (g * kh + i) * kw + j;
                    const double *oy = offsets + (b * 2 * G * T + 2 * tap) * HWo;
                    const double *ox = oy + HWo;
                    const double *mm = mask ? mask + (b * G * T + tap) * HWo : NULL;
                    for (int64_t oh = 0; oh < H_out; ++oh)
                        for (int64_t ow = 0; ow < W_out; ++ow) {
                            const int64_t q = oh * W_out + ow;
                            int64_t r0, c0;
                            double fy, fx;
                            split_position(oh * sh - ph + i * dh, oy[q], &r0, &fy);
                            split_position(ow * sw - pw + j * dw, ox[q], &c0, &fx);
                            double v = (1.0 - fy) * (1.0 - fx) * x_ext2(plane, H, W, r0, c0) +
                                       (1.0 - fy) * fx * x_ext2(plane, H, W, r0, c0 + 1) +
                                       fy * (1.0 - fx) * x_ext2(plane, H, W, r0 + 1, c0) +
                                       fy * fx * x_ext2(plane, H, W, r0 + 1, c0 + 1);
                            if (mm)
                                v *= mm[q];
                            S[((b * C_in + ci) * T + i * kw + j) * HWo + q] = v;
                        }
                }
        }
    /* Stage 2 */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t co = 0; co < C_out; ++co) {
            const int64_t grp = co / opg;
            for (int64_t q = 0; q < HWo; ++q) {
                double acc = 0.0;
                for (int64_t cl = 0; cl < cpg; ++cl)
                    for (int64_t t = 0; t < T; ++t)
                        acc += weight[(co * cpg + cl) * T + t] * S[((b * C_in + grp * cpg + cl) * T + t) * HWo + q];
                out[(b * C_out + co) * HWo + q] = acc + (bias ? bias[co] : 0.0);
            }
        }
    free(S);
    return OR_OK;
}
