/*
 * awq_oracle.c -- CPU oracle for the AWQ per-layer scale search.
 *
 * TEST INFRASTRUCTURE ONLY: plain, slow and written to be checked by eye
 * against the pages (see awq_oracle.h for the sources). Nothing here is tuned;
 * the only parallelism is an OpenMP loop over output rows whose per-row results
 * are combined afterwards in ascending row order. Built with
 * -O2 -ffp-contract=off and without fast-math, so every fp32/fp64 operation is
 * one IEEE operation with round-half-to-even.
 */
#include "awq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define REF_OK 0
#define REF_EINVAL (-1)
#define REF_ENONFINITE (-4)

/* ---------------------------------------------------------------------------
 * Step 1: s_X[j] = mean over tokens of |X[:, j]|, plus 1e-8.
 * [G] "How it works" step 1; [G] "The code, line by line" (the 1e-8 keeps a
 * channel that is always zero from getting a zero scale).
 * The pages use a library mean; the order of the fp64 sum is fixed here:
 * sequential inside consecutive 64-token chunks, then the chunk sums in order.
 * ------------------------------------------------------------------------- */
void awq_ref_act_stats(const float *X, int64_t tokens, int64_t in, float *xmag)
{
    for (int64_t j = 0; j < in; ++j) {
        double total = 0.0;
        for (int64_t t0 = 0; t0 < tokens; t0 += 64) {
            int64_t t1 = t0 + 64 < tokens ? t0 + 64 : tokens;
            double chunk = 0.0;
            for (int64_t t = t0; t < t1; ++t)
                chunk += fabs((double)X[t * in + j]);
            total += chunk;
        }
        double mean = total / (double)tokens;
        xmag[j] = (float)(mean + 1e-8);
    }
}

/* ---------------------------------------------------------------------------
 * Step 2: the alpha grid and the candidate scales.
 * [G] "The code, line by line": alpha runs over grid+1 evenly spaced values in
 * [0, 1] (0 included, so the grid contains plain RTN), s = s_X^alpha, then
 * s is divided by sqrt(max(s) * min(s)) so the scales are centred on 1 in log
 * scale. The power and the centring are fp64; s is rounded to fp32 once.
 * ------------------------------------------------------------------------- */
int awq_ref_s_table(const float *xmag, int64_t in, int grid, float *s_table)
{
    if (!xmag || !s_table || in < 1 || grid < 1)
        return REF_EINVAL;
    double *p = (double *)malloc((size_t)in * sizeof(double));
    if (!p)
        return REF_EINVAL;
    for (int k = 0; k <= grid; ++k) {
        double alpha = (double)k / (double)grid;
        for (int64_t j = 0; j < in; ++j)
            p[j] = pow((double)xmag[j], alpha);
        double pmax = p[0], pmin = p[0];
        for (int64_t j = 1; j < in; ++j) {
            if (p[j] > pmax) pmax = p[j];
            if (p[j] < pmin) pmin = p[j];
        }
        double centre = sqrt(pmax * pmin);
        for (int64_t j = 0; j < in; ++j)
            s_table[(int64_t)k * in + j] = (float)(p[j] / centre);
    }
    free(p);
    return REF_OK;
}

/* ---------------------------------------------------------------------------
 * Step 3a: round-to-nearest on one group, fp32.
 * Symmetric ([N] "Per-group symmetric int4 (RTN)" and its n-bit variant in
 * "Output MSE vs bit width"): levels L = 2^(b-1) - 1,
 *   scale = max(max|v| / L, 1e-8), q = clamp(round(v / scale), -L-1, L),
 *   dequantized = q * scale; stored code = q + 2^(b-1), zero = 2^(b-1)
 *   ([C] "The shared problem": symmetric variants fix the zero point).
 * Asymmetric ([C] group_params / rtn in "GPTQ: compensate the error you just
 * made"): maxq = 2^b - 1, lo = min(min v, 0), hi = max(max v, 0),
 *   scale = max((hi - lo) / maxq, 1e-8), zero = round(-lo / scale),
 *   code = clamp(round(v / scale) + zero, 0, maxq), dequantized = scale*(code - zero).
 * round() is half-to-even (numpy/torch round), i.e. rintf in the default mode.
 * ------------------------------------------------------------------------- */
int awq_ref_quant_group(const float *v, int64_t g, int bits, int mode,
                        int32_t *code, float *scale_out, int32_t *zero_out, float *what)
{
    if (!v || g < 1 || bits < 2 || bits > 8 || (mode != AWQ_REF_SYM && mode != AWQ_REF_ASYM))
        return REF_EINVAL;
    if (mode == AWQ_REF_SYM) {
        const float levels = (float)((1 << (bits - 1)) - 1);
        const int32_t offset = 1 << (bits - 1);
        float amax = 0.0f;
        for (int64_t i = 0; i < g; ++i) {
            float a = fabsf(v[i]);
            if (a > amax) amax = a;
        }
        float scale = amax / levels;
        if (scale < 1e-8f) scale = 1e-8f;
        for (int64_t i = 0; i < g; ++i) {
            float q = rintf(v[i] / scale);
            if (q < -levels - 1.0f) q = -levels - 1.0f;
            if (q > levels) q = levels;
            if (code) code[i] = (int32_t)q + offset;
            if (what) what[i] = q * scale;
        }
        if (scale_out) *scale_out = scale;
        if (zero_out) *zero_out = offset;
    } else {
        const float maxq = (float)((1 << bits) - 1);
        float lo = v[0], hi = v[0];
        for (int64_t i = 1; i < g; ++i) {
            if (v[i] < lo) lo = v[i];
            if (v[i] > hi) hi = v[i];
        }
        if (lo > 0.0f) lo = 0.0f;
        if (hi < 0.0f) hi = 0.0f;
        float scale = (hi - lo) / maxq;
        if (scale < 1e-8f) scale = 1e-8f;
        float zero = rintf(-lo / scale);
        for (int64_t i = 0; i < g; ++i) {
            float q = rintf(v[i] / scale) + zero;
            if (q < 0.0f) q = 0.0f;
            if (q > maxq) q = maxq;
            if (code) code[i] = (int32_t)q;
            if (what) what[i] = scale * (q - zero);
        }
        if (scale_out) *scale_out = scale;
        if (zero_out) *zero_out = (int32_t)zero;
    }
    return REF_OK;
}

static int check_layer(int64_t out, int64_t in, int bits, int group, int mode)
{
    if (out < 1 || in < 1 || group < 1 || in % group != 0)
        return REF_EINVAL;
    if (bits < 2 || bits > 8 || (mode != AWQ_REF_SYM && mode != AWQ_REF_ASYM))
        return REF_EINVAL;
    return REF_OK;
}

/* ---------------------------------------------------------------------------
 * Step 3b: fake quantization Q(W diag(s)) / s.
 * [G] "The code, line by line": column j is multiplied by s[j] (fp32 product),
 * each row is quantized group by group, and the result is divided by s again
 * (here in fp64), which is the deployed layer with the fold done inside W.
 * ------------------------------------------------------------------------- */
int awq_ref_fake_quant(const float *W, int64_t out, int64_t in, const float *s,
                       int bits, int group, int mode, double *wq)
{
    if (!W || !s || !wq || check_layer(out, in, bits, group, mode) != REF_OK)
        return REF_EINVAL;
    int bad = 0;
#pragma omp parallel
    {
        float *v = (float *)malloc((size_t)group * sizeof(float));
        float *what = (float *)malloc((size_t)group * sizeof(float));
        if (!v || !what) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t o = 0; o < out; ++o) {
                for (int64_t g0 = 0; g0 < in; g0 += group) {
                    for (int64_t i = 0; i < group; ++i)
                        v[i] = W[o * in + g0 + i] * s[g0 + i];
                    awq_ref_quant_group(v, group, bits, mode, NULL, NULL, NULL, what);
                    for (int64_t i = 0; i < group; ++i)
                        wq[o * in + g0 + i] = (double)what[i] / (double)s[g0 + i];
                }
            }
        }
        free(v);
        free(what);
    }
    return bad ? REF_EINVAL : REF_OK;
}

/* X as fp64 (exact) and ref = X W^T as fp64 [out][tokens]. */
static double *to_f64(const float *a, int64_t n)
{
    double *r = (double *)malloc((size_t)n * sizeof(double));
    if (r)
        for (int64_t i = 0; i < n; ++i)
            r[i] = (double)a[i];
    return r;
}

static double dot(const double *a, const double *b, int64_t n)
{
    double acc = 0.0;
    for (int64_t i = 0; i < n; ++i)
        acc += a[i] * b[i];
    return acc;
}

/* Sum over tokens and rows of (X wq^T - ref)^2, rows combined in ascending
 * order. ref: fp64[out][tokens] holding X W^T. */
static double output_sse(const double *x64, const double *ref, const double *wq,
                         int64_t out, int64_t in, int64_t tokens, double *row_sse,
                         int nthreads)
{
    if (nthreads <= 0) {
#ifdef _OPENMP
        nthreads = omp_get_max_threads();
#else
        nthreads = 1;
#endif
    }
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t o = 0; o < out; ++o) {
        double sse = 0.0;
        for (int64_t t = 0; t < tokens; ++t) {
            double y = dot(x64 + t * in, wq + o * in, in);
            double e = y - ref[o * tokens + t];
            sse += e * e;
        }
        row_sse[o] = sse;
    }
    double total = 0.0;
    for (int64_t o = 0; o < out; ++o)
        total += row_sse[o];
    return total;
}

static double *reference_output(const double *x64, const float *W, int64_t out,
                                int64_t in, int64_t tokens, int nthreads)
{
    double *ref = (double *)malloc((size_t)(out * tokens) * sizeof(double));
    double *w64 = to_f64(W, out * in);
    if (!ref || !w64) {
        free(ref);
        free(w64);
        return NULL;
    }
    if (nthreads <= 0) {
#ifdef _OPENMP
        nthreads = omp_get_max_threads();
#else
        nthreads = 1;
#endif
    }
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t o = 0; o < out; ++o)
        for (int64_t t = 0; t < tokens; ++t)
            ref[o * tokens + t] = dot(x64 + t * in, w64 + o * in, in);
    free(w64);
    return ref;
}

/* ---------------------------------------------------------------------------
 * Step 3c: output error, mean((X Wq^T - X W^T)^2) over all tokens and outputs.
 * [G] "How it works" step 3 and the err line of "The code, line by line";
 * [C] "The shared problem" (both methods minimise ||W X - W_hat X||^2).
 * ------------------------------------------------------------------------- */
double awq_ref_output_mse(const float *W, const double *wq, const float *X,
                          int64_t out, int64_t in, int64_t tokens, int nthreads)
{
    if (!W || !wq || !X || out < 1 || in < 1 || tokens < 1)
        return NAN;
    double *x64 = to_f64(X, tokens * in);
    double *row = (double *)malloc((size_t)out * sizeof(double));
    double *ref = x64 ? reference_output(x64, W, out, in, tokens, nthreads) : NULL;
    double mse = NAN;
    if (x64 && row && ref)
        mse = output_sse(x64, ref, wq, out, in, tokens, row, nthreads) /
              ((double)tokens * (double)out);
    free(x64);
    free(row);
    free(ref);
    return mse;
}

/* ---------------------------------------------------------------------------
 * Steps 2-4: the search ([G] "Source code", awq() listing; [C] awq_scales()).
 * For each alpha on the grid, in increasing order: the s-table row, the fake
 * quantized weight, its output MSE; a candidate replaces the best one only
 * when its error is strictly smaller, so the lowest alpha wins ties and a NaN
 * error is never chosen. Because alpha = 0 (s = 1, plain RTN) is on the grid,
 * the chosen error is never above RTN's ([G] "The code, line by line").
 * ------------------------------------------------------------------------- */
int awq_ref_search(const float *W, const float *X, int64_t out, int64_t in,
                   int64_t tokens, const float *xmag, int bits, int group,
                   int grid, int mode, double *mse, int32_t *best,
                   float *s_best, int nthreads)
{
    if (!W || !X || !xmag || !mse || !best || !s_best || tokens < 1 || grid < 1 ||
        check_layer(out, in, bits, group, mode) != REF_OK)
        return REF_EINVAL;
    const int n_alpha = grid + 1;
    float *s_table = (float *)malloc((size_t)n_alpha * (size_t)in * sizeof(float));
    double *wq = (double *)malloc((size_t)(out * in) * sizeof(double));
    double *row = (double *)malloc((size_t)out * sizeof(double));
    double *x64 = to_f64(X, tokens * in);
    double *ref = x64 ? reference_output(x64, W, out, in, tokens, nthreads) : NULL;
    int status = REF_OK;
    if (!s_table || !wq || !row || !x64 || !ref) {
        status = REF_EINVAL;
        goto done;
    }
    awq_ref_s_table(xmag, in, grid, s_table);

    int32_t best_k = -1;
    double best_err = INFINITY;
    for (int k = 0; k < n_alpha; ++k) {
        const float *s = s_table + (int64_t)k * in;
        awq_ref_fake_quant(W, out, in, s, bits, group, mode, wq);
        double err = output_sse(x64, ref, wq, out, in, tokens, row, nthreads) /
                     ((double)tokens * (double)out);
        mse[k] = err;
        if (err < best_err) {
            best_err = err;
            best_k = k;
        }
    }
    *best = best_k;
    if (best_k >= 0) {
        memcpy(s_best, s_table + (int64_t)best_k * in, (size_t)in * sizeof(float));
    } else {
        for (int64_t j = 0; j < in; ++j)
            s_best[j] = 1.0f;
        status = REF_ENONFINITE;
    }
done:
    free(s_table);
    free(wq);
    free(row);
    free(x64);
    free(ref);
    return status;
}

/* ---------------------------------------------------------------------------
 * Clipping-range search. [G] "Simplifications" names a per-group clipping
 * threshold that shrinks the max range to cut rounding error; [C] "AWQ: move
 * the error away from what matters" describes a second search after the
 * alpha search that shrinks each group's clipping range a little when that
 * lowers output error, then plain RTN. The pages fix no numbers; the readings
 * used here:
 *   - shrink ratios r_i = fl32(1 - i * max_shrink / n_clip), i = 0..n_clip-1,
 *     computed in fp64 and rounded once (r_0 = 1: no clipping);
 *   - the clipping range of a group is the quantizer's own range scaled by r:
 *     symmetric [-r*A, r*A] with A = max|v|; asymmetric [r*lo, r*hi] with
 *     lo = min(min v, 0), hi = max(max v, 0); values are clamped into it and
 *     the scale (and zero) are those of the clipped range;
 *   - the error of a choice is the group's own squared output error over the
 *     calibration tokens, sum_t (sum_{j in group} X[t,j] (wq_j - w_j))^2 with
 *     wq = fake-quantized weight / s (fp64), groups taken one at a time;
 *   - per (row, group) the first strict minimum over i wins (NaN never).
 * ------------------------------------------------------------------------- */
float awq_ref_clip_ratio(int i, int n_clip, float max_shrink)
{
    return (float)(1.0 - (double)i * (double)max_shrink / (double)n_clip);
}

int awq_ref_quant_group_clip(const float *v, int64_t g, int bits, int mode, float ratio,
                             int32_t *code, float *scale_out, int32_t *zero_out, float *what)
{
    if (!v || g < 1 || bits < 2 || bits > 8 || (mode != AWQ_REF_SYM && mode != AWQ_REF_ASYM))
        return REF_EINVAL;
    if (mode == AWQ_REF_SYM) {
        const float levels = (float)((1 << (bits - 1)) - 1);
        const int32_t offset = 1 << (bits - 1);
        float amax = 0.0f;
        for (int64_t i = 0; i < g; ++i) {
            float a = fabsf(v[i]);
            if (a > amax) amax = a;
        }
        const float mx = ratio * amax;          /* clipped range [-mx, mx] */
        float scale = mx / levels;
        if (scale < 1e-8f) scale = 1e-8f;
        for (int64_t i = 0; i < g; ++i) {
            float x = v[i];
            if (x > mx) x = mx;
            if (x < -mx) x = -mx;
            float q = rintf(x / scale);
            if (q < -levels - 1.0f) q = -levels - 1.0f;
            if (q > levels) q = levels;
            if (code) code[i] = (int32_t)q + offset;
            if (what) what[i] = q * scale;
        }
        if (scale_out) *scale_out = scale;
        if (zero_out) *zero_out = offset;
    } else {
        const float maxq = (float)((1 << bits) - 1);
        float lo = v[0], hi = v[0];
        for (int64_t i = 1; i < g; ++i) {
            if (v[i] < lo) lo = v[i];
            if (v[i] > hi) hi = v[i];
        }
        if (lo > 0.0f) lo = 0.0f;
        if (hi < 0.0f) hi = 0.0f;
        lo = ratio * lo;                          /* clipped range [lo, hi] */
        hi = ratio * hi;
        float scale = (hi - lo) / maxq;
        if (scale < 1e-8f) scale = 1e-8f;
        float zero = rintf(-lo / scale);
        for (int64_t i = 0; i < g; ++i) {
            float x = v[i];
            if (x > hi) x = hi;
            if (x < lo) x = lo;
            float q = rintf(x / scale) + zero;
            if (q < 0.0f) q = 0.0f;
            if (q > maxq) q = maxq;
            if (code) code[i] = (int32_t)q;
            if (what) what[i] = scale * (q - zero);
        }
        if (scale_out) *scale_out = scale;
        if (zero_out) *zero_out = (int32_t)zero;
    }
    return REF_OK;
}

int awq_ref_clip_search(const float *W, const float *X, int64_t out, int64_t in, int64_t tokens,
                        const float *s, int bits, int group, int mode, int n_clip,
                        float max_shrink, float *clip, double *sse, int nthreads)
{
    if (!W || !X || !s || !clip || tokens < 1 || n_clip < 1 || !(max_shrink >= 0.0f) ||
        max_shrink >= 1.0f || check_layer(out, in, bits, group, mode) != REF_OK)
        return REF_EINVAL;
    const int64_t ngroups = in / group;
    double *x64 = to_f64(X, tokens * in);
    if (!x64)
        return REF_EINVAL;
    int bad = 0;
    if (nthreads <= 0) {
#ifdef _OPENMP
        nthreads = omp_get_max_threads();
#else
        nthreads = 1;
#endif
    }
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t o = 0; o < out; ++o) {
        float *v = (float *)malloc((size_t)group * sizeof(float));
        float *what = (float *)malloc((size_t)group * sizeof(float));
        double *d = (double *)malloc((size_t)group * sizeof(double));
        if (!v || !what || !d) {
#pragma omp atomic write
            bad = 1;
            free(v);
            free(what);
            free(d);
            continue;
        }
        for (int64_t gi = 0; gi < ngroups; ++gi) {
            const int64_t g0 = gi * group;
            for (int64_t j = 0; j < group; ++j)
                v[j] = W[o * in + g0 + j] * s[g0 + j];
            int best = 0;
            double best_e = INFINITY;
            for (int i = 0; i < n_clip; ++i) {
                const float r = awq_ref_clip_ratio(i, n_clip, max_shrink);
                awq_ref_quant_group_clip(v, group, bits, mode, r, NULL, NULL, NULL, what);
                for (int64_t j = 0; j < group; ++j)
                    d[j] = (double)what[j] / (double)s[g0 + j] - (double)W[o * in + g0 + j];
                double e = 0.0;
                for (int64_t t = 0; t < tokens; ++t) {
                    const double y = dot(x64 + t * in + g0, d, group);
                    e += y * y;
                }
                if (sse)
                    sse[(o * ngroups + gi) * n_clip + i] = e;
                if (e < best_e) {
                    best_e = e;
                    best = i;
                }
            }
            clip[o * ngroups + gi] = awq_ref_clip_ratio(best, n_clip, max_shrink);
        }
        free(v);
        free(what);
        free(d);
    }
    free(x64);
    return bad ? REF_EINVAL : REF_OK;
}

/* ---------------------------------------------------------------------------
 * Final RTN of W diag(s) and packing. What is stored follows [C] "What lands
 * on disk" (integer codes packed into 32-bit words, one scale and one zero per
 * group and output row); the bit order and axis are this library's own: code i
 * of row o occupies bits [i*bits, (i+1)*bits) of that row's little-endian
 * stream of 32-bit words.
 * ------------------------------------------------------------------------- */
int awq_ref_quantize_pack(const float *W, int64_t out, int64_t in, const float *s,
                          int bits, int group, int mode, uint32_t *qweight,
                          float *scales, uint8_t *zeros)
{
    return awq_ref_quantize_pack_clip(W, out, in, s, NULL, bits, group, mode, qweight, scales, zeros);
}

int awq_ref_quantize_pack_clip(const float *W, int64_t out, int64_t in, const float *s,
                               const float *clip, int bits, int group, int mode,
                               uint32_t *qweight, float *scales, uint8_t *zeros)
{
    if (!W || !s || !qweight || !scales || !zeros ||
        check_layer(out, in, bits, group, mode) != REF_OK)
        return REF_EINVAL;
    const int64_t words = (in * bits + 31) / 32;
    const int64_t ngroups = in / group;
    float *v = (float *)malloc((size_t)group * sizeof(float));
    int32_t *code = (int32_t *)malloc((size_t)group * sizeof(int32_t));
    if (!v || !code) {
        free(v);
        free(code);
        return REF_EINVAL;
    }
    for (int64_t o = 0; o < out; ++o) {
        uint32_t *rowq = qweight + o * words;
        memset(rowq, 0, (size_t)words * sizeof(uint32_t));
        for (int64_t gi = 0; gi < ngroups; ++gi) {
            const int64_t g0 = gi * group;
            for (int64_t i = 0; i < group; ++i)
                v[i] = W[o * in + g0 + i] * s[g0 + i];
            float scale;
            int32_t zero;
            if (clip)
                awq_ref_quant_group_clip(v, group, bits, mode, clip[o * ngroups + gi], code, &scale,
                                         &zero, NULL);
            else
                awq_ref_quant_group(v, group, bits, mode, code, &scale, &zero, NULL);
            scales[o * ngroups + gi] = scale;
            zeros[o * ngroups + gi] = (uint8_t)zero;
            for (int64_t i = 0; i < group; ++i) {
                uint64_t bit = (uint64_t)(g0 + i) * (uint64_t)bits;
                uint64_t word = bit / 32, shift = bit % 32;
                uint32_t c = (uint32_t)code[i];
                rowq[word] |= c << shift;
                if (shift + (uint64_t)bits > 32)
                    rowq[word + 1] |= c >> (32 - shift);
            }
        }
    }
    free(v);
    free(code);
    return REF_OK;
}

/* ---------------------------------------------------------------------------
 * Folding s into the model ([G] "How it works" step 5 and the transformer
 * paragraph; [C] "AWQ: move the error away from what matters": W is multiplied
 * by s and the previous operation divided by it). The identity behind it is
 * W x = (W diag(s)) (diag(s)^-1 x) ([C] "AWQ: move the error ..."; [G] "The
 * code, line by line"). The pages do not say how the result is stored; here:
 * one fp32 operation, then one rounding to the model's storage type.
 * ------------------------------------------------------------------------- */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
uint16_t awq_ref_f32_to_f16(float x)
{
    uint32_t b;
    memcpy(&b, &x, sizeof b);
    const uint32_t sign = (b >> 16) & 0x8000u;
    const int32_t exp = (int32_t)((b >> 23) & 0xffu);
    const uint32_t frac = b & 0x7fffffu;
    if (exp == 0xff)                                   /* inf, NaN (kept quiet) */
        return (uint16_t)(sign | 0x7c00u | (frac ? 0x200u | (frac >> 13) : 0u));
    if (exp == 0)                                      /* fp32 zero or subnormal: < 2^-126 */
        return (uint16_t)sign;
    const uint32_t m = frac | 0x800000u;               /* value = m * 2^(exp - 150) */
    const int32_t e16 = exp - 127 + 15;
    if (e16 >= 31)
        return (uint16_t)(sign | 0x7c00u);
    uint32_t shift, q;
    if (e16 >= 1) {
        shift = 13;                                    /* keep 11 significant bits */
        q = ((uint32_t)e16 << 10) | ((m >> 13) & 0x3ffu);
    } else {
        /* subnormal: units of 2^-24, value / 2^-24 = m * 2^(exp - 126) */
        shift = (uint32_t)(126 - exp);
        if (shift > 24)
            return (uint16_t)sign;                     /* below a quarter unit */
        q = m >> shift;
    }
    const uint32_t rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1;                                        /* a carry moves up one binade (or to inf) */
    return (uint16_t)(sign | q);
}

/* bfloat16: the upper half of the fp32 pattern, rounded half to even. */
uint16_t awq_ref_f32_to_bf16(float x)
{
    uint32_t b;
    memcpy(&b, &x, sizeof b);
    if ((b & 0x7f800000u) == 0x7f800000u && (b & 0x7fffffu))
        return (uint16_t)((b >> 16) | 0x40u);          /* NaN, quiet */
    const uint32_t lower = b & 0xffffu, upper = b >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        return (uint16_t)(upper + 1u);
    return (uint16_t)upper;
}

static void store_one(void *out, int64_t i, int storage, float v)
{
    if (storage == AWQ_REF_STORE_F32)
        ((float *)out)[i] = v;
    else if (storage == AWQ_REF_STORE_F16)
        ((uint16_t *)out)[i] = awq_ref_f32_to_f16(v);
    else
        ((uint16_t *)out)[i] = awq_ref_f32_to_bf16(v);
}

int awq_ref_fold_rows(const float *A, int64_t rows, int64_t cols, const float *s, int storage,
                      void *out)
{
    if (!A || !s || !out || rows < 1 || cols < 1 || storage < 0 || storage > 2)
        return REF_EINVAL;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            store_one(out, r * cols + c, storage, A[r * cols + c] / s[r]);
    return REF_OK;
}

int awq_ref_scale_cols(const float *W, int64_t rows, int64_t cols, const float *s, int storage,
                       void *out)
{
    if (!W || !s || !out || rows < 1 || cols < 1 || storage < 0 || storage > 2)
        return REF_EINVAL;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            store_one(out, r * cols + c, storage, W[r * cols + c] * s[c]);
    return REF_OK;
}

/* ---------------------------------------------------------------------------
 * Deployment: Y = X Wd^T with Wd the dequantized packed weights ([C] "What
 * lands on disk": codes plus one scale and one zero per group and output row;
 * "From checkpoint to kernel": the serving kernel consumes them directly).
 * Dequantization is scale * (code - zero) (for symmetric layers the stored
 * zero is 2^(bits-1)), taken exactly in fp64.
 * ------------------------------------------------------------------------- */
uint32_t awq_ref_unpack_code(const uint32_t *row, int64_t k, int bits)
{
    uint32_t code = 0;
    for (int b = 0; b < bits; ++b) {
        const uint64_t bit = (uint64_t)k * (uint64_t)bits + (uint64_t)b;
        code |= ((row[bit / 32] >> (bit % 32)) & 1u) << b;
    }
    return code;
}

int awq_ref_qgemm(const float *X, int64_t M, int64_t in, const uint32_t *qweight,
                  const float *scales, const uint8_t *zeros, int64_t out, int bits, int group,
                  double *Y)
{
    if (!X || !qweight || !scales || !zeros || !Y || M < 1 ||
        check_layer(out, in, bits, group, AWQ_REF_SYM) != REF_OK)
        return REF_EINVAL;
    const int64_t words = (in * bits + 31) / 32;
    const int64_t ngroups = in / group;
    double *wd = (double *)malloc((size_t)in * sizeof(double));
    if (!wd)
        return REF_EINVAL;
    for (int64_t n = 0; n < out; ++n) {
        const uint32_t *row = qweight + n * words;
        for (int64_t k = 0; k < in; ++k) {
            const int64_t g = k / group;
            const double code = (double)awq_ref_unpack_code(row, k, bits);
            wd[k] = (double)scales[n * ngroups + g] * (code - (double)zeros[n * ngroups + g]);
        }
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < in; ++k)
                acc += (double)X[m * in + k] * wd[k];
            Y[m * out + n] = acc;
        }
    }
    free(wd);
    return REF_OK;
}
