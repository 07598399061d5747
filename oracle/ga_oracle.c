/*
 * ga_oracle.c -- plain, slow, fp64 CPU oracle for the fused gated activations.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * constant generator with the HIP library: it is written from the definitions
 * on the pages, one step per line, so a reader can check it by eye.
 *
 * Sources (the pages):
 *   - vLLM PR 48498 "[Performance] Add Triton kernel for Gemma3n sparse GELU",
 *     section "Purpose": one row-wise op that takes the per-row mean and
 *     variance of the gate, thresholds it with a Gaussian cutoff, applies the
 *     tanh GELU and multiplies by the up half.
 *   - Megatron-LM PR 6328 "Size MoE activation kernel grid to the row count",
 *     section "What changed and why": an elementwise silu(gate) * up over the
 *     live rows of a capture-sized MoE buffer, bounded by a device row count.
 *   - the same vLLM page, section Purpose: the provider is chosen per
 *     "approximation mode", so plain GELU-and-multiply exists in a tanh and
 *     an exact (erf) form; Megatron-LM PR 6328, section Scope and risks:
 *     the squared-ReLU activation kernel shares the bounded-row pattern.
 *   - the vLLM page, Test Result, Correctness: the activation's output feeds
 *     the layer's downstream projection, which a fused build keeps in order;
 *     here the product with the projection's weights, in double.
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes): the std is the population std (divide by d); the cutoff is
 * mean + z * std with z = inverse normal CDF of the target sparsity, passed in
 * as a float; "tanh GELU" is the textbook tanh approximation with constants
 * sqrt(2/pi) and 0.044715; the gate is the first half of each input row and
 * up the second; the result is computed in double and rounded ONCE, to
 * nearest-even, straight from double to the output type.
 *
 * Parity is pinned (not by re-running this file) in tests/test_oracle_pins.py:
 * codec against numpy / exhaustive search, GELU and SiLU against torch's fp64
 * routines and closed forms, row statistics against numpy and exact rational
 * arithmetic, the whole op against an fp64 torch composition, survival
 * fractions against 1 - Phi(z), the down projection against exact rational
 * sums, numpy's fp64 product and weights that pick out single elements, and
 * planted-mistake (mutant) runs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element types.  The numbering is the library's public dtype numbering,
 * restated here (an interface value, not shared code). */
enum { GAO_F32 = 0, GAO_F16 = 1, GAO_BF16 = 2 };

/* Field widths of a binary IEEE-style format: exponent bits, stored mantissa
 * bits.  bf16 is the top half of an IEEE binary32. */
static int fmt_bits(int dtype, int *ebits, int *mbits)
{
    switch (dtype) {
    case GAO_F32:  *ebits = 8; *mbits = 23; return 0;
    case GAO_F16:  *ebits = 5; *mbits = 10; return 0;
    case GAO_BF16: *ebits = 8; *mbits = 7;  return 0;
    default: return -1;
    }
}

size_t gao_elem_size(int dtype)
{
    return dtype == GAO_F32 ? 4 : (dtype == GAO_F16 || dtype == GAO_BF16) ? 2 : 0;
}

/* Bits -> exact double, from the format's definition:
 *   exponent field 0:          (-1)^s * m * 2^(emin - mbits)   (subnormal)
 *   exponent field all ones:   inf (m == 0) or NaN
 *   otherwise:                 (-1)^s * (2^mbits + m) * 2^(e - bias - mbits)  */
double gao_decode(uint32_t bits, int dtype)
{
    int ebits, mbits;
    if (fmt_bits(dtype, &ebits, &mbits)) return NAN;
    const int bias = (1 << (ebits - 1)) - 1;
    const uint32_t mant = bits & ((1u << mbits) - 1u);
    const uint32_t expf = (bits >> mbits) & ((1u << ebits) - 1u);
    const int sign = (bits >> (mbits + ebits)) & 1u;
    double mag;
    if (expf == 0)
        mag = ldexp((double)mant, 1 - bias - mbits);
    else if (expf == (1u << ebits) - 1u)
        mag = mant ? NAN : INFINITY;
    else
        mag = ldexp((double)((1u << mbits) + mant), (int)expf - bias - mbits);
    return sign ? -mag : mag;
}

/* double -> nearest representable value of the format, ties to even, in one
 * rounding step (no detour through float).  Overflow gives +-inf, NaN gives a
 * quiet NaN, subnormals are produced where the format has them. */
uint32_t gao_encode_rne(double v, int dtype)
{
    int ebits, mbits;
    if (fmt_bits(dtype, &ebits, &mbits)) return 0;
    const int bias = (1 << (ebits - 1)) - 1;
    const int emin = 1 - bias;
    const uint32_t expmax = (1u << ebits) - 1u;
    const uint32_t sign = signbit(v) ? (1u << (ebits + mbits)) : 0u;
    if (isnan(v)) return sign | (expmax << mbits) | (1u << (mbits - 1));
    double x = fabs(v);
    if (isinf(x)) return sign | (expmax << mbits);
    if (x == 0.0) return sign;

    int e2;
    frexp(x, &e2);            /* x = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;           /* x in [2^E, 2^(E+1)) */
    if (E < emin) E = emin;   /* subnormal range shares emin's quantum */
    /* x / quantum, exact (power-of-two scaling); rint rounds half to even. */
    double r = rint(ldexp(x, mbits - E));
    if (r == ldexp(1.0, mbits + 1)) {   /* rounded up into the next binade */
        r = ldexp(1.0, mbits);
        E += 1;
    }
    uint32_t expfield, mant;
    if (r >= ldexp(1.0, mbits)) {
        expfield = (uint32_t)(E + bias);
        mant = (uint32_t)(r - ldexp(1.0, mbits));
    } else {                            /* subnormal (only when E == emin) */
        expfield = 0;
        mant = (uint32_t)r;
    }
    if (expfield >= expmax) return sign | (expmax << mbits);
    return sign | (expfield << mbits) | mant;
}

static double load_elem(const void *base, int64_t i, int dtype)
{
    if (dtype == GAO_F32) return gao_decode(((const uint32_t *)base)[i], dtype);
    return gao_decode(((const uint16_t *)base)[i], dtype);
}

static void store_elem(void *base, int64_t i, int dtype, double v)
{
    uint32_t b = gao_encode_rne(v, dtype);
    if (dtype == GAO_F32) ((uint32_t *)base)[i] = b;
    else ((uint16_t *)base)[i] = (uint16_t)b;
}

/* tanh-approximate GELU: 0.5 s (1 + tanh( sqrt(2/pi) (s + 0.044715 s^3) )). */
double gao_gelu_tanh(double s)
{
    const double k = sqrt(2.0 / M_PI);
    return 0.5 * s * (1.0 + tanh(k * (s + 0.044715 * s * s * s)));
}

/* Exact GELU: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)). */
double gao_gelu_erf(double x)
{
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

/* Squared ReLU: max(x, 0)^2. */
double gao_squared_relu(double x)
{
    const double r = x > 0.0 ? x : 0.0;
    return r * r;
}

/* SiLU: x * sigmoid(x) = x / (1 + e^-x). */
double gao_silu(double x)
{
    return x / (1.0 + exp(-x));
}

/* Per-row statistics of the gate: mean = sum/d, population variance =
 * sum (g - mean)^2 / d (second pass over the row), std = sqrt(variance). */
void gao_row_stats(const double *g, int64_t d, double *mean, double *std)
{
    double s = 0.0;
    for (int64_t i = 0; i < d; ++i) s += g[i];
    const double mu = s / (double)d;
    double q = 0.0;
    for (int64_t i = 0; i < d; ++i) q += (g[i] - mu) * (g[i] - mu);
    *mean = mu;
    *std = sqrt(q / (double)d);
}

static int64_t clamp_live(int64_t live, int64_t rows)
{
    return live < 0 ? 0 : (live > rows ? rows : live);
}

/* Sparse GELU-and-multiply over rows [0, live) of in[T, 2d] (gate = columns
 * [0, d), up = columns [d, 2d)); out[T, d].  Rows >= live are not written.
 * Optional outputs (any may be NULL): out_f64[T*d] = the unrounded product,
 * row_mean / row_std / row_cut [T] = the per-row statistics and cutoff.
 * Returns 0, or -1 on bad arguments. */
int gao_gelu_and_mul_sparse(const void *in, void *out, int64_t T, int64_t d,
                            int dtype, float z, int64_t live, double *out_f64,
                            double *row_mean, double *row_std, double *row_cut)
{
    if (!in || !out || T < 0 || d < 1 || !gao_elem_size(dtype)) return -1;
    const int64_t n = clamp_live(live, T);
    double *g = (double *)malloc(sizeof(double) * (size_t)d);
    if (!g) return -1;
    for (int64_t r = 0; r < n; ++r) {
        const int64_t row = r * 2 * d;
        for (int64_t i = 0; i < d; ++i) g[i] = load_elem(in, row + i, dtype);
        double mean, std;
        gao_row_stats(g, d, &mean, &std);
        const double cut = mean + (double)z * std;
        if (row_mean) row_mean[r] = mean;
        if (row_std) row_std[r] = std;
        if (row_cut) row_cut[r] = cut;
        for (int64_t i = 0; i < d; ++i) {
            double s = g[i] - cut;
            if (!(s > 0.0)) s = 0.0;                 /* relu */
            const double up = load_elem(in, row + d + i, dtype);
            const double y = gao_gelu_tanh(s) * up;
            if (out_f64) out_f64[r * d + i] = y;
            store_elem(out, r * d + i, dtype, y);
        }
    }
    free(g);
    return 0;
}

/* Round a double to the element type and back (the value a tensor of that
 * type would hold). */
static double round_to(double v, int dtype)
{
    return gao_decode(gao_encode_rne(v, dtype), dtype);
}

/* Sparse GELU-and-multiply in "round-trip" form: the native composition of
 * the op keeps every intermediate tensor in the input type (vLLM PR 48498,
 * Test Result, "Cross-architecture warp and dtype validation": the Triton
 * kernel rounds intermediates to reproduce native PyTorch's rounding at
 * operation boundaries).  Reading taken: each of mean, std, z, z * std,
 * cutoff = mean + z * std, gate - cutoff, gelu_tanh(.) and the product is
 * rounded to the element type; each step is computed exactly (in double)
 * from already-rounded operands.  cut_in (may be NULL): per-row cutoffs to
 * use instead of computing them (already in the element type).
 * Optional outputs: row_mean / row_std (exact, before rounding), row_cut
 * (the rounded cutoff used). */
int gao_gelu_and_mul_sparse_rt(const void *in, void *out, int64_t T, int64_t d, int dtype, float z,
                               int64_t live, const double *cut_in, double *row_mean, double *row_std,
                               double *row_cut)
{
    if (!in || !out || T < 0 || d < 1 || !gao_elem_size(dtype)) return -1;
    const int64_t n = clamp_live(live, T);
    double *g = (double *)malloc(sizeof(double) * (size_t)d);
    if (!g) return -1;
    for (int64_t r = 0; r < n; ++r) {
        const int64_t row = r * 2 * d;
        for (int64_t i = 0; i < d; ++i) g[i] = load_elem(in, row + i, dtype);
        double mean, std;
        gao_row_stats(g, d, &mean, &std);
        double cut;
        if (cut_in) {
            cut = cut_in[r];
        } else {
            const double mean_t = round_to(mean, dtype);
            const double std_t = round_to(std, dtype);
            const double z_t = round_to((double)z, dtype);
            const double zs_t = round_to(z_t * std_t, dtype);
            cut = round_to(mean_t + zs_t, dtype);
        }
        if (row_mean) row_mean[r] = mean;
        if (row_std) row_std[r] = std;
        if (row_cut) row_cut[r] = cut;
        for (int64_t i = 0; i < d; ++i) {
            double s = round_to(g[i] - cut, dtype);
            if (!(s > 0.0)) s = 0.0;                 /* relu */
            const double h = round_to(gao_gelu_tanh(s), dtype);
            const double up = load_elem(in, row + d + i, dtype);
            store_elem(out, r * d + i, dtype, h * up);
        }
    }
    free(g);
    return 0;
}

/* Bounded SiLU-and-multiply: rows [0, clamp(live, 0, M)) of in[M, 2d] give
 * out[r, i] = silu(gate) * up; rows beyond the live count are not written. */
int gao_silu_and_mul_bounded(const void *in, void *out, int64_t M, int64_t d,
                             int dtype, int64_t live, double *out_f64)
{
    if (!in || !out || M < 0 || d < 1 || !gao_elem_size(dtype)) return -1;
    const int64_t n = clamp_live(live, M);
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t i = 0; i < d; ++i) {
            const double gate = load_elem(in, r * 2 * d + i, dtype);
            const double up = load_elem(in, r * 2 * d + d + i, dtype);
            const double y = gao_silu(gate) * up;
            if (out_f64) out_f64[r * d + i] = y;
            store_elem(out, r * d + i, dtype, y);
        }
    }
    return 0;
}

/* GELU-and-multiply without the sparsity step: out = gelu(gate) * up on rows
 * [0, clamp(live, 0, T)) of in[T, 2d]; approximate != 0 selects the tanh
 * form, 0 the exact erf form.  Rows beyond the live count are not written. */
int gao_gelu_and_mul(const void *in, void *out, int64_t T, int64_t d, int dtype,
                     int approximate, int64_t live, double *out_f64)
{
    if (!in || !out || T < 0 || d < 1 || !gao_elem_size(dtype)) return -1;
    const int64_t n = clamp_live(live, T);
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t i = 0; i < d; ++i) {
            const double gate = load_elem(in, r * 2 * d + i, dtype);
            const double up = load_elem(in, r * 2 * d + d + i, dtype);
            const double act = approximate ? gao_gelu_tanh(gate) : gao_gelu_erf(gate);
            const double y = act * up;
            if (out_f64) out_f64[r * d + i] = y;
            store_elem(out, r * d + i, dtype, y);
        }
    }
    return 0;
}

/* Sparse GELU-and-multiply followed by the layer's down projection: the
 * matrix product that consumes the activation (the vLLM page, Test Result,
 * Correctness: the standalone regression keeps the upstream projection, the
 * activation's write and the downstream projection in that order).  For each
 * live row r < clamp(live, 0, T) and output feature h < H:
 *     a[r, k] = gelu_and_mul_sparse(gu)[r, k]   as stored: rounded once
 *     y[r, h] = sum over k of a[r, k] * w[h, k]  in double, rounded once
 * gu is [T, 2d], w is [H, d] row-major (one row of d weights per output
 * feature, a linear layer's layout), y is [T, H].  y_f64 (may be NULL) gets
 * the unrounded sums and abs_f64 (may be NULL) the sums of |a[r,k] w[h,k]|
 * (the scale of any rounding error in the sum).  Rows beyond the live count
 * are not written. */
int gao_gelu_and_mul_sparse_down(const void *gu, const void *w, void *y, int64_t T, int64_t d,
                                 int64_t H, int dtype, float z, int64_t live, double *y_f64,
                                 double *abs_f64)
{
    if (!gu || !w || !y || T < 0 || d < 1 || H < 1 || !gao_elem_size(dtype)) return -1;
    const int64_t n = clamp_live(live, T);
    if (n == 0) return 0;
    const size_t es = gao_elem_size(dtype);
    void *a_bits = malloc(es * (size_t)(n * d));
    double *a = (double *)malloc(sizeof(double) * (size_t)(n * d));
    double *wrow = (double *)malloc(sizeof(double) * (size_t)d);
    int rc = -1;
    if (!a_bits || !a || !wrow) goto done;
    /* the activation, exactly as its own op stores it */
    if (gao_gelu_and_mul_sparse(gu, a_bits, n, d, dtype, z, n, NULL, NULL, NULL, NULL)) goto done;
    for (int64_t i = 0; i < n * d; ++i) a[i] = load_elem(a_bits, i, dtype);
    for (int64_t h = 0; h < H; ++h) {
        for (int64_t k = 0; k < d; ++k) wrow[k] = load_elem(w, h * d + k, dtype);
        for (int64_t r = 0; r < n; ++r) {
            double s = 0.0, m = 0.0;
            for (int64_t k = 0; k < d; ++k) {
                s += a[r * d + k] * wrow[k];
                m += fabs(a[r * d + k] * wrow[k]);
            }
            if (y_f64) y_f64[r * H + h] = s;
            if (abs_f64) abs_f64[r * H + h] = m;
            store_elem(y, r * H + h, dtype, s);
        }
    }
    rc = 0;
done:
    free(a_bits);
    free(a);
    free(wrow);
    return rc;
}

/* Bounded squared ReLU (not gated): in[M, d] -> out[M, d] = max(x, 0)^2 on
 * rows [0, clamp(live, 0, M)); the other rows are not written. */
int gao_squared_relu_bounded(const void *in, void *out, int64_t M, int64_t d, int dtype,
                             int64_t live, double *out_f64)
{
    if (!in || !out || M < 0 || d < 1 || !gao_elem_size(dtype)) return -1;
    const int64_t n = clamp_live(live, M);
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t i = 0; i < d; ++i) {
            const double y = gao_squared_relu(load_elem(in, r * d + i, dtype));
            if (out_f64) out_f64[r * d + i] = y;
            store_elem(out, r * d + i, dtype, y);
        }
    }
    return 0;
}

/* Array helpers so the pins can test each step over many points at once. */
void gao_decode_array(const void *bits, int64_t n, int dtype, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = load_elem(bits, i, dtype);
}

void gao_encode_array(const double *v, int64_t n, int dtype, void *bits)
{
    for (int64_t i = 0; i < n; ++i) store_elem(bits, i, dtype, v[i]);
}

void gao_gelu_tanh_array(const double *s, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = gao_gelu_tanh(s[i]);
}

void gao_silu_array(const double *x, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = gao_silu(x[i]);
}

void gao_gelu_erf_array(const double *x, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = gao_gelu_erf(x[i]);
}

void gao_squared_relu_array(const double *x, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = gao_squared_relu(x[i]);
}
