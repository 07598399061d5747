/* Host driver for the sanitizer build of the CPU oracle (test
 * infrastructure; built and run by tests/test_oracle_sanitized.py).  Every
 * entry point of oracle/ga_oracle.c runs on exactly sized heap buffers over
 * small shapes, live counts below, at and past the row count, and all three
 * element types, so that AddressSanitizer sees any access past a buffer and
 * UndefinedBehaviorSanitizer any undefined arithmetic.  Prints "ok". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

size_t gao_elem_size(int dtype);
double gao_decode(uint32_t bits, int dtype);
uint32_t gao_encode_rne(double v, int dtype);
int gao_gelu_and_mul_sparse(const void *in, void *out, int64_t T, int64_t d, int dtype, float z, int64_t live,
                            double *out_f64, double *row_mean, double *row_std, double *row_cut);
int gao_gelu_and_mul_sparse_rt(const void *in, void *out, int64_t T, int64_t d, int dtype, float z,
                               int64_t live, const double *cut_in, double *row_mean, double *row_std,
                               double *row_cut);
int gao_silu_and_mul_bounded(const void *in, void *out, int64_t M, int64_t d, int dtype, int64_t live,
                             double *out_f64);
int gao_gelu_and_mul(const void *in, void *out, int64_t T, int64_t d, int dtype, int approximate, int64_t live,
                     double *out_f64);
int gao_squared_relu_bounded(const void *in, void *out, int64_t M, int64_t d, int dtype, int64_t live,
                             double *out_f64);
void gao_decode_array(const void *bits, int64_t n, int dtype, double *out);
void gao_encode_array(const double *v, int64_t n, int dtype, void *bits);

static uint64_t state = 0x9E3779B97F4A7C15ull;

static double next_normal(void) {
    /* splitmix64 -> two uniforms -> Box-Muller (one output) */
    double u[2];
    for (int k = 0; k < 2; ++k) {
        uint64_t x = (state += 0x9E3779B97F4A7C15ull);
        x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
        x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
        x ^= x >> 31;
        u[k] = ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    }
    return sqrt(-2.0 * log(u[0])) * cos(6.283185307179586 * u[1]);
}

static void *random_rows(int64_t n, int dtype, double scale) {
    const size_t es = gao_elem_size(dtype);
    unsigned char *p = (unsigned char *)malloc(n > 0 ? (size_t)n * es : 1);
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t b = gao_encode_rne(scale * next_normal(), dtype);
        memcpy(p + (size_t)i * es, &b, es); /* little-endian: the low bytes hold the pattern */
    }
    return p;
}

static int failures = 0;
#define EXPECT(c) do { if (!(c)) { printf("FAILED line %d: %s\n", __LINE__, #c); ++failures; } } while (0)

int main(void) {
    static const int64_t ds[] = {1, 2, 7, 8, 31, 257};
    static const int64_t Ts[] = {0, 1, 5};
    for (int dtype = 0; dtype <= 2; ++dtype) {
        const size_t es = gao_elem_size(dtype);
        for (size_t di = 0; di < sizeof ds / sizeof ds[0]; ++di) {
            for (size_t ti = 0; ti < sizeof Ts / sizeof Ts[0]; ++ti) {
                const int64_t d = ds[di], T = Ts[ti];
                void *in = random_rows(T * 2 * d, dtype, 1.5);
                void *in1 = random_rows(T * d, dtype, 1.5);
                void *out = malloc(T > 0 ? (size_t)(T * d) * es : 1);
                double *f64 = (double *)malloc(T > 0 ? sizeof(double) * (size_t)(T * d) : 1);
                double *mean = (double *)malloc(T > 0 ? sizeof(double) * (size_t)T : 1);
                double *sd = (double *)malloc(T > 0 ? sizeof(double) * (size_t)T : 1);
                double *cut = (double *)malloc(T > 0 ? sizeof(double) * (size_t)T : 1);
                const int64_t lives[] = {-3, 0, T / 2, T, T + 5};
                for (size_t li = 0; li < 5; ++li) {
                    const int64_t live = lives[li];
                    EXPECT(gao_gelu_and_mul_sparse(in, out, T, d, dtype, 1.6448536f, live, f64, mean, sd, cut) == 0);
                    EXPECT(gao_gelu_and_mul_sparse(in, out, T, d, dtype, 0.0f, live, NULL, NULL, NULL, NULL) == 0);
                    EXPECT(gao_gelu_and_mul_sparse_rt(in, out, T, d, dtype, 2.3263479f, live, NULL, mean, sd, cut) == 0);
                    EXPECT(gao_gelu_and_mul_sparse_rt(in, out, T, d, dtype, 1.6448536f, live, cut, NULL, NULL, NULL) == 0);
                    EXPECT(gao_silu_and_mul_bounded(in, out, T, d, dtype, live, f64) == 0);
                    EXPECT(gao_gelu_and_mul(in, out, T, d, dtype, 1, live, f64) == 0);
                    EXPECT(gao_gelu_and_mul(in, out, T, d, dtype, 0, live, NULL) == 0);
                    EXPECT(gao_squared_relu_bounded(in1, out, T, d, dtype, live, f64) == 0);
                }
                free(in); free(in1); free(out); free(f64); free(mean); free(sd); free(cut);
            }
        }
        /* rejected arguments */
        unsigned char buf[64] = {0};
        EXPECT(gao_gelu_and_mul_sparse(NULL, buf, 1, 4, dtype, 1.0f, 1, NULL, NULL, NULL, NULL) == -1);
        EXPECT(gao_gelu_and_mul_sparse(buf, buf, -1, 4, dtype, 1.0f, 1, NULL, NULL, NULL, NULL) == -1);
        EXPECT(gao_silu_and_mul_bounded(buf, buf, 1, 0, dtype, 1, NULL) == -1);
        EXPECT(gao_gelu_and_mul(buf, buf, 1, 4, 7, 1, 1, NULL) == -1);
    }
    /* the codecs over every 16-bit pattern and special values */
    {
        uint16_t *bits = (uint16_t *)malloc(sizeof(uint16_t) * 65536);
        double *v = (double *)malloc(sizeof(double) * 65536);
        uint16_t *back = (uint16_t *)malloc(sizeof(uint16_t) * 65536);
        for (int i = 0; i < 65536; ++i) bits[i] = (uint16_t)i;
        for (int dtype = 1; dtype <= 2; ++dtype) {
            gao_decode_array(bits, 65536, dtype, v);
            gao_encode_array(v, 65536, dtype, back);
            for (int i = 0; i < 65536; ++i)
                if (!isnan(v[i])) EXPECT(back[i] == bits[i] || (v[i] == 0.0 && (back[i] & 0x7FFF) == 0));
        }
        free(bits); free(v); free(back);
        const double specials[] = {0.0, -0.0, INFINITY, -INFINITY, NAN, 1e308, -1e308, 1e-310, 5e-324,
                                   65504.0, 65520.0, 3.4028234663852886e38, 3.5e38, 1e-45, 1.401298464324817e-45};
        for (int dtype = 0; dtype <= 2; ++dtype)
            for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i) {
                const uint32_t b = gao_encode_rne(specials[i], dtype);
                (void)gao_decode(b, dtype);
            }
    }
    if (failures == 0) printf("ok\n");
    return failures == 0 ? 0 : 1;
}
