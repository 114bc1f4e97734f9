/* Drives every oracle function once on small inputs; built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by the test suite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_sumsq_accum(double state[2], const float *g, int64_t n);
double oracle_sumsq_finish(const double state[2]);
double oracle_grad_norm(const float *g, int64_t n);
float oracle_clip_scale(double norm, float clip);
void oracle_scalars(int32_t t, float lr, float wd, float *bc1, float *bc2, float *decay);
void oracle_adamw_elems(float *w, const float *g, float *m, float *v, int64_t n, float s,
                        float bc1, float bc2, float decay, float lr);
void oracle_scale_grads(float *g, int64_t n, float scale);
int oracle_adamw_clip_step(float *w, const float *g, float *m, float *v, int64_t n, int32_t t,
                           float lr, float wd, float clip, double *norm_out);
int oracle_adamw_clip_step_f64(double *w, const double *g, double *m, double *v, int64_t n,
                               int32_t t, double lr, double wd, double clip, double *norm_out);
int64_t oracle_ckpt_bytes(int64_t n);
int oracle_ckpt_pack(int32_t step, int64_t n, const float *w, const float *m, const float *v,
                     uint8_t *buf, int64_t len);
int oracle_ckpt_header(const uint8_t *buf, int64_t len, int32_t *step, int32_t *n);
int oracle_ckpt_unpack(const uint8_t *buf, int64_t len, int64_t n_expected, int32_t *step_out,
                       float *w, float *m, float *v);
int oracle_subnormals_kept(void);

#define N 1003
#define EXPECT(c)                                                   \
    do {                                                            \
        if (!(c)) {                                                 \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #c);  \
            return 1;                                               \
        }                                                           \
    } while (0)

int main(void) {
    float *w = malloc(N * 4), *g = malloc(N * 4), *m = calloc(N, 4), *v = calloc(N, 4);
    float *w2 = malloc(N * 4), *m2 = malloc(N * 4), *v2 = malloc(N * 4);
    for (int i = 0; i < N; ++i) {
        w[i] = 0.02f * (float)((i % 17) - 8);
        g[i] = 0.3f * (float)((i % 29) - 14);
    }
    double norm = 0.0;
    EXPECT(oracle_adamw_clip_step(w, g, m, v, N, 1, 3e-3f, 0.01f, 1.0f, &norm) == 0);
    EXPECT(norm > 1.0 && isfinite(norm));
    double st[2] = {0.0, 0.0};
    oracle_sumsq_accum(st, g, 500);
    oracle_sumsq_accum(st, g + 500, N - 500);
    EXPECT(sqrt(oracle_sumsq_finish(st)) == oracle_grad_norm(g, N));
    float bc1, bc2, decay;
    oracle_scalars(2, 3e-3f, 0.01f, &bc1, &bc2, &decay);
    oracle_adamw_elems(w, g, m, v, N, oracle_clip_scale(norm, 1.0f), bc1, bc2, decay, 3e-3f);
    oracle_scale_grads(g, N, 0.5f);
    double w64 = 2.0, g64 = 0.5, m64 = 0.0, v64 = 0.0, n64 = 0.0;
    EXPECT(oracle_adamw_clip_step_f64(&w64, &g64, &m64, &v64, 1, 1, 0.1, 0.01, 1.0, &n64) == 0);
    EXPECT(fabs(w64 - 1.898) < 1e-7 && n64 == 0.5);
    const int64_t len = oracle_ckpt_bytes(N);
    uint8_t *buf = malloc((size_t)len);
    EXPECT(oracle_ckpt_pack(7, N, w, m, v, buf, len) == 0);
    int32_t step = -1, n = -1;
    EXPECT(oracle_ckpt_header(buf, len, &step, &n) == 0 && step == 7 && n == N);
    EXPECT(oracle_ckpt_unpack(buf, len, N, &step, w2, m2, v2) == 0);
    EXPECT(memcmp(w, w2, N * 4) == 0 && memcmp(m, m2, N * 4) == 0 && memcmp(v, v2, N * 4) == 0);
    EXPECT(oracle_ckpt_unpack(buf, len - 1, N, &step, w2, m2, v2) == -2);
    EXPECT(oracle_ckpt_unpack(buf, 7, N, &step, w2, m2, v2) == -2);
    EXPECT(oracle_subnormals_kept() == 1);
    free(w); free(g); free(m); free(v); free(w2); free(m2); free(v2); free(buf);
    printf("oracle driver ok\n");
    return 0;
}
