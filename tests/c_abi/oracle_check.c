/* Drives the C oracle (oracle/kdaref.c) through its entry points on small
 * inputs, for a build under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every dtype, a ragged head count, several threads, the epilogue with and
 * without projection, and the argument errors.  The one-token case is checked
 * against its closed form: from S0 = 0, S_1 = beta k v^T, so
 * o_1 = beta (k . q) v. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kdaref_forward(const void* q, const void* k, const void* v, const void* z, const void* beta, int dt_in,
                   double g_min, const void* s0, int dt_s0, double* o, double* s_final, int B, int T, int H,
                   int dk, int dv, int nthreads);
int kdaref_out_gate(const void* o, int dt_o, const void* gate, int dt_gate, double eps, const void* w, int dt_w,
                    double* out, int B, int T, int H, int dv, int d_model, int nthreads);

enum { F64 = 0, F32 = 1, BF16 = 2 };

static int failures = 0;
#define CHECK(c)                                                     \
    do {                                                             \
        if (!(c)) {                                                  \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                              \
        }                                                            \
    } while (0)

static double urand(unsigned* s) {
    *s = *s * 1664525u + 1013904223u;
    return ((*s >> 8) / 16777216.0) * 2.0 - 1.0;
}

static uint16_t to_bf16(float f) {   /* truncation is enough for test inputs */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int main(void) {
    const int B = 2, T = 37, H = 3, dk = 8, dv = 6, d_model = 5;
    const size_t nk = (size_t)B * T * H * dk, nv = (size_t)B * T * H * dv, nb = (size_t)B * T * H;
    unsigned seed = 12345u;
    double *q = malloc(nk * 8), *k = malloc(nk * 8), *z = malloc(nk * 8), *v = malloc(nv * 8), *beta = malloc(nb * 8);
    double* s0 = malloc((size_t)B * H * dk * dv * 8);
    for (size_t i = 0; i < nk; ++i) {
        q[i] = 0.3 * urand(&seed);
        k[i] = 0.3 * urand(&seed);
        z[i] = urand(&seed);
    }
    for (size_t i = 0; i < nv; ++i) v[i] = urand(&seed);
    for (size_t i = 0; i < nb; ++i) beta[i] = 0.5 + 0.4 * urand(&seed);
    for (size_t i = 0; i < (size_t)B * H * dk * dv; ++i) s0[i] = 0.1 * urand(&seed);

    double* o = malloc(nv * 8);
    double* sf = malloc((size_t)B * H * dk * dv * 8);
    for (int nt = 1; nt <= 4; nt *= 2) {
        CHECK(kdaref_forward(q, k, v, z, beta, F64, -5.0, s0, F64, o, sf, B, T, H, dk, dv, nt) == 0);
        CHECK(kdaref_forward(q, k, v, z, beta, F64, -5.0, NULL, F64, o, NULL, B, T, H, dk, dv, nt) == 0);
        CHECK(kdaref_forward(q, k, v, z, beta, F64, -5.0, s0, F64, NULL, sf, B, T, H, dk, dv, nt) == 0);
    }
    /* fp32 and bf16 copies of the same inputs */
    float *qf = malloc(nk * 4), *kf = malloc(nk * 4), *zf = malloc(nk * 4), *vf = malloc(nv * 4), *bf = malloc(nb * 4);
    float* s0f = malloc((size_t)B * H * dk * dv * 4);
    uint16_t *qh = malloc(nk * 2), *kh = malloc(nk * 2), *zh = malloc(nk * 2), *vh = malloc(nv * 2), *bh = malloc(nb * 2);
    for (size_t i = 0; i < nk; ++i) {
        qf[i] = (float)q[i], kf[i] = (float)k[i], zf[i] = (float)z[i];
        qh[i] = to_bf16(qf[i]), kh[i] = to_bf16(kf[i]), zh[i] = to_bf16(zf[i]);
    }
    for (size_t i = 0; i < nv; ++i) vf[i] = (float)v[i], vh[i] = to_bf16(vf[i]);
    for (size_t i = 0; i < nb; ++i) bf[i] = (float)beta[i], bh[i] = to_bf16(bf[i]);
    for (size_t i = 0; i < (size_t)B * H * dk * dv; ++i) s0f[i] = (float)s0[i];
    CHECK(kdaref_forward(qf, kf, vf, zf, bf, F32, -5.0, s0f, F32, o, sf, B, T, H, dk, dv, 3) == 0);
    CHECK(kdaref_forward(qh, kh, vh, zh, bh, BF16, -5.0, s0, F64, o, sf, B, T, H, dk, dv, 3) == 0);

    /* one token from S0 = 0: o = beta (k . q) v */
    CHECK(kdaref_forward(q, k, v, z, beta, F64, -5.0, NULL, F64, o, sf, 1, 1, 1, dk, dv, 1) == 0);
    double kq = 0.0;
    for (int c = 0; c < dk; ++c) kq += k[c] * q[c];
    for (int j = 0; j < dv; ++j) CHECK(fabs(o[j] - beta[0] * kq * v[j]) < 1e-14);

    /* epilogue, with and without projection */
    double* gate = malloc(nv * 8);
    double* w = malloc((size_t)d_model * H * dv * 8);
    double* y = malloc((size_t)B * T * (H * dv > d_model ? H * dv : d_model) * 8);
    for (size_t i = 0; i < nv; ++i) gate[i] = urand(&seed);
    for (size_t i = 0; i < (size_t)d_model * H * dv; ++i) w[i] = 0.2 * urand(&seed);
    CHECK(kdaref_forward(q, k, v, z, beta, F64, -5.0, s0, F64, o, sf, B, T, H, dk, dv, 2) == 0);
    CHECK(kdaref_out_gate(o, F64, gate, F64, 1e-6, NULL, F64, y, B, T, H, dv, 0, 2) == 0);
    CHECK(kdaref_out_gate(o, F64, gate, F64, 1e-6, w, F64, y, B, T, H, dv, d_model, 3) == 0);
    CHECK(kdaref_out_gate(o, F64, gate, F64, 1e-6, NULL, F64, y, 0, T, H, dv, 0, 2) == 0);

    /* argument errors */
    CHECK(kdaref_forward(NULL, k, v, z, beta, F64, -5.0, NULL, F64, o, sf, B, T, H, dk, dv, 1) < 0);
    CHECK(kdaref_forward(q, k, v, z, beta, 7, -5.0, NULL, F64, o, sf, B, T, H, dk, dv, 1) < 0);
    CHECK(kdaref_forward(q, k, v, z, beta, F64, -5.0, NULL, F64, o, sf, -1, T, H, dk, dv, 1) < 0);
    CHECK(kdaref_forward(q, k, v, z, beta, F64, -5.0, NULL, F64, o, sf, 0, T, H, dk, dv, 1) == 0);
    CHECK(kdaref_out_gate(NULL, F64, gate, F64, 1e-6, NULL, F64, y, B, T, H, dv, 0, 1) < 0);

    free(q), free(k), free(z), free(v), free(beta), free(s0), free(o), free(sf);
    free(qf), free(kf), free(zf), free(vf), free(bf), free(s0f);
    free(qh), free(kh), free(zh), free(vh), free(bh);
    free(gate), free(w), free(y);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
