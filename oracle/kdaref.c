/*
 * kdaref.c -- fp64 CPU oracle for the Kimi Delta Attention (KDA) operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this file.  Only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark use it.
 * It shares no code, header, table or helper with the HIP path.
 *
 * What it computes, and where the pages define it:
 *
 *  - State update, "Kimi Linear: An Expressive, Efficient Attention
 *    Architecture" (tech report), section 3, Eq. 1:
 *        S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *    with S_t of shape d_k x d_v, and the readout o_t = S_t^T q_t.  The same
 *    equation appears in "Diagonal-Plus-Low-Rank Matrices and Kimi Delta
 *    Attention", section 2, and in the "KDA Recurrence" problem statement.
 *
 *  - The token step is evaluated in the order of the fused recurrent decode
 *    kernel described in the agentlenshq blog "Kimi Delta Attention builds on
 *    DeltaNet with per-channel forgetting" (section on efficient execution):
 *    decay the state, predict p = S'^T k, form the residual r = beta (v - p),
 *    add k r^T, then read out.  With S' = Diag(alpha) S this is Eq. 1
 *    rearranged without any approximation:
 *        (I - b k k^T) S' + b k v^T = S' + k (b (v - S'^T k))^T.
 *
 *  - Decay parametrisation, "KDA Recurrence" problem statement:
 *        alpha_t = exp(g_min * sigmoid(z_t)),  g_min < 0,
 *    one decay logit per key channel.
 *
 *  - Readout from the UPDATED state (o_t = S_t^T q_t, not S_{t-1}), "KDA
 *    Recurrence" problem statement.  No extra query scale is applied here:
 *    q is used exactly as given.
 *
 *  - Output epilogue, "KDA Recurrence" problem statement and its first worked
 *    example: per (batch, token, head) RMS normalisation over the d_v values
 *    with eps inside the square root and no learnable weight, times
 *    sigmoid(output-gate logit), heads concatenated to width H*d_v, then the
 *    supplied projection W of shape (d_model, H*d_v):  out = y W^T, no bias.
 *
 * All arithmetic is IEEE double.  Inputs may be given as double, float or
 * bfloat16 bit patterns; each is widened exactly to double before use.
 * Build with -O2 -ffp-contract=off so that no fused multiply-add changes the
 * rounding order written here.
 *
 * Tensor layouts (contiguous, row-major):
 *   q, k, z      (B, T, H, d_k)
 *   v            (B, T, H, d_v)
 *   beta         (B, T, H)
 *   s0, s_final  (B, H, d_k, d_v)
 *   o            (B, T, H, d_v)       written as double
 *   gate         (B, T, H, d_v)
 *   W            (d_model, H*d_v)
 *   out          (B, T, d_model) or (B, T, H*d_v) when W is NULL
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { REF_F64 = 0, REF_F32 = 1, REF_BF16 = 2 };

/* Widen element idx of a tensor stored in the given dtype to double. */
static double ref_load(const void* p, int dtype, size_t idx) {
    if (dtype == REF_F64) return ((const double*)p)[idx];
    if (dtype == REF_F32) return (double)((const float*)p)[idx];
    /* bfloat16: the upper 16 bits of an IEEE binary32. */
    uint32_t bits = ((uint32_t)((const uint16_t*)p)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int ref_dtype_ok(int dtype) {
    return dtype == REF_F64 || dtype == REF_F32 || dtype == REF_BF16;
}

/* ------------------------------------------------------------------------ */
/* Recurrence                                                                */
/* ------------------------------------------------------------------------ */

typedef struct {
    const void *q, *k, *v, *z, *beta, *s0;
    int dt_in, dt_s0;
    double g_min;
    double* o;
    double* s_final;
    int B, T, H, dk, dv;
    int nsplit;           /* d_v columns are cut into nsplit blocks */
    int units;            /* B * H * nsplit */
    int next;             /* next unit to claim */
    pthread_mutex_t lock;
} fwd_job;

/* One unit: batch b, head h, value columns [j0, j1).  The columns of S are
 * independent under Eq. 1 (the transition multiplies S only from the left),
 * so a column block can be run on its own. */
static void fwd_unit(fwd_job* jb, int unit) {
    const int dk = jb->dk, dv = jb->dv, H = jb->H, T = jb->T;
    const int bh = unit / jb->nsplit, part = unit % jb->nsplit;
    const int b = bh / H, h = bh % H;
    const int nb = dv / jb->nsplit;
    const int j0 = part * nb;

    double* S = (double*)malloc(sizeof(double) * (size_t)dk * nb);
    double* alpha = (double*)malloc(sizeof(double) * dk);
    double* kk = (double*)malloc(sizeof(double) * dk);
    double* qq = (double*)malloc(sizeof(double) * dk);
    double* p = (double*)malloc(sizeof(double) * nb);
    double* r = (double*)malloc(sizeof(double) * nb);

    /* S <- S0 (zeros when absent). */
    for (int c = 0; c < dk; ++c)
        for (int j = 0; j < nb; ++j) {
            size_t si = (((size_t)b * H + h) * dk + c) * dv + j0 + j;
            S[(size_t)c * nb + j] = jb->s0 ? ref_load(jb->s0, jb->dt_s0, si) : 0.0;
        }

    for (int t = 0; t < T; ++t) {
        const size_t tok = ((size_t)b * T + t) * H + h;   /* (b, t, h) row */
        const double beta = ref_load(jb->beta, jb->dt_in, tok);
        for (int c = 0; c < dk; ++c) {
            const double zc = ref_load(jb->z, jb->dt_in, tok * dk + c);
            const double sig = 1.0 / (1.0 + exp(-zc));
            alpha[c] = exp(jb->g_min * sig);
            kk[c] = ref_load(jb->k, jb->dt_in, tok * dk + c);
            qq[c] = ref_load(jb->q, jb->dt_in, tok * dk + c);
        }
        /* S' = Diag(alpha) S */
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < nb; ++j) S[(size_t)c * nb + j] *= alpha[c];
        /* p = S'^T k */
        for (int j = 0; j < nb; ++j) p[j] = 0.0;
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < nb; ++j) p[j] += S[(size_t)c * nb + j] * kk[c];
        /* r = beta (v - p) */
        for (int j = 0; j < nb; ++j)
            r[j] = beta * (ref_load(jb->v, jb->dt_in, tok * dv + j0 + j) - p[j]);
        /* S = S' + k r^T */
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < nb; ++j) S[(size_t)c * nb + j] += kk[c] * r[j];
        /* o_t = S_t^T q_t, read from the updated state */
        if (jb->o) {
            for (int j = 0; j < nb; ++j) p[j] = 0.0;
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < nb; ++j) p[j] += S[(size_t)c * nb + j] * qq[c];
            for (int j = 0; j < nb; ++j) jb->o[tok * dv + j0 + j] = p[j];
        }
    }

    if (jb->s_final)
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < nb; ++j)
                jb->s_final[(((size_t)b * H + h) * dk + c) * dv + j0 + j] = S[(size_t)c * nb + j];

    free(S); free(alpha); free(kk); free(qq); free(p); free(r);
}

static void* fwd_worker(void* arg) {
    fwd_job* jb = (fwd_job*)arg;
    for (;;) {
        pthread_mutex_lock(&jb->lock);
        int u = jb->next++;
        pthread_mutex_unlock(&jb->lock);
        if (u >= jb->units) break;
        fwd_unit(jb, u);
    }
    return NULL;
}

/* Run units [0, units) of a job on nthreads threads (the caller counts as
 * one of them). */
static void run_job(fwd_job* jb, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > jb->units) nthreads = jb->units;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, fwd_worker, jb) == 0) ++started;
    fwd_worker(jb);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
}

/*
 * kdaref_forward: the KDA recurrence over T tokens for every (batch, head).
 *   dt_in  dtype of q, k, v, z, beta (REF_F64 / REF_F32 / REF_BF16)
 *   dt_s0  dtype of s0 (REF_F64 / REF_F32); s0 may be NULL (zeros)
 *   o, s_final  double outputs; either may be NULL to skip it
 *   nthreads    worker threads (>= 1)
 * Returns 0 on success, a negative code on invalid arguments.
 */
int kdaref_forward(const void* q, const void* k, const void* v, const void* z,
                   const void* beta, int dt_in, double g_min,
                   const void* s0, int dt_s0, double* o, double* s_final,
                   int B, int T, int H, int dk, int dv, int nthreads) {
    if (!q || !k || !v || !z || !beta) return -1;
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1) return -2;
    if (!ref_dtype_ok(dt_in) || (s0 && dt_s0 != REF_F64 && dt_s0 != REF_F32)) return -3;
    if (B == 0 || H == 0) return 0;
    fwd_job jb;
    memset(&jb, 0, sizeof jb);
    jb.q = q; jb.k = k; jb.v = v; jb.z = z; jb.beta = beta; jb.s0 = s0;
    jb.dt_in = dt_in; jb.dt_s0 = dt_s0; jb.g_min = g_min;
    jb.o = o; jb.s_final = s_final;
    jb.B = B; jb.T = T; jb.H = H; jb.dk = dk; jb.dv = dv;
    /* Split d_v only as far as needed to give every thread a unit. */
    jb.nsplit = 1;
    while (B * H * jb.nsplit < nthreads && dv % (jb.nsplit * 2) == 0 && dv / (jb.nsplit * 2) >= 8)
        jb.nsplit *= 2;
    jb.units = B * H * jb.nsplit;
    pthread_mutex_init(&jb.lock, NULL);
    run_job(&jb, nthreads);
    pthread_mutex_destroy(&jb.lock);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Epilogue: RMSNorm x sigmoid gate, concat over heads, optional projection  */
/* ------------------------------------------------------------------------ */

typedef struct {
    const void *o, *gate, *w;
    int dt_o, dt_gate, dt_w;
    double eps;
    double* out;
    long rows;            /* B * T */
    int H, dv, d_model;
    long next;
    pthread_mutex_t lock;
} gate_job;

static void gate_row(gate_job* jb, long row, double* y) {
    const int H = jb->H, dv = jb->dv, width = H * dv;
    for (int h = 0; h < H; ++h) {
        const size_t base = ((size_t)row * H + h) * dv;
        double ss = 0.0;
        for (int j = 0; j < dv; ++j) {
            double x = ref_load(jb->o, jb->dt_o, base + j);
            ss += x * x;
        }
        const double inv = 1.0 / sqrt(ss / dv + jb->eps);
        for (int j = 0; j < dv; ++j) {
            double x = ref_load(jb->o, jb->dt_o, base + j);
            double g = ref_load(jb->gate, jb->dt_gate, base + j);
            double sig = 1.0 / (1.0 + exp(-g));
            y[h * dv + j] = x * inv * sig;
        }
    }
    if (!jb->w) {
        memcpy(jb->out + (size_t)row * width, y, sizeof(double) * (size_t)width);
        return;
    }
    /* out[row, m] = sum_c y[c] * W[m, c] */
    for (int m = 0; m < jb->d_model; ++m) {
        double acc = 0.0;
        for (int c = 0; c < width; ++c)
            acc += y[c] * ref_load(jb->w, jb->dt_w, (size_t)m * width + c);
        jb->out[(size_t)row * jb->d_model + m] = acc;
    }
}

static void* gate_worker(void* arg) {
    gate_job* jb = (gate_job*)arg;
    double* y = (double*)malloc(sizeof(double) * (size_t)jb->H * jb->dv);
    for (;;) {
        pthread_mutex_lock(&jb->lock);
        long r = jb->next;
        jb->next += 16;
        pthread_mutex_unlock(&jb->lock);
        if (r >= jb->rows) break;
        long r1 = r + 16 < jb->rows ? r + 16 : jb->rows;
        for (; r < r1; ++r) gate_row(jb, r, y);
    }
    free(y);
    return NULL;
}

/*
 * kdaref_out_gate: out = concat_h( RMSNorm(o_h) * sigmoid(gate_h) ) W^T.
 *   o      (B, T, H, dv) in dt_o
 *   gate   (B, T, H, dv) in dt_gate
 *   w      (d_model, H*dv) in dt_w, or NULL: out is then (B, T, H*dv)
 *   out    double
 * Returns 0 on success, a negative code on invalid arguments.
 */
int kdaref_out_gate(const void* o, int dt_o, const void* gate, int dt_gate,
                    double eps, const void* w, int dt_w, double* out,
                    int B, int T, int H, int dv, int d_model, int nthreads) {
    if (!o || !gate || !out) return -1;
    if (B < 0 || T < 0 || H < 1 || dv < 1 || (w && d_model < 1)) return -2;
    if (!ref_dtype_ok(dt_o) || !ref_dtype_ok(dt_gate) || (w && !ref_dtype_ok(dt_w))) return -3;
    gate_job jb;
    memset(&jb, 0, sizeof jb);
    jb.o = o; jb.gate = gate; jb.w = w;
    jb.dt_o = dt_o; jb.dt_gate = dt_gate; jb.dt_w = dt_w;
    jb.eps = eps; jb.out = out;
    jb.rows = (long)B * T; jb.H = H; jb.dv = dv; jb.d_model = d_model;
    if (jb.rows == 0) return 0;
    pthread_mutex_init(&jb.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    long maxt = (jb.rows + 15) / 16;
    if (nthreads > maxt) nthreads = (int)maxt;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, gate_worker, &jb) == 0) ++started;
    gate_worker(&jb);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&jb.lock);
    return 0;
}
