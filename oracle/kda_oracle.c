/*
 * Plain fp64 CPU oracle for the Kimi Delta Attention (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do. It shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes (per batch b and head h, state S of shape dk x dv):
 *
 *   g_t   <- g_t clamped to [-5, 0]          (the decay floor: "K3 tech report"
 *                                              transcript, the exchange on the
 *                                              lower log-decay bound of minus five;
 *                                              "Kimi K3 goes trillion-scale ..."
 *                                              subtitles, cue 14: the floored,
 *                                              lower-bounded sigmoid decay)
 *   P     =  Diag(exp(g_t)) S                (channel-wise forgetting, one factor
 *                                              per key channel = per row of S)
 *   u     =  beta_t (v_t - P^T k_t)          (delta rule: write strength times
 *                                              prediction error)
 *   S     =  P + k_t u^T                     == (I - beta k k^T) Diag(e^g) S + beta k v^T
 *   o_t   =  S^T q_t                         (read after the write, no scaling)
 *
 * The delta rule with channel-wise forget gate and fixed-size state is the one
 * described in "177: Kimi K3 in Detail", section 15, and in the same subtitle
 * cue 14. Every step is taken in the order written above, one token at a time,
 * in double precision. NaN in any input propagates (the clamp compares, it does
 * not use fmin/fmax).
 *
 * Gate option (gate = 1): g holds raw gate logits x instead of log-decays, and
 * the log-decay is -5 sigmoid(x) = -5 / (1 + exp(-x)) before the clamp (which
 * then only passes NaN). The pages state the bound (retention floored at
 * e^-5, a "lower-bounded sigmoid" decay) but not the formula; a sigmoid
 * scaled to the bound is the reading taken (same subtitle cue 14).
 *
 * Inputs may be fp32 or bf16 bit patterns; they are widened to double exactly.
 * Layout: q, k, g are [B, T, H, dk]; v is [B, T, H, dv]; beta is [B, T, H];
 * S0 and S_T are [B, H, dk, dv] (double); o is [B, T, H, dv] (double).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_GATE_LOG_DECAY 0
#define ORACLE_GATE_SIGMOID 1

static double widen(const void* base, int dtype, size_t idx) {
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double clamp_decay(double x) {
    if (x < -5.0) return -5.0;
    if (x > 0.0) return 0.0;
    return x;
}

/* Per-channel log-decay of one g entry under the gate option. */
static double log_decay(double x, int gate) {
    if (gate == ORACLE_GATE_SIGMOID) x = -5.0 / (1.0 + exp(-x));
    return clamp_decay(x);
}

typedef struct {
    const void *q, *k, *v, *g, *beta;
    int dtype, gate;
    const double* S0;  /* [B,H,dk,dv] or NULL */
    double* o;         /* [B,T,H,dv] or NULL */
    double* ST;        /* [B,H,dk,dv] or NULL */
    long B, T, H, dk, dv;
    long next_unit;    /* shared work counter */
    pthread_mutex_t lock;
} fwd_job;

/* One (b, h) unit: the per-token recurrence over all T tokens. */
static void run_unit(fwd_job* J, long unit, double* S, double* gq, double* gk,
                     double* e, double* u) {
    const long b = unit / J->H, h = unit % J->H;
    const long dk = J->dk, dv = J->dv, H = J->H, T = J->T;
    if (J->S0) memcpy(S, J->S0 + (size_t)unit * dk * dv, sizeof(double) * dk * dv);
    else memset(S, 0, sizeof(double) * dk * dv);
    for (long t = 0; t < T; ++t) {
        const size_t tok = (size_t)(b * T + t) * H + h;
        for (long i = 0; i < dk; ++i) {
            e[i] = exp(log_decay(widen(J->g, J->dtype, tok * dk + i), J->gate));
            gk[i] = widen(J->k, J->dtype, tok * dk + i);
            gq[i] = widen(J->q, J->dtype, tok * dk + i);
        }
        const double bt = widen(J->beta, J->dtype, tok);
        /* P = Diag(e) S */
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j) S[i * dv + j] *= e[i];
        /* u = beta (v - P^T k) */
        for (long j = 0; j < dv; ++j) {
            double r = 0.0;
            for (long i = 0; i < dk; ++i) r += S[i * dv + j] * gk[i];
            u[j] = bt * (widen(J->v, J->dtype, tok * dv + j) - r);
        }
        /* S = P + k u^T */
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j) S[i * dv + j] += gk[i] * u[j];
        /* o = S^T q */
        if (J->o) {
            for (long j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * gq[i];
                J->o[tok * dv + j] = acc;
            }
        }
    }
    if (J->ST) memcpy(J->ST + (size_t)unit * dk * dv, S, sizeof(double) * dk * dv);
}

static void* worker(void* arg) {
    fwd_job* J = (fwd_job*)arg;
    double* S = (double*)malloc(sizeof(double) * J->dk * J->dv);
    double* gq = (double*)malloc(sizeof(double) * J->dk);
    double* gk = (double*)malloc(sizeof(double) * J->dk);
    double* e = (double*)malloc(sizeof(double) * J->dk);
    double* u = (double*)malloc(sizeof(double) * J->dv);
    for (;;) {
        pthread_mutex_lock(&J->lock);
        long unit = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (unit >= J->B * J->H) break;
        run_unit(J, unit, S, gq, gk, e, u);
    }
    free(S); free(gq); free(gk); free(e); free(u);
    return NULL;
}

/* Full forward. Returns 0 on success, nonzero on bad arguments. */
int kda_oracle_fwd(const void* q, const void* k, const void* v, const void* g,
                   const void* beta, int dtype, int gate, const double* S0, double* o,
                   double* ST, long B, long T, long H, long dk, long dv,
                   int nthreads) {
    if (!q || !k || !v || !g || !beta) return 1;
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1) return 2;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return 3;
    if (gate != ORACLE_GATE_LOG_DECAY && gate != ORACLE_GATE_SIGMOID) return 3;
    fwd_job J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.dtype = dtype; J.gate = gate;
    J.S0 = S0; J.o = o; J.ST = ST;
    J.B = B; J.T = T; J.H = H; J.dk = dk; J.dv = dv; J.next_unit = 0;
    pthread_mutex_init(&J.lock, NULL);
    long units = B * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return 0;
}

/*
 * The same recurrence for one (b, h) restricted to a subset of value columns.
 * Column j of S, of u and of o only ever involves column j (the decay scales
 * rows, the erase and the readout contract over rows), so these columns equal
 * the corresponding columns of the full computation. Used to check sampled
 * columns of very long sequences. S0c is [dk, ncols] (or NULL); oc is
 * [T, ncols]; STc is [dk, ncols] (either may be NULL).
 */
int kda_oracle_fwd_cols(const void* q, const void* k, const void* v, const void* g,
                        const void* beta, int dtype, int gate, long B, long T, long H,
                        long dk, long dv, long b, long h, const long* cols,
                        long ncols, const double* S0c, double* oc, double* STc) {
    if (!q || !k || !v || !g || !beta || !cols) return 1;
    if (b < 0 || b >= B || h < 0 || h >= H || ncols < 1) return 2;
    if (gate != ORACLE_GATE_LOG_DECAY && gate != ORACLE_GATE_SIGMOID) return 3;
    for (long c = 0; c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= dv) return 2;
    double* S = (double*)calloc((size_t)dk * ncols, sizeof(double));
    double* e = (double*)malloc(sizeof(double) * dk);
    double* gk = (double*)malloc(sizeof(double) * dk);
    double* gq = (double*)malloc(sizeof(double) * dk);
    if (S0c) memcpy(S, S0c, sizeof(double) * dk * ncols);
    for (long t = 0; t < T; ++t) {
        const size_t tok = (size_t)(b * T + t) * H + h;
        for (long i = 0; i < dk; ++i) {
            e[i] = exp(log_decay(widen(g, dtype, tok * dk + i), gate));
            gk[i] = widen(k, dtype, tok * dk + i);
            gq[i] = widen(q, dtype, tok * dk + i);
        }
        const double bt = widen(beta, dtype, tok);
        for (long c = 0; c < ncols; ++c) {
            double r = 0.0;
            for (long i = 0; i < dk; ++i) {
                S[i * ncols + c] *= e[i];
                r += S[i * ncols + c] * gk[i];
            }
            const double uj = bt * (widen(v, dtype, tok * dv + cols[c]) - r);
            double acc = 0.0;
            for (long i = 0; i < dk; ++i) {
                S[i * ncols + c] += gk[i] * uj;
                acc += S[i * ncols + c] * gq[i];
            }
            if (oc) oc[t * ncols + c] = acc;
        }
    }
    if (STc) memcpy(STc, S, sizeof(double) * dk * ncols);
    free(S); free(e); free(gk); free(gq);
    return 0;
}
