/*
 * KDA prefill oracle: plain, slow, double-precision, token by token.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library.
 *
 * What it computes (Kimi Delta Attention, the gated delta rule with a decay
 * per key channel; the pages name KDA -- pegainfer PR #970 "cross-process CP
 * whale gang", commit text on the whale lane's "KDA (M,D) packages"; kern
 * PR #44, "k3: flash-kda builds a varlen variant", one state block per
 * sequence -- but do not write the recurrence out, so it is stated here):
 *
 *   for each sequence n and head h, S = S0[n,h] (zeros if absent), dk x dv
 *   for each token t of the sequence, in order:
 *       qn = scale * q_t / sqrt(|q_t|^2 + 1e-6)      (when qk_l2norm)
 *       kn =         k_t / sqrt(|k_t|^2 + 1e-6)
 *       S  = Diag(exp(g_t)) S                         decay first
 *       S  = S + beta_t kn (v_t - S^T kn)^T           erase along kn, then write
 *       o_t = S^T qn                                  read the updated state
 *   which is S_t = (I - beta_t kn kn^T) Diag(alpha_t) S_{t-1} + beta_t kn v_t^T
 *   with alpha_t = exp(g_t).
 *
 * Checkpoints (ROCm/ATOM PR #2709 "PP8 prefill for P/D serving", Changes:
 * KDA state checkpoints on a chunk grid): after the p-th token of a sequence
 * with p = m*interval (m >= 1) the state is stored at row
 * ckpt_offsets[n] + m - 1 of a [rows, H, dk, dv] buffer.
 *
 * Segment packages (pegainfer PR #970, whale-lane commit text: "KDA (M,D)
 * packages"): over a token range [a, b) of one sequence the state map is
 * affine, S_b = M S_a + D.  M is the product of the per-token linear maps
 * (the recurrence run on a dk x dk matrix started at I with v = 0) and D is
 * the recurrence run from S = 0.
 *
 * Layouts: q, k, g [T,H,dk]; v, o [T,H,dv]; beta [T,H]; states [.,H,dk,dv]
 * (key-major); all row-major, all double.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KDA_ORACLE_EPS 1e-6

typedef struct {
    int64_t T;
    int32_t H, dk, dv;
    const double *q, *k, *v, *g, *beta;
    double scale;
    int32_t l2norm;
} problem_t;

/* Normalised copies of q_t and k_t for head h. */
static void normalise(const problem_t *P, int64_t t, int32_t h, double *qn, double *kn) {
    const double *qt = P->q + (t * P->H + h) * P->dk;
    const double *kt = P->k + (t * P->H + h) * P->dk;
    double sq = 0.0, sk = 0.0;
    for (int i = 0; i < P->dk; ++i) { sq += qt[i] * qt[i]; sk += kt[i] * kt[i]; }
    double fq = P->scale, fk = 1.0;
    if (P->l2norm) { fq = P->scale / sqrt(sq + KDA_ORACLE_EPS); fk = 1.0 / sqrt(sk + KDA_ORACLE_EPS); }
    for (int i = 0; i < P->dk; ++i) { qn[i] = qt[i] * fq; kn[i] = kt[i] * fk; }
}

/*
 * One token step on a dk x ncol matrix S (row-major, leading dimension ncol).
 * When vt is NULL the written value is zero (the value-free linear part).
 */
static void token_step(const problem_t *P, int64_t t, int32_t h, const double *kn,
                       const double *vt, double *S, int ncol, double *r) {
    const double *gt = P->g + (t * P->H + h) * P->dk;
    const double b = P->beta[t * P->H + h];
    for (int i = 0; i < P->dk; ++i) {
        const double a = exp(gt[i]);
        for (int j = 0; j < ncol; ++j) S[i * ncol + j] *= a;
    }
    for (int j = 0; j < ncol; ++j) r[j] = 0.0;
    for (int i = 0; i < P->dk; ++i)
        for (int j = 0; j < ncol; ++j) r[j] += kn[i] * S[i * ncol + j];
    for (int i = 0; i < P->dk; ++i)
        for (int j = 0; j < ncol; ++j) {
            const double vj = vt ? vt[j] : 0.0;
            S[i * ncol + j] += b * kn[i] * (vj - r[j]);
        }
}

static void read_out(const problem_t *P, const double *qn, const double *S, double *ot) {
    for (int j = 0; j < P->dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < P->dk; ++i) acc += S[i * P->dv + j] * qn[i];
        ot[j] = acc;
    }
}

/* ------------------------------------------------------------------------- */
/* Work distribution over independent (sequence, head) units                  */
/* ------------------------------------------------------------------------- */
typedef struct {
    problem_t P;
    const int64_t *cu;
    int32_t N;
    const double *S0;
    int32_t interval;
    const int64_t *ckpt_off;
    double *ckpt, *o, *S_final;
    int64_t next;   /* atomic unit counter */
    int failed;
} prefill_job_t;

static void prefill_unit(prefill_job_t *J, int32_t n, int32_t h) {
    const problem_t *P = &J->P;
    const int dk = P->dk, dv = P->dv;
    const size_t ss = (size_t)dk * dv;
    double *S = (double *)calloc(ss, sizeof(double));
    double *qn = (double *)malloc(sizeof(double) * dk);
    double *kn = (double *)malloc(sizeof(double) * dk);
    double *r = (double *)malloc(sizeof(double) * dv);
    if (!S || !qn || !kn || !r) { J->failed = 1; free(S); free(qn); free(kn); free(r); return; }
    if (J->S0) memcpy(S, J->S0 + ((size_t)n * P->H + h) * ss, ss * sizeof(double));
    const int64_t a = J->cu[n], b = J->cu[n + 1];
    for (int64_t t = a; t < b; ++t) {
        normalise(P, t, h, qn, kn);
        token_step(P, t, h, kn, P->v + (t * P->H + h) * dv, S, dv, r);
        read_out(P, qn, S, J->o + (t * P->H + h) * dv);
        const int64_t p = t - a + 1;
        if (J->ckpt && J->interval > 0 && p % J->interval == 0) {
            const int64_t row = J->ckpt_off[n] + p / J->interval - 1;
            memcpy(J->ckpt + ((size_t)row * P->H + h) * ss, S, ss * sizeof(double));
        }
    }
    if (J->S_final) memcpy(J->S_final + ((size_t)n * P->H + h) * ss, S, ss * sizeof(double));
    free(S); free(qn); free(kn); free(r);
}

static void *prefill_worker(void *arg) {
    prefill_job_t *J = (prefill_job_t *)arg;
    const int64_t units = (int64_t)J->N * J->P.H;
    for (;;) {
        const int64_t u = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (u >= units) break;
        prefill_unit(J, (int32_t)(u / J->P.H), (int32_t)(u % J->P.H));
    }
    return NULL;
}

static int run_threads(void *(*fn)(void *), void *job, int32_t nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads == 1) { fn(job); return 0; }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    if (!th) return -1;
    int started = 0;
    for (int i = 0; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, fn, job) == 0) ++started;
    if (started == 0) fn(job);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    return 0;
}

/*
 * Token-by-token prefill over N packed sequences (cu_seqlens[N+1] row offsets).
 * S0, ckpt, S_final may be NULL.  Returns 0 on success, -1 on bad arguments
 * or allocation failure.
 */
int kda_oracle_prefill(int64_t T, int32_t H, int32_t dk, int32_t dv,
                       const double *q, const double *k, const double *v,
                       const double *g, const double *beta,
                       const int64_t *cu_seqlens, int32_t N, const double *S0,
                       double scale, int32_t qk_l2norm,
                       int32_t interval, const int64_t *ckpt_offsets, double *ckpt,
                       double *o, double *S_final, int32_t nthreads) {
    if (T < 0 || H <= 0 || dk <= 0 || dv <= 0 || N < 0 || !cu_seqlens) return -1;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return -1;
    if (ckpt && (interval <= 0 || !ckpt_offsets)) return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
    for (int32_t n = 0; n < N; ++n) if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    prefill_job_t J;
    memset(&J, 0, sizeof(J));
    J.P.T = T; J.P.H = H; J.P.dk = dk; J.P.dv = dv;
    J.P.q = q; J.P.k = k; J.P.v = v; J.P.g = g; J.P.beta = beta;
    J.P.scale = scale; J.P.l2norm = qk_l2norm;
    J.cu = cu_seqlens; J.N = N; J.S0 = S0; J.interval = interval;
    J.ckpt_off = ckpt_offsets; J.ckpt = ckpt; J.o = o; J.S_final = S_final;
    if (run_threads(prefill_worker, &J, nthreads) != 0) return -1;
    return J.failed ? -1 : 0;
}

/* ------------------------------------------------------------------------- */
/* Segment package (M, D) and the segment's outputs from a zero state         */
/* ------------------------------------------------------------------------- */
typedef struct {
    problem_t P;
    int64_t a, b;
    double *M, *D, *o_local;
    int64_t next;
    int failed;
} package_job_t;

static void package_head(package_job_t *J, int32_t h) {
    const problem_t *P = &J->P;
    const int dk = P->dk, dv = P->dv;
    double *M = (double *)calloc((size_t)dk * dk, sizeof(double));
    double *D = (double *)calloc((size_t)dk * dv, sizeof(double));
    double *qn = (double *)malloc(sizeof(double) * dk);
    double *kn = (double *)malloc(sizeof(double) * dk);
    double *r = (double *)malloc(sizeof(double) * (dk > dv ? dk : dv));
    if (!M || !D || !qn || !kn || !r) { J->failed = 1; goto out; }
    for (int i = 0; i < dk; ++i) M[i * dk + i] = 1.0;
    for (int64_t t = J->a; t < J->b; ++t) {
        normalise(P, t, h, qn, kn);
        token_step(P, t, h, kn, NULL, M, dk, r);
        token_step(P, t, h, kn, P->v + (t * P->H + h) * dv, D, dv, r);
        if (J->o_local) read_out(P, qn, D, J->o_local + (t * P->H + h) * dv);
    }
    memcpy(J->M + (size_t)h * dk * dk, M, sizeof(double) * dk * dk);
    memcpy(J->D + (size_t)h * dk * dv, D, sizeof(double) * dk * dv);
out:
    free(M); free(D); free(qn); free(kn); free(r);
}

static void *package_worker(void *arg) {
    package_job_t *J = (package_job_t *)arg;
    for (;;) {
        const int64_t u = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (u >= J->P.H) break;
        package_head(J, (int32_t)u);
    }
    return NULL;
}

/*
 * Package of the token range [a, b): M [H,dk,dk], D [H,dk,dv]; o_local (may be
 * NULL) receives rows a..b-1 of the outputs computed from a zero state.
 */
int kda_oracle_package(int64_t T, int32_t H, int32_t dk, int32_t dv,
                       const double *q, const double *k, const double *v,
                       const double *g, const double *beta,
                       int64_t a, int64_t b, double scale, int32_t qk_l2norm,
                       double *M, double *D, double *o_local, int32_t nthreads) {
    if (H <= 0 || dk <= 0 || dv <= 0 || a < 0 || b < a || b > T || !M || !D) return -1;
    if (b > a && (!q || !k || !v || !g || !beta)) return -1;
    package_job_t J;
    memset(&J, 0, sizeof(J));
    J.P.T = T; J.P.H = H; J.P.dk = dk; J.P.dv = dv;
    J.P.q = q; J.P.k = k; J.P.v = v; J.P.g = g; J.P.beta = beta;
    J.P.scale = scale; J.P.l2norm = qk_l2norm;
    J.a = a; J.b = b; J.M = M; J.D = D; J.o_local = o_local;
    if (run_threads(package_worker, &J, nthreads) != 0) return -1;
    return J.failed ? -1 : 0;
}
