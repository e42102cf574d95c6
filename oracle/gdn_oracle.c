/*
 * gdn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, token-sequential double-precision gated delta rule.  It is the
 * parity oracle for the GPU library and nothing else: only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg load it.  It shares no code,
 * header or constant with the GPU path.
 *
 * What it computes (SANA-Streaming pages: the Korean review, section 1 "Key
 * Terms", defines GDN as a fixed-size state that is updated recursively from
 * the previous state; the Chinese summary, "Method steps", step 2, says the
 * streaming model runs a forward scan that carries the previous chunk's cache
 * plus a backward scan inside the chunk).  The pages name Gated DeltaNet but do
 * not print its update; the published Gated DeltaNet rule is used:
 *
 *     S_t = a_t * S_{t-1} * (I - beta_t * k_t k_t^T) + beta_t * v_t k_t^T
 *     o_t = scale * S_t q_t                     (state after the update)
 *
 * with S in R^{Dv x Dk}.  When l2norm is set, q_t and k_t are first replaced by
 * x / sqrt(sum(x^2) + eps).  The reverse scan is the same rule applied to the
 * tokens in the order T-1, ..., 0 (each token keeps its own a_t, beta_t), and
 * o_t is stored at the token's own position.
 *
 * Work is split over (stream b, head h, block of state rows) because rows of S
 * evolve independently; time is strictly sequential.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t B, T, H, Dk, Dv;
    const double *q, *k, *v, *a, *beta, *S0;
    int reverse, l2norm;
    double eps, scale;
    double *o, *S_final;
    int64_t row_block;     /* state rows per work item */
    int64_t n_items;       /* B * H * ceil(Dv / row_block) */
    int64_t next_item;     /* shared counter, guarded by mu */
    pthread_mutex_t mu;
} job_t;

/* x / sqrt(sum(x^2) + eps), or a plain copy when normalisation is off. */
static void normalise(const double* x, int64_t n, int on, double eps, double* out) {
    if (!on) {
        memcpy(out, x, (size_t)n * sizeof(double));
        return;
    }
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss + eps);
    for (int64_t i = 0; i < n; ++i) out[i] = x[i] * inv;
}

/* One work item: stream b, head h, state rows [r0, r1). */
static void run_item(const job_t* J, int64_t b, int64_t h, int64_t r0, int64_t r1,
                     double* S, double* kh, double* qh, double* x) {
    const int64_t Dk = J->Dk, Dv = J->Dv, H = J->H, T = J->T;
    const int64_t nr = r1 - r0;

    /* start state: rows [r0, r1) of S0[b, h], or zero */
    for (int64_t r = 0; r < nr; ++r)
        for (int64_t c = 0; c < Dk; ++c)
            S[r * Dk + c] = J->S0 ? J->S0[((b * H + h) * Dv + (r0 + r)) * Dk + c] : 0.0;

    for (int64_t step = 0; step < T; ++step) {
        const int64_t t = J->reverse ? (T - 1 - step) : step;
        const int64_t tok = (b * T + t) * H + h;       /* [B, T, H] index */
        const double at = J->a[tok];
        const double bt = J->beta[tok];
        const double* vt = J->v + tok * Dv;

        normalise(J->k + tok * Dk, Dk, J->l2norm, J->eps, kh);
        normalise(J->q + tok * Dk, Dk, J->l2norm, J->eps, qh);

        /* x = S_{t-1} k_t  (rows of this block) */
        for (int64_t r = 0; r < nr; ++r) {
            double s = 0.0;
            for (int64_t c = 0; c < Dk; ++c) s += S[r * Dk + c] * kh[c];
            x[r] = s;
        }
        /* S_t = a_t * (S_{t-1} - beta_t * x k_t^T) + beta_t * v_t k_t^T
         *     = a_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T   */
        for (int64_t r = 0; r < nr; ++r) {
            const double vr = vt[r0 + r];
            for (int64_t c = 0; c < Dk; ++c) {
                const double erased = S[r * Dk + c] - bt * x[r] * kh[c];
                S[r * Dk + c] = at * erased + bt * vr * kh[c];
            }
        }
        /* o_t = scale * S_t q_t */
        for (int64_t r = 0; r < nr; ++r) {
            double s = 0.0;
            for (int64_t c = 0; c < Dk; ++c) s += S[r * Dk + c] * qh[c];
            J->o[tok * Dv + (r0 + r)] = J->scale * s;
        }
    }

    if (J->S_final)
        for (int64_t r = 0; r < nr; ++r)
            for (int64_t c = 0; c < Dk; ++c)
                J->S_final[((b * H + h) * Dv + (r0 + r)) * Dk + c] = S[r * Dk + c];
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    const int64_t nblk = (J->Dv + J->row_block - 1) / J->row_block;
    double* S = (double*)malloc((size_t)(J->row_block * J->Dk) * sizeof(double));
    double* kh = (double*)malloc((size_t)J->Dk * sizeof(double));
    double* qh = (double*)malloc((size_t)J->Dk * sizeof(double));
    double* x = (double*)malloc((size_t)J->row_block * sizeof(double));
    if (!S || !kh || !qh || !x) {
        free(S); free(kh); free(qh); free(x);
        return (void*)1;
    }
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t it = J->next_item++;
        pthread_mutex_unlock(&J->mu);
        if (it >= J->n_items) break;
        const int64_t blk = it % nblk;
        const int64_t bh = it / nblk;
        const int64_t r0 = blk * J->row_block;
        const int64_t r1 = (r0 + J->row_block < J->Dv) ? r0 + J->row_block : J->Dv;
        run_item(J, bh / J->H, bh % J->H, r0, r1, S, kh, qh, x);
    }
    free(S); free(kh); free(qh); free(x);
    return NULL;
}

/*
 * Run the scan over all (b, h).  Arrays are C-contiguous:
 *   q, k [B, T, H, Dk]; v, o [B, T, H, Dv]; a, beta [B, T, H];
 *   S0, S_final [B, H, Dv, Dk] (S0 NULL = zero start, S_final NULL = not wanted).
 * Returns 0 on success, -1 on bad arguments, -2 if a thread or buffer failed.
 */
int gdn_oracle_scan(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                    const double* q, const double* k, const double* v,
                    const double* a, const double* beta, const double* S0,
                    int reverse, int l2norm, double eps, double scale,
                    double* o, double* S_final, int nthreads, int64_t row_block) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    if (T > 0 && (!q || !k || !v || !a || !beta || !o)) return -1;
    if (row_block <= 0 || row_block > Dv) row_block = Dv;
    if (nthreads <= 0) nthreads = 1;

    job_t J;
    J.B = B; J.T = T; J.H = H; J.Dk = Dk; J.Dv = Dv;
    J.q = q; J.k = k; J.v = v; J.a = a; J.beta = beta; J.S0 = S0;
    J.reverse = reverse; J.l2norm = l2norm; J.eps = eps; J.scale = scale;
    J.o = o; J.S_final = S_final;
    J.row_block = row_block;
    J.n_items = B * H * ((Dv + row_block - 1) / row_block);
    J.next_item = 0;
    pthread_mutex_init(&J.mu, NULL);

    if (nthreads > J.n_items) nthreads = (int)(J.n_items > 0 ? J.n_items : 1);
    int rc = 0;
    if (nthreads == 1) {
        if (worker(&J) != NULL) rc = -2;
    } else {
        pthread_t* th = (pthread_t*)malloc((size_t)nthreads * sizeof(pthread_t));
        int started = 0;
        if (!th) rc = -2;
        for (int i = 0; th && i < nthreads; ++i) {
            if (pthread_create(&th[i], NULL, worker, &J) != 0) { rc = -2; break; }
            ++started;
        }
        for (int i = 0; i < started; ++i) {
            void* ret = NULL;
            pthread_join(th[i], &ret);
            if (ret != NULL) rc = -2;
        }
        free(th);
    }
    pthread_mutex_destroy(&J.mu);
    return rc;
}

/*
 * Gradient of the same scan (reverse-mode through the per-token rule, in double
 * precision).  The pages print no training procedure; this is the derivative of
 * the recurrence above, written out.  With G = dL/dS_t (the incoming gradient of
 * the state after token t, plus the output term scale * do_t q_t^T), x = S_{t-1} k_t
 * and gk = G k_t (k_t, q_t normalised when l2norm is set):
 *
 *     dq_t   = scale * S_t^T do_t
 *     dv_t   = beta_t * gk
 *     da_t   = <G, S_{t-1}> - beta_t * gk . x
 *     dbeta_t = gk . (v_t - a_t * x)
 *     dk_t   = beta_t * G^T v_t - a_t * beta_t * (S_{t-1}^T gk + G^T x)
 *     dL/dS_{t-1} = a_t * (G - beta_t * gk k_t^T)
 *
 * and, when l2norm is set, dx = (dxh - xh * (xh . dxh)) / sqrt(sum(x^2) + eps) maps
 * the gradient of a normalised vector xh back to its input x.  The reverse scan is
 * differentiated in its own processing order (t = T-1 .. 0).  One work item per
 * (b, h); the item keeps all T + 1 states.
 */
typedef struct {
    int64_t B, T, H, Dk, Dv;
    const double *q, *k, *v, *a, *beta, *S0, *dO, *dSf;
    int reverse, l2norm;
    double eps, scale;
    double *dq, *dk, *dv, *da, *dbeta, *dS0;
    int64_t next_item;
    pthread_mutex_t mu;
} bjob_t;

static int run_bitem(const bjob_t* J, int64_t b, int64_t h) {
    const int64_t Dk = J->Dk, Dv = J->Dv, H = J->H, T = J->T, DD = Dv * Dk;
    double* S = (double*)malloc((size_t)((T + 1) * DD) * sizeof(double));   /* S[p] = state before step p */
    double* G = (double*)malloc((size_t)DD * sizeof(double));
    double* kh = (double*)malloc((size_t)(T * Dk) * sizeof(double));
    double* qh = (double*)malloc((size_t)(T * Dk) * sizeof(double));
    double* x = (double*)malloc((size_t)Dv * sizeof(double));
    double* gk = (double*)malloc((size_t)Dv * sizeof(double));
    double* gq = (double*)malloc((size_t)Dk * sizeof(double));
    double* gkh = (double*)malloc((size_t)Dk * sizeof(double));
    int rc = 0;
    if (!S || !G || !kh || !qh || !x || !gk || !gq || !gkh) { rc = -2; goto done; }

    for (int64_t i = 0; i < DD; ++i) S[i] = J->S0 ? J->S0[(b * H + h) * DD + i] : 0.0;
    /* forward, keeping every state; kh, qh indexed by processing step */
    for (int64_t p = 0; p < T; ++p) {
        const int64_t t = J->reverse ? (T - 1 - p) : p;
        const int64_t tok = (b * T + t) * H + h;
        const double at = J->a[tok], bt = J->beta[tok];
        const double* vt = J->v + tok * Dv;
        const double *kt = J->k + tok * Dk, *qt = J->q + tok * Dk;
        normalise(kt, Dk, J->l2norm, J->eps, kh + p * Dk);
        normalise(qt, Dk, J->l2norm, J->eps, qh + p * Dk);
        const double* Sp = S + p * DD;
        double* Sn = S + (p + 1) * DD;
        const double* kp = kh + p * Dk;
        for (int64_t r = 0; r < Dv; ++r) {
            double s = 0.0;
            for (int64_t c = 0; c < Dk; ++c) s += Sp[r * Dk + c] * kp[c];
            for (int64_t c = 0; c < Dk; ++c)
                Sn[r * Dk + c] = at * (Sp[r * Dk + c] - bt * s * kp[c]) + bt * vt[r] * kp[c];
        }
    }
    /* backward */
    for (int64_t i = 0; i < DD; ++i) G[i] = J->dSf ? J->dSf[(b * H + h) * DD + i] : 0.0;
    for (int64_t p = T - 1; p >= 0; --p) {
        const int64_t t = J->reverse ? (T - 1 - p) : p;
        const int64_t tok = (b * T + t) * H + h;
        const double at = J->a[tok], bt = J->beta[tok];
        const double* vt = J->v + tok * Dv;
        const double* dot = J->dO + tok * Dv;
        const double* Sp = S + p * DD;        /* S_{t-1} in processing order */
        const double* Sc = S + (p + 1) * DD;  /* S_t */
        const double* kp = kh + p * Dk;
        const double* qp = qh + p * Dk;
        /* output term */
        for (int64_t c = 0; c < Dk; ++c) {
            double s = 0.0;
            for (int64_t r = 0; r < Dv; ++r) s += Sc[r * Dk + c] * dot[r];
            gq[c] = s * J->scale;
        }
        for (int64_t r = 0; r < Dv; ++r)
            for (int64_t c = 0; c < Dk; ++c) G[r * Dk + c] += J->scale * dot[r] * qp[c];
        /* the update */
        double da = 0.0, db = 0.0;
        for (int64_t r = 0; r < Dv; ++r) {
            double sx = 0.0, sg = 0.0, gs = 0.0;
            for (int64_t c = 0; c < Dk; ++c) {
                sx += Sp[r * Dk + c] * kp[c];
                sg += G[r * Dk + c] * kp[c];
                gs += G[r * Dk + c] * Sp[r * Dk + c];
            }
            x[r] = sx;
            gk[r] = sg;
            da += gs - bt * sg * sx;
            db += sg * (vt[r] - at * sx);
            J->dv[tok * Dv + r] = bt * sg;
        }
        for (int64_t c = 0; c < Dk; ++c) {
            double s = 0.0;
            for (int64_t r = 0; r < Dv; ++r)
                s += bt * G[r * Dk + c] * vt[r] - at * bt * (Sp[r * Dk + c] * gk[r] + G[r * Dk + c] * x[r]);
            gkh[c] = s;
        }
        J->da[tok] = da;
        J->dbeta[tok] = db;
        for (int64_t r = 0; r < Dv; ++r)
            for (int64_t c = 0; c < Dk; ++c) G[r * Dk + c] = at * (G[r * Dk + c] - bt * gk[r] * kp[c]);
        /* back through the normalisation */
        const double* xs[2] = {J->k + tok * Dk, J->q + tok * Dk};
        const double* hs[2] = {kp, qp};
        double* gs2[2] = {gkh, gq};
        double* outs[2] = {J->dk + tok * Dk, J->dq + tok * Dk};
        for (int w = 0; w < 2; ++w) {
            if (!J->l2norm) {
                memcpy(outs[w], gs2[w], (size_t)Dk * sizeof(double));
                continue;
            }
            double ss = 0.0, hg = 0.0;
            for (int64_t c = 0; c < Dk; ++c) {
                ss += xs[w][c] * xs[w][c];
                hg += hs[w][c] * gs2[w][c];
            }
            const double inv = 1.0 / sqrt(ss + J->eps);
            for (int64_t c = 0; c < Dk; ++c) outs[w][c] = (gs2[w][c] - hs[w][c] * hg) * inv;
        }
    }
    if (J->dS0)
        for (int64_t i = 0; i < DD; ++i) J->dS0[(b * H + h) * DD + i] = G[i];
done:
    free(S); free(G); free(kh); free(qh); free(x); free(gk); free(gq); free(gkh);
    return rc;
}

static void* bworker(void* arg) {
    bjob_t* J = (bjob_t*)arg;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t it = J->next_item++;
        pthread_mutex_unlock(&J->mu);
        if (it >= J->B * J->H) break;
        if (run_bitem(J, it / J->H, it % J->H) != 0) return (void*)1;
    }
    return NULL;
}

/*
 * Gradients of the scan for the loss whose gradients with respect to o and to the final
 * state are dO [B, T, H, Dv] and dS_final [B, H, Dv, Dk] (NULL = zero).  Same layouts and
 * arguments as gdn_oracle_scan; outputs dq, dk [B, T, H, Dk], dv [B, T, H, Dv], da, dbeta
 * [B, T, H] and dS0 [B, H, Dv, Dk] (the gradient of the start state; NULL = not wanted).
 * Returns 0 on success, -1 on bad arguments, -2 if a thread or buffer failed.
 */
int gdn_oracle_backward(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                        const double* q, const double* k, const double* v,
                        const double* a, const double* beta, const double* S0,
                        const double* dO, const double* dS_final,
                        int reverse, int l2norm, double eps, double scale,
                        double* dq, double* dk, double* dv, double* da, double* dbeta, double* dS0,
                        int nthreads) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    if (T > 0 && (!q || !k || !v || !a || !beta || !dO || !dq || !dk || !dv || !da || !dbeta)) return -1;
    if (nthreads <= 0) nthreads = 1;
    bjob_t J;
    J.B = B; J.T = T; J.H = H; J.Dk = Dk; J.Dv = Dv;
    J.q = q; J.k = k; J.v = v; J.a = a; J.beta = beta; J.S0 = S0; J.dO = dO; J.dSf = dS_final;
    J.reverse = reverse; J.l2norm = l2norm; J.eps = eps; J.scale = scale;
    J.dq = dq; J.dk = dk; J.dv = dv; J.da = da; J.dbeta = dbeta; J.dS0 = dS0;
    J.next_item = 0;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads > B * H) nthreads = (int)(B * H > 0 ? B * H : 1);
    int rc = 0;
    if (nthreads == 1) {
        if (bworker(&J) != NULL) rc = -2;
    } else {
        pthread_t* th = (pthread_t*)malloc((size_t)nthreads * sizeof(pthread_t));
        int started = 0;
        if (!th) rc = -2;
        for (int i = 0; th && i < nthreads; ++i) {
            if (pthread_create(&th[i], NULL, bworker, &J) != 0) { rc = -2; break; }
            ++started;
        }
        for (int i = 0; i < started; ++i) {
            void* ret = NULL;
            pthread_join(th[i], &ret);
            if (ret != NULL) rc = -2;
        }
        free(th);
    }
    pthread_mutex_destroy(&J.mu);
    return rc;
}
