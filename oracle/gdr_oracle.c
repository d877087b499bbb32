/*
 * gdr_oracle.c -- plain fp64 CPU reference for chunk-free gated delta-rule
 * attention: the token-by-token recurrence and its hand-derived reverse mode.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code, header
 * or constant with the GPU library and never calls it.
 *
 * What it computes (ReWY paper, Sec. 2.2 and Table 1; Sec. 4.5 names an
 * independent CPU FP64 recurrence as the reference for every gradient):
 *   forward  o_t and the final state ht of the recurrence in token_fwd_body.h;
 *   backward the exact gradients of  <o, dO> + <ht, dht>  with respect to
 *            q, k, v, the log decay g, the write weight beta and h0.
 * Gradients are taken against exactly these inputs: g is the log decay
 * (a = exp(g)) and beta the post-activation weight; any normalisation or
 * activation in front of them is the caller's chain rule (Sec. 2.2 leaves
 * normalisation and gate activations to the surrounding chain rule).
 *
 * Layouts (row-major): q, k [B,T,H,DK]; v, o, dO [B,T,H,DV]; g [B,T,H]
 * (scalar gate) or [B,T,H,DK] (vector gate); beta [B,T,H];
 * h0, ht, dht, dh0 [B,H,DK,DV] (key-major, i.e. the transpose of the
 * value-by-key state X used inside).
 *
 * Reverse mode, per token t from last to first, with Xb the adjoint of X_t:
 *   Xb  += dO_t q_t^T            dq_t = X_t^T dO_t
 *   w    = Xb k_t                eb = beta_t w   (adjoint of e)
 *   dk_t = beta_t Xb^T e - P^T eb
 *   dbeta_t = <w, e>             (undivided form: defined at beta = 0,
 *                                 paper Sec. 3.1 and App. B.3)
 *   dv_t = eb
 *   Pb   = Xb - eb k_t^T
 *   abar_j = sum_v X_{t-1}[v,j] Pb[v,j]     dg = abar * a  (summed over j
 *                                           for a scalar gate, App. E.1)
 *   Xb  <- Pb Diag(a_t)
 * and dh0 = Xb^T at the start. The states needed in reverse are rebuilt from
 * checkpoints taken every 64 tokens.
 *
 * GDN2 (gdr_oracle_gdn2_*; paper Table 1: vector decay with independent
 * vector erase and write gates, Sec. 3.1 keeps their gradients separate;
 * the step is in token_fwd_body.h). Per token, with s = Xb k_t after the
 * output adjoint is added, P = X_{t-1} Diag(a_t) and e = wrt o v - P (ers o k):
 *   dv_t = wrt_t o s              dwrt_t = v_t o s
 *   dk_t = Xb^T e - ers_t o (P^T s)          ders_t = -k_t o (P^T s)
 *   Pb   = Xb - s (ers_t o k_t)^T
 * and the decay and state adjoints as above.
 *
 * Threads split the work over (b, h, block of value rows); per-row-block
 * partial sums of dq, dk, dbeta and dg are added in a fixed order, so the
 * result does not depend on the thread count or scheduling.
 */
#include <complex.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define FWD_NAME fwd_rows_d
#define SCALAR double
#define SEXP exp
#include "token_fwd_body.h"
#undef FWD_NAME
#undef SCALAR
#undef SEXP

#define FWD_NAME fwd_rows_z
#define SCALAR double complex
#define SEXP cexp
#include "token_fwd_body.h"
#undef FWD_NAME
#undef SCALAR
#undef SEXP

#define CKPT 64

typedef struct {
    int64_t B, T, H, DK, DV;
    int vec_gate;
    int64_t nvb, rows;  /* value-row blocks per head, rows per block */
    const double *q, *k, *v, *g, *beta, *h0, *dO, *dht;
    const double *ers, *wrt;   /* GDN2 gates (NULL otherwise) */
    double *o, *ht, *dq, *dk, *dv, *dg, *dbeta, *dh0;
    double *ders, *dwrt;       /* GDN2 gate gradients */
    double* part;       /* per-item partials when nvb > 1 */
    int64_t part_w;     /* doubles per token in a partial row */
    int64_t next;       /* work counter (atomic) */
    int64_t nitems;
    int err;
} job_t;

static int64_t take(job_t* J) { return __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED); }

/* ---------------- forward ---------------- */

static void* fwd_worker(void* arg)
{
    job_t* J = (job_t*)arg;
    double* X = (double*)malloc(sizeof(double) * (size_t)(J->rows * J->DK + J->DK));
    if (!X) { J->err = 1; return NULL; }
    for (int64_t it; (it = take(J)) < J->nitems;) {
        const int64_t bh = it / J->nvb, vb = it % J->nvb;
        const int64_t b = bh / J->H, h = bh % J->H;
        const int64_t v0 = vb * J->rows;
        int64_t v1 = v0 + J->rows;
        if (v1 > J->DV) v1 = J->DV;
        if (v0 >= v1) continue;
        fwd_rows_d(J->T, J->H, J->DK, J->DV, J->vec_gate, b, h, v0, v1, J->q, J->k, J->v,
                   J->g, J->beta, J->ers, J->wrt, J->h0, J->o, J->ht, X, X + J->rows * J->DK);
    }
    free(X);
    return NULL;
}

static int run_threads(job_t* J, void* (*fn)(void*), int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > J->nitems) nthreads = (int)J->nitems;
    if (nthreads <= 1) { fn(J); return J->err; }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return 1;
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, fn, J) != 0) break;
        ++started;
    }
    if (started == 0) fn(J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    return J->err;
}

/* The row split depends on the shape only (about 32 work items when there
 * are fewer than 32 heads), never on the thread count, so the fixed-order
 * reduction gives the same bits for any number of threads. */
#define TARGET_ITEMS 32
static void split_rows(job_t* J)
{
    int64_t bh = J->B * J->H;
    int64_t nvb = 1;
    if (bh < TARGET_ITEMS) {
        nvb = (TARGET_ITEMS + bh - 1) / bh;
        if (nvb > J->DV) nvb = J->DV;
    }
    J->rows = (J->DV + nvb - 1) / nvb;
    J->nvb = (J->DV + J->rows - 1) / J->rows;
    J->nitems = bh * J->nvb;
}

static int fwd_any(int64_t B, int64_t T, int64_t H, int64_t DK, int64_t DV, int vec_gate,
                   const double* q, const double* k, const double* v, const double* g,
                   const double* beta, const double* ers, const double* wrt, const double* h0,
                   double* o, double* ht, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || DK < 1 || DV < 1) return 1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.DK = DK; J.DV = DV; J.vec_gate = vec_gate;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0; J.o = o; J.ht = ht;
    J.ers = ers; J.wrt = wrt;
    if (B * H == 0) return 0;
    split_rows(&J);
    return run_threads(&J, fwd_worker, nthreads);
}

int gdr_oracle_fwd(int64_t B, int64_t T, int64_t H, int64_t DK, int64_t DV, int vec_gate,
                   const double* q, const double* k, const double* v, const double* g,
                   const double* beta, const double* h0, double* o, double* ht, int nthreads)
{
    return fwd_any(B, T, H, DK, DV, vec_gate, q, k, v, g, beta, NULL, NULL, h0, o, ht, nthreads);
}

/* GDN2: per-key-channel log decay g [B,T,H,DK], erase gate ers [B,T,H,DK],
 * write gate wrt [B,T,H,DV]. */
int gdr_oracle_gdn2_fwd(int64_t B, int64_t T, int64_t H, int64_t DK, int64_t DV,
                        const double* q, const double* k, const double* v, const double* g,
                        const double* ers, const double* wrt, const double* h0, double* o,
                        double* ht, int nthreads)
{
    if (!ers || !wrt) return 1;
    return fwd_any(B, T, H, DK, DV, 1, q, k, v, g, NULL, ers, wrt, h0, o, ht, nthreads);
}

/* Complex-step forward: same recurrence in double complex, single thread.
 * Arrays are interleaved (re, im) pairs, the layout of C99 double complex. */
int gdr_oracle_fwd_complex(int64_t B, int64_t T, int64_t H, int64_t DK, int64_t DV, int vec_gate,
                           const double complex* q, const double complex* k,
                           const double complex* v, const double complex* g,
                           const double complex* beta, const double complex* h0,
                           double complex* o, double complex* ht)
{
    if (B < 0 || T < 0 || H < 0 || DK < 1 || DV < 1) return 1;
    double complex* X = (double complex*)malloc(sizeof(double complex) * (size_t)(DV * DK + DK));
    if (!X) return 1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            fwd_rows_z(T, H, DK, DV, vec_gate, b, h, 0, DV, q, k, v, g, beta, NULL, NULL, h0, o, ht,
                       X, X + DV * DK);
    free(X);
    return 0;
}

int gdr_oracle_gdn2_fwd_complex(int64_t B, int64_t T, int64_t H, int64_t DK, int64_t DV,
                                const double complex* q, const double complex* k,
                                const double complex* v, const double complex* g,
                                const double complex* ers, const double complex* wrt,
                                const double complex* h0, double complex* o, double complex* ht)
{
    if (B < 0 || T < 0 || H < 0 || DK < 1 || DV < 1 || !ers || !wrt) return 1;
    double complex* X = (double complex*)malloc(sizeof(double complex) * (size_t)(DV * DK + DK));
    if (!X) return 1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            fwd_rows_z(T, H, DK, DV, 1, b, h, 0, DV, q, k, v, g, NULL, ers, wrt, h0, o, ht, X,
                       X + DV * DK);
    free(X);
    return 0;
}

/* ---------------- backward ---------------- */

/* Advance the value rows X (nr x DK) of one head over token t.
 */
static void step_fwd(const job_t* J, int64_t b, int64_t h, int64_t t, int64_t v0, int64_t nr,
                     double* X, double* a)
{
    const int64_t DK = J->DK;
    const int64_t tok = (b * J->T + t) * J->H + h;
    const double* kt = J->k + tok * DK;
    const double* vt = J->v + tok * J->DV;
    for (int64_t j = 0; j < DK; ++j) a[j] = exp(J->vec_gate ? J->g[tok * DK + j] : J->g[tok]);
    if (J->ers) {
        /* GDN2: u = P (ers o k), e = wrt o v - u, X = P + e k^T */
        const double* et = J->ers + tok * DK;
        const double* wt = J->wrt + tok * J->DV;
        for (int64_t r = 0; r < nr; ++r) {
            double* x = X + r * DK;
            double u = 0;
            for (int64_t j = 0; j < DK; ++j) { x[j] *= a[j]; u += x[j] * (et[j] * kt[j]); }
            const double e = wt[v0 + r] * vt[v0 + r] - u;
            for (int64_t j = 0; j < DK; ++j) x[j] += e * kt[j];
        }
        return;
    }
    const double bt = J->beta[tok];
    for (int64_t r = 0; r < nr; ++r) {
        double* x = X + r * DK;
        double u = 0;
        for (int64_t j = 0; j < DK; ++j) { x[j] *= a[j]; u += x[j] * kt[j]; }
        const double e = vt[v0 + r] - u;
        for (int64_t j = 0; j < DK; ++j) x[j] += bt * e * kt[j];
    }
}

static void* bwd_worker(void* arg)
{
    job_t* J = (job_t*)arg;
    const int64_t DK = J->DK, DV = J->DV, T = J->T, H = J->H, R = J->rows;
    const int64_t nck = (T + CKPT - 1) / CKPT;
    const size_t st = (size_t)(R * DK);
    /* checkpoints, one segment of states, adjoint, scratch */
    double* ck = (double*)malloc(sizeof(double) * st * (size_t)(nck + 1));
    double* seg = (double*)malloc(sizeof(double) * st * (CKPT + 1));
    double* Xb = (double*)malloc(sizeof(double) * st);
    double* Pm = (double*)malloc(sizeof(double) * st);
    double* a = (double*)malloc(sizeof(double) * (size_t)DK);
    double* e = (double*)malloc(sizeof(double) * (size_t)R);
    double* w = (double*)malloc(sizeof(double) * (size_t)R);
    double* acc = (double*)malloc(sizeof(double) * (size_t)J->part_w);
    if (!ck || !seg || !Xb || !Pm || !a || !e || !w || !acc) {
        J->err = 1;
        goto out;
    }
    for (int64_t it; (it = take(J)) < J->nitems;) {
        const int64_t bh = it / J->nvb, vb = it % J->nvb;
        const int64_t b = bh / H, h = bh % H;
        const int64_t v0 = vb * R;
        int64_t v1 = v0 + R;
        if (v1 > DV) v1 = DV;
        if (v0 >= v1) continue;
        const int64_t nr = v1 - v0;
        const int direct = (J->nvb == 1);

        /* forward sweep storing checkpoints of X at t = 0, CKPT, 2 CKPT, ... */
        double* X = ck;
        for (int64_t r = 0; r < nr; ++r)
            for (int64_t j = 0; j < DK; ++j)
                X[r * DK + j] = J->h0 ? J->h0[((b * H + h) * DK + j) * DV + v0 + r] : 0.0;
        for (int64_t c = 0; c < nck; ++c) {
            double* nxt = ck + (size_t)(c + 1) * st;
            memcpy(nxt, ck + (size_t)c * st, sizeof(double) * (size_t)(nr * DK));
            const int64_t te = (c + 1) * CKPT < T ? (c + 1) * CKPT : T;
            for (int64_t t = c * CKPT; t < te; ++t) step_fwd(J, b, h, t, v0, nr, nxt, a);
        }
        /* adjoint of the final state: Xb = dht^T */
        for (int64_t r = 0; r < nr; ++r)
            for (int64_t j = 0; j < DK; ++j)
                Xb[r * DK + j] = J->dht ? J->dht[((b * H + h) * DK + j) * DV + v0 + r] : 0.0;

        for (int64_t c = nck - 1; c >= 0; --c) {
            const int64_t ts = c * CKPT;
            const int64_t te = (c + 1) * CKPT < T ? (c + 1) * CKPT : T;
            memcpy(seg, ck + (size_t)c * st, sizeof(double) * (size_t)(nr * DK));
            for (int64_t t = ts; t < te; ++t) {
                memcpy(seg + (size_t)(t - ts + 1) * st, seg + (size_t)(t - ts) * st,
                       sizeof(double) * (size_t)(nr * DK));
                step_fwd(J, b, h, t, v0, nr, seg + (size_t)(t - ts + 1) * st, a);
            }
            for (int64_t t = te - 1; t >= ts; --t) {
                const int64_t tok = (b * T + t) * H + h;
                const double* qt = J->q + tok * DK;
                const double* kt = J->k + tok * DK;
                const double* vt = J->v + tok * DV;
                const double* dot = J->dO + tok * DV;
                const double* Xp = seg + (size_t)(t - ts) * st;      /* X_{t-1} */
                const double* Xc = seg + (size_t)(t - ts + 1) * st;  /* X_t */
                const int64_t gw = J->vec_gate ? DK : 1;
                memset(acc, 0, sizeof(double) * (size_t)J->part_w);
                for (int64_t j = 0; j < DK; ++j) a[j] = exp(J->vec_gate ? J->g[tok * DK + j] : J->g[tok]);
                if (J->ers) {
                    /* GDN2; acc layout: [dq DK | dk DK | ders DK | dg DK] */
                    const double* et = J->ers + tok * DK;
                    const double* wt = J->wrt + tok * DV;
                    double* adq = acc;
                    double* adk = acc + DK;
                    double* ade = acc + 2 * DK;
                    double* adg = acc + 3 * DK;
                    for (int64_t r = 0; r < nr; ++r) {
                        double u = 0;
                        for (int64_t j = 0; j < DK; ++j) {
                            Pm[r * DK + j] = Xp[r * DK + j] * a[j];
                            u += Pm[r * DK + j] * (et[j] * kt[j]);
                        }
                        e[r] = wt[v0 + r] * vt[v0 + r] - u;
                    }
                    for (int64_t r = 0; r < nr; ++r) {
                        const double dor = dot[v0 + r];
                        double* xb = Xb + r * DK;
                        double sr = 0;
                        for (int64_t j = 0; j < DK; ++j) {
                            xb[j] += dor * qt[j];                 /* Xb += dO q^T */
                            adq[j] += Xc[r * DK + j] * dor;       /* dq = X_t^T dO */
                            sr += xb[j] * kt[j];                  /* s = Xb k (adjoint of e) */
                        }
                        J->dv[tok * DV + v0 + r] = wt[v0 + r] * sr;     /* dv = wrt o s */
                        J->dwrt[tok * DV + v0 + r] = vt[v0 + r] * sr;   /* dwrt = v o s */
                        for (int64_t j = 0; j < DK; ++j) {
                            const double ps = Pm[r * DK + j] * sr;       /* (P^T s)_j part */
                            adk[j] += xb[j] * e[r] - et[j] * ps;
                            ade[j] -= kt[j] * ps;
                            const double pb = xb[j] - sr * (et[j] * kt[j]);  /* Pb */
                            adg[j] += Xp[r * DK + j] * pb * a[j];
                            xb[j] = pb * a[j];                           /* Xb <- Pb Diag(a) */
                        }
                    }
                    if (direct) {
                        for (int64_t j = 0; j < DK; ++j) {
                            J->dq[tok * DK + j] = adq[j];
                            J->dk[tok * DK + j] = adk[j];
                            J->ders[tok * DK + j] = ade[j];
                            J->dg[tok * DK + j] = adg[j];
                        }
                    } else {
                        double* p = J->part + ((size_t)(bh * J->nvb + vb) * (size_t)T + (size_t)t) *
                                                  (size_t)J->part_w;
                        memcpy(p, acc, sizeof(double) * (size_t)J->part_w);
                    }
                    continue;
                }
                const double bt = J->beta[tok];
                /* acc layout: [dq DK | dk DK | dbeta 1 | dg gw] */
                double* adq = acc;
                double* adk = acc + DK;
                double* adb = acc + 2 * DK;
                double* adg = acc + 2 * DK + 1;
                /* P = X_{t-1} Diag(a), e = v - P k */
                for (int64_t r = 0; r < nr; ++r) {
                    double u = 0;
                    for (int64_t j = 0; j < DK; ++j) {
                        Pm[r * DK + j] = Xp[r * DK + j] * a[j];
                        u += Pm[r * DK + j] * kt[j];
                    }
                    e[r] = vt[v0 + r] - u;
                }
                for (int64_t r = 0; r < nr; ++r) {
                    const double dor = dot[v0 + r];
                    double* xb = Xb + r * DK;
                    double wr = 0;
                    for (int64_t j = 0; j < DK; ++j) {
                        xb[j] += dor * qt[j];                 /* Xb += dO q^T */
                        adq[j] += Xc[r * DK + j] * dor;       /* dq = X_t^T dO */
                        wr += xb[j] * kt[j];                  /* w = Xb k */
                    }
                    w[r] = wr;
                    const double ebr = bt * wr;
                    *adb += wr * e[r];                        /* dbeta = <w, e> */
                    J->dv[tok * DV + v0 + r] = ebr;           /* dv = eb */
                    for (int64_t j = 0; j < DK; ++j) {
                        adk[j] += bt * xb[j] * e[r] - Pm[r * DK + j] * ebr;
                        const double pb = xb[j] - ebr * kt[j];   /* Pb */
                        const double ab = Xp[r * DK + j] * pb;   /* abar_j part */
                        if (J->vec_gate) adg[j] += ab * a[j]; else adg[0] += ab * a[j];
                        xb[j] = pb * a[j];                       /* Xb <- Pb Diag(a) */
                    }
                }
                if (direct) {
                    for (int64_t j = 0; j < DK; ++j) {
                        J->dq[tok * DK + j] = adq[j];
                        J->dk[tok * DK + j] = adk[j];
                    }
                    J->dbeta[tok] = *adb;
                    for (int64_t j = 0; j < gw; ++j) J->dg[tok * gw + j] = adg[j];
                } else {
                    double* p = J->part + ((size_t)(bh * J->nvb + vb) * (size_t)T + (size_t)t) *
                                              (size_t)J->part_w;
                    memcpy(p, acc, sizeof(double) * (size_t)J->part_w);
                }
            }
        }
        if (J->dh0)
            for (int64_t r = 0; r < nr; ++r)
                for (int64_t j = 0; j < DK; ++j)
                    J->dh0[((b * H + h) * DK + j) * DV + v0 + r] = Xb[r * DK + j];
    }
out:
    free(ck); free(seg); free(Xb); free(Pm); free(a); free(e); free(w); free(acc);
    return NULL;
}

static int bwd_any(int64_t B, int64_t T, int64_t H, int64_t DK, int64_t DV, int vec_gate,
                   const double* q, const double* k, const double* v, const double* g,
                   const double* beta, const double* ers, const double* wrt, const double* h0,
                   const double* dO, const double* dht, double* dq, double* dk, double* dv,
                   double* dg, double* dbeta, double* ders, double* dwrt, double* dh0,
                   int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || DK < 1 || DV < 1) return 1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.DK = DK; J.DV = DV; J.vec_gate = vec_gate;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0; J.dO = dO; J.dht = dht;
    J.dq = dq; J.dk = dk; J.dv = dv; J.dg = dg; J.dbeta = dbeta; J.dh0 = dh0;
    J.ers = ers; J.wrt = wrt; J.ders = ders; J.dwrt = dwrt;
    if (B * H == 0) return 0;
    if (T == 0) {
        if (dh0)
            for (int64_t i = 0; i < B * H * DK * DV; ++i) dh0[i] = dht ? dht[i] : 0.0;
        return 0;
    }
    split_rows(&J);
    const int gdn2 = ers != NULL;
    const int64_t gw = vec_gate ? DK : 1;
    J.part_w = gdn2 ? 4 * DK : 2 * DK + 1 + gw;
    if (J.nvb > 1) {
        J.part = (double*)malloc(sizeof(double) * (size_t)(B * H * J.nvb) * (size_t)T *
                                 (size_t)J.part_w);
        if (!J.part) return 1;
    }
    int rc = run_threads(&J, bwd_worker, nthreads);
    if (rc == 0 && J.nvb > 1) {
        /* fixed-order reduction over value-row blocks */
        for (int64_t bh = 0; bh < B * H; ++bh) {
            const int64_t b = bh / H, h = bh % H;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t tok = (b * T + t) * H + h;
                for (int64_t x = 0; x < J.part_w; ++x) {
                    double s = 0;
                    for (int64_t vb = 0; vb < J.nvb; ++vb)
                        s += J.part[((size_t)(bh * J.nvb + vb) * (size_t)T + (size_t)t) *
                                        (size_t)J.part_w + (size_t)x];
                    if (x < DK) dq[tok * DK + x] = s;
                    else if (x < 2 * DK) dk[tok * DK + x - DK] = s;
                    else if (gdn2 && x < 3 * DK) ders[tok * DK + x - 2 * DK] = s;
                    else if (gdn2) dg[tok * DK + x - 3 * DK] = s;
                    else if (x == 2 * DK) dbeta[tok] = s;
                    else dg[tok * gw + (x - 2 * DK - 1)] = s;
                }
            }
        }
    }
    free(J.part);
    return rc;
}

int gdr_oracle_bwd(int64_t B, int64_t T, int64_t H, int64_t DK, int64_t DV, int vec_gate,
                   const double* q, const double* k, const double* v, const double* g,
                   const double* beta, const double* h0, const double* dO, const double* dht,
                   double* dq, double* dk, double* dv, double* dg, double* dbeta, double* dh0,
                   int nthreads)
{
    return bwd_any(B, T, H, DK, DV, vec_gate, q, k, v, g, beta, NULL, NULL, h0, dO, dht, dq, dk,
                   dv, dg, dbeta, NULL, NULL, dh0, nthreads);
}

int gdr_oracle_gdn2_bwd(int64_t B, int64_t T, int64_t H, int64_t DK, int64_t DV,
                        const double* q, const double* k, const double* v, const double* g,
                        const double* ers, const double* wrt, const double* h0, const double* dO,
                        const double* dht, double* dq, double* dk, double* dv, double* dg,
                        double* ders, double* dwrt, double* dh0, int nthreads)
{
    if (!ers || !wrt || !ders || !dwrt) return 1;
    return bwd_any(B, T, H, DK, DV, 1, q, k, v, g, NULL, ers, wrt, h0, dO, dht, dq, dk, dv, dg,
                   NULL, ders, dwrt, dh0, nthreads);
}
