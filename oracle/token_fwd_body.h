/*
 * Forward body of the token-by-token gated delta rule, written once and
 * instantiated twice by gdr_oracle.c: with SCALAR = double (the reference
 * itself) and with SCALAR = double complex (complex-step derivative checks).
 *
 * TEST INFRASTRUCTURE: part of the fp64 CPU oracle. Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.
 *
 * Recurrence (ReWY paper, Sec. 2.2 "Delta-rule operators" and Table 1): per
 * head, with the state X in value-by-key form (DV x DK),
 *     P   = X_{t-1} Diag(a_t)              decay first, a_t = exp(g_t)
 *     u   = P k_t                          prediction from the decayed state
 *     e   = v_t - u                        correction
 *     X_t = P + beta_t e k_t^T             rank-one write along k_t
 *     o_t = X_t q_t                        the output reads the updated state
 * This equals X_t = X_{t-1} Diag(a_t)(I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
 * A scalar gate (GDN) broadcasts one log decay over the DK channels; a vector
 * gate (KDA) carries one log decay per key channel.
 *
 * GDN2 (Table 1: vector decay, independent vector erase and write gates;
 * ers and wrt non-NULL, beta unused): the prediction reads the decayed state
 * with the erase-gated key, the correction starts from the write-gated value,
 * and the write goes along k itself:
 *     u = P (ers_t o k_t),   e = wrt_t o v_t - u,   X_t = P + e k_t^T
 * (ers_t per key channel, wrt_t per value channel). With ers_t = wrt_t =
 * beta_t in every channel this is the KDA step above.
 *
 * The body works on the value rows [v0, v1) of one (b, h): the rows of X are
 * independent in the forward pass, so a caller may split them across threads.
 */
#ifndef FWD_NAME
#error "define FWD_NAME, SCALAR and SEXP before including token_fwd_body.h"
#endif

static void FWD_NAME(int64_t T, int64_t H, int64_t DK, int64_t DV, int vec_gate,
                     int64_t b, int64_t h, int64_t v0, int64_t v1,
                     const SCALAR* q, const SCALAR* k, const SCALAR* v,
                     const SCALAR* g, const SCALAR* beta, const SCALAR* ers,
                     const SCALAR* wrt, const SCALAR* h0,
                     SCALAR* o, SCALAR* ht, SCALAR* X, SCALAR* a)
{
    const int64_t nr = v1 - v0;
    /* X[r][j] = h0[b,h,j,v0+r]  (h0 is stored key-major: [B,H,DK,DV]) */
    for (int64_t r = 0; r < nr; ++r)
        for (int64_t j = 0; j < DK; ++j)
            X[r * DK + j] = h0 ? h0[((b * H + h) * DK + j) * DV + v0 + r] : (SCALAR)0;

    for (int64_t t = 0; t < T; ++t) {
        const int64_t tok = (b * T + t) * H + h;
        const SCALAR* qt = q + tok * DK;
        const SCALAR* kt = k + tok * DK;
        const SCALAR* vt = v + tok * DV;
        for (int64_t j = 0; j < DK; ++j)
            a[j] = SEXP(vec_gate ? g[tok * DK + j] : g[tok]);
        if (ers) {
            /* GDN2 */
            const SCALAR* et = ers + tok * DK;
            const SCALAR* wt = wrt + tok * DV;
            for (int64_t r = 0; r < nr; ++r) {
                SCALAR* x = X + r * DK;
                SCALAR u = 0;
                for (int64_t j = 0; j < DK; ++j) {
                    x[j] = x[j] * a[j];               /* P = X Diag(a) */
                    u += x[j] * (et[j] * kt[j]);      /* u = P (ers o k) */
                }
                const SCALAR e = wt[v0 + r] * vt[v0 + r] - u;
                SCALAR out = 0;
                for (int64_t j = 0; j < DK; ++j) {
                    x[j] = x[j] + e * kt[j];          /* X = P + e k^T */
                    out += x[j] * qt[j];              /* o = X q */
                }
                o[tok * DV + v0 + r] = out;
            }
            continue;
        }
        const SCALAR bt = beta[tok];
        for (int64_t r = 0; r < nr; ++r) {
            SCALAR* x = X + r * DK;
            SCALAR u = 0;
            for (int64_t j = 0; j < DK; ++j) {
                x[j] = x[j] * a[j];          /* P = X Diag(a) */
                u += x[j] * kt[j];           /* u = P k */
            }
            const SCALAR e = vt[v0 + r] - u;
            SCALAR out = 0;
            for (int64_t j = 0; j < DK; ++j) {
                x[j] = x[j] + bt * e * kt[j];  /* X = P + beta e k^T */
                out += x[j] * qt[j];            /* o = X q */
            }
            o[tok * DV + v0 + r] = out;
        }
    }
    if (ht)
        for (int64_t r = 0; r < nr; ++r)
            for (int64_t j = 0; j < DK; ++j)
                ht[((b * H + h) * DK + j) * DV + v0 + r] = X[r * DK + j];
}
