/*
 * kdn_oracle.c -- fp64 CPU oracle of the gated delta-rule / diagonal-Kalman
 * associative-memory recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU
 * baseline leg of the benchmark are the only users of this file.  The HIP
 * library and its Python binding never load, link or call it, and the two
 * share no source: no header, no helper, no constant.
 *
 * What it computes is the plain token-by-token recurrence, in double
 * precision, in the order the pages give the steps.  No blocking, no chunking,
 * no reordering.  Pages cited (title, then the section used):
 *
 *   [TAB] "Внимание в LLM · часть 11 -- Память с поправкой" (tutorial on the
 *         delta rule): section "Сначала решить, сколько прошлого оставить"
 *         (gated state S_t = a_t S_{t-1} + w_t) and section "Записать не новое
 *         значение, а ошибку памяти" (read v^ = S^T k, compare e = v - v^,
 *         correct S += beta k e^T).
 *   [KDA] "معماری KDA: حذف تداخل حافظه با قانون دلتا در توالی‌های بلند" (Kimi
 *         Delta Attention article): section "تکامل قانون دلتا" (delta rule,
 *         beta = 1 replaces exactly) and section "از فراموشی کلی به فراموشی
 *         جزئی" (scalar retention applied to the whole state before the delta
 *         write; vector retention, one rate per key channel).
 *   [KDN] "给记忆装一个信任度探测器：Kalman Delta Networks 如何让AI知道自己
 *         "记得准不准"" (write-up of Kalman Delta Networks): section
 *         "把记忆问题重新想成一个滤波问题" (predict, then update with a gain
 *         derived from memory uncertainty and observation reliability) and
 *         section "对角近似：把矩阵压扁成一个向量" (diagonal covariance,
 *         per-channel update, mean-field projection whose mean is exact,
 *         information scaling mu of the precision increment).
 *         Isotropic KDN: section "各向同性近似：把整个头压缩成一个数" (one
 *         uncertainty scalar per head; the delta-rule form is kept and its
 *         scalar write strength is derived from the accumulated uncertainty
 *         and the observation reliability; otherwise shaped like KDA; the
 *         variance recursion is a Mobius map).
 *   [AFS] "Kalman Delta Networks: Uncertainty-aware Associative Memory"
 *         (explainer): section "Approximation 1: Diagonal KDN (Mean-Field
 *         Variational Inference)" and section "Approximation 2: Isotropic
 *         KDN (Single Scalar Uncertainty)".
 *
 * Readings of points the pages leave open (each is argued in the design
 * notes of the repository):
 *   - S is d_k x d_v and the read is v^ = S^T k.
 *   - The decay is applied before the read (Kalman predict, then update).
 *   - The output is read after the write: o_t = S_t^T q_t, with no scale.
 *   - Diagonal KDN predict: p- = a*a*p + xi (process noise xi per channel).
 *   - Gain: w = p- (.) k / s with s = r + sum_i p-_i k_i^2; this is the exact
 *     Kalman update of the mean under the diagonal prior, so the mean is exact.
 *   - Projection: the diagonal precision gains mu k_i^2 / r, i.e.
 *     p_i <- p-_i r / (r + mu p-_i k_i^2).  mu scales only the variance
 *     update, never the current write.
 *   - Degenerate values: s == 0 gives w = 0; r + mu p-_i k_i^2 == 0 leaves
 *     p_i = p-_i.
 *   - Isotropic KDN (covariance p I): the predict p I -> diag(a^2) p +
 *     diag(xi) is brought back to a multiple of I by the mean of its
 *     diagonal, p- = mean(a^2) p + mean(xi); the gain is exact under p- I,
 *     w = p- k / s with s = r + p- |k|^2 (write strength p- / s times k);
 *     the posterior precision I / p- + k k^T / r is brought back to a
 *     multiple of I by the mean of its diagonal, scaled by mu like the
 *     diagonal variant: 1/p = 1/p- + mu |k|^2 / (d_k r), i.e.
 *     p <- p- r / (r + (mu / d_k) p- |k|^2).  Degenerate values as above.
 *
 * Layouts (row-major, contiguous):
 *   q, k            [B, T, H, dk]       v, o        [B, T, H, dv]
 *   alpha           GDN: [B, T, H]      KDA/KDN:    [B, T, H, dk]
 *   beta            [B, T, H]           (not KDN)
 *   xi (proc noise) [B, T, H, dk]       r (obs noise) [B, T, H]   (KDN only)
 *   S0, S           [B, H, dk, dv]      p0, p       [B, H, dk] (isotropic: [B, H])
 *   xi and r as for diagonal KDN for the isotropic variant too.
 *
 * Variant codes: 0 DeltaNet, 1 Gated DeltaNet, 2 KDA, 3 diagonal KDN,
 * 4 isotropic KDN.
 */
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_DELTANET = 0, ORC_GATED_DELTANET = 1, ORC_KDA = 2, ORC_DIAG_KDN = 3,
       ORC_ISO_KDN = 4 };

/* One (batch, head) stream, tokens 0..T-1.  S (dk x dv) and p (dk; one value
 * for isotropic KDN) are the running state and are updated in place. */
static void run_stream(int variant, long T, long H, long dk, long dv, double mu,
                       const double *q, const double *k, const double *v,
                       const double *alpha, const double *beta,
                       const double *xi, const double *r,
                       long b, long h, double *S, double *p, double *o,
                       double *a, double *w, double *e, double *pm)
{
    for (long t = 0; t < T; ++t) {
        const long tok = (b * T + t) * H + h;          /* index of (b,t,h) */
        const double *kt = k + tok * dk;
        const double *qt = q + tok * dk;
        const double *vt = v + tok * dv;

        /* 1. Decay vector: none, one rate for the whole state, or one rate
         *    per key channel ([TAB] gated state; [KDA] scalar -> vector). */
        for (long i = 0; i < dk; ++i) {
            if (variant == ORC_DELTANET)
                a[i] = 1.0;
            else if (variant == ORC_GATED_DELTANET)
                a[i] = alpha[tok];
            else
                a[i] = alpha[tok * dk + i];
        }

        /* 2. Write vector. */
        if (variant == ORC_DIAG_KDN) {
            /* Kalman predict of the per-channel variance ([KDN] filtering
             * section: predict tracks uncertainty under the drift). */
            for (long i = 0; i < dk; ++i)
                pm[i] = a[i] * a[i] * p[i] + xi[tok * dk + i];
            /* Innovation variance and gain under the diagonal prior ([KDN]
             * gain from uncertainty and observation reliability; diagonal
             * section: the projected mean is exact). */
            const double rt = r[tok];
            double s = rt;
            for (long i = 0; i < dk; ++i)
                s += pm[i] * kt[i] * kt[i];
            for (long i = 0; i < dk; ++i)
                w[i] = (s != 0.0) ? pm[i] * kt[i] / s : 0.0;
            /* Mean-field projection back to a diagonal: precision of channel
             * i grows by mu * k_i^2 / r ([KDN] diagonal section, information
             * scaling; [AFS] Approximation 1). */
            for (long i = 0; i < dk; ++i) {
                const double den = rt + mu * pm[i] * kt[i] * kt[i];
                p[i] = (den != 0.0) ? pm[i] * rt / den : pm[i];
            }
        } else if (variant == ORC_ISO_KDN) {
            /* One variance for the whole head ([KDN] isotropic section):
             * predict, brought back to a multiple of the identity by the mean
             * of the diagonal. */
            double a2 = 0.0, xm = 0.0, kk = 0.0;
            for (long i = 0; i < dk; ++i) {
                a2 += a[i] * a[i];
                xm += xi[tok * dk + i];
                kk += kt[i] * kt[i];
            }
            const double pmi = (a2 / (double)dk) * p[0] + xm / (double)dk;
            /* Exact gain under the isotropic prior: the delta rule with the
             * write strength pmi / s derived from the uncertainty and the
             * observation reliability. */
            const double rt = r[tok];
            const double s = rt + pmi * kk;
            for (long i = 0; i < dk; ++i)
                w[i] = (s != 0.0) ? pmi * kt[i] / s : 0.0;
            /* Precision gain averaged over the key channels, scaled by mu. */
            const double den = rt + (mu / (double)dk) * pmi * kk;
            p[0] = (den != 0.0) ? pmi * rt / den : pmi;
        } else {
            /* Delta rule write strength beta ([TAB] correct step). */
            const double bt = beta[tok];
            for (long i = 0; i < dk; ++i)
                w[i] = bt * kt[i];
        }

        /* 3. Decay the memory before the delta write ([KDA] forgetting). */
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] *= a[i];

        /* 4. Read and compare: e = v - S^T k ([TAB] steps 1 and 2). */
        for (long j = 0; j < dv; ++j)
            e[j] = 0.0;
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                e[j] += S[i * dv + j] * kt[i];
        for (long j = 0; j < dv; ++j)
            e[j] = vt[j] - e[j];

        /* 5. Correct: S += w e^T ([TAB] step 3). */
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                S[i * dv + j] += w[i] * e[j];

        /* 6. Read the output from the updated memory: o = S^T q. */
        double *ot = o + tok * dv;
        for (long j = 0; j < dv; ++j)
            ot[j] = 0.0;
        for (long i = 0; i < dk; ++i)
            for (long j = 0; j < dv; ++j)
                ot[j] += S[i * dv + j] * qt[i];
    }
}

/* Returns 0 on success, a negative code on a bad argument.  S0 may be NULL
 * (zero initial memory); p0 and p are used by diagonal KDN only.  S and p
 * receive the final state and may alias S0 and p0 exactly.  nthreads <= 0
 * uses the OpenMP default. */
int kdn_oracle_recurrence(int variant, long B, long T, long H, long dk, long dv,
                          double mu,
                          const double *q, const double *k, const double *v,
                          const double *alpha, const double *beta,
                          const double *xi, const double *r,
                          const double *S0, const double *p0,
                          double *o, double *S, double *p, int nthreads)
{
    if (variant < ORC_DELTANET || variant > ORC_ISO_KDN)
        return -1;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -2;
    if (!q || !k || !v || !o || !S)
        return -3;
    if (variant != ORC_DELTANET && !alpha)
        return -4;
    const int kdn = variant == ORC_DIAG_KDN || variant == ORC_ISO_KDN;
    const long np = variant == ORC_DIAG_KDN ? dk : 1;   /* variances per stream */
    if (!kdn && !beta)
        return -5;
    if (kdn && (!xi || !r || !p0 || !p))
        return -6;

    const long BH = B * H;
    int fail = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (long bh = 0; bh < BH; ++bh) {
        const long b = bh / H, h = bh % H;
        double *Sb = S + bh * dk * dv;
        double *pb = kdn ? p + bh * np : NULL;
        if (S0) {
            if (S0 + bh * dk * dv != Sb)
                memcpy(Sb, S0 + bh * dk * dv, sizeof(double) * dk * dv);
        } else {
            memset(Sb, 0, sizeof(double) * dk * dv);
        }
        if (pb && p0 + bh * np != pb)
            memcpy(pb, p0 + bh * np, sizeof(double) * np);

        double *scratch = (double *)malloc(sizeof(double) * (3 * dk + dv));
        if (!scratch) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            fail = 1;
            continue;
        }
        double *a = scratch, *w = scratch + dk, *pm = scratch + 2 * dk;
        double *e = scratch + 3 * dk;
        run_stream(variant, T, H, dk, dv, mu, q, k, v, alpha, beta, xi, r,
                   b, h, Sb, pb, o, a, w, e, pm);
        free(scratch);
    }
    return fail ? -7 : 0;
}

/* Number of threads an OpenMP region started here would use. */
int kdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* --------------------------------------------------------------------------
 * Gradients of the recurrence for the write-strength variants (DeltaNet,
 * Gated DeltaNet, KDA).
 *
 * The pages give no gradient.  What is computed here is the exact derivative
 * of the recurrence above by reverse-mode differentiation of its steps, token
 * by token in reverse order.  For a scalar loss L with dL/do_t = do_t and
 * dL/dS_T = dS_T (S_t: the memory after token t, S_0 the initial one):
 *   step 6  o_t = S_t^T q_t:         dS_t += q_t do_t^T,  dq_t = S_t do_t
 *   step 5  S_t = S- + w e^T:        dw = dS_t e_t,  de = dS_t^T w,  dv_t = de
 *   step 4  e = v_t - S-^T k_t:      dS- = dS_t - k_t de^T,  dk_t = -S- de
 *   step 2  w = beta_t k_t:          dk_t += beta_t dw,  dbeta_t = k_t . dw
 *   step 3  S- = diag(a_t) S_{t-1}:  da_t,i = sum_j dS-[i,j] S_{t-1}[i,j],
 *                                    dS_{t-1} = diag(a_t) dS-
 * and dS_0 is the gradient of the initial memory.  The decay gradient is
 * returned per token for Gated DeltaNet (sum over channels of da_t) and per
 * token and channel for KDA.  The memories S_0 .. S_T of one stream are kept
 * (T + 1 matrices of dk x dv).
 * ------------------------------------------------------------------------ */

/* Steps 1-5 of one token for the write-strength variants: S_prev -> S_next,
 * with S- (the decayed memory) and the error e left in Sm and e. */
static void step_beta(int variant, long dk, long dv, long tok, const double *k,
                      const double *v, const double *alpha, const double *beta,
                      const double *S_prev, double *S_next, double *Sm,
                      double *a, double *e)
{
    const double *kt = k + tok * dk;
    const double *vt = v + tok * dv;
    for (long i = 0; i < dk; ++i)
        a[i] = variant == ORC_DELTANET ? 1.0
             : (variant == ORC_GATED_DELTANET ? alpha[tok] : alpha[tok * dk + i]);
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j)
            Sm[i * dv + j] = a[i] * S_prev[i * dv + j];
    for (long j = 0; j < dv; ++j) {
        double r = 0.0;
        for (long i = 0; i < dk; ++i)
            r += Sm[i * dv + j] * kt[i];
        e[j] = vt[j] - r;
    }
    const double bt = beta[tok];
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j)
            S_next[i * dv + j] = Sm[i * dv + j] + bt * kt[i] * e[j];
}

/* Returns 0 on success, a negative code on a bad argument.  S0 and dS_T may
 * be NULL (zero).  Gradients: dq, dk [B,T,H,dk]; dv [B,T,H,dv]; dalpha
 * [B,T,H] (Gated DeltaNet) or [B,T,H,dk] (KDA), NULL for DeltaNet; dbeta
 * [B,T,H]; dS0 [B,H,dk,dv]. */
int kdn_oracle_backward(int variant, long B, long T, long H, long dk, long dv,
                        const double *q, const double *k, const double *v,
                        const double *alpha, const double *beta, const double *S0,
                        const double *dO, const double *dS_T,
                        double *dq, double *dk_out, double *dv_out,
                        double *dalpha, double *dbeta, double *dS0, int nthreads)
{
    if (variant < ORC_DELTANET || variant > ORC_KDA)
        return -1;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -2;
    if (!q || !k || !v || !beta || !dO || !dq || !dk_out || !dv_out || !dbeta || !dS0)
        return -3;
    if (variant != ORC_DELTANET && (!alpha || !dalpha))
        return -4;

    const long BH = B * H, SZ = dk * dv;
    int fail = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (long bh = 0; bh < BH; ++bh) {
        const long b = bh / H, h = bh % H;
        double *Sall = (double *)malloc(sizeof(double) * (T + 1) * SZ);
        double *buf = (double *)malloc(sizeof(double) * (3 * SZ + 2 * dk + 2 * dv));
        if (!Sall || !buf) {
            free(Sall);
            free(buf);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            fail = 1;
            continue;
        }
        double *Sm = buf, *dS = buf + SZ, *dSm = buf + 2 * SZ;
        double *a = buf + 3 * SZ, *dw = a + dk, *e = dw + dk, *de = e + dv;

        /* forward: the memories after every token */
        if (S0)
            memcpy(Sall, S0 + bh * SZ, sizeof(double) * SZ);
        else
            memset(Sall, 0, sizeof(double) * SZ);
        for (long t = 0; t < T; ++t) {
            const long tok = (b * T + t) * H + h;
            step_beta(variant, dk, dv, tok, k, v, alpha, beta, Sall + t * SZ,
                      Sall + (t + 1) * SZ, Sm, a, e);
        }

        /* reverse */
        if (dS_T)
            memcpy(dS, dS_T + bh * SZ, sizeof(double) * SZ);
        else
            memset(dS, 0, sizeof(double) * SZ);
        for (long t = T - 1; t >= 0; --t) {
            const long tok = (b * T + t) * H + h;
            const double *qt = q + tok * dk, *kt = k + tok * dk;
            const double *dot = dO + tok * dv;
            const double *St = Sall + (t + 1) * SZ, *Sp = Sall + t * SZ;
            /* step 6 */
            for (long i = 0; i < dk; ++i) {
                double r = 0.0;
                for (long j = 0; j < dv; ++j) {
                    dS[i * dv + j] += qt[i] * dot[j];
                    r += St[i * dv + j] * dot[j];
                }
                dq[tok * dk + i] = r;
            }
            /* recompute S- and e of this token (dSm receives the recomputed
             * S_t, unused, and is overwritten below) */
            step_beta(variant, dk, dv, tok, k, v, alpha, beta, Sp, dSm, Sm, a, e);
            const double bt = beta[tok];
            /* step 5 */
            for (long i = 0; i < dk; ++i) {
                double r = 0.0;
                for (long j = 0; j < dv; ++j)
                    r += dS[i * dv + j] * e[j];
                dw[i] = r;
            }
            for (long j = 0; j < dv; ++j) {
                double r = 0.0;
                for (long i = 0; i < dk; ++i)
                    r += dS[i * dv + j] * bt * kt[i];
                de[j] = r;
                dv_out[tok * dv + j] = r;
            }
            /* steps 4 and 2 */
            double db = 0.0;
            for (long i = 0; i < dk; ++i) {
                double r = 0.0;
                for (long j = 0; j < dv; ++j) {
                    dSm[i * dv + j] = dS[i * dv + j] - kt[i] * de[j];
                    r += Sm[i * dv + j] * de[j];
                }
                dk_out[tok * dk + i] = -r + bt * dw[i];
                db += kt[i] * dw[i];
            }
            dbeta[tok] = db;
            /* step 3 */
            double dag = 0.0;
            for (long i = 0; i < dk; ++i) {
                double r = 0.0;
                for (long j = 0; j < dv; ++j) {
                    r += dSm[i * dv + j] * Sp[i * dv + j];
                    dS[i * dv + j] = a[i] * dSm[i * dv + j];
                }
                if (variant == ORC_KDA)
                    dalpha[tok * dk + i] = r;
                dag += r;
            }
            if (variant == ORC_GATED_DELTANET)
                dalpha[tok] = dag;
        }
        memcpy(dS0 + bh * SZ, dS, sizeof(double) * SZ);
        free(Sall);
        free(buf);
    }
    return fail ? -7 : 0;
}

/* --------------------------------------------------------------------------
 * Gradients for isotropic KDN.  The write strength is derived, per token,
 * from the head variance (forward step 2, isotropic branch):
 *   p- = a2 p + xm,  s = r + p- kk,  beta = p- / s (0 if s = 0),
 *   den = r + m p- kk (m = mu / dk),  p' = p- r / den (p- if den = 0),
 * with a2 = mean(a^2), xm = mean(xi), kk = |k|^2.  Reverse mode: the memory
 * part is the write-strength backward above with that beta, giving dbeta_t;
 * then, with dp the gradient of p' (from the later tokens, dp_T at the end):
 *   s != 0:   dp- += dbeta r / s^2,  dkk -= dbeta p-^2 / s^2,  dr -= dbeta p- / s^2
 *   den != 0: dp- += dp r^2 / den^2, dkk -= dp m p-^2 r / den^2,
 *             dr += dp m p-^2 kk / den^2;        den = 0: dp- += dp
 *   da2 = dp- p,  dxm = dp-,  and the gradient of the previous p is dp- a2;
 *   dalpha_i += da2 2 a_i / dk,  dxi_i = dxm / dk,  dk_i += dkk 2 k_i.
 * dp0 is the gradient of the initial variance.
 * ------------------------------------------------------------------------ */
int kdn_oracle_backward_iso(long B, long T, long H, long dk, long dv, double mu,
                            const double *q, const double *k, const double *v,
                            const double *alpha, const double *xi, const double *r,
                            const double *S0, const double *p0,
                            const double *dO, const double *dS_T, const double *dp_T,
                            double *dq, double *dk_out, double *dv_out, double *dalpha,
                            double *dxi, double *dr, double *dS0, double *dp0,
                            int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -2;
    if (!q || !k || !v || !alpha || !xi || !r || !p0 || !dO || !dq || !dk_out ||
        !dv_out || !dalpha || !dxi || !dr || !dS0 || !dp0)
        return -3;
    const long BH = B * H, SZ = dk * dv;
    const long NTOK = B * T * H;
    /* the derived write strengths, as a beta tensor for the memory part */
    double *beta = (double *)malloc(sizeof(double) * (NTOK > 0 ? NTOK : 1));
    double *dbeta = (double *)malloc(sizeof(double) * (NTOK > 0 ? NTOK : 1));
    double *pprev = (double *)malloc(sizeof(double) * (NTOK > 0 ? NTOK : 1));
    if (!beta || !dbeta || !pprev) {
        free(beta); free(dbeta); free(pprev);
        return -7;
    }
    const double m = mu / (double)dk;
    for (long bh = 0; bh < BH; ++bh) {
        const long b = bh / H, h = bh % H;
        double p = p0[bh];
        for (long t = 0; t < T; ++t) {
            const long tok = (b * T + t) * H + h;
            double a2 = 0.0, xm = 0.0, kk = 0.0;
            for (long i = 0; i < dk; ++i) {
                a2 += alpha[tok * dk + i] * alpha[tok * dk + i];
                xm += xi[tok * dk + i];
                kk += k[tok * dk + i] * k[tok * dk + i];
            }
            a2 /= (double)dk;
            xm /= (double)dk;
            pprev[tok] = p;
            const double pm = a2 * p + xm;
            const double s = r[tok] + pm * kk;
            beta[tok] = (s != 0.0) ? pm / s : 0.0;
            const double den = r[tok] + m * pm * kk;
            p = (den != 0.0) ? pm * r[tok] / den : pm;
        }
    }
    int rc = kdn_oracle_backward(ORC_KDA, B, T, H, dk, dv, q, k, v, alpha, beta, S0, dO,
                                 dS_T, dq, dk_out, dv_out, dalpha, dbeta, dS0, nthreads);
    if (rc == 0) {
        for (long bh = 0; bh < BH; ++bh) {
            const long b = bh / H, h = bh % H;
            double dp = dp_T ? dp_T[bh] : 0.0;
            for (long t = T - 1; t >= 0; --t) {
                const long tok = (b * T + t) * H + h;
                double a2 = 0.0, xm = 0.0, kk = 0.0;
                for (long i = 0; i < dk; ++i) {
                    a2 += alpha[tok * dk + i] * alpha[tok * dk + i];
                    xm += xi[tok * dk + i];
                    kk += k[tok * dk + i] * k[tok * dk + i];
                }
                a2 /= (double)dk;
                xm /= (double)dk;
                const double pp = pprev[tok], rt = r[tok];
                const double pm = a2 * pp + xm;
                const double s = rt + pm * kk, den = rt + m * pm * kk;
                const double db = dbeta[tok];
                double dpm = 0.0, dkk = 0.0, drt = 0.0;
                if (s != 0.0) {
                    dpm += db * rt / (s * s);
                    dkk -= db * pm * pm / (s * s);
                    drt -= db * pm / (s * s);
                }
                if (den != 0.0) {
                    dpm += dp * rt * rt / (den * den);
                    dkk -= dp * m * pm * pm * rt / (den * den);
                    drt += dp * m * pm * pm * kk / (den * den);
                } else {
                    dpm += dp;
                }
                const double da2 = dpm * pp;
                for (long i = 0; i < dk; ++i) {
                    dalpha[tok * dk + i] += da2 * 2.0 * alpha[tok * dk + i] / (double)dk;
                    dxi[tok * dk + i] = dpm / (double)dk;
                    dk_out[tok * dk + i] += dkk * 2.0 * k[tok * dk + i];
                }
                dr[tok] = drt;
                dp = dpm * a2;
            }
            dp0[bh] = dp;
        }
    }
    free(beta);
    free(dbeta);
    free(pprev);
    return rc;
}

/* --------------------------------------------------------------------------
 * Gradients for diagonal KDN.  Per token the write vector is the gain
 *   p-_i = a_i^2 p_i + xi_i,  s = r + sum_i p-_i k_i^2,  w_i = p-_i k_i / s,
 * and the variance update is p'_i = p-_i r / den_i, den_i = r + mu p-_i k_i^2
 * (s = 0: w = 0; den_i = 0: p'_i = p-_i).  Reverse mode: first the memory with
 * the write vector as given (as in the write-strength backward, without the
 * beta factor), which yields dw_t; then, per token in reverse, with dp_i the
 * gradient of p'_i from the later tokens (dp_T at the end):
 *   u_i = p-_i k_i:  du_i = dw_i / s,  ds = -sum_i dw_i u_i / s^2   (s != 0)
 *   dp-_i = du_i k_i + ds k_i^2 + dp_i r^2 / den_i^2    (dp_i if den_i = 0)
 *   dk_i += du_i p-_i + 2 ds p-_i k_i - 2 dp_i mu p-_i^2 r k_i / den_i^2
 *   dr = ds + sum_i dp_i mu p-_i^2 k_i^2 / den_i^2
 *   dalpha_i += 2 a_i p_i dp-_i,  dxi_i = dp-_i,  previous dp_i = a_i^2 dp-_i.
 * dp0 is the gradient of the initial variances.
 * ------------------------------------------------------------------------ */

/* Memory part for a given write vector W [B,T,H,dk] and per-channel decay:
 * the write-strength backward's steps 6, 5, 4 and 3 with w = W_t; returns dW
 * in place of dbeta and only the read term in dk. */
static int backward_memory_w(long B, long T, long H, long dk, long dv,
                             const double *q, const double *k, const double *v,
                             const double *alpha, const double *W, const double *S0,
                             const double *dO, const double *dS_T, double *dq,
                             double *dk_out, double *dv_out, double *dalpha, double *dW,
                             double *dS0)
{
    const long BH = B * H, SZ = dk * dv;
    for (long bh = 0; bh < BH; ++bh) {
        const long b = bh / H, h = bh % H;
        double *Sall = (double *)malloc(sizeof(double) * (T + 1) * SZ);
        double *buf = (double *)malloc(sizeof(double) * (3 * SZ + 2 * dv));
        if (!Sall || !buf) {
            free(Sall);
            free(buf);
            return -7;
        }
        double *Sm = buf, *dS = buf + SZ, *dSm = buf + 2 * SZ, *e = buf + 3 * SZ, *de = e + dv;
        if (S0)
            memcpy(Sall, S0 + bh * SZ, sizeof(double) * SZ);
        else
            memset(Sall, 0, sizeof(double) * SZ);
        /* forward: S_t = diag(a) S_{t-1} + w (v - (diag(a) S_{t-1})^T k)^T */
        for (long t = 0; t < T; ++t) {
            const long tok = (b * T + t) * H + h;
            const double *Sp = Sall + t * SZ;
            double *Sn = Sall + (t + 1) * SZ;
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j)
                    Sm[i * dv + j] = alpha[tok * dk + i] * Sp[i * dv + j];
            for (long j = 0; j < dv; ++j) {
                double rr = 0.0;
                for (long i = 0; i < dk; ++i)
                    rr += Sm[i * dv + j] * k[tok * dk + i];
                e[j] = v[tok * dv + j] - rr;
            }
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j)
                    Sn[i * dv + j] = Sm[i * dv + j] + W[tok * dk + i] * e[j];
        }
        if (dS_T)
            memcpy(dS, dS_T + bh * SZ, sizeof(double) * SZ);
        else
            memset(dS, 0, sizeof(double) * SZ);
        for (long t = T - 1; t >= 0; --t) {
            const long tok = (b * T + t) * H + h;
            const double *qt = q + tok * dk, *kt = k + tok * dk, *wt = W + tok * dk;
            const double *dot = dO + tok * dv;
            const double *St = Sall + (t + 1) * SZ, *Sp = Sall + t * SZ;
            for (long i = 0; i < dk; ++i) {
                double rr = 0.0;
                for (long j = 0; j < dv; ++j) {
                    dS[i * dv + j] += qt[i] * dot[j];
                    rr += St[i * dv + j] * dot[j];
                }
                dq[tok * dk + i] = rr;
            }
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j)
                    Sm[i * dv + j] = alpha[tok * dk + i] * Sp[i * dv + j];
            for (long j = 0; j < dv; ++j) {
                double rr = 0.0, rd = 0.0;
                for (long i = 0; i < dk; ++i) {
                    rr += Sm[i * dv + j] * kt[i];
                    rd += dS[i * dv + j] * wt[i];
                }
                e[j] = v[tok * dv + j] - rr;
                de[j] = rd;
                dv_out[tok * dv + j] = rd;
            }
            for (long i = 0; i < dk; ++i) {
                double rw = 0.0, rk = 0.0;
                for (long j = 0; j < dv; ++j) {
                    rw += dS[i * dv + j] * e[j];
                    dSm[i * dv + j] = dS[i * dv + j] - kt[i] * de[j];
                    rk += Sm[i * dv + j] * de[j];
                }
                dW[tok * dk + i] = rw;
                dk_out[tok * dk + i] = -rk;
            }
            for (long i = 0; i < dk; ++i) {
                double ra = 0.0;
                for (long j = 0; j < dv; ++j) {
                    ra += dSm[i * dv + j] * Sp[i * dv + j];
                    dS[i * dv + j] = alpha[tok * dk + i] * dSm[i * dv + j];
                }
                dalpha[tok * dk + i] = ra;
            }
        }
        memcpy(dS0 + bh * SZ, dS, sizeof(double) * SZ);
        free(Sall);
        free(buf);
    }
    return 0;
}

int kdn_oracle_backward_diag(long B, long T, long H, long dk, long dv, double mu,
                             const double *q, const double *k, const double *v,
                             const double *alpha, const double *xi, const double *r,
                             const double *S0, const double *p0,
                             const double *dO, const double *dS_T, const double *dp_T,
                             double *dq, double *dk_out, double *dv_out, double *dalpha,
                             double *dxi, double *dr, double *dS0, double *dp0)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -2;
    if (!q || !k || !v || !alpha || !xi || !r || !p0 || !dO || !dq || !dk_out ||
        !dv_out || !dalpha || !dxi || !dr || !dS0 || !dp0)
        return -3;
    const long BH = B * H, NTOK = B * T * H;
    const long NV = (NTOK > 0 ? NTOK : 1) * dk;
    double *W = (double *)malloc(sizeof(double) * NV);
    double *dW = (double *)malloc(sizeof(double) * NV);
    double *pprev = (double *)malloc(sizeof(double) * NV);
    double *dp = (double *)malloc(sizeof(double) * dk);
    if (!W || !dW || !pprev || !dp) {
        free(W); free(dW); free(pprev); free(dp);
        return -7;
    }
    /* forward: the gains and the variances before every token */
    for (long bh = 0; bh < BH; ++bh) {
        const long b = bh / H, h = bh % H;
        for (long i = 0; i < dk; ++i)
            dp[i] = p0[bh * dk + i];                       /* running p */
        for (long t = 0; t < T; ++t) {
            const long tok = (b * T + t) * H + h;
            const double *a = alpha + tok * dk, *kt = k + tok * dk, *x = xi + tok * dk;
            double s = r[tok];
            for (long i = 0; i < dk; ++i) {
                pprev[tok * dk + i] = dp[i];
                const double pm = a[i] * a[i] * dp[i] + x[i];
                s += pm * kt[i] * kt[i];
            }
            for (long i = 0; i < dk; ++i) {
                const double pm = a[i] * a[i] * dp[i] + x[i];
                W[tok * dk + i] = (s != 0.0) ? pm * kt[i] / s : 0.0;
                const double den = r[tok] + mu * pm * kt[i] * kt[i];
                dp[i] = (den != 0.0) ? pm * r[tok] / den : pm;
            }
        }
    }
    int rc = backward_memory_w(B, T, H, dk, dv, q, k, v, alpha, W, S0, dO, dS_T, dq, dk_out,
                               dv_out, dalpha, dW, dS0);
    if (rc == 0) {
        for (long bh = 0; bh < BH; ++bh) {
            const long b = bh / H, h = bh % H;
            for (long i = 0; i < dk; ++i)
                dp[i] = dp_T ? dp_T[bh * dk + i] : 0.0;
            for (long t = T - 1; t >= 0; --t) {
                const long tok = (b * T + t) * H + h;
                const double *a = alpha + tok * dk, *kt = k + tok * dk, *x = xi + tok * dk;
                const double *pp = pprev + tok * dk, *dwt = dW + tok * dk;
                const double rt = r[tok];
                double s = rt;
                for (long i = 0; i < dk; ++i) {
                    const double pm = a[i] * a[i] * pp[i] + x[i];
                    s += pm * kt[i] * kt[i];
                }
                double ds = 0.0;
                if (s != 0.0)
                    for (long i = 0; i < dk; ++i) {
                        const double pm = a[i] * a[i] * pp[i] + x[i];
                        ds -= dwt[i] * pm * kt[i] / (s * s);
                    }
                double drt = ds;
                for (long i = 0; i < dk; ++i) {
                    const double pm = a[i] * a[i] * pp[i] + x[i];
                    const double du = (s != 0.0) ? dwt[i] / s : 0.0;
                    const double den = rt + mu * pm * kt[i] * kt[i];
                    double dpm = du * kt[i] + ds * kt[i] * kt[i];
                    double dki = du * pm + 2.0 * ds * pm * kt[i];
                    if (den != 0.0) {
                        dpm += dp[i] * rt * rt / (den * den);
                        dki -= 2.0 * dp[i] * mu * pm * pm * rt * kt[i] / (den * den);
                        drt += dp[i] * mu * pm * pm * kt[i] * kt[i] / (den * den);
                    } else {
                        dpm += dp[i];
                    }
                    dk_out[tok * dk + i] += dki;
                    dalpha[tok * dk + i] += 2.0 * a[i] * pp[i] * dpm;
                    dxi[tok * dk + i] = dpm;
                    dp[i] = a[i] * a[i] * dpm;
                }
                dr[tok] = drt;
            }
            for (long i = 0; i < dk; ++i)
                dp0[bh * dk + i] = dp[i];
        }
    }
    free(W);
    free(dW);
    free(pprev);
    free(dp);
    return rc;
}
